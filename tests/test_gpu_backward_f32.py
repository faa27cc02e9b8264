"""fp32 backward against the fp64 oracle at max-abs 1e-4 per gradient element.

The fp32 backward runs the same gradient kernels as bf16 (instantiated on fp32 tiles
and fp32 MFMA products), so these cases check their pattern logic at a bar that a pair
counted twice or dropped cannot pass: a global key inside a row's window (counted
once), duplicate global indices, global keys on and off a dilated lattice, rows and
sequences without keys, windows that cover the sequence, the one-sided window, the
relative position bias and its table gradient, random blocks, per-sequence global sets
and separate global projections.  The bf16 gradient bars (relative to the reference's
own scale) are in test_gpu_backward.py.
"""

import numpy as np
import pytest
import torch

from oracle import longformer_oracle as orc
from sparse_long_sequence_longformer_amd.workloads import make_bias, make_custom, make_random_blocks
from tests.gpu_common import log, to_dev

pytestmark = pytest.mark.gpu

TOL = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_long_sequence_longformer_amd import binding

    binding.load_library()
    yield


def _pad(B, L, lens):
    if lens is None:
        return None
    if lens == "rand":
        return (np.random.default_rng(7).random((B, L)) < 0.3).astype(np.uint8)
    return (np.arange(L)[None, :] >= np.asarray(lens)[:, None]).astype(np.uint8)


def _padd(pad):
    return None if pad is None else torch.from_numpy(np.ascontiguousarray(pad)).to("cuda")


def _dout(B, H, L, seed):
    return torch.from_numpy(np.random.default_rng(seed + 9000).standard_normal((B, H, L, 64), dtype=np.float32))


def _check(got, ref, what):
    g = got.cpu().to(torch.float64).numpy()
    assert g.shape == ref.shape
    assert np.all(np.isfinite(g)), f"{what}: non-finite"
    err = np.abs(g - ref)
    mx = float(err.max()) if err.size else 0.0
    log(f"  {what}: max-abs {mx:.3e} (scale {float(np.abs(ref).max()) if ref.size else 0.0:.3e})")
    assert mx <= TOL, f"{what}: max-abs {mx} > {TOL}"


def _globals(spec, L, seed):
    if isinstance(spec, str) and spec.startswith("many"):
        n = int(spec[4:])
        return sorted(np.random.default_rng(seed).choice(L, n, replace=False).tolist())
    return spec


# (name, B, H, L, w, dil, globals, pad lengths or "rand", global-key scale, causal)
CASES = [
    ("w0", 1, 1, 200, 0, [1], [], None, 1.0, False),
    ("w0_globals", 1, 2, 130, 0, [1, 3], [7, 7, 129], None, 1.0, False),
    ("window_covers_all", 1, 2, 150, 200, [1, 2], [], None, 1.0, False),
    ("wdil_ge_L", 1, 1, 96, 40, [3], [50], None, 1.0, False),
    ("ragged_1000", 1, 1, 1000, 45, [1], [], None, 1.0, False),
    ("global_in_window_large_score", 1, 1, 333, 20, [1], [100, 101, 300], None, 4.0, False),
    ("globals_on_off_lattice", 1, 3, 400, 17, [3, 2, 4], [30, 31, 32, 33, 200], None, 3.0, False),
    ("dup_globals", 1, 1, 257, 9, [1], [5, 5, 200, 5, 200, 256], None, 1.0, False),
    ("band_fully_padded_rows", 2, 1, 500, 10, [1], [], [500, 120], 1.0, False),
    ("global_in_padding", 2, 2, 300, 12, [1, 2], [3, 250, 299], [300, 200], 2.0, False),
    ("random_padding", 2, 2, 384, 30, [1, 2], [0, 191, 383], "rand", 1.0, False),
    ("many_globals_100", 1, 2, 700, 25, [1, 2], "many100", None, 1.0, False),
    ("mixed_dilations", 1, 4, 640, 21, [1, 2, 3, 5], [10, 11, 320, 639], None, 1.0, False),
    ("tiny_L1", 1, 1, 1, 3, [1], [], None, 1.0, False),
    ("tiny_L2_global", 1, 1, 2, 0, [1], [1], None, 1.0, False),
    ("short_L33", 2, 1, 33, 4, [2], [0], [33, 20], 1.0, False),
    ("all_padded_sequence", 2, 1, 100, 5, [1], [3], [100, 0], 1.0, False),
    ("qa_like_1024", 1, 2, 1024, 256, [1, 1], list(range(16)), None, 1.0, False),
    ("causal_globals_dil", 1, 3, 400, 20, [1, 2, 3], [0, 7, 200, 399], None, 2.0, True),
    ("causal_padded", 2, 2, 333, 24, [1, 2], [3, 250], [333, 200], 1.0, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_f32_backward(case):
    from sparse_long_sequence_longformer_amd import binding

    name, B, H, L, w, dil, Gs, lens, gscale, causal = case
    log(f"case f32 backward {name}: B={B} H={H} L={L} w={w} dil={dil} causal={causal}")
    q, k, v = make_custom(B, H, L, dtype="f32", seed=len(name) + 50)
    G = _globals(Gs, L, len(name))
    if gscale != 1.0 and G:
        k[:, :, G] *= gscale  # global keys with large scores
    do = _dout(B, H, L, len(name))
    pad = _pad(B, L, lens)
    qd, kd, vd, dod = to_dev(q, k, v, do)
    out, lse = binding.forward_lse(qd, kd, vd, w, dil, G, _padd(pad), causal=causal)
    dq, dk, dv = binding.backward(qd, kd, vd, out, dod, lse, w, dil, G, _padd(pad), causal=causal)
    torch.cuda.synchronize()
    rq, rk, rv = orc.attention_backward(q, k, v, do, w, dil, G, pad, causal=causal)
    _check(dq, rq, f"{name} dq")
    _check(dk, rk, f"{name} dk")
    _check(dv, rv, f"{name} dv")


@pytest.mark.parametrize("causal", [False, True])
def test_f32_backward_bias_and_table_gradient(causal):
    from sparse_long_sequence_longformer_amd import binding

    B, H, L, w, dil, G = 2, 2, 500, 30, [1, 2], [0, 9, 250, 499]
    q, k, v = make_custom(B, H, L, dtype="f32", seed=61)
    do = _dout(B, H, L, 61)
    pad = _pad(B, L, [500, 320])
    tab = make_bias(H, w, seed=5, scale=2.0)
    qd, kd, vd, dod = to_dev(q, k, v, do)
    bd = torch.from_numpy(tab).to("cuda")
    out, lse = binding.forward_lse(qd, kd, vd, w, dil, G, _padd(pad), causal=causal, bias=bd)
    dq, dk, dv, db = binding.backward(qd, kd, vd, out, dod, lse, w, dil, G, _padd(pad), causal=causal, bias=bd,
                                      dbias=True)
    torch.cuda.synchronize()
    rq, rk, rv = orc.attention_backward(q, k, v, do, w, dil, G, pad, causal=causal, bias=tab)
    _check(dq, rq, "bias dq")
    _check(dk, rk, "bias dk")
    _check(dv, rv, "bias dv")
    # the table gradient sums about L * B terms per entry: same bar relative to its scale
    rdb = orc.attention_bias_grad(q, k, v, do, w, dil, G, pad, causal=causal, bias=tab)
    err = float(np.abs(db.cpu().double().numpy() - rdb).max())
    log(f"  dbias: max-abs {err:.3e} (scale {float(np.abs(rdb).max()):.3e})")
    assert err <= TOL * max(1.0, float(np.abs(rdb).max()))


def test_f32_backward_random_blocks():
    from sparse_long_sequence_longformer_amd import binding

    B, H, L, w, G = 2, 2, 640, 40, [0, 333]
    q, k, v = make_custom(B, H, L, dtype="f32", seed=62)
    do = _dout(B, H, L, 62)
    pad = _pad(B, L, [640, 500])
    rnd = make_random_blocks(H, L, 3, seed=13)
    qd, kd, vd, dod = to_dev(q, k, v, do)
    for causal in (False, True):
        out, lse = binding.forward_lse(qd, kd, vd, w, [1, 1], G, _padd(pad), causal=causal, rand=rnd)
        dq, dk, dv = binding.backward(qd, kd, vd, out, dod, lse, w, [1, 1], G, _padd(pad), causal=causal, rand=rnd)
        torch.cuda.synchronize()
        rq, rk, rv = orc.attention_backward(q, k, v, do, w, [1, 1], G, pad, causal=causal, rand=rnd)
        _check(dq, rq, f"random causal={causal} dq")
        _check(dk, rk, f"random causal={causal} dk")
        _check(dv, rv, f"random causal={causal} dv")


def test_f32_backward_per_sequence_globals():
    from sparse_long_sequence_longformer_amd import binding

    B, H, L, w, dil = 3, 2, 400, 20, [1, 2]
    G = np.array([[0, 5, 5, 399], [200, -1, -1, -1], [-1, -1, -1, -1]], dtype=np.int32)
    q, k, v = make_custom(B, H, L, dtype="f32", seed=63)
    do = _dout(B, H, L, 63)
    pad = _pad(B, L, [400, 300, 400])
    qd, kd, vd, dod = to_dev(q, k, v, do)
    out, lse = binding.forward_lse(qd, kd, vd, w, dil, G, _padd(pad))
    dq, dk, dv = binding.backward(qd, kd, vd, out, dod, lse, w, dil, G, _padd(pad))
    torch.cuda.synchronize()
    rq, rk, rv = orc.attention_backward(q, k, v, do, w, dil, G, pad)
    _check(dq, rq, "per-sequence dq")
    _check(dk, rk, "per-sequence dk")
    _check(dv, rv, "per-sequence dv")


def test_f32_backward_global_proj():
    from sparse_long_sequence_longformer_amd import binding

    B, H, L, w, dil, G = 2, 2, 500, 30, [1, 2], [0, 9, 250, 499] + list(range(100, 140))
    q, k, v = make_custom(B, H, L, dtype="f32", seed=64)
    qg, kg, vg = make_custom(B, H, L, dtype="f32", seed=65)
    do = _dout(B, H, L, 64)
    pad = _pad(B, L, [500, 320])
    dev = to_dev(q, k, v, qg, kg, vg, do)
    out, lse = binding.forward_global_proj_lse(*dev[:6], w, dil, G, _padd(pad))
    grads = binding.backward_global_proj(*dev[:6], out, dev[6], lse, w, dil, G, _padd(pad))
    torch.cuda.synchronize()
    refs = orc.attention_backward_global_proj(q, k, v, qg, kg, vg, do, w, dil, G, pad)
    for n, g, r in zip(("dq", "dk", "dv", "dq_g", "dk_g", "dv_g"), grads, refs):
        _check(g, r, f"global_proj {n}")


def test_f32_backward_deterministic():
    from sparse_long_sequence_longformer_amd import binding

    B, H, L, w, dil, G = 1, 2, 700, 25, [1, 2], [3, 400, 401]
    q, k, v = make_custom(B, H, L, dtype="f32", seed=66)
    do = _dout(B, H, L, 66)
    qd, kd, vd, dod = to_dev(q, k, v, do)
    out, lse = binding.forward_lse(qd, kd, vd, w, dil, G)
    a = binding.backward(qd, kd, vd, out, dod, lse, w, dil, G)
    b = binding.backward(qd, kd, vd, out, dod, lse, w, dil, G)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)

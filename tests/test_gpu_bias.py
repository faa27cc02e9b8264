"""Relative position bias on the window scores: HIP path (handle with a bias table)
against the fp64 oracle with the same table.

Forward tolerances as everywhere (fp32 max-abs 1e-4; bf16 max-abs 2e-2, mean-abs
2e-3), log-sum-exp max-abs 1e-4 / 2e-2, gradients max-abs 2e-2 and mean-abs 1e-2 of
the reference scale.  Tables are N(0, s^2): s = 1 for a learned-looking bias, s = 4
to push window scores far above and below the unbiased ones (the running maximum
then moves inside a tile), plus a table with a -30 row that switches offsets off.
"""

import numpy as np
import pytest
import torch

from oracle import longformer_oracle as orc
from oracle import layer_oracle as lorc
from sparse_long_sequence_longformer_amd.workloads import make_bias, make_custom
from tests.gpu_common import compare, log, sample_rows, to_dev
from tests.test_gpu_backward import _compare_grad, _dout

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_long_sequence_longformer_amd import binding

    binding.load_library()
    yield


def _pad_from_lengths(B, L, lengths):
    if lengths is None:
        return None
    return (np.arange(L)[None, :] >= np.asarray(lengths)[:, None]).astype(np.uint8)


def _padd(pad):
    return None if pad is None else torch.from_numpy(np.ascontiguousarray(pad)).to("cuda")


def _table(H, w, seed, scale):
    t = make_bias(H, w, seed=seed, scale=scale)
    if scale < 0:  # a table that switches every third offset off
        t = np.abs(t)
        t[:, ::3] = -30.0
    return t


def _check_lse(lse, ref, dtype):
    got = lse.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isneginf(got), np.isneginf(ref))
    fin = np.isfinite(ref)
    if fin.any():
        e = np.abs(got[fin] - ref[fin]).max()
        log(f"  lse max-abs {e:.3e}")
        assert e <= (1e-4 if dtype == "f32" else 2e-2)


# (name, dtype, B, H, L, w, dil, globals, pad lengths, causal, bias scale)
FWD_CASES = [
    ("f32_plain", "f32", 1, 2, 300, 20, [1, 1], [], None, False, 1.0),
    ("f32_globals_dil", "f32", 1, 3, 400, 17, [1, 2, 3], [0, 31, 200, 399], None, False, 1.0),
    ("f32_padded_big", "f32", 2, 2, 350, 25, [1, 2], [5, 300], [350, 210], False, 4.0),
    ("f32_off_rows", "f32", 1, 2, 384, 30, [1, 3], [0, 191], None, False, -1.0),
    ("f32_w_ge_L", "f32", 1, 1, 150, 300, [1], [7], None, False, 1.0),
    ("f32_w0", "f32", 1, 1, 130, 0, [1], [64], None, False, 2.0),
    ("f32_causal", "f32", 1, 3, 400, 17, [1, 2, 3], [0, 31, 200, 399], None, True, 1.0),
    ("f32_causal_big_pad", "f32", 2, 2, 350, 25, [1, 2], [5, 300], [350, 210], True, 4.0),
    ("bf16_plain", "bf16", 1, 2, 700, 64, [1, 2], [3, 400], None, False, 1.0),
    ("bf16_lm_like_2048", "bf16", 1, 4, 2048, 512, [1, 1, 2, 3], [], None, False, 1.0),
    ("bf16_qa_like_1500", "bf16", 2, 2, 1500, 256, [1, 2], list(range(16)), [1500, 900], False, 4.0),
    ("bf16_causal_1024", "bf16", 1, 2, 1024, 256, [1, 2], [0, 500], None, True, 1.0),
    ("bf16_max_w", "bf16", 1, 1, 2300, 1024, [1], [100], None, False, 1.0),
]


@pytest.mark.parametrize("case", FWD_CASES, ids=[c[0] for c in FWD_CASES])
def test_bias_forward(case):
    from sparse_long_sequence_longformer_amd import binding

    name, dtype, B, H, L, w, dil, G, lens, causal, scale = case
    log(f"case bias forward {name}: B={B} H={H} L={L} w={w} dil={dil} causal={causal} scale={scale}")
    q, k, v = make_custom(B, H, L, dtype=dtype, seed=len(name) + 400)
    tab = _table(H, w, len(name), scale)
    pad = _pad_from_lengths(B, L, lens)
    qd, kd, vd = to_dev(q, k, v)
    bd = torch.from_numpy(tab).to("cuda")
    out, lse = binding.forward_lse(qd, kd, vd, w, dil, G, _padd(pad), causal=causal, bias=bd)
    plain = binding.forward(qd, kd, vd, w, dil, G, _padd(pad), causal=causal, bias=bd)
    torch.cuda.synchronize()
    assert torch.equal(out, plain)
    if L * L * B * H <= 6_000_000:
        compare(out.cpu(), orc.attention(q, k, v, w, dil, G, pad, causal=causal, bias=tab), dtype, name)
        _check_lse(lse, orc.attention_lse(q, k, w, dil, G, pad, causal=causal, bias=tab), dtype)
    else:
        smp = sample_rows(B, H, L, G, pad, 160, seed=len(name))
        ref = orc.attention_sampled(q, k, v, w, dil, G, pad, smp, causal=causal, bias=tab)
        got = torch.stack([out[b, h, i].cpu() for b, h, i in smp])
        compare(got, ref, dtype, f"{name} sampled")


def test_bias_zero_table_is_unbiased():
    """A zero table gives the unbiased result bit for bit (a zero add changes no score)
    on the same tiling (the biased forward always runs 128-row work-groups)."""
    from sparse_long_sequence_longformer_amd import binding

    B, H, L, w, dil, G = 1, 2, 600, 40, [1, 2], [0, 299]
    q, k, v = make_custom(B, H, L, dtype="bf16", seed=77)
    qd, kd, vd = to_dev(q, k, v)
    zero = torch.zeros(H, 2 * w + 1, dtype=torch.float32, device="cuda")
    h = binding.LfAttn("bf16")
    h.set_tile_rows(128)
    a = binding.forward(qd, kd, vd, w, dil, G, bias=zero, handle=h)
    b = binding.forward(qd, kd, vd, w, dil, G, handle=h)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_bias_handle_setting_and_restore():
    """A bias set on a handle applies to every call; a per-call table restores it."""
    from sparse_long_sequence_longformer_amd import binding

    B, H, L, w, dil, G = 1, 2, 400, 30, [1, 1], [10]
    q, k, v = make_custom(B, H, L, dtype="f32", seed=78)
    qd, kd, vd = to_dev(q, k, v)
    t1, t2 = make_bias(H, w, seed=1), make_bias(H, w, seed=2)
    h = binding.LfAttn("f32")
    try:
        h.set_position_bias(torch.from_numpy(t1).to("cuda"))
        o1 = binding.forward(qd, kd, vd, w, dil, G, handle=h)
        o2 = binding.forward(qd, kd, vd, w, dil, G, handle=h, bias=torch.from_numpy(t2).to("cuda"))
        o1b = binding.forward(qd, kd, vd, w, dil, G, handle=h)
        torch.cuda.synchronize()
        assert torch.equal(o1, o1b)
        compare(o1.cpu(), orc.attention(q, k, v, w, dil, G, bias=t1), "f32", "handle table")
        compare(o2.cpu(), orc.attention(q, k, v, w, dil, G, bias=t2), "f32", "per-call table")
        with pytest.raises(binding.LfAttnError):
            binding.forward(qd, kd, vd, w + 1, dil, G, handle=h)
        h.set_position_bias(None)
        o0 = binding.forward(qd, kd, vd, w, dil, G, handle=h)
        torch.cuda.synchronize()
        compare(o0.cpu(), orc.attention(q, k, v, w, dil, G), "f32", "removed")
    finally:
        h.close()


def test_bias_global_proj():
    from sparse_long_sequence_longformer_amd import binding

    B, H, L, w, dil, G = 2, 2, 500, 30, [1, 2], [0, 9, 250, 499] + list(range(100, 140))
    q, k, v = make_custom(B, H, L, dtype="f32", seed=401)
    qg, kg, vg = make_custom(B, H, L, dtype="f32", seed=402)
    pad = _pad_from_lengths(B, L, [500, 320])
    tab = make_bias(H, w, seed=3, scale=2.0)
    out = binding.forward_global_proj(*to_dev(q, k, v, qg, kg, vg), w, dil, G, _padd(pad),
                                      bias=torch.from_numpy(tab).to("cuda"))
    torch.cuda.synchronize()
    compare(out.cpu(), orc.attention_global_proj(q, k, v, qg, kg, vg, w, dil, G, pad, bias=tab), "f32",
            "global_proj + bias")


BWD_CASES = [
    ("plain", 1, 2, 300, 16, [1, 1], [], None, False, 1.0),
    ("globals_dil", 1, 3, 400, 20, [1, 2, 3], [0, 7, 200, 399], None, False, 1.0),
    ("padded_big", 2, 2, 333, 24, [1, 2], [3, 250], [333, 200], False, 4.0),
    ("off_rows", 1, 2, 384, 30, [1, 3], [0, 191], None, False, -1.0),
    ("w_ge_L", 1, 1, 150, 200, [1], [5], None, False, 1.0),
    ("causal_globals", 1, 3, 400, 20, [1, 2, 3], [0, 7, 200, 399], None, True, 1.0),
    ("causal_padded", 2, 2, 333, 24, [1, 2], [3, 250], [333, 200], True, 2.0),
    ("lm_like_1024", 1, 2, 1024, 256, [1, 2], [], None, False, 1.0),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_bias_backward(case):
    from sparse_long_sequence_longformer_amd import binding

    name, B, H, L, w, dil, G, lens, causal, scale = case
    log(f"case bias backward {name}: B={B} H={H} L={L} w={w} dil={dil} causal={causal} scale={scale}")
    q, k, v = make_custom(B, H, L, dtype="bf16", seed=len(name) + 500)
    do = _dout(B, H, L, len(name) + 500)
    tab = _table(H, w, len(name) + 1, scale)
    pad = _pad_from_lengths(B, L, lens)
    qd, kd, vd, dod = to_dev(q, k, v, do)
    bd = torch.from_numpy(tab).to("cuda")
    out, lse = binding.forward_lse(qd, kd, vd, w, dil, G, _padd(pad), causal=causal, bias=bd)
    dq, dk, dv = binding.backward(qd, kd, vd, out, dod, lse, w, dil, G, _padd(pad), causal=causal, bias=bd)
    torch.cuda.synchronize()
    rq, rk, rv = orc.attention_backward(q, k, v, do, w, dil, G, pad, causal=causal, bias=tab)
    _compare_grad(dq.cpu(), rq, f"{name} dq")
    _compare_grad(dk.cpu(), rk, f"{name} dk")
    _compare_grad(dv.cpu(), rv, f"{name} dv")


def test_bias_layer():
    """The layer passes the handle's table to its attention (scale 4: the bias moves
    the output well beyond the tolerance, checked against the unbiased oracle)."""
    from sparse_long_sequence_longformer_amd import binding
    from tests.test_gpu_layer import TOL_MAX, TOL_MEAN, _weights

    B, L, E, F, w, dil, G = 1, 512, 128, 256, 48, [1, 2], [0, 300]
    H = E // 64
    x = torch.from_numpy(np.random.default_rng(5).standard_normal((B, L, E), dtype=np.float32)).bfloat16()
    W = _weights(E, F, 6, scale=0.1)
    tab = make_bias(H, w, seed=4, scale=4.0)
    out = binding.layer_forward(x.cuda(), {n: t.cuda() for n, t in W.items()}, w, dil, G,
                                bias=torch.from_numpy(tab).cuda())
    torch.cuda.synchronize()
    ref = lorc.layer_forward(x, W, H, w, dil, G, bias=tab)
    got = out.cpu().double().numpy()
    err = np.abs(got - ref)
    log(f"  layer + bias: max-abs {err.max():.3e} mean-abs {err.mean():.3e}")
    assert err.max() <= TOL_MAX and err.mean() <= TOL_MEAN
    moved = np.abs(lorc.layer_forward(x, W, H, w, dil, G) - ref).max()
    log(f"  bias moves the layer output by {moved:.3e}")
    assert moved > 10 * TOL_MAX


# Gradient of the table (lf_attn_backward_bias) against the oracle's, with the bars of
# the other gradients (relative to the reference's own scale); dq, dk, dv must equal
# those of the plain backward bit for bit (the table gradient only adds sums).
DBIAS_CASES = BWD_CASES + [
    ("qa_like_1500", 2, 2, 1500, 256, [1, 2], list(range(16)), [1500, 900], False, 1.0),
    ("max_w_2300", 1, 1, 2300, 1024, [1], [100], None, False, 1.0),
]


@pytest.mark.parametrize("case", DBIAS_CASES, ids=[c[0] for c in DBIAS_CASES])
def test_bias_table_gradient(case):
    from sparse_long_sequence_longformer_amd import binding

    name, B, H, L, w, dil, G, lens, causal, scale = case
    log(f"case bias table gradient {name}: B={B} H={H} L={L} w={w} dil={dil} causal={causal} scale={scale}")
    q, k, v = make_custom(B, H, L, dtype="bf16", seed=len(name) + 600)
    do = _dout(B, H, L, len(name) + 600)
    tab = _table(H, w, len(name) + 2, scale)
    pad = _pad_from_lengths(B, L, lens)
    qd, kd, vd, dod = to_dev(q, k, v, do)
    bd = torch.from_numpy(tab).to("cuda")
    out, lse = binding.forward_lse(qd, kd, vd, w, dil, G, _padd(pad), causal=causal, bias=bd)
    dq, dk, dv, db = binding.backward(qd, kd, vd, out, dod, lse, w, dil, G, _padd(pad), causal=causal, bias=bd,
                                      dbias=True)
    pq, pk, pv = binding.backward(qd, kd, vd, out, dod, lse, w, dil, G, _padd(pad), causal=causal, bias=bd)
    db2 = torch.full_like(db, float("nan"))
    binding.backward(qd, kd, vd, out, dod, lse, w, dil, G, _padd(pad), causal=causal, bias=bd, dbias=db2)
    torch.cuda.synchronize()
    assert torch.equal(dq, pq) and torch.equal(dk, pk) and torch.equal(dv, pv)
    assert torch.equal(db, db2), "table gradient differs between two calls"
    ref = orc.attention_bias_grad(q, k, v, do, w, dil, G, pad, causal=causal, bias=tab)
    _compare_grad(db.cpu(), ref, f"{name} dbias")


def test_bias_table_gradient_random_blocks():
    """Pairs that enter through a random block carry no bias and add nothing."""
    from sparse_long_sequence_longformer_amd import binding
    from sparse_long_sequence_longformer_amd.workloads import make_random_blocks

    B, H, L, w, G = 2, 2, 640, 40, [0, 333]
    q, k, v = make_custom(B, H, L, dtype="bf16", seed=610)
    do = _dout(B, H, L, 610)
    tab = _table(H, w, 11, 2.0)
    pad = _pad_from_lengths(B, L, [640, 500])
    rnd = make_random_blocks(H, L, 3, seed=12)
    qd, kd, vd, dod = to_dev(q, k, v, do)
    bd = torch.from_numpy(tab).to("cuda")
    for causal in (False, True):
        out, lse = binding.forward_lse(qd, kd, vd, w, [1, 1], G, _padd(pad), causal=causal, bias=bd, rand=rnd)
        *_, db = binding.backward(qd, kd, vd, out, dod, lse, w, [1, 1], G, _padd(pad), causal=causal, bias=bd,
                                  rand=rnd, dbias=True)
        torch.cuda.synchronize()
        ref = orc.attention_bias_grad(q, k, v, do, w, [1, 1], G, pad, causal=causal, bias=tab, rand=rnd)
        _compare_grad(db.cpu(), ref, f"random causal={causal} dbias")


def test_bias_table_gradient_needs_table():
    from sparse_long_sequence_longformer_amd import binding

    B, H, L, w = 1, 1, 200, 10
    q, k, v = make_custom(B, H, L, dtype="bf16", seed=620)
    qd, kd, vd = to_dev(q, k, v)
    out, lse = binding.forward_lse(qd, kd, vd, w, [1], [])
    with pytest.raises(binding.LfAttnError):
        binding.backward(qd, kd, vd, out, out, lse, w, [1], [], dbias=True)
    with pytest.raises(ValueError):
        binding.backward(qd, kd, vd, out, out, lse, w, [1], [], bias=torch.zeros(H, 2 * w + 1, device="cuda"),
                         dbias=torch.zeros(H, 2 * w, device="cuda"))

"""Random key blocks (BigBird-style random attention): HIP path (handle with random
draws) against the fp64 oracle with the same draws.

Tolerances as everywhere: fp32 max-abs 1e-4; bf16 max-abs 2e-2 and mean-abs 2e-3;
gradients max-abs 2e-2 and mean-abs 1e-2 of the reference scale;
log-sum-exp max-abs 1e-4 / 2e-2.  Draws come from the seeded generator (r distinct
key blocks per head and query block), plus hand-made tables with duplicates, unused
entries, every block, and each row's own block.
"""

import numpy as np
import pytest
import torch

from oracle import layer_oracle as lorc
from oracle import longformer_oracle as orc
from sparse_long_sequence_longformer_amd.workloads import make_bias, make_custom, make_random_blocks
from tests.gpu_common import compare, log, sample_rows, to_dev

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


def _draws(kind, H, L, seed):
    n = (L + 63) // 64
    if isinstance(kind, int):
        return make_random_blocks(H, L, kind, seed=seed)
    rng = np.random.default_rng(seed)
    if kind == "dups":  # duplicates and unused entries
        return rng.integers(-1, n, size=(H, n, 5)).astype(np.int32)
    if kind == "every":
        return np.tile(np.arange(n, dtype=np.int32), (H, n, 1))
    if kind == "own":
        return np.tile(np.arange(n, dtype=np.int32)[:, None], (H, 1, 1))
    if kind == "max":
        return np.stack([np.stack([rng.choice(n, 16, replace=False) for _ in range(n)]) for _ in range(H)]).astype(
            np.int32)
    raise ValueError(kind)


def _check_lse(lse, ref, dtype):
    got = lse.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isneginf(got), np.isneginf(ref))
    fin = np.isfinite(ref)
    if fin.any():
        e = np.abs(got[fin] - ref[fin]).max()
        log(f"  lse max-abs {e:.3e}")
        assert e <= (1e-4 if dtype == "f32" else 2e-2)


# (name, dtype, B, H, L, w, globals, pad lengths, causal, draws)
FWD_CASES = [
    ("f32_ragged_300", "f32", 1, 2, 300, 20, [0, 150], None, False, 2),
    ("f32_padded", "f32", 2, 2, 384, 16, [5, 200], [384, 230], False, 3),
    ("f32_causal", "f32", 1, 2, 400, 24, [0, 99, 399], None, True, 2),
    ("f32_causal_padded", "f32", 2, 1, 333, 10, [7], [333, 150], True, 4),
    ("f32_w0", "f32", 1, 2, 256, 0, [], None, False, 4),
    ("f32_dups", "f32", 1, 3, 500, 30, [0, 1, 2], None, False, "dups"),
    ("f32_every_block", "f32", 1, 1, 256, 5, [], None, False, "every"),
    ("f32_own_block", "f32", 1, 2, 320, 70, [64], None, False, "own"),
    ("f32_small_L", "f32", 1, 1, 50, 3, [], None, False, "every"),
    ("f32_many_globals", "f32", 1, 2, 640, 20, list(range(0, 640, 9)), None, False, 3),
    ("bf16_1024", "bf16", 1, 2, 1024, 128, [0, 511], None, False, 3),
    ("bf16_causal_1024", "bf16", 1, 2, 1024, 128, [0, 511], None, True, 3),
    ("bf16_max_draws_2048", "bf16", 1, 2, 2048, 64, [3], None, False, "max"),
    ("bf16_qa_like_4096", "bf16", 2, 2, 4096, 256, list(range(16)), [4096, 3000], False, 3),
]


@pytest.mark.parametrize("case", FWD_CASES, ids=[c[0] for c in FWD_CASES])
def test_random_forward(case):
    from sparse_long_sequence_longformer_amd import binding

    name, dtype, B, H, L, w, G, lens, causal, kind = case
    log(f"case random forward {name}: B={B} H={H} L={L} w={w} causal={causal} draws={kind}")
    q, k, v = make_custom(B, H, L, dtype=dtype, seed=len(name) + 600)
    rnd = _draws(kind, H, L, len(name))
    pad = _pad_from_lengths(B, L, lens)
    qd, kd, vd = to_dev(q, k, v)
    dil = [1] * H
    out, lse = binding.forward_lse(qd, kd, vd, w, dil, G, _padd(pad), causal=causal, rand=rnd)
    plain = binding.forward(qd, kd, vd, w, dil, G, _padd(pad), causal=causal, rand=rnd)
    torch.cuda.synchronize()
    assert torch.equal(out, plain)
    if L * L * B * H <= 6_000_000:
        compare(out.cpu(), orc.attention(q, k, v, w, dil, G, pad, causal=causal, rand=rnd), dtype, name)
        _check_lse(lse, orc.attention_lse(q, k, w, dil, G, pad, causal=causal, rand=rnd), dtype)
    else:
        smp = sample_rows(B, H, L, G, pad, 160, seed=len(name))
        ref = orc.attention_sampled(q, k, v, w, dil, G, pad, smp, causal=causal, rand=rnd)
        got = torch.stack([out[b, h, i].cpu() for b, h, i in smp])
        compare(got, ref, dtype, f"{name} sampled")
    if kind not in ("own",):  # the draws change the result
        base = binding.forward(qd, kd, vd, w, dil, G, _padd(pad), causal=causal)
        torch.cuda.synchronize()
        assert not torch.equal(base, out)


def test_random_own_block_is_window():
    """Drawing each row's own block with w >= 63 adds no key: bit-identical output on
    the same tiling (the forward with random blocks always runs 128-row work-groups)."""
    from sparse_long_sequence_longformer_amd import binding

    B, H, L, w, G = 1, 2, 700, 64, [3, 400]
    q, k, v = make_custom(B, H, L, dtype="bf16", seed=81)
    qd, kd, vd = to_dev(q, k, v)
    h = binding.LfAttn("bf16")
    h.set_tile_rows(128)
    a = binding.forward(qd, kd, vd, w, [1, 1], G, rand=_draws("own", H, L, 0), handle=h)
    b = binding.forward(qd, kd, vd, w, [1, 1], G, handle=h)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_random_with_bias_and_global_proj():
    from sparse_long_sequence_longformer_amd import binding

    B, H, L, w, G = 2, 2, 448, 24, [0, 9, 250]
    q, k, v = make_custom(B, H, L, dtype="f32", seed=82)
    qg, kg, vg = make_custom(B, H, L, dtype="f32", seed=83)
    pad = _pad_from_lengths(B, L, [448, 300])
    rnd = make_random_blocks(H, L, 3, seed=5)
    tab = make_bias(H, w, seed=6, scale=2.0)
    bd = torch.from_numpy(tab).to("cuda")
    out = binding.forward(*to_dev(q, k, v), w, [1, 1], G, _padd(pad), bias=bd, rand=rnd)
    gp = binding.forward_global_proj(*to_dev(q, k, v, qg, kg, vg), w, [1, 1], G, _padd(pad), bias=bd, rand=rnd)
    torch.cuda.synchronize()
    compare(out.cpu(), orc.attention(q, k, v, w, [1, 1], G, pad, bias=tab, rand=rnd), "f32", "random + bias")
    ref = orc.attention_global_proj(q, k, v, qg, kg, vg, w, [1, 1], G, pad, bias=tab, rand=rnd)
    compare(gp.cpu(), ref, "f32", "global proj + random + bias")


def test_random_handle_errors_and_reuse():
    from sparse_long_sequence_longformer_amd import binding

    B, H, L, w = 1, 2, 512, 16
    q, k, v = make_custom(B, H, L, dtype="f32", seed=84)
    qd, kd, vd = to_dev(q, k, v)
    h = binding.LfAttn("f32")
    try:
        r1, r2 = make_random_blocks(H, L, 2, seed=1), make_random_blocks(H, L, 2, seed=2)
        h.set_random_blocks(r1)
        o1 = binding.forward(qd, kd, vd, w, [1, 1], handle=h)
        h.set_random_blocks(r2)
        o2 = binding.forward(qd, kd, vd, w, [1, 1], handle=h)
        torch.cuda.synchronize()
        compare(o1.cpu(), orc.attention(q, k, v, w, [1, 1], rand=r1), "f32", "first draws")
        compare(o2.cpu(), orc.attention(q, k, v, w, [1, 1], rand=r2), "f32", "second draws")
        with pytest.raises(binding.LfAttnError):
            binding.forward(qd, kd, vd, w, [1, 2], handle=h)  # dilated head
        q2, k2, v2 = to_dev(*make_custom(B, H, L + 64, dtype="f32", seed=85))
        with pytest.raises(binding.LfAttnError):
            binding.forward(q2, k2, v2, w, [1, 1], handle=h)  # another number of query blocks
        h.set_random_blocks(None)
        o0 = binding.forward(qd, kd, vd, w, [1, 1], handle=h)
        torch.cuda.synchronize()
        compare(o0.cpu(), orc.attention(q, k, v, w, [1, 1]), "f32", "removed")
    finally:
        h.close()


def test_random_layer():
    from sparse_long_sequence_longformer_amd import binding
    from tests.test_gpu_layer import TOL_MAX, TOL_MEAN, _weights

    B, L, E, F, w, G = 1, 512, 128, 256, 32, [0, 300]
    H = E // 64
    x = torch.from_numpy(np.random.default_rng(8).standard_normal((B, L, E), dtype=np.float32)).bfloat16()
    W = _weights(E, F, 9, scale=0.1)
    rnd = make_random_blocks(H, L, 3, seed=7)
    out = binding.layer_forward(x.cuda(), {n: t.cuda() for n, t in W.items()}, w, [1] * H, G, rand=rnd)
    torch.cuda.synchronize()
    ref = lorc.layer_forward(x, W, H, w, [1] * H, G, rand=rnd)
    err = np.abs(out.cpu().double().numpy() - ref)
    log(f"  layer + random: max-abs {err.max():.3e} mean-abs {err.mean():.3e}")
    assert err.max() <= TOL_MAX and err.mean() <= TOL_MEAN


# (name, B, H, L, w, globals, pad lengths, causal, draws)
BWD_CASES = [
    ("plain_ragged", 1, 2, 300, 16, [], None, False, 2),
    ("globals_padded", 2, 2, 384, 20, [0, 7, 200, 383], [384, 250], False, 3),
    ("causal_globals", 1, 2, 400, 24, [0, 99, 399], None, True, 3),
    ("causal_padded_dups", 2, 1, 333, 10, [7, 150], [333, 150], True, "dups"),
    ("w0_every_block", 1, 1, 256, 0, [5], None, False, "every"),
    ("many_globals", 1, 2, 640, 20, list(range(0, 640, 9)), None, False, 3),
    ("lm_like_1024", 1, 2, 1024, 128, [0, 511], None, False, 3),
    ("max_draws_1024", 1, 1, 1024, 32, [3], None, False, "max"),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_random_backward(case):
    from sparse_long_sequence_longformer_amd import binding
    from tests.test_gpu_backward import _compare_grad, _dout

    name, B, H, L, w, G, lens, causal, kind = case
    log(f"case random backward {name}: B={B} H={H} L={L} w={w} causal={causal} draws={kind}")
    q, k, v = make_custom(B, H, L, dtype="bf16", seed=len(name) + 700)
    do = _dout(B, H, L, len(name) + 700)
    rnd = _draws(kind, H, L, len(name) + 1)
    pad = _pad_from_lengths(B, L, lens)
    qd, kd, vd, dod = to_dev(q, k, v, do)
    dil = [1] * H
    out, lse = binding.forward_lse(qd, kd, vd, w, dil, G, _padd(pad), causal=causal, rand=rnd)
    dq, dk, dv = binding.backward(qd, kd, vd, out, dod, lse, w, dil, G, _padd(pad), causal=causal, rand=rnd)
    torch.cuda.synchronize()
    rq, rk, rv = orc.attention_backward(q, k, v, do, w, dil, G, pad, causal=causal, rand=rnd)
    _compare_grad(dq.cpu(), rq, f"{name} dq")
    _compare_grad(dk.cpu(), rk, f"{name} dk")
    _compare_grad(dv.cpu(), rv, f"{name} dv")


@pytest.mark.parametrize("row", [0, 70, 200, 299])
def test_random_backward_structure_exact(row):
    """dO on one row only: dK, dV exactly zero off that row's key set (window, globals
    and its query block's draws), nonzero on it; dQ zero on every other row."""
    from oracle import brute
    from sparse_long_sequence_longformer_amd import binding
    from tests.test_gpu_backward import _dout

    B, H, L, w, G = 1, 2, 300, 6, [7, 200]
    pad = np.zeros((B, L), dtype=np.uint8)
    pad[0, [20, 150, 151, 290]] = 1
    rnd = make_random_blocks(H, L, 2, seed=11)
    q, k, v = make_custom(B, H, L, dtype="bf16", seed=53)
    do = torch.zeros(B, H, L, 64, dtype=torch.bfloat16)
    do[:, :, row] = _dout(B, H, 1, row)[:, :, 0]
    qd, kd, vd, dod = to_dev(q, k, v, do)
    out, lse = binding.forward_lse(qd, kd, vd, w, [1, 1], G, _padd(pad), rand=rnd)
    dq, dk, dv = (t.cpu() for t in binding.backward(qd, kd, vd, out, dod, lse, w, [1, 1], G, _padd(pad), rand=rnd))
    for h in range(H):
        keys = set(brute.key_set(row, L, w, 1, G, pad[0].astype(bool).tolist(), rand=rnd[h], rand_block=64))
        off = torch.from_numpy(np.array([j not in keys for j in range(L)]))
        assert torch.all(dk[0, h][off] == 0) and torch.all(dv[0, h][off] == 0), (h, row)
        assert bool((dv[0, h][~off].abs().amax(dim=1) > 0).all()), (h, row)
        others = torch.ones(L, dtype=torch.bool)
        others[row] = False
        assert torch.all(dq[0, h][others] == 0), (h, row)


def test_random_backward_with_bias():
    from sparse_long_sequence_longformer_amd import binding
    from tests.test_gpu_backward import _compare_grad, _dout

    B, H, L, w, G = 1, 2, 448, 24, [0, 250]
    q, k, v = make_custom(B, H, L, dtype="bf16", seed=91)
    do = _dout(B, H, L, 91)
    rnd = make_random_blocks(H, L, 3, seed=12)
    tab = make_bias(H, w, seed=13, scale=2.0)
    bd = torch.from_numpy(tab).to("cuda")
    qd, kd, vd, dod = to_dev(q, k, v, do)
    out, lse = binding.forward_lse(qd, kd, vd, w, [1, 1], G, bias=bd, rand=rnd)
    dq, dk, dv = binding.backward(qd, kd, vd, out, dod, lse, w, [1, 1], G, bias=bd, rand=rnd)
    torch.cuda.synchronize()
    rq, rk, rv = orc.attention_backward(q, k, v, do, w, [1, 1], G, bias=tab, rand=rnd)
    _compare_grad(dq.cpu(), rq, "bias+random dq")
    _compare_grad(dk.cpu(), rk, "bias+random dk")
    _compare_grad(dv.cpu(), rv, "bias+random dv")

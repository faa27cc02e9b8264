"""Backward pass (``lf_attn_forward_lse`` + ``lf_attn_backward``) against the fp64
oracle on seeded inputs.

Parity bar (bf16 inputs and outputs, fp32 accumulation), per gradient tensor:
max-abs error <= 2e-2 * max|ref| and mean-abs error <= 1e-2 * mean|ref| (the bf16
rounding of the recomputed weights, of dS and of the stored gradient is 2^-9
relative per term).  The forward's log-sum-exp: max-abs 1e-4 for fp32 inputs,
2e-2 for bf16; -inf exactly on rows without keys.  Sparsity structure is checked
exactly: with dO nonzero on one row only, every gradient entry outside that row's
key set is exactly zero.
"""

import numpy as np
import pytest
import torch

from oracle import longformer_oracle as orc
from oracle import brute
from sparse_long_sequence_longformer_amd import workloads
from sparse_long_sequence_longformer_amd.workloads import make_custom, make_qkv
from tests.gpu_common import log, to_dev

pytestmark = pytest.mark.gpu

GRAD_MAX_REL = 2e-2
GRAD_MEAN_REL = 1e-2


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


def _dout(B, H, L, seed):
    g = np.random.default_rng(seed + 5000).standard_normal((B, H, L, 64), dtype=np.float32)
    return torch.from_numpy(g).to(torch.bfloat16)


def _run_fwd_bwd(q, k, v, do, w, dil, G, pad):
    from sparse_long_sequence_longformer_amd import binding

    qd, kd, vd, dod = to_dev(q, k, v, do)
    padd = None if pad is None else torch.from_numpy(np.ascontiguousarray(pad)).to("cuda")
    out, lse = binding.forward_lse(qd, kd, vd, w, dil, G, padd)
    dq, dk, dv = binding.backward(qd, kd, vd, out, dod, lse, w, dil, G, padd)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu(), dq.cpu(), dk.cpu(), dv.cpu()


def _compare_grad(got, ref, what):
    g = got.to(torch.float64).numpy()
    assert np.all(np.isfinite(g)), f"{what}: non-finite"
    err = np.abs(g - ref)
    scale_max = float(np.abs(ref).max()) if ref.size else 0.0
    scale_mean = float(np.abs(ref).mean()) if ref.size else 0.0
    mx, mean = float(err.max()), float(err.mean())
    log(f"  {what}: max-abs {mx:.3e} (scale {scale_max:.3e}) mean-abs {mean:.3e} (scale {scale_mean:.3e})")
    assert mx <= GRAD_MAX_REL * scale_max + 1e-6, f"{what}: max-abs {mx} > {GRAD_MAX_REL} * {scale_max}"
    assert mean <= GRAD_MEAN_REL * scale_mean + 1e-7, f"{what}: mean-abs {mean} > {GRAD_MEAN_REL} * {scale_mean}"


# (name, B, H, L, w, dil, globals, pad lengths or "rand")
CASES = [
    ("no_globals_300", 1, 2, 300, 16, [1, 1], [], None),
    ("globals_dil", 1, 3, 400, 20, [1, 2, 3], [0, 7, 200, 399], None),
    ("padded", 2, 2, 333, 24, [1, 2], [3, 250], [333, 200]),
    ("rand_pad", 2, 1, 384, 30, [2], [0, 191, 383], "rand"),
    ("many_globals_70", 1, 2, 700, 25, [1, 2], "many70", None),
    ("w_ge_L", 1, 1, 150, 200, [1], [5], None),
    ("w0_globals", 1, 2, 130, 0, [1, 3], [7, 129], None),
    ("tiny_L2", 1, 1, 2, 0, [1], [1], None),
    ("qa_like_1024", 1, 2, 1024, 256, [1, 1], list(range(16)), None),
    ("all_padded_sequence", 2, 1, 100, 5, [1], [3], [100, 0]),
]


def _globals_for(spec, L, seed):
    if isinstance(spec, str) and spec.startswith("many"):
        n = int(spec[4:])
        return sorted(np.random.default_rng(seed).choice(L, n, replace=False).tolist())
    return list(spec)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_full_compare(case):
    name, B, H, L, w, dil, Gs, lens = case
    log(f"case backward {name}: B={B} H={H} L={L} w={w} dil={dil}")
    q, k, v = make_custom(B, H, L, dtype="bf16", seed=len(name))
    do = _dout(B, H, L, len(name))
    G = _globals_for(Gs, L, len(name))
    if lens == "rand":
        pad = (np.random.default_rng(9).random((B, L)) < 0.3).astype(np.uint8)
    else:
        pad = _pad_from_lengths(B, L, lens)
    out, lse, dq, dk, dv = _run_fwd_bwd(q, k, v, do, w, dil, G, pad)
    ref_lse = orc.attention_lse(q, k, w, dil, G, pad)
    lse_np = lse.numpy().astype(np.float64)
    assert np.array_equal(np.isneginf(lse_np), np.isneginf(ref_lse)), f"{name}: -inf rows differ"
    fin = np.isfinite(ref_lse)
    if fin.any():
        e = np.abs(lse_np[fin] - ref_lse[fin]).max()
        log(f"  lse: max-abs {e:.3e}")
        assert e <= 2e-2
    rq, rk, rv = orc.attention_backward(q, k, v, do, w, dil, G, pad)
    _compare_grad(dq, rq, f"{name} dq")
    _compare_grad(dk, rk, f"{name} dk")
    _compare_grad(dv, rv, f"{name} dv")


def test_forward_lse_f32():
    """fp32 forward with its log-sum-exp output."""
    from sparse_long_sequence_longformer_amd import binding

    B, H, L = 2, 2, 500
    q, k, v = make_custom(B, H, L, dtype="f32", seed=41)
    pad = _pad_from_lengths(B, L, [500, 300])
    pad[0, 100:140] = 1
    G = [0, 250, 499]
    qd, kd, vd = to_dev(q, k, v)
    out, lse = binding.forward_lse(qd, kd, vd, 10, [1, 2], G, torch.from_numpy(pad).to("cuda"))
    ref = orc.attention_lse(q, k, 10, [1, 2], G, pad)
    got = lse.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isneginf(got), np.isneginf(ref))
    fin = np.isfinite(ref)
    e = np.abs(got[fin] - ref[fin]).max()
    log(f"  f32 lse max-abs {e:.3e}")
    assert e <= 1e-4
    plain = binding.forward(qd, kd, vd, 10, [1, 2], G, torch.from_numpy(pad).to("cuda"))
    torch.cuda.synchronize()
    assert torch.equal(plain, out)


@pytest.mark.parametrize("row", [0, 7, 150, 299, 205])
def test_backward_sparsity_structure_exact(row):
    """dO nonzero on one row only: dK, dV are exactly zero off that row's key set
    and dQ exactly zero on every other row."""
    B, H, L, w, dil, G = 1, 2, 300, 12, [1, 3], [7, 200]
    pad = np.zeros((B, L), dtype=np.uint8)
    pad[0, [20, 150, 151, 290]] = 1
    q, k, v = make_custom(B, H, L, dtype="bf16", seed=51)
    do = torch.zeros(B, H, L, 64, dtype=torch.bfloat16)
    do[:, :, row] = _dout(B, H, 1, row)[:, :, 0]
    _, _, dq, dk, dv = _run_fwd_bwd(q, k, v, do, w, dil, G, pad)
    for h in range(H):
        keys = set(brute.key_set(row, L, w, dil[h], G, pad[0].astype(bool).tolist()))
        off = np.array([j not in keys for j in range(L)])
        assert torch.all(dk[0, h][torch.from_numpy(off)] == 0), (h, row)
        assert torch.all(dv[0, h][torch.from_numpy(off)] == 0), (h, row)
        on = torch.from_numpy(~off)
        assert bool((dv[0, h][on].abs().amax(dim=1) > 0).all()), (h, row)
        others = torch.ones(L, dtype=torch.bool)
        others[row] = False
        assert torch.all(dq[0, h][others] == 0), (h, row)


def test_backward_deterministic():
    from sparse_long_sequence_longformer_amd import binding

    B, H, L = 1, 4, 2048
    q, k, v = make_custom(B, H, L, dtype="bf16", seed=61)
    do = _dout(B, H, L, 61)
    qd, kd, vd, dod = to_dev(q, k, v, do)
    G = list(range(16))
    out, lse = binding.forward_lse(qd, kd, vd, 512, [1] * H, G)
    a = binding.backward(qd, kd, vd, out, dod, lse, 512, [1] * H, G)
    b = binding.backward(qd, kd, vd, out, dod, lse, 512, [1] * H, G)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("name", ["qa_4k", "dilated_8k"])
def test_backward_workload_slices(name):
    """Full-size workload: every gradient of three (b, h) slices against the oracle."""
    wl = workloads.WORKLOADS[name]
    log(f"case backward workload {name}: {wl.desc}")
    q, k, v = make_qkv(wl)
    do = _dout(wl.B, wl.H, wl.L, 7)
    G = wl.global_positions()
    pad = wl.pad_mask()
    out, lse, dq, dk, dv = _run_fwd_bwd(q, k, v, do, wl.w, wl.dil_list(), G, pad)
    slices = [(0, 0), (wl.B - 1, wl.H - 1), (0, wl.H // 2 + 1)]
    for b, h in slices:
        pr = None if pad is None else pad[b]
        rq, rk, rv = orc.attention_backward_bh(q[b, h], k[b, h], v[b, h], do[b, h], wl.w, wl.dil[h], G, pr)
        _compare_grad(dq[b, h], rq, f"{name} ({b},{h}) dq")
        _compare_grad(dk[b, h], rk, f"{name} ({b},{h}) dk")
        _compare_grad(dv[b, h], rv, f"{name} ({b},{h}) dv")

"""Shared helpers of the GPU parity tests: run the HIP path through the C-ABI binding
and compare with the fp64 oracle on the same seeded inputs."""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from oracle import longformer_oracle as orc
from sparse_long_sequence_longformer_amd import binding

# Tolerances of the forward against the fp64 oracle, over all B*H*L*64 outputs.
TOL_F32_MAX = 1e-4
TOL_BF16_MAX = 2e-2
TOL_BF16_MEAN = 2e-3


def log(msg):
    print(msg, flush=True)


def to_dev(*ts):
    return tuple(t.to("cuda").contiguous() for t in ts)


def run_gpu(q, k, v, w, dil, G, pad):
    """q, k, v: CPU tensors.  pad: numpy uint8 [B, L] or None.  Returns CPU tensor."""
    qd, kd, vd = to_dev(q, k, v)
    padd = None if pad is None else torch.from_numpy(np.ascontiguousarray(pad)).to("cuda")
    out = binding.forward(qd, kd, vd, w, dil, G, padd)
    torch.cuda.synchronize()
    return out.cpu()


def compare(got, ref, dtype, what=""):
    """got: torch CPU tensor (any float dtype); ref: numpy float64.  Returns (max, mean)."""
    g = got.to(torch.float64).numpy()
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - ref)
    mx = float(err.max()) if err.size else 0.0
    mean = float(err.mean()) if err.size else 0.0
    log(f"  {what}: max-abs {mx:.3e} mean-abs {mean:.3e}")
    if dtype == "f32":
        assert mx <= TOL_F32_MAX, f"{what}: max-abs {mx} > {TOL_F32_MAX}"
    else:
        assert mx <= TOL_BF16_MAX, f"{what}: max-abs {mx} > {TOL_BF16_MAX}"
        assert mean <= TOL_BF16_MEAN, f"{what}: mean-abs {mean} > {TOL_BF16_MEAN}"
    return mx, mean


# Gradients (bf16 in and out, fp32 accumulation), per tensor: relative to its scale.
GRAD_MAX_REL = 2e-2
GRAD_MEAN_REL = 1e-2


def compare_grad(got, ref, what):
    """max-abs <= 2e-2 * max|ref| and mean-abs <= 1e-2 * mean|ref|; on a tensor with
    fewer than 16 rows that are not zero by definition each bar is at least the
    forward's absolute bf16 bar (2e-2, 2e-3): the error of such a tensor is a few
    per-row numbers (the rounding of D = dO . O from the stored bf16 output moves a
    row whose dS terms cancel by 1-2 % of their size), not an average."""
    live_rows = int(np.count_nonzero(np.abs(ref).max(axis=-1))) if ref.size else 0
    g = got.to(torch.float64).numpy()
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite"
    err = np.abs(g - ref)
    scale_max = float(np.abs(ref).max()) if ref.size else 0.0
    scale_mean = float(np.abs(ref).mean()) if ref.size else 0.0
    mx = float(err.max()) if err.size else 0.0
    mean = float(err.mean()) if err.size else 0.0
    log(f"  {what}: max-abs {mx:.3e} (scale {scale_max:.3e}) mean-abs {mean:.3e} (scale {scale_mean:.3e})")
    tol_max, tol_mean = GRAD_MAX_REL * scale_max + 1e-6, GRAD_MEAN_REL * scale_mean + 1e-7
    if live_rows < 16:
        tol_max, tol_mean = max(tol_max, TOL_BF16_MAX), max(tol_mean, TOL_BF16_MEAN)
    assert mx <= tol_max, f"{what}: max-abs {mx} > {tol_max}"
    assert mean <= tol_mean, f"{what}: mean-abs {mean} > {tol_mean}"


def full_parity(q, k, v, w, dil, G, pad, dtype, what=""):
    got = run_gpu(q, k, v, w, dil, G, pad)
    ref = orc.attention(q, k, v, w, dil, G, pad)
    compare(got, ref, dtype, what)
    return got, ref


def sample_rows(B, H, L, G, pad, n_random, seed, extra_rows=()):
    """(b, h, i) samples: every global row, sequence ends, tile edges, padding edges,
    plus seeded random rows."""
    rng = np.random.default_rng(seed)
    rows = set()
    edges = [0, 1, 31, 32, 63, 64, 127, 128, 255, 256, L // 2, L - 129, L - 128, L - 2, L - 1, *extra_rows]
    for b in range(B):
        hs = [0, H - 1, int(rng.integers(0, H))]
        for h in hs:
            for i in edges:
                if 0 <= i < L:
                    rows.add((b, h, i))
            for g in G:
                rows.add((b, h, int(g)))
            if pad is not None:
                n = int((pad[b] == 0).sum())
                for i in (n - 2, n - 1, n, n + 1, n + 300):
                    if 0 <= i < L:
                        rows.add((b, h, i))
    for _ in range(n_random):
        rows.add((int(rng.integers(0, B)), int(rng.integers(0, H)), int(rng.integers(0, L))))
    return sorted(rows)


def oracle_threads() -> int:
    """Host threads for the oracle: the CPU share of this process, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_slices(fn, slices):
    """Run fn(b, h) for each (b, h) in ``slices`` on a thread pool with BLAS limited to
    one thread per call (numpy releases the interpreter lock in its array work).
    Returns the results in order."""
    from threadpoolctl import threadpool_limits

    with threadpool_limits(limits=1), ThreadPoolExecutor(oracle_threads()) as ex:
        return list(ex.map(lambda bh: fn(*bh), slices))


def oracle_full(q, k, v, w, dil, G, pad, slices=None, causal=False):
    """orc.attention on the (b, h) slices given (default: all), computed slice by slice
    on a thread pool: float64 [len(slices), L, d] (or [B, H, L, d] when all)."""
    B, H = q.shape[:2]
    padn = None if pad is None else np.asarray(pad) != 0
    every = slices is None
    slices = [(b, h) for b in range(B) for h in range(H)] if every else list(slices)

    def one(b, h):  # widened to float64 slice by slice (inside the oracle)
        return orc.attention_bh(q[b, h], k[b, h], v[b, h], w, dil[h], orc.globals_of(G, b),
                                None if padn is None else padn[b], causal=causal)

    res = oracle_slices(one, slices)
    out = np.stack(res)
    return out.reshape(B, H, *out.shape[1:]) if every else out

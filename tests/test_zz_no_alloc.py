"""The allocation-free forward (lf_attn_forward_static) through the C-ABI, against
lf_attn_forward on the same inputs: two calls in a row on one handle, the second with
a smaller input (the static scratch array keeps the first call's partials), then a
third call whose partials exceed the array, rejected before anything is enqueued.
Same kernels, so the outputs must be bit-identical (and within the bf16 bar of the
oracle on the small case)."""

import ctypes

import numpy as np
import pytest
import torch

from oracle import longformer_oracle as orc
from sparse_long_sequence_longformer_amd import binding
from sparse_long_sequence_longformer_amd.workloads import make_custom
from tests.gpu_common import compare, log, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load_library()
    yield


def _c_call(fn, h, q, k, v, out, w, dil, G, pad):
    B, H, L, d = q.shape
    dil_a = (ctypes.c_int32 * H)(*dil)
    g_a = (ctypes.c_int32 * max(1, len(G)))(*G)
    i32p = ctypes.POINTER(ctypes.c_int32)
    return fn(h.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, L, d, w,
              ctypes.cast(dil_a, i32p), ctypes.cast(g_a, i32p) if G else None, len(G),
              None if pad is None else pad.data_ptr(), torch.cuda.current_stream().cuda_stream)


def test_static_forward_matches_forward_twice():
    lib = binding.load_library()
    h = binding.LfAttn("bf16")
    cases = [
        # (B, H, L, w, dil, globals, padded lengths): the L=4096, w=512 shape, then a smaller one
        (2, 12, 4096, 512, [1] * 12, list(range(16)), None),
        (2, 3, 1000, 64, [1, 2, 3], [0, 5, 999, 400], [1000, 613]),
    ]
    for n, (B, H, L, w, dil, G, lens) in enumerate(cases):
        log(f"case static forward call {n}: B={B} H={H} L={L} w={w} dil={dil} globals={len(G)}")
        q, k, v = make_custom(B, H, L, dtype="bf16", seed=40 + n)
        qd, kd, vd = to_dev(q, k, v)
        pad = None
        padd = None
        if lens is not None:
            pad = (np.arange(L)[None, :] >= np.asarray(lens)[:, None]).astype(np.uint8)
            padd = torch.from_numpy(pad).cuda()
        ref = torch.empty_like(qd)
        got = torch.full_like(qd, float("nan"))
        assert _c_call(lib.lf_attn_forward, h, qd, kd, vd, ref, w, dil, G, padd) == 0
        assert _c_call(lib.lf_attn_forward_static, h, qd, kd, vd, got, w, dil, G, padd) == 0, \
            lib.lf_attn_last_error(h.handle).decode()
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"call {n}: static forward differs from lf_attn_forward"
        if n == 1:
            compare(got.cpu(), orc.attention(q, k, v, w, dil, G, pad), "bf16", "static forward vs oracle")
    h.close()


def test_static_forward_rejects_oversized_partials():
    lib = binding.load_library()
    h = binding.LfAttn("bf16")
    # B=4, H=16, L=32768 with 16 globals: 64 x 256 tiles x 32 queries x 264 bytes > 16 MiB.
    B, H, L = 4, 16, 32768
    qd = torch.zeros((B, H, L, 64), dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(qd, 3.0)
    st = _c_call(lib.lf_attn_forward_static, h, qd, qd, qd, out, 256, [1] * H, list(range(16)), None)
    msg = lib.lf_attn_last_error(h.handle).decode()
    log(f"  oversized: status {st}: {msg}")
    assert st == 2 and "allocation-free" in msg
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)  # nothing was enqueued
    h.close()

"""Failure paths forced from the host (LF_ATTN_FAULT, read when a handle is created):
a failed workspace allocation returns LF_ERR_OOM and a failed launch LF_ERR_HIP, both
before anything is enqueued, so the output buffer keeps its contents; the same handle
then completes the next call, and its result matches the oracle."""

import os

import numpy as np
import pytest
import torch

from oracle import longformer_oracle as orc
from sparse_long_sequence_longformer_amd import binding
from sparse_long_sequence_longformer_amd.workloads import make_custom
from tests.gpu_common import compare, log, to_dev

pytestmark = pytest.mark.gpu

LF_ERR_HIP, LF_ERR_OOM = 3, 4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load_library()
    yield


def _handle_with_fault(kind):
    old = os.environ.get("LF_ATTN_FAULT")
    os.environ["LF_ATTN_FAULT"] = kind
    try:
        return binding.LfAttn("bf16")
    finally:
        if old is None:
            del os.environ["LF_ATTN_FAULT"]
        else:
            os.environ["LF_ATTN_FAULT"] = old


@pytest.mark.parametrize("kind,code", [("alloc", LF_ERR_OOM), ("launch", LF_ERR_HIP)])
def test_fault_then_recovery(kind, code):
    B, H, L, w, dil, G = 2, 2, 500, 40, [1, 2], [0, 7, 300]
    log(f"case fault {kind}: B={B} H={H} L={L} w={w}")
    q, k, v = make_custom(B, H, L, dtype="bf16", seed=70)
    qd, kd, vd = to_dev(q, k, v)
    h = _handle_with_fault(kind)
    out = torch.full_like(qd, 5.0)
    with pytest.raises(binding.LfAttnError) as err:
        binding.forward(qd, kd, vd, w, dil, G, out=out, handle=h)
    assert err.value.status == code, err.value
    assert f"LF_ATTN_FAULT={kind}" in str(err.value)
    torch.cuda.synchronize()
    assert torch.all(out == 5.0), "output touched by a call that failed before enqueueing"
    # the same handle completes the next call
    binding.forward(qd, kd, vd, w, dil, G, out=out, handle=h)
    torch.cuda.synchronize()
    compare(out.cpu(), orc.attention(q, k, v, w, dil, G), "bf16", f"after {kind} fault")
    h.close()

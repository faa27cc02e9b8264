"""The forward and backward captured in a HIP graph (torch.cuda.CUDAGraph over the
library's launches) and replayed: every replay equals the eager result bit for bit,
with eager work and synchronisations between the replays.  The handle's workspace
is allocated by an eager call first (capture cannot allocate)."""

import numpy as np
import pytest
import torch

from sparse_long_sequence_longformer_amd import workloads
from sparse_long_sequence_longformer_amd.workloads import make_custom

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_long_sequence_longformer_amd import binding

    binding.load_library()
    yield


def test_forward_graph_replays():
    from sparse_long_sequence_longformer_amd import binding

    wl = workloads.WORKLOADS["qa_4k"]
    q, k, v = (t.cuda() for t in workloads.make_qkv(wl))
    h = binding.LfAttn("bf16")
    G = wl.global_positions()
    out = torch.empty_like(q)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        binding.forward(q, k, v, wl.w, wl.dil_list(), G, out=out, handle=h)  # allocates the workspace
    s.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        binding.forward(q, k, v, wl.w, wl.dil_list(), G, out=out, handle=h)
    for r in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r}"
        _ = (q.float() * 2).sum().item()  # eager work between replays


def test_backward_graph_replays():
    from sparse_long_sequence_longformer_amd import binding

    B, H, L = 1, 4, 1024
    q, k, v = (t.cuda() for t in make_custom(B, H, L, dtype="bf16", seed=5))
    do = torch.from_numpy(np.random.default_rng(1).standard_normal((B, H, L, 64), dtype=np.float32)).bfloat16().cuda()
    h = binding.LfAttn("bf16")
    G = list(range(8))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out, lse = binding.forward_lse(q, k, v, 128, [1] * H, G, handle=h)
        dq, dk, dv = binding.backward(q, k, v, out, do, lse, 128, [1] * H, G, handle=h)
    s.synchronize()
    ref = [t.clone() for t in (out, lse, dq, dk, dv)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        binding.forward_lse(q, k, v, 128, [1] * H, G, out=out, lse=lse, handle=h)
        binding.backward(q, k, v, out, do, lse, 128, [1] * H, G, dq=dq, dk=dk, dv=dv, handle=h)
    for r in range(3):
        for t in (out, dq, dk, dv):
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((out, lse, dq, dk, dv), ref):
            assert torch.equal(a, b), f"replay {r}"


def test_variant_graph_replays():
    """Causal mode, a bias table and random blocks set on the handle: after one eager call
    (workspaces allocated, draws uploaded) the forward and backward capture and replay
    bit for bit."""
    from sparse_long_sequence_longformer_amd import binding

    B, H, L, w = 1, 2, 1024, 96
    q, k, v = (t.cuda() for t in make_custom(B, H, L, dtype="bf16", seed=6))
    do = torch.from_numpy(np.random.default_rng(2).standard_normal((B, H, L, 64), dtype=np.float32)).bfloat16().cuda()
    h = binding.LfAttn("bf16")
    h.set_causal(True)
    h.set_position_bias(torch.from_numpy(workloads.make_bias(H, w, seed=3)).cuda())
    h.set_random_blocks(workloads.make_random_blocks(H, L, 2, seed=4))
    G = [0, 500]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out, lse = binding.forward_lse(q, k, v, w, [1] * H, G, handle=h, causal=True)
        dq, dk, dv = binding.backward(q, k, v, out, do, lse, w, [1] * H, G, handle=h, causal=True)
    s.synchronize()
    ref = [t.clone() for t in (out, lse, dq, dk, dv)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        binding.forward_lse(q, k, v, w, [1] * H, G, out=out, lse=lse, handle=h, causal=True)
        binding.backward(q, k, v, out, do, lse, w, [1] * H, G, dq=dq, dk=dk, dv=dv, handle=h, causal=True)
    for r in range(3):
        for t in (out, dq, dk, dv):
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((out, lse, dq, dk, dv), ref):
            assert torch.equal(a, b), f"replay {r}"
        _ = (q.float() * 2).sum().item()  # eager work between replays
    h.close()

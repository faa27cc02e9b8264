"""Whole-tensor parity at full size, and the band-mask refill of padded windows wider
than 64 stages, against the fp64 oracle (computed slice by slice on host threads).

* The L=4096 (w=256 and w=512) and L=8192 dilated workloads: every output element.
* The padded L=32768 workload: every row of the (b, h) slices (0, 0), (1, 5), (2, 10)
  and (3, 15), one head of each true length 32768, 20000, 9000 and 4096.
* Padding with w = 2100: a tile's window band spans more than 64 stages of 64 keys,
  so the kernels rebuild the invalid-key bits of their band stages in a second round
  (forward fp32 and bf16, backward bf16).

Bars: fp32 max-abs 1e-4; bf16 max-abs 2e-2 and mean-abs 2e-3 over every compared
element; gradients max-abs 2e-2 max|ref| and mean-abs 1e-2 mean|ref| per tensor.
"""

import numpy as np
import pytest
import torch

from oracle import longformer_oracle as orc
from sparse_long_sequence_longformer_amd import workloads
from sparse_long_sequence_longformer_amd.workloads import make_custom, make_qkv
from tests.gpu_common import compare, compare_grad, log, oracle_full, oracle_slices, run_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_long_sequence_longformer_amd import binding

    binding.load_library()
    yield


@pytest.mark.parametrize("name", ["cls_4k", "qa_4k", "dilated_8k"])
def test_workload_whole_tensor(name):
    wl = workloads.WORKLOADS[name]
    log(f"case workload whole tensor {name}: {wl.desc}")
    q, k, v = make_qkv(wl)
    G, pad = wl.global_positions(), wl.pad_mask()
    got = run_gpu(q, k, v, wl.w, wl.dil_list(), G, pad)
    ref = oracle_full(q, k, v, wl.w, wl.dil_list(), G, pad)
    compare(got, ref, "bf16", f"{name} (all {got.numel()} outputs)")


PADDED_SLICES = [(0, 0), (1, 5), (2, 10), (3, 15)]


def test_padded_32k_whole_slices():
    wl = workloads.WORKLOADS["padded_32k"]
    log(f"case padded_32k whole slices {PADDED_SLICES}: {wl.desc}")
    q, k, v = make_qkv(wl)
    G, pad = wl.global_positions(), wl.pad_mask()
    got = run_gpu(q, k, v, wl.w, wl.dil_list(), G, pad)
    ref = oracle_full(q, k, v, wl.w, wl.dil_list(), G, pad, slices=PADDED_SLICES)
    sel = torch.stack([got[b, h] for b, h in PADDED_SLICES])
    compare(sel, ref, "bf16", f"padded_32k slices {PADDED_SLICES}")


# Padding with a window band of more than 64 stages (head 0: 128 + 2*2100 keys, 68
# stages; head 1 with dilation 2 stays within 64).
REFILL_B, REFILL_H, REFILL_L, REFILL_W = 2, 2, 8192, 2100
REFILL_DIL = [1, 2]
REFILL_G = [0, 4000, 4001, 8191]


def _refill_pad():
    pad = np.zeros((REFILL_B, REFILL_L), dtype=np.uint8)
    pad[0, 7000:] = 1
    pad[1] = np.random.default_rng(17).random(REFILL_L) < 0.2
    pad[1, 6000:] = 1
    pad[1, 4000] = 0  # one global key unpadded, the other (4001) maybe padded
    return pad


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_refill_forward(dtype):
    """Both forward tilings (64-row split work-groups, which the library picks for this
    grid, and 128-row ones) against one oracle result."""
    from sparse_long_sequence_longformer_amd import binding

    log(f"case refill forward {dtype}: B={REFILL_B} H={REFILL_H} L={REFILL_L} w={REFILL_W} dil={REFILL_DIL}")
    q, k, v = make_custom(REFILL_B, REFILL_H, REFILL_L, dtype=dtype, seed=31)
    pad = _refill_pad()
    ref = oracle_full(q, k, v, REFILL_W, REFILL_DIL, REFILL_G, pad)
    qd, kd, vd = to_dev(q, k, v)
    padd = torch.from_numpy(pad).to("cuda")
    for rows in (64, 128):
        h = binding.LfAttn(dtype)
        h.set_tile_rows(rows)
        got = binding.forward(qd, kd, vd, REFILL_W, REFILL_DIL, REFILL_G, padd, handle=h)
        torch.cuda.synchronize()
        compare(got.cpu(), ref, dtype, f"refill forward {dtype} rows={rows}")


def test_refill_backward():
    from sparse_long_sequence_longformer_amd import binding

    log(f"case refill backward bf16: B={REFILL_B} H={REFILL_H} L={REFILL_L} w={REFILL_W} dil={REFILL_DIL}")
    q, k, v = make_custom(REFILL_B, REFILL_H, REFILL_L, dtype="bf16", seed=32)
    g = np.random.default_rng(33).standard_normal((REFILL_B, REFILL_H, REFILL_L, 64), dtype=np.float32)
    do = torch.from_numpy(g).to(torch.bfloat16)
    pad = _refill_pad()
    qd, kd, vd, dod = to_dev(q, k, v, do)
    padd = torch.from_numpy(pad).to("cuda")
    out, lse = binding.forward_lse(qd, kd, vd, REFILL_W, REFILL_DIL, REFILL_G, padd)
    grads = binding.backward(qd, kd, vd, out, dod, lse, REFILL_W, REFILL_DIL, REFILL_G, padd)
    torch.cuda.synchronize()
    padb = pad != 0

    def one(b, h):
        return orc.attention_backward_bh(q[b, h], k[b, h], v[b, h], do[b, h], REFILL_W, REFILL_DIL[h], REFILL_G,
                                         padb[b])

    slices = [(b, h) for b in range(REFILL_B) for h in range(REFILL_H)]
    res = oracle_slices(one, slices)
    for n, name in enumerate(("dq", "dk", "dv")):
        ref = np.stack([r[n] for r in res]).reshape(REFILL_B, REFILL_H, REFILL_L, 64)
        compare_grad(grads[n].cpu(), ref, f"refill backward {name}")

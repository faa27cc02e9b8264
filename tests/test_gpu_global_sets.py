"""Per-sequence global sets (LF_GLOBALS_PER_SEQUENCE): every entry point against the
fp64 oracle with one global row per sequence (negative entries unused).  Same
tolerances as the shared-set tests."""

import numpy as np
import pytest
import torch

from oracle import layer_oracle as lo
from oracle import longformer_oracle as orc
from sparse_long_sequence_longformer_amd.workloads import make_custom
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


def _pad(B, L, lens):
    return None if lens is None else (np.arange(L)[None, :] >= np.asarray(lens)[:, None]).astype(np.uint8)


def _padd(pad):
    return None if pad is None else torch.from_numpy(pad).to("cuda")


def _sets(rows):
    n = max(len(r) for r in rows)
    return np.array([list(r) + [-1] * (n - len(r)) for r in rows], dtype=np.int64)


# (name, dtype, H, L, w, dil, per-sequence rows, pad lengths, causal)
CASES = [
    ("f32_three_rows", "f32", 2, 300, 12, [1, 2], [[0, 150], [7, 7, 299], []], [300, 250, 120], False),
    ("f32_many_in_one_row", "f32", 1, 600, 8, [1], [list(range(0, 600, 9)), [5]], None, False),
    ("f32_causal", "f32", 2, 400, 20, [1, 3], [[3, 200, 399], [100]], None, True),
    ("bf16_question_spans", "bf16", 4, 2048, 256, [1] * 4, [list(range(16)), list(range(40)), list(range(3))],
     [2048, 1500, 2048], False),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_global_sets_forward(case):
    from sparse_long_sequence_longformer_amd import binding

    name, dtype, H, L, w, dil, rows, lens, causal = case
    B = len(rows)
    log(f"case per-sequence globals {name}: B={B} H={H} L={L} w={w} counts={[len(r) for r in rows]}")
    q, k, v = make_custom(B, H, L, dtype=dtype, seed=len(name) + 300)
    pad = _pad(B, L, lens)
    qd, kd, vd = to_dev(q, k, v)
    out, lse = binding.forward_lse(qd, kd, vd, w, dil, rows, _padd(pad), causal=causal)
    torch.cuda.synchronize()
    sets = _sets(rows)
    compare(out.cpu(), orc.attention(q, k, v, w, dil, sets, pad, causal=causal), dtype, name)
    ref = orc.attention_lse(q, k, w, dil, sets, pad, causal=causal)
    got = lse.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isneginf(got), np.isneginf(ref))
    fin = np.isfinite(ref)
    assert np.abs(got[fin] - ref[fin]).max() <= (1e-4 if dtype == "f32" else 2e-2)


def test_global_sets_match_shared_when_rows_agree():
    from sparse_long_sequence_longformer_amd import binding

    B, H, L = 2, 2, 500
    q, k, v = make_custom(B, H, L, dtype="bf16", seed=77)
    qd, kd, vd = to_dev(q, k, v)
    a = binding.forward(qd, kd, vd, 30, [1, 2], [4, 90, 91])
    b = binding.forward(qd, kd, vd, 30, [1, 2], [[91, 4, 90], [90, 91, 4, -1]])
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("causal", [False, True])
def test_global_sets_backward(causal):
    from sparse_long_sequence_longformer_amd import binding

    rows = [[0, 9, 200], list(range(100, 145)), []]
    B, H, L, w, dil = 3, 2, 400, 20, [1, 2]
    q, k, v = make_custom(B, H, L, dtype="bf16", seed=88)
    do = _dout(B, H, L, 88)
    pad = _pad(B, L, [400, 330, 400])
    qd, kd, vd, dod = to_dev(q, k, v, do)
    out, lse = binding.forward_lse(qd, kd, vd, w, dil, rows, _padd(pad), causal=causal)
    dq, dk, dv = binding.backward(qd, kd, vd, out, dod, lse, w, dil, rows, _padd(pad), causal=causal)
    torch.cuda.synchronize()
    rq, rk, rv = orc.attention_backward(q, k, v, do, w, dil, _sets(rows), pad, causal=causal)
    _compare_grad(dq.cpu(), rq, f"per-sequence dq causal={causal}")
    _compare_grad(dk.cpu(), rk, f"per-sequence dk causal={causal}")
    _compare_grad(dv.cpu(), rv, f"per-sequence dv causal={causal}")


def test_global_sets_layer():
    from sparse_long_sequence_longformer_amd import binding
    from tests.test_gpu_layer import TOL_MAX, TOL_MEAN, _weights

    B, L, E, F, w = 2, 300, 128, 256, 16
    rows = [[0, 5], list(range(40))]
    x = torch.from_numpy(np.random.default_rng(3).standard_normal((B, L, E), dtype=np.float32)).bfloat16()
    W = _weights(E, F, 4)
    out = binding.layer_forward(x.cuda(), {kk: vv.cuda() for kk, vv in W.items()}, w, [1, 2], rows)
    torch.cuda.synchronize()
    ref = lo.layer_forward(x, W, E // 64, w, [1, 2], _sets(rows), None)
    err = np.abs(out.cpu().double().numpy() - ref)
    log(f"  per-sequence layer: max-abs {err.max():.3e} mean-abs {err.mean():.3e}")
    assert err.max() <= TOL_MAX and err.mean() <= TOL_MEAN


def test_global_sets_qa_workload_sampled():
    """B=2, L=4096, w=512 with question spans of 16 and 48 tokens: sampled rows."""
    from sparse_long_sequence_longformer_amd import binding
    from sparse_long_sequence_longformer_amd import workloads

    wl = workloads.WORKLOADS["qa_4k"]
    q, k, v = workloads.make_qkv(wl)
    rows = [list(range(16)), list(range(48))]
    qd, kd, vd = to_dev(q, k, v)
    out = binding.forward(qd, kd, vd, wl.w, wl.dil_list(), rows).cpu()
    samples = sample_rows(wl.B, wl.H, wl.L, list(range(48)), None, n_random=32, seed=9)
    ref = orc.attention_sampled(q, k, v, wl.w, wl.dil_list(), _sets(rows), None, samples)
    compare(torch.stack([out[b, h, i] for b, h, i in samples]), ref, "bf16",
            f"per-sequence qa_4k ({len(samples)} sampled rows)")

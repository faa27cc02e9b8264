"""Both forward tilings against the fp64 oracle, forced on one handle each through
lf_attn_set_tile_rows: 128-row work-groups (four waves of 32 rows) and the 64-row
split form (two waves per 32 rows, each taking every other 32-key sub-tile of a
stage, their partial softmax states merged before the store).  Left to itself the
library picks the split form for grids that fill at most half of the GPU, i.e. for
most small shapes of the other tests; here each form runs the whole fp32 battery
(max-abs 1e-4), the bf16 cases (2e-2 / 2e-3), the one-sided variant, per-sequence
global sets and the log-sum-exp output, and the automatic choice is checked to be
bit-identical to the form it should pick.
"""

import numpy as np
import pytest
import torch

from oracle import longformer_oracle as orc
from sparse_long_sequence_longformer_amd import workloads
from sparse_long_sequence_longformer_amd.workloads import make_custom, make_qkv
from tests.gpu_common import compare, log, to_dev
from tests.test_gpu_parity import BF16_CASES, F32_CASES, _globals_for, _pad_from_lengths

pytestmark = pytest.mark.gpu

_handles = {}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_long_sequence_longformer_amd import binding

    binding.load_library()  # fail loudly if the HIP library is missing
    yield
    _handles.clear()


def _handle(dtype, rows, causal=False, per_seq=False):
    from sparse_long_sequence_longformer_amd import binding

    key = (dtype, rows, causal, per_seq)
    if key not in _handles:
        h = binding.LfAttn(dtype)
        h.set_tile_rows(rows)
        if causal:
            h.set_causal(True)
        if per_seq:
            h.set_per_sequence_globals(True)
        _handles[key] = h
    return _handles[key]


def _padd(pad):
    return None if pad is None else torch.from_numpy(np.ascontiguousarray(pad)).to("cuda")


def _run(q, k, v, w, dil, G, pad, dtype, rows, causal=False, per_seq=False):
    from sparse_long_sequence_longformer_amd import binding

    qd, kd, vd = to_dev(q, k, v)
    out = binding.forward(qd, kd, vd, w, dil, G, _padd(pad), handle=_handle(dtype, rows, causal, per_seq),
                          causal=causal)
    torch.cuda.synchronize()
    return out.cpu()


@pytest.mark.parametrize("rows", [64, 128])
@pytest.mark.parametrize("case", F32_CASES, ids=[c[0] for c in F32_CASES])
def test_f32_battery_both_tilings(case, rows):
    name, B, H, L, w, dil, Gs, lens, gscale = case
    log(f"case f32 {name} rows={rows}: B={B} H={H} L={L} w={w} dil={dil}")
    q, k, v = make_custom(B, H, L, dtype="f32", seed=len(name))
    G = _globals_for(Gs, L, len(name))
    if gscale != 1.0 and G:
        k[:, :, G] *= gscale
    pad = (np.random.default_rng(7).random((B, L)) < 0.3).astype(np.uint8) if lens == "rand" \
        else _pad_from_lengths(B, L, lens)
    got = _run(q, k, v, w, dil, G, pad, "f32", rows)
    compare(got, orc.attention(q, k, v, w, dil, G, pad), "f32", f"{name} rows={rows}")


@pytest.mark.parametrize("rows", [64, 128])
@pytest.mark.parametrize("case", BF16_CASES, ids=[c[0] for c in BF16_CASES])
def test_bf16_both_tilings(case, rows):
    name, B, H, L, w, dil, G, lens = case
    log(f"case bf16 {name} rows={rows}: B={B} H={H} L={L} w={w} dil={dil}")
    q, k, v = make_custom(B, H, L, dtype="bf16", seed=11)
    pad = _pad_from_lengths(B, L, lens)
    got = _run(q, k, v, w, dil, G, pad, "bf16", rows)
    compare(got, orc.attention(q, k, v, w, dil, G, pad), "bf16", f"{name} rows={rows}")


# (name, dtype, B, H, L, w, dil, globals, pad)
CAUSAL_CASES = [
    ("f32_mixed", "f32", 2, 3, 700, 70, [1, 2, 3], [0, 5, 350, 699], "rand"),
    ("f32_wide", "f32", 1, 2, 520, 300, [1, 1], [17, 400], None),
    ("bf16_1500", "bf16", 2, 2, 1500, 256, [1, 2], [0, 1, 2, 800], [1500, 1100]),
]


@pytest.mark.parametrize("rows", [64, 128])
@pytest.mark.parametrize("case", CAUSAL_CASES, ids=[c[0] for c in CAUSAL_CASES])
def test_causal_and_lse_both_tilings(case, rows):
    from sparse_long_sequence_longformer_amd import binding

    name, dtype, B, H, L, w, dil, G, lens = case
    log(f"case causal {name} rows={rows}: B={B} H={H} L={L} w={w} dil={dil}")
    q, k, v = make_custom(B, H, L, dtype=dtype, seed=len(name) + 40)
    pad = (np.random.default_rng(3).random((B, L)) < 0.25).astype(np.uint8) if lens == "rand" \
        else _pad_from_lengths(B, L, lens)
    qd, kd, vd = to_dev(q, k, v)
    h = _handle(dtype, rows, causal=True)
    out, lse = binding.forward_lse(qd, kd, vd, w, dil, G, _padd(pad), handle=h, causal=True)
    torch.cuda.synchronize()
    compare(out.cpu(), orc.attention(q, k, v, w, dil, G, pad, causal=True), dtype, f"{name} rows={rows}")
    ref = orc.attention_lse(q, k, w, dil, G, pad, causal=True)
    got = lse.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isneginf(got), np.isneginf(ref))
    fin = np.isfinite(ref)
    err = float(np.abs(got[fin] - ref[fin]).max()) if fin.any() else 0.0
    log(f"  lse max-abs {err:.3e}")
    assert err <= (1e-4 if dtype == "f32" else 2e-2)


@pytest.mark.parametrize("rows", [64, 128])
def test_per_sequence_globals_both_tilings(rows):
    B, H, L, w = 3, 2, 900, 60
    dil = [1, 2]
    rows_g = [[0, 1, 2, 450], [899, -1, -1, -1], [-1, -1, 300, 301]]  # negative: unused
    q, k, v = make_custom(B, H, L, dtype="f32", seed=77)
    pad = _pad_from_lengths(B, L, [900, 620, 333])
    got = _run(q, k, v, w, dil, rows_g, pad, "f32", rows, per_seq=True)
    compare(got, orc.attention(q, k, v, w, dil, rows_g, pad), "f32", f"per-sequence globals rows={rows}")


@pytest.mark.parametrize("name,expect", [("cls_4k", 64), ("qa_4k", 128)])
def test_automatic_choice(name, expect):
    """cls_4k's 384 work-groups of 128 rows fill half of the 768 slots: split form;
    qa_4k's 768 fill them all: 128 rows.  The automatic result is bit-identical to the
    forced one (same kernel, same inputs)."""
    from sparse_long_sequence_longformer_amd import binding

    wl = workloads.WORKLOADS[name]
    qd, kd, vd = to_dev(*make_qkv(wl))
    G = wl.global_positions()
    auto = binding.forward(qd, kd, vd, wl.w, wl.dil_list(), G)
    forced = binding.forward(qd, kd, vd, wl.w, wl.dil_list(), G, handle=_handle("bf16", expect))
    other = binding.forward(qd, kd, vd, wl.w, wl.dil_list(), G, handle=_handle("bf16", 192 - expect))
    torch.cuda.synchronize()
    assert torch.equal(auto, forced)
    assert not torch.equal(auto, other)  # the two forms round differently somewhere

"""Separate global projections (``lf_attn_forward_global_proj``) against the fp64
oracle ``attention_global_proj`` on seeded inputs, plus properties that tie the
variant to the single-projection forward.  Same tolerances as the forward:
fp32 max-abs 1e-4; bf16 max-abs 2e-2 and mean-abs 2e-3."""

import numpy as np
import pytest
import torch

from oracle import longformer_oracle as orc
from sparse_long_sequence_longformer_amd import workloads
from sparse_long_sequence_longformer_amd.workloads import make_custom, make_global_proj, make_qkv
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


def _run(q, k, v, qg, kg, vg, w, dil, G, pad):
    from sparse_long_sequence_longformer_amd import binding

    dev = to_dev(q, k, v, qg, kg, vg)
    padd = None if pad is None else torch.from_numpy(np.ascontiguousarray(pad)).to("cuda")
    out = binding.forward_global_proj(*dev, w, dil, G, padd)
    torch.cuda.synchronize()
    return out.cpu()


def _inputs(B, H, L, dtype, seed):
    q, k, v = make_custom(B, H, L, dtype=dtype, seed=seed)
    qg, kg, vg = make_custom(B, H, L, dtype=dtype, seed=seed + 1000)
    return q, k, v, qg, kg, vg


# (name, dtype, B, H, L, w, dil, globals, pad lengths or "rand")
CASES = [
    ("f32_basic", "f32", 1, 2, 300, 12, [1, 2], [0, 150, 299], None),
    ("f32_padded", "f32", 2, 2, 400, 20, [1, 3], [3, 250, 399], [400, 260]),
    ("f32_rand_pad", "f32", 2, 1, 384, 30, [2], [0, 191, 383], "rand"),
    ("f32_many_globals_70", "f32", 1, 2, 700, 25, [1, 2], "many70", None),
    ("f32_max_globals_256", "f32", 1, 1, 600, 8, [1], "many256", [450]),
    ("f32_tiny_L2", "f32", 1, 1, 2, 0, [1], [1], None),
    ("f32_no_globals", "f32", 1, 1, 200, 10, [1], [], None),
    ("bf16_qa_like_2048", "bf16", 1, 4, 2048, 512, [1] * 4, list(range(16)), None),
    ("bf16_mixed_1000", "bf16", 2, 3, 1000, 40, [1, 2, 3], [0, 5, 500, 999], [1000, 777]),
    ("bf16_many_globals_90", "bf16", 1, 2, 1300, 64, [1, 2], "many90", [1300]),
]


def _globals_for(spec, L, seed):
    if isinstance(spec, str) and spec.startswith("many"):
        n = int(spec[4:])
        return sorted(np.random.default_rng(seed).choice(L, n, replace=False).tolist())
    return list(spec)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_global_proj_full_compare(case):
    name, dtype, B, H, L, w, dil, Gs, lens = case
    log(f"case global_proj {name}: B={B} H={H} L={L} w={w} dil={dil}")
    q, k, v, qg, kg, vg = _inputs(B, H, L, dtype, seed=len(name))
    G = _globals_for(Gs, L, len(name))
    if lens == "rand":
        pad = (np.random.default_rng(9).random((B, L)) < 0.3).astype(np.uint8)
    else:
        pad = _pad_from_lengths(B, L, lens)
    got = _run(q, k, v, qg, kg, vg, w, dil, G, pad)
    ref = orc.attention_global_proj(q, k, v, qg, kg, vg, w, dil, G, pad)
    compare(got, ref, dtype, name)


def test_global_proj_same_tensors_equal_forward():
    """q_g = q, k_g = k, v_g = v reproduces lf_attn_forward bit for bit."""
    from sparse_long_sequence_longformer_amd import binding

    B, H, L = 2, 2, 900
    q, k, v = make_custom(B, H, L, dtype="bf16", seed=31)
    pad = _pad_from_lengths(B, L, [900, 500])
    qd, kd, vd = to_dev(q, k, v)
    padd = torch.from_numpy(pad).to("cuda")
    G = [0, 7, 450, 899] + list(range(100, 140))  # two 32-query blocks of globals
    a = binding.forward(qd, kd, vd, 60, [1, 2], G, padd)
    b = binding.forward_global_proj(qd, kd, vd, qd, kd, vd, 60, [1, 2], G, padd)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("name", ["qa_4k", "padded_32k"])
def test_global_proj_workload(name):
    """Full-size workload: global rows against the oracle row by row, every other row
    bit-identical to the single-projection forward (it never reads q_g, k_g, v_g)."""
    from sparse_long_sequence_longformer_amd import binding

    wl = workloads.WORKLOADS[name]
    log(f"case global_proj workload {name}: {wl.desc}")
    q, k, v = make_qkv(wl)
    qg, kg, vg = make_global_proj(wl)
    G = wl.global_positions()
    pad = wl.pad_mask()
    qd, kd, vd, qgd, kgd, vgd = to_dev(q, k, v, qg, kg, vg)
    padd = None if pad is None else torch.from_numpy(pad).to("cuda")
    got = binding.forward_global_proj(qd, kd, vd, qgd, kgd, vgd, wl.w, wl.dil_list(), G, padd)
    base = binding.forward(qd, kd, vd, wl.w, wl.dil_list(), G, padd)
    torch.cuda.synchronize()
    is_g = torch.zeros(wl.L, dtype=torch.bool, device="cuda")
    is_g[G] = True
    assert torch.equal(got[:, :, ~is_g], base[:, :, ~is_g])
    del base
    got = got.cpu()
    heads = range(wl.H) if wl.L <= 4096 else (0, 7, wl.H - 1)
    samples = [(b, h, g) for b in range(wl.B) for h in heads for g in G]
    samples += [s for s in sample_rows(wl.B, wl.H, wl.L, [], pad, n_random=16, seed=6)][:24]
    ref = orc.attention_global_proj_sampled(q, k, v, qg, kg, vg, wl.w, wl.dil_list(), G, pad, samples)
    sel = torch.stack([got[b, h, i] for b, h, i in samples])
    compare(sel, ref, "bf16", f"{name} global projections ({len(samples)} sampled rows)")

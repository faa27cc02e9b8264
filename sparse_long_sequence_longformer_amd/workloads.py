"""Seeded synthetic workloads for the Longformer attention forward.

This module only draws inputs; it holds none of the attention arithmetic, so
both the HIP path and the fp64 oracle can take their inputs from it.

Recipe (fixed, shared by every consumer):
  1. rng = numpy.random.default_rng(seed) with seed 0;
  2. q, k, v drawn in that order as float32 standard normals of shape
     (B, H, L, 64); optionally scaled (0.5 for the CLS workload);
  3. bf16 workloads are rounded to bfloat16 by torch (round to nearest even);
  4. random global positions use numpy.random.default_rng(1).choice(L, n, replace=False), sorted;
  5. the key padding mask is pad[b, j] = (j >= length[b]) (uint8, 1 = padded);
  6. separate global projections q_g, k_g, v_g (when used) follow steps 1-3 with
     seed + 1000.
  7. a relative-position-bias table (when used) is [H, 2w + 1] float32 standard
     normals times a scale, from numpy.random.default_rng(seed + 7919).
  8. random key blocks (when used) are [H, ceil(L / 64), r] int32: for every head
     and query block, r distinct key blocks drawn uniformly from all of them by
     numpy.random.default_rng(seed + 104729).choice(n_blocks, r, replace=False).

The five shapes follow the pages' workloads: hidden size 768 = 12 heads x 64
(page "基于Block-Sparse Attention的Longformer" §6 example model), 4096-token
documents and windows of 512 per side (page "基于自注意力机制的长文本建模算法：
Longformer详解" §2, §9), a CLS-like single global token and a question-span of
global tokens (same page §2 and §7), and 8-16 global tokens with windows of
L/8..L/4 (page "Efficient Transformers: A Survey" commentary, §3.3).
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    L: int
    w: int
    dil: tuple
    dtype: str  # "f32" or "bf16"
    globals_: tuple = ()
    random_globals: int = 0  # if > 0, draw this many distinct positions with seed 1
    lengths: tuple = ()  # true lengths per sequence (empty: no padding)
    scale: float = 1.0
    seed: int = 0
    d: int = 64
    desc: str = field(default="", compare=False)

    def global_positions(self) -> list[int]:
        if self.random_globals:
            g = np.random.default_rng(1).choice(self.L, self.random_globals, replace=False)
            return sorted(int(x) for x in g)
        return list(self.globals_)

    def pad_mask(self):
        """uint8 [B, L] (1 = padded key) or None when every sequence is full."""
        if not self.lengths:
            return None
        j = np.arange(self.L)[None, :]
        lens = np.asarray(self.lengths)[:, None]
        return (j >= lens).astype(np.uint8)

    def dil_list(self) -> list[int]:
        return list(self.dil)


WORKLOADS = {
    "tiny_f32": Workload(
        "tiny_f32", B=1, H=1, L=256, w=32, dil=(1,), dtype="f32",
        desc="B=1 H=1 L=256 d=64 w=32 dil=1, no globals, no padding, fp32"),
    "cls_4k": Workload(
        "cls_4k", B=1, H=12, L=4096, w=256, dil=(1,) * 12, dtype="bf16", globals_=(0,), scale=0.5,
        desc="B=1 H=12 L=4096 d=64 w=256 dil=1, global {0}, bf16 0.5*N(0,1)"),
    "qa_4k": Workload(
        "qa_4k", B=2, H=12, L=4096, w=512, dil=(1,) * 12, dtype="bf16", globals_=tuple(range(16)),
        desc="B=2 H=12 L=4096 d=64 w=512 dil=1, globals 0..15, bf16 N(0,1)"),
    "dilated_8k": Workload(
        "dilated_8k", B=1, H=12, L=8192, w=128, dil=(1,) * 6 + (2,) * 6, dtype="bf16",
        random_globals=8,
        desc="B=1 H=12 L=8192 d=64 w=128 dil 1 (heads 0-5) / 2 (heads 6-11), 8 random globals, bf16"),
    "padded_32k": Workload(
        "padded_32k", B=4, H=16, L=32768, w=256, dil=(1,) * 16, dtype="bf16",
        globals_=tuple(range(16)), lengths=(32768, 20000, 9000, 4096),
        desc="B=4 H=16 L=32768 d=64 w=256 dil=1, globals 0..15, lengths 32768/20000/9000/4096, bf16"),
}

# The workload the throughput metric is quoted on (L=4096, w=512).
HEADLINE = "qa_4k"


def make_qkv(wl: Workload):
    """Return (q, k, v) as CPU torch tensors of the workload's dtype."""
    import torch

    rng = np.random.default_rng(wl.seed)
    shape = (wl.B, wl.H, wl.L, wl.d)
    arrs = []
    for _ in range(3):
        a = rng.standard_normal(shape, dtype=np.float32)
        if wl.scale != 1.0:
            a = a * np.float32(wl.scale)
        arrs.append(a)
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    return tuple(torch.from_numpy(a).to(tdt) for a in arrs)


def make_global_proj(wl: Workload):
    """Return (q_g, k_g, v_g), the global rows' own projections, drawn like make_qkv
    with seed + 1000."""
    from dataclasses import replace

    return make_qkv(replace(wl, seed=wl.seed + 1000))


def make_custom(B, H, L, dtype="bf16", seed=0, scale=1.0, d=64):
    """Seeded q, k, v of an arbitrary shape (same recipe as the named workloads)."""
    wl = Workload("custom", B=B, H=H, L=L, w=0, dil=(1,) * H, dtype=dtype, seed=seed, scale=scale, d=d)
    return make_qkv(wl)


def make_bias(H: int, w: int, seed: int = 0, scale: float = 1.0):
    """Seeded relative-position-bias table [H, 2w + 1] (float32): i.i.d. normal
    values times ``scale``, the shape of a learned per-head, per-offset scalar."""
    rng = np.random.default_rng(seed + 7919)
    return (rng.standard_normal((H, 2 * w + 1)) * scale).astype(np.float32)


def make_random_blocks(H: int, L: int, r: int, seed: int = 0, block: int = 64):
    """Seeded random key-block draws [H, ceil(L / block), r] (int32): for each head and
    query block, r distinct key blocks chosen uniformly among all ceil(L / block)."""
    n = (L + block - 1) // block
    if r > n:
        raise ValueError("more draws per query block than key blocks")
    rng = np.random.default_rng(seed + 104729)
    out = np.empty((H, n, r), dtype=np.int32)
    for h in range(H):
        for qb in range(n):
            out[h, qb] = rng.choice(n, r, replace=False)
    return out


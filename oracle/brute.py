"""Brute-force enumeration of Longformer window + global attention for tiny inputs.

TEST INFRASTRUCTURE ONLY (see ``oracle/longformer_oracle.py``).  A second,
independent statement of the same definition, used to pin the fp64 oracle:
for each query row the key set is listed element by element from the pattern
definitions, and the softmax-weighted sum is formed with Python floats,
``math.exp`` and ``math.fsum``.  Meant for L <= 64.

Key set of query i (page "基于自注意力机制的长文本建模算法：Longformer详解",
§2: sliding window of w keys per side, dilation factor d giving positions
i-d*w ... i, ... i+d*w, global tokens that see and are seen by every position;
§4: the patterns are combined into one attention):
  * if i is global: every position 0..L-1;
  * otherwise: {i + m*dil : m = -w..w} intersected with [0, L), plus every global;
  * random blocks (BigBird's random attention, survey commentary on "Efficient
    Transformers" §3.1-§3.2): a non-global i also gets every key of the key blocks
    [kb*bs, kb*bs + bs) listed in rand[i // bs] (entries < 0 unused);
  * minus padded keys;
  * in the one-sided (causal) variant, minus every key after i.
"""

from __future__ import annotations

import math


def key_set(i: int, L: int, w: int, dil: int, globals_, pad_row=None, causal: bool = False,
            rand=None, rand_block: int = 64) -> list[int]:
    G = set(int(g) for g in (globals_ or []))
    if i in G:
        keys = set(range(L))
    else:
        keys = set()
        for m in range(-w, w + 1):
            j = i + m * dil
            if 0 <= j < L:
                keys.add(j)
        keys |= G
        if rand is not None:
            for kb in rand[i // rand_block]:
                if kb >= 0:
                    keys |= {j for j in range(kb * rand_block, (kb + 1) * rand_block) if j < L}
    if pad_row is not None:
        keys = {j for j in keys if not pad_row[j]}
    if causal:  # one-sided variant: no key after its query
        keys = {j for j in keys if j <= i}
    return sorted(keys)


def attention_row(q_i, k, v, keys) -> list[float]:
    """softmax(q_i . k_j / sqrt(d)) over ``keys``, applied to v; zeros if no key."""
    d = len(q_i)
    if not keys:
        return [0.0] * d
    scores = [math.fsum(q_i[t] * k[j][t] for t in range(d)) / math.sqrt(d) for j in keys]
    top = max(scores)
    weights = [math.exp(s - top) for s in scores]
    total = math.fsum(weights)
    return [math.fsum(weights[n] * v[j][t] for n, j in enumerate(keys)) / total for t in range(d)]


def attention_bh(q, k, v, w: int, dil: int, globals_=None, pad_row=None, causal: bool = False,
                 rand=None, rand_block: int = 64) -> list[list[float]]:
    """q, k, v: nested lists [L][d] of floats.  Returns [L][d]."""
    L = len(k)
    return [attention_row(q[i], k, v, key_set(i, L, w, dil, globals_, pad_row, causal, rand, rand_block))
            for i in range(L)]


def pair_count(L: int, w: int, dil: int, globals_=None, pad_row=None, causal: bool = False,
               rand=None, rand_block: int = 64) -> int:
    return sum(len(key_set(i, L, w, dil, globals_, pad_row, causal, rand, rand_block)) for i in range(L))

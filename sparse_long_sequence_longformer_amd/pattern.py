"""Host-side accounting of the attention pattern: attended-pair counts.

The effective work of one forward is 4*d_h FLOP per attended (query, key) pair
(d_h multiply-adds for q.k and d_h for p.v); exponentials and masked tile
entries are not counted.  Pair counts follow the pattern's complexity
statements: O(n*w) for the window and O(n*g) for globals (page
"基于Block-Sparse Attention的Longformer" §3 and §4).

Counts are formed without building the L x L mask: per residue class of the
dilation, a prefix sum over unpadded keys gives each row's window count in
O(1), and the few global keys are checked against the window directly.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass
class PairCounts:
    band: int  # non-global rows, keys in their window
    global_col: int  # non-global rows, global keys outside their window
    global_row: int  # global rows, every unpadded key
    random: int = 0  # non-global rows, keys of their random blocks outside window and globals

    @property
    def total(self) -> int:
        return self.band + self.global_col + self.global_row + self.random

    @property
    def band_kernel(self) -> int:
        """Pairs handled by the band kernel (window, global-column fold, random blocks)."""
        return self.band + self.global_col + self.random


def _unique_globals(global_idx, L):
    if global_idx is None:
        return np.zeros(0, dtype=np.int64)
    g = np.unique(np.asarray(global_idx, dtype=np.int64).reshape(-1))
    if g.size and (g[0] < 0 or g[-1] >= L):
        raise ValueError("global index out of range")
    return g


def _random_pairs(L: int, w: int, dil: int, is_g: np.ndarray, valid: np.ndarray, causal: bool, rand,
                  block: int) -> int:
    """Random-block pairs of non-global rows that neither the window nor the globals
    already give: one (query block x key block) rectangle at a time."""
    n_kb = (L + block - 1) // block
    key_ok = valid & ~is_g
    tot = 0
    for qb, row in enumerate(np.asarray(rand, dtype=np.int64)):
        i = np.arange(qb * block, min(L, qb * block + block), dtype=np.int64)
        i = i[~is_g[i]]
        if i.size == 0:
            continue
        for kb in np.unique(row[(row >= 0) & (row < n_kb)]):
            j = np.arange(kb * block, min(L, kb * block + block), dtype=np.int64)
            j = j[key_ok[j]]
            diff = j[None, :] - i[:, None]
            win = (diff % dil == 0) & (diff >= -w * dil) & (diff <= (0 if causal else w * dil))
            ok = ~win
            if causal:
                ok &= diff <= 0
            tot += int(ok.sum())
    return tot


def count_pairs_bh(L: int, w: int, dil: int, G: np.ndarray, valid: np.ndarray, causal: bool = False,
                   rand=None, rand_block: int = 64) -> PairCounts:
    """Pair counts for one (sequence, head).  ``valid[j]`` is True for unpadded keys.

    ``causal``: the one-sided variant, every pair with its key after its query removed
    (window keys i - m*dil for m = 0..w, global keys g <= i, global rows see j <= g).
    """
    is_g = np.zeros(L, dtype=bool)
    is_g[G] = True
    band = 0
    gcol = 0
    Gv = G[valid[G]] if G.size else G  # unpadded global keys
    for r in range(min(dil, L)):
        pos = np.arange(r, L, dil, dtype=np.int64)  # rows/keys of this residue class
        n = pos.size
        pref = np.concatenate([[0], np.cumsum(valid[pos].astype(np.int64))])
        i = np.arange(n, dtype=np.int64)
        lo = np.maximum(i - w, 0)
        hi = i if causal else np.minimum(i + w, n - 1)
        win = pref[hi + 1] - pref[lo]
        rows = ~is_g[pos]
        band += int(win[rows].sum())
        if Gv.size:
            # globals inside row's window: same residue and g' - i in [-w, w] ([-w, 0] causal)
            same = Gv[(Gv % dil) == r]
            gp = (same - r) // dil
            inside = np.zeros(n, dtype=np.int64)
            for g in gp:
                inside[max(0, g if causal else g - w):min(n, g + w + 1)] += 1
            # global keys the row sees at all: every one, or those at or before it (causal)
            seen = np.searchsorted(Gv, pos, side="right") if causal else np.full(n, Gv.size)
            gcol += int((seen - inside)[rows].sum())
    if causal:
        vpref = np.concatenate([[0], np.cumsum(valid.astype(np.int64))])
        grow = int(vpref[G + 1].sum()) if G.size else 0
    else:
        grow = int(G.size) * int(valid.sum())
    rnd = 0 if rand is None else _random_pairs(L, w, dil, is_g, valid, causal, rand, rand_block)
    return PairCounts(band, gcol, grow, rnd)


def count_pairs(L: int, w: int, dil_per_head, global_idx=None, key_pad_mask=None, B: int = 1,
                causal: bool = False, rand=None, rand_block: int = 64) -> PairCounts:
    """Attended pairs summed over B sequences and all heads.

    ``key_pad_mask`` is an array-like [B, L] (nonzero = padded) or None.
    ``global_idx``: one set for every sequence, or one row per sequence ([B][n],
    negative entries unused).
    ``rand``: random key blocks per head ([H][n_query_blocks][r], negative unused).
    """
    per_seq = global_idx is not None and np.asarray(global_idx).ndim == 2
    dils = [int(x) for x in np.asarray(dil_per_head).reshape(-1)]
    pad = None if key_pad_mask is None else (np.asarray(key_pad_mask) != 0)
    if pad is not None:
        B = pad.shape[0]
    if per_seq:
        B = np.asarray(global_idx).shape[0]
    tot = PairCounts(0, 0, 0, 0)
    cache = {}
    for b in range(B):
        if per_seq:
            row = np.asarray(global_idx, dtype=np.int64)[b]
            G = _unique_globals(row[row >= 0], L)
        else:
            G = _unique_globals(global_idx, L)
        valid = np.ones(L, dtype=bool) if pad is None else ~pad[b]
        key_b = b if (pad is not None or per_seq) else 0
        for hh, dl in enumerate(dils):
            key = (key_b, dl) if rand is None else (key_b, dl, hh)
            if key not in cache:
                cache[key] = count_pairs_bh(L, w, dl, G, valid, causal,
                                            None if rand is None else rand[hh], rand_block)
            c = cache[key]
            tot.band += c.band
            tot.global_col += c.global_col
            tot.global_row += c.global_row
            tot.random += c.random
    return tot


def effective_flops(pairs: int, d: int = 64) -> float:
    return 4.0 * d * pairs

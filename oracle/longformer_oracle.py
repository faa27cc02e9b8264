"""Plain fp64 CPU oracle for Longformer window + global sparse self-attention (forward).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library and imports nothing from it.

What it computes (per batch b and head h, with inputs widened to float64):

* Key set of query i (the attention pattern):
  - sliding / dilated window: keys j = i + m*dil for m in [-w, w], 0 <= j < L.
    Page "基于自注意力机制的长文本建模算法：Longformer详解" (Longformer explained),
    §2 "local sliding window" (w neighbours on each side, e.g. 512 each side)
    and §2 "dilated sliding window" (positions i-d*w ... i-d, i, i+d ... i+d*w).
  - global, symmetric: a global query attends to every position and every
    query attends to every global key.  Same page §2 "global attention"; page
    "基于Block-Sparse Attention的Longformer" (Block-Sparse Longformer) §2 and §4,
    which state both directions.
  - the union of these sets (each key counted once), Longformer explained §4
    (the three patterns are combined in one attention).
  - key padding: a padded key is never attended to (library convention; the
    pages only truncate inputs).
* Scores S = Q K^T / sqrt(d_h), masked entries set to -inf, row softmax, then
  O = P V: the textbook scaled dot-product attention of page
  "Reformer哈希：突破Transformer计算瓶颈的高效注意力机制详解" (Reformer hashing),
  §"core principle", restricted to the key set above.
* A query row whose key set is empty gives an all-zero output row.
* One-sided (causal) variant (``causal=True`` everywhere): every pair with a key
  after its query is removed, i.e. the key set above intersected with {j <= i}:
  window keys i - m*dil for m = 0..w, global keys g <= i, and a global row sees
  the keys j <= g.  This is the pattern of autoregressive language modelling,
  which the Longformer-explained page lists among the pretraining tasks (§6); the
  pages give no rule for it, and a mask on top of the union is the plainest one.
* Relative position bias (``bias``: one table of 2w+1 values per head): a window
  pair j = i + m*dil of a non-global row i scores S_ij + beta_h[m + w]; pairs that
  enter through the global pattern (global rows, global keys outside the window)
  get no bias.  Page "基于自注意力机制的长文本建模算法：Longformer详解" §5 names a
  relative position bias that strengthens the local attention.
* Random blocks (``rand``: per head, one row of key-block indices per query block;
  entries < 0 unused; block size ``rand_block``, 64 by default): a non-global row i
  also attends every key of the key blocks [kb*bs, kb*bs + bs) that its query block
  i // bs drew, in the union with its window and the globals (each key once).  The
  survey page (commentary on "Efficient Transformers: A Survey", §3.1-§3.2) names
  BigBird's random attention on top of window + global; the draws are inputs here
  (the page asks for a fixed seed so that inference is repeatable).
* Per-sequence global sets: ``global_idx`` may hold one row per sequence
  ([B][n], negative entries unused); sequence b then uses its own row as G.
* Variant with separate global projections (``attention_global_proj``): the page
  "基于Block-Sparse Attention的Longformer" §4 gives global attention its own
  query, key and value projections.  Read inside the one-softmax formulation: a
  global query row attends every unpadded key with its own projections,
  softmax(q_g k_g^T / sqrt(d_h)) v_g; every other row is computed exactly as above
  from q, k, v (its global keys included).

* Per-row log-sum-exp (``attention_lse``): log of the sum over the key set of
  exp(S_ij); -inf for a row with no key.  It is the normaliser of the row's
  softmax, the quantity a backward pass reuses.
* Gradient of the relative position bias tables (``attention_bias_grad``): entry
  m + w of head h's table sums dS_ij (below) over the window pairs j = i + m*dil of
  the non-global rows, the pairs the entry is added to.
* Gradients (``attention_backward``): for an upstream gradient dO of the output,
  the textbook derivatives of O = P V with P the row softmax of S (Reformer
  hashing page, "core principle" formula; the same key sets):
      dV = P^T dO,   dP = dO V^T,   dS = P * (dP - rowsum(dP * P)),
      dQ = dS K / sqrt(d_h),   dK = dS^T Q / sqrt(d_h),
  with rowsum(dP * P) = rowsum(dO * O).  A row with no key has a constant zero
  output: it contributes nothing.

The mask is built explicitly as dense boolean rows (R rows x L keys at a time)
directly from the set definitions above; no banding, tiling or online softmax.
"""

from __future__ import annotations

import math

import numpy as np

ROW_BLOCK = 512


def _as_f64(x) -> np.ndarray:
    """Widen a numpy array or a CPU torch tensor (any float dtype) to float64."""
    if hasattr(x, "detach"):  # torch tensor
        x = x.detach().to("cpu")
        import torch  # local: torch is only needed when handed a tensor

        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def globals_of(global_idx, b: int) -> np.ndarray:
    """The global set of sequence b: ``global_idx`` is one set shared by every
    sequence (1-D), or one row per sequence (2-D [B][n], entries < 0 unused)."""
    if global_idx is None:
        return np.zeros(0, dtype=np.int64)
    arr = np.asarray(global_idx, dtype=np.int64)
    if arr.ndim == 2:
        row = arr[b]
        return global_set(row[row >= 0])
    return global_set(arr)


def global_set(global_idx) -> np.ndarray:
    """The designated global positions as a sorted set (duplicates ignored)."""
    if global_idx is None:
        return np.zeros(0, dtype=np.int64)
    return np.unique(np.asarray(global_idx, dtype=np.int64).reshape(-1))


def window_member(i: np.ndarray, j: np.ndarray, w: int, dil: int) -> np.ndarray:
    """True where key j lies in query i's (dilated) window: j = i + m*dil, |m| <= w.

    Longformer explained §2: the window reaches w positions on each side, and a
    dilation factor d spaces the attended positions d apart (i-d*w ... i+d*w).
    """
    diff = j - i
    return (np.abs(diff) <= w * dil) & (diff % dil == 0)


def random_member(rows: np.ndarray, L: int, rand, block: int) -> np.ndarray:
    """R[r, j]: key j lies in one of the key blocks drawn by the query block of row
    rows[r].  ``rand`` is [n_query_blocks, r] (entries < 0 unused)."""
    rand = np.asarray(rand, dtype=np.int64)
    n_kb = (L + block - 1) // block
    drawn = np.zeros((rand.shape[0], n_kb + 1), dtype=bool)  # last column: unused entries
    for qb in range(rand.shape[0]):
        for kb in rand[qb]:
            drawn[qb, kb if 0 <= kb < n_kb else n_kb] = True
    sel = drawn[np.asarray(rows, dtype=np.int64) // block, :n_kb]  # [R, n_kb]
    return sel[:, np.arange(L) // block]


def mask_rows(L: int, w: int, dil: int, G: np.ndarray, pad_row, rows: np.ndarray, causal: bool = False,
              rand=None, rand_block: int = 64) -> np.ndarray:
    """Explicit boolean mask M[r, j] for the query rows ``rows`` over all L keys.

    M[i, j] = not pad[j] and (i in G or j in G or j in window(i) or j in the random
    blocks of i's block) [and j <= i if causal].
    """
    rows = np.asarray(rows, dtype=np.int64)
    j = np.arange(L, dtype=np.int64)[None, :]
    i = rows[:, None]
    is_global_key = np.zeros(L, dtype=bool)
    is_global_key[G] = True
    is_global_query = is_global_key[rows][:, None]
    m = window_member(i, j, w, dil) | is_global_key[None, :] | is_global_query
    if rand is not None:
        m |= random_member(rows, L, rand, rand_block)
    if pad_row is not None:
        m &= ~np.asarray(pad_row, dtype=bool)[None, :]
    if causal:
        m &= j <= i
    return m


def window_bias(L: int, w: int, dil: int, G: np.ndarray, rows, beta) -> np.ndarray:
    """Additive bias [R, L]: beta[m + w] where key j = i + m*dil lies in the window of a
    non-global row i, else 0 (validity is the mask's business)."""
    rows = np.asarray(rows, dtype=np.int64)
    j = np.arange(L, dtype=np.int64)[None, :]
    diff = j - rows[:, None]
    win = window_member(rows[:, None], j, w, dil)
    is_g = np.zeros(L, dtype=bool)
    is_g[G] = True
    win &= ~is_g[rows][:, None]
    m = np.where(win, diff // dil + w, 0)
    return np.where(win, np.asarray(beta, dtype=np.float64)[m], 0.0)


def _attention_rows(q, k, v, m, extra=None):
    """Masked softmax attention of the query rows in ``q`` against all keys.

    q: [R, d], k, v: [L, d], m: [R, L] boolean, extra: additive scores or None.
    Returns (O [R, d], P [R, L]).
    """
    d = q.shape[1]
    s = (q @ k.T) / math.sqrt(d)
    if extra is not None:
        s = s + extra
    s = np.where(m, s, -np.inf)
    row_max = s.max(axis=1, keepdims=True)
    has_key = np.isfinite(row_max)
    row_max = np.where(has_key, row_max, 0.0)
    e = np.where(m, np.exp(s - row_max), 0.0)
    denom = e.sum(axis=1, keepdims=True)
    p = np.where(has_key, e / np.where(has_key, denom, 1.0), 0.0)
    return p @ v, p


def attention_bh(q, k, v, w: int, dil: int, global_idx=None, pad_row=None, rows=None,
                 return_probs: bool = False, causal: bool = False, bias=None, rand=None, rand_block: int = 64):
    """Oracle for one (batch, head) slice.

    q, k, v: [L, d] arrays (widened to float64).  ``rows`` selects query rows
    (default: all).  Returns O [len(rows), d] float64, and the attention
    weights P [len(rows), L] when ``return_probs``.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    L = k.shape[0]
    if w < 0 or dil < 1:
        raise ValueError("need w >= 0 and dil >= 1")
    G = global_set(global_idx)
    if G.size and (G.min() < 0 or G.max() >= L):
        raise ValueError("global index out of range")
    rows = np.arange(L, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, q.shape[1]), dtype=np.float64)
    probs = np.zeros((rows.size, L), dtype=np.float64) if return_probs else None
    for s0 in range(0, rows.size, ROW_BLOCK):
        blk = rows[s0:s0 + ROW_BLOCK]
        m = mask_rows(L, w, dil, G, pad_row, blk, causal=causal, rand=rand, rand_block=rand_block)
        extra = None if bias is None else window_bias(L, w, dil, G, blk, bias)
        o, p = _attention_rows(q[blk], k, v, m, extra) if extra is not None else _attention_rows(q[blk], k, v, m)
        out[s0:s0 + blk.size] = o
        if return_probs:
            probs[s0:s0 + blk.size] = p
    return (out, probs) if return_probs else out


def attention(q, k, v, w: int, dil_per_head, global_idx=None, key_pad_mask=None, causal: bool = False,
              bias=None, rand=None, rand_block: int = 64):
    """Oracle for the full [B, H, L, d] problem.  Returns float64 [B, H, L, d].

    ``dil_per_head`` has one dilation per head (w is shared by all heads);
    ``global_idx`` is one set shared by every sequence and head;
    ``key_pad_mask`` is [B, L], nonzero meaning a padded key (or None);
    ``rand``: random key blocks per head, [H, n_query_blocks, r], or None.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, H, L, d = q.shape
    dil = [int(x) for x in np.asarray(dil_per_head).reshape(-1)]
    if len(dil) != H:
        raise ValueError("need one dilation per head")
    pad = None if key_pad_mask is None else np.asarray(_as_f64(key_pad_mask) != 0)
    out = np.zeros((B, H, L, d), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            out[b, h] = attention_bh(q[b, h], k[b, h], v[b, h], w, dil[h], globals_of(global_idx, b),
                                     None if pad is None else pad[b], causal=causal,
                                     bias=None if bias is None else bias[h],
                                     rand=None if rand is None else rand[h], rand_block=rand_block)
    return out


def attention_sampled(q, k, v, w: int, dil_per_head, global_idx, key_pad_mask, samples, causal: bool = False,
                      bias=None, rand=None, rand_block: int = 64):
    """Oracle output rows for a list of (b, h, i) samples, computed one by one.

    Used to check full-size runs where the whole oracle would be too slow.
    Returns float64 [len(samples), d].
    """
    dil = [int(x) for x in np.asarray(dil_per_head).reshape(-1)]
    pad = None if key_pad_mask is None else np.asarray(_as_f64(key_pad_mask) != 0)
    res = []
    for b, h, i in samples:
        o = attention_bh(q[b, h], k[b, h], v[b, h], w, dil[h], globals_of(global_idx, b),
                         None if pad is None else pad[b], rows=[i], causal=causal,
                         bias=None if bias is None else bias[h],
                         rand=None if rand is None else rand[h], rand_block=rand_block)
        res.append(o[0])
    return np.stack(res) if res else np.zeros((0, q.shape[-1]))


def mask_count(L: int, w: int, dil_per_head, global_idx=None, key_pad_mask=None, B: int = 1,
               causal: bool = False, rand=None, rand_block: int = 64) -> int:
    """Number of attended (query, key) pairs, summed over batch and heads: sum of M."""
    dil = [int(x) for x in np.asarray(dil_per_head).reshape(-1)]
    pad = None if key_pad_mask is None else np.asarray(_as_f64(key_pad_mask) != 0)
    total = 0
    for b in range(B):
        G = globals_of(global_idx, b)
        for h, d in enumerate(dil):
            for s0 in range(0, L, ROW_BLOCK):
                rows = np.arange(s0, min(L, s0 + ROW_BLOCK))
                total += int(mask_rows(L, w, d, G, None if pad is None else pad[b], rows, causal=causal,
                                       rand=None if rand is None else rand[h], rand_block=rand_block).sum())
    return total


def attention_global_proj(q, k, v, q_g, k_g, v_g, w: int, dil_per_head, global_idx=None, key_pad_mask=None,
                          causal: bool = False, bias=None, rand=None, rand_block: int = 64):
    """Oracle for the variant with separate global projections.  float64 [B, H, L, d].

    Rows not in the global set: ``attention(q, k, v, ...)``.  A global row g:
    masked softmax over the unpadded keys of q_g[g] . k_g^T / sqrt(d_h), times v_g
    (page "基于Block-Sparse Attention的Longformer" §4, global attention with its own
    projections; every global row sees every position, §2).  ``bias`` and ``rand``
    reach only the other rows, as in ``attention``.
    """
    out = attention(q, k, v, w, dil_per_head, global_idx, key_pad_mask, causal=causal, bias=bias, rand=rand,
                    rand_block=rand_block)
    q_g, k_g, v_g = _as_f64(q_g), _as_f64(k_g), _as_f64(v_g)
    B, H, L, d = q_g.shape
    pad = None if key_pad_mask is None else np.asarray(_as_f64(key_pad_mask) != 0)
    for b in range(B):
        G = globals_of(global_idx, b)
        if G.size == 0:
            continue
        keep = np.ones((G.size, L), dtype=bool)
        if pad is not None:
            keep &= ~pad[b][None, :]
        if causal:
            keep &= np.arange(L)[None, :] <= G[:, None]
        for h in range(H):
            o, _ = _attention_rows(q_g[b, h][G], k_g[b, h], v_g[b, h], keep)
            out[b, h][G] = o
    return out


def attention_global_proj_sampled(q, k, v, q_g, k_g, v_g, w: int, dil_per_head, global_idx, key_pad_mask,
                                  samples):
    """``attention_global_proj`` output rows for a list of (b, h, i) samples, one by one."""
    dil = [int(x) for x in np.asarray(dil_per_head).reshape(-1)]
    pad = None if key_pad_mask is None else np.asarray(_as_f64(key_pad_mask) != 0)
    res = []
    for b, h, i in samples:
        Gb = globals_of(global_idx, b)
        if i in set(int(x) for x in Gb):
            L = k_g.shape[2]
            keep = np.ones((1, L), dtype=bool)
            if pad is not None:
                keep &= ~pad[b][None, :]
            o, _ = _attention_rows(_as_f64(q_g[b, h][i:i + 1]), _as_f64(k_g[b, h]), _as_f64(v_g[b, h]), keep)
        else:
            o = attention_bh(q[b, h], k[b, h], v[b, h], w, dil[h], Gb,
                             None if pad is None else pad[b], rows=[i])
        res.append(o[0])
    return np.stack(res) if res else np.zeros((0, q.shape[-1]))


def _scores_rows(q, k, m, extra=None):
    """Masked scores S = Q K^T / sqrt(d) (+ extra) (-inf off the mask) of the query rows in q."""
    d = q.shape[1]
    s = (q @ k.T) / math.sqrt(d)
    if extra is not None:
        s = s + extra
    return np.where(m, s, -np.inf)


def attention_lse_bh(q, k, w: int, dil: int, global_idx=None, pad_row=None, causal: bool = False,
                     bias=None, rand=None, rand_block: int = 64) -> np.ndarray:
    """log sum_{j in keys(i)} exp(q_i . k_j / sqrt(d)) of every row; -inf without keys."""
    q, k = _as_f64(q), _as_f64(k)
    L = k.shape[0]
    G = global_set(global_idx)
    out = np.empty(L, dtype=np.float64)
    for s0 in range(0, L, ROW_BLOCK):
        blk = np.arange(s0, min(L, s0 + ROW_BLOCK))
        s = _scores_rows(q[blk], k, mask_rows(L, w, dil, G, pad_row, blk, causal=causal, rand=rand,
                                              rand_block=rand_block),
                         None if bias is None else window_bias(L, w, dil, G, blk, bias))
        top = s.max(axis=1)
        has = np.isfinite(top)
        safe = np.where(has, top, 0.0)
        tot = np.exp(s - safe[:, None]).sum(axis=1)
        out[s0:s0 + blk.size] = np.where(has, safe + np.log(np.where(has, tot, 1.0)), -np.inf)
    return out


def attention_lse(q, k, w: int, dil_per_head, global_idx=None, key_pad_mask=None, causal: bool = False,
                  bias=None, rand=None, rand_block: int = 64) -> np.ndarray:
    """Per-row log-sum-exp of the full problem: float64 [B, H, L]."""
    q, k = _as_f64(q), _as_f64(k)
    B, H, L, _ = q.shape
    dil = [int(x) for x in np.asarray(dil_per_head).reshape(-1)]
    pad = None if key_pad_mask is None else np.asarray(_as_f64(key_pad_mask) != 0)
    out = np.zeros((B, H, L), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            out[b, h] = attention_lse_bh(q[b, h], k[b, h], w, dil[h], globals_of(global_idx, b),
                                         None if pad is None else pad[b], causal=causal,
                                         bias=None if bias is None else bias[h],
                                         rand=None if rand is None else rand[h], rand_block=rand_block)
    return out


def attention_backward_bh(q, k, v, dout, w: int, dil: int, global_idx=None, pad_row=None, causal: bool = False,
                          bias=None, rand=None, rand_block: int = 64):
    """Gradients (dQ, dK, dV) of one (batch, head) slice for the upstream gradient dout.

    Row blocks of the explicit mask; dK and dV collect every block's contribution.
    """
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(dout)
    L, d = q.shape
    G = global_set(global_idx)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for s0 in range(0, L, ROW_BLOCK):
        blk = np.arange(s0, min(L, s0 + ROW_BLOCK))
        m = mask_rows(L, w, dil, G, pad_row, blk, causal=causal, rand=rand, rand_block=rand_block)
        extra = None if bias is None else window_bias(L, w, dil, G, blk, bias)
        o, p = _attention_rows(q[blk], k, v, m, extra) if extra is not None else _attention_rows(q[blk], k, v, m)
        dv += p.T @ do[blk]
        dp = do[blk] @ v.T
        delta = (do[blk] * o).sum(axis=1, keepdims=True)
        ds = p * (dp - delta)
        dq[blk] = ds @ k / math.sqrt(d)
        dk += ds.T @ q[blk] / math.sqrt(d)
    return dq, dk, dv


def attention_bias_grad_bh(q, k, v, dout, w: int, dil: int, global_idx=None, pad_row=None, causal: bool = False,
                           bias=None, rand=None, rand_block: int = 64) -> np.ndarray:
    """Gradient of sum(O * dout) with respect to one head's relative position bias table
    (2w+1 entries, reading of page "基于自注意力机制的长文本建模算法：Longformer详解" §5):
    entry m + w sums dS_ij over the window pairs j = i + m*dil of the non-global rows i
    that are in the key set (the pairs the entry was added to), with dS = P (dP - D) the
    gradient of the row's scaled scores."""
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(dout)
    L = q.shape[0]
    G = global_set(global_idx)
    is_g = np.zeros(L, dtype=bool)
    is_g[G] = True
    beta = np.zeros(2 * w + 1) if bias is None else np.asarray(bias, dtype=np.float64)
    db = np.zeros(2 * w + 1, dtype=np.float64)
    for s0 in range(0, L, ROW_BLOCK):
        blk = np.arange(s0, min(L, s0 + ROW_BLOCK))
        m = mask_rows(L, w, dil, G, pad_row, blk, causal=causal, rand=rand, rand_block=rand_block)
        o, p = _attention_rows(q[blk], k, v, m, window_bias(L, w, dil, G, blk, beta))
        dp = do[blk] @ v.T
        ds = p * (dp - (do[blk] * o).sum(axis=1, keepdims=True))
        j = np.arange(L)[None, :]
        win = window_member(blk[:, None], j, w, dil) & m & ~is_g[blk][:, None]
        idx = (j - blk[:, None]) // dil + w
        np.add.at(db, idx[win], ds[win])
    return db


def attention_bias_grad(q, k, v, dout, w: int, dil_per_head, global_idx=None, key_pad_mask=None,
                        causal: bool = False, bias=None, rand=None, rand_block: int = 64) -> np.ndarray:
    """Gradient of the relative position bias tables of the full problem: float64 [H, 2w+1],
    summed over the batch."""
    q = _as_f64(q)
    B, H, L, d = q.shape
    dil = [int(x) for x in np.asarray(dil_per_head).reshape(-1)]
    pad = None if key_pad_mask is None else np.asarray(_as_f64(key_pad_mask) != 0)
    out = np.zeros((H, 2 * w + 1), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            out[h] += attention_bias_grad_bh(q[b, h], k[b, h], v[b, h], dout[b, h], w, dil[h],
                                             globals_of(global_idx, b), None if pad is None else pad[b],
                                             causal=causal, bias=None if bias is None else bias[h],
                                             rand=None if rand is None else rand[h], rand_block=rand_block)
    return out


def _grads_rows(q_rows, k, v, do_rows, m, extra=None):
    """Gradients of O = softmax(q_rows k^T / sqrt(d) (+ extra), masked by m) v for the
    upstream gradient do_rows: (dQ of these rows, dK and dV contributions)."""
    d = q_rows.shape[1]
    o, p = _attention_rows(q_rows, k, v, m, extra) if extra is not None else _attention_rows(q_rows, k, v, m)
    dv = p.T @ do_rows
    dp = do_rows @ v.T
    delta = (do_rows * o).sum(axis=1, keepdims=True)
    ds = p * (dp - delta)
    return ds @ k / math.sqrt(d), ds.T @ q_rows / math.sqrt(d), dv


def attention_backward_global_proj_bh(q, k, v, q_g, k_g, v_g, dout, w: int, dil: int, global_idx=None,
                                      pad_row=None, causal: bool = False, bias=None, rand=None,
                                      rand_block: int = 64):
    """Gradients of one (batch, head) slice of ``attention_global_proj``: six arrays
    (dQ, dK, dV, dQ_g, dK_g, dV_g).  Rows outside the global set attend with q, k, v
    (their key sets as in ``attention``), so they give dQ of those rows and dK, dV; a
    global row attends every unpadded key (up to itself in the one-sided variant) with
    q_g, k_g, v_g, so it gives dQ_g of that row and dK_g, dV_g.  dQ of a global row and
    dQ_g of any other row are zero (those inputs are not read)."""
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(dout)
    q_g, k_g, v_g = _as_f64(q_g), _as_f64(k_g), _as_f64(v_g)
    L, d = q.shape
    G = global_set(global_idx)
    is_g = np.zeros(L, dtype=bool)
    is_g[G] = True
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dq_g, dk_g, dv_g = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    others = np.nonzero(~is_g)[0]
    for s0 in range(0, others.size, ROW_BLOCK):
        blk = others[s0:s0 + ROW_BLOCK]
        m = mask_rows(L, w, dil, G, pad_row, blk, causal=causal, rand=rand, rand_block=rand_block)
        extra = None if bias is None else window_bias(L, w, dil, G, blk, bias)
        a, b_, c = _grads_rows(q[blk], k, v, do[blk], m, extra)
        dq[blk] = a
        dk += b_
        dv += c
    if G.size:
        keep = np.ones((G.size, L), dtype=bool)
        if pad_row is not None:
            keep &= ~np.asarray(pad_row, dtype=bool)[None, :]
        if causal:
            keep &= np.arange(L)[None, :] <= G[:, None]
        a, b_, c = _grads_rows(q_g[G], k_g, v_g, do[G], keep)
        dq_g[G] = a
        dk_g += b_
        dv_g += c
    return dq, dk, dv, dq_g, dk_g, dv_g


def attention_backward_global_proj(q, k, v, q_g, k_g, v_g, dout, w: int, dil_per_head, global_idx=None,
                                   key_pad_mask=None, causal: bool = False, bias=None, rand=None,
                                   rand_block: int = 64):
    """Gradients of the full separate-projection problem: six float64 [B, H, L, d]
    arrays (dQ, dK, dV, dQ_g, dK_g, dV_g)."""
    q = _as_f64(q)
    B, H, L, d = q.shape
    dil = [int(x) for x in np.asarray(dil_per_head).reshape(-1)]
    pad = None if key_pad_mask is None else np.asarray(_as_f64(key_pad_mask) != 0)
    res = [np.zeros((B, H, L, d), dtype=np.float64) for _ in range(6)]
    for b in range(B):
        for h in range(H):
            parts = attention_backward_global_proj_bh(
                q[b, h], k[b, h], v[b, h], q_g[b, h], k_g[b, h], v_g[b, h], dout[b, h], w, dil[h],
                globals_of(global_idx, b), None if pad is None else pad[b], causal=causal,
                bias=None if bias is None else bias[h], rand=None if rand is None else rand[h],
                rand_block=rand_block)
            for r, x in zip(res, parts):
                r[b, h] = x
    return tuple(res)


def attention_backward(q, k, v, dout, w: int, dil_per_head, global_idx=None, key_pad_mask=None,
                       causal: bool = False, bias=None, rand=None, rand_block: int = 64):
    """Gradients of the full problem: three float64 [B, H, L, d] arrays (dQ, dK, dV)."""
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(dout)
    B, H, L, d = q.shape
    dil = [int(x) for x in np.asarray(dil_per_head).reshape(-1)]
    if len(dil) != H:
        raise ValueError("need one dilation per head")
    pad = None if key_pad_mask is None else np.asarray(_as_f64(key_pad_mask) != 0)
    dq, dk, dv = (np.zeros((B, H, L, d), dtype=np.float64) for _ in range(3))
    for b in range(B):
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h] = attention_backward_bh(
                q[b, h], k[b, h], v[b, h], do[b, h], w, dil[h], globals_of(global_idx, b),
                None if pad is None else pad[b], causal=causal, bias=None if bias is None else bias[h],
                rand=None if rand is None else rand[h], rand_block=rand_block)
    return dq, dk, dv

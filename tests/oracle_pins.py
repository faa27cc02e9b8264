"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
what the pages or the mathematics fix.  They are collected as tests by
``test_oracle_pins.py`` and re-run against deliberately broken copies of the
oracle by ``test_oracle_mutations.py`` (a pin set that cannot tell a broken
oracle from the right one proves nothing).
"""

from __future__ import annotations

import math
import os

import numpy as np
import torch

from oracle import brute
from oracle import longformer_oracle as orc

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _textbook_attention(q, k, v):
    """softmax(Q K^T / sqrt(d)) V by torch's CPU routine in float64 (page
    "Reformer哈希" §"core principle" formula)."""
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x))[None, None] for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)
    return out[0, 0].numpy()


def read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append(line.split())
    return rows


# ---------------------------------------------------------------- brute force

BRUTE_CASES = [
    # (L, d, w, dil, globals, pad_len or pad pattern seed, seed)
    (1, 8, 0, 1, [], None, 1),
    (7, 8, 2, 1, [], None, 2),
    (16, 8, 3, 2, [5], None, 3),
    (24, 8, 4, 3, [0, 23, 7, 7], None, 4),
    (33, 8, 5, 1, [2, 30], "rand", 5),
    (40, 8, 2, 4, [9, 39, 13], "rand", 6),
    (48, 8, 60, 1, [], None, 7),
    (31, 8, 0, 2, [4, 4, 17], "rand", 8),
    (20, 8, 3, 2, [1], "allbut", 9),
    (12, 64, 2, 3, [11], "suffix", 10),
]


def _pad_for(kind, L, seed):
    if kind is None:
        return None
    if kind == "rand":
        return np.random.default_rng(100 + seed).random(L) < 0.3
    if kind == "suffix":
        return np.arange(L) >= (2 * L) // 3
    if kind == "allbut":
        p = np.ones(L, dtype=bool)
        p[L // 2] = False
        return p
    raise ValueError(kind)


def pin_brute_force():
    """The oracle equals element-by-element enumeration with math.fsum (L <= 64)."""
    for L, d, w, dil, G, padk, seed in BRUTE_CASES:
        q, k, v = (_rand((L, d), seed * 3 + t) for t in range(3))
        pad = _pad_for(padk, L, seed)
        got = orc.attention_bh(q, k, v, w, dil, G, pad)
        ref = np.array(brute.attention_bh(q.tolist(), k.tolist(), v.tolist(), w, dil, G,
                                          None if pad is None else pad.tolist()))
        err = np.abs(got - ref).max() if L else 0.0
        assert err < 1e-12, f"brute force mismatch {err} for L={L} w={w} dil={dil} G={G}"


def pin_pair_counts_brute():
    """Mask sums equal the enumerated key-set sizes."""
    for L, d, w, dil, G, padk, seed in BRUTE_CASES:
        pad = _pad_for(padk, L, seed)
        n_brute = brute.pair_count(L, w, dil, G, None if pad is None else pad.tolist())
        n_orc = orc.mask_count(L, w, [dil], G, None if pad is None else pad[None, :])
        assert n_brute == n_orc, (L, w, dil, G, n_brute, n_orc)


# ---------------------------------------------------------- closed-form limits

def pin_full_attention_limit():
    """w >= L with dil = 1 is full attention: the textbook formula."""
    for L, w, seed in [(64, 64, 11), (100, 1000, 12), (37, 36, 13)]:
        q, k, v = (_rand((L, 64), seed * 3 + t) for t in range(3))
        got = orc.attention_bh(q, k, v, w, 1)
        ref = _textbook_attention(q, k, v)
        assert np.abs(got - ref).max() < 1e-12


def pin_all_global():
    """Every position global is full attention, whatever the window."""
    L = 50
    q, k, v = (_rand((L, 32), 20 + t) for t in range(3))
    for w, dil in [(0, 1), (3, 2)]:
        got = orc.attention_bh(q, k, v, w, dil, list(range(L)))
        assert np.abs(got - _textbook_attention(q, k, v)).max() < 1e-12


def pin_w0_identity():
    """w = 0, no globals, dil = 1, no padding: each query sees only itself, O = V exactly."""
    L = 45
    q, k, v = (_rand((L, 64), 30 + t) for t in range(3))
    got = orc.attention_bh(q, k, v, 0, 1)
    assert np.array_equal(got, v)


def pin_constant_v():
    """Constant V along the sequence gives that constant on every row with a key."""
    L = 70
    q, k = _rand((L, 16), 40), _rand((L, 16), 41)
    row = _rand((16,), 42)
    v = np.tile(row, (L, 1))
    pad = np.zeros(L, dtype=bool)
    pad[60:] = True
    got = orc.attention_bh(q, k, v, 3, 2, [5, 66], pad)
    assert np.abs(got - row[None, :]).max() < 1e-12


def pin_rows_sum_to_one():
    """Attention weights: each row sums to 1, is zero off the key set, and an empty
    key set gives a zero row (output zero)."""
    L = 60
    q, k, v = (_rand((L, 16), 50 + t) for t in range(3))
    pad = np.zeros(L, dtype=bool)
    pad[10:30] = True  # rows 10..29 with w=2, dil=1 have every window key padded
    G = [40]
    o, p = orc.attention_bh(q, k, v, 2, 1, G, pad, return_probs=True)
    s = p.sum(axis=1)
    for i in range(L):
        keys = brute.key_set(i, L, 2, 1, G, pad.tolist())
        off = np.ones(L, dtype=bool)
        off[keys] = False
        assert np.all(p[i, off] == 0.0)
        if keys:
            assert abs(s[i] - 1.0) < 1e-12
        else:
            assert s[i] == 0.0 and np.all(o[i] == 0.0)
    # with the global key padded as well, rows 12..27 have no key at all
    pad2 = pad.copy()
    pad2[40] = True
    o2 = orc.attention_bh(q, k, v, 2, 1, G, pad2)
    assert np.all(o2[12:28] == 0.0) and np.all(np.isfinite(o2))


# ------------------------------------------------------------- reductions

def pin_dilation_residues():
    """With no globals or padding and dil | L, the dilated window on residue class r
    is the plain window on the subsequence r, r+dil, ... (closed-form reduction)."""
    L, dil, w = 48, 3, 4
    q, k, v = (_rand((L, 16), 60 + t) for t in range(3))
    got = orc.attention_bh(q, k, v, w, dil)
    for r in range(dil):
        sub = orc.attention_bh(q[r::dil], k[r::dil], v[r::dil], w, 1)
        assert np.abs(got[r::dil] - sub).max() < 1e-12


def pin_padding_truncation():
    """Suffix padding: the rows before the true length equal the unpadded run on the
    truncated sequence."""
    L, n = 64, 41
    q, k, v = (_rand((L, 16), 70 + t) for t in range(3))
    pad = np.arange(L) >= n
    G = [3, 20]
    got = orc.attention_bh(q, k, v, 5, 2, G, pad)
    ref = orc.attention_bh(q[:n], k[:n], v[:n], 5, 2, G)
    assert np.abs(got[:n] - ref).max() < 1e-12


def pin_duplicate_globals():
    """Duplicated global indices are the same set (each key counted once)."""
    L = 40
    q, k, v = (_rand((L, 16), 80 + t) for t in range(3))
    a = orc.attention_bh(q, k, v, 3, 1, [7, 7, 30, 7, 30])
    b = orc.attention_bh(q, k, v, 3, 1, [30, 7])
    assert np.abs(a - b).max() == 0.0


def pin_global_in_window_counted_once():
    """A global key inside a row's window enters that row's softmax once: compare one
    row against its hand-listed key set."""
    L = 30
    q, k, v = (_rand((L, 8), 90 + t) for t in range(3))
    i, G = 10, [12]
    o = orc.attention_bh(q, k, v, 2, 1, G, rows=[i])[0]
    keys = [8, 9, 10, 11, 12]  # window of 10 with w=2; the global 12 already inside it
    s = np.array([q[i] @ k[j] for j in keys]) / math.sqrt(8)
    p = np.exp(s - s.max())
    p /= p.sum()
    assert np.abs(o - p @ v[keys]).max() < 1e-12


def pin_head_permutation():
    """Heads are independent: permuting heads together with their dilations permutes
    the outputs."""
    B, H, L, d = 2, 3, 24, 8
    q, k, v = (_rand((B, H, L, d), 100 + t) for t in range(3))
    dil = [1, 2, 3]
    pad = np.zeros((B, L), dtype=np.uint8)
    pad[1, 18:] = 1
    o = orc.attention(q, k, v, 2, dil, [4], pad)
    perm = [2, 0, 1]
    o2 = orc.attention(q[:, perm], k[:, perm], v[:, perm], 2, [dil[p] for p in perm], [4], pad)
    assert np.abs(o2 - o[:, perm]).max() == 0.0


# ------------------------------------------------------------- page values

def pin_dense_counts_golden():
    """The full-attention limit reproduces the dense counts the pages print."""
    for L, printed, rel, *_ in read_table("dense_pair_counts.txt"):
        L, printed, rel = int(L), float(printed), float(rel)
        n = orc.mask_count(L, L, [1])
        assert n == L * L
        assert abs(n - printed) <= rel * printed + 0.5, (L, n, printed)


def pin_window_example_golden():
    """512 keys per side: interior rows see 1025 keys, edge rows are truncated."""
    for L, w, dil, i, expect in read_table("window_example.txt"):
        L, w, dil, i, expect = map(int, (L, w, dil, i, expect))
        m = orc.mask_rows(L, w, dil, np.zeros(0, dtype=np.int64), None, np.array([i]))
        assert int(m.sum()) == expect
        assert len(brute.key_set(i, L, w, dil, [])) == expect


# ------------------------------------------- separate global projections

GP_CASES = [
    # (L, d, w, dils, globals, pad kind, seed)
    (24, 8, 3, [1, 2], [0, 9], None, 200),
    (33, 8, 2, [3, 1], [32, 4, 4], "rand", 201),
    (16, 8, 0, [1, 1], [7], "suffix", 202),
    (20, 8, 3, [2, 2], [], None, 203),
]


def _gp_inputs(L, d, H, seed):
    return [_rand((1, H, L, d), seed * 7 + t) for t in range(6)]


def pin_global_proj_brute():
    """Separate global projections: global rows are brute-force attention of q_g over
    every unpadded key of k_g, v_g; every other row is brute force over its own key
    set with q, k, v."""
    for L, d, w, dils, G, padk, seed in GP_CASES:
        H = len(dils)
        q, k, v, qg, kg, vg = _gp_inputs(L, d, H, seed)
        pad = _pad_for(padk, L, seed)
        got = orc.attention_global_proj(q, k, v, qg, kg, vg, w, dils, G,
                                        None if pad is None else pad[None, :])
        Gs = set(G)
        padl = None if pad is None else pad.tolist()
        for h in range(H):
            for i in range(L):
                keys = brute.key_set(i, L, w, dils[h], G, padl)
                if i in Gs:
                    ref = brute.attention_row(qg[0, h, i].tolist(), kg[0, h].tolist(), vg[0, h].tolist(), keys)
                else:
                    ref = brute.attention_row(q[0, h, i].tolist(), k[0, h].tolist(), v[0, h].tolist(), keys)
                err = np.abs(got[0, h, i] - np.array(ref)).max()
                assert err < 1e-12, (L, w, dils[h], G, i, err)


def pin_global_proj_dependence():
    """Global rows depend only on (q_g, k_g, v_g), the other rows only on (q, k, v):
    perturbing one triple leaves the other rows bit-identical and moves these rows."""
    L, d, w, dils, G = 40, 8, 3, [1, 2], [5, 31]
    q, k, v, qg, kg, vg = _gp_inputs(L, d, 2, 210)
    pad = np.zeros((1, L), dtype=bool)
    pad[0, 35:] = True
    base = orc.attention_global_proj(q, k, v, qg, kg, vg, w, dils, G, pad)
    is_g = np.zeros(L, dtype=bool)
    is_g[G] = True
    a = orc.attention_global_proj(q + 1.0, k * 1.5, v - 2.0, qg, kg, vg, w, dils, G, pad)
    assert np.array_equal(a[:, :, is_g], base[:, :, is_g])
    assert np.abs(a[:, :, ~is_g] - base[:, :, ~is_g]).min(axis=-1).max() > 0
    b = orc.attention_global_proj(q, k, v, qg + 1.0, kg * 1.5, vg - 2.0, w, dils, G, pad)
    assert np.array_equal(b[:, :, ~is_g], base[:, :, ~is_g])
    assert np.abs(b[:, :, is_g] - base[:, :, is_g]).min() > 0


def pin_global_proj_closed_forms():
    """k_g = 0 makes a global row the mean of the unpadded v_g rows; k_g = k, v_g = v,
    q_g = q is the single-projection attention."""
    L, d, w, dils, G = 30, 8, 2, [1, 3], [0, 17]
    q, k, v, qg, kg, vg = _gp_inputs(L, d, 2, 220)
    pad = np.zeros((1, L), dtype=bool)
    pad[0, [3, 4, 25]] = True
    got = orc.attention_global_proj(q, k, v, qg, np.zeros_like(kg), vg, w, dils, G, pad)
    mean = vg[0][:, ~pad[0]].mean(axis=1)  # [H, d]
    for g in G:
        assert np.abs(got[0, :, g] - mean).max() < 1e-12
    same = orc.attention_global_proj(q, k, v, q, k, v, w, dils, G, pad)
    ref = orc.attention(q, k, v, w, dils, G, pad)
    assert np.abs(same - ref).max() < 1e-12


def pin_global_proj_sampled():
    """The row-by-row sampler agrees with the full computation."""
    L, d, w, dils, G = 36, 8, 4, [2, 1], [1, 20, 35]
    q, k, v, qg, kg, vg = _gp_inputs(L, d, 2, 230)
    pad = np.zeros((1, L), dtype=bool)
    pad[0, 30:] = True
    full = orc.attention_global_proj(q, k, v, qg, kg, vg, w, dils, G, pad)
    samples = [(0, 0, 1), (0, 1, 20), (0, 1, 2), (0, 0, 33), (0, 1, 35)]
    got = orc.attention_global_proj_sampled(q, k, v, qg, kg, vg, w, dils, G, pad, samples)
    ref = np.stack([full[b, h, i] for b, h, i in samples])
    assert np.abs(got - ref).max() < 1e-12


# ------------------------------------------------------- backward and log-sum-exp

BWD_CASES = [
    # (L, d, w, dil, globals, pad kind, seed)
    (16, 8, 2, 1, [], None, 300),
    (24, 8, 3, 2, [5], None, 301),
    (33, 8, 4, 1, [2, 30, 30], "rand", 302),
    (40, 8, 2, 3, [9, 39], "suffix", 303),
    (20, 8, 3, 2, [1], "allbut", 304),
    (30, 8, 40, 1, [], None, 305),
]


def _torch_dense_attention(q, k, v, keysets):
    """softmax(Q K^T / sqrt(d)) V in torch float64 with the key sets given as lists
    (enumerated by brute.key_set); rows without keys give zeros."""
    L, d = q.shape
    m = torch.zeros(L, L, dtype=torch.bool)
    for i, ks in enumerate(keysets):
        m[i, ks] = True
    s = (q @ k.T) / math.sqrt(d)
    s = s.masked_fill(~m, float("-inf"))
    p = torch.softmax(s, dim=1)
    p = torch.where(m.any(dim=1, keepdim=True), p, torch.zeros_like(p))
    return p @ v


def pin_backward_autograd():
    """Analytic gradients equal torch autograd of a dense masked attention whose key
    sets come from the brute-force enumerator."""
    for L, d, w, dil, G, padk, seed in BWD_CASES:
        q, k, v, do = (_rand((L, d), seed * 5 + t) for t in range(4))
        pad = _pad_for(padk, L, seed)
        padl = None if pad is None else pad.tolist()
        keysets = [brute.key_set(i, L, w, dil, G, padl) for i in range(L)]
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        out = _torch_dense_attention(tq, tk, tv, keysets)
        (out * torch.from_numpy(do)).sum().backward()
        dq, dk, dv = orc.attention_backward_bh(q, k, v, do, w, dil, G, pad)
        for name, a, b in (("dq", dq, tq.grad), ("dk", dk, tk.grad), ("dv", dv, tv.grad)):
            err = np.abs(a - b.numpy()).max()
            assert err < 1e-12, (name, L, w, dil, G, padk, err)


def pin_backward_finite_differences():
    """Central differences of sum(O * dO) in float64 match every gradient entry."""
    L, d, w, dil, G = 10, 4, 2, 2, [3]
    q, k, v, do = (_rand((L, d), 320 + t) for t in range(4))
    pad = np.zeros(L, dtype=bool)
    pad[[1, 8]] = True
    dq, dk, dv = orc.attention_backward_bh(q, k, v, do, w, dil, G, pad)

    def loss(q_, k_, v_):
        return float((orc.attention_bh(q_, k_, v_, w, dil, G, pad) * do).sum())

    eps = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        for i in range(L):
            for c in range(d):
                args = [q.copy(), k.copy(), v.copy()]
                args[which][i, c] += eps
                up = loss(*args)
                args[which][i, c] -= 2 * eps
                dn = loss(*args)
                fd = (up - dn) / (2 * eps)
                assert abs(fd - grad[i, c]) < 1e-7, (which, i, c, fd, grad[i, c])


def pin_backward_structure():
    """With dO nonzero on one row only, dK and dV vanish exactly off that row's key
    set and not on it, and dQ vanishes on every other row."""
    L, d, w, dil, G = 36, 8, 3, 2, [4, 30]
    q, k, v = (_rand((L, d), 330 + t) for t in range(3))
    pad = np.zeros(L, dtype=bool)
    pad[[10, 25]] = True
    for i in (0, 4, 12, 30, 35):
        do = np.zeros((L, d))
        do[i] = _rand((d,), 340 + i)
        dq, dk, dv = orc.attention_backward_bh(q, k, v, do, w, dil, G, pad)
        keys = set(brute.key_set(i, L, w, dil, G, pad.tolist()))
        for j in range(L):
            if j in keys:
                assert np.abs(dv[j]).max() > 0 and np.abs(dk[j]).max() > 0, (i, j)
            else:
                assert np.all(dv[j] == 0) and np.all(dk[j] == 0), (i, j)
            if j != i:
                assert np.all(dq[j] == 0), (i, j)


def pin_backward_invariants():
    """Shift invariance of the softmax: adding one vector to every key leaves O
    unchanged, so the dK rows sum to zero; adding c to every value adds c to each row
    with a key, so the dV rows sum to the dO rows of rows with keys.  w = 0 without
    globals or padding is O = V: dV = dO, dQ = dK = 0 (up to rounding)."""
    L, d = 44, 8
    q, k, v, do = (_rand((L, d), 350 + t) for t in range(4))
    pad = np.zeros(L, dtype=bool)
    pad[12:20] = True  # with w = 1, dil = 1, rows 13..18 have no key
    dq, dk, dv = orc.attention_backward_bh(q, k, v, do, 1, 1, None, pad)
    assert np.abs(dk.sum(axis=0)).max() < 1e-12
    has = np.array([len(brute.key_set(i, L, 1, 1, [], pad.tolist())) > 0 for i in range(L)])
    assert not has[13:19].any() and has[:12].all()
    assert np.abs(dv.sum(axis=0) - do[has].sum(axis=0)).max() < 1e-12
    dq0, dk0, dv0 = orc.attention_backward_bh(q, k, v, do, 0, 1)
    # dS = 1 * (do_i . v_i - do_i . o_i) with o_i = v_i: zero up to the rounding of the
    # two dot products
    assert np.array_equal(dv0, do) and np.abs(dq0).max() < 1e-13 and np.abs(dk0).max() < 1e-13


def pin_lse_brute():
    """Per-row log-sum-exp equals log(fsum(exp)) over the enumerated key set, and
    torch's logsumexp in the full-attention limit."""
    for L, d, w, dil, G, padk, seed in BWD_CASES:
        q, k = _rand((L, d), seed * 5), _rand((L, d), seed * 5 + 1)
        pad = _pad_for(padk, L, seed)
        got = orc.attention_lse_bh(q, k, w, dil, G, pad)
        for i in range(L):
            keys = brute.key_set(i, L, w, dil, G, None if pad is None else pad.tolist())
            if not keys:
                assert got[i] == -np.inf
                continue
            sc = [math.fsum(q[i, t] * k[j, t] for t in range(d)) / math.sqrt(d) for j in keys]
            top = max(sc)
            ref = top + math.log(math.fsum(math.exp(x - top) for x in sc))
            assert abs(got[i] - ref) < 1e-12, (L, i, got[i], ref)
    L = 50
    q, k = _rand((L, 16), 360), _rand((L, 16), 361)
    ref = torch.logsumexp(torch.from_numpy(q @ k.T / 4.0), dim=1).numpy()
    assert np.abs(orc.attention_lse_bh(q, k, L, 1) - ref).max() < 1e-12


# ------------------------------------------------------ one-sided (causal) variant

def pin_causal_brute():
    """Causal variant: the oracle equals brute-force enumeration of the key sets with
    every key after its query removed; log-sum-exp as well."""
    for L, d, w, dil, G, padk, seed in BRUTE_CASES:
        q, k, v = (_rand((L, d), seed * 3 + t) for t in range(3))
        pad = _pad_for(padk, L, seed)
        padl = None if pad is None else pad.tolist()
        got = orc.attention_bh(q, k, v, w, dil, G, pad, causal=True)
        ref = np.array(brute.attention_bh(q.tolist(), k.tolist(), v.tolist(), w, dil, G, padl, causal=True))
        err = np.abs(got - ref).max() if L else 0.0
        assert err < 1e-12, (L, w, dil, G, err)
        assert orc.mask_count(L, w, [dil], G, None if pad is None else pad[None, :], causal=True) == \
            brute.pair_count(L, w, dil, G, padl, causal=True)
        lse = orc.attention_lse_bh(q, k, w, dil, G, pad, causal=True)
        for i in range(L):
            keys = brute.key_set(i, L, w, dil, G, padl, causal=True)
            if not keys:
                assert lse[i] == -np.inf
                continue
            sc = [math.fsum(q[i, t] * k[j, t] for t in range(d)) / math.sqrt(d) for j in keys]
            top = max(sc)
            assert abs(lse[i] - (top + math.log(math.fsum(math.exp(x - top) for x in sc)))) < 1e-12


def pin_causal_textbook():
    """w >= L, dil = 1, no globals: causal attention as computed by torch's CPU
    scaled_dot_product_attention(is_causal=True) in float64; row 0 is V_0 exactly."""
    for L, w in [(64, 64), (37, 100)]:
        q, k, v = (_rand((L, 32), 400 + L + t) for t in range(3))
        got = orc.attention_bh(q, k, v, w, 1, causal=True)
        tq, tk, tv = (torch.from_numpy(x)[None, None] for x in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)[0, 0].numpy()
        assert np.abs(got - ref).max() < 1e-12
        assert np.array_equal(got[0], v[0])


def pin_causal_prefix():
    """A causal row never depends on later positions: changing Q, K, V from position n
    on leaves rows < n bit-identical, with globals and padding."""
    L, n, w, dil, G = 60, 35, 4, 2, [3, 40, 50]
    q, k, v = (_rand((L, 8), 410 + t) for t in range(3))
    pad = np.zeros(L, dtype=bool)
    pad[[7, 45]] = True
    a = orc.attention_bh(q, k, v, w, dil, G, pad, causal=True)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    for x in (q2, k2, v2):
        x[n:] += 3.0
    b = orc.attention_bh(q2, k2, v2, w, dil, G, pad, causal=True)
    assert np.array_equal(a[:n], b[:n])
    assert np.abs(a[n:] - b[n:]).min(axis=1).max() > 0


def pin_causal_backward_autograd():
    """Causal gradients equal torch autograd of a dense masked attention whose key
    sets come from the causal brute-force enumeration."""
    for L, d, w, dil, G, padk, seed in BWD_CASES:
        q, k, v, do = (_rand((L, d), seed * 5 + 10 + t) for t in range(4))
        pad = _pad_for(padk, L, seed)
        padl = None if pad is None else pad.tolist()
        keysets = [brute.key_set(i, L, w, dil, G, padl, causal=True) for i in range(L)]
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        out = _torch_dense_attention(tq, tk, tv, keysets)
        (out * torch.from_numpy(do)).sum().backward()
        dq, dk, dv = orc.attention_backward_bh(q, k, v, do, w, dil, G, pad, causal=True)
        for name, a, b in (("dq", dq, tq.grad), ("dk", dk, tk.grad), ("dv", dv, tv.grad)):
            err = np.abs(a - b.numpy()).max()
            assert err < 1e-12, (name, L, w, dil, G, padk, err)


# ------------------------------------------------------------- the layer

def _layer_weights(E, F, seed, scale=0.05):
    rng = np.random.default_rng(seed)
    W = {
        "w_qkv": rng.standard_normal((3 * E, E)) * scale, "b_qkv": rng.standard_normal(3 * E) * scale,
        "w_o": rng.standard_normal((E, E)) * scale, "b_o": rng.standard_normal(E) * scale,
        "ln1_g": 1.0 + rng.standard_normal(E) * 0.1, "ln1_b": rng.standard_normal(E) * 0.1,
        "w_1": rng.standard_normal((F, E)) * scale, "b_1": rng.standard_normal(F) * scale,
        "w_2": rng.standard_normal((E, F)) * scale, "b_2": rng.standard_normal(E) * scale,
        "ln2_g": 1.0 + rng.standard_normal(E) * 0.1, "ln2_b": rng.standard_normal(E) * 0.1,
    }
    return W


def pin_layer_torch_encoder():
    """Full-attention limit (w >= L, no globals, dil = 1): the layer equals torch's
    nn.TransformerEncoderLayer (post-LayerNorm, GELU, no dropout) in float64 with the
    same weights, with and without key padding."""
    from oracle import layer_oracle as lo

    B, L, H, F = 2, 40, 2, 96
    E = 64 * H
    W = _layer_weights(E, F, 500)
    x = _rand((B, L, E), 501)
    enc = torch.nn.TransformerEncoderLayer(E, H, dim_feedforward=F, dropout=0.0, activation="gelu",
                                           batch_first=True, norm_first=False, dtype=torch.float64)
    with torch.no_grad():
        enc.self_attn.in_proj_weight.copy_(torch.from_numpy(W["w_qkv"]))
        enc.self_attn.in_proj_bias.copy_(torch.from_numpy(W["b_qkv"]))
        enc.self_attn.out_proj.weight.copy_(torch.from_numpy(W["w_o"]))
        enc.self_attn.out_proj.bias.copy_(torch.from_numpy(W["b_o"]))
        enc.linear1.weight.copy_(torch.from_numpy(W["w_1"]))
        enc.linear1.bias.copy_(torch.from_numpy(W["b_1"]))
        enc.linear2.weight.copy_(torch.from_numpy(W["w_2"]))
        enc.linear2.bias.copy_(torch.from_numpy(W["b_2"]))
        enc.norm1.weight.copy_(torch.from_numpy(W["ln1_g"]))
        enc.norm1.bias.copy_(torch.from_numpy(W["ln1_b"]))
        enc.norm2.weight.copy_(torch.from_numpy(W["ln2_g"]))
        enc.norm2.bias.copy_(torch.from_numpy(W["ln2_b"]))
    enc.eval()
    pad = np.zeros((B, L), dtype=bool)
    pad[1, 30:] = True
    for mask in (None, pad):
        with torch.no_grad():
            ref = enc(torch.from_numpy(x), src_key_padding_mask=None if mask is None else torch.from_numpy(mask))
        got = lo.layer_forward(x, W, H, L, [1] * H, None, mask)
        assert np.abs(got - ref.numpy()).max() < 1e-10


def pin_layer_norm_rows():
    """With unit gains and zero shifts every output row has mean 0 and variance
    1 / (1 + eps / var): LayerNorm's own definition, checked on the layer output."""
    from oracle import layer_oracle as lo

    B, L, H, F = 1, 30, 1, 64
    E = 64 * H
    W = _layer_weights(E, F, 510)
    for n in ("ln1_g", "ln2_g"):
        W[n] = np.ones(E)
    for n in ("ln1_b", "ln2_b"):
        W[n] = np.zeros(E)
    x = _rand((B, L, E), 511)
    out = lo.layer_forward(x, W, H, 5, [2], [3], None, eps=0.0)
    assert np.abs(out.mean(axis=-1)).max() < 1e-12
    assert np.abs(out.var(axis=-1) - 1.0).max() < 1e-12


# -------------------------------------------------------- per-sequence global sets

def pin_global_sets_per_sequence():
    """Per-sequence global sets: each sequence equals brute-force enumeration with its
    own set; identical rows equal the shared set; -1 entries are ignored."""
    B, H, L, d, w = 3, 2, 36, 8, 3
    dil = [1, 2]
    q, k, v = (_rand((B, H, L, d), 600 + t) for t in range(3))
    sets = np.array([[0, 17, -1, -1], [5, 5, 30, 2], [-1, -1, -1, -1]])
    pad = np.zeros((B, L), dtype=bool)
    pad[1, 31:] = True
    got = orc.attention(q, k, v, w, dil, sets, pad)
    for b in range(B):
        G = [int(g) for g in sets[b] if g >= 0]
        for h in range(H):
            ref = np.array(brute.attention_bh(q[b, h].tolist(), k[b, h].tolist(), v[b, h].tolist(), w, dil[h], G,
                                              pad[b].tolist()))
            assert np.abs(got[b, h] - ref).max() < 1e-12, (b, h)
    same = np.array([[4, 20]] * B)
    assert np.array_equal(orc.attention(q, k, v, w, dil, same, pad), orc.attention(q, k, v, w, dil, [4, 20], pad))
    n = orc.mask_count(L, w, dil, sets, pad, B=B)
    assert n == sum(brute.pair_count(L, w, dd, [int(g) for g in sets[b] if g >= 0], pad[b].tolist())
                    for b in range(B) for dd in dil)


# ------------------------------------------------------ relative position bias

def pin_bias_sdpa():
    """Full-window limit (no globals, dil = 1): the biased attention equals torch's CPU
    scaled_dot_product_attention with the additive mask B[i, j] = beta[j - i + w] in
    float64; its log-sum-exp and autograd gradients agree as well."""
    L, w, d = 40, 40, 16
    q, k, v, do = (_rand((L, d), 700 + t) for t in range(4))
    beta = _rand((2 * w + 1,), 704)
    i = np.arange(L)
    Bm = beta[(i[None, :] - i[:, None]) + w]
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq[None, None], tk[None, None], tv[None, None],
                                                           attn_mask=torch.from_numpy(Bm)[None, None])[0, 0]
    got = orc.attention_bh(q, k, v, w, 1, bias=beta)
    assert np.abs(got - ref.detach().numpy()).max() < 1e-12
    lse = orc.attention_lse_bh(q, k, w, 1, bias=beta)
    s = q @ k.T / math.sqrt(d) + Bm
    assert np.abs(lse - (s.max(1) + np.log(np.exp(s - s.max(1, keepdims=True)).sum(1)))).max() < 1e-12
    (ref * torch.from_numpy(do)).sum().backward()
    dq, dk, dv = orc.attention_backward_bh(q, k, v, do, w, 1, bias=beta)
    for a, b in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.abs(a - b.numpy()).max() < 1e-12


def pin_bias_shift_and_scope():
    """A constant bias changes nothing without globals (softmax shift invariance); with
    globals, only window pairs of non-global rows are biased: a global row is unchanged,
    and a brute-force listing of one non-global row's scores matches."""
    L, w, dil, d = 36, 3, 2, 8
    q, k, v = (_rand((L, d), 710 + t) for t in range(3))
    pad = np.zeros(L, dtype=bool)
    pad[[5, 30]] = True
    base = orc.attention_bh(q, k, v, w, dil, None, pad)
    const = orc.attention_bh(q, k, v, w, dil, None, pad, bias=np.full(2 * w + 1, 2.5))
    assert np.abs(base - const).max() < 1e-12
    G = [4, 33]
    beta = _rand((2 * w + 1,), 713)
    got = orc.attention_bh(q, k, v, w, dil, G, pad, bias=beta)
    assert np.array_equal(got[G], orc.attention_bh(q, k, v, w, dil, G, pad)[G])
    i = 14
    keys = brute.key_set(i, L, w, dil, G, pad.tolist())
    sc = []
    for j in keys:
        t = math.fsum(q[i, c] * k[j, c] for c in range(d)) / math.sqrt(d)
        if (j - i) % dil == 0 and abs(j - i) <= w * dil:
            t += beta[(j - i) // dil + w]
        sc.append(t)
    e = np.exp(np.array(sc) - max(sc))
    assert np.abs(got[i] - (e / e.sum()) @ v[keys]).max() < 1e-12



# ------------------------------------------------------------- random blocks

# (L, d, w, dil, globals, pad kind, block, draws per query block, causal, seed)
RAND_CASES = [
    (16, 8, 1, 1, [], None, 4, 1, False, 1),
    (40, 8, 2, 1, [3, 31], None, 8, 2, False, 2),
    (37, 8, 3, 2, [0, 36], "rand", 4, 3, False, 3),
    (48, 8, 2, 1, [10], "suffix", 8, 2, True, 4),
    (29, 8, 0, 1, [], "rand", 4, 4, True, 5),
    (64, 16, 5, 3, [7, 7, 50], "rand", 16, 2, False, 6),
]


def _draws(L, block, r, seed):
    """Key-block draws per query block with duplicates and unused (-1) entries."""
    n = (L + block - 1) // block
    return np.random.default_rng(700 + seed).integers(-1, n, size=(n, r))


def pin_random_brute():
    """Random blocks: the oracle (output, log-sum-exp, mask sum) equals brute-force
    enumeration of window + globals + the key blocks each query block drew."""
    for L, d, w, dil, G, padk, bs, r, causal, seed in RAND_CASES:
        q, k, v = (_rand((L, d), 900 + seed * 3 + t) for t in range(3))
        pad = _pad_for(padk, L, seed)
        padl = None if pad is None else pad.tolist()
        rnd = _draws(L, bs, r, seed)
        got = orc.attention_bh(q, k, v, w, dil, G, pad, causal=causal, rand=rnd, rand_block=bs)
        ref = np.array(brute.attention_bh(q.tolist(), k.tolist(), v.tolist(), w, dil, G, padl, causal, rnd, bs))
        assert np.abs(got - ref).max() < 1e-12, (L, w, dil, bs, causal)
        assert orc.mask_count(L, w, [dil], G, None if pad is None else pad[None, :], causal=causal, rand=[rnd],
                              rand_block=bs) == brute.pair_count(L, w, dil, G, padl, causal, rnd, bs)
        lse = orc.attention_lse_bh(q, k, w, dil, G, pad, causal=causal, rand=rnd, rand_block=bs)
        for i in range(L):
            keys = brute.key_set(i, L, w, dil, G, padl, causal, rnd, bs)
            if not keys:
                assert lse[i] == -np.inf
                continue
            sc = [math.fsum(q[i, t] * k[j, t] for t in range(d)) / math.sqrt(d) for j in keys]
            top = max(sc)
            assert abs(lse[i] - (top + math.log(math.fsum(math.exp(x - top) for x in sc)))) < 1e-12


def pin_random_limits():
    """Every query block drawing every key block is full attention (torch SDPA, and its
    causal form); a draw of each row's own block with w >= block - 1 adds no key (the
    result is bit-identical to no draws); global rows ignore the draws."""
    L, bs = 40, 8
    n = L // bs
    q, k, v = (_rand((L, 16), 950 + t) for t in range(3))
    every = np.tile(np.arange(n), (n, 1))
    got = orc.attention_bh(q, k, v, 0, 1, rand=every, rand_block=bs)
    assert np.abs(got - _textbook_attention(q, k, v)).max() < 1e-12
    tq, tk, tv = (torch.from_numpy(x)[None, None] for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)[0, 0].numpy()
    assert np.abs(orc.attention_bh(q, k, v, 0, 1, rand=every, rand_block=bs, causal=True) - ref).max() < 1e-12
    own = np.arange(n)[:, None]
    pad = _pad_for("rand", L, 3)
    for w in (bs - 1, bs + 3):
        a = orc.attention_bh(q, k, v, w, 1, [5, 30], pad, rand=own, rand_block=bs)
        b = orc.attention_bh(q, k, v, w, 1, [5, 30], pad)
        assert np.array_equal(a, b)
    # a strictly smaller window loses keys that the own-block draw puts back
    a = orc.attention_bh(q, k, v, 1, 1, rand=own, rand_block=bs)
    assert np.abs(a - orc.attention_bh(q, k, v, 1, 1)).max() > 1e-3
    G = [2, 17]
    far = np.full((n, 1), n - 1)
    a = orc.attention_bh(q, k, v, 1, 1, G, rand=far, rand_block=bs)
    b = orc.attention_bh(q, k, v, 1, 1, G)
    assert np.array_equal(a[G], b[G])


def pin_random_backward_autograd():
    """Random-block gradients equal torch autograd of the dense masked attention whose
    key sets come from the brute-force enumeration."""
    for L, d, w, dil, G, padk, bs, r, causal, seed in RAND_CASES:
        q, k, v, do = (_rand((L, d), 980 + seed * 5 + t) for t in range(4))
        pad = _pad_for(padk, L, seed)
        padl = None if pad is None else pad.tolist()
        rnd = _draws(L, bs, r, seed)
        keysets = [brute.key_set(i, L, w, dil, G, padl, causal, rnd, bs) for i in range(L)]
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        out = _torch_dense_attention(tq, tk, tv, keysets)
        (out * torch.from_numpy(do)).sum().backward()
        dq, dk, dv = orc.attention_backward_bh(q, k, v, do, w, dil, G, pad, causal=causal, rand=rnd,
                                               rand_block=bs)
        for name, a, b in (("dq", dq, tq.grad), ("dk", dk, tk.grad), ("dv", dv, tv.grad)):
            err = np.abs(a - b.numpy()).max()
            assert err < 1e-12, (name, L, w, dil, G, padk, err)



# ---------------------------------------- backward of the separate global projections

def pin_global_proj_backward_autograd():
    """Gradients of the separate-projection variant equal torch autograd of a dense
    formulation: other rows attend their brute-force key sets with q, k, v, global rows
    every unpadded key (up to themselves when one-sided) with q_g, k_g, v_g."""
    cases = [(24, 8, 3, 2, [0, 7, 7, 23], "rand", False), (33, 8, 4, 1, [5, 30], None, True),
             (40, 16, 2, 3, [1, 20, 39], "suffix", False)]
    for L, d, w, dil, G, padk, causal in cases:
        pad = _pad_for(padk, L, L)
        padl = None if pad is None else pad.tolist()
        arrs = [_rand((L, d), 1300 + L + t) for t in range(7)]
        q, k, v, qg, kg, vg, do = arrs
        Gs = sorted(set(G))
        keysets = [brute.key_set(i, L, w, dil, G, padl, causal=causal) for i in range(L)]
        ts = [torch.tensor(x, requires_grad=True) for x in (q, k, v, qg, kg, vg)]
        base = _torch_dense_attention(ts[0], ts[1], ts[2], keysets)
        gkeys = [[j for j in range(L) if (padl is None or not padl[j]) and (not causal or j <= i)] for i in range(L)]
        glob = _torch_dense_attention(ts[3], ts[4], ts[5], gkeys)
        rows = torch.zeros(L, 1, dtype=torch.float64)
        rows[Gs] = 1.0
        out = base * (1 - rows) + glob * rows
        (out * torch.from_numpy(do)).sum().backward()
        got = orc.attention_backward_global_proj_bh(q, k, v, qg, kg, vg, do, w, dil, G, pad, causal=causal)
        for name, a, t in zip(("dq", "dk", "dv", "dq_g", "dk_g", "dv_g"), got, ts):
            err = np.abs(a - t.grad.numpy()).max()
            assert err < 1e-12, (name, L, w, dil, G, causal, err)


def pin_global_proj_backward_reduces():
    """With q_g = q, k_g = k, v_g = v the two gradient sets add up to the single-projection
    gradients (each global row's pairs move from one set to the other)."""
    L, d, w, dil, G = 36, 8, 3, 2, [0, 11, 35]
    pad = _pad_for("rand", L, 5)
    q, k, v, do = (_rand((L, d), 1400 + t) for t in range(4))
    parts = orc.attention_backward_global_proj_bh(q, k, v, q, k, v, do, w, dil, G, pad)
    ref = orc.attention_backward_bh(q, k, v, do, w, dil, G, pad)
    for a, b_, r in zip(parts[:3], parts[3:], ref):
        assert np.abs(a + b_ - r).max() < 1e-12
    assert np.all(parts[0][G] == 0) and np.all(np.delete(parts[3], G, axis=0) == 0)


# ------------------------------------ full-problem wrappers (per-(b, h) indexing)
#
# attention_sampled, attention_lse, attention_backward and
# attention_backward_global_proj carry the per-slice indexing themselves: pad[b],
# dil[h], the global set of sequence b, bias[h], rand[h].  Every sequence and every
# head below differs in each of these, and B = H, so a swapped b and h gives wrong
# numbers (not an index error).

WRAP_B, WRAP_H, WRAP_L, WRAP_D, WRAP_W, WRAP_BS = 3, 3, 40, 8, 3, 8
WRAP_DIL = [1, 2, 3]


def _wrap_case(seed):
    """Inputs of the wrapper pins: per-sequence padding and global sets, per-head
    dilation, bias table and random draws (blocks of 8 keys)."""
    B, H, L, d, w = WRAP_B, WRAP_H, WRAP_L, WRAP_D, WRAP_W
    arrs = [_rand((B, H, L, d), seed + t) for t in range(7)]
    pad = np.zeros((B, L), dtype=bool)
    pad[0, 33:] = True           # suffix
    pad[1, [3, 17, 29]] = True   # scattered; sequence 2 unpadded
    sets = np.array([[0, 21, -1], [5, 5, 38], [-1, -1, -1]])
    bias = _rand((H, 2 * w + 1), seed + 20)
    rand = np.stack([_draws(L, WRAP_BS, 2, seed + 30 + h) for h in range(H)])
    return arrs, pad, sets, bias, rand


def _wrap_keys(b, h, i, pad, sets, rand, causal):
    G = [int(g) for g in sets[b] if g >= 0]
    return brute.key_set(i, WRAP_L, WRAP_W, WRAP_DIL[h], G, pad[b].tolist(), causal, rand[h], WRAP_BS)


def _wrap_bias(b, h, i, j, sets, bias):
    """Bias of pair (i, j) listed from the definition: a window pair j = i + m*dil of a
    non-global row gets beta_h[m + w]."""
    dil, w = WRAP_DIL[h], WRAP_W
    if i in set(int(g) for g in sets[b] if g >= 0):
        return 0.0
    if (j - i) % dil == 0 and abs(j - i) <= w * dil:
        return float(bias[h][(j - i) // dil + w])
    return 0.0


def _wrap_scores(q, k, b, h, i, keys, sets, bias):
    d = q.shape[-1]
    return [math.fsum(q[b, h, i, c] * k[b, h, j, c] for c in range(d)) / math.sqrt(d)
            + _wrap_bias(b, h, i, j, sets, bias) for j in keys]


def pin_wrapper_sampled():
    """attention_sampled at every (b, h, i) equals a brute-force row (listed key set,
    listed bias, math.fsum), in both window modes."""
    (q, k, v, *_), pad, sets, bias, rand = _wrap_case(1500)
    samples = [(b, h, i) for b in range(WRAP_B) for h in range(WRAP_H) for i in range(WRAP_L)]
    for causal in (False, True):
        got = orc.attention_sampled(q, k, v, WRAP_W, WRAP_DIL, sets, pad, samples, causal=causal, bias=bias,
                                    rand=rand, rand_block=WRAP_BS)
        for n, (b, h, i) in enumerate(samples):
            keys = _wrap_keys(b, h, i, pad, sets, rand, causal)
            if not keys:
                assert np.all(got[n] == 0), (b, h, i)
                continue
            sc = _wrap_scores(q, k, b, h, i, keys, sets, bias)
            top = max(sc)
            e = [math.exp(x - top) for x in sc]
            tot = math.fsum(e)
            ref = [math.fsum(e[t] * v[b, h, j, c] for t, j in enumerate(keys)) / tot for c in range(WRAP_D)]
            assert np.abs(got[n] - np.array(ref)).max() < 1e-12, (causal, b, h, i)


def pin_wrapper_lse():
    """attention_lse of the full problem equals log(fsum(exp)) over each row's listed
    key set (with the listed bias), -inf for rows without keys."""
    (q, k, *_), pad, sets, bias, rand = _wrap_case(1600)
    for causal in (False, True):
        got = orc.attention_lse(q, k, WRAP_W, WRAP_DIL, sets, pad, causal=causal, bias=bias, rand=rand,
                                rand_block=WRAP_BS)
        for b in range(WRAP_B):
            for h in range(WRAP_H):
                for i in range(WRAP_L):
                    keys = _wrap_keys(b, h, i, pad, sets, rand, causal)
                    if not keys:
                        assert got[b, h, i] == -np.inf, (b, h, i)
                        continue
                    sc = _wrap_scores(q, k, b, h, i, keys, sets, bias)
                    top = max(sc)
                    ref = top + math.log(math.fsum(math.exp(x - top) for x in sc))
                    assert abs(got[b, h, i] - ref) < 1e-12, (causal, b, h, i)


def _wrap_dense(tq, tk, tv, b, h, pad, sets, bias, rand, causal, rows=None):
    """Dense masked attention of slice (b, h) in torch float64: listed key sets and
    bias entries; rows without keys give zeros.  rows: restrict the queries."""
    L = WRAP_L
    m = torch.zeros(L, L, dtype=torch.bool)
    extra = torch.zeros(L, L, dtype=torch.float64)
    for i in range(L):
        for j in _wrap_keys(b, h, i, pad, sets, rand, causal):
            m[i, j] = True
            extra[i, j] = _wrap_bias(b, h, i, j, sets, bias)
    s = (tq @ tk.T) / math.sqrt(tq.shape[1]) + extra
    s = s.masked_fill(~m, float("-inf"))
    p = torch.softmax(s, dim=1)
    p = torch.where(m.any(dim=1, keepdim=True), p, torch.zeros_like(p))
    return p @ tv


def pin_wrapper_backward():
    """attention_backward of the full problem equals torch autograd, slice by slice, of
    the dense masked attention built from the listed key sets and bias entries."""
    (q, k, v, do, *_), pad, sets, bias, rand = _wrap_case(1700)
    for causal in (False, True):
        got = orc.attention_backward(q, k, v, do, WRAP_W, WRAP_DIL, sets, pad, causal=causal, bias=bias, rand=rand,
                                     rand_block=WRAP_BS)
        for b in range(WRAP_B):
            for h in range(WRAP_H):
                ts = [torch.tensor(x[b, h], requires_grad=True) for x in (q, k, v)]
                out = _wrap_dense(*ts, b, h, pad, sets, bias, rand, causal)
                (out * torch.from_numpy(do[b, h])).sum().backward()
                for name, a, t in zip(("dq", "dk", "dv"), got, ts):
                    err = np.abs(a[b, h] - t.grad.numpy()).max()
                    assert err < 1e-12, (name, causal, b, h, err)


def pin_wrapper_backward_global_proj():
    """attention_backward_global_proj of the full problem equals torch autograd, slice by
    slice: other rows attend their listed key sets (with the listed bias) with q, k, v;
    global rows attend every unpadded key (up to themselves when one-sided) with q_g,
    k_g, v_g."""
    (q, k, v, qg, kg, vg, do), pad, sets, bias, rand = _wrap_case(1800)
    L = WRAP_L
    for causal in (False, True):
        got = orc.attention_backward_global_proj(q, k, v, qg, kg, vg, do, WRAP_W, WRAP_DIL, sets, pad,
                                                 causal=causal, bias=bias, rand=rand, rand_block=WRAP_BS)
        for b in range(WRAP_B):
            Gs = sorted(set(int(g) for g in sets[b] if g >= 0))
            for h in range(WRAP_H):
                ts = [torch.tensor(x[b, h], requires_grad=True) for x in (q, k, v, qg, kg, vg)]
                base = _wrap_dense(ts[0], ts[1], ts[2], b, h, pad, sets, bias, rand, causal)
                gm = torch.zeros(L, L, dtype=torch.bool)
                for i in range(L):
                    for j in range(L):
                        gm[i, j] = not pad[b, j] and (not causal or j <= i)
                s = ((ts[3] @ ts[4].T) / math.sqrt(WRAP_D)).masked_fill(~gm, float("-inf"))
                p = torch.softmax(s, dim=1)
                p = torch.where(gm.any(dim=1, keepdim=True), p, torch.zeros_like(p))
                glob = p @ ts[5]
                rows = torch.zeros(L, 1, dtype=torch.float64)
                rows[Gs] = 1.0
                out = base * (1 - rows) + glob * rows
                (out * torch.from_numpy(do[b, h])).sum().backward()
                for name, a, t in zip(("dq", "dk", "dv", "dq_g", "dk_g", "dv_g"), got, ts):
                    err = np.abs(a[b, h] - t.grad.numpy()).max()
                    assert err < 1e-12, (name, causal, b, h, err)


# ------------------------------------------------- gradient of the position bias table

def _bias_dense_torch(q, k, v, table, L, w, dil, G, padl, causal, rand, bs):
    """Dense masked attention in torch float64 with the bias table gathered onto the
    window pairs of non-global rows, pairs listed by brute force."""
    d = q.shape[1]
    Gs = set(int(g) for g in G)
    m = torch.zeros(L, L, dtype=torch.bool)
    idx = torch.zeros(L, L, dtype=torch.long)
    use = torch.zeros(L, L, dtype=torch.bool)
    for i in range(L):
        for j in brute.key_set(i, L, w, dil, G, padl, causal, rand, bs):
            m[i, j] = True
            if i not in Gs and (j - i) % dil == 0 and abs(j - i) <= w * dil:
                use[i, j] = True
                idx[i, j] = (j - i) // dil + w
    s = (q @ k.T) / math.sqrt(d) + torch.where(use, table[idx], torch.zeros((), dtype=torch.float64))
    s = s.masked_fill(~m, float("-inf"))
    p = torch.softmax(s, dim=1)
    p = torch.where(m.any(dim=1, keepdim=True), p, torch.zeros_like(p))
    return p @ v


BIAS_GRAD_CASES = [
    # (L, d, w, dil, globals, pad kind, causal, random draws (block, r) or None)
    (30, 8, 3, 1, [], None, False, None),
    (36, 8, 4, 2, [4, 5, 33], "rand", False, None),
    (40, 8, 5, 1, [0, 9, 9, 39], "suffix", True, None),
    (48, 8, 2, 3, [7, 20], None, False, None),
    (40, 8, 2, 1, [3, 31], "rand", False, (8, 2)),
]


def pin_bias_grad_autograd():
    """The bias-table gradient equals torch autograd of the dense formulation (window
    pairs of non-global rows listed by brute force), with dilation, globals inside and
    outside the window, padding, the one-sided mode and random blocks (no bias on
    them); the full-problem wrapper sums the slices of every sequence per head."""
    for n, (L, d, w, dil, G, padk, causal, rnd) in enumerate(BIAS_GRAD_CASES):
        q, k, v, do = (_rand((L, d), 1500 + 10 * n + t) for t in range(4))
        beta = _rand((2 * w + 1,), 1509 + 10 * n)
        pad = _pad_for(padk, L, n)
        padl = None if pad is None else pad.tolist()
        bs, draws = 64, None
        if rnd is not None:
            bs = rnd[0]
            draws = _draws(L, bs, rnd[1], n)
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        tb = torch.tensor(beta, requires_grad=True)
        out = _bias_dense_torch(tq, tk, tv, tb, L, w, dil, G, padl, causal, draws, bs)
        (out * torch.from_numpy(do)).sum().backward()
        got = orc.attention_bias_grad_bh(q, k, v, do, w, dil, G, pad, causal=causal, bias=beta, rand=draws,
                                         rand_block=bs)
        err = np.abs(got - tb.grad.numpy()).max()
        assert err < 1e-12, (n, err)
    # wrapper: B = 2 sequences, H = 2 heads, per-sequence padding and dilation per head
    B, H, L, d, w = 2, 2, 24, 8, 3
    dil = [1, 2]
    q, k, v, do = (_rand((B, H, L, d), 1590 + t) for t in range(4))
    beta = _rand((H, 2 * w + 1), 1595)
    pad = np.zeros((B, L), dtype=bool)
    pad[1, 19:] = True
    got = orc.attention_bias_grad(q, k, v, do, w, dil, [2, 15], pad, bias=beta)
    for h in range(H):
        ref = np.zeros(2 * w + 1)
        for b in range(B):
            tb = torch.tensor(beta[h], requires_grad=True)
            out = _bias_dense_torch(*(torch.from_numpy(x[b, h]) for x in (q, k, v)), tb, L, w, dil[h], [2, 15],
                                    pad[b].tolist(), False, None, 64)
            (out * torch.from_numpy(do[b, h])).sum().backward()
            ref += tb.grad.numpy()
        assert np.abs(got[h] - ref).max() < 1e-12, h


def pin_bias_grad_finite_differences():
    """Central differences of sum(O * dO) with respect to each table entry."""
    L, d, w, dil, G = 14, 4, 2, 2, [5]
    q, k, v, do = (_rand((L, d), 1600 + t) for t in range(4))
    beta = _rand((2 * w + 1,), 1605)
    pad = np.zeros(L, dtype=bool)
    pad[[2, 11]] = True
    got = orc.attention_bias_grad_bh(q, k, v, do, w, dil, G, pad, bias=beta)
    eps = 1e-6
    for m in range(2 * w + 1):
        up, dn = beta.copy(), beta.copy()
        up[m] += eps
        dn[m] -= eps
        fd = (float((orc.attention_bh(q, k, v, w, dil, G, pad, bias=up) * do).sum())
              - float((orc.attention_bh(q, k, v, w, dil, G, pad, bias=dn) * do).sum())) / (2 * eps)
        assert abs(fd - got[m]) < 1e-7, (m, fd, got[m])


ALL_PINS = [
    pin_brute_force,
    pin_pair_counts_brute,
    pin_full_attention_limit,
    pin_all_global,
    pin_w0_identity,
    pin_constant_v,
    pin_rows_sum_to_one,
    pin_dilation_residues,
    pin_padding_truncation,
    pin_duplicate_globals,
    pin_global_in_window_counted_once,
    pin_head_permutation,
    pin_dense_counts_golden,
    pin_window_example_golden,
    pin_global_proj_brute,
    pin_global_proj_dependence,
    pin_global_proj_closed_forms,
    pin_global_proj_sampled,
    pin_backward_autograd,
    pin_backward_finite_differences,
    pin_backward_structure,
    pin_backward_invariants,
    pin_lse_brute,
    pin_causal_brute,
    pin_causal_textbook,
    pin_causal_prefix,
    pin_causal_backward_autograd,
    pin_global_sets_per_sequence,
    pin_bias_sdpa,
    pin_bias_shift_and_scope,
    pin_random_brute,
    pin_random_limits,
    pin_random_backward_autograd,
    pin_global_proj_backward_autograd,
    pin_global_proj_backward_reduces,
    pin_wrapper_sampled,
    pin_wrapper_lse,
    pin_wrapper_backward,
    pin_wrapper_backward_global_proj,
    pin_bias_grad_autograd,
    pin_bias_grad_finite_differences,
    pin_layer_torch_encoder,
    pin_layer_norm_rows,
]

"""Plant plausible mistakes in the oracle (on the CPU) and check the pins catch each one.

Every mutant replaces one helper of ``oracle.longformer_oracle`` for the duration of
a test; the brute-force enumerator, the textbook routine and the golden tables are
untouched, so a pin that still passes against a mutant would be blind to that mistake.
"""

import math

import numpy as np
import pytest

from oracle import longformer_oracle as orc
from tests import oracle_pins as P

_orig_window = orc.window_member
_orig_mask = orc.mask_rows
_orig_rows = orc._attention_rows


def _window_strict(i, j, w, dil):  # off by one at the window edge
    diff = j - i
    return (np.abs(diff) < w * dil) & (diff % dil == 0)


def _window_no_lattice(i, j, w, dil):  # dilation span kept, spacing dropped
    diff = j - i
    return np.abs(diff) <= w * dil


def _window_no_span(i, j, w, dil):  # spacing kept, span not stretched by dil
    diff = j - i
    return (np.abs(diff) <= w) & (diff % dil == 0)


def _window_sign(i, j, w, dil):  # one-sided window (a causal reading)
    diff = j - i
    return (diff <= 0) & (-diff <= w * dil) & (diff % dil == 0)


def _causal(m, rows, L, causal):
    if causal:
        m &= np.arange(L)[None, :] <= np.asarray(rows)[:, None]
    return m


def _mask_rows_only(L, w, dil, G, pad_row, rows, causal=False, rand=None, rand_block=64):  # global rows only, no global columns
    rows = np.asarray(rows, dtype=np.int64)
    j = np.arange(L)[None, :]
    isg = np.zeros(L, dtype=bool)
    isg[G] = True
    m = orc.window_member(rows[:, None], j, w, dil) | isg[rows][:, None]
    if rand is not None:
        m |= orc.random_member(rows, L, rand, rand_block)
    if pad_row is not None:
        m &= ~np.asarray(pad_row, dtype=bool)[None, :]
    return _causal(m, rows, L, causal)


def _mask_cols_only(L, w, dil, G, pad_row, rows, causal=False, rand=None, rand_block=64):  # global columns only, no global rows
    rows = np.asarray(rows, dtype=np.int64)
    j = np.arange(L)[None, :]
    isg = np.zeros(L, dtype=bool)
    isg[G] = True
    m = orc.window_member(rows[:, None], j, w, dil) | isg[None, :]
    if rand is not None:
        m |= orc.random_member(rows, L, rand, rand_block)
    if pad_row is not None:
        m &= ~np.asarray(pad_row, dtype=bool)[None, :]
    return _causal(m, rows, L, causal)


def _mask_pad_queries(L, w, dil, G, pad_row, rows, causal=False, rand=None, rand_block=64):  # padding applied to query rows
    m = _orig_mask(L, w, dil, G, None, rows, causal=causal, rand=rand, rand_block=rand_block)
    if pad_row is not None:
        m &= ~np.asarray(pad_row, dtype=bool)[np.asarray(rows)][:, None]
    return m


def _mask_pad_ignored(L, w, dil, G, pad_row, rows, causal=False, rand=None, rand_block=64):
    return _orig_mask(L, w, dil, G, None, rows, causal=causal, rand=rand, rand_block=rand_block)


def _rows_scale_d(q, k, v, m, extra=None):  # 1/d instead of 1/sqrt(d)
    return _orig_rows(q / math.sqrt(q.shape[1]), k, v, m, extra)


def _rows_transposed(q, k, v, m, extra=None):  # S^T = K Q^T used where S = Q K^T was meant
    d = q.shape[1]
    if q.shape[0] != k.shape[0]:
        raise ValueError("transposed scores need a square block")
    s = np.where(m, (k @ q.T) / math.sqrt(d), -np.inf)
    mx = np.max(s, axis=1, keepdims=True)
    ok = np.isfinite(mx)
    e = np.where(m, np.exp(s - np.where(ok, mx, 0.0)), 0.0)
    den = e.sum(axis=1, keepdims=True)
    p = np.where(ok, e / np.where(ok, den, 1.0), 0.0)
    return p @ v, p


def _rows_pk(q, k, v, m, extra=None):  # weights applied to K instead of V
    o, p = _orig_rows(q, k, v, m)
    return p @ k, p


def _rows_zero_fill(q, k, v, m, extra=None):  # out-of-pattern scores left at 0 instead of excluded
    d = q.shape[1]
    s = np.where(m, (q @ k.T) / math.sqrt(d), 0.0)
    e = np.exp(s - s.max(axis=1, keepdims=True))
    p = e / e.sum(axis=1, keepdims=True)
    return p @ v, p


def _rows_nan_empty(q, k, v, m, extra=None):  # no guard for rows without keys
    d = q.shape[1]
    s = np.where(m, (q @ k.T) / math.sqrt(d), -np.inf)
    with np.errstate(invalid="ignore", divide="ignore"):
        e = np.exp(s - s.max(axis=1, keepdims=True))
        p = e / e.sum(axis=1, keepdims=True)
    return p @ v, p


_GP = orc.attention_global_proj


def _gp_uses_k(q, k, v, q_g, k_g, v_g, *a, **kw):  # global rows scored against k, not k_g
    return _GP(q, k, v, q_g, k, v_g, *a, **kw)


def _gp_uses_q(q, k, v, q_g, k_g, v_g, *a, **kw):  # global rows with the window query q
    return _GP(q, k, v, q, k_g, v_g, *a, **kw)


def _gp_uses_v(q, k, v, q_g, k_g, v_g, *a, **kw):  # global rows weight v, not v_g
    return _GP(q, k, v, q_g, k_g, v, *a, **kw)


def _bwd_mutant(kind):
    """attention_backward_bh with one plausible mistake planted."""

    def fn(q, k, v, dout, w, dil, global_idx=None, pad_row=None, causal=False):
        q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dout))
        L, d = q.shape
        G = orc.global_set(global_idx)
        m = orc.mask_rows(L, w, dil, G, pad_row, np.arange(L), causal=causal)
        o, p = orc._attention_rows(q, k, v, m)
        dv = p.T @ do
        dp = do @ v.T
        delta = (do * o).sum(axis=1, keepdims=True)
        if kind == "no_delta":
            ds = p * dp
        elif kind == "delta_from_dp":  # rowsum of dP instead of rowsum(P * dP)
            ds = p * (dp - dp.sum(axis=1, keepdims=True))
        else:
            ds = p * (dp - delta)
        dq = ds @ k / math.sqrt(d)
        dk = ds.T @ q / math.sqrt(d)
        if kind == "dk_unscaled":
            dk = ds.T @ q
        if kind == "dq_from_v":
            dq = ds @ v / math.sqrt(d)
        if kind == "dv_unmasked_softmax":  # dV from weights over every key
            s = (q @ k.T) / math.sqrt(d)
            e = np.exp(s - s.max(axis=1, keepdims=True))
            dv = (e / e.sum(axis=1, keepdims=True)).T @ do
        return dq, dk, dv

    return fn


def _mask_causal_window_only(L, w, dil, G, pad_row, rows, causal=False, rand=None, rand_block=64):  # future global keys kept
    m = _orig_mask(L, w, dil, G, pad_row, rows, causal=causal, rand=rand, rand_block=rand_block)
    if causal:
        rows = np.asarray(rows, dtype=np.int64)
        extra = np.zeros((rows.size, L), dtype=bool)
        extra[:, np.asarray(G, dtype=np.int64)] = True
        if pad_row is not None:
            extra &= ~np.asarray(pad_row, dtype=bool)[None, :]
        m |= extra
    return m


def _mask_causal_strict(L, w, dil, G, pad_row, rows, causal=False, rand=None, rand_block=64):  # self excluded (j < i)
    m = _orig_mask(L, w, dil, G, pad_row, rows, causal=causal, rand=rand, rand_block=rand_block)
    if causal:
        m &= np.arange(L)[None, :] != np.asarray(rows)[:, None]
    return m


_orig_random = orc.random_member


def _random_transposed(rows, L, rand, block):  # row i gets key j when j's block drew i's block
    rows = np.asarray(rows, dtype=np.int64)
    t = _orig_random(np.arange(L), L, rand, block)  # [L, L]: t[j, i] = i in the blocks j's block drew
    return t.T[rows]


def _random_next_block(rows, L, rand, block):  # block kb read as kb + 1
    r = np.asarray(rand, dtype=np.int64)
    return _orig_random(rows, L, np.where(r >= 0, r + 1, r), block)


def _random_first_draw_only(rows, L, rand, block):  # only the first draw of each query block
    return _orig_random(rows, L, np.asarray(rand)[:, :1], block)


def _grads_rows_no_delta(q_rows, k, v, do_rows, m, extra=None):  # dS = P * dP (the D term dropped)
    d = q_rows.shape[1]
    o, p = _orig_rows(q_rows, k, v, m, extra) if extra is not None else _orig_rows(q_rows, k, v, m)
    ds = p * (do_rows @ v.T)
    return ds @ k / math.sqrt(d), ds.T @ q_rows / math.sqrt(d), p.T @ do_rows


from oracle import layer_oracle as _lo  # noqa: E402

_orig_ln = _lo.layer_norm


def _ln_unbiased(y, gamma, beta, eps):  # sample variance (n - 1) instead of the biased one
    mu = y.mean(axis=-1, keepdims=True)
    var = ((y - mu) ** 2).sum(axis=-1, keepdims=True) / (y.shape[-1] - 1)
    return (y - mu) / np.sqrt(var + eps) * gamma + beta


def _gelu_tanh(t):  # the tanh approximation of GELU
    return 0.5 * t * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (t + 0.044715 * t ** 3)))


def _split_interleaved(t, H):  # head h takes every H-th feature
    B, L, E = t.shape
    return t.reshape(B, L, E // H, H).transpose(0, 3, 1, 2)


def _bias_reversed(L, w, dil, G, rows, beta):  # table read backwards (m -> -m)
    return _orig_bias(L, w, dil, G, rows, np.asarray(beta)[::-1])


def _bias_on_global_rows(L, w, dil, G, rows, beta):  # global rows biased too
    return _orig_bias(L, w, dil, np.zeros(0, dtype=np.int64), rows, beta)


_orig_bias = orc.window_bias

# b and h swapped in the per-slice indexing of the full-problem wrappers (one field
# at a time): the padding row, the dilation, the global set, the bias table or the
# random draws of the wrong slice.
def _slice_ix(which, b, h):
    """(pad row, dilation, global set, bias, rand) indices of slice (b, h)."""
    ix = {"pad": b, "dil": h, "glob": b, "bias": h, "rand": h}
    swap = {"pad": h, "dil": b, "glob": h, "bias": b, "rand": b}
    ix[which] = swap[which]
    return ix


def _pad_of(key_pad_mask):
    return None if key_pad_mask is None else np.asarray(orc._as_f64(key_pad_mask) != 0)


def _sampled_swap(which):
    def f(q, k, v, w, dil_per_head, global_idx, key_pad_mask, samples, causal=False, bias=None, rand=None,
          rand_block=64):
        dil = [int(x) for x in np.asarray(dil_per_head).reshape(-1)]
        pad = _pad_of(key_pad_mask)
        res = []
        for b, h, i in samples:
            x = _slice_ix(which, b, h)
            o = orc.attention_bh(q[b, h], k[b, h], v[b, h], w, dil[x["dil"]], orc.globals_of(global_idx, x["glob"]),
                                 None if pad is None else pad[x["pad"]], rows=[i], causal=causal,
                                 bias=None if bias is None else bias[x["bias"]],
                                 rand=None if rand is None else rand[x["rand"]], rand_block=rand_block)
            res.append(o[0])
        return np.stack(res)
    return f


def _lse_swap(which):
    def f(q, k, w, dil_per_head, global_idx=None, key_pad_mask=None, causal=False, bias=None, rand=None,
          rand_block=64):
        q, k = orc._as_f64(q), orc._as_f64(k)
        B, H, L, _ = q.shape
        dil = [int(x) for x in np.asarray(dil_per_head).reshape(-1)]
        pad = _pad_of(key_pad_mask)
        out = np.zeros((B, H, L))
        for b in range(B):
            for h in range(H):
                x = _slice_ix(which, b, h)
                out[b, h] = orc.attention_lse_bh(q[b, h], k[b, h], w, dil[x["dil"]],
                                                 orc.globals_of(global_idx, x["glob"]),
                                                 None if pad is None else pad[x["pad"]], causal=causal,
                                                 bias=None if bias is None else bias[x["bias"]],
                                                 rand=None if rand is None else rand[x["rand"]], rand_block=rand_block)
        return out
    return f


def _bwd_swap(which):
    def f(q, k, v, dout, w, dil_per_head, global_idx=None, key_pad_mask=None, causal=False, bias=None, rand=None,
          rand_block=64):
        q, k, v, do = (orc._as_f64(t) for t in (q, k, v, dout))
        B, H, L, d = q.shape
        dil = [int(x) for x in np.asarray(dil_per_head).reshape(-1)]
        pad = _pad_of(key_pad_mask)
        res = [np.zeros((B, H, L, d)) for _ in range(3)]
        for b in range(B):
            for h in range(H):
                x = _slice_ix(which, b, h)
                parts = orc.attention_backward_bh(q[b, h], k[b, h], v[b, h], do[b, h], w, dil[x["dil"]],
                                                  orc.globals_of(global_idx, x["glob"]),
                                                  None if pad is None else pad[x["pad"]], causal=causal,
                                                  bias=None if bias is None else bias[x["bias"]],
                                                  rand=None if rand is None else rand[x["rand"]],
                                                  rand_block=rand_block)
                for r, t in zip(res, parts):
                    r[b, h] = t
        return tuple(res)
    return f


def _gp_bwd_swap(which):
    def f(q, k, v, q_g, k_g, v_g, dout, w, dil_per_head, global_idx=None, key_pad_mask=None, causal=False,
          bias=None, rand=None, rand_block=64):
        q = orc._as_f64(q)
        B, H, L, d = q.shape
        dil = [int(x) for x in np.asarray(dil_per_head).reshape(-1)]
        pad = _pad_of(key_pad_mask)
        res = [np.zeros((B, H, L, d)) for _ in range(6)]
        for b in range(B):
            for h in range(H):
                x = _slice_ix(which, b, h)
                parts = orc.attention_backward_global_proj_bh(
                    q[b, h], k[b, h], v[b, h], q_g[b, h], k_g[b, h], v_g[b, h], dout[b, h], w, dil[x["dil"]],
                    orc.globals_of(global_idx, x["glob"]), None if pad is None else pad[x["pad"]], causal=causal,
                    bias=None if bias is None else bias[x["bias"]], rand=None if rand is None else rand[x["rand"]],
                    rand_block=rand_block)
                for r, t in zip(res, parts):
                    r[b, h] = t
        return tuple(res)
    return f


_WRAPPERS = {"attention_sampled": _sampled_swap, "attention_lse": _lse_swap,
             "attention_backward": _bwd_swap, "attention_backward_global_proj": _gp_bwd_swap}


def _bias_grad_mutant(kind):
    """attention_bias_grad_bh with one plausible mistake."""
    def f(q, k, v, dout, w, dil, global_idx=None, pad_row=None, causal=False, bias=None, rand=None, rand_block=64):
        q, k, v, do = (orc._as_f64(t) for t in (q, k, v, dout))
        L = q.shape[0]
        G = orc.global_set(global_idx)
        is_g = np.zeros(L, dtype=bool)
        is_g[G] = True
        beta = np.zeros(2 * w + 1) if bias is None else np.asarray(bias, dtype=np.float64)
        db = np.zeros(2 * w + 1)
        blk = np.arange(L)
        m = orc.mask_rows(L, w, dil, G, pad_row, blk, causal=causal, rand=rand, rand_block=rand_block)
        o, p = orc._attention_rows(q, k, v, m, orc.window_bias(L, w, dil, G, blk, beta))
        dp = do @ v.T
        delta = 0.0 if kind == "no_delta" else (do * o).sum(axis=1, keepdims=True)
        ds = p * (dp - delta)
        j = np.arange(L)[None, :]
        win = orc.window_member(blk[:, None], j, w, dil) & m
        if kind != "global_rows":
            win &= ~is_g[:, None]
        idx = (j - blk[:, None]) // dil + w
        if kind == "reversed":
            idx = 2 * w - idx
        np.add.at(db, idx[win], ds[win])
        return db
    return f


MUTANTS = {
    "window_strict_edge": ("window_member", _window_strict),
    "window_no_lattice": ("window_member", _window_no_lattice),
    "window_span_not_dilated": ("window_member", _window_no_span),
    "window_one_sided": ("window_member", _window_sign),
    "global_rows_only": ("mask_rows", _mask_rows_only),
    "global_cols_only": ("mask_rows", _mask_cols_only),
    "pad_on_queries": ("mask_rows", _mask_pad_queries),
    "pad_ignored": ("mask_rows", _mask_pad_ignored),
    "causal_future_globals": ("mask_rows", _mask_causal_window_only),
    "causal_excludes_self": ("mask_rows", _mask_causal_strict),
    "scale_1_over_d": ("_attention_rows", _rows_scale_d),
    "transposed_scores": ("_attention_rows", _rows_transposed),
    "weights_times_k": ("_attention_rows", _rows_pk),
    "zero_fill_softmax": ("_attention_rows", _rows_zero_fill),
    "nan_empty_rows": ("_attention_rows", _rows_nan_empty),
    "global_proj_uses_k": ("attention_global_proj", _gp_uses_k),
    "global_proj_uses_q": ("attention_global_proj", _gp_uses_q),
    "global_proj_uses_v": ("attention_global_proj", _gp_uses_v),
    "bias_reversed": ("window_bias", _bias_reversed),
    "bias_on_global_rows": ("window_bias", _bias_on_global_rows),
    "random_transposed": ("random_member", _random_transposed),
    "random_next_block": ("random_member", _random_next_block),
    "random_first_draw_only": ("random_member", _random_first_draw_only),
    "gp_bwd_no_delta": ("_grads_rows", _grads_rows_no_delta),
    "layer_ln_unbiased": ("layer:layer_norm", _ln_unbiased),
    "layer_gelu_tanh": ("layer:gelu", _gelu_tanh),
    "layer_heads_interleaved": ("layer:split_heads", _split_interleaved),
    "bwd_no_delta": ("attention_backward_bh", _bwd_mutant("no_delta")),
    "bwd_delta_from_dp": ("attention_backward_bh", _bwd_mutant("delta_from_dp")),
    "bwd_dk_unscaled": ("attention_backward_bh", _bwd_mutant("dk_unscaled")),
    "bwd_dq_from_v": ("attention_backward_bh", _bwd_mutant("dq_from_v")),
    "bwd_dv_unmasked": ("attention_backward_bh", _bwd_mutant("dv_unmasked_softmax")),
}
for _kind in ("no_delta", "global_rows", "reversed"):
    MUTANTS[f"bias_grad_{_kind}"] = ("attention_bias_grad_bh", _bias_grad_mutant(_kind))
for _fn, _make in _WRAPPERS.items():
    for _field in ("pad", "dil", "glob", "bias", "rand"):
        MUTANTS[f"{_fn}_swap_{_field}"] = (_fn, _make(_field))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    if attr.startswith("layer:"):
        monkeypatch.setattr(_lo, attr[len("layer:"):], fn)
    else:
        monkeypatch.setattr(orc, attr, fn)
    caught = []
    for pin in P.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
            break
    assert caught, f"no pin detects mutant {name}"

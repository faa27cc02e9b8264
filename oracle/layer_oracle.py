"""Plain fp64 CPU oracle of one Longformer layer around the sparse attention.

TEST INFRASTRUCTURE ONLY (see ``oracle/longformer_oracle.py``): only the test
suite and the bench's CPU leg use it; it shares no code with the HIP library.

The layer (post-LayerNorm transformer block; the page "基于自注意力机制的长文本建模
算法：Longformer详解" §6 starts Longformer from RoBERTa's weights, so its layers are
RoBERTa's with the self-attention replaced; page "基于Block-Sparse Attention的
Longformer" §6 shows the same order: attention, residual, LayerNorm, feed-forward,
residual, LayerNorm), for x [B, L, E] with E = H * 64:

    q, k, v = split_heads(x W_qkv^T + b_qkv)          # rows of W_qkv: q, then k, then v
    a       = merge_heads(attention(q, k, v))         # the window + global attention
    x1      = LN1(x + a W_o^T + b_o)
    out     = LN2(x1 + GELU(x1 W_1^T + b_1) W_2^T + b_2)

LN(y) = (y - mean(y)) / sqrt(var(y) + eps) * gamma + beta over the last axis
(biased variance); GELU(t) = t * Phi(t) = 0.5 t (1 + erf(t / sqrt(2))).
Head h of q, k, v holds features 64h .. 64h + 63.  Everything is computed in
float64 from the given (already rounded) inputs and weights.
"""

from __future__ import annotations

import math

import numpy as np

from . import longformer_oracle as orc

WEIGHT_NAMES = ("w_qkv", "b_qkv", "w_o", "b_o", "ln1_g", "ln1_b", "w_1", "b_1", "w_2", "b_2", "ln2_g", "ln2_b")


def _f64(x):
    return orc._as_f64(x)


def layer_norm(y, gamma, beta, eps: float):
    """Normalise over the last axis with the biased variance, then scale and shift."""
    mu = y.mean(axis=-1, keepdims=True)
    var = ((y - mu) ** 2).mean(axis=-1, keepdims=True)
    return (y - mu) / np.sqrt(var + eps) * gamma + beta


def gelu(t):
    """t * Phi(t), with the standard normal CDF written through erf."""
    erf = np.vectorize(math.erf)
    return 0.5 * t * (1.0 + erf(t / math.sqrt(2.0)))


def split_heads(t, H: int):
    """[B, L, H*d] -> [B, H, L, d] (head h = features d*h .. d*h + d - 1)."""
    B, L, E = t.shape
    return t.reshape(B, L, H, E // H).transpose(0, 2, 1, 3)


def merge_heads(t):
    """[B, H, L, d] -> [B, L, H*d]."""
    B, H, L, d = t.shape
    return t.transpose(0, 2, 1, 3).reshape(B, L, H * d)


def layer_forward(x, weights: dict, H: int, w: int, dil_per_head, global_idx=None, key_pad_mask=None,
                  eps: float = 1e-5, causal: bool = False, bias=None, rand=None):
    """One layer on x [B, L, E]; ``weights`` maps WEIGHT_NAMES to arrays (nn.Linear
    layout: weight [out, in]); ``bias``: the attention's relative position bias
    ([H, 2w + 1]) or None; ``rand``: its random key blocks ([H, n_blocks, r]) or None.
    Returns float64 [B, L, E]."""
    x = _f64(x)
    W = {k: _f64(v) for k, v in weights.items()}
    E = x.shape[-1]
    qkv = x @ W["w_qkv"].T + W["b_qkv"]
    q, k, v = (split_heads(qkv[..., i * E:(i + 1) * E], H) for i in range(3))
    a = merge_heads(orc.attention(q, k, v, w, dil_per_head, global_idx, key_pad_mask, causal=causal,
                                    bias=bias, rand=rand))
    x1 = layer_norm(x + a @ W["w_o"].T + W["b_o"], W["ln1_g"], W["ln1_b"], eps)
    f = gelu(x1 @ W["w_1"].T + W["b_1"]) @ W["w_2"].T + W["b_2"]
    return layer_norm(x1 + f, W["ln2_g"], W["ln2_b"], eps)

"""One transformer layer applied to a block of masked positions.

A denoising round runs every position of the block through the model; block
queries see the whole prefix KV cache and every key of their own block, with
no mask inside the block ([ORL-blog] "What shipped": generation proceeds in
blocks whose still-unresolved tokens are predicted together; [ORL-card] "The
paper's evaluation pipeline": block decoding against a prefix KV cache).

Readings where the pages are silent (each one the plainest the rest supports):
  * pre-norm decoder layer: RMSNorm, no biases, no QK-norm, eps = 1e-6, gains 1;
  * RoPE in its rotate-half form, pairs (j, j + D/2), theta_j = pos * base^(-2j/D),
    base 1e4, at absolute positions;
  * grouped-query attention: query head h uses kv head floor(h / (Hq/Hkv)),
    softmax scale 1/sqrt(D);
  * SwiGLU FFN: down(silu(gate f) * up f).
All are pinned by tests/test_oracle_block.py (brute force and invariants).
"""
from __future__ import annotations

import numpy as np

from .numerics import Prec


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * g along the last axis."""
    ms = (x * x).mean(axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def rope(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotate-half rotary embedding of x [..., n, H, D] at positions pos [n].

    Pair (j, j + D/2) is rotated by the angle pos * base^(-2j/D).  The angle is
    formed in float64 whatever the compute type.
    """
    D = x.shape[-1]
    half = D // 2
    j = np.arange(half, dtype=np.float64)
    inv = base ** (-2.0 * j / D)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]      # [n, D/2]
    c = np.cos(ang)[:, None, :].astype(x.dtype)
    s = np.sin(ang)[:, None, :].astype(x.dtype)
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Block attention with every key visible.

    q [B, Hq, D]; k, v [Hkv, N, D] (the N keys: prefix followed by the block).
    Returns o [B, Hq, D] with o[i, h] = softmax_j(scale * q[i,h].k[g,j]) v[g, j],
    g = h // (Hq // Hkv).
    """
    B, Hq, D = q.shape
    Hkv = k.shape[0]
    group = Hq // Hkv
    o = np.empty_like(q)
    for h in range(Hq):
        g = h // group
        s = (q[:, h, :] @ k[g].T) * scale          # [B, N]
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        o[:, h, :] = p @ v[g]
    return o


def swiglu(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    return gate / (1.0 + np.exp(-gate)) * up


def attention_sublayer(x, lw, kc, vc, L, shape, prec: Prec, pos=None):
    """Pre-norm attention with residual; writes this block's K/V into the cache.

    x [B, d] residual stream; kc/vc [Hkv, cap, D] caches (modified in place at
    rows [L, L+B)); returns x + o Wo^T.
    """
    B = x.shape[0]
    Hq, Hkv, D = shape.hq, shape.hkv, shape.head_dim
    if pos is None:
        pos = np.arange(L, L + B)
    a = prec.act(rmsnorm(x, lw["attn_norm"], shape.eps))
    q = (a @ lw["wq"].T).reshape(B, Hq, D)
    k = (a @ lw["wk"].T).reshape(B, Hkv, D)
    v = (a @ lw["wv"].T).reshape(B, Hkv, D)
    q = prec.act(rope(q, pos, shape.rope_base))
    k = prec.act(rope(k, pos, shape.rope_base))
    v = prec.act(v)
    kc[:, L:L + B, :] = prec.kv_store(k, 0).transpose(1, 0, 2)
    vc[:, L:L + B, :] = prec.kv_store(v, 1).transpose(1, 0, 2)
    o = attention(q, kc[:, :L + B, :], vc[:, :L + B, :], 1.0 / np.sqrt(D))
    o = prec.act(o.reshape(B, Hq * D))
    return x + o @ lw["wo"].T


def dense_ffn_sublayer(h, lw, shape, prec: Prec):
    f = prec.act(rmsnorm(h, lw["ffn_norm"], shape.eps))
    act = prec.act(swiglu(f @ lw["wg"].T, f @ lw["wu"].T))
    return h + act @ lw["wd"].T


def dense_layer(x, lw, kc, vc, L, shape, prec: Prec):
    h = attention_sublayer(x, lw, kc, vc, L, shape, prec)
    return dense_ffn_sublayer(h, lw, shape, prec)


def forward_block(model, x, kv, L, prec: Prec, skip_last_ffn: bool = False):
    """Run the block's residual stream x [B, d] through every layer.

    kv: KVCache; each layer's block K/V is written at [L, L+B).  With
    skip_last_ffn the last layer stops after writing its K/V (used by the
    commit pass, whose last-layer output feeds nothing).
    """
    from .moe import moe_ffn_sublayer
    shape = model.shape
    h = x
    for i in range(shape.n_layers):
        lw = model.layer(i)
        last = i == shape.n_layers - 1
        if skip_last_ffn and last:
            attention_sublayer(h, lw, kv.k[i], kv.v[i], L, shape, prec)
            return None
        h = attention_sublayer(h, lw, kv.k[i], kv.v[i], L, shape, prec)
        if shape.moe:
            h = moe_ffn_sublayer(h, model, i, prec)
        else:
            h = dense_ffn_sublayer(h, lw, shape, prec)
    return h

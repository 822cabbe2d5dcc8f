"""Routed-expert FFN with 4-bit expert weights (the MoE model's FFN).

The pages run routed experts in 4-bit floating point on the GPU's FP4 matrix
units ([ORL-blog] "What shipped": routed experts in NVFP4 on FP4 tensor cores;
[ORL-news] on the MoE results).  The MI355X reading uses the OCP
Microscaling formats instead of NVFP4:
  * expert weights MXFP4: e2m1 elements, one e8m0 power-of-two scale per 32
    consecutive elements along the input axis;
  * activations MXFP8: e4m3 elements with an e8m0 scale per 32 along the
    contraction axis, scale exponent floor(log2(amax)) - 8 (e4m3's largest
    exponent is 8), elements rounded to nearest-even and saturated at 448;
  * router: r = f W_r^T from the bf16 normed hidden state, softmax over all
    experts, top-k by (probability desc, expert id asc), the selected
    probabilities used as mixing weights without renormalisation; shared
    experts always added with weight 1.
Every e2m1 x 2^e value is exact in float64, so the oracle decodes weights
exactly.  Pinned by tests/test_oracle_moe.py (format tables, round trips, a
top-k equal to all experts reducing to a dense mixture, one-hot routing) and by
tests/test_oracle_moe_expert.py: one expert and the whole sublayer (norm,
router, top-k, shared expert, residual) against scalar-loop brute force with an
independently enumerated e4m3 table, on MXFP4-exact weights; the same checks
reject copies with gate and up swapped, the activation re-quantisation dropped,
the shared expert dropped or the norm gain ignored.
"""
from __future__ import annotations

import numpy as np

from .numerics import Prec
from .block import rmsnorm, swiglu

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def mxfp4_decode(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Decode MXFP4 [..., K/2] bytes (element 2j in the low nibble) and
    [..., K/32] e8m0 scales to float64 [..., K]."""
    packed = np.asarray(packed, dtype=np.uint8)
    lo = packed & 0x0F
    hi = packed >> 4
    codes = np.stack([lo, hi], axis=-1).reshape(packed.shape[:-1] + (packed.shape[-1] * 2,))
    mag = E2M1[codes & 0x7]
    val = np.where(codes & 0x8, -mag, mag)
    sc = np.exp2(np.asarray(scales, dtype=np.float64) - 127.0)
    K = val.shape[-1]
    val = val.reshape(val.shape[:-1] + (K // 32, 32)) * sc[..., None]
    return val.reshape(val.shape[:-2] + (K,))


def e4m3_round(v: np.ndarray) -> np.ndarray:
    """Nearest-even e4m3 (OCP, bias 7, 3 mantissa bits, max 448, subnormals
    down to 2^-9), saturating; float64 in and out."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)                      # below 2^-6 the spacing stays 2^-9
    quantum = np.exp2(e - 3.0)
    q = np.round(a / quantum) * quantum          # np.round: halves to even
    q = np.minimum(q, 448.0)
    return np.where(v < 0, -q, q)


def mxfp8_quant_dequant(x: np.ndarray) -> np.ndarray:
    """Quantise [..., K] to MXFP8 (e4m3 + e8m0 per 32 along K) and decode back."""
    x = np.asarray(x, dtype=np.float64)
    K = x.shape[-1]
    blk = x.reshape(x.shape[:-1] + (K // 32, 32))
    amax = np.abs(blk).max(axis=-1)
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 8.0, -127.0)
    e = np.clip(e, -127.0, 127.0)
    sc = np.exp2(e)[..., None]
    q = e4m3_round(blk / sc) * sc
    return q.reshape(x.shape)


def router_topk(f: np.ndarray, w_router: np.ndarray, top_k: int):
    """Softmax routing: returns (expert ids [R, k], weights [R, k], probs [R, E])
    with ids ordered by (prob desc, id asc)."""
    r = f @ w_router.T
    r = r - r.max(axis=1, keepdims=True)
    p = np.exp(r)
    p = p / p.sum(axis=1, keepdims=True)
    E = p.shape[1]
    ids = np.empty((p.shape[0], top_k), np.int64)
    for i in range(p.shape[0]):
        order = sorted(range(E), key=lambda e: (-p[i, e], e))
        ids[i] = order[:top_k]
    w = np.take_along_axis(p, ids, axis=1)
    return ids, w, p


def expert_ffn(xq: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray) -> np.ndarray:
    """One expert on MXFP8-quantised inputs xq [R, d] with decoded weights."""
    act = swiglu(xq @ wg.T, xq @ wu.T)
    return mxfp8_quant_dequant(act) @ wd.T


def moe_ffn(f: np.ndarray, w_router: np.ndarray, experts, shared, top_k: int):
    """y = sum over the top-k experts of p_e * expert_e(f) + sum of shared experts.

    f [R, d] bf16-valued normed hidden; experts(e) -> (wg, wu, wd) decoded
    float64 matrices; shared: list of (wg, wu, wd).  Returns (y, ids, weights).
    """
    ids, w, _ = router_topk(f, w_router, top_k)
    xq = mxfp8_quant_dequant(f)
    y = np.zeros_like(f)
    for i in range(f.shape[0]):
        for j in range(top_k):
            wg, wu, wd = experts(int(ids[i, j]))
            y[i] += w[i, j] * expert_ffn(xq[i:i + 1], wg, wu, wd)[0]
    for (wg, wu, wd) in shared:
        y += expert_ffn(xq, wg, wu, wd)
    return y, ids, w


def moe_ffn_sublayer(h, model, layer: int, prec: Prec):
    """h + MoE(RMSNorm(h)) for layer `layer` of a MoE OracleModel."""
    s = model.shape
    f = prec.act(rmsnorm(h, model.get(f"l{layer}.ffn_norm"), s.eps))
    cache = {}

    def dec(e):
        if e not in cache:
            mats = []
            for which in ("wg", "wu", "wd"):
                pk, sc = model.src.expert(layer, e, which)
                mats.append(mxfp4_decode(pk, sc).astype(prec.compute))
            cache[e] = tuple(mats)
        return cache[e]

    shared = [dec(s.n_experts + j) for j in range(s.n_shared)]
    y, _, _ = moe_ffn(f, model.get(f"l{layer}.router"), dec, shared, s.top_k)
    return h + y

"""FP8 KV cache: keys and values stored as e4m3 codes with one scale per cache.

[ORL-blog] "What shipped" states that the engine keeps its KV cache in FP8 on
Blackwell; [ORL-card] "The paper's evaluation pipeline" decodes blocks against
a prefix KV cache.  No element format or scaling is given.  The reading taken
here is the plainest one: every stored K (V) element
is an OCP FP8 e4m3 code (bias 7, 3 mantissa bits, subnormals down to 2^-9,
largest finite 448, codes 0x7F / 0xFF NaN, no infinities), and the cache as a
whole has one float scale, k_scale (v_scale), so that the stored key is
k_scale * e4m3(code).  Attention then runs on the decoded keys and values
exactly as in the bf16 cache.

Pinned by tests/test_oracle_kvcache.py: the code table against values of the
format definition (tests/golden/mx_formats.json), decode against the
independently written nearest-even rounding (every finite code is a fixed point
of it, and the codes are ordered), the encoder as its inverse on every finite
code and its nearest-even ties, and the attention against the float64 oracle
attention on decoded caches, including the closed forms of the two scales.
"""
from __future__ import annotations

import numpy as np

from .block import attention
from .moe import e4m3_round


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """float64 values of e4m3 codes (uint8), from the format's bit fields."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """e4m3 codes of v: nearest-even rounding, saturating at 448 (NaN stays NaN)."""
    v = np.asarray(v, dtype=np.float64)
    q = e4m3_round(np.nan_to_num(v, nan=0.0))
    a = np.abs(q)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    sub = a < 2.0 ** -6
    m_sub = np.round(a / 2.0 ** -9)
    m_nrm = np.round((a / np.exp2(e) - 1.0) * 8.0)
    mag = np.where(sub, m_sub, ((e + 7.0) * 8.0) + m_nrm).astype(np.int64)
    code = (np.where(np.signbit(q), 0x80, 0) | mag).astype(np.uint8)
    return np.where(np.isnan(v), np.uint8(0x7F), code)


def attention_fp8_cache(q: np.ndarray, k_codes: np.ndarray, v_codes: np.ndarray, k_scale: float, v_scale: float,
                        scale: float) -> np.ndarray:
    """Block attention over an FP8 cache: q [B, Hq, D] (float), k_codes / v_codes [Hkv, N, D]
    uint8 e4m3 codes of the N visible keys, stored values k_scale * e4m3(code) and
    v_scale * e4m3(code)."""
    k = k_scale * e4m3_decode(k_codes)
    v = v_scale * e4m3_decode(v_codes)
    return attention(np.asarray(q, dtype=np.float64), k, v, scale)

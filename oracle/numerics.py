"""Storage-format helpers of the oracle (its own code; shares nothing with the library)."""
from __future__ import annotations

import dataclasses

import numpy as np


def _f64_to_f32_rne(x: np.ndarray) -> np.ndarray:
    # numpy's float64 -> float32 cast rounds to nearest-even.
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round to bf16 the way the GPU stores an activation: the value is first
    an fp32 number (nearest-even from float64), then rounded to the nearest
    bf16 (ties to even).  Returned in float64."""
    f = _f64_to_f32_rne(x)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    nan = np.isnan(f)
    out = r.astype(np.uint32).view(np.float32).astype(np.float64)
    if nan.any():
        out[nan] = np.nan
    return out


def decode_storage(a: np.ndarray, dtype=np.float64) -> np.ndarray:
    """A stored tensor (float32 values, or uint16 bf16 bit patterns) as floats."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(dtype)
    return a.astype(dtype)


@dataclasses.dataclass(frozen=True)
class Prec:
    """Numerics of one oracle run.

    storage: "f32" (every tensor an fp32 value, no activation rounding) or
             "bf16" (activations rounded to bf16 at the library's storage points).
    compute: np.float64 for parity, np.float32 for the CPU timing baseline.
    kv_scales: None (the KV cache holds the stored k and v), or (k_scale, v_scale) for an
             FP8 cache: the cache then holds scale * e4m3(value / scale), the value being the
             bf16 k (v) after RoPE, rounded to nearest-even e4m3 with saturation (NaN stays
             NaN), the quotient value / scale being the single-precision quotient of the
             stored bf16 value and the single-precision scale (the scale is a float of the
             cache format; oracle/kvcache.py states the format reading).
    """
    storage: str = "f32"
    compute: type = np.float64
    kv_scales: tuple | None = None

    def kv_store(self, x: np.ndarray, which: int) -> np.ndarray:
        """What the KV cache holds for the stored keys (which = 0) or values (which = 1)."""
        if self.kv_scales is None:
            return x
        from .moe import e4m3_round
        s = np.float32(self.kv_scales[which])
        quot = (np.asarray(x, dtype=np.float64).astype(np.float32) / s).astype(np.float64)
        return (float(s) * e4m3_round(quot)).astype(self.compute, copy=False)

    def act(self, x: np.ndarray) -> np.ndarray:
        """Round an activation at a storage point."""
        if self.storage == "bf16":
            return bf16_round(x).astype(self.compute, copy=False)
        return np.asarray(x, dtype=self.compute)

    def w(self, stored: np.ndarray) -> np.ndarray:
        return decode_storage(stored, self.compute)

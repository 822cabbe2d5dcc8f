"""Seeded synthetic inputs for the block-diffusion denoising round.

This module only draws random numbers and encodes them in the storage formats
the library consumes (fp32, bf16 bit patterns, MXFP4 bytes).  It holds no step
of the decoding method itself, so both the CPU oracle and the GPU path can take
their inputs from here without sharing any of the method's arithmetic.

Generator: numpy ``PCG64`` seeded with ``SeedSequence(seed, spawn_key=(crc32(name),
chunk))``.  Every tensor is identified by a stable string name; big tensors are
drawn in chunks of ``CHUNK`` elements, each chunk from its own child stream, so
they can be drawn in parallel and the bytes do not depend on the thread count.
Normal draws use numpy's float32 ziggurat, are scaled by ``std`` in float32,
and bf16 tensors are then rounded to nearest-even from those float32 values.
"""
from __future__ import annotations

import dataclasses
import os
import zlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 22
_THREADS = max(1, min(16, os.cpu_count() or 1))


# --------------------------------------------------------------------------
# model shapes (the workloads the pages measure, at random init)
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class ModelShape:
    name: str
    n_layers: int
    d: int
    hq: int
    hkv: int
    head_dim: int
    ffn: int            # dense FFN width (0 for MoE layers)
    vocab: int
    dtype: str          # "f32" or "bf16" storage of weights and activations
    block: int = 32
    rope_base: float = 1e4
    eps: float = 1e-6
    n_experts: int = 0
    expert_ffn: int = 0
    top_k: int = 0
    n_shared: int = 0
    std: float = 0.02

    @property
    def moe(self) -> bool:
        return self.n_experts > 0


TINY = ModelShape("tiny-fp32", n_layers=2, d=256, hq=4, hkv=2, head_dim=64, ffn=768,
                  vocab=4096, dtype="f32")
QWEN4B = ModelShape("qwen3-4b-shaped", n_layers=36, d=2560, hq=32, hkv=8, head_dim=128,
                    ffn=9728, vocab=151936, dtype="bf16")
MOE16B = ModelShape("moe-16b-a1b", n_layers=20, d=2048, hq=16, hkv=4, head_dim=128, ffn=0,
                    vocab=157184, dtype="bf16", n_experts=256, expert_ffn=512, top_k=8,
                    n_shared=1)

SHAPES = {s.name: s for s in (TINY, QWEN4B, MOE16B)}
SEEDS = (1234, 1235, 1236)


def small_shape(base: ModelShape, **kw) -> ModelShape:
    """A reduced copy of a shape (for tests that must finish in seconds)."""
    return dataclasses.replace(base, **kw)


# --------------------------------------------------------------------------
# raw draws
# --------------------------------------------------------------------------
def _ss(seed: int, name: str, chunk: int) -> np.random.Generator:
    key = zlib.crc32(name.encode("utf-8"))
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(key, chunk))))


def _chunks(n: int):
    return [(c, c * CHUNK, min(n, (c + 1) * CHUNK)) for c in range((n + CHUNK - 1) // CHUNK)]


def normal_f32(seed: int, name: str, shape, std: float = 1.0) -> np.ndarray:
    """float32 N(0, std^2) draws of the given shape."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.float32)
    s32 = np.float32(std)

    def fill(args):
        c, a, b = args
        out[a:b] = _ss(seed, name, c).standard_normal(b - a, dtype=np.float32) * s32

    parts = _chunks(n)
    if len(parts) > 1:
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(fill, parts))
    else:
        for p in parts:
            fill(p)
    return out.reshape(shape)


def uniform_ints(seed: int, name: str, n: int, high: int) -> np.ndarray:
    """int32 ids uniform in [0, high)."""
    return _ss(seed, name, 0).integers(0, high, size=n, dtype=np.int64).astype(np.int32)


def e4m3_codes(seed: int, name: str, shape, max_mag_code: int = 0x4F) -> np.ndarray:
    """uint8 FP8 e4m3 codes: a random sign bit over magnitude codes drawn uniformly from
    [0, max_mag_code] (0x4F is 7.5; the NaN codes 0x7F / 0xFF are never drawn)."""
    n = int(np.prod(shape))
    r = _ss(seed, name, 0)
    mag = r.integers(0, max_mag_code + 1, size=n, dtype=np.int64)
    sgn = r.integers(0, 2, size=n, dtype=np.int64) << 7
    return (mag | sgn).astype(np.uint8).reshape(shape)


def permutation(seed: int, name: str, n: int) -> np.ndarray:
    return _ss(seed, name, 0).permutation(n).astype(np.int32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest-even) and return the 16-bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def stored_normal(seed: int, name: str, shape, std: float, dtype: str) -> np.ndarray:
    """A normal tensor in its storage format: float32 array or uint16 bf16 bits."""
    x = normal_f32(seed, name, shape, std)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# MXFP4 storage (OCP Microscaling v1.0: e2m1 elements, e8m0 scale per 32)
# --------------------------------------------------------------------------
_E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def encode_mxfp4(x: np.ndarray):
    """Encode a [..., K] float32 array as MXFP4 along its last axis.

    Per block of 32 elements: shared exponent e = floor(log2(amax)) - 2 (the
    e2m1 maximum exponent is 2), stored as the e8m0 byte e + 127 (an all-zero
    block stores 0); each element x / 2^e is rounded to the nearest e2m1 value
    (ties to the even code), magnitudes above 6 saturate to 6.  Two codes per
    byte: element 2j in the low nibble, element 2j+1 in the high nibble; the
    code is sign << 3 | magnitude index.  Returns (packed uint8 [..., K/2],
    scales uint8 [..., K/32]).  This is checkpoint encoding of synthetic
    weights, not a step of the decode.
    """
    x = np.asarray(x, dtype=np.float32)
    K = x.shape[-1]
    assert K % 32 == 0
    blk = x.astype(np.float64).reshape(x.shape[:-1] + (K // 32, 32))
    amax = np.abs(blk).max(axis=-1)
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, -127)
    e = np.clip(e, -127, 127)
    scaled = blk / np.exp2(e)[..., None]
    mag = np.minimum(np.abs(scaled), 6.0)
    # nearest grid point, ties to the even index (even index == even mantissa bit): the number
    # of midpoints below mag is the lower neighbour's index; a value exactly on a midpoint
    # between an odd and an even index moves to the even one
    mids = (_E2M1_GRID[1:] + _E2M1_GRID[:-1]) / 2
    idx = np.searchsorted(mids, mag, side="left")
    on_mid = mag == mids[np.minimum(idx, len(mids) - 1)]
    idx = np.where(on_mid & (idx % 2 == 1), idx + 1, idx)
    sign = (scaled < 0) & (idx > 0)
    code = (sign.astype(np.uint8) << 3) | idx.astype(np.uint8)
    code = code.reshape(x.shape[:-1] + (K,))
    packed = (code[..., 0::2] | (code[..., 1::2] << 4)).astype(np.uint8)
    scales = (e + 127).astype(np.uint8)
    return packed, scales


# --------------------------------------------------------------------------
# model weights
# --------------------------------------------------------------------------
class Weights:
    """Lazily drawn random-init weights of one model, in storage format.

    Dense matrices use the [out, in] convention.  Norm gains are ones.  Names:
    ``emb`` [V,d], ``mask_emb`` [d], ``w_sc`` [d,d], ``final_norm`` [d];
    per layer ``l{i}.attn_norm``, ``l{i}.wq`` [Hq*D,d], ``l{i}.wk``/``l{i}.wv``
    [Hkv*D,d], ``l{i}.wo`` [d,Hq*D], ``l{i}.ffn_norm``; dense FFN ``l{i}.wg``/
    ``l{i}.wu`` [F,d], ``l{i}.wd`` [d,F]; MoE ``l{i}.router`` [E,d] (bf16) and
    expert FFNs ``l{i}.x{e}.{wg,wu,wd}`` (e = expert id, shared experts use ids
    E..E+n_shared-1) as MXFP4 (packed, scales) pairs along the input axis.
    """

    def __init__(self, shape: ModelShape, seed: int = 1234, cache: bool = True):
        self.shape = shape
        self.seed = seed
        self._cache = {} if cache else None

    def _get(self, name, fn):
        if self._cache is None:
            return fn()
        if name not in self._cache:
            self._cache[name] = fn()
        return self._cache[name]

    def names_dense(self):
        s = self.shape
        out = ["emb", "mask_emb", "w_sc", "final_norm"]
        for i in range(s.n_layers):
            out += [f"l{i}.{n}" for n in ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm")]
            if not s.moe:
                out += [f"l{i}.{n}" for n in ("wg", "wu", "wd")]
            else:
                out += [f"l{i}.router"]
        return out

    def shape_of(self, name: str):
        s = self.shape
        base = name.split(".")[-1]
        table = {
            "emb": (s.vocab, s.d), "mask_emb": (s.d,), "w_sc": (s.d, s.d), "final_norm": (s.d,),
            "attn_norm": (s.d,), "ffn_norm": (s.d,), "wq": (s.hq * s.head_dim, s.d),
            "wk": (s.hkv * s.head_dim, s.d), "wv": (s.hkv * s.head_dim, s.d),
            "wo": (s.d, s.hq * s.head_dim), "router": (s.n_experts, s.d),
        }
        if ".x" in name:
            f = s.expert_ffn
            return {"wg": (f, s.d), "wu": (f, s.d), "wd": (s.d, f)}[base]
        if base in ("wg", "wu"):
            return (s.ffn, s.d)
        if base == "wd":
            return (s.d, s.ffn)
        return table[base]

    def __getitem__(self, name: str) -> np.ndarray:
        s = self.shape
        base = name.split(".")[-1]
        shp = self.shape_of(name)
        if base.endswith("norm"):
            one = np.ones(shp, dtype=np.float32)
            return self._get(name, lambda: one if s.dtype == "f32" else f32_to_bf16_bits(one))
        if ".x" in name:
            raise KeyError("expert weights are read with expert()")
        return self._get(name, lambda: stored_normal(self.seed, name, shp, s.std, s.dtype))

    def expert(self, layer: int, e: int, which: str):
        """(packed uint8, scales uint8) MXFP4 of one expert matrix."""
        name = f"l{layer}.x{e}.{which}"
        shp = self.shape_of(name)
        return self._get(name, lambda: encode_mxfp4(normal_f32(self.seed, name, shp, self.shape.std)))

    def expert_stack(self, layer: int, which: str):
        """All routed + shared experts of one layer stacked: packed [E+S, out, in/2], scales [E+S, out, in/32]."""
        s = self.shape
        n = s.n_experts + s.n_shared
        parts = [self.expert(layer, e, which) for e in range(n)]
        return np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts])


# --------------------------------------------------------------------------
# op-level inputs
# --------------------------------------------------------------------------
def prompt_ids(shape: ModelShape, n: int, seed: int = 1234) -> np.ndarray:
    return uniform_ints(seed, "prompt", n, shape.vocab)


def unit_rms_rows(seed: int, name: str, rows: int, d: int) -> np.ndarray:
    """float32 rows drawn N(0,1) and then scaled to root-mean-square 1 (rows on
    the sphere of radius sqrt(d)); the distribution of hidden states after a
    unit-gain RMS normalisation."""
    x = normal_f32(seed, name, (rows, d), 1.0).astype(np.float64)
    x = x / np.sqrt((x * x).mean(axis=1, keepdims=True))
    return x.astype(np.float32)


def committed_mask(seed: int, rows: int, n_committed: int) -> np.ndarray:
    """uint8 mask with exactly n_committed ones at seeded-permutation positions."""
    m = np.zeros(rows, dtype=np.uint8)
    m[permutation(seed, "committed", rows)[:n_committed]] = 1
    return m

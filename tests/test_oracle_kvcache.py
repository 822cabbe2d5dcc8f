"""Pins of the oracle's FP8 (e4m3) KV cache: code table, rounding, encoder, attention."""
import json
import math
import os

import numpy as np

import synth
import oracle
from oracle import Prec
from oracle import attention, e4m3_decode, e4m3_encode, attention_fp8_cache
from oracle.moe import e4m3_round

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mx_formats.json")


def test_e4m3_code_table():
    """Codes from the OCP format definition (bias 7, 3 mantissa bits, subnormals, NaN)."""
    with open(GOLDEN) as f:
        table = json.load(f)["e4m3"]["values_by_code"]
    for code, want in table.items():
        got = e4m3_decode(np.array([int(code, 16)], np.uint8))[0]
        if want == "nan":
            assert math.isnan(got), code
        else:
            assert got == want and math.copysign(1.0, got) == math.copysign(1.0, want), (code, got, want)


def test_e4m3_decode_against_rounding():
    """Every finite code is a fixed point of the independently written nearest-even rounding,
    the 127 non-negative finite codes are strictly increasing, and the extremes match the
    rounding's saturation and smallest subnormal."""
    codes = np.arange(256, dtype=np.uint8)
    vals = e4m3_decode(codes)
    finite = ~np.isnan(vals)
    assert finite.sum() == 254
    np.testing.assert_array_equal(e4m3_round(vals[finite]), vals[finite])
    pos = vals[:0x7F]
    assert np.all(np.diff(pos) > 0)
    np.testing.assert_array_equal(vals[0x80:0xFF], -pos)
    assert pos[-1] == e4m3_round(np.array([1e9]))[0] == 448.0
    assert pos[1] == 2.0 ** -9


def test_e4m3_encode_inverts_decode_and_ties():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF, 0x80)], np.uint8)
    np.testing.assert_array_equal(e4m3_encode(e4m3_decode(codes)), codes)
    # midpoints between neighbours go to the even mantissa, and beyond 448 saturates
    v = np.array([1.0625, 1.1875, 3 * 2.0 ** -10, 464.0, 1e6, -1e6, -1.0625])
    np.testing.assert_array_equal(e4m3_decode(e4m3_encode(v)), [1.0, 1.25, 2.0 ** -8, 448.0, 448.0, -448.0, -1.0])
    assert e4m3_encode(np.array([np.nan]))[0] == 0x7F


def _case(seed, B=5, hq=4, hkv=2, N=70, D=16):
    q = synth.normal_f32(seed, "kv8.q", (B, hq, D)).astype(np.float64)
    kc = synth.e4m3_codes(seed, "kv8.k", (hkv, N, D))
    vc = synth.e4m3_codes(seed, "kv8.v", (hkv, N, D))
    return q, kc, vc


def test_attention_fp8_cache_reduces_to_attention():
    """Unit scales: the same as the float64 attention over the decoded values; a key scale is
    a softmax-scale factor; a value scale multiplies the output."""
    q, kc, vc = _case(11)
    k, v = e4m3_decode(kc), e4m3_decode(vc)
    s = 0.25
    np.testing.assert_allclose(attention_fp8_cache(q, kc, vc, 1.0, 1.0, s), attention(q, k, v, s), rtol=0, atol=0)
    np.testing.assert_allclose(attention_fp8_cache(q, kc, vc, 0.125, 1.0, s), attention(q, k, v, s * 0.125),
                               rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(attention_fp8_cache(q, kc, vc, 1.0, 0.03, s), 0.03 * attention(q, k, v, s),
                               rtol=1e-12, atol=1e-14)


def test_attention_fp8_cache_one_key_and_equal_keys():
    """One visible key returns v_scale times its value row; identical keys average the values."""
    q, kc, vc = _case(12, N=1)
    o = attention_fp8_cache(q, kc, vc, 0.5, 0.25, 1.0)
    for h in range(q.shape[1]):
        np.testing.assert_array_equal(o[:, h], np.broadcast_to(0.25 * e4m3_decode(vc[h // 2, 0]), o[:, h].shape))
    q, kc, vc = _case(13, N=6)
    kc[:] = kc[:, :1]
    o = attention_fp8_cache(q, kc, vc, 1.0, 1.0, 1.0)
    np.testing.assert_allclose(o[:, 0], np.broadcast_to(e4m3_decode(vc[0]).mean(axis=0), o[:, 0].shape), rtol=1e-12)


def _tiny_layer():
    from oracle import KVCache
    s = synth.small_shape(synth.TINY, n_layers=1, d=8, hq=2, hkv=1, head_dim=4, ffn=6, vocab=16, block=3)
    rng = np.random.default_rng(7)
    W = {n: rng.standard_normal(shp) * 0.5 for n, shp in [
        ("wq", (8, 8)), ("wk", (4, 8)), ("wv", (4, 8)), ("wo", (8, 8)), ("wg", (6, 8)), ("wu", (6, 8)),
        ("wd", (8, 6))]}
    W["attn_norm"] = rng.uniform(0.5, 1.5, 8)
    W["ffn_norm"] = rng.uniform(0.5, 1.5, 8)
    return s, W, rng, KVCache


def test_fp8_cache_write_quantises_the_stored_kv():
    """With an FP8 cache the rows a layer writes are scale * e4m3(bf16 k or v / scale), the
    bf16 values being those the bf16-cache run writes; earlier rows are untouched."""
    from oracle import dense_layer, Prec
    s, W, rng, KVCache = _tiny_layer()
    L = 2
    x = rng.standard_normal((3, 8))
    runs = {}
    for name, prec in (("bf16", Prec("bf16")), ("fp8", Prec("bf16", kv_scales=(0.25, 0.5)))):
        kv = KVCache.empty(s, 8)
        kv.k[0][:, :L] = 0.25 * e4m3_decode(synth.e4m3_codes(3, "kv8.kprev", (1, L, 4)))
        kv.v[0][:, :L] = 0.5 * e4m3_decode(synth.e4m3_codes(3, "kv8.vprev", (1, L, 4)))
        dense_layer(x, W, kv.k[0], kv.v[0], L, s, prec)
        runs[name] = kv
    k16, v16 = runs["bf16"].k[0], runs["bf16"].v[0]
    k8, v8 = runs["fp8"].k[0], runs["fp8"].v[0]
    np.testing.assert_array_equal(k8[:, :L], k16[:, :L])
    np.testing.assert_array_equal(k8[:, L:L + 3], 0.25 * e4m3_round(k16[:, L:L + 3] / 0.25))
    np.testing.assert_array_equal(v8[:, L:L + 3], 0.5 * e4m3_round(v16[:, L:L + 3] / 0.5))
    # every written value is a code of the format times its scale
    codes = e4m3_encode(k8[:, L:L + 3] / 0.25)
    np.testing.assert_array_equal(0.25 * e4m3_decode(codes), k8[:, L:L + 3])


def test_fp8_cache_layer_equals_bf16_cache_on_representable_values():
    """When every k and v the layer stores is already a scale * e4m3 value (here: values of
    zero, a weight matrix of zeros), the FP8 cache changes nothing."""
    from oracle import dense_layer, Prec
    s, W, rng, KVCache = _tiny_layer()
    W["wk"] = np.zeros_like(W["wk"])
    W["wv"] = np.zeros_like(W["wv"])
    L = 2
    x = rng.standard_normal((3, 8))
    outs = []
    for prec in (Prec("bf16"), Prec("bf16", kv_scales=(0.125, 2.0))):
        kv = KVCache.empty(s, 8)
        kv.k[0][:, :L] = 0.125 * e4m3_decode(synth.e4m3_codes(4, "kv8.kprev", (1, L, 4)))
        kv.v[0][:, :L] = 2.0 * e4m3_decode(synth.e4m3_codes(4, "kv8.vprev", (1, L, 4)))
        outs.append(dense_layer(x, W, kv.k[0], kv.v[0], L, s, prec))
    np.testing.assert_array_equal(outs[0], outs[1])


def test_fp8_cache_quotient_is_single_precision():
    """The code written for a cached value is that of the single-precision quotient of the
    bf16 value and the cache scale (a float of the cache format).  For v = 0.02490234375 and
    scale 1.7f the exact quotient lies just below the midpoint 0.0146484375 of two e4m3
    values, while its single-precision rounding is the midpoint, which ties to the even code
    0x08 (0.015625) instead of 0x07 (0.013671875)."""
    import torch
    v = np.array([0.02490234375])
    s = float(np.float32(1.7))
    q32 = (torch.tensor(v, dtype=torch.float32) / torch.tensor(s, dtype=torch.float32)).item()
    assert q32 == 0.0146484375 and v[0] / s < 0.0146484375
    prec = Prec("bf16", kv_scales=(1.7, 1.0))
    stored = prec.kv_store(v, 0)
    assert stored[0] == s * 0.015625
    assert oracle.e4m3_encode(stored / s)[0] == 0x08
    # NaN stays NaN (the encoder maps it to the NaN code)
    assert np.isnan(prec.kv_store(np.array([np.nan]), 0)[0])
    assert oracle.e4m3_encode(np.array([np.nan]))[0] == 0x7F

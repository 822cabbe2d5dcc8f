"""Pins of the oracle's MX formats and routed-expert FFN."""
import json
import math
import os

import numpy as np

import synth
from oracle import mxfp4_decode, mxfp8_quant_dequant, router_topk, moe_ffn
from oracle.moe import e4m3_round, expert_ffn

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mx_formats.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_e2m1_code_table():
    g = _golden()
    codes = np.arange(16, dtype=np.uint8)
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    packed = np.concatenate([packed, np.zeros(8, np.uint8)])        # one block of 32 elements
    vals = mxfp4_decode(packed[None], np.array([[127]], np.uint8))[0][:16]
    assert list(vals) == g["e2m1_values_by_code"]


def test_e8m0_scale_and_roundtrip():
    rng = np.random.default_rng(0)
    grid = np.array(_golden()["e2m1_values_by_code"][:8])
    # exactly representable blocks round-trip through the synthetic encoder and the oracle decoder
    for e in (-3, 0, 5):
        x = rng.choice(np.concatenate([grid, -grid]), size=(3, 64)) * 2.0 ** e
        x[:, 0] = 6.0 * 2.0 ** e            # block amax pins the scale exponent
        x[:, 32] = -6.0 * 2.0 ** e
        pk, sc = synth.encode_mxfp4(x.astype(np.float32))
        assert np.all(sc == e + 127)
        np.testing.assert_array_equal(mxfp4_decode(pk, sc), x)


def test_e4m3_values():
    g = _golden()["e4m3"]
    assert e4m3_round(np.array([g["max"]]))[0] == g["max"]
    assert e4m3_round(np.array([1e6]))[0] == g["max"]              # saturates
    assert e4m3_round(np.array([g["min_subnormal"]]))[0] == g["min_subnormal"]
    assert e4m3_round(np.array([g["min_subnormal"] * 0.5]))[0] == 0.0    # halfway to zero: even
    for v, r in g["ties_to_even"]:
        assert e4m3_round(np.array([v]))[0] == r
    # every normal e4m3 value is a fixed point
    for ex in range(-6, 9):
        for m in range(8):
            v = (1 + m / 8) * 2.0 ** ex
            if v <= g["max"]:
                assert e4m3_round(np.array([v, -v])).tolist() == [v, -v]


def test_mxfp8_roundtrip_exact_values():
    rng = np.random.default_rng(1)
    x = rng.integers(-14, 15, size=(2, 64)).astype(np.float64) / 8.0
    x[:, 0] = 1.75
    x[:, 32] = -1.75
    np.testing.assert_array_equal(mxfp8_quant_dequant(x), x)
    # the shared exponent puts the block maximum in [256, 512) before rounding, so a
    # maximum above 448 * 2^e is clamped to 448 * 2^e (1000 -> 2 * 448)
    y = np.full((1, 32), 0.001)
    y[0, 5] = 1000.0
    q = mxfp8_quant_dequant(y)
    assert q[0, 5] == 896.0
    assert q[0, 0] == 0.0                 # 0.001 / 2 is below half the smallest subnormal


def test_router_topk_order_and_ties():
    f = np.array([[1.0, 0.0], [0.0, 1.0]])
    W = np.array([[2.0, 0.0], [1.0, 0.0], [2.0, 0.0], [0.0, 3.0]])
    ids, w, p = router_topk(f, W, 2)
    assert ids[0].tolist() == [0, 2]           # equal probabilities: lower id first
    assert ids[1].tolist() == [3, 0]
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-15)
    np.testing.assert_allclose(w, np.take_along_axis(p, ids, 1))


def test_topk_all_experts_is_dense_mixture_and_one_hot():
    rng = np.random.default_rng(2)
    d, F, E = 32, 32, 4
    mats = [tuple(rng.standard_normal(s) * 0.3 for s in ((F, d), (F, d), (d, F))) for _ in range(E)]
    f = rng.standard_normal((3, d))
    Wr = rng.standard_normal((E, d))
    y, ids, w = moe_ffn(f, Wr, lambda e: mats[e], [], E)
    _, _, p = router_topk(f, Wr, E)
    xq = mxfp8_quant_dequant(f)
    dense = sum(p[:, e:e + 1] * expert_ffn(xq, *mats[e]) for e in range(E))
    np.testing.assert_allclose(y, dense, atol=1e-12)
    # a router that is one-hot on expert 2 (logit 1e3 above the others) with top-1
    # (one extra block of 32 input features; only its first feature is non-zero)
    Wr1 = np.zeros((E, d + 32))
    Wr1[2, d] = 1.0
    f1 = np.concatenate([f, np.zeros((3, 32))], axis=1)
    f1[:, d] = 1e3
    mats1 = [(np.pad(a, ((0, 0), (0, 32))), np.pad(b, ((0, 0), (0, 32))), np.pad(c, ((0, 32), (0, 0))))
             for a, b, c in mats]
    y1, ids1, w1 = moe_ffn(f1, Wr1, lambda e: mats1[e], [], 1)
    assert ids1[:, 0].tolist() == [2, 2, 2] and np.all(w1 == 1.0)
    np.testing.assert_allclose(y1, expert_ffn(mxfp8_quant_dequant(f1), *mats1[2]), atol=1e-12)
    # the shared expert is added with weight one
    y2, _, _ = moe_ffn(f1, Wr1, lambda e: mats1[e], [mats1[0]], 1)
    np.testing.assert_allclose(y2 - y1, expert_ffn(mxfp8_quant_dequant(f1), *mats1[0]), atol=1e-12)


def test_synth_mxfp4_encoder_rounding():
    # the encoder (checkpoint side) rounds to the nearest e2m1 value, ties to even, and
    # saturates; the oracle decoder reads back what the encoder wrote
    x = np.zeros((1, 32), np.float32)
    x[0, :6] = [4.0, 0.25, 0.75, 5.0, 2.5, -1.25]     # amax 4 -> scale 2^0
    pk, sc = synth.encode_mxfp4(x)
    assert sc[0, 0] == 127
    np.testing.assert_array_equal(mxfp4_decode(pk, sc)[0, :6], [4.0, 0.0, 1.0, 4.0, 2.0, -1.0])
    x[0, 0] = 7.9                                       # amax 7.9 -> scale 2^0, saturate to 6
    pk, sc = synth.encode_mxfp4(x)
    assert mxfp4_decode(pk, sc)[0, 0] == 6.0 and math.isclose(2 ** (int(sc[0, 0]) - 127), 1.0)

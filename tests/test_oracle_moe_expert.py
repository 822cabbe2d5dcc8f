"""Pins of the oracle's routed-expert path against scalar-loop brute force.

The oracle's expert FFN (oracle/moe.py) is checked here against code written
independently from the definitions, not by re-calling it:
  * the e4m3 values are enumerated from the format (sign, 4 exponent bits with
    bias 7, 3 mantissa bits, subnormals at exponent field 0, the all-ones code
    is NaN) and rounding picks the nearest value, ties to the code with an
    even mantissa, saturating at the largest finite value (OCP MX v1.0,
    sections 5 and 6.3);
  * the MXFP8 shared exponent is found by an integer search for
    2^e <= amax < 2^(e+1) (no log2), minus e4m3's largest exponent 8;
  * one expert is y = down(q8(silu(gate x) * up x)) with q8 the MXFP8
    round trip, x itself MXFP8-rounded, every product a Python loop;
  * the MoE sublayer is h + sum_k p_k expert_k(bf16(rmsnorm(h) g)) + shared.
The pages run routed experts in 4-bit floating point ([ORL-blog] "What shipped";
[ORL-news] on the MoE results); the MX reading is the oracle's.

Each comparison is also run against a copy of the oracle's function with a
mistake planted in it (gate and up swapped, the activation re-quantisation
dropped, the shared expert dropped, the norm gain ignored), and must reject it.
"""
import math

import numpy as np
import torch

import oracle
from oracle import Prec
from oracle.moe import expert_ffn, moe_ffn, moe_ffn_sublayer, mxfp8_quant_dequant, swiglu, router_topk

TOL = 1e-12


# ------------------------------------------------------------------ independent formats
def _e4m3_values():
    """(value, code) for every finite e4m3 code, from the format definition."""
    out = []
    for code in range(256):
        s, e, m = code >> 7, (code >> 3) & 0xF, code & 7
        if e == 15 and m == 7:
            continue                                   # NaN
        mag = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
        out.append((-mag if s else mag, code))
    return out


_E4M3 = _e4m3_values()


def _e4m3_nearest_even(x: float) -> float:
    best_v, best_c, best_d = None, None, None
    for v, c in _E4M3:
        dist = abs(x - v)
        if best_d is None or dist < best_d or (dist == best_d and (c & 1) == 0 and (best_c & 1) == 1):
            best_v, best_c, best_d = v, c, dist
    return 0.0 if best_v == 0.0 else best_v           # +0 for -0


def _floor_log2(a: float) -> int:
    e = 0
    while 2.0 ** e > a:
        e -= 1
    while 2.0 ** (e + 1) <= a:
        e += 1
    return e


def _mxfp8_brute(row):
    row = [float(v) for v in row]
    out = []
    for b in range(0, len(row), 32):
        blk = row[b:b + 32]
        amax = max(abs(v) for v in blk)
        if amax == 0.0:
            out += [0.0] * 32
            continue
        sc = 2.0 ** (_floor_log2(amax) - 8)
        out += [_e4m3_nearest_even(v / sc) * sc for v in blk]
    return out


def _expert_brute(x, wg, wu, wd):
    """One expert on rows x (float64 [R, d]) with float64 weights, by loops."""
    R, d = x.shape
    F = wg.shape[0]
    y = np.zeros((R, wd.shape[0]))
    for i in range(R):
        xq = _mxfp8_brute(x[i])
        act = []
        for j in range(F):
            g = sum(xq[k] * wg[j, k] for k in range(d))
            u = sum(xq[k] * wu[j, k] for k in range(d))
            act.append(g / (1.0 + math.exp(-g)) * u)
        aq = _mxfp8_brute(act)
        for n in range(wd.shape[0]):
            y[i, n] = sum(aq[j] * wd[n, j] for j in range(F))
    return y


def _bf16_lib(x):
    """fp64 -> fp32 -> bf16 (nearest-even twice) through torch's own conversions."""
    return torch.from_numpy(np.asarray(x, np.float64)).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()


def _mxfp4_weights(rng, shape, exp_lo=-3, exp_hi=-1):
    """Float64 matrices whose every 32-element block along the input axis is e2m1 values
    times one power of two (so an MXFP4 checkpoint holds them exactly)."""
    e2m1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    mag = rng.choice(e2m1, size=shape)
    sgn = rng.choice([-1.0, 1.0], size=shape)
    sc = 2.0 ** rng.integers(exp_lo, exp_hi + 1, size=shape[:-1] + (shape[-1] // 32,))
    return (mag * sgn).reshape(shape[:-1] + (shape[-1] // 32, 32)) * sc[..., None]


def _reshape(w, shape):
    return w.reshape(shape)


def _mats(rng, d, F):
    wg = _reshape(_mxfp4_weights(rng, (F, d)), (F, d))
    wu = _reshape(_mxfp4_weights(rng, (F, d)), (F, d))
    wd = _reshape(_mxfp4_weights(rng, (d, F)), (d, F))
    return wg, wu, wd


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ------------------------------------------------------------------ the planted mistakes
def _expert_gate_up_swapped(xq, wg, wu, wd):
    return mxfp8_quant_dequant(swiglu(xq @ wu.T, xq @ wg.T)) @ wd.T


def _expert_no_act_quant(xq, wg, wu, wd):
    return swiglu(xq @ wg.T, xq @ wu.T) @ wd.T


# ------------------------------------------------------------------ tests
def test_e4m3_brute_table_against_golden_codes():
    """The enumerated table agrees with the OCP code values stored in the golden file."""
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "mx_formats.json")))["e4m3"]
    table = {c: v for v, c in _E4M3}
    for code, val in g["values_by_code"].items():
        c = int(code, 16)
        if val == "nan":
            assert c not in table
        else:
            assert table[c] == val
    assert max(v for v, _ in _E4M3) == g["max"]


def test_brute_mxfp8_agrees_with_oracle_quantiser():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((3, 96)) * np.array([1e-3, 1.0, 300.0]).repeat(32)[None, :]
    x[0, 5] = 0.0
    got = mxfp8_quant_dequant(x)
    want = np.array([_mxfp8_brute(r) for r in x])
    np.testing.assert_array_equal(got, want)


def test_expert_ffn_matches_brute_force():
    rng = np.random.default_rng(12)
    d, F = 64, 64
    wg, wu, wd = _mats(rng, d, F)
    x = _bf16_lib(rng.standard_normal((3, d)))
    want = _expert_brute(x, wg, wu, wd)
    got = expert_ffn(mxfp8_quant_dequant(x), wg, wu, wd)
    assert _rel(got, want) < TOL
    # the same comparison rejects the planted mistakes
    assert _rel(_expert_gate_up_swapped(mxfp8_quant_dequant(x), wg, wu, wd), want) > 1e-3
    assert _rel(_expert_no_act_quant(mxfp8_quant_dequant(x), wg, wu, wd), want) > 1e-4
    assert _rel(expert_ffn(x, wg, wu, wd), want) > 1e-4           # input not MXFP8-rounded


class _Src:
    """A one-layer MoE source: expert(layer, e, which) -> MXFP4 (packed, scales)."""

    def __init__(self, mats):
        self.mats = mats

    def expert(self, layer, e, which):
        import synth
        m = self.mats[e][("wg", "wu", "wd").index(which)]
        pk, sc = synth.encode_mxfp4(m.astype(np.float32))
        np.testing.assert_array_equal(oracle.mxfp4_decode(pk, sc), m)     # held exactly
        return pk, sc


class _Model:
    def __init__(self, shape, src, dense):
        self.shape = shape
        self.src = src
        self.dense = dense

    def get(self, name):
        return self.dense[name]


def _moe_shape(d, F, E, top_k, n_shared):
    import synth
    return synth.small_shape(synth.MOE16B, n_layers=1, d=d, hq=2, hkv=1, expert_ffn=F, n_experts=E,
                             top_k=top_k, n_shared=n_shared, vocab=64)


def _sublayer_brute(h, gain, eps, w_router, mats, top_k, n_shared, E):
    """h + MoE(bf16(rmsnorm(h) g)) with the router's softmax and top-k by loops."""
    R, d = h.shape
    y = np.array(h, dtype=np.float64)
    for i in range(R):
        ms = sum(v * v for v in h[i]) / d
        f = _bf16_lib(np.array([h[i, k] / math.sqrt(ms + eps) * gain[k] for k in range(d)]))
        logits = [sum(f[k] * w_router[e, k] for k in range(d)) for e in range(E)]
        mx = max(logits)
        ex = [math.exp(v - mx) for v in logits]
        p = [v / sum(ex) for v in ex]
        chosen = sorted(range(E), key=lambda e: (-p[e], e))[:top_k]
        for e in chosen:
            y[i] += p[e] * _expert_brute(f[None, :], *mats[e])[0]
        for s in range(n_shared):
            y[i] += _expert_brute(f[None, :], *mats[E + s])[0]
    return y


def test_moe_sublayer_one_hot_top1_is_the_dense_expert():
    """A router that is one-hot on expert e (its logit far above the others) with top-1 and no
    shared expert: the MoE sublayer is h + that expert applied to bf16(rmsnorm(h) g), weight 1."""
    rng = np.random.default_rng(13)
    d, F, E = 64, 32, 4
    mats = [_mats(rng, d, F) for _ in range(E)]
    h = (np.abs(rng.standard_normal((2, d))) + 0.5) * 3.0     # positive rows
    gain = _bf16_lib(1.0 + 0.25 * rng.uniform(-1, 1, d))
    eps = 1e-6
    f = _bf16_lib(h / np.sqrt((h * h).mean(axis=1, keepdims=True) + eps) * gain)
    w_router = np.zeros((E, d))
    w_router[2] = 10.0                                     # logit of expert 2 in the hundreds, others 0
    shape = _moe_shape(d, F, E, 1, 0)
    model = _Model(shape, _Src(mats), {"l0.ffn_norm": gain, "l0.router": w_router})
    ids, w, _ = router_topk(f, w_router, 1)
    assert ids[:, 0].tolist() == [2, 2] and np.all(w == 1.0)
    got = moe_ffn_sublayer(h, model, 0, Prec("bf16"))
    want = h + _expert_brute(f, *mats[2])
    assert _rel(got - h, want - h) < TOL
    # a plain dense SwiGLU FFN with the same matrices (bf16 activation rounding in place of MXFP8)
    # is a different function: the MX roundings are part of the expert path
    dense = h + _bf16_lib(swiglu(f @ mats[2][0].T, f @ mats[2][1].T)) @ mats[2][2].T
    assert _rel(got - h, dense - h) > 1e-4


def test_moe_sublayer_matches_brute_force_top2_with_shared():
    rng = np.random.default_rng(14)
    d, F, E, S = 64, 32, 4, 1
    mats = [_mats(rng, d, F) for _ in range(E + S)]
    h = rng.standard_normal((3, d))
    gain = _bf16_lib(1.0 + 0.25 * rng.standard_normal(d))
    w_router = _bf16_lib(rng.standard_normal((E, d)) * 0.3)
    shape = _moe_shape(d, F, E, 2, S)
    model = _Model(shape, _Src(mats), {"l0.ffn_norm": gain, "l0.router": w_router})
    got = moe_ffn_sublayer(h, model, 0, Prec("bf16"))
    want = _sublayer_brute(h, gain, shape.eps, w_router, mats, 2, S, E)
    assert _rel(got - h, want - h) < 1e-11

    # planted mistakes in a copy of the sublayer: shared expert dropped, norm gain ignored
    def sub_no_shared(hh):
        f = Prec("bf16").act(oracle.rmsnorm(hh, gain, shape.eps))
        y, _, _ = moe_ffn(f, w_router, lambda e: mats[e], [], 2)
        return hh + y

    def sub_no_gain(hh):
        f = Prec("bf16").act(oracle.rmsnorm(hh, np.ones(d), shape.eps))
        y, _, _ = moe_ffn(f, w_router, lambda e: mats[e], [mats[E]], 2)
        return hh + y

    assert _rel(sub_no_shared(h) - h, want - h) > 1e-3
    assert _rel(sub_no_gain(h) - h, want - h) > 1e-3

"""Pins of the oracle's layer pieces against brute force, closed forms and invariants."""
import math

import numpy as np
import pytest

import synth
from oracle import rmsnorm, rope, attention, Prec
from oracle.block import dense_layer, swiglu
from oracle.loop import KVCache


def test_rmsnorm_unit_rms_and_gain():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 64)) * 3.0
    y = rmsnorm(x, np.ones(64), 0.0)
    np.testing.assert_allclose(np.sqrt((y * y).mean(axis=1)), 1.0, rtol=1e-13)
    g = rng.standard_normal(64)
    np.testing.assert_allclose(rmsnorm(x, g, 1e-6), rmsnorm(x, np.ones(64), 1e-6) * g, rtol=1e-13)
    # brute force with eps on one row
    row = x[2]
    ms = sum(float(v) * float(v) for v in row) / len(row)
    ref = [float(v) / math.sqrt(ms + 1e-6) * float(gg) for v, gg in zip(row, g)]
    np.testing.assert_allclose(rmsnorm(x, g, 1e-6)[2], ref, rtol=1e-13)


def test_rope_identity_norm_relative():
    rng = np.random.default_rng(1)
    D = 16
    x = rng.standard_normal((3, 2, D))
    np.testing.assert_allclose(rope(x, np.zeros(3), 1e4), x, atol=0)
    y = rope(x, np.array([5, 17, 300]), 1e4)
    # each rotate-half pair keeps its length
    n0 = x[..., :D // 2] ** 2 + x[..., D // 2:] ** 2
    n1 = y[..., :D // 2] ** 2 + y[..., D // 2:] ** 2
    np.testing.assert_allclose(n1, n0, rtol=1e-12)
    # q.k depends only on the position difference
    q = rng.standard_normal((1, 1, D))
    k = rng.standard_normal((1, 1, D))
    for a, b in [(3, 10), (100, 107), (1000, 1007)]:
        s = (rope(q, np.array([b]), 1e4) * rope(k, np.array([a]), 1e4)).sum()
        s0 = (rope(q, np.array([7]), 1e4) * rope(k, np.array([0]), 1e4)).sum()
        assert abs(s - s0) < 1e-12


def test_rope_matches_complex_rotation():
    # independent derivation: the pair (x_j, x_{j+D/2}) is the complex number
    # x_j + i x_{j+D/2} multiplied by exp(i * pos * base^(-2j/D))
    rng = np.random.default_rng(2)
    D, base = 8, 10000.0
    x = rng.standard_normal((1, 1, D))
    pos = 37
    y = rope(x, np.array([pos]), base)[0, 0]
    for j in range(D // 2):
        z = complex(x[0, 0, j], x[0, 0, j + D // 2]) * complex(math.cos(pos * base ** (-2 * j / D)),
                                                                  math.sin(pos * base ** (-2 * j / D)))
        assert abs(y[j] - z.real) < 1e-12 and abs(y[j + D // 2] - z.imag) < 1e-12


def _attn_brute(q, k, v, scale):
    B, Hq, D = q.shape
    Hkv, N, _ = k.shape
    out = np.zeros_like(q)
    for i in range(B):
        for h in range(Hq):
            g = h * Hkv // Hq
            s = [scale * sum(q[i, h, t] * k[g, j, t] for t in range(D)) for j in range(N)]
            mx = max(s)
            w = [math.exp(a - mx) for a in s]
            z = sum(w)
            for t in range(D):
                out[i, h, t] = sum(w[j] * v[g, j, t] for j in range(N)) / z
    return out


@pytest.mark.parametrize("L,B", [(0, 1), (0, 3), (1, 1), (5, 3), (5, 1)])
def test_attention_brute_force(L, B):
    rng = np.random.default_rng(10 + L * 7 + B)
    Hq, Hkv, D = 4, 2, 8
    q = rng.standard_normal((B, Hq, D))
    k = rng.standard_normal((Hkv, L + B, D))
    v = rng.standard_normal((Hkv, L + B, D))
    np.testing.assert_allclose(attention(q, k, v, 1 / math.sqrt(D)), _attn_brute(q, k, v, 1 / math.sqrt(D)),
                               atol=1e-12, rtol=0)


def test_attention_special_cases():
    rng = np.random.default_rng(3)
    Hq, Hkv, D = 4, 2, 8
    # a single key gives o = v
    q = rng.standard_normal((2, Hq, D))
    k = rng.standard_normal((Hkv, 1, D))
    v = rng.standard_normal((Hkv, 1, D))
    o = attention(q, k, v, 0.3)
    for h in range(Hq):
        np.testing.assert_allclose(o[:, h], np.broadcast_to(v[h // 2, 0], (2, D)), atol=1e-15)
    # q = 0 gives the mean of V
    k = rng.standard_normal((Hkv, 6, D))
    v = rng.standard_normal((Hkv, 6, D))
    o = attention(np.zeros((3, Hq, D)), k, v, 0.3)
    for h in range(Hq):
        np.testing.assert_allclose(o[:, h], np.broadcast_to(v[h // 2].mean(axis=0), (3, D)), atol=1e-14)
    # Hkv = Hq is multi-head attention: each head on its own kv head
    q = rng.standard_normal((3, 2, D))
    k = rng.standard_normal((2, 5, D))
    v = rng.standard_normal((2, 5, D))
    o = attention(q, k, v, 0.5)
    for h in range(2):
        np.testing.assert_allclose(o[:, h:h + 1], attention(q[:, h:h + 1], k[h:h + 1], v[h:h + 1], 0.5), atol=1e-15)
    # Hkv = 1 is multi-query attention: every head uses kv head 0
    o = attention(q, k[:1], v[:1], 0.5)
    np.testing.assert_allclose(o[:, 1:2], attention(q[:, 1:2], k[:1], v[:1], 0.5), atol=1e-15)


def test_swiglu_closed_form():
    for g, u in [(0.0, 3.0), (1.0, 2.0), (-2.5, 0.5), (10.0, -1.0)]:
        ref = g / (1 + math.exp(-g)) * u
        assert abs(float(swiglu(np.array(g), np.array(u))) - ref) < 1e-15


def _layer_brute(x, W, kprev, vprev, L, s):
    """Scalar-loop pre-norm layer written from the definitions."""
    B, d = x.shape
    Hq, Hkv, D, F = s.hq, s.hkv, s.head_dim, s.ffn

    def norm(row, g):
        ms = sum(t * t for t in row) / len(row)
        return [row[j] / math.sqrt(ms + s.eps) * g[j] for j in range(len(row))]

    def matvec(Wm, vec):
        return [sum(Wm[o][i] * vec[i] for i in range(len(vec))) for o in range(len(Wm))]

    def rot(vec, pos):
        out = list(vec)
        for j in range(D // 2):
            th = pos * s.rope_base ** (-2.0 * j / D)
            a, b = vec[j], vec[j + D // 2]
            out[j] = a * math.cos(th) - b * math.sin(th)
            out[j + D // 2] = b * math.cos(th) + a * math.sin(th)
        return out

    qs, ks, vs = [], [], []
    for i in range(B):
        a = norm(list(x[i]), W["attn_norm"])
        q = matvec(W["wq"], a)
        k = matvec(W["wk"], a)
        v = matvec(W["wv"], a)
        qs.append([rot(q[h * D:(h + 1) * D], L + i) for h in range(Hq)])
        ks.append([rot(k[h * D:(h + 1) * D], L + i) for h in range(Hkv)])
        vs.append([v[h * D:(h + 1) * D] for h in range(Hkv)])
    keys = [[list(kprev[g, j]) for j in range(L)] + [ks[i][g] for i in range(B)] for g in range(Hkv)]
    vals = [[list(vprev[g, j]) for j in range(L)] + [vs[i][g] for i in range(B)] for g in range(Hkv)]
    out = np.zeros((B, d))
    for i in range(B):
        o = []
        for h in range(Hq):
            g = h // (Hq // Hkv)
            sc = [sum(qs[i][h][t] * keys[g][j][t] for t in range(D)) / math.sqrt(D) for j in range(L + B)]
            mx = max(sc)
            w = [math.exp(c - mx) for c in sc]
            z = sum(w)
            o += [sum(w[j] * vals[g][j][t] for j in range(L + B)) / z for t in range(D)]
        hres = [x[i, j] + sum(W["wo"][j][t] * o[t] for t in range(Hq * D)) for j in range(d)]
        f = norm(hres, W["ffn_norm"])
        gt = matvec(W["wg"], f)
        up = matvec(W["wu"], f)
        act = [gt[j] / (1 + math.exp(-gt[j])) * up[j] for j in range(F)]
        out[i] = [hres[j] + sum(W["wd"][j][t] * act[t] for t in range(F)) for j in range(d)]
    return out


def test_dense_layer_brute_force():
    s = synth.small_shape(synth.TINY, n_layers=1, d=8, hq=2, hkv=1, head_dim=4, ffn=6, vocab=16, block=3)
    rng = np.random.default_rng(4)
    W = {n: rng.standard_normal(shp) * 0.5 for n, shp in [
        ("wq", (8, 8)), ("wk", (4, 8)), ("wv", (4, 8)), ("wo", (8, 8)), ("wg", (6, 8)), ("wu", (6, 8)),
        ("wd", (8, 6))]}
    W["attn_norm"] = rng.uniform(0.5, 1.5, 8)   # non-unit gains catch swapped norms
    W["ffn_norm"] = rng.uniform(0.5, 1.5, 8)
    L = 2
    kv = KVCache.empty(s, 8)
    kv.k[0][:, :L] = rng.standard_normal((1, L, 4))
    kv.v[0][:, :L] = rng.standard_normal((1, L, 4))
    kprev, vprev = kv.k[0].copy(), kv.v[0].copy()
    x = rng.standard_normal((3, 8))
    y = dense_layer(x, W, kv.k[0], kv.v[0], L, s, Prec())
    np.testing.assert_allclose(y, _layer_brute(x, W, kprev, vprev, L, s), atol=1e-12, rtol=0)


def test_bf16_round_points():
    from oracle import bf16_round
    # exact bf16 values are fixed points; halfway cases go to even
    assert bf16_round(np.array([1.0]))[0] == 1.0
    assert bf16_round(np.array([1.0 + 2 ** -8]))[0] == 1.0               # halfway, even is 1.0
    assert bf16_round(np.array([1.0 + 3 * 2 ** -8]))[0] == 1.0 + 2 ** -6   # halfway, even is up
    assert bf16_round(np.array([1.0 + 2 ** -8 + 2 ** -20]))[0] == 1.0 + 2 ** -7
    assert bf16_round(np.array([-3.0]))[0] == -3.0


def test_bf16_round_matches_library_conversion():
    """On fp32 values (random magnitudes over 24 binades, both signs, plus exact halfway
    cases) the oracle's rounding equals torch's float32 -> bfloat16 conversion, which rounds
    to nearest even."""
    import torch
    from oracle import bf16_round
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(200000) * np.exp2(rng.integers(-12, 12, 200000))).astype(np.float32)
    # halfway between two bf16 values: a bf16 value plus half its unit in the last place
    base = torch.from_numpy(x[:1000]).to(torch.bfloat16).float().numpy()
    half = (base.view(np.uint32) | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, half])
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy().astype(np.float64)
    assert np.array_equal(bf16_round(x.astype(np.float64)), ref)


def test_decode_storage_matches_library_widening():
    import torch
    from oracle import decode_storage
    bits = np.random.default_rng(12).integers(0, 1 << 16, 100000, dtype=np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]          # finite values only
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy().astype(np.float64)
    assert np.array_equal(decode_storage(bits), ref)

"""Pins of the oracle's head statistics: brute force, closed forms and invariants."""
import math

import numpy as np

from oracle import head_rowstats


def _brute(h, E):
    out = []
    for row in h:
        l = [sum(row[t] * e[t] for t in range(len(row))) for e in E]
        mx = max(l)
        am = l.index(mx)
        w = [math.exp(a - mx) for a in l]
        s = sum(w)
        p = [a / s for a in w]
        ent = -sum(pp * math.log(pp) for pp in p if pp > 0)
        pe = [sum(p[v] * E[v][t] for v in range(len(E))) for t in range(len(row))]
        out.append((mx + math.log(s), ent, max(p), am, pe))
    return out


def test_head_brute_force():
    rng = np.random.default_rng(0)
    h = rng.standard_normal((3, 6))
    E = rng.standard_normal((11, 6))
    st = head_rowstats(h, E, want_logits=True)
    for i, (lse, ent, mp, am, pe) in enumerate(_brute(h, E)):
        assert abs(st["lse"][i] - lse) < 1e-12
        assert abs(st["entropy"][i] - ent) < 1e-12
        assert abs(st["maxprob"][i] - mp) < 1e-12
        assert st["argmax"][i] == am
        np.testing.assert_allclose(st["pe"][i], pe, atol=1e-12)
    # probabilities sum to one
    p = np.exp(st["logits"] - st["lse"][:, None])
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-12)


def test_entropy_range_and_uniform():
    rng = np.random.default_rng(1)
    V, d = 50, 8
    E = rng.standard_normal((V, d))
    h = rng.standard_normal((4, d)) * 3
    st = head_rowstats(h, E)
    assert np.all(st["entropy"] >= 0) and np.all(st["entropy"] <= math.log(V) + 1e-12)
    # all logits equal (h = 0): H = ln V, maxprob = 1/V, argmax = 0, lse = ln V, pe = mean row
    st = head_rowstats(np.zeros((2, d)), E)
    np.testing.assert_allclose(st["entropy"], math.log(V), atol=1e-12)
    np.testing.assert_allclose(st["maxprob"], 1.0 / V, atol=1e-15)
    assert list(st["argmax"]) == [0, 0]
    np.testing.assert_allclose(st["lse"], math.log(V), atol=1e-12)
    np.testing.assert_allclose(st["pe"], np.broadcast_to(E.mean(axis=0), (2, d)), atol=1e-12)


def test_two_logit_closed_form():
    for a, b in [(0.3, -1.2), (2.0, 2.5), (-7.0, 4.0)]:
        E = np.array([[a], [b]])
        st = head_rowstats(np.array([[1.0]]), E)
        p0 = 1.0 / (1.0 + math.exp(b - a))
        H = -(p0 * math.log(p0) + (1 - p0) * math.log(1 - p0))
        assert abs(st["entropy"][0] - H) < 1e-12
        assert abs(st["lse"][0] - (max(a, b) + math.log1p(math.exp(-abs(a - b))))) < 1e-12
        assert abs(st["maxprob"][0] - max(p0, 1 - p0)) < 1e-12
        assert st["argmax"][0] == (0 if a >= b else 1)
        np.testing.assert_allclose(st["pe"][0], [p0 * a + (1 - p0) * b], atol=1e-12)


def test_shift_and_permutation_invariance():
    rng = np.random.default_rng(2)
    V, d = 40, 6
    E = rng.standard_normal((V, d))
    h = rng.standard_normal((3, d))
    st = head_rowstats(h, E)
    # shift: an extra coordinate equal to 1 in every E row and c in h adds c to every logit
    c = 2.75
    E1 = np.concatenate([E, np.ones((V, 1))], axis=1)
    h1 = np.concatenate([h, np.full((3, 1), c)], axis=1)
    st1 = head_rowstats(h1, E1)
    np.testing.assert_allclose(st1["lse"], st["lse"] + c, atol=1e-12)
    np.testing.assert_allclose(st1["entropy"], st["entropy"], atol=1e-12)
    np.testing.assert_allclose(st1["maxprob"], st["maxprob"], atol=1e-14)
    assert list(st1["argmax"]) == list(st["argmax"])
    np.testing.assert_allclose(st1["pe"][:, :d], st["pe"], atol=1e-12)
    # permuting E's rows permutes argmax and leaves the rest unchanged
    perm = rng.permutation(V)
    st2 = head_rowstats(h, E[perm])
    inv = np.argsort(perm)
    assert list(st2["argmax"]) == [int(inv[a]) for a in st["argmax"]]
    np.testing.assert_allclose(st2["lse"], st["lse"], atol=1e-12)
    np.testing.assert_allclose(st2["entropy"], st["entropy"], atol=1e-12)
    np.testing.assert_allclose(st2["pe"], st["pe"], atol=1e-12)


def test_one_hot_pe_is_embedding_row():
    rng = np.random.default_rng(3)
    V, d = 30, 5
    E = rng.standard_normal((V, d))
    # make token 17's logit 1e3 above the rest: append a coordinate that only row 17 has
    E1 = np.concatenate([E, np.zeros((V, 1))], axis=1)
    E1[17, -1] = 1.0
    h = np.concatenate([np.zeros((1, d)), [[1e3]]], axis=1)
    st = head_rowstats(h, E1)
    assert st["argmax"][0] == 17
    np.testing.assert_allclose(st["pe"][0], E1[17], atol=1e-12)
    assert st["maxprob"][0] > 1 - 1e-12 and st["entropy"][0] < 1e-12


def test_argmax_tie_lowest_id_and_committed_sentinels():
    rng = np.random.default_rng(4)
    V, d = 12, 4
    E = rng.standard_normal((V, d)) * 0.1
    E[3] = E[7] = np.array([5.0, 0, 0, 0])
    h = np.array([[1.0, 0, 0, 0], [1.0, 0, 0, 0], [0.5, 0.1, 0, 0]])
    committed = np.array([0, 1, 0], np.uint8)
    st = head_rowstats(h, E, committed)
    assert st["argmax"][0] == 3
    assert st["argmax"][1] == -1 and st["lse"][1] == 0 and st["entropy"][1] == 0 and st["maxprob"][1] == 0
    assert not st["pe"][1].any()
    st_open = head_rowstats(h[[0, 2]], E)
    np.testing.assert_allclose(st["lse"][[0, 2]], st_open["lse"], atol=0)

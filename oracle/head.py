"""Tied-embedding head with per-row statistics and the p.E feedback mix.

Each round yields, for every still-unresolved position, a predictive
distribution over the vocabulary ([ORL-blog] "What shipped").  The head is the
tied embedding E used as the output matrix ([ORL-blog] "What shipped": the
self-conditioning adapter sits on the tied embedding), and the statistics the
commit rule needs are computed per row ([ORL-card] "The paper's evaluation
pipeline" names fused row statistics).

Readings: entropy in nats (range [0, ln V]); confidence = max probability;
argmax ties go to the lowest token id; the previous distribution is fed back
only through p.E = sum_v p_v E_v (d numbers per row), never as p itself.
Committed rows get the sentinels argmax = -1, lse = entropy = maxprob = 0 and
a zero pe row.  Pinned by tests/test_oracle_head.py.
"""
from __future__ import annotations

import numpy as np

from .numerics import Prec

_VCHUNK = 16384


def head_rowstats(hn: np.ndarray, emb_stored: np.ndarray, committed=None, prec: Prec = Prec(),
                  want_pe: bool = True, want_logits: bool = False):
    """Row statistics of softmax(hn E^T) for the open rows.

    hn [R, d] final-normed hidden rows (already at their storage precision);
    emb_stored [V, d] the stored embedding.  Returns a dict with lse, entropy,
    maxprob [R] (compute dtype), argmax [R] int32, pe [R, d] and optionally
    logits [R, V] (open rows only, others zero) plus the top-2 logit gap per
    row (diagnostic for near-ties).
    """
    R, d = hn.shape
    V = emb_stored.shape[0]
    dt = prec.compute
    if committed is None:
        committed = np.zeros(R, dtype=np.uint8)
    open_rows = np.nonzero(np.asarray(committed) == 0)[0]
    out = {
        "lse": np.zeros(R, dt), "entropy": np.zeros(R, dt), "maxprob": np.zeros(R, dt),
        "argmax": np.full(R, -1, np.int32), "pe": np.zeros((R, d), dt),
        "top2_gap": np.full(R, np.inf),
    }
    if want_logits:
        out["logits"] = np.zeros((R, V), dt)
    if open_rows.size == 0:
        return out
    h = np.asarray(hn[open_rows], dtype=dt)
    # logits, one vocabulary chunk at a time (the whole [M, V] is kept; it is small)
    l = np.empty((open_rows.size, V), dt)
    for a in range(0, V, _VCHUNK):
        b = min(V, a + _VCHUNK)
        l[:, a:b] = h @ prec.w(emb_stored[a:b]).T
    m = l.max(axis=1)
    am = l.argmax(axis=1)                   # first maximum == lowest token id
    z = l - m[:, None]
    e = np.exp(z)
    s = e.sum(axis=1)
    p = e / s[:, None]
    lse = m + np.log(s)
    with np.errstate(divide="ignore", invalid="ignore"):
        plogp = np.where(p > 0, p * np.log(np.where(p > 0, p, 1.0)), 0.0)
    ent = -plogp.sum(axis=1)
    maxprob = p.max(axis=1)
    srt = np.partition(l, V - 2, axis=1)[:, -2:] if V >= 2 else np.stack([m, m], 1)
    gap = np.abs(srt[:, 1] - srt[:, 0])
    out["lse"][open_rows] = lse
    out["entropy"][open_rows] = ent
    out["maxprob"][open_rows] = maxprob
    out["argmax"][open_rows] = am.astype(np.int32)
    out["top2_gap"][open_rows] = gap
    if want_logits:
        out["logits"][open_rows] = l
    if want_pe:
        pe = np.zeros((open_rows.size, d), dt)
        for a in range(0, V, _VCHUNK):
            b = min(V, a + _VCHUNK)
            pe += p[:, a:b] @ prec.w(emb_stored[a:b])
        out["pe"][open_rows] = pe
    return out

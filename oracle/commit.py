"""Confidence commit: which open positions become final this round.

Each round commits the positions that clear the commit bar; more clearing
means fewer rounds per block ([ORL-blog] "What shipped", last paragraph of the
entropy-contraction item; [ORL-news] "dLLM 是什么": many positions predicted at
once, then revised by confidence).  The pages give no bar value and no
selection rule beyond this, so the readings are:

  THRESHOLD: commit every open row with maxprob >= tau, plus (forced_top1) the
             open row with the largest maxprob, so every round commits >= 1.
  FIXED_K:   commit the min(k, n_open) open rows with the largest maxprob
             (random weights make a threshold degenerate, so a fixed count
             stands in for the learned tokens-per-forward).
  Ties rank the lower position first; NaN maxprob ranks as -inf.
  A committed position is never reopened; the token is the row's argmax.
  In the last allowed round (round == max_rounds - 1) every open row is
  committed at its argmax and FLAG_HIT_MAX_ROUNDS is set if that committed
  more than the rule would have.
Pinned by tests/test_oracle_commit.py (crafted cases and loop invariants).
"""
from __future__ import annotations

import dataclasses

import numpy as np

THRESHOLD = 0
FIXED_K = 1
FLAG_HIT_MAX_ROUNDS = 1
FLAG_NONFINITE = 2


@dataclasses.dataclass(frozen=True)
class CommitRule:
    mode: int = THRESHOLD
    tau: float = 0.9
    k: int = 1
    forced_top1: bool = True
    max_rounds: int = 32


def _rank_key(mp: float) -> float:
    return -np.inf if np.isnan(mp) else float(mp)


def commit(rule: CommitRule, maxprob, argmax, committed, tokens, round_idx: int):
    """Apply one round's commit in place.

    maxprob [B] (float), argmax [B] (int), committed [B] (uint8, modified),
    tokens [B] (int32, modified).  Returns (indices committed this round,
    flags).  The threshold comparison and the ranking use the values as given
    (the caller decides their precision).
    """
    B = len(committed)
    open_idx = [i for i in range(B) if not committed[i]]
    flags = 0
    if any(not np.isfinite(maxprob[i]) for i in open_idx):
        flags |= FLAG_NONFINITE
    order = sorted(open_idx, key=lambda i: (-_rank_key(maxprob[i]), i))
    if rule.mode == THRESHOLD:
        sel = {i for i in open_idx if maxprob[i] >= rule.tau}
        if rule.forced_top1 and order:
            sel.add(order[0])
    elif rule.mode == FIXED_K:
        sel = set(order[:min(rule.k, len(order))])
    else:
        raise ValueError(rule.mode)
    if round_idx >= rule.max_rounds - 1:
        forced = set(open_idx) - sel
        if forced:
            flags |= FLAG_HIT_MAX_ROUNDS
        sel = set(open_idx)
    for i in sel:
        tokens[i] = argmax[i]
        committed[i] = 1
    return sorted(sel), flags

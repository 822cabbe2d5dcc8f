"""Pins of the commit rule on crafted cases."""
import math

import numpy as np
import pytest

from oracle import CommitRule, commit, THRESHOLD, FIXED_K, FLAG_HIT_MAX_ROUNDS, FLAG_NONFINITE


def _run(rule, mp, committed=None, round_idx=0):
    n = len(mp)
    committed = np.zeros(n, np.uint8) if committed is None else np.array(committed, np.uint8)
    tokens = np.full(n, -5, np.int32)
    argmax = np.arange(100, 100 + n, dtype=np.int32)
    sel, flags = commit(rule, np.array(mp, dtype=np.float64), argmax, committed, tokens, round_idx)
    return sel, flags, committed, tokens


def test_threshold_plus_top1():
    rule = CommitRule(THRESHOLD, tau=0.9, forced_top1=True, max_rounds=32)
    sel, flags, c, t = _run(rule, [0.95, 0.5, 0.91, 0.2])
    assert sel == [0, 2] and flags == 0
    assert list(c) == [1, 0, 1, 0] and list(t) == [100, -5, 102, -5]
    # nobody clears the bar: the top-1 is committed, ties to the lower position
    sel, _, _, _ = _run(rule, [0.3, 0.6, 0.6, 0.1])
    assert sel == [1]
    # threshold is inclusive
    sel, _, _, _ = _run(rule, [0.9, 0.1])
    assert sel == [0]
    # without forced top-1 nothing may be committed
    sel, _, _, _ = _run(CommitRule(THRESHOLD, tau=0.9, forced_top1=False), [0.3, 0.6])
    assert sel == []


def test_committed_rows_are_not_candidates():
    rule = CommitRule(THRESHOLD, tau=0.9)
    sel, _, c, t = _run(rule, [0.99, 0.4, 0.3], committed=[1, 0, 0])
    assert sel == [1] and t[0] == -5      # row 0 was already committed: left alone


@pytest.mark.parametrize("k", [1, 2, 3, 6, 11, 32])
def test_fixed_k_counts(k):
    rule = CommitRule(FIXED_K, k=k)
    rng = np.random.default_rng(k)
    committed = np.zeros(32, np.uint8)
    tokens = np.zeros(32, np.int32)
    rounds = 0
    while not committed.all():
        n_open = int((committed == 0).sum())
        mp = rng.uniform(size=32)
        before = committed.copy()
        sel, flags = commit(rule, mp, np.arange(32), committed, tokens, rounds)
        assert len(sel) == min(k, n_open) and flags == 0
        assert np.all(committed >= before)                    # never reopened
        opened = [i for i in range(32) if not before[i]]
        best = sorted(opened, key=lambda i: (-mp[i], i))[:len(sel)]
        assert sorted(best) == sel
        rounds += 1
    assert rounds == math.ceil(32 / k)


def test_fixed_k_ties_lower_position():
    sel, _, _, _ = _run(CommitRule(FIXED_K, k=2), [0.5, 0.7, 0.5, 0.5])
    assert sel == [0, 1]


def test_nan_ranks_last_and_flags():
    sel, flags, _, _ = _run(CommitRule(THRESHOLD, tau=0.9), [float("nan"), 0.2, 0.1])
    assert sel == [1] and flags & FLAG_NONFINITE
    sel, _, _, _ = _run(CommitRule(FIXED_K, k=1), [float("nan"), float("nan")])
    assert sel == [0]


def test_max_rounds_commits_all():
    rule = CommitRule(THRESHOLD, tau=0.9, forced_top1=True, max_rounds=4)
    sel, flags, c, _ = _run(rule, [0.1, 0.2, 0.3], round_idx=3)
    assert sel == [0, 1, 2] and c.all() and flags & FLAG_HIT_MAX_ROUNDS
    # when the rule itself would commit everything, no flag
    sel, flags, _, _ = _run(rule, [0.3], round_idx=3)
    assert sel == [0] and flags == 0

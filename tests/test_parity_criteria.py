"""The attention parity criterion (tests/parity.py) accepts the roundings of a correct bf16
path and rejects the failures it is meant to catch: an output missing one key split of the
long-prefix plan, an all-zero output, and an output whose value scale is off.  Run on the
CPU with the oracle's attention as the exact result."""
import math

import numpy as np
import pytest

import oracle
import synth
from tests.parity import attention_ok, attention_errors, kernel_attention_model, split_bounds

B, HQ, HKV, D = 32, 4, 1, 128


def _inputs(L, seed):
    q = oracle.decode_storage(synth.stored_normal(seed, "crit.q", (B, HQ, D), 1.0, "bf16"))
    k = oracle.decode_storage(synth.stored_normal(seed, "crit.k", (HKV, L + B, D), 1.0, "bf16"))
    v = oracle.decode_storage(synth.stored_normal(seed, "crit.v", (HKV, L + B, D), 1.0, "bf16"))
    return q, k, v


def _emulated_bf16_path(q, k, v, drop=None):
    """The library's bf16 roundings on the oracle's inputs, the combined output rounded to
    bf16 as the library stores it."""
    return oracle.bf16_round(kernel_attention_model(q, k, v, 1.0 / math.sqrt(D), drop=drop))


@pytest.mark.parametrize("L", [512, 4096, 32768])
def test_criterion_accepts_the_bf16_roundings(L):
    q, k, v = _inputs(L, 1250)
    ref = oracle.attention(q, k, v, 1.0 / math.sqrt(D))
    got = _emulated_bf16_path(q, k, v)
    rel, elem = attention_errors(got, ref)
    assert attention_ok(got, ref), (rel, elem)
    assert rel < 5e-3                   # the derivation's 2e-3, with room for the worst row


@pytest.mark.parametrize("L", [4096, 32768])
def test_criterion_rejects_a_dropped_split(L):
    q, k, v = _inputs(L, 1251)
    ref = oracle.attention(q, k, v, 1.0 / math.sqrt(D))
    n = len(split_bounds(L + B))
    assert n >= 22
    for drop in (0, n // 2, n - 2):
        assert not attention_ok(_emulated_bf16_path(q, k, v, drop=drop), ref), drop


def test_criterion_rejects_zero_and_scaled_outputs():
    q, k, v = _inputs(32768, 1252)
    ref = oracle.attention(q, k, v, 1.0 / math.sqrt(D))
    assert not attention_ok(np.zeros_like(ref), ref)
    assert not attention_ok(ref * 1.03, ref)            # a 3 % value-scale error (e.g. an FP8 scale)
    assert attention_ok(oracle.bf16_round(ref), ref)


def test_criterion_rejects_a_wrong_kv_head():
    # GQA with 2 kv heads: reading the other kv head's values for every query head
    L = 1024
    q = oracle.decode_storage(synth.stored_normal(1253, "crit.q2", (B, 8, D), 1.0, "bf16"))
    k = oracle.decode_storage(synth.stored_normal(1253, "crit.k2", (2, L + B, D), 1.0, "bf16"))
    v = oracle.decode_storage(synth.stored_normal(1253, "crit.v2", (2, L + B, D), 1.0, "bf16"))
    ref = oracle.attention(q, k, v, 1.0 / math.sqrt(D))
    wrong = oracle.attention(q, k, v[::-1].copy(), 1.0 / math.sqrt(D))
    assert not attention_ok(wrong, ref)


@pytest.mark.parametrize("n", [1, 64, 65, 2047, 2048, 2049, 2336, 4128, 32800])
def test_split_plan_partitions_the_keys(n):
    """The kernel's split plan as the error model takes it: the passes of all splits cover
    [0, n) once, in 64-key passes, within 32 splits; split s starts with pass s (keys
    [64 s, 64 s + 64)) and takes every nsplit-th pass after it."""
    splits = split_bounds(n)
    assert 1 <= len(splits) <= 32
    cover = sorted(p for sp in splits for p in sp)
    assert cover == [(c, min(n, c + 64)) for c in range(0, n, 64)]
    for s, sp in enumerate(splits):
        assert sp[0][0] == 64 * s
        assert all(b[0] - a[0] == 64 * len(splits) for a, b in zip(sp, sp[1:]))

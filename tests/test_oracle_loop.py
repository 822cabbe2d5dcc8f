"""Pins of the self-conditioning input, the cached block loop, prefill and resume."""
import numpy as np
import pytest

import synth
from oracle import (OracleModel, KVCache, Prec, CommitRule, THRESHOLD, FIXED_K, selfcond, decode_block,
                    prefill, generate, blockcausal_reference)

SMALL = synth.small_shape(synth.TINY, n_layers=2, d=64, hq=4, hkv=2, head_dim=16, ffn=96, vocab=97, block=8)


def _model(shape=SMALL, seed=1234, **over):
    return OracleModel(shape, synth.Weights(shape, seed), Prec("f32", np.float64), overrides=over)


def test_selfcond_inert_and_identity():
    s = SMALL
    rng = np.random.default_rng(0)
    m = _model(w_sc=np.zeros((s.d, s.d)))
    tokens = np.array([5, 0, 9, 0, 0, 1, 0, 0], np.int32)
    committed = np.array([1, 0, 1, 0, 0, 1, 0, 0], np.uint8)
    pe = rng.standard_normal((8, s.d))
    x = selfcond(m, tokens, committed, pe, Prec())
    mask = m.get("mask_emb")
    E = m.emb_rows(np.arange(s.vocab))
    for i in range(8):
        np.testing.assert_array_equal(x[i], E[tokens[i]] if committed[i] else mask)
    # first round: no previous distribution, every open row is the mask vector
    x0 = selfcond(_model(), tokens, np.zeros(8, np.uint8), None, Prec())
    np.testing.assert_array_equal(x0, np.broadcast_to(mask, (8, s.d)))
    # identity adapter with a one-hot distribution on token 11: x = m + E[11]
    mi = _model(w_sc=np.eye(s.d))
    pe1 = np.broadcast_to(E[11], (8, s.d))
    x1 = selfcond(mi, tokens, committed, pe1, Prec())
    for i in range(8):
        if not committed[i]:
            np.testing.assert_allclose(x1[i], mask + E[11], atol=1e-15)


def test_cache_equals_blockcausal_recompute():
    m = _model()
    prompt = synth.prompt_ids(SMALL, 16, 1234)
    rule = CommitRule(THRESHOLD, tau=0.9, forced_top1=True, max_rounds=8)
    toks, blocks, kv = generate(m, prompt, 2, rule, Prec(), cap=64)
    seq = np.concatenate([prompt, toks])
    ks, vs = blockcausal_reference(m, seq, Prec())
    N = len(seq)
    assert kv.length == N
    for li in range(SMALL.n_layers):
        np.testing.assert_allclose(kv.k[li][:, :N], ks[li], atol=1e-10, rtol=0)
        np.testing.assert_allclose(kv.v[li][:, :N], vs[li], atol=1e-10, rtol=0)


def test_prefill_equals_blockcausal():
    m = _model()
    prompt = synth.prompt_ids(SMALL, 24, 99)
    kv = KVCache.empty(SMALL, 32)
    prefill(m, kv, prompt, Prec())
    ks, vs = blockcausal_reference(m, prompt, Prec())
    for li in range(SMALL.n_layers):
        np.testing.assert_allclose(kv.k[li][:, :24], ks[li], atol=1e-10, rtol=0)
        np.testing.assert_allclose(kv.v[li][:, :24], vs[li], atol=1e-10, rtol=0)


def test_loop_invariants_threshold():
    m = _model()
    prompt = synth.prompt_ids(SMALL, 8, 7)
    rule = CommitRule(THRESHOLD, tau=0.9, forced_top1=True, max_rounds=8)
    kv = KVCache.empty(SMALL, 64)
    prefill(m, kv, prompt, Prec())
    br = decode_block(m, kv, rule, Prec(), keep_trace=True)
    assert 1 <= br.rounds <= rule.max_rounds
    assert all(n >= 1 for n in br.n_new) and sum(br.n_new) == SMALL.block
    prev = np.zeros(SMALL.block, np.uint8)
    for open_before, res in br.trace:
        assert np.array_equal(open_before, prev)
        now = set(res.committed_now)
        assert all(not prev[i] for i in now)                  # only open rows commit
        for i in now:
            assert res.stats["argmax"][i] >= 0
        prev = prev.copy()
        prev[list(now)] = 1
    assert prev.all()
    for open_before, res in br.trace:
        for i in res.committed_now:
            assert br.tokens[i] == res.stats["argmax"][i]     # token = argmax of its commit round


@pytest.mark.parametrize("k", [1, 3, 8])
def test_loop_fixed_k_rounds(k):
    m = _model()
    kv = KVCache.empty(SMALL, 32)
    prefill(m, kv, synth.prompt_ids(SMALL, 8, 3), Prec())
    br = decode_block(m, kv, CommitRule(FIXED_K, k=k, max_rounds=8), Prec())
    assert br.rounds == -(-SMALL.block // k)
    assert br.n_new == [min(k, SMALL.block - k * r) for r in range(br.rounds)]


def test_resume_from_block_boundary():
    m = _model()
    prompt = synth.prompt_ids(SMALL, 8, 5)
    rule = CommitRule(THRESHOLD, tau=0.9, forced_top1=True, max_rounds=8)
    full, _, _ = generate(m, prompt, 3, rule, Prec(), cap=64)
    part, _, kv = generate(m, prompt, 1, rule, Prec(), cap=64)
    # restart from (tokens so far, KV cache, length) in a fresh copy
    kv2 = kv.copy()
    rest = [decode_block(m, kv2, rule, Prec()).tokens for _ in range(2)]
    np.testing.assert_array_equal(np.concatenate([part] + rest), full)


def test_max_rounds_cap_commits_everything():
    m = _model()
    kv = KVCache.empty(SMALL, 32)
    prefill(m, kv, synth.prompt_ids(SMALL, 8, 3), Prec())
    rule = CommitRule(THRESHOLD, tau=1.5, forced_top1=False, max_rounds=3)   # nobody can clear tau
    br = decode_block(m, kv, rule, Prec())
    assert br.rounds == 3 and br.n_new == [0, 0, SMALL.block]
    from oracle import FLAG_HIT_MAX_ROUNDS
    assert br.flags & FLAG_HIT_MAX_ROUNDS

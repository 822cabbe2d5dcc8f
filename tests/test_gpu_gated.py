"""GPU: the gated threshold block decode (dlm_decode_block_gated) produces what
dlm_decode_block produces -- tokens, round state and the whole KV cache, bitwise -- whatever
the segment length, for blocks that end in round 0, in a few rounds and at max_rounds."""
import sys

import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import require_gpu, storage

pytestmark = pytest.mark.gpu

SMALL = synth.small_shape(synth.QWEN4B, name="small-bf16", n_layers=2, d=512, hq=8, hkv=2, head_dim=64, ffn=1024,
                          vocab=3001)


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _dlm():
    require_gpu()
    import block_diffusion_decoding_denoise_amd as dlm
    dlm.lib()
    return dlm


def _run(dlm, m, prompt, n_blocks, rule, gated, seg):
    m.set_len(0)
    for x in m.k + m.v:
        x.zero_()
    m.prefill(torch.from_numpy(prompt))
    toks, states = [], []
    for _ in range(n_blocks):
        if gated:
            m.decode_block_gated(rule, seg_rounds=seg)
        else:
            m.decode_block(rule)
        torch.cuda.synchronize()
        toks.append(m.tokens.clone())
        states.append(dlm.state_dict(m.state))
    return torch.stack(toks), states, [x.clone() for x in m.k], [x.clone() for x in m.v]


@pytest.mark.parametrize("tau,max_rounds,seg", [(0.0, 32, 1), (0.0, 32, 4), (0.9, 32, 3), (0.9, 5, 2), (0.9, 7, 16)],
                         ids=["round0-seg1", "round0-seg4", "32rounds-seg3", "maxrounds5-seg2", "seg-longer-than-block"])
def test_gated_equals_block_graph(tau, max_rounds, seg):
    dlm = _dlm()
    _say(f"gated decode: tau {tau}, max rounds {max_rounds}, segments of {seg}")
    w = synth.Weights(SMALL, 1320)
    m = dlm.Model(SMALL, {n: storage(w[n], "bf16") for n in w.names_dense()}, cap=64 + 3 * 32)
    prompt = synth.prompt_ids(SMALL, 64, 1320)
    rule = dlm.CommitRule.threshold(tau, True, max_rounds)
    t0, s0, k0, v0 = _run(dlm, m, prompt, 2, rule, False, seg)
    t1, s1, k1, v1 = _run(dlm, m, prompt, 2, rule, True, seg)
    assert s0 == s1
    assert torch.equal(t0, t1)
    for a, b in zip(k0 + v0, k1 + v1):
        assert torch.equal(a, b)
    _say(f"  rounds per block {[st['round'] for st in s1]}")


def test_gated_fixed_k_takes_the_block_graph():
    dlm = _dlm()
    w = synth.Weights(SMALL, 1321)
    m = dlm.Model(SMALL, {n: storage(w[n], "bf16") for n in w.names_dense()}, cap=64 + 3 * 32)
    prompt = synth.prompt_ids(SMALL, 64, 1321)
    rule = dlm.CommitRule.fixed_k(6)
    t0, s0, _, _ = _run(dlm, m, prompt, 1, rule, False, 2)
    n_graphs = dlm.lib().dlm_model_graph_count(m.handle)
    t1, s1, _, _ = _run(dlm, m, prompt, 1, rule, True, 2)
    assert torch.equal(t0, t1) and s0 == s1
    assert dlm.lib().dlm_model_graph_count(m.handle) == n_graphs     # the same cached graph


def test_gated_rejects_bad_segment_length():
    dlm = _dlm()
    w = synth.Weights(SMALL, 1322)
    m = dlm.Model(SMALL, {n: storage(w[n], "bf16") for n in w.names_dense()}, cap=96)
    with pytest.raises(RuntimeError):
        m.decode_block_gated(dlm.CommitRule.threshold(0.5, True, 8), seg_rounds=0)

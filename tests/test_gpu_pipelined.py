"""GPU: a block's commit pass carried by the next block's round 0 (dlm_decode_block_pipelined).

The pipelined sequence must give the same tokens, round states and KV cache as decoding each
block with its own commit pass.  For dense bf16 models with 32-row blocks the commit rows and
round 0 share one 64-row forward; every row of it runs the same arithmetic in the same order
as in the separate passes (each row's GEMM outputs come from their own matrix-core columns
with the same contraction order, the attention of each query block sees the same keys and
splits), so the comparison is bitwise.  The f32 model runs the commit pass on its own and is
compared with the oracle.
"""
import sys

import numpy as np
import pytest
import torch

import synth
import oracle
from oracle import Prec, OracleModel, CommitRule as OCommitRule
from tests.gpu_util import require_gpu, storage

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _dlm():
    require_gpu()
    import block_diffusion_decoding_denoise_amd as dlm
    dlm.lib()
    return dlm


def _model(shape, seed, cap, kv_scales=None, fused_layers=False):
    """fused_layers: False (per-op kernels), True (one launch per sublayer) or "attn-out"
    (per-op kernels with the attention-output projection inside the attention launch)."""
    dlm = _dlm()
    w = synth.Weights(shape, seed)
    up = {n: storage(w[n], shape.dtype) for n in w.names_dense()}
    if fused_layers == "attn-out":
        return dlm.Model(shape, up, cap=cap, kv_scales=kv_scales, layer_path=dlm.DLM_LAYERS_ATTN_OUT), w
    return dlm.Model(shape, up, cap=cap, kv_scales=kv_scales, fused_layers=fused_layers), w


def _run(dlm, m, prompt, n_blocks, rule, pipelined):
    toks, states = m.generate(torch.from_numpy(prompt), n_blocks, rule, pipelined=pipelined)
    torch.cuda.synchronize()
    n = len(prompt) + 32 * n_blocks
    assert int(m.len_dev.item()) == n
    k = [x[:, :n].clone() for x in m.k]
    v = [dlm.v_cache_to_natural(x)[:, :n].clone() for x in m.v]
    return toks, states, k, v


SMALL = synth.small_shape(synth.QWEN4B, name="small-bf16", n_layers=2, d=512, hq=8, hkv=2, head_dim=64, ffn=1024,
                          vocab=3001)
# the 4B layer shapes (row-owned gate/up with 3 sub-tiles, QKV with 24 rows per workgroup,
# stream-K attention-output and down projections with their real partial counts)
QWEN4B_2L = synth.small_shape(synth.QWEN4B, name="qwen4b-2-layers", n_layers=2)
# the smallest model on the fused layer path (8 kv heads, one per XCD, 4 query heads of 128 each)
FUSED_SMALL = synth.small_shape(synth.QWEN4B, name="fused-small", n_layers=2, d=512, ffn=1024, vocab=3001)


@pytest.mark.parametrize("shape,seed,prompt_len,n_blocks,rule_args,kv_scales,fused", [
    (SMALL, 1234, 64, 3, ("fixed_k", 6), None, False),
    (SMALL, 1235, 32, 2, ("threshold", 0.5, True, 32), None, False),
    (SMALL, 1236, 96, 2, ("fixed_k", 32), None, False),
    (QWEN4B_2L, 1234, 256, 3, ("fixed_k", 6), None, False),
    (SMALL, 1237, 64, 3, ("fixed_k", 6), (0.125, 0.0625), False),
    (QWEN4B_2L, 1238, 256, 2, ("fixed_k", 6), (0.25, 0.125), False),
    (FUSED_SMALL, 1241, 64, 3, ("fixed_k", 6), None, True),
    (FUSED_SMALL, 1242, 32, 2, ("threshold", 0.5, True, 32), None, True),
    (FUSED_SMALL, 1243, 64, 2, ("fixed_k", 6), (0.07, 0.11), True),
    (QWEN4B_2L, 1245, 256, 3, ("fixed_k", 6), None, True),
    (FUSED_SMALL, 1246, 64, 3, ("fixed_k", 6), None, "attn-out"),
    (FUSED_SMALL, 1247, 32, 2, ("threshold", 0.5, True, 32), (0.07, 0.11), "attn-out"),
    (QWEN4B_2L, 1248, 256, 2, ("fixed_k", 6), None, "attn-out"),
], ids=["small-k6", "small-threshold", "small-k32", "qwen4b-2l-k6", "small-k6-fp8-cache", "qwen4b-2l-k6-fp8-cache",
        "fused-small-k6", "fused-small-threshold", "fused-small-k6-fp8-cache", "fused-qwen4b-2l-k6",
        "attn-out-small-k6", "attn-out-small-threshold-fp8-cache", "attn-out-qwen4b-2l-k6"])
def test_pipelined_bitexact_bf16(shape, seed, prompt_len, n_blocks, rule_args, kv_scales, fused):
    dlm = _dlm()
    _say(f"pipelined vs separate commit passes: {shape.name} seed {seed} prompt {prompt_len} "
         f"blocks {n_blocks} rule {rule_args} kv_scales {kv_scales} fused layers {fused}")
    m, _ = _model(shape, seed, cap=prompt_len + 32 * n_blocks, kv_scales=kv_scales, fused_layers=fused)
    rule = getattr(dlm.CommitRule, rule_args[0])(*rule_args[1:])
    prompt = synth.prompt_ids(shape, prompt_len, seed)
    t0, s0, k0, v0 = _run(dlm, m, prompt, n_blocks, rule, pipelined=False)
    t1, s1, k1, v1 = _run(dlm, m, prompt, n_blocks, rule, pipelined=True)
    assert s0 == s1
    assert torch.equal(t0, t1)
    for l in range(shape.n_layers):
        assert torch.equal(k0[l], k1[l]), f"layer {l} keys"
        assert torch.equal(v0[l], v1[l]), f"layer {l} values"
    # replaying the captured graphs gives the same again
    t2, s2, k2, _ = _run(dlm, m, prompt, n_blocks, rule, pipelined=True)
    assert torch.equal(t1, t2) and s1 == s2
    assert all(torch.equal(a, b) for a, b in zip(k1, k2))


MOE_SMALL = synth.small_shape(synth.MOE16B, name="moe-small-pipelined", n_layers=2, d=256, hq=4, hkv=2, head_dim=64,
                              vocab=1000, n_experts=32, expert_ffn=128, top_k=4, n_shared=1)
# the MoE model's per-layer shapes (256 experts, top-8, d 2048), two layers
MOE_E256 = synth.small_shape(synth.MOE16B, name="moe-e256-2-layers", n_layers=2, vocab=4096)


@pytest.mark.parametrize("shape,seed,prompt_len,n_blocks,rule_args,kv_scales", [
    (MOE_SMALL, 1234, 64, 3, ("fixed_k", 6), None),
    (MOE_SMALL, 1235, 32, 2, ("threshold", 0.5, True, 32), None),
    (MOE_E256, 1236, 64, 3, ("fixed_k", 6), None),
    (MOE_SMALL, 1240, 64, 3, ("fixed_k", 6), (0.125, 0.125)),
], ids=["moe-small-k6", "moe-small-threshold", "moe-e256-k6", "moe-small-k6-fp8-cache"])
def test_pipelined_bitexact_moe(shape, seed, prompt_len, n_blocks, rule_args, kv_scales):
    """MoE models: the 64-row fused pass routes the previous block's commit rows and round 0's
    rows together (up to 64 rows per expert, shared experts in two slots); every row's routing,
    expert products and slot outputs are those of the separate passes, so tokens, round states
    and caches are bitwise equal."""
    dlm = _dlm()
    _say(f"pipelined MoE vs separate commit passes: {shape.name} seed {seed} prompt {prompt_len} "
         f"blocks {n_blocks} rule {rule_args}")
    from tests.gpu_util import moe_device_weights
    w = synth.Weights(shape, seed)
    dev = {n: storage(w[n], "bf16") for n in w.names_dense() if not n.endswith(".router")}
    dev.update(moe_device_weights(w))
    m = dlm.Model(shape, dev, cap=prompt_len + 32 * n_blocks, kv_scales=kv_scales)
    rule = getattr(dlm.CommitRule, rule_args[0])(*rule_args[1:])
    prompt = synth.prompt_ids(shape, prompt_len, seed)
    t0, s0, k0, v0 = _run(dlm, m, prompt, n_blocks, rule, pipelined=False)
    t1, s1, k1, v1 = _run(dlm, m, prompt, n_blocks, rule, pipelined=True)
    assert s0 == s1
    assert torch.equal(t0, t1)
    for l in range(shape.n_layers):
        assert torch.equal(k0[l], k1[l]), f"layer {l} keys"
        assert torch.equal(v0[l], v1[l]), f"layer {l} values"


@pytest.mark.parametrize("shape,seed,prompt_len,fused", [(SMALL, 1237, 96, False), (QWEN4B_2L, 1238, 64, False),
                                                         (MOE_SMALL, 1239, 160, False), (FUSED_SMALL, 1244, 160, True),
                                                         (FUSED_SMALL, 1249, 160, "attn-out")],
                         ids=["small-3blocks", "qwen4b-2l", "moe-small-5blocks", "fused-small-5blocks",
                              "attn-out-small-5blocks"])
def test_prefill_pairs_bitexact(shape, seed, prompt_len, fused):
    """Prefill with 64-row forwards (two prompt blocks per pass, dlm_prefill_rows with 64 rows):
    the cache equals the one built block by block (one prefill call per block), bitwise."""
    dlm = _dlm()
    _say(f"prefill in block pairs vs block by block: {shape.name} seed {seed} prompt {prompt_len}")
    if shape.n_experts:
        from tests.gpu_util import moe_device_weights
        w = synth.Weights(shape, seed)
        dev = {n: storage(w[n], "bf16") for n in w.names_dense() if not n.endswith(".router")}
        dev.update(moe_device_weights(w))
        m = dlm.Model(shape, dev, cap=prompt_len + 32)
    else:
        m, _ = _model(shape, seed, cap=prompt_len + 32, fused_layers=fused)
    prompt = torch.from_numpy(synth.prompt_ids(shape, prompt_len, seed))
    m.set_len(0)
    m.prefill(prompt, max_rows=64)
    torch.cuda.synchronize()
    assert int(m.len_dev.item()) == prompt_len
    k0 = [x[:, :prompt_len].clone() for x in m.k]
    v0 = [dlm.v_cache_to_natural(x)[:, :prompt_len].clone() for x in m.v]
    m.set_len(0)
    for b in range(prompt_len // 32):
        m.prefill(prompt[32 * b:32 * (b + 1)])
    torch.cuda.synchronize()
    assert int(m.len_dev.item()) == prompt_len
    for l in range(shape.n_layers):
        assert torch.equal(k0[l], m.k[l][:, :prompt_len]), f"layer {l} keys"
        assert torch.equal(v0[l], dlm.v_cache_to_natural(m.v[l])[:, :prompt_len]), f"layer {l} values"


def test_pipelined_tiny_fp32_matches_oracle():
    """f32: the pending commit pass runs on its own; tokens and rounds bit-exact with the
    oracle's block loop, and the final cache equal to the oracle's."""
    dlm = _dlm()
    s = synth.TINY
    _say("pipelined tiny fp32, seed 1234")
    m, w = _model(s, 1234, cap=64 + 4 * 32)
    prompt = synth.prompt_ids(s, 64, 1234)
    rule = dlm.CommitRule.threshold(0.9, True, 32)
    toks, states, k, v = _run(dlm, m, prompt, 4, rule, pipelined=True)
    om = OracleModel(s, w, Prec("f32"))
    ref, blocks, kv = oracle.generate(om, prompt, 4, OCommitRule(0, 0.9, 1, True, 32), Prec("f32"))
    np.testing.assert_array_equal(toks.numpy(), ref)
    for b, (st, br) in enumerate(zip(states, blocks)):
        assert st["round"] == br.rounds and st["n_new"] == br.n_new and st["flags"] == br.flags, f"block {b}"
    n = 64 + 4 * 32
    for l in range(s.n_layers):
        np.testing.assert_allclose(k[l].cpu().numpy(), kv.k[l][:, :n], atol=2e-5, rtol=1e-4)
        np.testing.assert_allclose(v[l].cpu().numpy(), kv.v[l][:, :n], atol=2e-5, rtol=1e-4)


def test_pipelined_rejects_aliased_tokens():
    dlm = _dlm()
    m, _ = _model(SMALL, 1234, cap=128)
    rule = dlm.CommitRule.fixed_k(6)
    with pytest.raises(dlm.DlmError):
        m.decode_block_pipelined(rule, m.tokens, m.tokens)

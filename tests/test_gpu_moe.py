"""GPU parity of the routed-expert (MXFP4 / MXFP8) FFN inside the denoising round."""
import sys

import numpy as np
import pytest
import torch

import synth
import oracle
from oracle import Prec, OracleModel, KVCache
from tests.gpu_util import require_gpu, storage, moe_device_weights, to_bits
from tests.test_gpu_model import _lockstep, _unpack_act

pytestmark = pytest.mark.gpu


# Residual-stream tolerance with MXFP8 activations: both sides quantise to e4m3 (3 mantissa
# bits, one step = 2^-3 relative) from inputs that differ at bf16 precision, so a few percent of
# the codes land one step apart; their effect on a row's residual is a few percent of its norm.
MX_RESID_TOL = 5e-2


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _moe_shape(**kw):
    base = dict(name="moe-small", n_layers=2, d=256, hq=4, hkv=2, head_dim=64, vocab=1000, n_experts=32,
                expert_ffn=128, top_k=4, n_shared=1)
    base.update(kw)
    return synth.small_shape(synth.MOE16B, **base)


def _model(shape, seed, cap):
    require_gpu()
    import block_diffusion_decoding_denoise_amd as dlm
    dlm.lib()
    w = synth.Weights(shape, seed)
    dev = {n: storage(w[n], "bf16") for n in w.names_dense() if not n.endswith(".router")}
    dev.update(moe_device_weights(w))
    return dlm, dlm.Model(shape, dev, cap=cap), w


def _round0_residual(shape, seed, prompt_len):
    """Round 0 of the first block after a prefill: the residual stream after the last layer,
    GPU against the oracle (same bf16 KV cache from the GPU prefill)."""
    dlm, m, w = _model(shape, seed, cap=prompt_len + 64)
    prompt = synth.prompt_ids(shape, prompt_len, seed)
    m.set_len(0)
    m.prefill(torch.from_numpy(prompt))
    m.decode_begin()
    torch.cuda.synchronize()
    L = int(m.len_dev.item())
    kv = KVCache([t.float().cpu().numpy().astype(np.float64) for t in m.k],
                 [dlm.v_cache_to_natural(t).float().cpu().numpy().astype(np.float64) for t in m.v], L)
    m.decode_round(dlm.CommitRule.fixed_k(4))
    torch.cuda.synchronize()
    gx = m.view("x", (shape.block, shape.d), torch.float32).cpu().numpy()
    om = OracleModel(shape, w, Prec("bf16"))
    prec = Prec("bf16")
    x0 = np.tile(om.get("mask_emb"), (shape.block, 1))          # round 0: every row open, x = m
    h = oracle.forward_block(om, x0, kv, L, prec)
    return gx, h


def _e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """OCP e4m3 code -> value (bias 7, 3 mantissa bits, exponent field 0 = subnormal)."""
    c = codes.astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 7
    return s * np.where(e == 0, m / 8.0 * 2.0 ** -6, (1 + m / 8.0) * np.exp2(e - 7.0))


MOE_ROUTING_SHAPE = dict(name="moe-1l-e256", n_layers=1, d=2048, hq=16, hkv=4, head_dim=128, n_experts=256,
                         expert_ffn=512, top_k=8, n_shared=1)


@pytest.mark.parametrize("kw", [dict(name="moe-1l", n_layers=1), MOE_ROUTING_SHAPE], ids=["small", "e256-top8"])
def test_moe_stages_one_layer(kw):
    """One MoE layer, round 0: router logits, MXFP8 input codes, the top-k routing, the per-row
    output slots, each against the oracle's own step from the oracle's input.  The second case
    has the MoE model's routing shape (256 routed experts, top-8, d 2048)."""
    s = _moe_shape(**kw)
    _say(f"moe stages {s.name}: d={s.d} E={s.n_experts} top{s.top_k}")
    dlm, m, w = _model(s, 1234, cap=96)
    prompt = synth.prompt_ids(s, 32, 1234)
    m.set_len(0)
    m.prefill(torch.from_numpy(prompt))
    m.decode_begin()
    torch.cuda.synchronize()
    L = int(m.len_dev.item())
    kv = KVCache([t.float().cpu().numpy().astype(np.float64) for t in m.k],
                 [dlm.v_cache_to_natural(t).float().cpu().numpy().astype(np.float64) for t in m.v], L)
    m.decode_round(dlm.CommitRule.fixed_k(4))
    torch.cuda.synchronize()
    B, d, E, NS, F = s.block, s.d, s.n_experts, s.top_k + s.n_shared, s.expert_ffn
    prec = Prec("bf16")
    om = OracleModel(s, w, prec)
    x0 = np.tile(om.get("mask_emb"), (B, 1))
    h1 = oracle.block.attention_sublayer(x0, om.layer(0), kv.k[0], kv.v[0], L, s, prec)
    f = prec.act(oracle.block.rmsnorm(h1, om.get("l0.ffn_norm"), s.eps))
    # the GPU's own MoE input (packed bf16) agrees with the oracle's to bf16 precision (the
    # attention kernel's internal roundings are not mirrored); the later stages are checked
    # from the GPU's input
    f_gpu = _unpack_act(to_bits(m.view("xn", (32, d), torch.bfloat16)), d)[:B]
    assert np.linalg.norm(f_gpu - f) / np.linalg.norm(f) < 1e-2
    # router logits from that input
    g_logits = m.view("moe_logits", (32, E), torch.float32).cpu().numpy()[:B]
    np.testing.assert_allclose(g_logits, f_gpu @ om.get("l0.router").T, atol=1e-4, rtol=1e-4)
    # MXFP8 input: the exact MX rule applied to the GPU's input
    xq = _e4m3_decode(m.view("moe_xq", (32, d), torch.uint8).cpu().numpy()[:B])
    xs = m.view("moe_xs", (32, d // 32), torch.uint8).cpu().numpy()[:B].astype(np.float64)
    g_x = (xq.reshape(B, d // 32, 32) * np.exp2(xs - 127)[..., None]).reshape(B, d)
    np.testing.assert_array_equal(g_x, oracle.mxfp8_quant_dequant(f_gpu))
    f = f_gpu
    # routing: each row's top-k by rank, with its probabilities
    ids, wts, probs = oracle.router_topk(f, om.get("l0.router"), s.top_k)
    g_ids = m.view("moe_ids", (32, s.top_k), torch.int32).cpu().numpy()[:B]
    g_w = m.view("moe_wts", (32, s.top_k), torch.float32).cpu().numpy()[:B].astype(np.float64)
    # the same experts in the same ranks, except where the oracle's own probabilities are within
    # 1e-3 (relative) of each other around the difference (near ties, counted)
    near = 0
    for i in range(B):
        if (g_ids[i] == ids[i]).all():
            continue
        p_sorted = np.sort(probs[i])[::-1]
        gaps = np.abs(np.diff(p_sorted[:s.top_k + 1])) / p_sorted[:s.top_k + 1].max()
        assert gaps.min() < 1e-3, f"row {i}: routing {g_ids[i]} vs {ids[i]}"
        near += 1
    assert near <= B // 4
    np.testing.assert_allclose(g_w[g_ids == ids], wts[g_ids == ids], rtol=1e-4)
    # per-slot outputs from the GPU's own MXFP8 input and routing: routed expert j of row i,
    # weighted, and the shared expert
    y = m.view("moe_y", (32 * NS, d), torch.float32).cpu().numpy()
    aq = _e4m3_decode(m.view("moe_aq", (32 * NS, F), torch.uint8).cpu().numpy())
    asc = m.view("moe_as", (32 * NS, F // 32), torch.uint8).cpu().numpy().astype(np.float64)
    g_act = (aq.reshape(-1, F // 32, 32) * np.exp2(asc - 127)[..., None]).reshape(-1, F)
    dec = {}
    for i in range(B):
        for j in range(NS):
            e = g_ids[i, j] if j < s.top_k else E + (j - s.top_k)
            if e not in dec:
                dec[e] = [oracle.mxfp4_decode(*w.expert(0, e, which)) for which in ("wg", "wu", "wd")]
            wg, wu, wd = dec[e]
            # act in MXFP8: the oracle's quantisation of its own act; codes differ only where the
            # f32 and f64 act values fall on different sides of an e4m3 rounding boundary
            act = oracle.mxfp8_quant_dequant(oracle.block.swiglu(g_x[i] @ wg.T, g_x[i] @ wu.T))
            a_err = np.linalg.norm(g_act[i * NS + j] - act) / np.linalg.norm(act)
            assert a_err < 1e-2, ("act", i, j, e, a_err)
            ref = oracle.moe.expert_ffn(g_x[i:i + 1], wg, wu, wd)[0] * (g_w[i, j] if j < s.top_k else 1.0)
            got = y[i * NS + j]
            err = np.linalg.norm(got - ref) / np.linalg.norm(ref)
            assert err < 2e-2, ("y", i, j, e, err)


def test_moe_small_round0_residual():
    s = _moe_shape()
    _say(f"moe round-0 residual d={s.d} E={s.n_experts} top{s.top_k}")
    gx, h = _round0_residual(s, 1234, 32)
    err = np.linalg.norm(gx - h, axis=1) / np.linalg.norm(h, axis=1)
    assert err.max() < MX_RESID_TOL, err.max()


def test_moe_expert_shape_round0_residual():
    """d 2048, expert FFN 512, top-8 + 1 shared expert: the MoE model's per-expert shapes."""
    s = _moe_shape(name="moe-d2048", n_layers=1, d=2048, hq=16, hkv=4, head_dim=128, n_experts=32,
                   expert_ffn=512, top_k=8, n_shared=1)
    _say(f"moe round-0 residual d={s.d} E={s.n_experts} F={s.expert_ffn} top{s.top_k}")
    gx, h = _round0_residual(s, 1235, 32)
    err = np.linalg.norm(gx - h, axis=1) / np.linalg.norm(h, axis=1)
    assert err.max() < MX_RESID_TOL, err.max()


def test_moe_lockstep():
    """Every round of a block: head statistics and commits against the oracle recomputed from
    the GPU's own round-start state."""
    require_gpu()
    import tests.test_gpu_model as tg
    s = _moe_shape()
    orig = tg._upload
    tg._upload = lambda w: {**{n: storage(w[n], "bf16") for n in w.names_dense() if not n.endswith(".router")},
                            **moe_device_weights(w)}
    try:
        _lockstep(s, 1236, 32, 1, (1, 0.0, 6, 0, 32))
    finally:
        tg._upload = orig

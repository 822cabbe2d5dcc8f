"""GPU: the prompt in wide forwards (dlm_prefill: up to 8 blocks, 256 rows, per forward on
dense bf16 models) against the oracle's prefill, which runs one commit pass per block.

Layer 0 reads only the prompt's embedding rows, so its K/V must agree to a bf16 rounding.
Later layers carry the attention kernel's bf16 probabilities (which the oracle keeps exact):
their relative deviation must stay within twice that of the oracle's prefill under the
kernel-arithmetic error model (tests/parity.py), plus 1e-3."""
import sys

import numpy as np
import pytest
import torch

import synth
import oracle
from oracle import Prec, OracleModel, KVCache
from tests.gpu_util import require_gpu, storage
from tests.test_gpu_model import _kernel_arithmetic

pytestmark = pytest.mark.gpu

SMALL = synth.small_shape(synth.QWEN4B, name="small-bf16", n_layers=2, d=512, hq=8, hkv=2, head_dim=64, ffn=1024,
                          vocab=3001)
QWEN4B_2L = synth.small_shape(synth.QWEN4B, name="qwen4b-2-layers", n_layers=2)


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _dlm():
    require_gpu()
    import block_diffusion_decoding_denoise_amd as dlm
    dlm.lib()
    return dlm


def _model(dlm, s, seed, cap):
    w = synth.Weights(s, seed)
    return dlm.Model(s, {n: storage(w[n], "bf16") for n in w.names_dense()}, cap=cap), w


def _gpu_cache(dlm, m, n):
    ks = [m.k[l][:, :n].float().cpu().numpy().astype(np.float64) for l in range(len(m.k))]
    vs = [dlm.v_cache_to_natural(m.v[l])[:, :n].float().cpu().numpy().astype(np.float64) for l in range(len(m.v))]
    return ks, vs


def _check_against_oracle(s, w, prompt, ks, vs):
    n = len(prompt)
    om = OracleModel(s, w, Prec("bf16"))
    kv = KVCache.empty(s, n)
    oracle.prefill(om, kv, prompt, Prec("bf16"))
    kvm = KVCache.empty(s, n)
    with _kernel_arithmetic():
        oracle.prefill(om, kvm, prompt, Prec("bf16"))
    for l in range(s.n_layers):
        for which, g, o, mo in (("k", ks[l], kv.k[l][:, :n], kvm.k[l][:, :n]),
                                ("v", vs[l], kv.v[l][:, :n], kvm.v[l][:, :n])):
            e_gpu = np.linalg.norm(g - o) / np.linalg.norm(o)
            e_model = np.linalg.norm(mo - o) / np.linalg.norm(o)
            _say(f"  layer {l} {which}: GPU vs oracle {e_gpu:.3e}, model vs oracle {e_model:.3e}")
            assert e_gpu <= 2 * e_model + 1e-3, (l, which, e_gpu, e_model)
            if l == 0:
                # identical bf16 inputs: a value differs only where fp32 and fp64 round it to
                # different sides of a bf16 rounding boundary (one unit in the last place); a
                # result that nearly cancels (|o| far below its summands) also carries the fp32
                # summation error, well under 1e-5 of the values' RMS
                ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(o), 1e-30))) - 7)
                floor = 1e-5 * np.sqrt(np.mean(o * o))
                bad = np.argwhere(np.abs(g - o) > 1.01 * ulp + floor)
                for i in bad[:8]:
                    i = tuple(i)
                    _say(f"    {which}{i}: gpu {g[i]:.8g} oracle {o[i]:.8g} ulp {ulp[i]:.3g}")
                assert len(bad) == 0, f"{len(bad)} elements beyond one bf16 ulp"
                assert np.mean(g != o) < 1e-2, np.mean(g != o)


@pytest.mark.parametrize("n_blocks", [1, 2, 3, 8, 11], ids=["1block", "2blocks", "3blocks", "8blocks", "11blocks"])
def test_wide_prefill_matches_oracle_small(n_blocks):
    """1 and 2 blocks take the commit-pass and pair paths, 3 and 8 one wide forward, 11 a wide
    forward of 8 blocks followed by one of 3 (which attends to the first 256 positions)."""
    dlm = _dlm()
    n = 32 * n_blocks
    _say(f"wide prefill vs oracle: small model, {n} prompt tokens")
    m, w = _model(dlm, SMALL, 1300 + n_blocks, cap=n + 32)
    prompt = synth.prompt_ids(SMALL, n, 1300 + n_blocks)
    m.set_len(0)
    m.prefill(torch.from_numpy(prompt))
    torch.cuda.synchronize()
    assert int(m.len_dev.item()) == n
    ks, vs = _gpu_cache(dlm, m, n)
    _check_against_oracle(SMALL, w, prompt, ks, vs)


def test_wide_prefill_matches_oracle_qwen4b_layers():
    """The 4B layer shapes (2 layers): a 256-token prompt in one 256-row forward."""
    dlm = _dlm()
    _say("wide prefill vs oracle: 4B layer shapes, 256 prompt tokens")
    m, w = _model(dlm, QWEN4B_2L, 1310, cap=256 + 32)
    prompt = synth.prompt_ids(QWEN4B_2L, 256, 1310)
    m.set_len(0)
    m.prefill(torch.from_numpy(prompt))
    torch.cuda.synchronize()
    ks, vs = _gpu_cache(dlm, m, 256)
    _check_against_oracle(QWEN4B_2L, w, prompt, ks, vs)


@pytest.mark.parametrize("max_rows", [32, 64, 96, 256])
def test_prefill_rows_agree(max_rows):
    """dlm_prefill_rows at several forward widths against dlm_prefill (8-block forwards): the
    same cache up to float summation order -- layer 0 to one bf16 unit in the last place, the
    last layer within 1e-2 relative."""
    dlm = _dlm()
    s = QWEN4B_2L
    n = 320
    _say(f"prefill rows {max_rows} vs wide: 4B layer shapes, {n} tokens")
    m, w = _model(dlm, s, 1311, cap=n + 32)
    prompt = torch.from_numpy(synth.prompt_ids(s, n, 1311))
    m.set_len(0)
    m.prefill(prompt)
    torch.cuda.synchronize()
    k0, v0 = _gpu_cache(dlm, m, n)
    m.set_len(0)
    m.prefill(prompt, max_rows=max_rows)
    torch.cuda.synchronize()
    assert int(m.len_dev.item()) == n
    k1, v1 = _gpu_cache(dlm, m, n)
    for l in range(s.n_layers):
        for a, b in ((k0[l], k1[l]), (v0[l], v1[l])):
            if l == 0:
                ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(a), 1e-30))) - 7)
                assert np.all(np.abs(a - b) <= 1.01 * ulp + 1e-5 * np.sqrt(np.mean(a * a)))
            else:
                assert np.linalg.norm(a - b) / np.linalg.norm(a) < 1e-2


def test_prefill_rows_rejects_less_than_a_block():
    dlm = _dlm()
    m, _ = _model(dlm, SMALL, 1312, cap=96)
    prompt = torch.from_numpy(synth.prompt_ids(SMALL, 64, 1312))
    with pytest.raises(RuntimeError):
        m.prefill(prompt, max_rows=16)

"""GPU: the allocation-free attention call (dlm_block_attn_noalloc) gives the same bytes as
dlm_block_attn with a caller workspace, on two calls in a row (the second with a smaller input,
so the shared scratch holds the first call's partials when it starts)."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import require_gpu, storage

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _case(dlm, hq, hkv, D, B, L, cap, seed, fp8=False):
    _say(f"noalloc attention hq={hq} hkv={hkv} D={D} B={B} L={L} cap={cap} fp8={fp8} seed={seed}")
    q = storage(synth.stored_normal(seed, "na.q", (B, hq, D), 1.0, "bf16"), "bf16")
    if fp8:
        k = torch.from_numpy(synth.e4m3_codes(seed, "na.k8", (hkv, cap, D))).cuda()
        v = torch.from_numpy(synth.e4m3_codes(seed, "na.v8", (hkv, cap // 32, D, 32))).cuda()
        scales = (0.0625, 0.125)
    else:
        k = storage(synth.stored_normal(seed, "na.k", (hkv, cap, D), 1.0, "bf16"), "bf16")
        v = storage(synth.stored_normal(seed, "na.v", (hkv, cap // 32, D, 32), 1.0, "bf16"), "bf16")
        scales = None
    ref = dlm.block_attn(q, k, v, L, kv_scales=scales)
    got = dlm.block_attn_noalloc(q, k, v, L, kv_scales=scales)
    torch.cuda.synchronize()
    assert torch.isfinite(got.float()).all()
    assert torch.equal(got, ref), (got.float() - ref.float()).abs().max().item()


def test_noalloc_attention_two_calls_then_smaller():
    require_gpu()
    import block_diffusion_decoding_denoise_amd as dlm
    dlm.lib()
    assert dlm.lib().dlm_block_attn_noalloc_max_bytes() == 16 << 20
    _case(dlm, 32, 8, 128, 32, 4096, 4128, 1260)                 # 22 key splits per kv head
    _case(dlm, 16, 4, 128, 20, 300, 352, 1261)                   # a smaller call right after
    _case(dlm, 32, 8, 128, 32, 32768, 32800, 1262, fp8=True)     # the largest plan of the shape (32 splits)
    _case(dlm, 8, 2, 64, 7, 33, 96, 1263)


def test_noalloc_attention_rejects_a_plan_beyond_the_scratch():
    require_gpu()
    import block_diffusion_decoding_denoise_amd as dlm
    q = torch.zeros(32, 64, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(16, 32800, 128, dtype=torch.bfloat16, device="cuda")
    v = torch.zeros(16, 32800 // 32, 128, 32, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dlm.DlmError, match="split scratch"):
        dlm.block_attn_noalloc(q, k, v, 32768)

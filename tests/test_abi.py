"""CPU checks of the C-ABI library: it loads, exports every declared call, and rejects bad
arguments on the host before touching a device."""
import ctypes
import os
import re

import pytest

import block_diffusion_decoding_denoise_amd as dlm

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "dlm.h")

OK, ARG, SHAPE, DTYPE, WS, HIP, UNSUP = 0, -1, -2, -3, -4, -5, -6
FAKE = ctypes.c_void_p(0x10000)     # aligned, never dereferenced by a rejected call


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dlm_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_call():
    L = dlm.lib()
    names = _declared()
    assert len(names) >= 20
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing
    assert L.dlm_abi_version() == 2


def _attn(**kw):
    base = dict(dtype=dlm.DLM_BF16, hq=32, hkv=8, head_dim=128, block=32, cap=1024, softmax_scale=0.088,
                prefix_len=100, prefix_len_dev=None, max_prefix_len=100, kv_dtype=dlm.DLM_BF16, k_scale=1.0,
                v_scale=1.0)
    base.update(kw)
    return dlm.AttnDesc(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(hq=30), SHAPE), (dict(head_dim=96), SHAPE), (dict(block=33), SHAPE), (dict(prefix_len=1000), SHAPE),
    (dict(dtype=7), DTYPE), (dict(hkv=0), ARG), (dict(prefix_len=-1), ARG),
    (dict(kv_dtype=dlm.DLM_F32), DTYPE), (dict(dtype=dlm.DLM_F32, kv_dtype=dlm.DLM_FP8_E4M3), DTYPE),
    (dict(kv_dtype=dlm.DLM_FP8_E4M3, k_scale=0.0), ARG), (dict(kv_dtype=dlm.DLM_FP8_E4M3, v_scale=float("nan")), ARG),
    (dict(kv_dtype=dlm.DLM_FP8_E4M3, k_scale=float("inf")), ARG), (dict(kv_dtype=dlm.DLM_FP8_E4M3, head_dim=96), SHAPE),
])
def test_block_attn_validation(kw, code):
    d = _attn(**kw)
    L = dlm.lib()
    assert L.dlm_block_attn(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == code
    assert L.dlm_last_error()


def test_block_attn_null_and_workspace():
    L = dlm.lib()
    d = _attn()
    assert L.dlm_block_attn(None, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == ARG
    assert L.dlm_block_attn(ctypes.byref(d), None, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == ARG
    need = L.dlm_block_attn_ws_bytes(ctypes.byref(d))
    assert need > 0
    assert L.dlm_block_attn(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None) == WS
    misaligned = ctypes.c_void_p(0x10002)
    assert L.dlm_block_attn(ctypes.byref(d), misaligned, FAKE, FAKE, FAKE, FAKE, need, None) == ARG


def test_head_validation():
    L = dlm.lib()
    ok = dlm.HeadDesc(dlm.DLM_BF16, 32, 2560, 151936)
    need = L.dlm_head_rowstats_ws_bytes(ctypes.byref(ok))
    assert need > 151936 // 16
    args = [FAKE] * 9
    assert L.dlm_head_rowstats(ctypes.byref(dlm.HeadDesc(dlm.DLM_BF16, 65, 2560, 100)), *args, FAKE, need, None) == SHAPE
    assert L.dlm_head_rowstats(ctypes.byref(dlm.HeadDesc(dlm.DLM_BF16, 32, 2561, 100)), *args, FAKE, need, None) == SHAPE
    assert L.dlm_head_rowstats(ctypes.byref(dlm.HeadDesc(dlm.DLM_F32, 32, 512, 100)), *args, FAKE, need, None) == SHAPE
    assert L.dlm_head_rowstats(ctypes.byref(dlm.HeadDesc(5, 32, 256, 100)), *args, FAKE, need, None) == DTYPE
    assert L.dlm_head_rowstats(ctypes.byref(ok), *args, FAKE, need - 1, None) == WS
    assert L.dlm_head_rowstats(ctypes.byref(ok), None, *args[1:], FAKE, need, None) == ARG


def test_commit_validation():
    L = dlm.lib()
    r = dlm.CommitRule.fixed_k(0)
    assert L.dlm_commit(ctypes.byref(r), 32, FAKE, FAKE, FAKE, FAKE, FAKE, None) == ARG
    r = dlm.CommitRule.threshold(max_rounds=65)
    assert L.dlm_commit(ctypes.byref(r), 32, FAKE, FAKE, FAKE, FAKE, FAKE, None) == ARG
    r = dlm.CommitRule.threshold()
    assert L.dlm_commit(ctypes.byref(r), 65, FAKE, FAKE, FAKE, FAKE, FAKE, None) == SHAPE
    assert L.dlm_commit(ctypes.byref(r), 32, None, FAKE, FAKE, FAKE, FAKE, None) == ARG


def test_model_desc_validation():
    L = dlm.lib()
    good = dlm.ModelDesc(dlm.DLM_BF16, 36, 2560, 32, 8, 128, 9728, 151936, 32, 1e4, 1e-6, 0, 0, 0, 0)
    assert L.dlm_packed_bytes(ctypes.byref(good)) > 7_000_000_000
    bad = dlm.ModelDesc(dlm.DLM_BF16, 36, 2560, 32, 7, 128, 9728, 151936, 32, 1e4, 1e-6, 0, 0, 0, 0)
    assert L.dlm_packed_bytes(ctypes.byref(bad)) == 0
    layers = (dlm.LayerWeights * 36)()
    h = ctypes.c_void_p()
    assert L.dlm_model_create(ctypes.byref(good), FAKE, FAKE, FAKE, FAKE, layers, FAKE, ctypes.byref(h)) == ARG
    f32 = dlm.ModelDesc(dlm.DLM_F32, 2, 512, 4, 2, 64, 768, 4096, 32, 1e4, 1e-6, 0, 0, 0, 0)
    assert L.dlm_packed_bytes(ctypes.byref(f32)) == 0       # f32 models up to d = 256 only


def test_layer_path_packing():
    """Models whose attention-output projection runs inside the attention launch
    (DLM_LAYERS_ATTN_OUT) pack that matrix a second time, as 8 column slices: exactly one more
    d x (hq D) bf16 matrix per layer than the per-op path; models that launch does not serve
    pack the same bytes either way; an unknown layer path is rejected."""
    L = dlm.lib()

    def nbytes(path, d=2560, hq=32, hkv=8, D=128):
        desc = dlm.ModelDesc(dlm.DLM_BF16, 36, d, hq, hkv, D, 9728, 151936, 32, 1e4, 1e-6, 0, 0, 0, 0, path)
        return L.dlm_packed_bytes(ctypes.byref(desc))

    assert nbytes(dlm.DLM_LAYERS_ATTN_OUT) - nbytes(dlm.DLM_LAYERS_PER_OP) == 36 * 2560 * 4096 * 2
    for kw in ({"hkv": 4}, {"D": 64}, {"d": 3584}):          # not 8 groups of 4 x 128, or d > 3072
        assert nbytes(dlm.DLM_LAYERS_ATTN_OUT, **kw) == nbytes(dlm.DLM_LAYERS_PER_OP, **kw) > 0
    assert nbytes(3) == 0


def test_valid_call_without_device_is_unsupported():
    """A fully valid call reaches the device check; with no gfx950 device current it
    returns DLM_ERR_UNSUPPORTED (on a GPU machine this test is skipped)."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present")
    L = dlm.lib()
    r = dlm.CommitRule.threshold()
    assert L.dlm_commit(ctypes.byref(r), 32, FAKE, FAKE, FAKE, FAKE, FAKE, None) == UNSUP


def test_kv_cache_format_validation():
    """The KV descriptor's format is checked on the host before anything is enqueued: a cache
    in the model dtype or FP8 e4m3 (bf16 models) with finite positive scales is accepted; the
    workspace query returns 0 for anything else and leaves a message."""
    L = dlm.lib()
    desc = dlm.ModelDesc(dlm.DLM_BF16, 2, 256, 4, 2, 64, 512, 1000, 32, 1e4, 1e-6, 0, 0, 0, 0)
    layers = (dlm.LayerWeights * 2)()
    for lw in layers:
        for name, _ in dlm.LayerWeights._fields_[:9]:
            setattr(lw, name, FAKE.value)
    h = ctypes.c_void_p()
    assert L.dlm_model_create(ctypes.byref(desc), FAKE, FAKE, FAKE, FAKE, layers, FAKE, ctypes.byref(h)) == 0
    ptrs = (ctypes.c_void_p * 2)(FAKE.value, FAKE.value)
    try:
        def ws(kv_dtype, ks=1.0, vs=1.0):
            kv = dlm.KV(ptrs, ptrs, 256, FAKE.value, 256, kv_dtype, ks, vs)
            return L.dlm_decode_ws_bytes(h, ctypes.byref(kv))
        assert ws(dlm.DLM_BF16) > 0
        assert ws(dlm.DLM_FP8_E4M3, 0.125, 0.5) == ws(dlm.DLM_BF16)    # same workspace either way
        for bad in [(dlm.DLM_F32,), (dlm.DLM_MXFP4,), (dlm.DLM_FP8_E4M3, 0.0, 1.0), (dlm.DLM_FP8_E4M3, 1.0, -1.0),
                    (dlm.DLM_FP8_E4M3, float("nan"), 1.0), (dlm.DLM_FP8_E4M3, 1.0, float("inf"))]:
            assert ws(*bad) == 0, bad
            assert L.dlm_last_error()
    finally:
        L.dlm_model_destroy(h)


def test_graph_key_covers_cache_geometry_and_every_layer():
    """The key a block graph is cached under changes with the cache capacity, max_len, the FP8
    scales and any layer's K or V base (host only: a stale graph would replay wrong strides or
    write freed memory)."""
    L = dlm.lib()
    n_layers = 3
    desc = dlm.ModelDesc(dlm.DLM_BF16, n_layers, 256, 4, 2, 64, 512, 1000, 32, 1e4, 1e-6, 0, 0, 0, 0)
    layers = (dlm.LayerWeights * n_layers)()
    for lw in layers:
        for name, _ in dlm.LayerWeights._fields_[:9]:
            setattr(lw, name, FAKE.value)
    h = ctypes.c_void_p()
    assert L.dlm_model_create(ctypes.byref(desc), FAKE, FAKE, FAKE, FAKE, layers, FAKE, ctypes.byref(h)) == 0
    rule = dlm.CommitRule.fixed_k(6)
    words = (ctypes.c_uint64 * 256)()

    def key(k_ptrs, v_ptrs, cap=512, max_len=512, kv_dtype=dlm.DLM_BF16, ks=1.0, vs=1.0, pipelined=0):
        kp = (ctypes.c_void_p * n_layers)(*k_ptrs)
        vp = (ctypes.c_void_p * n_layers)(*v_ptrs)
        kv = dlm.KV(kp, vp, cap, FAKE.value, max_len, kv_dtype, ks, vs)
        n = L.dlm_block_graph_key(h, ctypes.byref(rule), ctypes.byref(kv), None, pipelined, FAKE, FAKE, FAKE,
                                  words, 256)
        assert n > 0, L.dlm_last_error()
        return tuple(words[:n])

    try:
        ks = [0x100000 * (i + 1) for i in range(n_layers)]
        vs = [0x1000000 * (i + 1) for i in range(n_layers)]
        base = key(ks, vs)
        assert key(ks, vs) == base
        assert key(ks, vs, cap=1024) != base
        assert key(ks, vs, max_len=256) != base
        assert key(ks[:2] + [0x900000], vs) != base          # the last layer's K reallocated
        assert key(ks, [vs[0], 0x9000000, vs[2]]) != base     # a middle layer's V reallocated
        assert key(ks, vs, kv_dtype=dlm.DLM_FP8_E4M3, ks=0.5, vs=0.5) != key(ks, vs, kv_dtype=dlm.DLM_FP8_E4M3,
                                                                           ks=0.25, vs=0.5)
        assert key(ks, vs, pipelined=1) != base
        small = (ctypes.c_uint64 * 2)()
        kv = dlm.KV((ctypes.c_void_p * n_layers)(*ks), (ctypes.c_void_p * n_layers)(*vs), 512, FAKE.value, 512,
                    dlm.DLM_BF16, 1.0, 1.0)
        assert L.dlm_block_graph_key(h, ctypes.byref(rule), ctypes.byref(kv), None, 0, FAKE, FAKE, FAKE, small,
                                     2) == ARG
        assert L.dlm_model_graph_count(h) == 0
    finally:
        L.dlm_model_destroy(h)

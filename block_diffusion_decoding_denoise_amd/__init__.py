"""Python binding of libdlm.so, the block-diffusion denoising-round library for MI355X.

Argument marshalling only: torch supplies device memory and the current HIP stream,
every step of the round runs in the library's HIP kernels.  The binding raises
DlmError when the library is missing or a call fails; there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libdlm.so")

DLM_F32, DLM_BF16, DLM_MXFP4, DLM_FP8_E4M3 = 0, 1, 2, 3
DLM_LAYERS_PER_OP, DLM_LAYERS_FUSED, DLM_LAYERS_ATTN_OUT = 0, 1, 2
THRESHOLD, FIXED_K = 0, 1
FLAG_HIT_MAX_ROUNDS, FLAG_NONFINITE = 1, 2
MAX_ROWS = 64
MAX_ROUNDS = 64


class DlmError(RuntimeError):
    pass


# ------------------------------------------------------------------ ABI structs
class AttnDesc(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("hq", ctypes.c_int), ("hkv", ctypes.c_int),
                ("head_dim", ctypes.c_int), ("block", ctypes.c_int), ("cap", ctypes.c_int),
                ("softmax_scale", ctypes.c_float), ("prefix_len", ctypes.c_int),
                ("prefix_len_dev", ctypes.c_void_p), ("max_prefix_len", ctypes.c_int),
                ("kv_dtype", ctypes.c_int), ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float)]


class HeadDesc(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("rows", ctypes.c_int), ("d", ctypes.c_int), ("vocab", ctypes.c_int)]


class SelfcondDesc(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("rows", ctypes.c_int), ("d", ctypes.c_int), ("vocab", ctypes.c_int)]


class CommitRule(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int), ("tau", ctypes.c_float), ("k", ctypes.c_int),
                ("forced_top1", ctypes.c_int), ("max_rounds", ctypes.c_int)]

    @classmethod
    def threshold(cls, tau=0.9, forced_top1=True, max_rounds=32):
        return cls(THRESHOLD, tau, 1, int(forced_top1), max_rounds)

    @classmethod
    def fixed_k(cls, k, max_rounds=32):
        return cls(FIXED_K, 0.0, k, 0, max_rounds)


class RoundState(ctypes.Structure):
    _fields_ = [("round", ctypes.c_int32), ("n_open", ctypes.c_int32), ("cont", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("n_new", ctypes.c_int32 * MAX_ROUNDS)]


ROUND_STATE_INTS = 4 + MAX_ROUNDS


class ModelDesc(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("n_layers", ctypes.c_int), ("d", ctypes.c_int), ("hq", ctypes.c_int),
                ("hkv", ctypes.c_int), ("head_dim", ctypes.c_int), ("ffn", ctypes.c_int), ("vocab", ctypes.c_int),
                ("block", ctypes.c_int), ("rope_base", ctypes.c_float), ("eps", ctypes.c_float),
                ("n_experts", ctypes.c_int), ("expert_ffn", ctypes.c_int), ("top_k", ctypes.c_int),
                ("n_shared", ctypes.c_int), ("layer_path", ctypes.c_int)]


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "wg", "wu", "wd",
                                               "router", "x_w13", "x_w13_scale", "x_w2", "x_w2_scale")]


class KV(ctypes.Structure):
    _fields_ = [("k", ctypes.POINTER(ctypes.c_void_p)), ("v", ctypes.POINTER(ctypes.c_void_p)),
                ("cap", ctypes.c_int), ("len_dev", ctypes.c_void_p), ("max_len", ctypes.c_int),
                ("kv_dtype", ctypes.c_int), ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float)]


class DecodeViews(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("x", "hn", "pe", "lse", "entropy", "maxprob", "argmax", "committed", "xn",
                                               "moe_logits", "moe_xq", "moe_xs", "moe_ids", "moe_wts", "moe_aq",
                                               "moe_as", "moe_y", "moe_hits", "sync_err")]


# ------------------------------------------------------------------ loading
_lib = None


def lib():
    """The loaded library (raises DlmError when it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise DlmError(f"{_LIB_PATH} is missing: build it with __graft_entry__.build() "
                       "or python block_diffusion_decoding_denoise_amd/build.py")
    L = ctypes.CDLL(_LIB_PATH)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    P = ctypes.POINTER
    sig = {
        "dlm_abi_version": (i, []),
        "dlm_last_error": (ctypes.c_char_p, []),
        "dlm_block_attn_ws_bytes": (sz, [P(AttnDesc)]),
        "dlm_block_attn": (i, [P(AttnDesc), vp, vp, vp, vp, vp, sz, vp]),
        "dlm_head_rowstats_ws_bytes": (sz, [P(HeadDesc)]),
        "dlm_head_rowstats": (i, [P(HeadDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "dlm_commit": (i, [P(CommitRule), i, vp, vp, vp, vp, vp, vp]),
        "dlm_block_reset": (i, [i, vp, vp, vp, vp]),
        "dlm_selfcond_ws_bytes": (sz, [P(SelfcondDesc)]),
        "dlm_selfcond": (i, [P(SelfcondDesc), vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "dlm_pack_matrix": (i, [vp, i, i, vp, vp, vp]),
        "dlm_linear_ws_bytes": (sz, [i, i]),
        "dlm_linear": (i, [vp, vp, i, i, i, vp, vp, sz, vp]),
        "dlm_pack_activations": (i, [vp, i, i, vp, vp]),
        "dlm_model_create": (i, [P(ModelDesc), vp, vp, vp, vp, P(LayerWeights), vp, P(vp)]),
        "dlm_model_destroy": (None, [vp]),
        "dlm_packed_bytes": (sz, [P(ModelDesc)]),
        "dlm_pack_ws_bytes": (sz, [P(ModelDesc)]),
        "dlm_pack_model": (i, [P(ModelDesc), vp, P(LayerWeights), vp, vp, sz, vp]),
        "dlm_decode_ws_bytes": (sz, [vp, P(KV)]),
        "dlm_decode_block": (i, [vp, P(CommitRule), P(KV), vp, vp, vp, sz, vp]),
        "dlm_decode_block_pipelined": (i, [vp, P(CommitRule), P(KV), vp, vp, vp, vp, sz, vp]),
        "dlm_prefill": (i, [vp, vp, i, P(KV), vp, sz, vp]),
        "dlm_prefill_rows": (i, [vp, vp, i, P(KV), vp, sz, i, vp]),
        "dlm_decode_block_gated": (i, [vp, P(CommitRule), P(KV), vp, vp, vp, sz, i, vp]),
        "dlm_decode_views_get": (i, [vp, P(KV), vp, sz, P(DecodeViews)]),
        "dlm_decode_round": (i, [vp, P(CommitRule), P(KV), vp, vp, vp, sz, vp]),
        "dlm_decode_begin": (i, [vp, P(KV), vp, vp, vp, sz, vp]),
        "dlm_commit_pass": (i, [vp, P(KV), vp, vp, sz, vp]),
        "dlm_ffn_gate_up_ws_bytes": (sz, [vp]),
        "dlm_ffn_gate_up": (i, [vp, i, vp, vp, vp, sz, vp]),
        "dlm_block_graph_key": (i, [vp, P(CommitRule), P(KV), vp, i, vp, vp, vp, P(ctypes.c_uint64), i]),
        "dlm_block_attn_noalloc_max_bytes": (sz, []),
        "dlm_block_attn_noalloc": (i, [P(AttnDesc), vp, vp, vp, vp, vp]),
        "dlm_model_graph_count": (i, [vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def exported_symbols():
    return [n for n in dir(lib()) if n.startswith("dlm_")]


def _check(rc: int, what: str):
    if rc != 0:
        msg = lib().dlm_last_error()
        raise DlmError(f"{what} failed ({rc}): {msg.decode() if msg else ''}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DLM_BF16
    if t.dtype == torch.float32:
        return DLM_F32
    raise DlmError(f"unsupported dtype {t.dtype}")


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda or not t.is_contiguous():
        raise DlmError(f"{name} must be a contiguous device tensor")


# ------------------------------------------------------------------ op calls
def block_attn(q, k_cache, v_cache, prefix_len, out=None, prefix_len_dev=None, max_prefix_len=None,
               scale=None, ws=None, kv_scales=None):
    """o = softmax(q K^T * scale) V over the L prefix keys and the B block keys (no mask).
    q [B, hq, D]; k_cache [hkv, cap, D]; v_cache in the blocked transposed layout
    [hkv, cap/32, D, 32] (v_cache_from_natural); returns out [B, hq, D].
    uint8 caches hold FP8 e4m3 codes (bf16 q); kv_scales = (k_scale, v_scale) then gives the
    stored values' scales."""
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, n)
    B, hq, D = q.shape
    hkv, cap, _ = k_cache.shape
    fp8 = k_cache.dtype == torch.uint8
    if fp8 != (v_cache.dtype == torch.uint8):
        raise ValueError("k_cache and v_cache must both be FP8 (uint8 codes) or neither")
    ks, vs = kv_scales if kv_scales is not None else (1.0, 1.0)
    d = AttnDesc(_dtype_code(q), hq, hkv, D, B, cap, scale if scale is not None else D ** -0.5,
                 int(prefix_len), _ptr(prefix_len_dev), int(max_prefix_len if max_prefix_len is not None else prefix_len),
                 DLM_FP8_E4M3 if fp8 else _dtype_code(q), float(ks), float(vs))
    if out is None:
        out = torch.empty_like(q)
    need = lib().dlm_block_attn_ws_bytes(ctypes.byref(d))
    if ws is None:
        ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=q.device)
    _check(lib().dlm_block_attn(ctypes.byref(d), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(ws),
                                ws.numel(), _stream()), "dlm_block_attn")
    return out


def block_attn_noalloc(q, k_cache, v_cache, prefix_len, out=None, prefix_len_dev=None, max_prefix_len=None,
                       scale=None, kv_scales=None):
    """block_attn through dlm_block_attn_noalloc: no workspace (the library's per-GPU scratch)."""
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, n)
    B, hq, D = q.shape
    hkv, cap, _ = k_cache.shape
    fp8 = k_cache.dtype == torch.uint8
    ks, vs = kv_scales if kv_scales is not None else (1.0, 1.0)
    d = AttnDesc(_dtype_code(q), hq, hkv, D, B, cap, scale if scale is not None else D ** -0.5,
                 int(prefix_len), _ptr(prefix_len_dev), int(max_prefix_len if max_prefix_len is not None else prefix_len),
                 DLM_FP8_E4M3 if fp8 else _dtype_code(q), float(ks), float(vs))
    if out is None:
        out = torch.empty_like(q)
    _check(lib().dlm_block_attn_noalloc(ctypes.byref(d), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out),
                                        _stream()), "dlm_block_attn_noalloc")
    return out


def head_rowstats(h, emb, committed=None, want_pe=True, logits=False, ws=None):
    """Row statistics of softmax(h E^T) for open rows.  Returns dict of lse, entropy,
    maxprob, argmax, pe (or None) and logits (or None)."""
    _dev(h, "h")
    _dev(emb, "emb")
    R, dm = h.shape
    V = emb.shape[0]
    desc = HeadDesc(_dtype_code(h), R, dm, V)
    dev = h.device
    f = lambda *s: torch.empty(*s, dtype=torch.float32, device=dev)  # noqa: E731
    out = {"lse": f(R), "entropy": f(R), "maxprob": f(R), "argmax": torch.empty(R, dtype=torch.int32, device=dev),
           "pe": f(R, dm) if want_pe else None, "logits": torch.full((R, V), float("nan"), device=dev) if logits else None}
    need = lib().dlm_head_rowstats_ws_bytes(ctypes.byref(desc))
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _check(lib().dlm_head_rowstats(ctypes.byref(desc), _ptr(h), _ptr(emb), _ptr(committed), _ptr(out["lse"]),
                                   _ptr(out["entropy"]), _ptr(out["maxprob"]), _ptr(out["argmax"]), _ptr(out["pe"]),
                                   _ptr(out["logits"]), _ptr(ws), ws.numel(), _stream()), "dlm_head_rowstats")
    return out


def new_round_state(device="cuda"):
    return torch.zeros(ROUND_STATE_INTS, dtype=torch.int32, device=device)


def block_reset(committed, tokens, state):
    _check(lib().dlm_block_reset(committed.numel(), _ptr(committed), _ptr(tokens), _ptr(state), _stream()),
           "dlm_block_reset")


def commit(rule: CommitRule, maxprob, argmax, committed, tokens, state):
    _check(lib().dlm_commit(ctypes.byref(rule), committed.numel(), _ptr(maxprob), _ptr(argmax), _ptr(committed),
                            _ptr(tokens), _ptr(state), _stream()), "dlm_commit")


def state_dict(state: torch.Tensor):
    s = state.cpu().tolist()
    return {"round": s[0], "n_open": s[1], "cont": s[2], "flags": s[3], "n_new": s[4:4 + s[0]]}


def pack_matrix(w: torch.Tensor, row_map=None):
    """Packed (matrix-core tile order) copy of a bf16 [N, K] matrix."""
    _dev(w, "w")
    N, K = w.shape
    out = torch.empty_like(w)
    _check(lib().dlm_pack_matrix(_ptr(w), N, K, _ptr(row_map), _ptr(out), _stream()), "dlm_pack_matrix")
    return out


def pack_activations(x):
    """Row-major bf16 [rows <= 32, k] -> the packed operand order of the skinny GEMM (32 x k)."""
    _dev(x, "x")
    rows, k = x.shape
    out = torch.empty(32, k, dtype=torch.bfloat16, device=x.device)
    _check(lib().dlm_pack_activations(_ptr(x), rows, k, _ptr(out), _stream()), "dlm_pack_activations")
    return out


def linear(w_packed, x_packed, m=32, y=None, ws=None):
    """y [m, n] f32 = x[:m] W^T with a packed bf16 W [n, k] and packed activations."""
    n, k = w_packed.shape
    x = x_packed
    if y is None:
        y = torch.empty(m, n, dtype=torch.float32, device=x.device)
    need = lib().dlm_linear_ws_bytes(n, k)
    if ws is None:
        ws = torch.zeros(need, dtype=torch.uint8, device=x.device)
    _check(lib().dlm_linear(_ptr(w_packed), _ptr(x), m, n, k, _ptr(y), _ptr(ws), ws.numel(), _stream()),
           "dlm_linear")
    return y


def selfcond(tokens, committed, emb, mask_emb, w_sc, pe_prev=None, ws=None):
    """Round input rows x [rows, d] f32.  w_sc: packed bf16 (pack_matrix) or f32 [d, d]."""
    rows = tokens.numel()
    dm = emb.shape[1]
    desc = SelfcondDesc(_dtype_code(emb), rows, dm, emb.shape[0])
    x = torch.empty(rows, dm, dtype=torch.float32, device=emb.device)
    need = lib().dlm_selfcond_ws_bytes(ctypes.byref(desc))
    if ws is None:
        ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=emb.device)
    _check(lib().dlm_selfcond(ctypes.byref(desc), _ptr(tokens), _ptr(committed), _ptr(emb), _ptr(mask_emb),
                              _ptr(w_sc), _ptr(pe_prev), _ptr(x), _ptr(ws), ws.numel(), _stream()), "dlm_selfcond")
    return x


# ------------------------------------------------------------------ model
class Model:
    """Device weights + the library's host handle + one KV cache and decode workspace.

    weights: mapping name -> torch tensor (device), names as in synth.Weights
    (``emb``, ``mask_emb``, ``w_sc``, ``final_norm``, ``l{i}.{attn_norm,wq,wk,wv,wo,ffn_norm,
    wg,wu,wd}``).  bf16 tensors are given as torch.bfloat16.
    kv_scales: None for a cache in the model dtype, or (k_scale, v_scale) for an FP8 e4m3
    cache (bf16 models): uint8 codes, stored value = scale * e4m3(code).
    fused_layers: one launch per sublayer (DLM_LAYERS_FUSED).  layer_path: the descriptor's value
    itself (DLM_LAYERS_PER_OP, DLM_LAYERS_FUSED or DLM_LAYERS_ATTN_OUT), overriding fused_layers.
    """

    def __init__(self, shape, weights, cap, max_len=None, device="cuda", kv_scales=None, fused_layers=False,
                 layer_path=None):
        self.shape = shape
        self.w = weights
        self.device = device
        s = shape
        dt = DLM_BF16 if s.dtype == "bf16" else DLM_F32
        self.desc = ModelDesc(dt, s.n_layers, s.d, s.hq, s.hkv, s.head_dim, s.ffn, s.vocab, s.block, s.rope_base,
                              s.eps, s.n_experts, s.expert_ffn, s.top_k, s.n_shared,
                              layer_path if layer_path is not None
                              else DLM_LAYERS_FUSED if fused_layers else DLM_LAYERS_PER_OP)
        L = lib()
        self._layers = (LayerWeights * s.n_layers)()
        for i in range(s.n_layers):
            lw = self._layers[i]
            for n in ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "wg", "wu", "wd", "router",
                      "x_w13", "x_w13_scale", "x_w2", "x_w2_scale"):
                t = weights.get(f"l{i}.{n}")
                setattr(lw, n, None if t is None else t.data_ptr())
        self.packed = None
        if dt == DLM_BF16:
            nb = L.dlm_packed_bytes(ctypes.byref(self.desc))
            self.packed = torch.empty(nb, dtype=torch.uint8, device=device)
            pws = torch.empty(L.dlm_pack_ws_bytes(ctypes.byref(self.desc)), dtype=torch.uint8, device=device)
            _check(L.dlm_pack_model(ctypes.byref(self.desc), _ptr(weights["w_sc"]), self._layers, _ptr(self.packed),
                                    _ptr(pws), pws.numel(), _stream()), "dlm_pack_model")
            torch.cuda.synchronize()
        h = ctypes.c_void_p()
        _check(L.dlm_model_create(ctypes.byref(self.desc), _ptr(weights["emb"]), _ptr(weights["mask_emb"]),
                                  _ptr(weights["w_sc"]), _ptr(weights["final_norm"]), self._layers,
                                  _ptr(self.packed), ctypes.byref(h)), "dlm_model_create")
        self.handle = h
        # KV cache and decode workspace
        tdt = torch.bfloat16 if dt == DLM_BF16 else torch.float32
        if kv_scales is not None:
            tdt = torch.uint8
        self.kv_scales = kv_scales
        self.cap = cap
        self.k = [torch.zeros(s.hkv, cap, s.head_dim, dtype=tdt, device=device) for _ in range(s.n_layers)]
        # V is cached transposed in 32-position blocks, [hkv, cap/32, D, 32]
        if cap % 32:
            raise DlmError("cap must be a multiple of 32")
        self.v = [torch.zeros(s.hkv, cap // 32, s.head_dim, 32, dtype=tdt, device=device) for _ in range(s.n_layers)]
        self._kptrs = (ctypes.c_void_p * s.n_layers)(*[t.data_ptr() for t in self.k])
        self._vptrs = (ctypes.c_void_p * s.n_layers)(*[t.data_ptr() for t in self.v])
        self.len_dev = torch.zeros(1, dtype=torch.int32, device=device)
        ks, vs = kv_scales if kv_scales is not None else (1.0, 1.0)
        self.kv = KV(self._kptrs, self._vptrs, cap, self.len_dev.data_ptr(), max_len or cap,
                     DLM_FP8_E4M3 if kv_scales is not None else dt, float(ks), float(vs))
        nb = L.dlm_decode_ws_bytes(self.handle, ctypes.byref(self.kv))
        if nb == 0:
            _check(-1, "dlm_decode_ws_bytes")
        self.ws = torch.zeros(nb, dtype=torch.uint8, device=device)
        self.tokens = torch.zeros(s.block, dtype=torch.int32, device=device)
        self.state = new_round_state(device)
        v = DecodeViews()
        _check(L.dlm_decode_views_get(self.handle, ctypes.byref(self.kv), _ptr(self.ws), self.ws.numel(),
                                      ctypes.byref(v)), "dlm_decode_views_get")
        self.views = v

    def close(self):
        if getattr(self, "handle", None):
            lib().dlm_model_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # views into the decode workspace
    def view(self, name, shape, dtype):
        ptr = getattr(self.views, name)
        n = 1
        for x in shape:
            n *= x
        itemsize = torch.tensor([], dtype=dtype).element_size()
        off = ptr - self.ws.data_ptr()
        return self.ws[off:off + n * itemsize].view(dtype).view(*shape)

    def ffn_gate_up(self, layer, x_packed, act=None, ws=None):
        """The round's gate/up + SwiGLU sublayer of `layer` alone: packed bf16 32 x d in,
        packed bf16 32 x ffn out (dlm_ffn_gate_up)."""
        if act is None:
            act = torch.empty(32, self.shape.ffn, dtype=torch.bfloat16, device=x_packed.device)
        if ws is None:
            ws = torch.zeros(max(lib().dlm_ffn_gate_up_ws_bytes(self.handle), 256), dtype=torch.uint8,
                             device=x_packed.device)
        _check(lib().dlm_ffn_gate_up(self.handle, layer, _ptr(x_packed), _ptr(act), _ptr(ws), ws.numel(),
                                     _stream()), "dlm_ffn_gate_up")
        return act

    def set_len(self, n):
        self.len_dev.fill_(int(n))

    def prefill(self, ids, max_rows=None):
        """Append the prompt's K/V (dlm_prefill; with max_rows, dlm_prefill_rows: at most that
        many rows per forward)."""
        ids = ids.to(device=self.device, dtype=torch.int32).contiguous()
        if max_rows is None:
            _check(lib().dlm_prefill(self.handle, _ptr(ids), ids.numel(), ctypes.byref(self.kv), _ptr(self.ws),
                                     self.ws.numel(), _stream()), "dlm_prefill")
        else:
            _check(lib().dlm_prefill_rows(self.handle, _ptr(ids), ids.numel(), ctypes.byref(self.kv), _ptr(self.ws),
                                          self.ws.numel(), int(max_rows), _stream()), "dlm_prefill_rows")

    def decode_block(self, rule: CommitRule, tokens=None, state=None):
        tokens = self.tokens if tokens is None else tokens
        state = self.state if state is None else state
        _check(lib().dlm_decode_block(self.handle, ctypes.byref(rule), ctypes.byref(self.kv), _ptr(tokens),
                                      _ptr(state), _ptr(self.ws), self.ws.numel(), _stream()), "dlm_decode_block")
        return tokens

    def decode_block_gated(self, rule: CommitRule, seg_rounds=1, tokens=None, state=None):
        """dlm_decode_block without the rounds after the block is done (threshold rules): round
        segments of seg_rounds, the host checking the continue flag between them; blocks the
        calling thread until the commit pass is enqueued (dlm_decode_block_gated)."""
        tokens = self.tokens if tokens is None else tokens
        state = self.state if state is None else state
        _check(lib().dlm_decode_block_gated(self.handle, ctypes.byref(rule), ctypes.byref(self.kv), _ptr(tokens),
                                            _ptr(state), _ptr(self.ws), self.ws.numel(), int(seg_rounds),
                                            _stream()), "dlm_decode_block_gated")
        return tokens

    def decode_block_pipelined(self, rule: CommitRule, prev_tokens, tokens, state=None):
        """Decode one block into `tokens`, first completing the pending commit pass of the
        previous block (prev_tokens, or None); this block's commit pass is left pending
        (dlm_decode_block_pipelined)."""
        state = self.state if state is None else state
        _check(lib().dlm_decode_block_pipelined(self.handle, ctypes.byref(rule), ctypes.byref(self.kv),
                                                None if prev_tokens is None else _ptr(prev_tokens), _ptr(tokens),
                                                _ptr(state), _ptr(self.ws), self.ws.numel(), _stream()),
               "dlm_decode_block_pipelined")
        return tokens

    def decode_begin(self):
        _check(lib().dlm_decode_begin(self.handle, ctypes.byref(self.kv), _ptr(self.tokens), _ptr(self.state),
                                      _ptr(self.ws), self.ws.numel(), _stream()), "dlm_decode_begin")

    def decode_round(self, rule: CommitRule):
        _check(lib().dlm_decode_round(self.handle, ctypes.byref(rule), ctypes.byref(self.kv), _ptr(self.tokens),
                                      _ptr(self.state), _ptr(self.ws), self.ws.numel(), _stream()), "dlm_decode_round")

    def commit_pass(self, tokens=None):
        tokens = self.tokens if tokens is None else tokens
        _check(lib().dlm_commit_pass(self.handle, ctypes.byref(self.kv), _ptr(tokens), _ptr(self.ws), self.ws.numel(),
                                     _stream()), "dlm_commit_pass")

    def check_sync(self):
        """Raise DlmError if a kernel that synchronises inside an XCD (the fused layer path,
        or the attention's in-launch split merge) reported a barrier wait that gave up or a
        workgroup off its group's XCD since the workspace was zeroed; the results are then not
        to be trusted.  No-op for models without such kernels.  Reads one word."""
        if not self.views.sync_err:
            return
        flags = int(self.view("sync_err", (1,), torch.int32).item())
        if flags:
            raise DlmError(f"XCD synchronisation failed (sync flags {flags}: 1 a barrier wait gave up, "
                           f"2 a workgroup ran off its group's XCD)")

    def generate(self, prompt_ids, n_blocks, rule: CommitRule, pipelined=False):
        """Prefill, then decode n_blocks blocks (one token readback per block).
        Returns (token ids [n_blocks * B], list of per-block round states).  pipelined: each
        block's commit pass rides along with the next block's round 0 (the last one runs on
        its own), with the same result.  Raises DlmError if an XCD-local synchronisation
        failed (check_sync)."""
        self.set_len(0)
        self.prefill(prompt_ids)
        out, states = [], []
        if not pipelined:
            for _ in range(n_blocks):
                self.decode_block(rule)
                out.append(self.tokens.cpu())
                states.append(state_dict(self.state))
            self.check_sync()
            return torch.cat(out), states
        bufs = [torch.zeros_like(self.tokens), torch.zeros_like(self.tokens)]
        prev = None
        for b in range(n_blocks):
            cur = bufs[b % 2]
            self.decode_block_pipelined(rule, prev, cur)
            out.append(cur.cpu())
            states.append(state_dict(self.state))
            prev = cur
        if prev is not None:
            self.commit_pass(prev)
        self.check_sync()
        return torch.cat(out), states


def v_cache_from_natural(v):
    """[hkv, cap, D] values -> the library's V cache layout [hkv, cap/32, D, 32] (torch)."""
    h, cap, D = v.shape
    return v.reshape(h, cap // 32, 32, D).transpose(2, 3).contiguous()


def v_cache_to_natural(vc):
    """The library's V cache [hkv, cap/32, D, 32] -> [hkv, cap, D] (torch)."""
    h, nb, D, _ = vc.shape
    return vc.transpose(2, 3).reshape(h, nb * 32, D)


def weights_to_device(w, names, device="cuda"):
    """Upload synth storage arrays (float32 or uint16 bf16 bits) as torch tensors."""
    import numpy as np
    out = {}
    for n in names:
        a = w[n]
        if a.dtype == np.uint16:
            out[n] = torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(device)
        else:
            out[n] = torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return out

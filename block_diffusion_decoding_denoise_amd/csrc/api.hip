// C ABI of the library: argument validation, workspace layout, the per-round sequence of
// kernels and the device-resident block loop captured in a HIP graph.
#include <stdarg.h>
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <map>
#include <mutex>
#include <tuple>
#include <vector>

#include "attn.h"
#include "gemm.h"
#include "head.h"
#include "small.h"
#include "moe.h"
#include "layer.h"

#include <cstddef>

// ------------------------------------------------------------------ errors
namespace dlm {
static thread_local char g_err[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int check_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return DLM_OK;
  return fail(DLM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool device_ok() {
  static int cached[64];
  static std::once_flag once[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
  std::call_once(once[dev], [dev]() {
    hipDeviceProp_t prop;
    cached[dev] = (hipGetDeviceProperties(&prop, dev) == hipSuccess &&
                   strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 0;
  });
  return cached[dev] == 1;
}
}  // namespace dlm

using namespace dlm;

#define DLM_DEVICE_CHECK() \
  do { if (!dlm::device_ok()) return dlm::fail(DLM_ERR_UNSUPPORTED, "no gfx950 device is current"); } while (0)

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

extern "C" int dlm_abi_version(void) { return DLM_ABI_VERSION; }
extern "C" const char* dlm_last_error(void) { return dlm::g_err; }

// ------------------------------------------------------------------ block attention op
static int check_attn(const dlm_attn_desc* d) {
  DLM_REQUIRE(d, DLM_ERR_ARG, "desc is null");
  DLM_REQUIRE(d->dtype == DLM_BF16 || d->dtype == DLM_F32, DLM_ERR_DTYPE, "attn dtype %d", d->dtype);
  DLM_REQUIRE(d->hq > 0 && d->hkv > 0 && d->block > 0 && d->cap > 0, DLM_ERR_ARG, "non-positive size");
  DLM_REQUIRE(d->cap % 32 == 0, DLM_ERR_SHAPE, "cap must be a multiple of 32 (blocked V cache)");
  DLM_REQUIRE(d->hq % d->hkv == 0, DLM_ERR_SHAPE, "hq %% hkv != 0");
  DLM_REQUIRE(d->head_dim == 64 || d->head_dim == 128, DLM_ERR_SHAPE, "head_dim must be 64 or 128");
  DLM_REQUIRE(d->kv_dtype == d->dtype || (d->kv_dtype == DLM_FP8_E4M3 && d->dtype == DLM_BF16), DLM_ERR_DTYPE,
              "kv_dtype %d with dtype %d (an FP8 cache needs bf16 queries)", d->kv_dtype, d->dtype);
  if (d->kv_dtype == DLM_FP8_E4M3)
    DLM_REQUIRE(isfinite(d->k_scale) && isfinite(d->v_scale) && d->k_scale > 0.f && d->v_scale > 0.f,
                DLM_ERR_ARG, "FP8 cache scales must be finite and positive");
  DLM_REQUIRE(d->block <= 32, DLM_ERR_SHAPE, "block must be <= 32");
  const int maxL = d->prefix_len_dev ? d->max_prefix_len : d->prefix_len;
  DLM_REQUIRE(maxL >= 0 && d->prefix_len >= 0, DLM_ERR_ARG, "negative prefix length");
  DLM_REQUIRE(maxL + d->block <= d->cap, DLM_ERR_SHAPE, "prefix + block exceeds cap");
  return DLM_OK;
}

extern "C" size_t dlm_block_attn_ws_bytes(const dlm_attn_desc* d) {
  if (check_attn(d) != DLM_OK) return 0;
  if (d->dtype == DLM_F32) return 256;
  const int maxL = d->prefix_len_dev ? d->max_prefix_len : d->prefix_len;
  return attn_ws_bytes(d->hq, d->hkv, d->head_dim, attn_plan(d->hq, d->hkv, d->head_dim, d->block, maxL));
}

static int block_attn_enqueue(const dlm_attn_desc* d, const void* q, const void* k, const void* v, void* out,
                              void* ws, void* stream);

extern "C" int dlm_block_attn(const dlm_attn_desc* d, const void* q, const void* k, const void* v, void* out,
                              void* ws, size_t ws_bytes, void* stream) {
  int rc = check_attn(d);
  if (rc) return rc;
  DLM_REQUIRE(q && k && v && out, DLM_ERR_ARG, "null tensor");
  DLM_REQUIRE(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(out), DLM_ERR_ARG, "tensors must be 16-byte aligned");
  const size_t need = dlm_block_attn_ws_bytes(d);
  DLM_REQUIRE(ws || need == 0, DLM_ERR_ARG, "null workspace");
  DLM_REQUIRE(ws_bytes >= need, DLM_ERR_WORKSPACE, "workspace %zu < %zu", ws_bytes, need);
  DLM_DEVICE_CHECK();
  return block_attn_enqueue(d, q, k, v, out, ws, stream);
}

// ------------------------------------------------------------------ allocation-free attention
// The split partials of dlm_block_attn_noalloc live in this file-scope device array (one copy
// per GPU, held until the process ends).  Host code never uses the array's name as an address:
// each device's copy is found once with hipGetSymbolAddress and that pointer is passed to the
// kernels.  The kernels overwrite every partial they later read, so nothing is cleared.
static constexpr size_t kAttnScratchBytes = (size_t)16 << 20;
__device__ __align__(256) uint8_t scratch[kAttnScratchBytes];

static void* attn_scratch_ptr(int* rc) {
  constexpr int kMaxDev = 64;
  static void* ptr[kMaxDev];
  static hipError_t err[kMaxDev];
  static std::once_flag once[kMaxDev];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) {
    *rc = fail(DLM_ERR_HIP, "no current device in [0, %d)", kMaxDev);
    return nullptr;
  }
  std::call_once(once[dev], [dev]() { err[dev] = hipGetSymbolAddress(&ptr[dev], HIP_SYMBOL(scratch)); });
  if (err[dev] != hipSuccess || ptr[dev] == nullptr) {
    *rc = fail(DLM_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
               err[dev] != hipSuccess ? hipGetErrorString(err[dev]) : "null address");
    return nullptr;
  }
  return ptr[dev];
}

extern "C" size_t dlm_block_attn_noalloc_max_bytes(void) { return kAttnScratchBytes; }

extern "C" int dlm_block_attn_noalloc(const dlm_attn_desc* d, const void* q, const void* k, const void* v, void* out,
                                      void* stream) {
  int rc = check_attn(d);
  if (rc) return rc;
  DLM_REQUIRE(q && k && v && out, DLM_ERR_ARG, "null tensor");
  DLM_REQUIRE(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(out), DLM_ERR_ARG, "tensors must be 16-byte aligned");
  const size_t need = dlm_block_attn_ws_bytes(d);
  DLM_REQUIRE(need <= kAttnScratchBytes, DLM_ERR_WORKSPACE,
              "this attention needs %zu bytes of split scratch; the allocation-free call holds %zu "
              "(use dlm_block_attn with a workspace)", need, kAttnScratchBytes);
  DLM_DEVICE_CHECK();
  void* ws = attn_scratch_ptr(&rc);
  if (!ws) return rc;
  return block_attn_enqueue(d, q, k, v, out, ws, stream);
}

static int block_attn_enqueue(const dlm_attn_desc* d, const void* q, const void* k, const void* v, void* out,
                              void* ws, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if (d->dtype == DLM_F32)
    return attn_f32((const float*)q, (const float*)k, (const float*)v, (float*)out, d->hq, d->hkv, d->head_dim,
                    d->block, d->cap, d->softmax_scale, d->prefix_len_dev, d->prefix_len, nullptr, st);
  const int maxL = d->prefix_len_dev ? d->max_prefix_len : d->prefix_len;
  return attn_bf16(q, k, v, out, d->hq, d->hkv, d->head_dim, d->block, 1, d->cap, d->softmax_scale,
                   d->prefix_len_dev, d->prefix_len, nullptr,
                   attn_plan(d->hq, d->hkv, d->head_dim, d->block, maxL), ws, /*out_packed=*/0, st,
                   AttnKv{d->kv_dtype == DLM_FP8_E4M3 ? 1 : 0, d->k_scale, d->v_scale});
}

// ------------------------------------------------------------------ head op
static int check_head(const dlm_head_desc* d) {
  DLM_REQUIRE(d, DLM_ERR_ARG, "desc is null");
  DLM_REQUIRE(d->dtype == DLM_BF16 || d->dtype == DLM_F32, DLM_ERR_DTYPE, "head dtype %d", d->dtype);
  DLM_REQUIRE(d->rows > 0 && d->d > 0 && d->vocab > 0, DLM_ERR_ARG, "non-positive size");
  DLM_REQUIRE(d->rows <= DLM_MAX_ROWS, DLM_ERR_SHAPE, "rows must be <= %d", DLM_MAX_ROWS);
  DLM_REQUIRE(d->d % 32 == 0 && d->d <= 4096, DLM_ERR_SHAPE, "d must be a multiple of 32 and <= 4096");
  DLM_REQUIRE(d->dtype == DLM_BF16 || d->d <= 256, DLM_ERR_SHAPE, "f32 head supports d <= 256");
  return DLM_OK;
}

extern "C" size_t dlm_head_rowstats_ws_bytes(const dlm_head_desc* d) {
  if (check_head(d) != DLM_OK) return 0;
  return head_ws_bytes(d->dtype, d->rows, d->d, d->vocab);
}

extern "C" int dlm_head_rowstats(const dlm_head_desc* d, const void* h, const void* emb, const uint8_t* committed,
                                 float* lse, float* entropy, float* maxprob, int32_t* argmax, float* pe,
                                 float* logits_dbg, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_head(d);
  if (rc) return rc;
  DLM_REQUIRE(h && emb && lse && entropy && maxprob && argmax && ws, DLM_ERR_ARG, "null pointer");
  DLM_REQUIRE(aligned16(h) && aligned16(emb), DLM_ERR_ARG, "h and emb must be 16-byte aligned");
  const size_t need = dlm_head_rowstats_ws_bytes(d);
  DLM_REQUIRE(ws_bytes >= need, DLM_ERR_WORKSPACE, "workspace %zu < %zu", ws_bytes, need);
  DLM_DEVICE_CHECK();
  return head_launch(d->dtype, h, emb, committed, d->rows, d->d, d->vocab, lse, entropy, maxprob, argmax, pe,
                     logits_dbg, ws, nullptr, (hipStream_t)stream);
}

// ------------------------------------------------------------------ commit op
static int check_rule(const dlm_commit_rule* r) {
  DLM_REQUIRE(r, DLM_ERR_ARG, "rule is null");
  DLM_REQUIRE(r->mode == DLM_COMMIT_THRESHOLD || r->mode == DLM_COMMIT_FIXED_K, DLM_ERR_ARG, "bad commit mode");
  DLM_REQUIRE(r->max_rounds >= 1 && r->max_rounds <= DLM_MAX_ROUNDS, DLM_ERR_ARG, "max_rounds out of range");
  DLM_REQUIRE(r->mode != DLM_COMMIT_FIXED_K || r->k >= 1, DLM_ERR_ARG, "k must be >= 1");
  return DLM_OK;
}

extern "C" int dlm_commit(const dlm_commit_rule* rule, int rows, const float* maxprob, const int32_t* argmax,
                          uint8_t* committed, int32_t* tokens, dlm_round_state* state, void* stream) {
  int rc = check_rule(rule);
  if (rc) return rc;
  DLM_REQUIRE(rows >= 1 && rows <= DLM_MAX_ROWS, DLM_ERR_SHAPE, "rows must be in [1, %d]", DLM_MAX_ROWS);
  DLM_REQUIRE(maxprob && argmax && committed && tokens && state, DLM_ERR_ARG, "null pointer");
  DLM_DEVICE_CHECK();
  return commit_launch(*rule, rows, maxprob, argmax, nullptr, nullptr, committed, tokens, state,
                       (hipStream_t)stream);
}

extern "C" int dlm_block_reset(int rows, uint8_t* committed, int32_t* tokens, dlm_round_state* state,
                               void* stream) {
  DLM_REQUIRE(rows >= 1 && rows <= DLM_MAX_ROWS, DLM_ERR_SHAPE, "rows must be in [1, %d]", DLM_MAX_ROWS);
  DLM_REQUIRE(committed && tokens && state, DLM_ERR_ARG, "null pointer");
  DLM_DEVICE_CHECK();
  return block_reset(rows, committed, tokens, state, nullptr, 0, (hipStream_t)stream);
}

// ------------------------------------------------------------------ self-conditioning op
static int check_sc(const dlm_selfcond_desc* d) {
  DLM_REQUIRE(d, DLM_ERR_ARG, "desc is null");
  DLM_REQUIRE(d->dtype == DLM_BF16 || d->dtype == DLM_F32, DLM_ERR_DTYPE, "selfcond dtype %d", d->dtype);
  DLM_REQUIRE(d->rows > 0 && d->d > 0 && d->vocab > 0, DLM_ERR_ARG, "non-positive size");
  DLM_REQUIRE(d->rows <= 32, DLM_ERR_SHAPE, "rows must be <= 32");
  DLM_REQUIRE(d->d % 32 == 0, DLM_ERR_SHAPE, "d must be a multiple of 32");
  return DLM_OK;
}

static size_t sc_gemm_ws(int d) { return gemm_ws_bytes(d, d, gemm_plan(d, d)); }

extern "C" size_t dlm_selfcond_ws_bytes(const dlm_selfcond_desc* d) {
  if (check_sc(d) != DLM_OK) return 0;
  const size_t el = d->dtype == DLM_BF16 ? 2 : 4;
  return align_up((size_t)32 * d->d * el, 256) + (d->dtype == DLM_BF16 ? sc_gemm_ws(d->d) : 0);
}

static EpiParams epi_zero() {
  EpiParams e;
  memset(&e, 0, sizeof(e));
  return e;
}

extern "C" int dlm_selfcond(const dlm_selfcond_desc* d, const int32_t* tokens, const uint8_t* committed,
                            const void* emb, const void* mask_emb, const void* w_sc, const float* pe_prev,
                            float* x_out, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_sc(d);
  if (rc) return rc;
  DLM_REQUIRE(tokens && committed && emb && mask_emb && w_sc && x_out && ws, DLM_ERR_ARG, "null pointer");
  DLM_REQUIRE(aligned16(w_sc) && aligned16(ws), DLM_ERR_ARG, "w_sc and ws must be 16-byte aligned");
  DLM_REQUIRE(ws_bytes >= dlm_selfcond_ws_bytes(d), DLM_ERR_WORKSPACE, "workspace too small");
  DLM_DEVICE_CHECK();
  hipStream_t st = (hipStream_t)stream;
  const int bf = d->dtype == DLM_BF16;
  const size_t el = bf ? 2 : 4;
  void* xsc = ws;
  void* gws = (char*)ws + align_up((size_t)32 * d->d * el, 256);
  rc = selfcond_prep(pe_prev, committed, xsc, d->rows, d->d, bf, nullptr, st);
  if (rc) return rc;
  EpiParams e = epi_zero();
  e.kind = EPI_SELFCOND;
  e.M = d->rows;
  e.bf16_out = bf;
  e.out = x_out;
  e.ld_out = d->d;
  e.mask_emb = mask_emb;
  e.emb = emb;
  e.tokens = tokens;
  e.committed = committed;
  e.vocab = d->vocab;
  if (bf) return gemm_bf16(w_sc, xsc, d->d, d->d, MAP_IDENTITY, e, gemm_plan(d->d, d->d), gws, st);
  F32Mats W{};
  W.w[0] = (const float*)w_sc;
  W.rows[0] = d->d;
  return gemm_f32(W, (const float*)xsc, d->d, d->d, MAP_IDENTITY, e, st);
}

// ------------------------------------------------------------------ packing
extern "C" int dlm_pack_matrix(const void* src, int n_rows, int k, const int32_t* row_map_dev, void* dst,
                               void* stream) {
  DLM_REQUIRE(src && dst, DLM_ERR_ARG, "null pointer");
  DLM_REQUIRE(n_rows > 0 && k > 0 && n_rows % 32 == 0 && k % 32 == 0, DLM_ERR_SHAPE,
              "n_rows %% 32 and k %% 32 must be 0");
  DLM_REQUIRE(aligned16(src) && aligned16(dst), DLM_ERR_ARG, "16-byte alignment required");
  DLM_DEVICE_CHECK();
  const void* s[1] = {src};
  int r[1] = {n_rows};
  return pack_bf16(s, r, 1, n_rows, k, row_map_dev, dst, (hipStream_t)stream);
}

// ------------------------------------------------------------------ plain linear
extern "C" size_t dlm_linear_ws_bytes(int n, int k) {
  if (n <= 0 || k <= 0 || n % 32 || k % 32) return 0;
  return gemm_ws_bytes(n, k, gemm_plan(n, k));
}

extern "C" int dlm_linear(const void* w_packed, const void* x, int m, int n, int k, float* y, void* ws,
                          size_t ws_bytes, void* stream) {
  DLM_REQUIRE(w_packed && x && y && ws, DLM_ERR_ARG, "null pointer");
  DLM_REQUIRE(m >= 1 && m <= 32, DLM_ERR_SHAPE, "m must be in [1, 32]");
  DLM_REQUIRE(n > 0 && k > 0 && n % 32 == 0 && k % 32 == 0, DLM_ERR_SHAPE, "n %% 32 and k %% 32 must be 0");
  DLM_REQUIRE(aligned16(w_packed) && aligned16(x) && aligned16(ws), DLM_ERR_ARG, "16-byte alignment required");
  DLM_REQUIRE(ws_bytes >= dlm_linear_ws_bytes(n, k), DLM_ERR_WORKSPACE, "workspace too small");
  DLM_DEVICE_CHECK();
  EpiParams e = epi_zero();
  e.kind = EPI_STORE_F32;
  e.M = m;
  e.bf16_out = 1;
  e.out = y;
  e.ld_out = n;
  return gemm_bf16(w_packed, x, n, k, MAP_IDENTITY, e, gemm_plan(n, k), ws, (hipStream_t)stream);
}

extern "C" int dlm_pack_activations(const void* x, int rows, int k, void* x_packed, void* stream) {
  DLM_REQUIRE(x && x_packed, DLM_ERR_ARG, "null pointer");
  DLM_REQUIRE(rows >= 1 && rows <= 32 && k > 0 && k % 32 == 0, DLM_ERR_SHAPE, "rows in [1, 32], k %% 32 == 0");
  DLM_DEVICE_CHECK();
  return pack_rows_bf16(x, rows, k, x_packed, (hipStream_t)stream);
}

// ------------------------------------------------------------------ model
// Everything a captured block graph bakes in: the rule, every buffer address the kernels
// take (tokens, state, workspace, prefix length, each layer's K and V base), and the cache
// geometry and format (capacity strides, the max_len-dependent attention split plan and
// workspace offsets, FP8 scales).  A launch whose key differs captures a new graph.
typedef std::vector<uint64_t> GraphKey;

struct dlm_model {
  dlm_model_desc d;
  const void* emb;
  const void* mask_emb;
  const void* w_sc;
  const void* final_norm;
  std::vector<dlm_layer_weights> layers;
  const void* packed;
  // packed offsets (bytes)
  size_t off_sc;
  std::vector<size_t> off_qkv, off_o, off_gu, off_dn, off_router, off_moe;
  size_t packed_bytes;
  GemmPlan pl_sc, pl_qkv, pl_o, pl_gu, pl_dn, pl_router;
  int n_qkv;
  // fused layer path (layer.hip): one launch per sublayer, XCD-local synchronisation; the
  // QKV, attention-output and down matrices are then packed in its layouts
  bool fused;
  FusedDims fd;
  // per-op path with the attention-output projection inside the attention launch (layer.hip
  // attn_out_xcd) for 32- and 64-row forwards, on request: the attention-output matrix is also
  // packed as the fused path's 8 column slices (off_ox); wide prefill forwards keep the
  // separate GEMM
  bool xo;
  std::vector<size_t> off_ox;
  std::mutex mu;
  std::map<GraphKey, hipGraphExec_t> graphs;
  std::vector<hipGraph_t> graph_objs;
  hipStream_t cap_stream = nullptr;
  // gated block decode (dlm_decode_block_gated): the continue flag after each round segment is
  // copied to pinned host memory and an event marks it; two slots (one segment in flight ahead)
  std::mutex gate_mu;
  int32_t* gate_flags = nullptr;
  hipEvent_t gate_ev[2] = {nullptr, nullptr};
  int gate_last = -1;   // slot of the last flag copy a call left in flight (-1: none)
};

static int check_model_desc(const dlm_model_desc* d) {
  DLM_REQUIRE(d, DLM_ERR_ARG, "desc is null");
  DLM_REQUIRE(d->dtype == DLM_BF16 || d->dtype == DLM_F32, DLM_ERR_DTYPE, "model dtype %d", d->dtype);
  DLM_REQUIRE(d->n_layers > 0 && d->d > 0 && d->hq > 0 && d->hkv > 0 && d->vocab > 0 && d->block > 0,
              DLM_ERR_ARG, "non-positive size");
  DLM_REQUIRE(d->hq % d->hkv == 0, DLM_ERR_SHAPE, "hq %% hkv != 0");
  DLM_REQUIRE(d->head_dim == 64 || d->head_dim == 128, DLM_ERR_SHAPE, "head_dim must be 64 or 128");
  DLM_REQUIRE(d->block <= 32, DLM_ERR_SHAPE, "block must be <= 32");
  DLM_REQUIRE(d->d % 32 == 0 && d->d <= 4096, DLM_ERR_SHAPE, "d must be a multiple of 32, <= 4096");
  DLM_REQUIRE(d->layer_path == DLM_LAYERS_PER_OP || d->layer_path == DLM_LAYERS_FUSED ||
                  d->layer_path == DLM_LAYERS_ATTN_OUT,
              DLM_ERR_ARG,
              "layer_path %d", d->layer_path);
  const bool moe = d->n_experts > 0;
  if (!moe) DLM_REQUIRE(d->ffn > 0 && d->ffn % 32 == 0, DLM_ERR_SHAPE, "ffn must be a positive multiple of 32");
  if (moe) {
    DLM_REQUIRE(d->dtype == DLM_BF16, DLM_ERR_DTYPE, "MoE models are bf16");
    DLM_REQUIRE(d->top_k >= 1 && d->top_k <= 8 && d->top_k <= d->n_experts && d->n_experts <= 256,
                DLM_ERR_SHAPE, "top_k in [1, 8], n_experts <= 256");
    DLM_REQUIRE(d->expert_ffn % 128 == 0 && d->expert_ffn > 0 && d->n_shared >= 0 && d->n_shared <= 2,
                DLM_ERR_SHAPE, "expert_ffn %% 128 == 0, n_shared <= 2");
    DLM_REQUIRE(d->n_experts % 32 == 0 && d->d % 256 == 0 && d->block <= 32 && d->n_layers <= 256, DLM_ERR_SHAPE,
                "MoE: n_experts %% 32 == 0, d %% 256 == 0, block <= 32, n_layers <= 256");
  }
  if (d->dtype == DLM_F32) DLM_REQUIRE(d->d <= 256, DLM_ERR_SHAPE, "f32 models support d <= 256");
  return DLM_OK;
}

// On request (DLM_LAYERS_ATTN_OUT), dense bf16 models with 8 kv heads of 4 query heads of 128,
// 32-row blocks, d % 512 == 0 and d <= 3072 (at most 96 output features per workgroup in the
// projection) take the attention and its output projection as one launch on the per-op path.
static bool xo_ok(const dlm_model_desc& d) {
  return d.layer_path == DLM_LAYERS_ATTN_OUT && d.dtype == DLM_BF16 && d.n_experts == 0 && d.hq == 32 &&
         d.hkv == 8 && d.head_dim == 128 && d.block == 32 && d.d % 512 == 0 && d.d <= 3072;
}

static void layout_packed(dlm_model* m) {
  const dlm_model_desc& d = m->d;
  const int D = d.head_dim;
  m->n_qkv = (d.hq + 2 * d.hkv) * D;
  m->xo = xo_ok(d);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align_up(bytes, 256); return o; };
  m->off_sc = take((size_t)d.d * d.d * 2);
  m->off_qkv.resize(d.n_layers);
  m->off_o.resize(d.n_layers);
  m->off_gu.resize(d.n_layers);
  m->off_dn.resize(d.n_layers);
  m->off_router.resize(d.n_layers);
  m->off_moe.resize(d.n_layers);
  m->off_ox.assign(d.n_layers, 0);
  for (int l = 0; l < d.n_layers; ++l) {
    m->off_qkv[l] = take((size_t)m->n_qkv * d.d * 2);
    m->off_o[l] = take((size_t)d.d * d.hq * D * 2);
    if (m->xo) m->off_ox[l] = take((size_t)d.d * d.hq * D * 2);
    if (d.n_experts == 0) {
      m->off_gu[l] = take((size_t)2 * d.ffn * d.d * 2);
      m->off_dn[l] = take((size_t)d.d * d.ffn * 2);
    } else {
      m->off_router[l] = take((size_t)d.n_experts * d.d * 2);
      m->off_moe[l] = take(moe_layer_packed_bytes(moe_dims(d)));
    }
  }
  m->packed_bytes = d.dtype == DLM_BF16 ? off : 0;
  m->pl_sc = gemm_plan_owned(d.d, d.d);
  m->pl_qkv = gemm_plan_owned(m->n_qkv, d.d);
  m->pl_o = gemm_plan(d.d, d.hq * D);
  if (d.n_experts == 0) {
    m->pl_gu = gemm_plan_owned(2 * d.ffn, d.d);
    m->pl_dn = gemm_plan(d.d, d.ffn);
  } else {
    m->pl_gu = m->pl_dn = GemmPlan{1, 1, 0};
  }
  m->pl_router = d.n_experts ? gemm_plan_owned(d.n_experts, d.d) : GemmPlan{1, 1, 0};
  m->fused = d.layer_path == DLM_LAYERS_FUSED &&
             layer_fused_ok(d.dtype, d.n_experts, d.d, d.hq, d.hkv, D, d.ffn, d.block) &&
             m->pl_gu.R == 2 * d.ffn / 256 && m->pl_gu.splits == 256;
  if (m->fused || m->xo) m->fd = fused_dims(d.d, d.ffn, d.hq, d.hkv, D);
}

extern "C" size_t dlm_packed_bytes(const dlm_model_desc* d) {
  if (check_model_desc(d) != DLM_OK) return 0;
  dlm_model m;
  m.d = *d;
  layout_packed(&m);
  return m.packed_bytes;
}

extern "C" size_t dlm_pack_ws_bytes(const dlm_model_desc* d) {
  if (check_model_desc(d) != DLM_OK) return 0;
  const size_t qkv = (size_t)(d->hq + 2 * d->hkv) * d->head_dim;
  return (qkv + 2 * (size_t)(d->ffn > 0 ? d->ffn : 0)) * 4 + 256;
}

static int check_layer(const dlm_model_desc* d, const dlm_layer_weights& L, int i) {
  DLM_REQUIRE(L.attn_norm && L.wq && L.wk && L.wv && L.wo && L.ffn_norm, DLM_ERR_ARG,
              "layer %d: null attention weight", i);
  if (d->n_experts == 0)
    DLM_REQUIRE(L.wg && L.wu && L.wd, DLM_ERR_ARG, "layer %d: null FFN weight", i);
  else
    DLM_REQUIRE(L.router && L.x_w13 && L.x_w13_scale && L.x_w2 && L.x_w2_scale, DLM_ERR_ARG,
                "layer %d: null MoE weight", i);
  return DLM_OK;
}

extern "C" int dlm_pack_model(const dlm_model_desc* d, const void* w_sc, const dlm_layer_weights* layers, void* dst,
                              void* row_map_ws, size_t ws_bytes, void* stream) {
  int rc = check_model_desc(d);
  if (rc) return rc;
  DLM_REQUIRE(d->dtype == DLM_BF16, DLM_ERR_DTYPE, "only bf16 models are packed");
  DLM_REQUIRE(w_sc && layers && dst && row_map_ws, DLM_ERR_ARG, "null pointer");
  DLM_REQUIRE(ws_bytes >= dlm_pack_ws_bytes(d), DLM_ERR_WORKSPACE, "row-map workspace too small");
  for (int i = 0; i < d->n_layers; ++i) {
    rc = check_layer(d, layers[i], i);
    if (rc) return rc;
  }
  DLM_DEVICE_CHECK();
  dlm_model m;
  m.d = *d;
  layout_packed(&m);
  hipStream_t st = (hipStream_t)stream;
  const int D = d->head_dim;
  std::vector<int32_t> maps((size_t)m.n_qkv + 2 * (size_t)(d->ffn > 0 ? d->ffn : 0));
  if (m.fused) build_xqkv_row_map(d->hq, d->hkv, D, maps.data());
  else build_row_map(MAP_QKV, m.n_qkv, d->hq, d->hkv, D, d->ffn, maps.data());
  if (d->n_experts == 0) build_row_map(MAP_GU, 2 * d->ffn, d->hq, d->hkv, D, d->ffn, maps.data() + m.n_qkv);
  int32_t* map_qkv = (int32_t*)row_map_ws;
  int32_t* map_gu = map_qkv + m.n_qkv;
  DLM_HIP(hipMemcpyAsync(row_map_ws, maps.data(), maps.size() * 4, hipMemcpyHostToDevice, st));
  DLM_HIP(hipStreamSynchronize(st));
  char* out = (char*)dst;
  {
    const void* s[1] = {w_sc};
    int r[1] = {d->d};
    rc = m.pl_sc.R ? pack_bf16_owned(s, r, 1, d->d, d->d, nullptr, m.pl_sc.R, out + m.off_sc, st)
                   : pack_bf16(s, r, 1, d->d, d->d, nullptr, out + m.off_sc, st);
    if (rc) return rc;
  }
  for (int l = 0; l < d->n_layers; ++l) {
    const dlm_layer_weights& L = layers[l];
    const void* s3[3] = {L.wq, L.wk, L.wv};
    int r3[3] = {d->hq * D, d->hkv * D, d->hkv * D};
    if (m.fused) {
      // QKV with each XCD's head group in its workgroups' blocks; the attention-output and down
      // matrices as 8 column slices (each XCD's contraction range) in the row-owned layout
      const FusedDims& fd = m.fd;
      if ((rc = pack_bf16_owned(s3, r3, 3, m.n_qkv, d->d, map_qkv, fd.rq, out + m.off_qkv[l], st))) return rc;
      for (int x = 0; x < 8; ++x) {
        const void* so[1] = {(const uint16_t*)L.wo + (size_t)x * fd.ko};
        int ro[1] = {d->d};
        if ((rc = pack_bf16_owned(so, ro, 1, d->d, fd.ko, nullptr, fd.ro,
                                  out + m.off_o[l] + (size_t)x * d->d * fd.ko * 2, st, d->hq * D)))
          return rc;
        const void* sd[1] = {(const uint16_t*)L.wd + (size_t)x * fd.kd};
        int rd[1] = {d->d};
        if ((rc = pack_bf16_owned(sd, rd, 1, d->d, fd.kd, nullptr, fd.ro,
                                  out + m.off_dn[l] + (size_t)x * d->d * fd.kd * 2, st, d->ffn)))
          return rc;
      }
      const void* s2[2] = {L.wg, L.wu};
      int r2[2] = {d->ffn, d->ffn};
      if ((rc = pack_bf16_owned(s2, r2, 2, 2 * d->ffn, d->d, map_gu, m.pl_gu.R, out + m.off_gu[l], st))) return rc;
      continue;
    }
    rc = m.pl_qkv.R ? pack_bf16_owned(s3, r3, 3, m.n_qkv, d->d, map_qkv, m.pl_qkv.R, out + m.off_qkv[l], st)
                    : pack_bf16(s3, r3, 3, m.n_qkv, d->d, map_qkv, out + m.off_qkv[l], st);
    if (rc) return rc;
    const void* so[1] = {L.wo};
    int ro[1] = {d->d};
    rc = m.pl_o.R ? pack_bf16_owned(so, ro, 1, d->d, d->hq * D, nullptr, m.pl_o.R, out + m.off_o[l], st)
                  : pack_bf16(so, ro, 1, d->d, d->hq * D, nullptr, out + m.off_o[l], st);
    if (rc) return rc;
    if (m.xo) {
      // the same matrix as 8 column slices (each XCD's query heads) for the fused attention output
      const FusedDims& fd = m.fd;
      for (int x = 0; x < 8; ++x) {
        const void* sx[1] = {(const uint16_t*)L.wo + (size_t)x * fd.ko};
        int rx[1] = {d->d};
        if ((rc = pack_bf16_owned(sx, rx, 1, d->d, fd.ko, nullptr, fd.ro,
                                  out + m.off_ox[l] + (size_t)x * d->d * fd.ko * 2, st, d->hq * D)))
          return rc;
      }
    }
    if (d->n_experts == 0) {
      const void* s2[2] = {L.wg, L.wu};
      int r2[2] = {d->ffn, d->ffn};
      rc = m.pl_gu.R ? pack_bf16_owned(s2, r2, 2, 2 * d->ffn, d->d, map_gu, m.pl_gu.R, out + m.off_gu[l], st)
                     : pack_bf16(s2, r2, 2, 2 * d->ffn, d->d, map_gu, out + m.off_gu[l], st);
      if (rc) return rc;
      const void* sd[1] = {L.wd};
      int rd[1] = {d->d};
      rc = m.pl_dn.R ? pack_bf16_owned(sd, rd, 1, d->d, d->ffn, nullptr, m.pl_dn.R, out + m.off_dn[l], st)
                     : pack_bf16(sd, rd, 1, d->d, d->ffn, nullptr, out + m.off_dn[l], st);
      if (rc) return rc;
    } else {
      const void* sr[1] = {L.router};
      int rr[1] = {d->n_experts};
      rc = m.pl_router.R
               ? pack_bf16_owned(sr, rr, 1, d->n_experts, d->d, nullptr, m.pl_router.R, out + m.off_router[l], st)
               : pack_bf16(sr, rr, 1, d->n_experts, d->d, nullptr, out + m.off_router[l], st);
      if (rc) return rc;
      if ((rc = moe_pack_layer(moe_dims(*d), L, out + m.off_moe[l], st))) return rc;
    }
  }
  return DLM_OK;
}

extern "C" int dlm_model_create(const dlm_model_desc* d, const void* emb, const void* mask_emb, const void* w_sc,
                                const void* final_norm, const dlm_layer_weights* layers, const void* packed,
                                dlm_model** out) {
  int rc = check_model_desc(d);
  if (rc) return rc;
  DLM_REQUIRE(out, DLM_ERR_ARG, "out is null");
  DLM_REQUIRE(emb && mask_emb && w_sc && final_norm && layers, DLM_ERR_ARG, "null model weight");
  DLM_REQUIRE(d->dtype == DLM_F32 || packed, DLM_ERR_ARG, "bf16 models need the packed buffer");
  for (int i = 0; i < d->n_layers; ++i) {
    rc = check_layer(d, layers[i], i);
    if (rc) return rc;
  }
  dlm_model* m = new dlm_model();
  m->d = *d;
  m->emb = emb;
  m->mask_emb = mask_emb;
  m->w_sc = w_sc;
  m->final_norm = final_norm;
  m->layers.assign(layers, layers + d->n_layers);
  m->packed = packed;
  layout_packed(m);
  *out = m;
  return DLM_OK;
}

extern "C" void dlm_model_destroy(dlm_model* m) {
  if (!m) return;
  for (auto& kv : m->graphs) hipGraphExecDestroy(kv.second);
  for (auto g : m->graph_objs) hipGraphDestroy(g);
  if (m->cap_stream) hipStreamDestroy(m->cap_stream);
  for (hipEvent_t e : m->gate_ev)
    if (e) hipEventDestroy(e);
  if (m->gate_flags) hipHostFree(m->gate_flags);
  delete m;
}

// ------------------------------------------------------------------ decode workspace
struct DecodeWs {
  float* x;
  void* xn;
  void* q;
  void* o;
  void* act;
  void* xsc;
  void* hn;
  float* pe;
  float* lse;
  float* ent;
  float* maxp;
  int32_t* amax;
  uint8_t* committed;
  void* gemm_ws;
  void* attn_ws;
  void* head_ws;
  void* moe_ws;
  // fused layer path: second residual buffer, the two sublayers' XCD partials, per-XCD normed
  // rows, XCD barrier counters and the sync error word
  float* x2;
  float* pa;
  float* pb;
  uint16_t* xn8;
  unsigned* bar;
  int* err;
  size_t total;
};

static AttnPlan model_attn_plan(const dlm_model* m, const dlm_kv* kv) {
  return attn_plan(m->d.hq, m->d.hkv, m->d.head_dim, m->d.block, kv->max_len - m->d.block);
}

// A round fused with the previous block's commit pass runs 64 rows through the layers: the
// bf16 models (dense and MoE) with 32-row blocks do so.
static bool fusable(const dlm_model* m) {
  return m->d.dtype == DLM_BF16 && m->d.block == 32;
}

// Dense bf16 models with 32-row blocks take the prompt in forwards of up to 256 rows (8 blocks,
// block-causal among themselves); the wide GEMMs split those rows over the waves.
constexpr int kWideBlocks = 8;
static bool wide_ok(const dlm_model* m) {
  return m->d.dtype == DLM_BF16 && m->d.block == 32 && m->d.n_experts == 0 && !m->fused;
}

// Decode rounds of bf16 models with 8 (kv head, query-head group) groups merge the attention's
// key splits inside its launch, behind XCD-local barriers whose counters and sync words live
// in the decode workspace (zeroed once by the caller).
static bool xcd_combine(const dlm_model* m) {
  return m->d.dtype == DLM_BF16 && attn_xcd_combine_ok(m->d.hq, m->d.hkv, m->d.block, 1);
}

static DecodeWs decode_layout(const dlm_model* m, const dlm_kv* kv, char* base) {
  const dlm_model_desc& d = m->d;
  const size_t el = d.dtype == DLM_BF16 ? 2 : 4;
  // buffers hold 32 rows (the GEMM B operand reads 32), the layer buffers 64 when a round can
  // carry the previous block's commit rows
  const int B = 32;
  const int BL = wide_ok(m) ? 32 * kWideBlocks : fusable(m) ? 64 : 32;
  const int qd = d.hq * d.head_dim;
  const int F = d.n_experts ? d.expert_ffn : d.ffn;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align_up(bytes, 256); return base + o; };
  DecodeWs w;
  w.x = (float*)take((size_t)BL * d.d * 4);
  w.xn = take((size_t)BL * d.d * el);
  w.q = take((size_t)BL * qd * el);
  w.o = take((size_t)BL * qd * el);
  w.act = take((size_t)BL * F * el);
  w.xsc = take((size_t)B * d.d * el);
  w.hn = take((size_t)B * d.d * el);
  w.pe = (float*)take((size_t)B * d.d * 4);
  w.lse = (float*)take(B * 4);
  w.ent = (float*)take(B * 4);
  w.maxp = (float*)take(B * 4);
  w.amax = (int32_t*)take(B * 4);
  w.committed = (uint8_t*)take(64);
  size_t g = 0;
  if (d.dtype == DLM_BF16) {
    g = std::max(g, gemm_ws_bytes(d.d, d.d, m->pl_sc));
    g = std::max(g, gemm_ws_bytes(m->n_qkv, d.d, m->pl_qkv));
    g = std::max(g, gemm_ws_bytes(d.d, qd, m->pl_o, BL));
    if (!d.n_experts) {
      g = std::max(g, gemm_ws_bytes(2 * d.ffn, d.d, m->pl_gu));
      g = std::max(g, gemm_ws_bytes(d.d, d.ffn, m->pl_dn, BL));
    } else {
      g = std::max(g, gemm_ws_bytes(d.n_experts, d.d, m->pl_router));
    }
  }
  w.gemm_ws = take(g + 256);
  w.attn_ws = take(d.dtype == DLM_BF16 ? attn_ws_bytes(d.hq, d.hkv, d.head_dim, model_attn_plan(m, kv), BL / 32)
                                       : 256);
  w.head_ws = take(head_ws_bytes(d.dtype, d.block, d.d, d.vocab));
  w.moe_ws = take(d.n_experts ? moe_ws_bytes(d) : 0);
  w.x2 = w.pa = w.pb = nullptr;
  w.xn8 = nullptr;
  w.bar = nullptr;
  w.err = nullptr;
  if (m->fused) {
    w.x2 = (float*)take((size_t)64 * d.d * 4);
    w.pa = (float*)take((size_t)64 * 8 * d.d * 4);
    w.pb = (float*)take((size_t)64 * 8 * d.d * 4);
    w.xn8 = (uint16_t*)take((size_t)8 * 64 * d.d * 2);
  }
  if (m->xo) w.pa = (float*)take((size_t)64 * 8 * d.d * 4);   // the attention output's XCD partials
  if (m->fused || m->xo || xcd_combine(m)) {
    w.bar = (unsigned*)take(8 * 64 * 4);
    w.err = (int*)take(9 * 128);
  }
  w.total = off;
  return w;
}

static int check_kv(const dlm_model* m, const dlm_kv* kv) {
  DLM_REQUIRE(m, DLM_ERR_ARG, "model is null");
  DLM_REQUIRE(kv && kv->k && kv->v && kv->len_dev, DLM_ERR_ARG, "kv is null");
  DLM_REQUIRE(kv->cap % 32 == 0, DLM_ERR_SHAPE, "cap must be a multiple of 32 (blocked V cache)");
  DLM_REQUIRE(kv->cap > 0 && kv->max_len >= m->d.block && kv->max_len <= kv->cap, DLM_ERR_SHAPE,
              "kv: need block <= max_len <= cap");
  for (int l = 0; l < m->d.n_layers; ++l)
    DLM_REQUIRE(kv->k[l] && kv->v[l] && aligned16(kv->k[l]) && aligned16(kv->v[l]), DLM_ERR_ARG,
                "kv layer %d: null or misaligned", l);
  DLM_REQUIRE(kv->kv_dtype == m->d.dtype || (kv->kv_dtype == DLM_FP8_E4M3 && m->d.dtype == DLM_BF16),
              DLM_ERR_DTYPE, "kv_dtype %d with a model of dtype %d", kv->kv_dtype, m->d.dtype);
  if (kv->kv_dtype == DLM_FP8_E4M3)
    DLM_REQUIRE(isfinite(kv->k_scale) && isfinite(kv->v_scale) && kv->k_scale > 0.f && kv->v_scale > 0.f,
                DLM_ERR_ARG, "FP8 cache scales must be finite and positive");
  return DLM_OK;
}

extern "C" size_t dlm_decode_ws_bytes(const dlm_model* m, const dlm_kv* kv) {
  if (check_kv(m, kv) != DLM_OK) return 0;
  return decode_layout(m, kv, nullptr).total;
}

extern "C" int dlm_decode_views_get(const dlm_model* m, const dlm_kv* kv, void* ws, size_t ws_bytes,
                                    dlm_decode_views* out) {
  int rc = check_kv(m, kv);
  if (rc) return rc;
  DLM_REQUIRE(ws && out, DLM_ERR_ARG, "null pointer");
  DecodeWs w = decode_layout(m, kv, (char*)ws);
  DLM_REQUIRE(ws_bytes >= w.total, DLM_ERR_WORKSPACE, "workspace too small");
  out->x = w.x;
  out->hn = w.hn;
  out->pe = w.pe;
  out->lse = w.lse;
  out->entropy = w.ent;
  out->maxprob = w.maxp;
  out->argmax = w.amax;
  out->committed = w.committed;
  out->xn = w.xn;
  memset(&out->moe_logits, 0, sizeof(dlm_decode_views) - offsetof(dlm_decode_views, moe_logits));
  if (m->d.n_experts) moe_views(moe_dims(m->d), w.moe_ws, out);
  out->sync_err = w.err;
  return DLM_OK;
}

// ------------------------------------------------------------------ the forward pass
// Runs the residual stream x through every layer.  last_kv_only: the last layer stops after
// its K/V are written (commit pass).  nqb = 2 (bf16, block 32): x holds 64 rows, the previous
// block's committed rows (positions L .. L + 31, whose K/V this pass appends) and then the
// current block's rows (positions L + 32 ..), which also attend to the first 32.
// The bf16 residual projections (attention output, FFN down) leave their sums as deferred
// GEMM partials, which the next RMSNorm adds into the residual stream; *pending describes the
// partials still to be added after the last layer (base == nullptr: none).
static int enqueue_layers(const dlm_model* m, const dlm_kv* kv, const DecodeWs& w, const int32_t* cont,
                          bool last_kv_only, hipStream_t st, PartialSrc* pending, int nqb = 1) {
  const dlm_model_desc& d = m->d;
  const int bf = d.dtype == DLM_BF16;
  const int D = d.head_dim, qd = d.hq * D;
  const int B = nqb == 1 ? d.block : 32 * nqb;   // rows through the GEMMs and norms
  const char* pk = (const char*)m->packed;
  int rc;
  PartialSrc ps{};
  if (m->fused) {
    // x (w.x) -> attention sublayer -> (w.x2, pa) -> FFN sublayer -> (w.x, pb) per layer
    const LayerBufs lb{w.xn8, (uint16_t*)w.q, (uint16_t*)w.o, (uint16_t*)w.act, w.attn_ws, w.bar, w.err};
    const AttnKv kvf{kv->kv_dtype == DLM_FP8_E4M3 ? 1 : 0, kv->k_scale, kv->v_scale};
    for (int l = 0; l < d.n_layers; ++l) {
      const dlm_layer_weights& L = m->layers[l];
      const bool kv_only = last_kv_only && l == d.n_layers - 1;
      EpiParams e = epi_zero();
      e.kind = EPI_QKV_ROPE;
      e.M = B;
      e.bf16_out = 1;
      e.k_cache = kv->k[l];
      e.v_cache = kv->v[l];
      e.hq = d.hq;
      e.hkv = d.hkv;
      e.D = D;
      e.cap = kv->cap;
      e.len_dev = kv->len_dev;
      e.rope_r = pow((double)d.rope_base, -2.0 / (double)D);
      e.kv8 = kvf.fp8;
      e.k_scale = kvf.fp8 ? kv->k_scale : 1.0f;
      e.v_scale = kvf.fp8 ? kv->v_scale : 1.0f;
      const LayerIO ioa{w.x, l ? w.pb : nullptr, w.x2, w.pa};
      if ((rc = fused_attn_sublayer(m->fd, nqb, (const uint16_t*)(pk + m->off_qkv[l]),
                                    (const uint16_t*)(pk + m->off_o[l]), L.attn_norm, d.eps, ioa, lb, e,
                                    model_attn_plan(m, kv), 1.0f / sqrtf((float)D), kvf, kv_only, cont, st)))
        return rc;
      if (kv_only) break;
      const LayerIO iof{w.x2, w.pa, w.x, w.pb};
      if ((rc = fused_ffn_sublayer(m->fd, nqb, (const uint16_t*)(pk + m->off_gu[l]),
                                   (const uint16_t*)(pk + m->off_dn[l]), L.ffn_norm, d.eps, iof, lb, cont, st)))
        return rc;
    }
    // the last FFN's 8 XCD partials are added into x by the final norm, in XCD order
    ps.slots = w.pb;
    ps.nslot = 8;
    *pending = ps;
    return DLM_OK;
  }
  for (int l = 0; l < d.n_layers; ++l) {
    const dlm_layer_weights& L = m->layers[l];
    const bool last = l == d.n_layers - 1;
    if ((rc = rmsnorm(w.x, L.attn_norm, w.xn, B, d.d, bf, bf, d.eps, cont, st, &ps))) return rc;
    ps = PartialSrc{};
    EpiParams e = epi_zero();
    e.kind = EPI_QKV_ROPE;
    e.M = B;
    e.bf16_out = bf;
    e.q_out = w.q;
    e.k_cache = kv->k[l];
    e.v_cache = kv->v[l];
    e.hq = d.hq;
    e.hkv = d.hkv;
    e.D = D;
    e.cap = kv->cap;
    e.len_dev = kv->len_dev;
    e.rope_r = pow((double)d.rope_base, -2.0 / (double)D);
    e.kv8 = kv->kv_dtype == DLM_FP8_E4M3;
    e.k_scale = e.kv8 ? kv->k_scale : 1.0f;
    e.v_scale = e.kv8 ? kv->v_scale : 1.0f;
    e.cont_dev = cont;
    if (bf) rc = gemm_bf16(pk + m->off_qkv[l], w.xn, m->n_qkv, d.d, MAP_QKV, e, m->pl_qkv, w.gemm_ws, st);
    else {
      F32Mats W{};
      W.w[0] = (const float*)L.wq; W.rows[0] = d.hq * D;
      W.w[1] = (const float*)L.wk; W.rows[1] = d.hkv * D;
      W.w[2] = (const float*)L.wv; W.rows[2] = d.hkv * D;
      rc = gemm_f32(W, (const float*)w.xn, m->n_qkv, d.d, MAP_QKV, e, st);
    }
    if (rc) return rc;
    if (last && last_kv_only) break;
    const float scale = 1.0f / sqrtf((float)D);
    if (m->xo && nqb <= 2) {
      // attention and output projection in one launch; its 8 XCD partials are added into x by
      // the next RMSNorm, in XCD order
      if ((rc = attn_out_xcd(m->fd, nqb, (const uint16_t*)(pk + m->off_ox[l]), (const uint16_t*)w.q, kv->k[l],
                             kv->v[l], (uint16_t*)w.o, w.attn_ws, w.pa, w.bar, w.err, kv->cap, kv->len_dev,
                             model_attn_plan(m, kv), scale,
                             AttnKv{kv->kv_dtype == DLM_FP8_E4M3 ? 1 : 0, kv->k_scale, kv->v_scale}, cont, st)))
        return rc;
      ps = PartialSrc{};
      ps.slots = w.pa;
      ps.nslot = 8;
    } else {
      if (bf) rc = attn_bf16(w.q, kv->k[l], kv->v[l], w.o, d.hq, d.hkv, D, d.block, nqb, kv->cap, scale, kv->len_dev,
                             0, cont, model_attn_plan(m, kv), w.attn_ws, /*out_packed=*/1, st,
                             AttnKv{kv->kv_dtype == DLM_FP8_E4M3 ? 1 : 0, kv->k_scale, kv->v_scale},
                             AttnXSync{w.bar, w.err});
      else rc = attn_f32((const float*)w.q, (const float*)kv->k[l], (const float*)kv->v[l], (float*)w.o, d.hq, d.hkv,
                         D, B, kv->cap, scale, kv->len_dev, 0, cont, st);
      if (rc) return rc;
      e = epi_zero();
      e.kind = bf && !m->pl_o.R ? EPI_PARTIAL : EPI_RESID;
      e.M = B;
      e.bf16_out = bf;
      e.out = w.x;
      e.ld_out = d.d;
      e.cont_dev = cont;
      if (bf) {
        rc = gemm_bf16(pk + m->off_o[l], w.o, d.d, qd, MAP_IDENTITY, e, m->pl_o, w.gemm_ws, st);
        if (!m->pl_o.R) ps = gemm_partials(d.d, qd, m->pl_o, w.gemm_ws, B);
      } else {
        F32Mats W{};
        W.w[0] = (const float*)L.wo; W.rows[0] = d.d;
        rc = gemm_f32(W, (const float*)w.o, d.d, qd, MAP_IDENTITY, e, st);
      }
      if (rc) return rc;
    }
    if ((rc = rmsnorm(w.x, L.ffn_norm, w.xn, B, d.d, bf, bf, d.eps, cont, st, &ps))) return rc;
    ps = PartialSrc{};
    if (d.n_experts) {
      // the experts' weighted outputs are added into x by the next RMSNorm, slot by slot
      MoeDims md = moe_dims(d);
      md.rows = B;
      if ((rc = moe_ffn(md, l, w.xn, pk + m->off_router[l], m->pl_router, pk + m->off_moe[l], w.moe_ws,
                        w.gemm_ws, cont, &ps, st)))
        return rc;
      continue;
    }
    e = epi_zero();
    e.kind = EPI_SWIGLU;
    e.M = B;
    e.bf16_out = bf;
    e.act_out = w.act;
    e.F = d.ffn;
    e.cont_dev = cont;
    if (bf) rc = gemm_bf16(pk + m->off_gu[l], w.xn, 2 * d.ffn, d.d, MAP_GU, e, m->pl_gu, w.gemm_ws, st);
    else {
      F32Mats W{};
      W.w[0] = (const float*)L.wg; W.rows[0] = d.ffn;
      W.w[1] = (const float*)L.wu; W.rows[1] = d.ffn;
      rc = gemm_f32(W, (const float*)w.xn, 2 * d.ffn, d.d, MAP_GU, e, st);
    }
    if (rc) return rc;
    e = epi_zero();
    e.kind = bf && !m->pl_dn.R ? EPI_PARTIAL : EPI_RESID;
    e.M = B;
    e.bf16_out = bf;
    e.out = w.x;
    e.ld_out = d.d;
    e.cont_dev = cont;
    if (bf) {
      rc = gemm_bf16(pk + m->off_dn[l], w.act, d.d, d.ffn, MAP_IDENTITY, e, m->pl_dn, w.gemm_ws, st);
      if (!m->pl_dn.R) ps = gemm_partials(d.d, d.ffn, m->pl_dn, w.gemm_ws, B);
    } else {
      F32Mats W{};
      W.w[0] = (const float*)L.wd; W.rows[0] = d.d;
      rc = gemm_f32(W, (const float*)w.act, d.d, d.ffn, MAP_IDENTITY, e, st);
    }
    if (rc) return rc;
  }
  *pending = ps;
  return DLM_OK;
}

static int enqueue_round(const dlm_model* m, const dlm_commit_rule& rule, const dlm_kv* kv, int32_t* tokens,
                         dlm_round_state* state, const DecodeWs& w, hipStream_t st) {
  const dlm_model_desc& d = m->d;
  const int bf = d.dtype == DLM_BF16;
  const int B = d.block;
  // A fixed-k rule enqueues exactly the rounds the block needs, so its kernels need not read
  // the continue flag; a threshold rule enqueues max_rounds rounds and every kernel of a round
  // after the block completed exits at once.
  const int32_t* cont = rule.mode == DLM_COMMIT_FIXED_K ? nullptr : &state->cont;
  int rc;
  // round input: E[tok] for committed rows, mask + W_sc bf(pe) for open rows
  if ((rc = selfcond_prep(w.pe, w.committed, w.xsc, B, d.d, bf, cont, st))) return rc;
  EpiParams e = epi_zero();
  e.kind = EPI_SELFCOND;
  e.M = B;
  e.bf16_out = bf;
  e.out = w.x;
  e.ld_out = d.d;
  e.mask_emb = m->mask_emb;
  e.emb = m->emb;
  e.tokens = tokens;
  e.committed = w.committed;
  e.vocab = d.vocab;
  e.cont_dev = cont;
  if (bf) rc = gemm_bf16((const char*)m->packed + m->off_sc, w.xsc, d.d, d.d, MAP_IDENTITY, e, m->pl_sc,
                         w.gemm_ws, st);
  else {
    F32Mats W{};
    W.w[0] = (const float*)m->w_sc;
    W.rows[0] = d.d;
    rc = gemm_f32(W, (const float*)w.xsc, d.d, d.d, MAP_IDENTITY, e, st);
  }
  if (rc) return rc;
  PartialSrc ps{};
  if ((rc = enqueue_layers(m, kv, w, cont, false, st, &ps))) return rc;
  if ((rc = rmsnorm(w.x, m->final_norm, w.hn, B, d.d, bf, 0, d.eps, cont, st, &ps))) return rc;
  if ((rc = head_launch(d.dtype, w.hn, m->emb, w.committed, B, d.d, d.vocab, w.lse, w.ent, w.maxp, w.amax, w.pe,
                        nullptr, w.head_ws, cont, st)))
    return rc;
  return commit_launch(rule, B, w.maxp, w.amax, w.lse, w.ent, w.committed, tokens, state, st);
}

static int enqueue_commit_pass(const dlm_model* m, const dlm_kv* kv, const int32_t* tokens, const DecodeWs& w,
                               hipStream_t st) {
  const dlm_model_desc& d = m->d;
  int rc;
  if ((rc = embed(tokens, m->emb, w.x, d.block, d.d, d.vocab, d.dtype == DLM_BF16, st))) return rc;
  PartialSrc ps{};
  if ((rc = enqueue_layers(m, kv, w, nullptr, true, st, &ps))) return rc;
  return len_add(kv->len_dev, d.block, st);
}

// Round 0 of a block fused with the commit pass of the previous block (prev_tokens, whose K/V
// are not yet in the cache): one 64-row pass whose first 32 rows are the previous block's
// committed tokens at positions L .. L + 31 and whose last 32 rows are round 0 of this block
// at L + 32 .., which attend to the prefix, to the previous block and to each other.  Every
// row computes what the separate commit pass and round would; the weights stream once.
static int enqueue_fused_round0(const dlm_model* m, const dlm_commit_rule& rule, const dlm_kv* kv,
                                const int32_t* prev_tokens, int32_t* tokens, dlm_round_state* state,
                                const DecodeWs& w, hipStream_t st) {
  const dlm_model_desc& d = m->d;
  const int B = d.block;
  const int32_t* cont = rule.mode == DLM_COMMIT_FIXED_K ? nullptr : &state->cont;
  int rc;
  float* x_round = w.x + (size_t)B * d.d;
  if ((rc = embed(prev_tokens, m->emb, w.x, B, d.d, d.vocab, 1, st))) return rc;
  if ((rc = selfcond_prep(w.pe, w.committed, w.xsc, B, d.d, 1, nullptr, st))) return rc;
  EpiParams e = epi_zero();
  e.kind = EPI_SELFCOND;
  e.M = B;
  e.bf16_out = 1;
  e.out = x_round;
  e.ld_out = d.d;
  e.mask_emb = m->mask_emb;
  e.emb = m->emb;
  e.tokens = tokens;
  e.committed = w.committed;
  e.vocab = d.vocab;
  if ((rc = gemm_bf16((const char*)m->packed + m->off_sc, w.xsc, d.d, d.d, MAP_IDENTITY, e, m->pl_sc, w.gemm_ws,
                      st)))
    return rc;
  PartialSrc ps{};
  if ((rc = enqueue_layers(m, kv, w, nullptr, false, st, &ps, /*nqb=*/2))) return rc;
  ps.row0 = B;   // the final norm serves the round's rows only
  if ((rc = rmsnorm(x_round, m->final_norm, w.hn, B, d.d, 1, 0, d.eps, nullptr, st, &ps))) return rc;
  if ((rc = len_add(kv->len_dev, B, st))) return rc;   // the previous block is now in the cache
  if ((rc = head_launch(d.dtype, w.hn, m->emb, w.committed, B, d.d, d.vocab, w.lse, w.ent, w.maxp, w.amax, w.pe,
                        nullptr, w.head_ws, cont, st)))
    return rc;
  return commit_launch(rule, B, w.maxp, w.amax, w.lse, w.ent, w.committed, tokens, state, st);
}

static int n_rounds(const dlm_model* m, const dlm_commit_rule& r) {
  if (r.mode == DLM_COMMIT_FIXED_K) {
    const int n = (m->d.block + r.k - 1) / r.k;
    return n < r.max_rounds ? n : r.max_rounds;
  }
  return r.max_rounds;
}

static int enqueue_block(const dlm_model* m, const dlm_commit_rule& rule, const dlm_kv* kv, int32_t* tokens,
                         dlm_round_state* state, const DecodeWs& w, hipStream_t st) {
  int rc;
  if ((rc = block_reset(m->d.block, w.committed, tokens, state, w.pe, 32 * m->d.d, st))) return rc;
  const int R = n_rounds(m, rule);
  for (int r = 0; r < R; ++r)
    if ((rc = enqueue_round(m, rule, kv, tokens, state, w, st))) return rc;
  return enqueue_commit_pass(m, kv, tokens, w, st);
}

// A block whose own commit pass is left to the next block (or to dlm_commit_pass): the
// previous block's pending commit pass runs fused into round 0 when the model allows it, else
// on its own before round 0.
static int enqueue_block_pipelined(const dlm_model* m, const dlm_commit_rule& rule, const dlm_kv* kv,
                                   const int32_t* prev_tokens, int32_t* tokens, dlm_round_state* state,
                                   const DecodeWs& w, hipStream_t st) {
  int rc;
  if ((rc = block_reset(m->d.block, w.committed, tokens, state, w.pe, 32 * m->d.d, st))) return rc;
  const int R = n_rounds(m, rule);
  int r = 0;
  if (prev_tokens && fusable(m)) {
    if ((rc = enqueue_fused_round0(m, rule, kv, prev_tokens, tokens, state, w, st))) return rc;
    r = 1;
  } else if (prev_tokens) {
    if ((rc = enqueue_commit_pass(m, kv, prev_tokens, w, st))) return rc;
  }
  for (; r < R; ++r)
    if ((rc = enqueue_round(m, rule, kv, tokens, state, w, st))) return rc;
  return DLM_OK;
}

static int check_decode(const dlm_model* m, const dlm_kv* kv, void* ws, size_t ws_bytes) {
  int rc = check_kv(m, kv);
  if (rc) return rc;
  DLM_REQUIRE(ws && aligned16(ws), DLM_ERR_ARG, "workspace null or misaligned");
  DLM_REQUIRE(ws_bytes >= decode_layout(m, kv, nullptr).total, DLM_ERR_WORKSPACE, "workspace too small");
  return DLM_OK;
}

extern "C" size_t dlm_ffn_gate_up_ws_bytes(const dlm_model* m) {
  if (!m || m->d.dtype != DLM_BF16 || m->d.n_experts) return 0;
  return gemm_ws_bytes(2 * m->d.ffn, m->d.d, m->pl_gu);
}

extern "C" int dlm_ffn_gate_up(const dlm_model* m, int layer, const void* x_packed, void* act_packed, void* ws,
                               size_t ws_bytes, void* stream) {
  DLM_REQUIRE(m && x_packed && act_packed && ws, DLM_ERR_ARG, "null pointer");
  DLM_REQUIRE(m->d.dtype == DLM_BF16 && m->d.n_experts == 0, DLM_ERR_DTYPE, "dense bf16 models only");
  DLM_REQUIRE(layer >= 0 && layer < m->d.n_layers, DLM_ERR_ARG, "layer out of range");
  DLM_REQUIRE(aligned16(x_packed) && aligned16(act_packed) && aligned16(ws), DLM_ERR_ARG,
              "16-byte alignment required");
  DLM_REQUIRE(ws_bytes >= dlm_ffn_gate_up_ws_bytes(m), DLM_ERR_WORKSPACE, "workspace too small");
  DLM_DEVICE_CHECK();
  EpiParams e = epi_zero();
  e.kind = EPI_SWIGLU;
  e.M = m->d.block;
  e.bf16_out = 1;
  e.act_out = act_packed;
  e.F = m->d.ffn;
  return gemm_bf16((const char*)m->packed + m->off_gu[layer], x_packed, 2 * m->d.ffn, m->d.d, MAP_GU, e, m->pl_gu,
                   ws, (hipStream_t)stream);
}

static void block_graph_key(const dlm_model* m, const dlm_commit_rule* rule, const dlm_kv* kv,
                            const int32_t* prev_tokens, int pipelined, const int32_t* tokens,
                            const dlm_round_state* state, const void* ws, GraphKey* key) {
  auto bits = [](float f) { uint32_t u; memcpy(&u, &f, 4); return (uint64_t)u; };
  auto ptr = [](const void* p) { return (uint64_t)(uintptr_t)p; };
  key->assign({(uint64_t)rule->mode, bits(rule->tau), (uint64_t)rule->k, (uint64_t)rule->forced_top1,
               (uint64_t)rule->max_rounds, ptr(tokens), ptr(state), ptr(ws), ptr(kv->len_dev), (uint64_t)pipelined,
               ptr(prev_tokens), (uint64_t)kv->kv_dtype, bits(kv->k_scale), bits(kv->v_scale), (uint64_t)kv->cap,
               (uint64_t)kv->max_len, (uint64_t)m->d.n_layers});
  for (int l = 0; l < m->d.n_layers; ++l) {
    key->push_back(ptr(kv->k[l]));
    key->push_back(ptr(kv->v[l]));
  }
}

extern "C" int dlm_block_graph_key(const dlm_model* m, const dlm_commit_rule* rule, const dlm_kv* kv,
                                   const int32_t* prev_tokens, int pipelined, const int32_t* tokens,
                                   const dlm_round_state* state, const void* ws, uint64_t* words, int max_words) {
  int rc = check_kv(m, kv);
  if (rc) return rc;
  if ((rc = check_rule(rule))) return rc;
  DLM_REQUIRE(words && max_words >= 0, DLM_ERR_ARG, "null key buffer");
  GraphKey key;
  block_graph_key(m, rule, kv, prev_tokens, pipelined, tokens, state, ws, &key);
  DLM_REQUIRE((size_t)max_words >= key.size(), DLM_ERR_ARG, "key needs %zu words", key.size());
  memcpy(words, key.data(), key.size() * sizeof(uint64_t));
  return (int)key.size();
}

extern "C" int dlm_model_graph_count(const dlm_model* m) {
  DLM_REQUIRE(m, DLM_ERR_ARG, "model is null");
  dlm_model* mm = const_cast<dlm_model*>(m);
  std::lock_guard<std::mutex> lock(mm->mu);
  return (int)mm->graphs.size();
}

// Captures (once per key) the work enq(stream) enqueues, and launches it.
template <class Enq>
static int launch_cached_graph(const dlm_model* m, const GraphKey& key, Enq enq, hipStream_t st) {
  dlm_model* mm = const_cast<dlm_model*>(m);
  std::lock_guard<std::mutex> lock(mm->mu);
  auto it = mm->graphs.find(key);
  if (it == mm->graphs.end()) {
    if (!mm->cap_stream) DLM_HIP(hipStreamCreateWithFlags(&mm->cap_stream, hipStreamNonBlocking));
    DLM_HIP(hipStreamBeginCapture(mm->cap_stream, hipStreamCaptureModeThreadLocal));
    int rc = enq(mm->cap_stream);
    hipGraph_t g = nullptr;
    hipError_t e2 = hipStreamEndCapture(mm->cap_stream, &g);
    if (rc) {
      if (g) hipGraphDestroy(g);
      return rc;
    }
    if (e2 != hipSuccess) return check_hip(e2, "hipStreamEndCapture");
    hipGraphExec_t ex = nullptr;
    hipError_t e3 = hipGraphInstantiate(&ex, g, nullptr, nullptr, 0);
    if (e3 != hipSuccess) {
      hipGraphDestroy(g);
      return check_hip(e3, "hipGraphInstantiate");
    }
    mm->graph_objs.push_back(g);
    it = mm->graphs.emplace(key, ex).first;
  }
  return check_hip(hipGraphLaunch(it->second, st), "hipGraphLaunch");
}

// Captures (once per key) and launches the graph of one block.
static int launch_block_graph(const dlm_model* m, const dlm_commit_rule* rule, const dlm_kv* kv,
                              const int32_t* prev_tokens, int pipelined, int32_t* tokens, dlm_round_state* state,
                              void* ws, hipStream_t st) {
  const DecodeWs w = decode_layout(m, kv, (char*)ws);
  GraphKey key;
  block_graph_key(m, rule, kv, prev_tokens, pipelined, tokens, state, ws, &key);
  return launch_cached_graph(m, key, [&](hipStream_t cs) {
    return pipelined ? enqueue_block_pipelined(m, *rule, kv, prev_tokens, tokens, state, w, cs)
                     : enqueue_block(m, *rule, kv, tokens, state, w, cs);
  }, st);
}

extern "C" int dlm_decode_block(const dlm_model* m, const dlm_commit_rule* rule, const dlm_kv* kv, int32_t* tokens,
                                dlm_round_state* state, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_decode(m, kv, ws, ws_bytes);
  if (rc) return rc;
  if ((rc = check_rule(rule))) return rc;
  DLM_REQUIRE(tokens && state, DLM_ERR_ARG, "null pointer");
  DLM_DEVICE_CHECK();
  return launch_block_graph(m, rule, kv, nullptr, 0, tokens, state, ws, (hipStream_t)stream);
}

extern "C" int dlm_decode_block_pipelined(const dlm_model* m, const dlm_commit_rule* rule, const dlm_kv* kv,
                                          const int32_t* prev_tokens, int32_t* tokens, dlm_round_state* state,
                                          void* ws, size_t ws_bytes, void* stream) {
  int rc = check_decode(m, kv, ws, ws_bytes);
  if (rc) return rc;
  if ((rc = check_rule(rule))) return rc;
  DLM_REQUIRE(tokens && state, DLM_ERR_ARG, "null pointer");
  DLM_REQUIRE(prev_tokens != tokens, DLM_ERR_ARG, "prev_tokens and tokens must be distinct buffers");
  DLM_DEVICE_CHECK();
  return launch_block_graph(m, rule, kv, prev_tokens, 1, tokens, state, ws, (hipStream_t)stream);
}

// A threshold block as graphs of seg_rounds rounds, one segment in flight ahead of the one the
// host waits on: after each segment the continue flag goes to pinned host memory behind an
// event, and no further segment is launched once a segment has ended the block.  At most one
// speculative segment runs without work (its kernels read the flag and exit); the commit pass
// follows as its own graph.  Graphs are cached under the block's key plus the segment kind.
extern "C" int dlm_decode_block_gated(const dlm_model* m, const dlm_commit_rule* rule, const dlm_kv* kv,
                                      int32_t* tokens, dlm_round_state* state, void* ws, size_t ws_bytes,
                                      int seg_rounds, void* stream) {
  int rc = check_decode(m, kv, ws, ws_bytes);
  if (rc) return rc;
  if ((rc = check_rule(rule))) return rc;
  DLM_REQUIRE(tokens && state, DLM_ERR_ARG, "null pointer");
  DLM_REQUIRE(seg_rounds >= 1, DLM_ERR_ARG, "seg_rounds must be at least 1");
  DLM_DEVICE_CHECK();
  hipStream_t st = (hipStream_t)stream;
  if (rule->mode == DLM_COMMIT_FIXED_K)   // the round count is known: no round runs without work
    return launch_block_graph(m, rule, kv, nullptr, 0, tokens, state, ws, st);
  dlm_model* mm = const_cast<dlm_model*>(m);
  std::lock_guard<std::mutex> gate_lock(mm->gate_mu);
  if (!mm->gate_flags) {
    DLM_HIP(hipHostMalloc((void**)&mm->gate_flags, 2 * sizeof(int32_t), hipHostMallocDefault));
    for (hipEvent_t& e : mm->gate_ev) DLM_HIP(hipEventCreateWithFlags(&e, hipEventDisableTiming));
  }
  // a flag copy the previous call left in flight (its last, speculative segment) must land
  // before this call's copies reuse the slots, whatever stream it ran on
  if (mm->gate_last >= 0) DLM_HIP(hipEventSynchronize(mm->gate_ev[mm->gate_last]));
  mm->gate_last = -1;
  const DecodeWs w = decode_layout(m, kv, (char*)ws);
  const int S = std::min(seg_rounds, rule->max_rounds);
  const int nseg = (rule->max_rounds + S - 1) / S;
  GraphKey base;
  block_graph_key(m, rule, kv, nullptr, 0, tokens, state, ws, &base);
  auto key_of = [&](uint64_t kind) {
    GraphKey k = base;
    k.push_back(0x6761746564ull);   // gated-decode graphs
    k.push_back(kind);
    k.push_back((uint64_t)S);
    return k;
  };
  auto launch_seg = [&](int j) -> int {
    int r2 = launch_cached_graph(m, key_of(j == 0 ? 0 : 1), [&](hipStream_t cs) {
      int r3;
      if (j == 0 && (r3 = block_reset(m->d.block, w.committed, tokens, state, w.pe, 32 * m->d.d, cs))) return r3;
      for (int r = 0; r < S; ++r)
        if ((r3 = enqueue_round(m, *rule, kv, tokens, state, w, cs))) return r3;
      return (int)DLM_OK;
    }, st);
    if (r2) return r2;
    DLM_HIP(hipMemcpyAsync(&mm->gate_flags[j & 1], &state->cont, sizeof(int32_t), hipMemcpyDeviceToHost, st));
    DLM_HIP(hipEventRecord(mm->gate_ev[j & 1], st));
    mm->gate_last = j & 1;
    return DLM_OK;
  };
  if ((rc = launch_seg(0))) return rc;
  if (nseg > 1 && (rc = launch_seg(1))) return rc;
  for (int j = 0; j < nseg; ++j) {
    DLM_HIP(hipEventSynchronize(mm->gate_ev[j & 1]));
    if (((volatile int32_t*)mm->gate_flags)[j & 1] == 0) break;   // segment j ended the block
    if (j + 2 < nseg && (rc = launch_seg(j + 2))) return rc;
  }
  return launch_cached_graph(m, key_of(2), [&](hipStream_t cs) { return enqueue_commit_pass(m, kv, tokens, w, cs); },
                             st);
}

extern "C" int dlm_decode_begin(const dlm_model* m, const dlm_kv* kv, int32_t* tokens, dlm_round_state* state,
                                void* ws, size_t ws_bytes, void* stream) {
  int rc = check_decode(m, kv, ws, ws_bytes);
  if (rc) return rc;
  DLM_REQUIRE(tokens && state, DLM_ERR_ARG, "null pointer");
  DLM_DEVICE_CHECK();
  DecodeWs w = decode_layout(m, kv, (char*)ws);
  return block_reset(m->d.block, w.committed, tokens, state, w.pe, 32 * m->d.d, (hipStream_t)stream);
}

extern "C" int dlm_decode_round(const dlm_model* m, const dlm_commit_rule* rule, const dlm_kv* kv, int32_t* tokens,
                                dlm_round_state* state, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_decode(m, kv, ws, ws_bytes);
  if (rc) return rc;
  if ((rc = check_rule(rule))) return rc;
  DLM_REQUIRE(tokens && state, DLM_ERR_ARG, "null pointer");
  DLM_DEVICE_CHECK();
  DecodeWs w = decode_layout(m, kv, (char*)ws);
  return enqueue_round(m, *rule, kv, tokens, state, w, (hipStream_t)stream);
}

extern "C" int dlm_commit_pass(const dlm_model* m, const dlm_kv* kv, const int32_t* tokens, void* ws,
                               size_t ws_bytes, void* stream) {
  int rc = check_decode(m, kv, ws, ws_bytes);
  if (rc) return rc;
  DLM_REQUIRE(tokens, DLM_ERR_ARG, "null tokens");
  DLM_DEVICE_CHECK();
  DecodeWs w = decode_layout(m, kv, (char*)ws);
  return enqueue_commit_pass(m, kv, tokens, w, (hipStream_t)stream);
}

// The prompt as forwards of up to max_blocks blocks: each forward's rows attend to the cached
// prefix and, block-causally, to each other (block j of the forward sees blocks 0 .. j), as a
// run of consecutive commit passes would.  Wide forwards (3 to 8 blocks) go to the dense bf16
// models, pairs to the models that run 64-row rounds, single blocks to every model.
static int enqueue_prefill(const dlm_model* m, const int32_t* ids, int nb, const dlm_kv* kv, const DecodeWs& w,
                           int max_blocks, hipStream_t st) {
  const dlm_model_desc& d = m->d;
  const int B = d.block;
  int rc;
  for (int b = 0; b < nb;) {
    int c = std::min(max_blocks, nb - b);
    if (c >= 3 && !wide_ok(m)) c = 2;
    if (c == 2 && !fusable(m)) c = 1;
    if (c == 1) {
      if ((rc = enqueue_commit_pass(m, kv, ids + (size_t)b * B, w, st))) return rc;
    } else {
      if ((rc = embed(ids + (size_t)b * B, m->emb, w.x, c * B, d.d, d.vocab, 1, st))) return rc;
      PartialSrc ps{};
      if ((rc = enqueue_layers(m, kv, w, nullptr, /*last_kv_only=*/true, st, &ps, /*nqb=*/c))) return rc;
      if ((rc = len_add(kv->len_dev, c * B, st))) return rc;
    }
    b += c;
  }
  return DLM_OK;
}

static int prefill_impl(const dlm_model* m, const int32_t* ids, int n, const dlm_kv* kv, void* ws, size_t ws_bytes,
                        int max_blocks, void* stream) {
  int rc = check_decode(m, kv, ws, ws_bytes);
  if (rc) return rc;
  DLM_REQUIRE(ids, DLM_ERR_ARG, "null ids");
  DLM_REQUIRE(n >= 0 && n % m->d.block == 0, DLM_ERR_SHAPE, "n must be a multiple of the block size");
  DLM_DEVICE_CHECK();
  const DecodeWs w = decode_layout(m, kv, (char*)ws);
  return enqueue_prefill(m, ids, n / m->d.block, kv, w, max_blocks, (hipStream_t)stream);
}

extern "C" int dlm_prefill(const dlm_model* m, const int32_t* ids, int n, const dlm_kv* kv, void* ws,
                           size_t ws_bytes, void* stream) {
  return prefill_impl(m, ids, n, kv, ws, ws_bytes, kWideBlocks, stream);
}

extern "C" int dlm_prefill_rows(const dlm_model* m, const int32_t* ids, int n, const dlm_kv* kv, void* ws,
                                size_t ws_bytes, int max_rows, void* stream) {
  DLM_REQUIRE(m, DLM_ERR_ARG, "model is null");
  DLM_REQUIRE(max_rows >= m->d.block, DLM_ERR_ARG, "max_rows must be at least one block");
  return prefill_impl(m, ids, n, kv, ws, ws_bytes, std::min(kWideBlocks, max_rows / m->d.block), stream);
}

// Block attention: B block queries attend to the L prefix keys and all B block keys,
// with no mask (a denoising round predicts the block's unresolved positions together,
// page "ORL: diffusion LLMs get a learnable 'tokens per forward'", section "What shipped").
//
// The V cache is stored transposed in 32-key blocks, [kv head][cap/32][D][32], so that 8
// consecutive keys of one value column are one 16-byte load and a 32-key tile of V^T is one
// contiguous run.
//
// bf16 path (attn_body.h).  One workgroup per (kv head, group of up to 4 query heads, key
// split), one wave per query head.  A split is processed in passes of two 32-key tiles: the
// pass's K and V^T tiles are loaded once per workgroup (non-temporal buffer loads into
// registers), staged into double-buffered LDS with padded rows, and shared by the waves while
// the next pass is in flight.  Scores are computed transposed, S^T = K Q^T, with
// v_mfma_f32_16x16x32_bf16; the K rows fed to the MFMA are permuted so that lane l owns one
// query (l % 16) and 8 consecutive keys of each tile, so the online-softmax statistics stay in
// the lane (two permlane-swap exchanges finish a row) and the probabilities are already the B operand of
// O^T = V^T P^T, whose A operand is one 16-byte LDS read of V^T.  The split count is chosen
// on the device from the prefix length (the fewest passes per split within 32 splits), and
// the 64-key passes are dealt to the splits in turn, so each split's first pass (keys
// [64 s, 64 s + 64)) is requested before the prefix length arrives.  With
// one split the normalised output is written directly; otherwise each split writes its
// normalised output (bf16) with its running max and sum, and a combine kernel merges the
// splits in index order.  Deterministic throughout.  An FP8 e4m3 cache is widened to bf16 on
// its way into LDS; the key scale is folded into the softmax scale, the value scale into the
// output.
//
// Decode rounds of models with exactly 8 (kv head, query-head group) groups merge the splits
// inside the attention launch instead: the 32 splits of group x are workgroups x, x + 8, ..,
// which the dispatcher places on one XCD, so after storing its split each workgroup meets the
// other 31 at an XCD-local barrier (xcd.h) and then merges 1/32 of the group's outputs from the
// XCD's L2, in the same split order and arithmetic as the combine kernel.  That removes one
// launch from every layer.
#include "attn.h"
#include "attn_body.h"
#include "xcd.h"

#include <algorithm>
#include <type_traits>

namespace dlm {

namespace {

template <int D, int WPG, bool KV8 = false>
__global__ __launch_bounds__(64 * WPG) __attribute__((amdgpu_waves_per_eu(2))) void attn_bf16_kernel(AttnP p) {
  DLM_TRACE_POINT(0);
  if (p.cont_dev && *p.cont_dev == 0) return;
  __shared__ __attribute__((aligned(16))) uint8_t smem[attn_smem_bytes<D, WPG>()];
  const int G = p.hq / p.hkv;
  const int HG = G / WPG;
  const int per_qb = p.hkv * HG * p.nsplit_max;
  const int qblk = blockIdx.x / per_qb, bx = blockIdx.x % per_qb;
  const int s = bx % p.nsplit_max, gh = bx / p.nsplit_max;
  attn_split_body<D, WPG, KV8, false>(p, qblk, gh / HG, gh % HG, s, smem);
}

// One workgroup per (group x = blockIdx % 8, split s = blockIdx / 8): the group's kWgPerXcd
// workgroups always launch (splits past the prefix's split count only take part in the
// merge), so every barrier counts kWgPerXcd arrivals whatever the plan.
template <int D, int WPG, bool KV8 = false>
__global__ __launch_bounds__(64 * WPG) __attribute__((amdgpu_waves_per_eu(2))) void attn_bf16_xcd_kernel(
    AttnP p, AttnXSync xs) {
  if (p.cont_dev && *p.cont_dev == 0) return;
  __shared__ __attribute__((aligned(16))) uint8_t smem[attn_smem_bytes<D, WPG>()];
  const int x = blockIdx.x & (kXcds - 1), s = blockIdx.x / kXcds;
  const int HG = (p.hq / p.hkv) / WPG;
  publish_placement(xs.err, x, s);
  attn_split_body<D, WPG, KV8, false>(p, 0, x / HG, x % HG, s, smem);
  // the split count, as every workgroup computes it; with one split the output is complete
  const int N = min((p.len_dev ? *p.len_dev : p.len_host) + p.B, p.cap);
  const int chunk = split_chunk(N, p.nsplit_max);
  if ((N + chunk - 1) / chunk <= 1) return;
  xcd_sync(xs.bar + 64 * x, xs.err);
  check_placement(xs.err, x);
  // group x's outputs: query heads WPG x .. WPG x + WPG - 1, D / 4 threads per (head, query)
  constexpr int TPQ = D / 4;
  const int items = WPG * p.B * TPQ;
  for (int it = s * 64 * WPG + (int)threadIdx.x; it < items; it += kWgPerXcd * 64 * WPG) {
    const int hl = it / (p.B * TPQ), qi = (it / TPQ) % p.B;
    attn_combine_item<D, true>(p, 0, WPG * x + hl, qi, 4 * (it % TPQ));
  }
}

template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnP p) {
  if (p.cont_dev && *p.cont_dev == 0) return;
  constexpr int TPQ = D / 4, PPW = 256 / TPQ;     // threads per (head, query), pairs per workgroup
  const int pair = blockIdx.x * PPW + threadIdx.x / TPQ;
  const int dv = 4 * (threadIdx.x % TPQ);
  const int qblk = pair / (p.hq * p.B), bx = pair % (p.hq * p.B);
  if (qblk >= p.nqb) return;
  attn_combine_item<D, false>(p, qblk, bx / p.B, bx % p.B, dv);
}

// ------------------------------------------------------------------ f32 reference-style path
struct AttnF32P {
  const float* q;
  const float* k;
  const float* v;
  float* out;
  int hq, hkv, B, cap, D;
  float scale;
  const int32_t* len_dev;
  int len_host;
  const int32_t* cont_dev;
};

// one workgroup (64 threads) per (head, query); two passes over the keys
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnF32P p) {
  if (p.cont_dev && *p.cont_dev == 0) return;
  const int L = p.len_dev ? *p.len_dev : p.len_host;
  const int N = min(L + p.B, p.cap);
  const int head = blockIdx.x / p.B, qi = blockIdx.x % p.B;
  const int g = head / (p.hq / p.hkv);
  const float* q = p.q + ((size_t)qi * p.hq + head) * p.D;
  const float* kb = p.k + (size_t)g * p.cap * p.D;
  const float* vb = p.v + (size_t)g * p.D * p.cap;   // this head's blocked V^T
  const int lane = threadIdx.x;
  float mx = -INFINITY;
  for (int j = lane; j < N; j += 64) {
    float s = 0.f;
    for (int t = 0; t < p.D; ++t) s = fmaf(q[t], kb[(size_t)j * p.D + t], s);
    mx = fmaxf(mx, s * p.scale);
  }
  mx = wave_max(mx);
  float den = 0.f;
  float acc[128];
  for (int t = 0; t < p.D; ++t) acc[t] = 0.f;
  for (int j = lane; j < N; j += 64) {
    float s = 0.f;
    for (int t = 0; t < p.D; ++t) s = fmaf(q[t], kb[(size_t)j * p.D + t], s);
    const float e = expf(s * p.scale - mx);
    den += e;
    for (int t = 0; t < p.D; ++t) acc[t] = fmaf(e, vb[vt_index(0, p.D, p.cap, j, t)], acc[t]);
  }
  den = wave_sum(den);
  for (int t = 0; t < p.D; ++t) {
    const float num = wave_sum(acc[t]);
    if (lane == 0) p.out[((size_t)qi * p.hq + head) * p.D + t] = num / den;
  }
}

}  // namespace

AttnPlan attn_plan(int hq, int hkv, int D, int B, int max_len) {
  (void)hq; (void)hkv; (void)D;
  AttnPlan pl;
  // the launch covers up to kMaxSplits splits of at least one pass; the kernels choose the
  // split length from the prefix length they read at run time
  const int N = max_len + B;
  pl.chunk = PT * TK;
  pl.nsplit_max = std::min(kMaxSplits, std::max(1, (N + PT * TK - 1) / (PT * TK)));
  return pl;
}

static int attn_wpg(int hq, int hkv) {
  const int G = hq / hkv;
  return G < 4 ? G : 4;
}

bool attn_xcd_combine_ok(int hq, int hkv, int B, int nqb) {
  const int wpg = attn_wpg(hq, hkv);
  return nqb == 1 && B == 32 && hkv * ((hq / hkv) / wpg) == kXcds;
}

size_t attn_ws_bytes(int hq, int hkv, int D, AttnPlan pl, int nqb) {
  const int G = hq / hkv;
  const size_t po = (size_t)nqb * hkv * pl.nsplit_max * G * 32 * D * 2;
  const size_t pm = (size_t)nqb * hkv * pl.nsplit_max * G * 32 * 2 * 4;
  return align_up(po, 256) + align_up(pm, 256);
}

int attn_bf16(const void* q, const void* k, const void* v, void* out, int hq, int hkv, int D,
              int B, int nqb, int cap, float scale, const int32_t* len_dev, int len_host,
              const int32_t* cont_dev, AttnPlan pl, void* ws, int out_packed, hipStream_t st, AttnKv kvf,
              AttnXSync xs) {
  if (nqb < 1 || nqb > 8 || (nqb > 1 && B != 32))
    return fail(DLM_ERR_SHAPE, "attention: one query block, or up to eight of 32 rows");
  AttnP p;
  p.out_packed = out_packed;
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.out = (uint16_t*)out;
  const int G = hq / hkv;
  const size_t po = (size_t)nqb * hkv * pl.nsplit_max * G * 32 * D * 2;
  p.part_o = (uint16_t*)ws;
  p.part_ml = (float*)((char*)ws + align_up(po, 256));
  p.hq = hq;
  p.hkv = hkv;
  p.B = B;
  p.nqb = nqb;
  p.cap = cap;
  p.chunk = pl.chunk;
  p.nsplit_max = pl.nsplit_max;
  p.scale_log2 = scale * (kvf.fp8 ? kvf.k_scale : 1.f) * 1.4426950408889634f;
  p.v_scale = kvf.fp8 ? kvf.v_scale : 1.f;
  p.len_dev = len_dev;
  p.len_host = len_host;
  p.cont_dev = cont_dev;
  const int WPG = attn_wpg(hq, hkv);
  if (G % WPG || (WPG != 1 && WPG != 2 && WPG != 4))
    return fail(DLM_ERR_SHAPE, "attention: query heads per kv head must be 1, 2 or a multiple of 4");
  if (pl.nsplit_max > kMaxSplits) return fail(DLM_ERR_SHAPE, "attention: more key splits than planned for");
  if (xs.bar && xs.err && attn_xcd_combine_ok(hq, hkv, B, nqb)) {
    // splits merged in the launch: kXcds groups x kWgPerXcd workgroups (kMaxSplits == kWgPerXcd)
    static_assert(kMaxSplits == kWgPerXcd, "one workgroup per split slot of a group");
    auto launch = [&](auto kern) {
      hipLaunchKernelGGL(kern, dim3(kXcds * kWgPerXcd), dim3(64 * WPG), 0, st, p, xs);
    };
#define DLM_ATTN_XCD(DD, KV)                                  \
  if (WPG == 4) launch(attn_bf16_xcd_kernel<DD, 4, KV>);      \
  else if (WPG == 2) launch(attn_bf16_xcd_kernel<DD, 2, KV>); \
  else launch(attn_bf16_xcd_kernel<DD, 1, KV>);
    if (D == 128) {
      if (kvf.fp8) { DLM_ATTN_XCD(128, true) } else { DLM_ATTN_XCD(128, false) }
    } else {
      if (kvf.fp8) { DLM_ATTN_XCD(64, true) } else { DLM_ATTN_XCD(64, false) }
    }
#undef DLM_ATTN_XCD
    return check_hip(hipGetLastError(), "attn_bf16 launch");
  }
  const int grid = nqb * hkv * (G / WPG) * pl.nsplit_max;
  auto launch = [&](auto kern, int threads) { hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), 0, st, p); };
  if (D == 128) {
    if (kvf.fp8) {
      if (WPG == 4) launch(attn_bf16_kernel<128, 4, true>, 256);
      else if (WPG == 2) launch(attn_bf16_kernel<128, 2, true>, 128);
      else launch(attn_bf16_kernel<128, 1, true>, 64);
    } else if (WPG == 4) launch(attn_bf16_kernel<128, 4>, 256);
    else if (WPG == 2) launch(attn_bf16_kernel<128, 2>, 128);
    else launch(attn_bf16_kernel<128, 1>, 64);
    hipLaunchKernelGGL(attn_combine_kernel<128>, dim3((nqb * hq * B + 7) / 8), dim3(256), 0, st, p);
  } else {
    if (kvf.fp8) {
      if (WPG == 4) launch(attn_bf16_kernel<64, 4, true>, 256);
      else if (WPG == 2) launch(attn_bf16_kernel<64, 2, true>, 128);
      else launch(attn_bf16_kernel<64, 1, true>, 64);
    } else if (WPG == 4) launch(attn_bf16_kernel<64, 4>, 256);
    else if (WPG == 2) launch(attn_bf16_kernel<64, 2>, 128);
    else launch(attn_bf16_kernel<64, 1>, 64);
    hipLaunchKernelGGL(attn_combine_kernel<64>, dim3((nqb * hq * B + 15) / 16), dim3(256), 0, st, p);
  }
  return check_hip(hipGetLastError(), "attn_bf16 launch");
}

int attn_f32(const float* q, const float* k, const float* v, float* out, int hq, int hkv, int D,
             int B, int cap, float scale, const int32_t* len_dev, int len_host,
             const int32_t* cont_dev, hipStream_t st) {
  AttnF32P p{q, k, v, out, hq, hkv, B, cap, D, scale, len_dev, len_host, cont_dev};
  hipLaunchKernelGGL(attn_f32_kernel, dim3(hq * B), dim3(64), 0, st, p);
  return check_hip(hipGetLastError(), "attn_f32 launch");
}

}  // namespace dlm

// Fused layer kernels: each sublayer of a dense block-diffusion layer (attention: RMSNorm,
// QKV + RoPE + K/V write, block attention, split combine, attention output; FFN: RMSNorm,
// gate/up + SwiGLU, down) runs as ONE launch of 256 workgroups, synchronised only inside
// each XCD.
//
// The chip's 256 compute units sit in 8 XCDs of 32, each with its own L2, and the workgroups
// of a 256-workgroup launch are dealt to the XCDs round-robin, so workgroups b and b + 8 share
// an XCD (every launch checks this with the XCC_ID hardware register).  The 4B-shaped model has 8 kv heads, so XCD x takes kv head x and everything that
// depends on it alone: the q, k and v rows of that head's group (QKV), the attention of its 4
// query heads over the prefix and the block (32 key splits, one per workgroup), the split
// combine, and the slice of the attention-output projection that contracts over those 4
// heads' columns.  The FFN splits the same way: XCD x owns 1/8 of the FFN columns (gate/up
// rows) and the matching 1/8 of the down projection's contraction.  Between the steps of a
// sublayer only the XCD's own 32 workgroups must agree, so a step boundary is an XCD-local
// barrier (an L2 atomic counter; about 1.3 us) instead of a kernel boundary, and the data a
// step hands to the next (normed rows, q, split partials, o, act) moves through the XCD's L2:
// producers store normally (stores write through to L2) and wait for completion before
// arriving; consumers read with sc1 loads, which bypass the compute unit's L1 and are served
// by the XCD's L2.
//
// Each XCD's projections (attention output, down) leave a partial sum of the full output row;
// the 8 partials are added, in XCD order, by the next sublayer's first step, which every XCD
// does for itself (workgroup w of each XCD completes and normalises row w), so no step ever
// waits on another XCD.  A sublayer is therefore 2 launches per layer where the per-op path
// takes 8, and each launch starts its first weight loads before it reads the residual.
//
// Weights are packed for this mapping at model load: QKV in the row-owned layout with the
// rows of XCD x's head group in workgroup blocks 32 x .. 32 x + 31 (x = blockIdx % 8: the
// workgroups of one such group share an XCD, in whatever order the groups map onto XCDs); the attention-output and
// down matrices as 8 column slices (XCD x's contraction range), each in the row-owned layout
// with d / 32 output rows per workgroup; gate/up in the per-op row-owned layout, whose block
// 32 x + w holds FFN columns [F/8 x + F/256 w, +F/256).
//
// Numerics are those of the per-op path: bf16 storage of the normed rows, q/k/v, o and act,
// fp32 residual and accumulation; only the order in which partial sums are added differs.
#include "layer.h"

#include <string.h>

#include "epilogue.h"
#include "xcd.h"

namespace dlm {

bool layer_fused_ok(int dtype, int n_experts, int d, int hq, int hkv, int D, int F, int block) {
  // d % 512: every wave's share of a d-long contraction is a whole number of ring turns
  return dtype == DLM_BF16 && n_experts == 0 && hkv == 8 && hq == 32 && D == 128 && block == 32 &&
         d % 512 == 0 && d <= 4096 && F % 256 == 0 && 2 * F / 256 <= 128;
}

FusedDims fused_dims(int d, int F, int hq, int hkv, int D) {
  FusedDims f;
  f.d = d;
  f.F = F;
  f.hq = hq;
  f.hkv = hkv;
  f.D = D;
  const int G = hq / hkv;
  f.rq = (G + 2) * D / 32;
  f.ro = d / 32;
  f.ko = G * D;
  f.rg = 2 * F / 256;
  f.kd = F / 8;
  return f;
}

void build_xqkv_row_map(int hq, int hkv, int D, int32_t* out) {
  const int G = hq / hkv, per = (G + 2) * D, Nq = hq * D, Nk = hkv * D;
  for (int p = 0; p < hkv * per; ++p) {
    const int x = p / per, r = p % per;
    auto pair = [&](int within) { return 16 * (within / 32) + (within % 32) / 2 + ((within % 32) % 2) * (D / 2); };
    if (r < G * D) out[p] = (G * x + r / D) * D + pair(r % D);
    else if (r < (G + 1) * D) out[p] = Nq + x * D + pair(r - G * D);
    else out[p] = Nq + Nk + x * D + (r - (G + 1) * D);
  }
}

// Optional per-workgroup phase timestamps for kernel studies (compiled out unless defined).
#ifndef DLM_LAYER_TRACE
#define DLM_LAYER_TRACE(kind, i)
#endif

namespace {

struct LayerP {
  int d, F, hq, hkv, D, mrows;
  FusedDims fd;
  float eps;
  LayerIO io;
  const uint16_t* gain;
  uint16_t* xn;
  // attention sublayer
  const uint16_t* wqkv;
  const uint16_t* wo;
  EpiParams epi;
  AttnP attn;
  int last_kv_only;
  // FFN sublayer
  const uint16_t* wgu;
  const uint16_t* wd;
  uint16_t* act;
  unsigned* bar;
  int* err;
  const int32_t* cont_dev;
};

// ------------------------------------------------------------------ residual + RMSNorm
// A row of the residual: h = base + part[0] + ... + part[7], written to base_out by one XCD
// only (x == row % 8), normalised into XCD x's copy of the packed normed rows (same formula as
// the per-op RMSNorm).  Split into the loads (row_issue) and the rest (row_finish) so that a
// weight prefetch can be issued in between: the row's loads are then ahead of it in the
// wave's in-order memory queue.
constexpr int kRowV = 4;             // d <= 4096: 4 float4 per thread

struct RowIn {
  f32x4_t h[kRowV];
  f32x4_t pv[kRowV][kXcds];
  u32x2_t gb[kRowV];
  int cc[kRowV];
  bool ok[kRowV];
};

__device__ __forceinline__ void row_issue(const LayerP& p, int row, RowIn& ri) {
  const int tid = threadIdx.x, d = p.d;
#pragma unroll
  for (int j = 0; j < kRowV; ++j) {
    const int c = 4 * (tid + 256 * j);
    ri.ok[j] = c < d;
    ri.cc[j] = ri.ok[j] ? c : 0;
    ri.h[j] = *(const f32x4_t*)(p.io.base_in + (size_t)row * d + ri.cc[j]);
  }
#pragma unroll
  for (int j = 0; j < kRowV; ++j) ri.gb[j] = *(const u32x2_t*)(p.gain + ri.cc[j]);
  if (p.io.part_in) {
#pragma unroll
    for (int j = 0; j < kRowV; ++j)
#pragma unroll
      for (int k = 0; k < kXcds; ++k)
        ri.pv[j][k] = *(const f32x4_t*)(p.io.part_in + ((size_t)row * kXcds + k) * d + ri.cc[j]);
  }
}

__device__ __forceinline__ void row_finish(const LayerP& p, int x, int row, RowIn& ri, float* red) {
  const int tid = threadIdx.x, d = p.d;
  if (p.io.part_in) {
#pragma unroll
    for (int j = 0; j < kRowV; ++j)
#pragma unroll
      for (int k = 0; k < kXcds; ++k) ri.h[j] += ri.pv[j][k];
  }
  if (x == (row & 7)) {
#pragma unroll
    for (int j = 0; j < kRowV; ++j)
      if (ri.ok[j]) *(f32x4_t*)(p.io.base_out + (size_t)row * d + ri.cc[j]) = ri.h[j];
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kRowV; ++j)
    if (ri.ok[j])
#pragma unroll
      for (int e = 0; e < 4; ++e) s = fmaf(ri.h[j][e], ri.h[j][e], s);
  s = wave_sum(s);
  if ((tid & 63) == 0) red[tid >> 6] = s;
  __syncthreads();
  const float tot = ((red[0] + red[1]) + red[2]) + red[3];
  __syncthreads();
  const float r = 1.0f / sqrtf(tot / (float)d + p.eps);
  uint16_t* xn = p.xn + (size_t)x * 64 * d;
#pragma unroll
  for (int j = 0; j < kRowV; ++j) {
    if (!ri.ok[j]) continue;
    const float g4[4] = {lo_bf(ri.gb[j][0]), hi_bf(ri.gb[j][0]), lo_bf(ri.gb[j][1]), hi_bf(ri.gb[j][1])};
    uint2 ow;
    ow.x = pack2bf(ri.h[j][0] * r * g4[0], ri.h[j][1] * r * g4[1]);
    ow.y = pack2bf(ri.h[j][2] * r * g4[2], ri.h[j][3] * r * g4[3]);
    *(uint2*)(xn + xpk_index_m(row, ri.cc[j], d)) = ow;
  }
}

// ------------------------------------------------------------------ row-owned GEMM pieces
// A wave's view of one row-owned weight block: R rows (NS sub-tiles of up to 32 rows), KT
// k-steps, each k-step R x 16 contiguous with its sub-tiles in matrix-core operand order.
// The 4 waves of a workgroup take every 4th k-step: wave step i is block k-step v + 4 i.
// Loads past the block read zeros (buffer range), so rings can run past the end.
template <int NS>
struct WBlk {
  __amdgpu_buffer_rsrc_t r;
  uint32_t wo[NS];
  uint32_t sb;
  int KT, v;
  __device__ __forceinline__ void init(const uint16_t* W, int R, int KT_, int v_) {
    sb = (uint32_t)R * 32u;
    KT = KT_;
    v = v_;
    r = make_rsrc(W, sb * (uint32_t)KT);
    const int lane = threadIdx.x & 63, i = lane & 31, h = lane >> 5;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int rows_s = min(32, R - 32 * s);
      wo[s] = i < rows_s ? (uint32_t)(512 * s + (i + rows_s * h) * 8) * 2u : 0x80000000u;
    }
  }
  __device__ __forceinline__ int steps() const { return (KT - v + 3) / 4; }
  __device__ __forceinline__ u32x4_t load(int i, int s) const {
    const int k = v + 4 * i;
    return bload16_nt(r, k < KT ? wo[s] + (uint32_t)k * sb : 0x80000000u);
  }
};

// The activation operand of a GEMM step: packed panels of xkt k-steps (32 rows each), the
// contraction covering k-steps kofs .. kofs + KT; read with L1-bypassing loads (written
// earlier in this kernel by the XCD's workgroups).
struct XOp {
  __amdgpu_buffer_rsrc_t r;
  uint32_t xo, xpanel;
  int KT, v;
  __device__ __forceinline__ void init(const uint16_t* X, int xkt, int kofs, int KT_, int v_, int mb) {
    xpanel = (uint32_t)xkt * 1024u;
    r = make_rsrc(X, (uint32_t)mb * xpanel);
    xo = (uint32_t)(threadIdx.x & 63) * 16u + (uint32_t)kofs * 1024u;
    KT = KT_;
    v = v_;
  }
  __device__ __forceinline__ u32x4_t load(int i, int mb) const {
    const int k = v + 4 * i;
    return ld16_xcd(r, (k < KT ? xo + (uint32_t)k * 1024u : 0x80000000u) + (uint32_t)mb * xpanel);
  }
};

// The 4 waves' accumulators added in LDS (red: [4][NS][MB][16][64]) in wave order; out:
// sums[s][mb][q] for accumulator register 4 v + q of sub-tile s, panel mb (register r of a
// 32 x 32 block holds output row 8 (r / 4) + 4 (lane / 32) + r % 4 of column lane % 32).
template <int NS, int MB>
__device__ __forceinline__ void wave_reduce(const f32x16_t (&acc)[NS][MB], float* red, float (&sums)[NS][MB][4]) {
  const int lane = threadIdx.x & 63;
  const int v = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  float (*rd)[NS][MB][16][64] = (float (*)[NS][MB][16][64])red;
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) rd[v][s][mb][r][lane] = acc[s][mb][r];
  __syncthreads();
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 4 * v + q;
        sums[s][mb][q] = ((rd[0][s][mb][r][lane] + rd[1][s][mb][r][lane]) + rd[2][s][mb][r][lane]) +
                         rd[3][s][mb][r][lane];
      }
  __syncthreads();
}

template <int NS, int MB>
__device__ __forceinline__ void zero_acc(f32x16_t (&acc)[NS][MB]) {
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[s][mb][r] = 0.f;
}

// A projection's partial sums for output features [R w, R w + R) of every row, stored as XCD
// x's slot of the partial buffer, [row][8][d].  sums hold the wave's quarter of the 16
// accumulator registers; they are parked in LDS so that each row's R features are stored as
// one contiguous run.
template <int NS, int MB>
__device__ __forceinline__ void store_partial(const LayerP& p, int x, int w, int R, const float (&sums)[NS][MB][4],
                                             float* stage) {
  const int lane = threadIdx.x & 63, v = threadIdx.x >> 6;
  // stage[m][n]: m < 32 MB rows, n < R features
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 4 * v + q;
        const int n = 32 * s + 8 * (r / 4) + 4 * (lane >> 5) + (r % 4);
        if (n < R) stage[(32 * mb + (lane & 31)) * R + n] = sums[s][mb][q];
      }
  __syncthreads();
  const int total = 32 * MB * R;
  for (int i = threadIdx.x; i < total; i += 256) {
    const int m = i / R, n = i % R;
    p.io.part_out[((size_t)m * kXcds + x) * p.d + (size_t)R * w + n] = stage[i];
  }
  __syncthreads();
}

// LDS: the largest of the attention's double-buffered tiles and the GEMM reduction buffer,
// and more than half of a compute unit's 160 KB, so that each compute unit holds exactly one
// workgroup (the 256 workgroups then fill the 256 compute units)
template <int MB>
constexpr int smem_bytes() {
  constexpr int a = attn_smem_bytes<128, 4>();
  constexpr int g = 4 * 3 * MB * 16 * 64 * 4;
  constexpr int m = a > g ? a : g;
  return m > 96 * 1024 ? m : 96 * 1024;
}

// ------------------------------------------------------------------ attention sublayer
constexpr int kRing = 8;     // weight steps in flight per wave

// Attention of kv head x's query heads (key split w of each query block), the split combine,
// and the slice of the attention-output projection that contracts over those heads' columns,
// left as XCD x's partial of every output row.  q and the K/V cache were written before: earlier
// in the same launch, or by the launch before.  check: verify the group's XCD placement after
// this function's first barrier (set when that barrier is the launch's first).
template <int MB, bool KV8>
__device__ __forceinline__ void attn_out_steps(const LayerP& p, int x, int w, int v, unsigned* bar, float* red,
                                               uint8_t* smem, bool check) {
  const int lane = threadIdx.x & 63;
  const int d = p.d, G = p.hq / p.hkv, D = p.D;
  // The attention output is computed by waves 2 and 3, the split combine by waves 0 and 1.
  // Waves 2 and 3 request all of this workgroup's attention-output weights (features
  // [ro w, +ro) over kv head x's G D columns; kNo steps each) as soon as the first query
  // block's first two key passes are in flight, so the weights stream while the attention
  // computes; only later passes of long prefixes queue behind them.
  constexpr int kNo = 16;           // (G D / 16) / 2 wave steps: G D = 512
  const int Ro = p.fd.ro, Ko = p.fd.ko;
  const int vo = v - 2;             // 0, 1 on the output waves
  WBlk<3> wob;
  wob.init(p.wo + ((size_t)x * d * Ko + (size_t)w * Ro * Ko), Ro, Ko / 16, 0);
  u32x4_t wo_r[kNo][3];
  auto o_step = [&](int i) { return vo + 2 * i; };     // block k-step of output-wave step i
  auto issue_wo = [&] {
    if (v >= 2) {
#pragma unroll
      for (int i = 0; i < kNo; ++i)
#pragma unroll
        for (int s = 0; s < 3; ++s)
          wo_r[i][s] = bload16_nt(wob.r, o_step(i) < Ko / 16 ? wob.wo[s] + (uint32_t)o_step(i) * wob.sb : 0x80000000u);
    }
  };

  // 3. attention: key split w of kv head x, for each query block
  attn_split_body<128, 4, KV8, true>(p.attn, 0, x, 0, w, smem, issue_wo);
  if (MB == 2) attn_split_body<128, 4, KV8, true>(p.attn, 1, x, 0, w, smem);
  DLM_LAYER_TRACE(0, 5);
  xcd_sync(bar, p.err);
  if (check) check_placement(p.err, x);
  DLM_LAYER_TRACE(0, 6);

  // 4. split combine of kv head x's (query block, head, query, 4 columns) items, waves 0 and 1
  if (v < 2) {
    for (int it = w * 128 + (int)threadIdx.x; it < MB * 4 * 32 * 32; it += kWgPerXcd * 128) {
      const int dvg = it & 31, qi = (it >> 5) & 31, hl = (it >> 10) & 3, qb = it >> 12;
      attn_combine_item<128, true>(p.attn, qb, G * x + hl, qi, 4 * dvg);
    }
  }
  DLM_LAYER_TRACE(0, 7);
  xcd_sync(bar, p.err);
  DLM_LAYER_TRACE(0, 8);

  // 5. attention output from the held weights (waves 2 and 3): partial sums over kv head x's
  // columns, the two waves' sums added in LDS
  {
    f32x16_t acc[3][MB];
    zero_acc(acc);
    if (v >= 2) {
      const __amdgpu_buffer_rsrc_t xr = make_rsrc(p.attn.out, (uint32_t)MB * (uint32_t)(p.hq * D / 16) * 1024u);
      const uint32_t xo = (uint32_t)lane * 16u + (uint32_t)(x * Ko / 16) * 1024u;
      const uint32_t xpanel = (uint32_t)(p.hq * D / 16) * 1024u;
      u32x4_t xf[kNo][MB];
#pragma unroll
      for (int i = 0; i < kNo; ++i)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          xf[i][mb] = ld16_xcd(xr, (o_step(i) < Ko / 16 ? xo + (uint32_t)o_step(i) * 1024u : 0x80000000u) + mb * xpanel);
#pragma unroll
      for (int i = 0; i < kNo; ++i)
#pragma unroll
        for (int s = 0; s < 3; ++s)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) acc[s][mb] = mfma32x32x16(wo_r[i][s], xf[i][mb], acc[s][mb]);
    }
    DLM_LAYER_TRACE(0, 9);
    float sums[3][MB][4];
    wave_reduce(acc, red, sums);        // waves 0 and 1 add zeros: same sums, fixed order
    store_partial<3, MB>(p, x, w, Ro, sums, red);
    DLM_LAYER_TRACE(0, 10);
  }
}

template <int MB, bool KV8>
__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void attn_sublayer_kernel(LayerP p) {
  if (p.cont_dev && *p.cont_dev == 0) return;
  __shared__ __attribute__((aligned(16))) uint8_t smem[smem_bytes<MB>()];
  float* red = (float*)smem;
  const int x = blockIdx.x & 7, w = blockIdx.x >> 3;
  const int lane = threadIdx.x & 63;
  const int v = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  publish_placement(p.err, x, w);
  unsigned* bar = p.bar + x * 64;
  const int d = p.d, G = p.hq / p.hkv, D = p.D;
  DLM_LAYER_TRACE(0, 0);

  // 1. complete and normalise row w of the residual (every XCD for itself); the QKV weight
  // ring (rows of kv head x's group) starts right behind the row's loads
  const int Rq = p.fd.rq;
  WBlk<1> wq;
  wq.init(p.wqkv + (size_t)(32 * x + w) * Rq * d, Rq, d / 16, v);
  u32x4_t wf[kRing];
  {
    RowIn ri;
    row_issue(p, w, ri);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kRing; ++u) wf[u] = wq.load(u, 0);
    __builtin_amdgcn_sched_barrier(0);
    row_finish(p, x, w, ri, red);
    if (MB == 2) {
      row_issue(p, w + 32, ri);
      row_finish(p, x, w + 32, ri, red);
    }
  }
  DLM_LAYER_TRACE(0, 1);
  xcd_sync(bar, p.err);
  check_placement(p.err, x);
  DLM_LAYER_TRACE(0, 2);

  // 2. QKV + RoPE + K/V write
  {
    XOp xq;
    xq.init(p.xn + (size_t)x * 64 * d, d / 16, 0, d / 16, v, MB);
    u32x4_t xf[kRing][MB];
#pragma unroll
    for (int u = 0; u < kRing; ++u)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) xf[u][mb] = xq.load(u, mb);
    f32x16_t acc[1][MB];
    zero_acc(acc);
    const int n = wq.steps();
    for (int k0 = 0; k0 < n; k0 += kRing) {
#pragma unroll
      for (int u = 0; u < kRing; ++u) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[0][mb] = mfma32x32x16(wf[u], xf[u][mb], acc[0][mb]);
        wf[u] = wq.load(k0 + u + kRing, 0);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) xf[u][mb] = xq.load(k0 + u + kRing, mb);
      }
    }
    DLM_LAYER_TRACE(0, 3);
    float sums[1][MB][4];
    wave_reduce(acc, red, sums);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = 32 * mb + (lane & 31);
#pragma unroll
      for (int q = 0; q < 4; q += 2) {
        const int r = 4 * v + q;
        const int row = 8 * (r / 4) + 4 * (lane >> 5) + (r % 4);
        if (row >= Rq) continue;
        const int pl = Rq * w + row;          // packed row within the XCD's block, even
        const float a = sums[0][mb][q], b = sums[0][mb][q + 1];
        auto jpair = [&](int within) { return 16 * (within / 32) + (within % 32) / 2; };
        if (pl < G * D) epi_qk_rope(p.epi, m, 0, G * x + pl / D, jpair(pl % D), a, b);
        else if (pl < (G + 1) * D) epi_qk_rope(p.epi, m, 1, x, jpair(pl - G * D), a, b);
        else {
          const int rel = x * D + (pl - (G + 1) * D);
          epi_v(p.epi, m, rel, a);
          epi_v(p.epi, m, rel + 1, b);
        }
      }
    }
  }
  if (p.last_kv_only) return;       // uniform: the commit pass's last layer needs only its K/V

  xcd_sync(bar, p.err);
  DLM_LAYER_TRACE(0, 4);
  attn_out_steps<MB, KV8>(p, x, w, v, bar, red, smem, false);
}

// The attention and its output projection alone, for the per-op path: q and the K/V cache come
// from the QKV launch before, and the 8 XCD partials go to the next RMSNorm, which adds them to
// the residual in XCD order.  One launch in place of two (attention, output projection).
template <int MB, bool KV8>
__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void attn_out_kernel(LayerP p) {
  if (p.cont_dev && *p.cont_dev == 0) return;
  __shared__ __attribute__((aligned(16))) uint8_t smem[smem_bytes<MB>()];
  const int x = blockIdx.x & 7, w = blockIdx.x >> 3;
  const int v = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  publish_placement(p.err, x, w);
  attn_out_steps<MB, KV8>(p, x, w, v, p.bar + x * 64, (float*)smem, smem, true);
}

// ------------------------------------------------------------------ FFN sublayer
// One weight stream per wave through the gate/up block (wave steps [0, n1)) and on into the
// down block (steps n1 ..), so the down projection's first weights are in flight while the
// SwiGLU outputs are exchanged (n1 is a multiple of the ring depth).
template <int MB>
__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void ffn_sublayer_kernel(LayerP p) {
  if (p.cont_dev && *p.cont_dev == 0) return;
  __shared__ __attribute__((aligned(16))) uint8_t smem[smem_bytes<MB>()];
  float* red = (float*)smem;
  const int x = blockIdx.x & 7, w = blockIdx.x >> 3;
  const int lane = threadIdx.x & 63;
  const int v = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  publish_placement(p.err, x, w);
  unsigned* bar = p.bar + x * 64;
  const int d = p.d;
  DLM_LAYER_TRACE(1, 0);

  const int Rg = p.fd.rg, Ro = p.fd.ro, Kd = p.fd.kd;
  WBlk<3> wg, wd;
  wg.init(p.wgu + (size_t)(32 * x + w) * Rg * d, Rg, d / 16, v);
  wd.init(p.wd + ((size_t)x * d * Kd + (size_t)w * Ro * Kd), Ro, Kd / 16, v);
  const int n1 = wg.steps(), n2 = wd.steps();
  auto wl = [&](int i, int s) -> u32x4_t { return i < n1 ? wg.load(i, s) : wd.load(i - n1, s); };
  u32x4_t wf[kRing][3];
  {
    RowIn ri;
    row_issue(p, w, ri);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kRing; ++u)
#pragma unroll
      for (int s = 0; s < 3; ++s) wf[u][s] = wl(u, s);
    __builtin_amdgcn_sched_barrier(0);
    row_finish(p, x, w, ri, red);
    if (MB == 2) {
      row_issue(p, w + 32, ri);
      row_finish(p, x, w + 32, ri, red);
    }
  }
  DLM_LAYER_TRACE(1, 1);
  xcd_sync(bar, p.err);
  check_placement(p.err, x);
  DLM_LAYER_TRACE(1, 2);

  // gate/up + SwiGLU: FFN columns [F/8 x + F/256 w, + F/256) as (gate, up) row pairs
  {
    XOp xg;
    xg.init(p.xn + (size_t)x * 64 * d, d / 16, 0, d / 16, v, MB);
    u32x4_t xf[kRing][MB];
#pragma unroll
    for (int u = 0; u < kRing; ++u)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) xf[u][mb] = xg.load(u, mb);
    f32x16_t acc[3][MB];
    zero_acc(acc);
    for (int k0 = 0; k0 < n1; k0 += kRing) {
#pragma unroll
      for (int u = 0; u < kRing; ++u) {
#pragma unroll
        for (int s = 0; s < 3; ++s)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) acc[s][mb] = mfma32x32x16(wf[u][s], xf[u][mb], acc[s][mb]);
#pragma unroll
        for (int s = 0; s < 3; ++s) wf[u][s] = wl(k0 + u + kRing, s);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) xf[u][mb] = xg.load(k0 + u + kRing, mb);
      }
    }
    DLM_LAYER_TRACE(1, 3);
    float sums[3][MB][4];
    wave_reduce(acc, red, sums);
    const int f0 = (32 * x + w) * (Rg / 2);
#pragma unroll
    for (int s = 0; s < 3; ++s)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int m = 32 * mb + (lane & 31);
#pragma unroll
        for (int q = 0; q < 4; q += 2) {
          const int r = 4 * v + q;
          const int row = 32 * s + 8 * (r / 4) + 4 * (lane >> 5) + (r % 4);
          if (row >= Rg) continue;
          epi_swiglu(p.epi, m, f0 + row / 2, sums[s][mb][q], sums[s][mb][q + 1]);
        }
      }
  }
  DLM_LAYER_TRACE(1, 4);
  // the down weights' next kRing wave steps go out while the XCD meets: with the ring's kRing
  // the down projection then has 2 kRing steps in flight
  u32x4_t wf2[kRing][3];
  xcd_sync(bar, p.err, [&] {
#pragma unroll
    for (int u = 0; u < kRing; ++u)
#pragma unroll
      for (int s = 0; s < 3; ++s) wf2[u][s] = wl(n1 + kRing + u, s);
  });
  DLM_LAYER_TRACE(1, 5);

  // down: features [ro w, +ro) over XCD x's F/8 columns of act (weight steps n1 .. of the
  // stream: wf holds steps n1 .. n1 + kRing - 1, wf2 the next kRing)
  {
    XOp xd;
    xd.init(p.act, p.F / 16, x * Kd / 16, Kd / 16, v, MB);
    u32x4_t xf[2 * kRing][MB];
#pragma unroll
    for (int u = 0; u < 2 * kRing; ++u)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) xf[u][mb] = xd.load(u, mb);
    f32x16_t acc[3][MB];
    zero_acc(acc);
    for (int k0 = 0; k0 < n2; k0 += 2 * kRing) {
#pragma unroll
      for (int u = 0; u < kRing; ++u) {
#pragma unroll
        for (int s = 0; s < 3; ++s)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) acc[s][mb] = mfma32x32x16(wf[u][s], xf[u][mb], acc[s][mb]);
#pragma unroll
        for (int s = 0; s < 3; ++s) wf[u][s] = wl(n1 + k0 + u + 2 * kRing, s);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) xf[u][mb] = xd.load(k0 + u + 2 * kRing, mb);
      }
#pragma unroll
      for (int u = 0; u < kRing; ++u) {
#pragma unroll
        for (int s = 0; s < 3; ++s)
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) acc[s][mb] = mfma32x32x16(wf2[u][s], xf[kRing + u][mb], acc[s][mb]);
#pragma unroll
        for (int s = 0; s < 3; ++s) wf2[u][s] = wl(n1 + k0 + kRing + u + 2 * kRing, s);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) xf[kRing + u][mb] = xd.load(k0 + kRing + u + 2 * kRing, mb);
      }
    }
    DLM_LAYER_TRACE(1, 6);
    float sums[3][MB][4];
    wave_reduce(acc, red, sums);
    store_partial<3, MB>(p, x, w, Ro, sums, red);
    DLM_LAYER_TRACE(1, 7);
  }
}

LayerP base_params(const FusedDims& fd, int mb, const void* gain, float eps, const LayerIO& io, const LayerBufs& b,
                   const int32_t* cont_dev) {
  LayerP p;
  memset(&p, 0, sizeof(p));
  p.d = fd.d;
  p.F = fd.F;
  p.hq = fd.hq;
  p.hkv = fd.hkv;
  p.D = fd.D;
  p.mrows = 32 * mb;
  p.fd = fd;
  p.eps = eps;
  p.io = io;
  p.gain = (const uint16_t*)gain;
  p.xn = b.xn;
  p.act = b.act;
  p.bar = b.bar;
  p.err = b.err;
  p.cont_dev = cont_dev;
  return p;
}

}  // namespace

int fused_attn_sublayer(const FusedDims& fd, int mb, const uint16_t* wqkv, const uint16_t* wo_slices,
                        const void* gain, float eps, const LayerIO& io, const LayerBufs& b, const EpiParams& qkv_epi,
                        AttnPlan plan, float softmax_scale, AttnKv kvf, int last_kv_only, const int32_t* cont_dev,
                        hipStream_t st) {
  if (mb != 1 && mb != 2) return fail(DLM_ERR_SHAPE, "fused layer: 32 or 64 rows");
  if (plan.nsplit_max > kWgPerXcd) return fail(DLM_ERR_SHAPE, "fused layer: more key splits than workgroups");
  LayerP p = base_params(fd, mb, gain, eps, io, b, cont_dev);
  p.wqkv = wqkv;
  p.wo = wo_slices;
  p.epi = qkv_epi;
  p.epi.q_out = b.q;
  p.epi.bf16_out = 1;
  p.last_kv_only = last_kv_only;
  AttnP& a = p.attn;
  a.q = b.q;
  a.k = (const uint16_t*)qkv_epi.k_cache;
  a.v = (const uint16_t*)qkv_epi.v_cache;
  a.out = b.o;
  const int G = fd.hq / fd.hkv;
  const size_t po = (size_t)mb * fd.hkv * plan.nsplit_max * G * 32 * fd.D * 2;
  a.part_o = (uint16_t*)b.attn_ws;
  a.part_ml = (float*)((char*)b.attn_ws + align_up(po, 256));
  a.hq = fd.hq;
  a.hkv = fd.hkv;
  a.B = 32;
  a.nqb = mb;
  a.cap = qkv_epi.cap;
  a.chunk = plan.chunk;
  a.nsplit_max = plan.nsplit_max;
  a.out_packed = 1;
  a.scale_log2 = softmax_scale * (kvf.fp8 ? kvf.k_scale : 1.f) * 1.4426950408889634f;
  a.v_scale = kvf.fp8 ? kvf.v_scale : 1.f;
  a.len_dev = qkv_epi.len_dev;
  a.len_host = qkv_epi.len_host;
  a.cont_dev = nullptr;
  auto launch = [&](auto kern) { hipLaunchKernelGGL(kern, dim3(256), dim3(256), 0, st, p); };
  if (mb == 1) {
    if (kvf.fp8) launch(attn_sublayer_kernel<1, true>);
    else launch(attn_sublayer_kernel<1, false>);
  } else {
    if (kvf.fp8) launch(attn_sublayer_kernel<2, true>);
    else launch(attn_sublayer_kernel<2, false>);
  }
  return check_hip(hipGetLastError(), "fused attention sublayer launch");
}

int attn_out_xcd(const FusedDims& fd, int mb, const uint16_t* wo_slices, const uint16_t* q, const void* k_cache,
                 const void* v_cache, uint16_t* o_packed, void* attn_ws, float* part_out, unsigned* bar, int* err,
                 int cap, const int32_t* len_dev, AttnPlan plan, float softmax_scale, AttnKv kvf,
                 const int32_t* cont_dev, hipStream_t st) {
  if (mb != 1 && mb != 2) return fail(DLM_ERR_SHAPE, "attention with output: 32 or 64 rows");
  if (plan.nsplit_max > kWgPerXcd) return fail(DLM_ERR_SHAPE, "attention with output: more key splits than workgroups");
  LayerIO io{};
  io.part_out = part_out;
  LayerBufs b{};
  b.bar = bar;
  b.err = err;
  LayerP p = base_params(fd, mb, nullptr, 0.f, io, b, cont_dev);
  p.wo = wo_slices;
  AttnP& a = p.attn;
  a.q = q;
  a.k = (const uint16_t*)k_cache;
  a.v = (const uint16_t*)v_cache;
  a.out = o_packed;
  const int G = fd.hq / fd.hkv;
  const size_t po = (size_t)mb * fd.hkv * plan.nsplit_max * G * 32 * fd.D * 2;
  a.part_o = (uint16_t*)attn_ws;
  a.part_ml = (float*)((char*)attn_ws + align_up(po, 256));
  a.hq = fd.hq;
  a.hkv = fd.hkv;
  a.B = 32;
  a.nqb = mb;
  a.cap = cap;
  a.chunk = plan.chunk;
  a.nsplit_max = plan.nsplit_max;
  a.out_packed = 1;
  a.scale_log2 = softmax_scale * (kvf.fp8 ? kvf.k_scale : 1.f) * 1.4426950408889634f;
  a.v_scale = kvf.fp8 ? kvf.v_scale : 1.f;
  a.len_dev = len_dev;
  a.len_host = 0;
  a.cont_dev = nullptr;
  auto launch = [&](auto kern) { hipLaunchKernelGGL(kern, dim3(256), dim3(256), 0, st, p); };
  if (mb == 1) {
    if (kvf.fp8) launch(attn_out_kernel<1, true>);
    else launch(attn_out_kernel<1, false>);
  } else {
    if (kvf.fp8) launch(attn_out_kernel<2, true>);
    else launch(attn_out_kernel<2, false>);
  }
  return check_hip(hipGetLastError(), "attention with output launch");
}

int fused_ffn_sublayer(const FusedDims& fd, int mb, const uint16_t* wgu, const uint16_t* wd_slices, const void* gain,
                       float eps, const LayerIO& io, const LayerBufs& b, const int32_t* cont_dev, hipStream_t st) {
  if (mb != 1 && mb != 2) return fail(DLM_ERR_SHAPE, "fused layer: 32 or 64 rows");
  LayerP p = base_params(fd, mb, gain, eps, io, b, cont_dev);
  p.wgu = wgu;
  p.wd = wd_slices;
  p.epi.act_out = b.act;
  p.epi.F = fd.F;
  p.epi.bf16_out = 1;
  if (mb == 1) hipLaunchKernelGGL(ffn_sublayer_kernel<1>, dim3(256), dim3(256), 0, st, p);
  else hipLaunchKernelGGL(ffn_sublayer_kernel<2>, dim3(256), dim3(256), 0, st, p);
  return check_hip(hipGetLastError(), "fused FFN sublayer launch");
}

}  // namespace dlm

// Routed-expert FFN of the MoE model (the FFN of every layer of the MoE configuration).
//
// Steps, per layer and round (all rows of the block):
//   1. router logits r = f W_r^T (bf16 stream-K GEMM, f32 out);
//   2. route: softmax over the E routed experts in f32, top-k by (probability desc, expert id
//      asc), the selected probabilities are the mixing weights (not renormalised); shared
//      experts take every row with weight 1.  The same launch quantises f to MXFP8 (e4m3
//      codes, one e8m0 scale per 32 along d);
//   3. up: per hit expert and 64 interleaved gate/up rows, act = silu(gate) * up over its rows
//      with v_mfma_scale_f32_16x16x128_f8f6f4 (A = MXFP4 weights, B = MXFP8 activations), the
//      32 act values of a row quantised to MXFP8 in the epilogue;
//   4. down: per hit expert and 64 output columns, y = act W_d^T, scaled by the row's mixing
//      weight and stored to the row's slot; the next RMSNorm adds the slots in order.
// The expert kernels read the whole top-k table: it gives each workgroup its expert's rows,
// in row order, and, in the up kernel, the expert itself (the experts hit, in id order, take
// the lowest workgroup slots after the shared ones); the up kernel leaves that list for the
// down kernel.
// Pages: [ORL-blog] "What shipped" runs routed experts in 4-bit floating point on the
// matrix units; the MI355X form uses the OCP microscaling formats (MXFP4 weights, MXFP8
// activations), which the scaled matrix-core instruction consumes directly.
//
// Packed expert matrix of R rows x K columns (R % 64 == 0, K % 128 == 0): for quad q (64 rows),
// step s (128 columns), row group gq (16 rows) and lane l, the 16 bytes at
// ((q S + s) 4 + gq) 1024 + 16 l hold the e2m1 codes (low nibble first) of row 64q + 16gq + l%16,
// columns 128s + 32(l/16) .. +32, and byte ((q S + s) 4 + gq) 64 + l of the scale array holds that
// 32-column block's e8m0.  That is the A-operand order of the scaled MFMA, so a wave loads one
// contiguous 1 KiB (+ 64 B of scales) per row group and step.  Gate/up rows are interleaved
// (packed row 2i = gate i, 2i + 1 = up i) so one lane holds both halves of a SwiGLU pair.
#include "moe.h"

#include <cstring>

namespace dlm {

MoeDims moe_dims(const dlm_model_desc& d) {
  MoeDims m;
  m.d = d.d;
  m.F = d.expert_ffn;
  m.E = d.n_experts;
  m.S = d.n_shared;
  m.top_k = d.top_k;
  m.NS = d.top_k + d.n_shared;
  m.rows = d.block;
  return m;
}

size_t moe_layer_packed_bytes(const MoeDims& m) { return (size_t)(m.E + m.S) * m.expert_bytes(); }

namespace {

constexpr int kMaxRows = 64;       // a round fused with the previous block's commit pass
constexpr int kMaxExperts = 512;
constexpr int kMaxLayers = 256;

// -------------------------------------------------------------------- MX number formats
// Shared exponent of a block for an element format whose largest exponent is emax:
// floor(log2(amax)) - emax, -127 for an all-zero block (OCP MX v1.0).
__device__ inline int mx_shared_exp(float amax, int emax) {
  if (!(amax > 0.f)) return -127;
  int ex;
  frexpf(amax, &ex);                     // amax = m 2^ex, m in [0.5, 1)
  return max(-127, min(127, ex - 1 - emax));
}

// SA: the byte of sa that holds the A scale (four row groups share one scale word)
template <int SA = 0>
__device__ inline f32x4_t mfma_mx(u32x4_t a_fp4, u32x4_t b_lo, u32x4_t b_hi, int sa, int sb, f32x4_t c) {
  typedef int v8i_t __attribute__((ext_vector_type(8)));
  v8i_t a, b;
  a[0] = (int)a_fp4[0]; a[1] = (int)a_fp4[1]; a[2] = (int)a_fp4[2]; a[3] = (int)a_fp4[3];
  a[4] = 0; a[5] = 0; a[6] = 0; a[7] = 0;
  b[0] = (int)b_lo[0]; b[1] = (int)b_lo[1]; b[2] = (int)b_lo[2]; b[3] = (int)b_lo[3];
  b[4] = (int)b_hi[0]; b[5] = (int)b_hi[1]; b[6] = (int)b_hi[2]; b[7] = (int)b_hi[3];
  // A format 4 = e2m1 (lane l: row l%16, columns 32(l/16) .. +32), B format 0 = e4m3 (lane l:
  // column l%16, rows 16(l/16) .. +16 then 64 + 16(l/16) .. +16); scales: lane 16b + i holds the
  // e8m0 of row / column i, 32-element block b, in byte SA of sa and byte 0 of sb.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 0, SA, sa, 0, sb);
}

__device__ inline uint32_t bload_u8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, 0);
}

// -------------------------------------------------------------------- packing
struct MxPackP {
  const uint8_t* src;         // [n_mats][R][K/2] codes, natural
  const uint8_t* src_scale;   // [n_mats][R][K/32]
  uint8_t* dst;
  uint8_t* dst_scale;
  int R, K, interleave;
  long long chunks;           // n_mats * R * K / 32
};

__global__ __launch_bounds__(256) void mx_pack_kernel(MxPackP p) {
  const long long c = (long long)blockIdx.x * 256 + threadIdx.x;
  if (c >= p.chunks) return;
  const long long per_mat = (long long)p.R * p.K / 32;
  const int mat = (int)(c / per_mat);
  int r = (int)(c % per_mat);
  const int lane = r % 64;
  int u = r / 64;
  const int gq = u % 4;
  u /= 4;
  const int S = p.K / 128;
  const int s = u % S, q = u / S;
  const int prow = 64 * q + 16 * gq + (lane & 15);
  const int srow = p.interleave ? ((prow & 1) ? p.R / 2 : 0) + prow / 2 : prow;
  const int k0 = 128 * s + 32 * (lane >> 4);
  const size_t so = (size_t)mat * p.R * (p.K / 2) + (size_t)srow * (p.K / 2) + k0 / 2;
  *(u32x4_t*)(p.dst + (size_t)c * 16) = *(const u32x4_t*)(p.src + so);
  // the four row groups' scales of one (quad, step, lane) share a 4-byte word, so that one
  // load per step brings them
  p.dst_scale[((c >> 8) * 64 + lane) * 4 + gq] = p.src_scale[(size_t)mat * p.R * (p.K / 32) + (size_t)srow * (p.K / 32) + k0 / 32];
}

// -------------------------------------------------------------------- route + quantise
struct Route {
  int* ids;        // [rows][top_k] expert of each rank, by (probability desc, id asc)
  float* wts;      // [rows][top_k] its probability (the mixing weight)
  int* hits;       // [n_layers] running count of distinct experts per layer (statistics)
  int* n_hit;      // number of distinct routed experts some row selected ...
  int* list;       // ... and their ids, ascending (256 entries); both written by the up kernel
};

struct RouteP {
  MoeDims m;
  const float* logits;     // [rows][E]
  const uint16_t* f;       // bf16 packed activations, rows x d in 32-row panels
  uint8_t* xq;             // [rows][d] e4m3 codes
  uint8_t* xs;             // [rows][d/32] e8m0
  Route ro;
  const int32_t* cont_dev;
};

// One workgroup per row of the block: the row's MXFP8 input, then its softmax over the E
// routed experts and the top-k by rank (rank of e = number of experts with a larger
// probability, or an equal one and a lower id), so no serial selection loop runs.
__global__ __launch_bounds__(256) void moe_route_kernel(RouteP p) {
  if (p.cont_dev && *p.cont_dev == 0) return;
  const MoeDims& m = p.m;
  const int row = blockIdx.x, tid = threadIdx.x;
  __shared__ __align__(16) unsigned long long s_key[256];
  __shared__ float red[4];
  const bool has = tid < m.E;
  const float r = has ? p.logits[(size_t)row * m.E + tid] : -INFINITY;   // issued before the MX work
  // MXFP8 of the row: four threads per 32-element block, 8 elements (one 16-byte packed run)
  // each; the block maximum is taken over the four lanes
  for (int b = tid >> 2; b < m.d / 32; b += 64) {
    const int j = tid & 3;
    const u32x4_t w = *(const u32x4_t*)(p.f + xpk_index_m(row, 32 * b + 8 * j, m.d));
    float v[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = lo_bf(w[e]);
      v[2 * e + 1] = hi_bf(w[e]);
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    const int e = mx_shared_exp(amax, 8);
    const float inv = ldexpf(1.f, -e);
    uint32_t words[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
      words[i] = e4m3_code(v[4 * i] * inv) | (e4m3_code(v[4 * i + 1] * inv) << 8) |
                 (e4m3_code(v[4 * i + 2] * inv) << 16) | (e4m3_code(v[4 * i + 3] * inv) << 24);
    *(u32x2_t*)(p.xq + (size_t)row * m.d + 32 * b + 8 * j) = u32x2_t{words[0], words[1]};
    if (j == 0) p.xs[(size_t)row * (m.d / 32) + b] = (uint8_t)(e + 127);
  }
  // softmax over the routed experts (thread t holds expert t; E <= 256)
  float mx = wave_max(r);
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  const float ex = has ? expf(r - mx) : 0.f;
  float sum = wave_sum(ex);
  if ((tid & 63) == 0) red[tid >> 6] = sum;
  __syncthreads();
  sum = ((red[0] + red[1]) + red[2]) + red[3];
  const float pr = ex / sum;
  // rank of expert tid = number of experts with a larger key, where the key is the
  // probability's bits (non-negative floats order as unsigned integers; not-a-number ranks
  // lowest) above 255 - id: key order is (probability desc, id asc), keys are distinct, so the
  // ranks are a permutation and one unsigned compare per expert decides
  const uint32_t pbits = pr >= 0.f ? __float_as_uint(pr) : 0u;
  const unsigned long long key = ((unsigned long long)pbits << 8) | (unsigned long long)(255 - tid);
  s_key[tid] = has ? key : 0ull;
  __syncthreads();
  if (has) {
    int rank = 0;
#pragma unroll 8
    for (int e = 0; e < m.E; ++e) rank += s_key[e] > key ? 1 : 0;
    if (rank < m.top_k) {
      p.ro.ids[row * m.top_k + rank] = tid;
      p.ro.wts[row * m.top_k + rank] = pr;
    }
  }
}

// -------------------------------------------------------------------- expert projections
struct ExpP {
  MoeDims m;
  int layer;
  const uint8_t* w;        // packed codes of this layer's matrix of expert 0
  const uint8_t* ws;       // packed scales of expert 0
  size_t w_stride, s_stride;   // bytes per expert
  int Q, S;                // quads (64 rows) and 128-column steps of the matrix
  const uint8_t* bq;       // B operand codes: [rows or slots][K]
  const uint8_t* bs;       // B operand scales: [rows or slots][K/32]
  int b_by_slot;           // B rows are indexed by slot (down) or by row (up)
  Route ro;
  uint8_t* aq;             // up: act codes [rows NS][F]
  uint8_t* as;             // up: act scales [rows NS][F/32]
  float* y;                // down: [rows NS][d]
  const int32_t* cont_dev;
};

// One single-wave workgroup per (expert, quad).  The wave first finds the block's rows routed
// to the expert (row order, from the top-k table; every row for a shared expert); a workgroup
// whose expert no row chose exits before touching its weights.  It then runs 4 row groups x up
// to 2 groups of 16 rows, K in steps of 128, PF weight steps in flight.
// PF: steps of 128 columns in flight per wave
template <int UP, int PF>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void moe_expert_kernel(ExpP p) {
  if (p.cont_dev && *p.cont_dev == 0) return;
  const MoeDims& m = p.m;
  // workgroup slots: the shared experts first, then the routed experts some row selected, in
  // id order.  The up kernel finds a slot's expert from the routing table (slots past the
  // experts hit exit once they have read it) and its first quad's workgroups write the list of
  // experts hit and their count for the down kernel, whose spare slots exit after one load.
  // a shared expert takes one slot per 32 rows of the block (two for a 64-row fused pass), so
  // that no shared-expert workgroup makes two passes over its weights
  const int per = (m.rows + 31) / 32, SV = per * m.S;
  const int slot_e = blockIdx.x / p.Q, q = blockIdx.x % p.Q;
  if (!UP && slot_e >= SV && slot_e - SV >= *p.ro.n_hit) return;
  const int lane = threadIdx.x;
  __shared__ int s_n;
  __shared__ int s_row[kMaxRows], s_slot[kMaxRows];
  __shared__ float s_w[kMaxRows];
  __shared__ uint32_t s_hb[8];
  int e;
  {
    int n = 0;
    if (slot_e < SV) {
      e = m.E + slot_e / per;
      const int r0 = 32 * (slot_e % per);
      if (lane < 32 && r0 + lane < m.rows) {
        s_row[lane] = r0 + lane;
        s_slot[lane] = (r0 + lane) * m.NS + m.top_k + (e - m.E);
        s_w[lane] = 1.f;
      }
      n = max(0, min(32, m.rows - r0));
    } else {
      // the (row, rank) table, <= 512 entries row-major: every id and weight is loaded at once
      // (entries past the table read zeros and are masked by the index test)
      constexpr int TC = kMaxRows * 8 / 64;      // 64-entry chunks of the largest table
      const int total = m.rows * m.top_k;
      const __amdgpu_buffer_rsrc_t ir = make_rsrc(p.ro.ids, (uint32_t)total * 4u);
      const __amdgpu_buffer_rsrc_t wtr = make_rsrc(p.ro.wts, (uint32_t)total * 4u);
      int idv[TC];
      float wv[TC];
#pragma unroll
      for (int c = 0; c < TC; ++c) {
        idv[c] = __builtin_amdgcn_raw_buffer_load_b32(ir, (64 * c + lane) * 4, 0, 0);
        wv[c] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(wtr, (64 * c + lane) * 4, 0, 0));
      }
      if (UP) {
        // this slot's expert: the (slot_e - SV)-th of the experts hit, in id order, from a
        // bitmap of the table (routed ids are < E <= 256)
        if (lane < 8) s_hb[lane] = 0u;
        __syncthreads();
#pragma unroll
        for (int c = 0; c < TC; ++c)
          if (64 * c + lane < total) atomicOr(&s_hb[idv[c] >> 5], 1u << (idv[c] & 31));
        __syncthreads();
        int j = slot_e - SV, word = -1, n_hit = 0;
        uint32_t bits = 0u;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t x = s_hb[i];
          const int c = __popc(x);
          if (word < 0) {
            if (j < c) { word = i; bits = x; }
            else j -= c;
          }
          n_hit += c;
        }
        if (word < 0) return;             // fewer experts hit than this slot (uniform)
        for (int t = 0; t < j; ++t) bits &= bits - 1u;
        e = 32 * word + __builtin_ctz(bits);
        if (q == 0 && lane == 0) {
          p.ro.list[slot_e - SV] = e;
          if (slot_e - SV == n_hit - 1) *p.ro.n_hit = n_hit;
        }
      } else {
        e = p.ro.list[slot_e - SV];
      }
#pragma unroll
      for (int c = 0; c < TC; ++c) {
        const int idx = 64 * c + lane;
        const bool hit = idx < total && idv[c] == e;
        const unsigned long long mask = __ballot(hit);
        if (hit) {
          const int pos = n + __popcll(mask & ((1ull << lane) - 1));
          const int i = idx / m.top_k;
          s_row[pos] = i;
          s_slot[pos] = i * m.NS + idx % m.top_k;
          s_w[pos] = wv[c];
        }
        n += __popcll(mask);
      }
    }
    if (lane == 0) {
      s_n = n;
      if (UP && q == 0 && n > 0 && (slot_e >= SV || slot_e % per == 0)) atomicAdd(&p.ro.hits[p.layer], 1);
    }
  }
  __syncthreads();
  const int n = s_n;
  if (n == 0) return;
  const int K = 128 * p.S;
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(p.w + e * p.w_stride + (size_t)q * p.S * 4096, (uint32_t)p.S * 4096u);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(p.ws + e * p.s_stride + (size_t)q * p.S * 256, (uint32_t)p.S * 256u);
  const int n_brows = p.b_by_slot ? m.rows * m.NS : m.rows;
  const __amdgpu_buffer_rsrc_t br = make_rsrc(p.bq, (uint32_t)(n_brows * K));
  const __amdgpu_buffer_rsrc_t bsr = make_rsrc(p.bs, (uint32_t)(n_brows * (K / 32)));
  // up to 32 of the expert's rows per pass over the weights (two column groups of 16); a routed
  // expert with more rows (only in a 64-row fused pass) makes a second pass, from L2
  for (int r0 = 0; r0 < n; r0 += 32) {
    const bool two = n - r0 > 16;
    int col[2], brow[2], slot[2];
#pragma unroll
    for (int cg = 0; cg < 2; ++cg) {
      col[cg] = r0 + 16 * cg + (lane & 15);
      brow[cg] = -1;
      slot[cg] = -1;
      if (col[cg] < n) {
        slot[cg] = s_slot[col[cg]];
        brow[cg] = p.b_by_slot ? slot[cg] : s_row[col[cg]];
      }
    }
    uint32_t bo[2], bso[2];
#pragma unroll
    for (int cg = 0; cg < 2; ++cg) {
      bo[cg] = brow[cg] >= 0 ? (uint32_t)(brow[cg] * K + 16 * (lane >> 4)) : 0x80000000u;
      bso[cg] = brow[cg] >= 0 ? (uint32_t)(brow[cg] * (K / 32) + (lane >> 4)) : 0x80000000u;
    }
    f32x4_t acc[2][4];
#pragma unroll
    for (int cg = 0; cg < 2; ++cg)
#pragma unroll
      for (int g = 0; g < 4; ++g) acc[cg][g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // ring of PF steps: weights (4 row groups) and the block rows' activations (2 column groups)
    u32x4_t wa[PF][4], blo[PF][2], bhi[PF][2];
    uint32_t wsc[PF], bsc[PF][2];
    auto fetch = [&](int u, int s) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        wa[u][g] = bload16_nt(wr, (uint32_t)((s * 4 + g) * 64 + lane) * 16u);
      }
      wsc[u] = __builtin_amdgcn_raw_buffer_load_b32(sr, (int)(s * 64 + lane) * 4, 0, 0);
#pragma unroll
      for (int cg = 0; cg < 2; ++cg) {
        if (cg == 1 && !two) break;
        const uint32_t off = s < p.S ? bo[cg] + 128u * s : 0x80000000u;
        blo[u][cg] = bload16(br, off);
        bhi[u][cg] = bload16(br, off + 64u);
        bsc[u][cg] = bload_u8(bsr, s < p.S ? bso[cg] + 4u * s : 0x80000000u);
      }
    };
#pragma unroll
    for (int u = 0; u < PF; ++u) fetch(u, u);
    for (int s0 = 0; s0 < p.S; s0 += PF) {
#pragma unroll
      for (int u = 0; u < PF; ++u) {
        const int s = s0 + u;
        if (s < p.S) {
#pragma unroll
          for (int cg = 0; cg < 2; ++cg) {
            if (cg == 1 && !two) break;
            acc[cg][0] = mfma_mx<0>(wa[u][0], blo[u][cg], bhi[u][cg], (int)wsc[u], (int)bsc[u][cg], acc[cg][0]);
            acc[cg][1] = mfma_mx<1>(wa[u][1], blo[u][cg], bhi[u][cg], (int)wsc[u], (int)bsc[u][cg], acc[cg][1]);
            acc[cg][2] = mfma_mx<2>(wa[u][2], blo[u][cg], bhi[u][cg], (int)wsc[u], (int)bsc[u][cg], acc[cg][2]);
            acc[cg][3] = mfma_mx<3>(wa[u][3], blo[u][cg], bhi[u][cg], (int)wsc[u], (int)bsc[u][cg], acc[cg][3]);
          }
        }
        fetch(u, s + PF);
      }
    }
    // epilogue.  acc[cg][g][r] = D[row 64q + 16g + 4(l/16) + r][column col[cg]]
#pragma unroll
    for (int cg = 0; cg < 2; ++cg) {
      if (cg == 1 && !two) break;
      const bool valid = col[cg] < n;
      if (UP) {
        // rows 2i / 2i + 1 are gate / up of intermediate column i = 32q + 8g + 2(l/16) + {0, 1}
        float act[4][2];
        float amax = 0.f;
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const float gt = acc[cg][g][2 * h], up = acc[cg][g][2 * h + 1];
            act[g][h] = gt / (1.0f + expf(-gt)) * up;
            amax = fmaxf(amax, fabsf(act[g][h]));
          }
        amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
        amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
        const int ex = mx_shared_exp(amax, 8);
        const float inv = ldexpf(1.f, -ex);
        if (valid) {
          uint8_t* dst = p.aq + (size_t)slot[cg] * m.F + 32 * q + 2 * (lane >> 4);
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *(uint16_t*)(dst + 8 * g) = (uint16_t)(e4m3_code(act[g][0] * inv) | (e4m3_code(act[g][1] * inv) << 8));
          if ((lane >> 4) == 0) p.as[(size_t)slot[cg] * (m.F / 32) + q] = (uint8_t)(ex + 127);
        }
      } else if (valid) {
        const float wgt = s_w[col[cg]];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4_t o;
#pragma unroll
          for (int r = 0; r < 4; ++r) o[r] = wgt * acc[cg][g][r];
          *(f32x4_t*)(p.y + (size_t)slot[cg] * m.d + 64 * q + 16 * g + 4 * (lane >> 4)) = o;
        }
      }
    }
  }
}

struct MoeWs {
  float* logits;
  uint8_t *xq, *xs, *aq, *as;
  float* y;
  Route ro;
  size_t total;
};

MoeWs moe_ws_layout(const MoeDims& m, char* base) {
  MoeWs w;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align_up(bytes, 256); return base ? base + o : nullptr; };
  w.logits = (float*)take((size_t)kMaxRows * m.E * 4);
  w.xq = (uint8_t*)take((size_t)kMaxRows * m.d);
  w.xs = (uint8_t*)take((size_t)kMaxRows * m.d / 32);
  w.aq = (uint8_t*)take((size_t)kMaxRows * m.NS * m.F);
  w.as = (uint8_t*)take((size_t)kMaxRows * m.NS * m.F / 32);
  w.y = (float*)take((size_t)kMaxRows * m.NS * m.d * 4);
  w.ro.ids = (int*)take((size_t)kMaxRows * 8 * 4);
  w.ro.wts = (float*)take((size_t)kMaxRows * 8 * 4);
  w.ro.hits = (int*)take((size_t)kMaxLayers * 4);
  w.ro.n_hit = (int*)take(4);
  w.ro.list = (int*)take(256 * 4);
  w.total = off;
  return w;
}

}  // namespace

size_t moe_ws_bytes(const dlm_model_desc& d) {
  if (!d.n_experts) return 0;
  return moe_ws_layout(moe_dims(d), nullptr).total;
}

void moe_views(const MoeDims& m, void* ws, dlm_decode_views* out) {
  MoeWs w = moe_ws_layout(m, (char*)ws);
  out->moe_logits = w.logits;
  out->moe_xq = w.xq;
  out->moe_xs = w.xs;
  out->moe_ids = w.ro.ids;
  out->moe_wts = w.ro.wts;
  out->moe_aq = w.aq;
  out->moe_as = w.as;
  out->moe_y = w.y;
  out->moe_hits = w.ro.hits;
}

int moe_pack_layer(const MoeDims& m, const dlm_layer_weights& L, void* dst, hipStream_t st) {
  const int ET = m.E + m.S;
  uint8_t* out = (uint8_t*)dst;
  // per expert: w13 codes, w13 scales, w2 codes, w2 scales
  // (packed as four arrays over all experts so each kernel sees a fixed expert stride)
  uint8_t* w13 = out;
  uint8_t* w13s = w13 + (size_t)ET * m.w13_bytes();
  uint8_t* w2 = w13s + (size_t)ET * m.w13_scale_bytes();
  uint8_t* w2s = w2 + (size_t)ET * m.w2_bytes();
  MxPackP p;
  p.src = (const uint8_t*)L.x_w13;
  p.src_scale = (const uint8_t*)L.x_w13_scale;
  p.dst = w13;
  p.dst_scale = w13s;
  p.R = 2 * m.F;
  p.K = m.d;
  p.interleave = 1;
  p.chunks = (long long)ET * p.R * p.K / 32;
  hipLaunchKernelGGL(mx_pack_kernel, dim3((unsigned)((p.chunks + 255) / 256)), dim3(256), 0, st, p);
  DLM_HIP(hipGetLastError());
  p.src = (const uint8_t*)L.x_w2;
  p.src_scale = (const uint8_t*)L.x_w2_scale;
  p.dst = w2;
  p.dst_scale = w2s;
  p.R = m.d;
  p.K = m.F;
  p.interleave = 0;
  p.chunks = (long long)ET * p.R * p.K / 32;
  hipLaunchKernelGGL(mx_pack_kernel, dim3((unsigned)((p.chunks + 255) / 256)), dim3(256), 0, st, p);
  return check_hip(hipGetLastError(), "moe pack launch");
}

int moe_ffn(const MoeDims& m, int layer, const void* f, const void* router_packed, GemmPlan router_plan,
            const void* experts, void* ws, void* gemm_ws, const int32_t* cont_dev, PartialSrc* out, hipStream_t st) {
  if (m.rows > kMaxRows || m.E + m.S > kMaxExperts || m.E > 256 || m.top_k > 8 || layer >= kMaxLayers)
    return fail(DLM_ERR_SHAPE, "moe: unsupported shape");
  MoeWs w = moe_ws_layout(m, (char*)ws);
  const int ET = m.E + m.S;
  // 1. router logits
  EpiParams e;
  memset(&e, 0, sizeof(e));
  e.kind = EPI_STORE_F32;
  e.M = m.rows;
  e.bf16_out = 1;
  e.out = w.logits;
  e.ld_out = m.E;
  e.cont_dev = cont_dev;
  int rc = gemm_bf16(router_packed, f, m.E, m.d, MAP_IDENTITY, e, router_plan, gemm_ws, st);
  if (rc) return rc;
  // 2. route + quantise, one workgroup per row
  RouteP rp;
  rp.m = m;
  rp.logits = w.logits;
  rp.f = (const uint16_t*)f;
  rp.xq = w.xq;
  rp.xs = w.xs;
  rp.ro = w.ro;
  rp.cont_dev = cont_dev;
  hipLaunchKernelGGL(moe_route_kernel, dim3(m.rows), dim3(256), 0, st, rp);
  DLM_HIP(hipGetLastError());
  // 3. up (gate/up + SwiGLU + MXFP8 of act)
  const uint8_t* base = (const uint8_t*)experts;
  ExpP up;
  up.m = m;
  up.layer = layer;
  up.w = base;
  up.ws = base + (size_t)ET * m.w13_bytes();
  up.w_stride = m.w13_bytes();
  up.s_stride = m.w13_scale_bytes();
  up.Q = 2 * m.F / 64;
  up.S = m.d / 128;
  up.bq = w.xq;
  up.bs = w.xs;
  up.b_by_slot = 0;
  up.ro = w.ro;
  up.aq = w.aq;
  up.as = w.as;
  up.y = nullptr;
  up.cont_dev = cont_dev;
  const int slots = m.E + (m.rows + 31) / 32 * m.S;   // shared experts: one slot per 32 rows
  hipLaunchKernelGGL((moe_expert_kernel<1, 4>), dim3(slots * up.Q), dim3(64), 0, st, up);
  DLM_HIP(hipGetLastError());
  // 4. down (weighted, per slot)
  ExpP dn = up;
  dn.w = base + (size_t)ET * (m.w13_bytes() + m.w13_scale_bytes());
  dn.ws = dn.w + (size_t)ET * m.w2_bytes();
  dn.w_stride = m.w2_bytes();
  dn.s_stride = m.w2_scale_bytes();
  dn.Q = m.d / 64;
  dn.S = m.F / 128;
  dn.bq = w.aq;
  dn.bs = w.as;
  dn.b_by_slot = 1;
  dn.aq = nullptr;
  dn.as = nullptr;
  dn.y = w.y;
  hipLaunchKernelGGL((moe_expert_kernel<0, 4>), dim3(slots * dn.Q), dim3(64), 0, st, dn);
  DLM_HIP(hipGetLastError());
  PartialSrc ps{};
  ps.slots = w.y;
  ps.nslot = m.NS;
  *out = ps;
  return DLM_OK;
}

}  // namespace dlm

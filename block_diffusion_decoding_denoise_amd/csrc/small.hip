// Small kernels of the round: RMSNorm, the commit rule, block reset, the self-conditioning
// operand, the embedding gather of the commit pass and the prefix-length update.
#include "small.h"

namespace dlm {

namespace {

// ------------------------------------------------------------------ RMSNorm
// One workgroup (NTH threads, 1024 as launched) per row; deterministic fixed-order reduction.  When the residual
// stream has pending GEMM partial sums (a residual projection with deferred output), the row is
// first completed as x + p_0 + p_1 + ... in contributor order and written back.
struct NormP {
  float* x;
  const void* g;
  void* out;
  int d, bf16, packed;
  float eps;
  const int32_t* cont_dev;
  PartialSrc ps;
};

__device__ inline int owner_unit(long long s, long long T, int NW) {
  return (int)(((s + 1) * NW - 1) / T);
}

// Sum over a wave's 64 lanes without LDS round trips: DPP moves reduce each 16-lane row
// (neighbour swap, pair swap, half-row mirror, row mirror; after the two swaps a quad holds one
// value, so each mirror adds two equal-valued groups), then the four rows' sums are read from
// lanes 0, 16, 32 and 48 and added in that order.  Every lane returns the same value.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_move<0xB1>(v);     // quad_perm [1, 0, 3, 2]
  v += dpp_move<0x4E>(v);     // quad_perm [2, 3, 0, 1]
  v += dpp_move<0x141>(v);    // row_half_mirror
  v += dpp_move<0x140>(v);    // row_mirror
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return ((a + b) + c) + d;
}

template <int NTH>
__global__ __launch_bounds__(NTH) void rmsnorm_kernel(NormP p) {
  if (p.cont_dev && *p.cont_dev == 0) return;
  constexpr int NWV = NTH / 64;
  __shared__ float red[NWV];
  const int row = blockIdx.x, tid = threadIdx.x;
  float* x = p.x + (size_t)row * p.d;
  // every load of the row (x, gains, pending partial sums) is issued, unconditionally, before
  // any arithmetic: addresses of columns past d are clamped to column 0 and their values
  // ignored, and partial slots past a tile's contributor count use out-of-range buffer
  // offsets, which read zeros (d <= 4096: <= 4096 / (4 NTH) float4 per thread)
  constexpr int MAXV = 4096 / 4 / NTH, NPF = 6;
  int cc[MAXV];
  bool valid[MAXV];
  f32x4_t xv[MAXV];
#pragma unroll
  for (int j = 0; j < MAXV; ++j) {
    const int c = 4 * (tid + NTH * j);
    valid[j] = c < p.d;
    cc[j] = valid[j] ? c : 0;
    xv[j] = *(const f32x4_t*)(x + cc[j]);
  }
  u32x2_t gb[MAXV];
  f32x4_t gf[MAXV];
#pragma unroll
  for (int j = 0; j < MAXV; ++j) {
    if (p.bf16) gb[j] = *(const u32x2_t*)((const uint16_t*)p.g + cc[j]);
    else gf[j] = *(const f32x4_t*)((const float*)p.g + cc[j]);
  }
  if (p.ps.base) {
    const long long T = (long long)p.ps.tiles * p.ps.KT;
    const __amdgpu_buffer_rsrc_t pr = make_rsrc(p.ps.base, (uint32_t)p.ps.bytes);
    int cnt[MAXV];
    uint32_t off[MAXV];
    f32x4_t pv[MAXV][NPF];
#pragma unroll
    for (int j = 0; j < MAXV; ++j) {
      const int t = cc[j] >> 5;
      const int fo = owner_unit((long long)t * p.ps.KT, T, p.ps.NW);
      cnt[j] = valid[j] ? owner_unit((long long)(t + 1) * p.ps.KT - 1, T, p.ps.NW) - fo + 1 : 0;
      off[j] = (uint32_t)((((size_t)t * p.ps.cmax) * p.ps.mstride + (row + p.ps.row0) * 32 + (cc[j] & 31)) * 4);
      const uint32_t cstep = (uint32_t)p.ps.mstride * 4u;    // bytes between contributors
#pragma unroll
      for (int i = 0; i < NPF; ++i)
        pv[j][i] = __builtin_bit_cast(f32x4_t, bload16(pr, i < cnt[j] ? off[j] + (uint32_t)i * cstep : 0x80000000u));
    }
#pragma unroll
    for (int j = 0; j < MAXV; ++j) {
#pragma unroll
      for (int i = 0; i < NPF; ++i) xv[j] += pv[j][i];      // slots past cnt read zeros
      for (int i = NPF; i < cnt[j]; ++i)
        xv[j] += __builtin_bit_cast(f32x4_t, bload16(pr, off[j] + (uint32_t)i * (uint32_t)p.ps.mstride * 4u));
    }
  } else if (p.ps.slots) {
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(p.ps.slots + (size_t)(row + p.ps.row0) * p.ps.nslot * p.d,
                                                (uint32_t)(p.ps.nslot * p.d * 4));
    constexpr int MAXSL = 10;
    f32x4_t sv[MAXV][MAXSL];
#pragma unroll
    for (int j = 0; j < MAXV; ++j)
#pragma unroll
      for (int i = 0; i < MAXSL; ++i)
        sv[j][i] = __builtin_bit_cast(
            f32x4_t, bload16(sr, valid[j] && i < p.ps.nslot ? (uint32_t)((i * p.d + cc[j]) * 4) : 0x80000000u));
#pragma unroll
    for (int j = 0; j < MAXV; ++j)
#pragma unroll
      for (int i = 0; i < MAXSL; ++i) xv[j] += sv[j][i];
  }
  if (p.ps.base || p.ps.slots) {
#pragma unroll
    for (int j = 0; j < MAXV; ++j)
      if (valid[j]) *(f32x4_t*)(x + cc[j]) = xv[j];
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < MAXV; ++j)
    if (valid[j])
#pragma unroll
      for (int e = 0; e < 4; ++e) s = fmaf(xv[j][e], xv[j][e], s);
  s = wave_sum_dpp(s);
  if ((tid & 63) == 0) red[tid >> 6] = s;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < NWV; ++i) tot += red[i];
  const float r = 1.0f / sqrtf(tot / (float)p.d + p.eps);
#pragma unroll
  for (int j = 0; j < MAXV; ++j) {
    if (!valid[j]) continue;
    const int c = cc[j];
    if (p.bf16) {
      const float g4[4] = {lo_bf(gb[j][0]), hi_bf(gb[j][0]), lo_bf(gb[j][1]), hi_bf(gb[j][1])};
      uint2 ow;
      ow.x = pack2bf(xv[j][0] * r * g4[0], xv[j][1] * r * g4[1]);
      ow.y = pack2bf(xv[j][2] * r * g4[2], xv[j][3] * r * g4[3]);
      // 4 consecutive columns stay contiguous in the packed operand order
      *(uint2*)((uint16_t*)p.out + (p.packed ? xpk_index_m(row, c, p.d) : (size_t)row * p.d + c)) = ow;
    } else {
      f32x4_t o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = xv[j][e] * r * gf[j][e];
      *(f32x4_t*)((float*)p.out + (size_t)row * p.d + c) = o;
    }
  }
}

// ------------------------------------------------------------------ commit
struct CommitP {
  dlm_commit_rule rule;
  int rows;
  const float* maxp;
  const int32_t* amax;
  const float* lse;
  const float* ent;
  uint8_t* committed;
  int32_t* tokens;
  dlm_round_state* st;
};

__device__ inline float rank_key(float v) { return v != v ? -INFINITY : v; }

// One wave, lane i = row i (rows <= 64): every row's statistics are loaded at once, and the
// selection is taken through wave ballots.  An open row's rank is the number of open rows
// ranked before it (larger max-prob first, NaN as -inf, lower index first among equals), so
// "rank < k" picks exactly the k rows that k successive picks of the best remaining row take.
__global__ __launch_bounds__(64) void commit_kernel(CommitP p) {
  dlm_round_state* st = p.st;
  if (st->cont == 0) return;
  const int round = st->round;
  const int lane = threadIdx.x;
  const bool in = lane < p.rows;
  const int i = in ? lane : 0;                 // rows >= 1: lanes past the block re-read row 0
  const bool is_open = in && !p.committed[i];
  const float mp = p.maxp[i];
  const float ls = p.lse ? p.lse[i] : 0.f;
  const float en = p.ent ? p.ent[i] : 0.f;
  const int32_t am = p.amax[i];
  const uint64_t open = __ballot(is_open);
  const int n_open = __popcll(open);
  int flags = __ballot(is_open && !(isfinite(mp) && isfinite(ls) && isfinite(en))) ? DLM_FLAG_NONFINITE : 0;
  const float key = rank_key(mp);
  int rank = 0;
  for (int j = 0; j < p.rows; ++j) {
    const float kj = __shfl(key, j, 64);
    rank += ((open >> j) & 1ull) && (kj > key || (kj == key && j < lane)) ? 1 : 0;
  }
  uint64_t sel;
  if (p.rule.mode == DLM_COMMIT_THRESHOLD) {
    sel = __ballot(is_open && mp >= p.rule.tau);
    if (p.rule.forced_top1 && n_open > 0) sel |= __ballot(is_open && rank == 0);
  } else {
    sel = __ballot(is_open && rank < min(p.rule.k, n_open));
  }
  if (round >= p.rule.max_rounds - 1) {
    if (open & ~sel) flags |= DLM_FLAG_HIT_MAX_ROUNDS;
    sel = open;
  }
  if (in && ((sel >> lane) & 1ull)) {
    p.tokens[lane] = am;
    p.committed[lane] = 1;
  }
  if (lane == 0) {
    const int n_new = __popcll(sel);
    if (round < DLM_MAX_ROUNDS) st->n_new[round] = n_new;
    st->round = round + 1;
    st->n_open = n_open - n_new;
    st->flags |= flags;
    st->cont = (st->n_open > 0 && round + 1 < p.rule.max_rounds) ? 1 : 0;
  }
}

// ------------------------------------------------------------------ block reset
__global__ __launch_bounds__(256) void reset_kernel(int rows, uint8_t* committed, int32_t* tokens,
                                                    dlm_round_state* st, float* pe, int pe_elems) {
  const int tid = blockIdx.x * 256 + threadIdx.x;
  if (tid < rows) {
    committed[tid] = 0;
    tokens[tid] = 0;
  }
  if (st && tid < DLM_MAX_ROUNDS) st->n_new[tid] = 0;
  if (st && tid == 0) {
    st->round = 0;
    st->n_open = rows;
    st->cont = 1;
    st->flags = 0;
  }
  if (pe)
    for (int i = tid; i < pe_elems; i += gridDim.x * 256) pe[i] = 0.f;
}

// ------------------------------------------------------------------ self-cond operand
// xsc = round(pe) for open rows, 0 for committed rows (so W_sc xsc = 0 there); bf16 output is
// in the packed operand order of the skinny GEMM
__global__ __launch_bounds__(256) void selfcond_prep_kernel(const float* pe, const uint8_t* committed,
                                                            void* xsc, int rows, int d, int bf16,
                                                            const int32_t* cont_dev) {
  if (cont_dev && *cont_dev == 0) return;
  const int n = (bf16 ? 32 : rows) * d;   // bf16: all 32 operand rows (rows >= `rows` are zero)
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) {
    const int r = i / d;
    const float v = (r < rows && pe && !(committed && committed[r])) ? pe[i] : 0.f;
    if (bf16) ((uint16_t*)xsc)[xpk_index(r, i - r * d)] = f2bf(v);
    else ((float*)xsc)[i] = v;
  }
}

// ------------------------------------------------------------------ embedding gather
__global__ __launch_bounds__(256) void embed_kernel(const int32_t* tokens, const void* E, float* x,
                                                    int rows, int d, int V, int bf16) {
  const int n = rows * d;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) {
    const int r = i / d, c = i % d;
    int tok = tokens[r];
    tok = (tok < 0 || tok >= V) ? 0 : tok;   // out-of-range ids read row 0 instead of faulting
    const size_t src = (size_t)tok * d + c;
    x[i] = bf16 ? bf2f(((const uint16_t*)E)[src]) : ((const float*)E)[src];
  }
}

// row-major bf16 [rows, k] -> packed skinny-GEMM operand order (rows < 32; other rows zero)
__global__ __launch_bounds__(256) void pack_rows_kernel(const uint16_t* x, int rows, int k, uint16_t* out) {
  const int n = 32 * k;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) {
    const int r = i / k, c = i % k;
    out[xpk_index(r, c)] = r < rows ? x[i] : (uint16_t)0;
  }
}

__global__ void len_add_kernel(int32_t* len, int add) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *len += add;
}

}  // namespace

int rmsnorm(float* x, const void* g, void* out, int rows, int d, int bf16, int packed, float eps,
            const int32_t* cont_dev, hipStream_t st, const PartialSrc* ps) {
  PartialSrc none{};
  NormP p{x, g, out, d, bf16, packed, eps, cont_dev, ps ? *ps : none};
  hipLaunchKernelGGL(rmsnorm_kernel<1024>, dim3(rows), dim3(1024), 0, st, p);
  return check_hip(hipGetLastError(), "rmsnorm launch");
}

int commit_launch(const dlm_commit_rule& rule, int rows, const float* maxp, const int32_t* amax,
                  const float* lse, const float* ent, uint8_t* committed, int32_t* tokens,
                  dlm_round_state* state, hipStream_t st) {
  CommitP p{rule, rows, maxp, amax, lse, ent, committed, tokens, state};
  hipLaunchKernelGGL(commit_kernel, dim3(1), dim3(64), 0, st, p);
  return check_hip(hipGetLastError(), "commit launch");
}

int block_reset(int rows, uint8_t* committed, int32_t* tokens, dlm_round_state* state, float* pe,
                int pe_elems, hipStream_t st) {
  const int grid = pe ? 64 : 1;
  hipLaunchKernelGGL(reset_kernel, dim3(grid), dim3(256), 0, st, rows, committed, tokens, state, pe,
                     pe_elems);
  return check_hip(hipGetLastError(), "reset launch");
}

int selfcond_prep(const float* pe, const uint8_t* committed, void* xsc, int rows, int d, int bf16,
                  const int32_t* cont_dev, hipStream_t st) {
  hipLaunchKernelGGL(selfcond_prep_kernel, dim3(64), dim3(256), 0, st, pe, committed, xsc, rows, d, bf16,
                     cont_dev);
  return check_hip(hipGetLastError(), "selfcond prep launch");
}

int embed(const int32_t* tokens, const void* E, float* x, int rows, int d, int V, int bf16, hipStream_t st) {
  hipLaunchKernelGGL(embed_kernel, dim3(64), dim3(256), 0, st, tokens, E, x, rows, d, V, bf16);
  return check_hip(hipGetLastError(), "embed launch");
}

int pack_rows_bf16(const void* x, int rows, int k, void* out, hipStream_t st) {
  hipLaunchKernelGGL(pack_rows_kernel, dim3(64), dim3(256), 0, st, (const uint16_t*)x, rows, k, (uint16_t*)out);
  return check_hip(hipGetLastError(), "pack rows launch");
}

int len_add(int32_t* len, int add, hipStream_t st) {
  hipLaunchKernelGGL(len_add_kernel, dim3(1), dim3(64), 0, st, len, add);
  return check_hip(hipGetLastError(), "len add launch");
}

}  // namespace dlm

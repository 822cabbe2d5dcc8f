// Skinny GEMMs of the denoising round: C[m][n] = sum_k X[m][k] W[n][k] for the block's
// M <= 32 rows (or 64: a round fused with the previous block's commit pass), with the consumer
// of C fused into the epilogue (RoPE + KV-cache write, SwiGLU, residual add, self-conditioning
// input).
//
// bf16 path (matrix cores).  W is packed once at model load: 32-row tile t, 16-column step
// kt is one contiguous 1 KiB run in which lane l's 16 bytes are
// W[row(32t + l%32)][16kt + 8(l/32) .. +8] -- the A operand of v_mfma_f32_32x32x16_bf16.
// The packed matrix is therefore one contiguous stream of (tile, step) units, and the kernel
// is stream-K over it: worker (wave) w owns the contiguous unit range
// [w T / NW, (w+1) T / NW) of the T = tiles x steps units, so every worker streams the same
// number of bytes with 1 KiB loads and no tile-count tail.  Each wave keeps a ring of P
// steps in flight (buffer loads, which return zeros past the range, so the ring runs without
// branches); the block's activations (bf16, 32 x K per panel, L2-resident) are the B operand
// (32 rows in one MFMA; a second panel of 32 rows reuses each weight fragment for a second
// product), stored in the packed operand order so each fragment is one contiguous 1 KiB.
// When a worker finishes a tile segment it runs the epilogue straight from its
// accumulator registers if it owned the whole tile, else it stores a partial and the last
// contributor of the tile (agent-scope counter) adds the partials in contributor order, so
// results are deterministic.  Partials are handed over with coherent stores and loads, never
// with whole-L2 fences.
//
// Row orders of fused matrices (packed row p, tile t = p/32, r = p%32):
//   QKV: q and k heads hold rotate-half pairs side by side, p = 2i -> j = 16t'+i,
//        p = 2i+1 -> j + D/2 (t' = tile within the head), so RoPE is applied to a pair of
//        accumulators held by one lane; v rows keep their order.
//   GU:  p = 2i -> gate row 16t + i, p = 2i+1 -> up row 16t + i, so SwiGLU takes a pair.
#include "gemm.h"
#include "epilogue.h"

// Optional per-workgroup timestamps for kernel studies (compiled out unless defined).
#ifndef DLM_TRACE_POINT
#define DLM_TRACE_POINT(i)
#endif

#include <vector>

namespace dlm {

void build_row_map(int kind, int n_rows, int hq, int hkv, int D, int F, int32_t* out) {
  for (int p = 0; p < n_rows; ++p) {
    if (kind == MAP_QKV) out[p] = qkv_logical(p, hq, hkv, D);
    else if (kind == MAP_GU) out[p] = gu_logical(p, F);
    else out[p] = p;
  }
}

// single logical output n of row m (identity-mapped kinds)
__device__ inline void epi_single(const EpiParams& e, int m, int n, float v) {
  const size_t o = (size_t)m * e.ld_out + n;
  switch (e.kind) {
    case EPI_STORE_F32: e.out[o] = v; break;
    case EPI_RESID: e.out[o] += v; break;
    case EPI_SELFCOND: {
      if (e.committed[m]) {
        int tok = e.tokens[m];
        tok = (tok < 0 || tok >= e.vocab) ? 0 : tok;   // ids are in range unless the caller broke them
        e.out[o] = load_act(e.emb, (size_t)tok * e.ld_out + n, e.bf16_out);
      }
      else e.out[o] = load_act(e.mask_emb, n, e.bf16_out) + v;
      break;
    }
    default: break;
  }
}

// pair of packed rows (p, p+1), p even
__device__ inline void epi_pair_packed(const EpiParams& e, int map, int p, int m, float a, float b) {
  if (map == MAP_QKV) {
    const int Nq = e.hq * e.D, Nk = e.hkv * e.D;
    if (p < Nq + Nk) {
      const int first = qkv_logical(p, e.hq, e.hkv, e.D);
      const int part = first < Nq ? 0 : 1;
      const int rel = first - (part ? Nq : 0);
      epi_qk_rope(e, m, part, rel / e.D, rel % e.D, a, b);
    } else {
      epi_v(e, m, p - Nq - Nk, a);
      epi_v(e, m, p + 1 - Nq - Nk, b);
    }
  } else if (map == MAP_GU) {
    epi_swiglu(e, m, gu_logical(p, e.F), a, b);
  } else {
    epi_single(e, m, p, a);
    epi_single(e, m, p + 1, b);
  }
}

// ------------------------------------------------------------------ bf16 kernel
// Workspace: a fixed block of per-tile counters at the start (shared by every GEMM that uses
// the same workspace; each GEMM leaves its counters at zero), then the partial sums.
constexpr int kMaxTiles = 4096;
constexpr size_t kCounterBytes = kMaxTiles * 4;

struct GemmP {
  const uint16_t* W;
  const uint16_t* X;
  int K, KT, tiles, NW, cmax, map;
  int R;             // row-owned mode: rows per workgroup (0: stream-K)
  float* partial;    // [tiles][cmax][16][64] (fixup) or [tiles][cmax][32 MB][32] (deferred)
  int* counters;     // [tiles]
  EpiParams ep;
};

// workgroup owning unit s when workgroup g owns [floor(g T / NW), floor((g+1) T / NW))
__device__ inline int owner_of(long long s, long long T, int NW) {
  return (int)(((s + 1) * NW - 1) / T);
}

__device__ inline void epilogue_quarter(const GemmP& p, int t, const float (&v4)[4], int wave, int lane) {
  const int m = lane & 31;
  if (m >= p.ep.M) return;
#pragma unroll
  for (int q = 0; q < 4; q += 2) {
    const int r = 4 * wave + q;
    const int row = 8 * (r / 4) + 4 * (lane >> 5) + (r % 4);
    epi_pair_packed(p.ep, p.map, t * 32 + row, m, v4[q], v4[q + 1]);
  }
}

// A workgroup is one stream-K worker: it owns the contiguous unit range [s0, s1), which covers
// at most MAXSEG tile segments (first and last possibly partial); its 4 waves take every 4th
// unit of it, each wave parks its accumulator in LDS at every tile boundary, and the wave
// results are added in LDS in a fixed order.  Then, per segment: with deferred output the sum
// is stored as this workgroup's partial and a later kernel adds the partials; otherwise a tile
// the workgroup owns entirely gets its epilogue here, and a shared tile is finished by its last
// contributor, which adds all partials in contributor order.
constexpr int MAXSEG = 4;

__device__ inline int contributors(const GemmP& p, int t, long long T, int* first) {
  const int fo = owner_of((long long)t * p.KT, T, p.NW);
  const int lo = owner_of((long long)(t + 1) * p.KT - 1, T, p.NW);
  *first = fo;
  return lo - fo + 1;
}

// MB: activation panels of 32 rows (2 only with deferred output).
template <int P, int MB>
__global__ __launch_bounds__(256, MB == 1 ? 2 : 1) void gemm_bf16_kernel(GemmP p) {
  if (p.ep.cont_dev && *p.ep.cont_dev == 0) return;
  __shared__ float red[4][MAXSEG][MB][16][64];
  __shared__ int s_last[MAXSEG];
  const int lane = threadIdx.x & 63;
  const int v = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = blockIdx.x;
  const long long T = (long long)p.tiles * p.KT;
  const int s0 = (int)((long long)g * T / p.NW), s1 = (int)((long long)(g + 1) * T / p.NW);
  const int n = s1 - s0;
  const int nv = (n - v + 3) / 4;             // units of this wave: WG units v, v+4, ...
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(p.W + (size_t)s0 * 512, (uint32_t)n * 1024u);
  const uint32_t xpanel = (uint32_t)(32 * p.K * 2);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(p.X, MB * xpanel);
  const uint32_t wo = (uint32_t)lane * 16u;
  const uint32_t xo = (uint32_t)lane * 16u;
  u32x4_t wf[P], xf[P][MB];
  int kpf = (s0 + v) % p.KT;   // step-in-tile of the next unit this wave prefetches
#pragma unroll
  for (int u = 0; u < P; ++u) {
    wf[u] = bload16_nt(wr, wo + (uint32_t)(v + 4 * u) * 1024u);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) xf[u][mb] = bload16(xr, xo + (uint32_t)kpf * 1024u + mb * xpanel);
    kpf += 4;
    if (kpf >= p.KT) kpf %= p.KT;
  }
  f32x16_t acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[mb][r] = 0.f;
  const int t0 = s0 / p.KT;
  const int nseg = (s1 - 1) / p.KT - t0 + 1;
  int seg = 0;
  int nextb = (t0 + 1) * p.KT - s0;   // WG-relative unit where segment seg + 1 begins
  // streaming loop: no stores to global memory inside, so the ring's memory-counter waits
  // stay exact; a tile boundary parks the accumulator in LDS
  for (int k0 = 0; k0 < nv; k0 += P) {
#pragma unroll
    for (int u = 0; u < P; ++u) {
      const int unit = v + 4 * (k0 + u);
      while (unit < n && unit >= nextb) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            red[v][seg][mb][r][lane] = acc[mb][r];
            acc[mb][r] = 0.f;
          }
        ++seg;
        nextb += p.KT;
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[mb] = mfma32x32x16(wf[u], xf[u][mb], acc[mb]);
      wf[u] = bload16_nt(wr, wo + (uint32_t)(v + 4 * (k0 + u + P)) * 1024u);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) xf[u][mb] = bload16(xr, xo + (uint32_t)kpf * 1024u + mb * xpanel);
      kpf += 4;
      if (kpf >= p.KT) kpf %= p.KT;
    }
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) red[v][seg][mb][r][lane] = acc[mb][r];
  for (int sg = seg + 1; sg < nseg; ++sg)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) red[v][sg][mb][r][lane] = 0.f;
  __syncthreads();
  bool need[MAXSEG];
  int cnt[MAXSEG];
  bool any = false;
  for (int sg = 0; sg < nseg; ++sg) {
    const int t = t0 + sg;
    int fo;
    cnt[sg] = contributors(p, t, T, &fo);
    need[sg] = false;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      float sums[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 4 * v + q;
        sums[q] = ((red[0][sg][mb][r][lane] + red[1][sg][mb][r][lane]) + red[2][sg][mb][r][lane]) +
                  red[3][sg][mb][r][lane];
      }
      if (p.ep.kind == EPI_PARTIAL) {
        // [tile][contributor][m][n] with n contiguous: rows n = 8v + 4(lane/32) + q of column m
        float* dst = p.partial + ((size_t)t * p.cmax + (g - fo)) * (1024 * MB) + (32 * mb + (lane & 31)) * 32 +
                     8 * v + 4 * (lane >> 5);
        *(f32x4_t*)dst = f32x4_t{sums[0], sums[1], sums[2], sums[3]};
      } else if constexpr (MB == 1) {
        if (cnt[sg] == 1) {
          epilogue_quarter(p, t, sums, v, lane);
        } else {
          need[sg] = any = true;
          float* dst = p.partial + ((size_t)t * p.cmax + (g - fo)) * 1024;
#pragma unroll
          for (int q = 0; q < 4; ++q) store_coherent(&dst[(4 * v + q) * 64 + lane], sums[q]);
        }
      }
    }
  }
  if constexpr (MB == 1) {
    if (!any) return;
    wait_stores();
    __syncthreads();
    if (threadIdx.x < nseg) {
      const int sg = threadIdx.x;
      s_last[sg] = need[sg] ? (atomic_add_agent(&p.counters[t0 + sg], 1) == cnt[sg] - 1) : 0;
    }
    __syncthreads();
    for (int sg = 0; sg < nseg; ++sg) {
      if (!s_last[sg]) continue;
      const int t = t0 + sg;
      const float* base = p.partial + (size_t)t * p.cmax * 1024;
      float tot[4] = {0.f, 0.f, 0.f, 0.f};
      for (int j = 0; j < cnt[sg]; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) tot[q] += load_coherent(&base[(size_t)j * 1024 + (4 * v + q) * 64 + lane]);
      if (threadIdx.x == 0) store_agent(&p.counters[t], 0);
      epilogue_quarter(p, t, tot, v, lane);
    }
  }
}

// Row-owned mode: workgroup g owns R = N / NW whole output rows (packed rows [gR, gR + R)) over
// the full K, so no tile is shared and no partial sums exist.  W is packed per workgroup:
// block g is R x K, k-step kt (16 columns) of it is R x 16 contiguous, split into sub-tiles of
// 32 rows (the last one holds R mod 32 rows); sub-tile s of the step is stored in matrix-core
// operand order, lane (i + rows_s * h) holding row 32s + i, columns 16 kt + 8h .. +8.  Lanes of a
// short sub-tile past its rows load zeros (out-of-range buffer offsets), so every workgroup
// moves exactly R K 2 bytes of weights and one activation fragment per step feeds all NS
// sub-tiles.  The 4 waves take every 4th step; their sums are added in LDS in fixed order.
__device__ inline void epilogue_rows(const GemmP& p, int rowbase, int rows_s, const float (&v4)[4], int wave,
                                     int lane, int mb) {
  const int m = 32 * mb + (lane & 31);
  if (m >= p.ep.M) return;
#pragma unroll
  for (int q = 0; q < 4; q += 2) {
    const int r = 4 * wave + q;
    const int row = 8 * (r / 4) + 4 * (lane >> 5) + (r % 4);
    if (row < rows_s) epi_pair_packed(p.ep, p.map, rowbase + row, m, v4[q], v4[q + 1]);
  }
}

// MB: activation panels of 32 rows; one weight fragment feeds NS x MB products.
template <int NS, int P, int MB>
__global__ __launch_bounds__(256, 1) void gemm_owned_kernel(GemmP p) {
  DLM_TRACE_POINT(0);
  if (p.ep.cont_dev && *p.ep.cont_dev == 0) return;
  __shared__ float red[4][NS][MB][16][64];
  const int lane = threadIdx.x & 63;
  const int v = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = blockIdx.x;
  const int R = p.R;
  const uint32_t step_bytes = (uint32_t)R * 32u;
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(p.W + (size_t)g * R * p.K, step_bytes * (uint32_t)p.KT);
  const uint32_t xpanel = (uint32_t)(32 * p.K * 2);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(p.X, MB * xpanel);
  uint32_t wo[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int rows_s = min(32, R - 32 * s);
    const int i = lane & 31, h = lane >> 5;
    wo[s] = i < rows_s ? (uint32_t)(512 * s + (i + rows_s * h) * 8) * 2u : 0x80000000u;
  }
  const uint32_t xo = (uint32_t)lane * 16u;
  const int nv = (p.KT - v + 3) / 4;           // steps of this wave: v, v + 4, ...
  // With several row sub-tiles per step (gate/up), workgroups start at different column
  // steps (rotated by g KT / NW) so that the activation block, freshly written by the
  // previous kernel, is not requested by every workgroup at the same address at the same
  // time; measured, this helps the long gate/up stream and slightly slows the single-sub-tile
  // QKV, which keeps the natural order.  A wave's i-th step is (v + 4 i + kofs) mod KT; steps
  // past the wave's count read zeros (offsets at or above 2^31 are past every range).
  const int kofs = NS >= 2 ? (int)(((long long)g * p.KT) / p.NW) : 0;
  auto step_of = [&](int i) -> int {
    const int k = v + 4 * i;
    if (k >= p.KT) return -1;
    return k + kofs >= p.KT ? k + kofs - p.KT : k + kofs;
  };
  auto w_off = [&](int i, int s) -> uint32_t {
    const int r = step_of(i);
    return r < 0 ? 0x80000000u : wo[s] + (uint32_t)r * step_bytes;
  };
  auto x_off = [&](int i) -> uint32_t {
    const int r = step_of(i);
    return r < 0 ? 0x80000000u : xo + (uint32_t)r * 1024u;
  };
  u32x4_t wf[P][NS], xf[P][MB];
#pragma unroll
  for (int u = 0; u < P; ++u) {
#pragma unroll
    for (int s = 0; s < NS; ++s) wf[u][s] = bload16_nt(wr, w_off(u, s));
    const uint32_t xa = x_off(u);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) xf[u][mb] = bload16(xr, xa + mb * xpanel);
  }
  f32x16_t acc[NS][MB];
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[s][mb][r] = 0.f;
  for (int k0 = 0; k0 < nv; k0 += P) {
    if (k0 == P) DLM_TRACE_POINT(1);
#pragma unroll
    for (int u = 0; u < P; ++u) {
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[s][mb] = mfma32x32x16(wf[u][s], xf[u][mb], acc[s][mb]);
#pragma unroll
      for (int s = 0; s < NS; ++s) wf[u][s] = bload16_nt(wr, w_off(k0 + u + P, s));
      const uint32_t xa = x_off(k0 + u + P);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) xf[u][mb] = bload16(xr, xa + mb * xpanel);
    }
  }
  DLM_TRACE_POINT(2);
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) red[v][s][mb][r][lane] = acc[s][mb][r];
  __syncthreads();
  DLM_TRACE_POINT(3);
#pragma unroll
  for (int s = 0; s < NS; ++s) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      float sums[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 4 * v + q;
        sums[q] = ((red[0][s][mb][r][lane] + red[1][s][mb][r][lane]) + red[2][s][mb][r][lane]) +
                  red[3][s][mb][r][lane];
      }
      epilogue_rows(p, g * R + 32 * s, min(32, R - 32 * s), sums, v, lane, mb);
    }
  }
  DLM_TRACE_POINT(4);
}

// ------------------------------------------------------------------ wide activation blocks
// 64 < M <= 256 rows (the prompt's forward passes).  The same packed weights and plans as the
// block's skinny GEMMs, but the 4 waves split the rows instead of the contraction: wave w
// takes the 32-row panels w and w + 4 and runs every step of its workgroup's weight range, so
// each wave's accumulators hold complete sums (no reduction between waves, no LDS).  The 4
// waves read the same weight fragments close together in time: one read from HBM, the rest
// from the compute unit's cache.  Each weight fragment feeds 2 (x NS) products.

__device__ inline void wide_epilogue(const GemmP& p, int rowbase, int rows_s, const f32x16_t& a, int panel,
                                     int lane) {
  const int m = 32 * panel + (lane & 31);
  if (m >= p.ep.M) return;
#pragma unroll
  for (int r = 0; r < 16; r += 2) {
    const int row = 8 * (r / 4) + 4 * (lane >> 5) + (r % 4);
    if (row < rows_s) epi_pair_packed(p.ep, p.map, rowbase + row, m, a[r], a[r + 1]);
  }
}

// Row-owned plan (the weights packed with pack_bf16_owned for p.R): workgroup g owns packed
// rows [g R, g R + R) over the full K.
template <int NS, int P>
__global__ __launch_bounds__(256, 1) void gemm_wide_owned_kernel(GemmP p) {
  if (p.ep.cont_dev && *p.ep.cont_dev == 0) return;
  const int lane = threadIdx.x & 63;
  const int v = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int npan = (p.ep.M + 31) / 32;
  if (v >= npan) return;                       // no barriers below: idle waves may leave
  const bool two = v + 4 < npan;
  const int g = blockIdx.x;
  const int R = p.R;
  const uint32_t step_bytes = (uint32_t)R * 32u;
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(p.W + (size_t)g * R * p.K, step_bytes * (uint32_t)p.KT);
  const uint32_t xpanel = (uint32_t)(32 * p.K * 2);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(p.X, (uint32_t)npan * xpanel);
  uint32_t wo[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int rows_s = min(32, R - 32 * s);
    const int i = lane & 31, h = lane >> 5;
    wo[s] = i < rows_s ? (uint32_t)(512 * s + (i + rows_s * h) * 8) * 2u : 0x80000000u;
  }
  // the wave's two panels (the second past the rows reads zeros)
  const uint32_t xo0 = (uint32_t)lane * 16u + (uint32_t)v * xpanel;
  const uint32_t xo1 = two ? xo0 + 4u * xpanel : 0x80000000u;
  // workgroups start at different steps (as in the skinny kernel) so the activation block is
  // not requested at one address by every workgroup at once
  const int kofs = (int)(((long long)g * p.KT) / p.NW);
  auto step_of = [&](int i) -> int {
    if (i >= p.KT) return -1;
    return i + kofs >= p.KT ? i + kofs - p.KT : i + kofs;
  };
  u32x4_t wf[P][NS], xf[P][2];
  auto issue = [&](int u, int i) {
    const int r = step_of(i);
#pragma unroll
    for (int s = 0; s < NS; ++s) wf[u][s] = bload16_nt(wr, r < 0 ? 0x80000000u : wo[s] + (uint32_t)r * step_bytes);
    xf[u][0] = bload16(xr, r < 0 ? 0x80000000u : xo0 + (uint32_t)r * 1024u);
    xf[u][1] = bload16(xr, r < 0 || !two ? 0x80000000u : xo1 + (uint32_t)r * 1024u);
  };
#pragma unroll
  for (int u = 0; u < P; ++u) issue(u, u);
  f32x16_t acc[NS][2];
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[s][j][r] = 0.f;
  for (int k0 = 0; k0 < p.KT; k0 += P) {
#pragma unroll
    for (int u = 0; u < P; ++u) {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        acc[s][0] = mfma32x32x16(wf[u][s], xf[u][0], acc[s][0]);
        acc[s][1] = mfma32x32x16(wf[u][s], xf[u][1], acc[s][1]);
      }
      issue(u, k0 + u + P);
    }
  }
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int rows_s = min(32, R - 32 * s);
    wide_epilogue(p, g * R + 32 * s, rows_s, acc[s][0], v, lane);
    if (two) wide_epilogue(p, g * R + 32 * s, rows_s, acc[s][1], v + 4, lane);
  }
}

// Stream-K plan (the weights in the (tile, step) unit stream), deferred output only: the wave
// runs its workgroup's unit range in order and, at the end of each tile segment, stores its
// panels' sums as the workgroup's partial of that tile ([tile][contributor][m][n], m over all
// panels); the RMSNorm that consumes the residual adds the partials.
template <int P>
__global__ __launch_bounds__(256, 1) void gemm_wide_streamk_kernel(GemmP p) {
  if (p.ep.cont_dev && *p.ep.cont_dev == 0) return;
  const int lane = threadIdx.x & 63;
  const int v = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int npan = (p.ep.M + 31) / 32;
  if (v >= npan) return;                       // no barriers below
  const bool two = v + 4 < npan;
  const int g = blockIdx.x;
  const long long T = (long long)p.tiles * p.KT;
  const int s0 = (int)((long long)g * T / p.NW), s1 = (int)((long long)(g + 1) * T / p.NW);
  const int n = s1 - s0;
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(p.W + (size_t)s0 * 512, (uint32_t)n * 1024u);
  const uint32_t xpanel = (uint32_t)(32 * p.K * 2);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(p.X, (uint32_t)npan * xpanel);
  const uint32_t xo0 = (uint32_t)lane * 16u + (uint32_t)v * xpanel;
  const uint32_t xo1 = two ? xo0 + 4u * xpanel : 0x80000000u;
  u32x4_t wf[P], xf[P][2];
  auto issue = [&](int u, int i) {
    const bool ok = i < n;
    const int kt = (s0 + i) % p.KT;
    wf[u] = bload16_nt(wr, ok ? (uint32_t)lane * 16u + (uint32_t)i * 1024u : 0x80000000u);
    xf[u][0] = bload16(xr, ok ? xo0 + (uint32_t)kt * 1024u : 0x80000000u);
    xf[u][1] = bload16(xr, ok && two ? xo1 + (uint32_t)kt * 1024u : 0x80000000u);
  };
  auto flush = [&](int t, f32x16_t (&a)[2]) {
    int fo;
    contributors(p, t, T, &fo);
    float* base = p.partial + ((size_t)t * p.cmax + (g - fo)) * (size_t)(1024 * npan);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (j == 1 && !two) break;
      const int m = 32 * (v + 4 * j) + (lane & 31);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *(f32x4_t*)(base + (size_t)m * 32 + 8 * q + 4 * (lane >> 5)) =
            f32x4_t{a[j][4 * q], a[j][4 * q + 1], a[j][4 * q + 2], a[j][4 * q + 3]};
#pragma unroll
      for (int r = 0; r < 16; ++r) a[j][r] = 0.f;
    }
  };
#pragma unroll
  for (int u = 0; u < P; ++u) issue(u, u);
  f32x16_t acc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  int tcur = s0 / p.KT;
  int nextb = (tcur + 1) * p.KT - s0;          // unit index where the next tile begins
  for (int k0 = 0; k0 < n; k0 += P) {
#pragma unroll
    for (int u = 0; u < P; ++u) {
      const int i = k0 + u;
      if (i < n) {
        if (i == nextb) {
          flush(tcur, acc);
          ++tcur;
          nextb += p.KT;
        }
        acc[0] = mfma32x32x16(wf[u], xf[u][0], acc[0]);
        acc[1] = mfma32x32x16(wf[u], xf[u][1], acc[1]);
      }
      issue(u, i + P);
    }
  }
  flush(tcur, acc);
}

// One workgroup per compute unit: the weight stream is split into equal contiguous ranges, so
// every CU moves the same bytes and the workgroups finish together.  A range covers at most
// MAXSEG tile segments (n <= 3 K/16 + 1 units).
constexpr int kNumCU = 256;
constexpr int kMaxSub = 4;   // row-owned mode: at most 4 sub-tiles (128 rows) per workgroup

GemmPlan gemm_plan(int N, int K) {
  GemmPlan pl;
  const long long tiles = N / 32, T = tiles * (K / 16);
  long long nw = kNumCU;
  if (nw < (tiles + 2) / 3) nw = (tiles + 2) / 3;
  if (nw > T) nw = T;                    // every workgroup owns at least one unit
  pl.tpw = 1;
  pl.splits = (int)nw;                   // number of stream-K workgroups
  pl.R = 0;
  return pl;
}

GemmPlan gemm_plan_owned(int N, int K) {
  // the most workgroups (<= one per CU) that split N into equal even row counts of at most 128
  for (int nw = kNumCU; nw >= 1; --nw) {
    if (N % nw) continue;
    const int R = N / nw;
    if (R % 2 || R > 32 * kMaxSub) continue;
    if (nw < kNumCU / 2 && N >= kNumCU) break;   // too few workgroups to stream well
    GemmPlan pl;
    pl.tpw = 1;
    pl.splits = nw;
    pl.R = R;
    return pl;
  }
  return gemm_plan(N, K);
}

static int gemm_cmax(int N, int K, int nw) {
  const long long T = (long long)(N / 32) * (K / 16);
  const long long minsteps = T / nw > 0 ? T / nw : 1;
  return (int)((K / 16) / minsteps + 2);
}

static int panels(int M) { return (M + 31) / 32; }

PartialSrc gemm_partials(int N, int K, GemmPlan plan, void* ws, int M) {
  PartialSrc ps;
  ps.base = (const float*)((char*)ws + kCounterBytes);
  ps.tiles = N / 32;
  ps.KT = K / 16;
  ps.NW = plan.splits;
  ps.cmax = gemm_cmax(N, K, plan.splits);
  ps.mstride = 1024 * panels(M);
  ps.row0 = 0;
  ps.bytes = (size_t)ps.tiles * ps.cmax * ps.mstride * 4;
  ps.slots = nullptr;
  ps.nslot = 0;
  return ps;
}

size_t gemm_ws_bytes(int N, int K, GemmPlan plan, int mrows) {
  if (plan.R > 0) return kCounterBytes;
  const size_t part = (size_t)(N / 32) * gemm_cmax(N, K, plan.splits) * 1024 * panels(mrows) * 4;
  return kCounterBytes + align_up(part, 256);
}

int gemm_bf16(const void* W, const void* X, int N, int K, int map_kind, const EpiParams& ep,
              GemmPlan plan, void* ws, hipStream_t st) {
  GemmP p;
  p.W = (const uint16_t*)W;
  p.X = (const uint16_t*)X;
  p.K = K;
  p.KT = K / 16;
  p.tiles = N / 32;
  p.NW = plan.splits;
  p.cmax = gemm_cmax(N, K, plan.splits);
  p.map = map_kind;
  if (p.tiles > kMaxTiles) return fail(DLM_ERR_SHAPE, "gemm: %d tiles exceed %d", p.tiles, kMaxTiles);
  const long long T = (long long)p.tiles * p.KT;
  if ((T + p.NW - 1) / p.NW > 3LL * p.KT + 1) return fail(DLM_ERR_SHAPE, "gemm: plan spans too many tiles");
  p.counters = (int*)ws;
  p.partial = (float*)((char*)ws + kCounterBytes);
  p.ep = ep;
  p.R = plan.R;
  if (ep.M < 1 || ep.M > 256) return fail(DLM_ERR_SHAPE, "gemm: %d rows (1..256 supported)", ep.M);
  const int mb = panels(ep.M);
  auto launch = [&](auto kern) { hipLaunchKernelGGL(kern, dim3(p.NW), dim3(256), 0, st, p); };
  if (ep.M > 64) {
    // wide blocks: row-owned plans with any row-owned epilogue, stream-K plans deferred only
    if (plan.R > 0) {
      if (ep.kind == EPI_PARTIAL) return fail(DLM_ERR_ARG, "gemm: row-owned plan has no partial sums");
      if (N != plan.R * plan.splits || plan.R % 2 || plan.R > 32 * kMaxSub)
        return fail(DLM_ERR_SHAPE, "gemm: bad row-owned plan");
      const int ns = (plan.R + 31) / 32;
      if (ns == 1) launch(gemm_wide_owned_kernel<1, 8>);
      else if (ns == 2) launch(gemm_wide_owned_kernel<2, 8>);
      else if (ns == 3) launch(gemm_wide_owned_kernel<3, 6>);
      else launch(gemm_wide_owned_kernel<4, 4>);
    } else {
      if (ep.kind != EPI_PARTIAL) return fail(DLM_ERR_ARG, "gemm: more than 64 rows on a stream-K plan need deferred output");
      launch(gemm_wide_streamk_kernel<8>);
    }
    return check_hip(hipGetLastError(), "gemm_bf16 launch");
  }
  if (plan.R > 0) {
    if (ep.kind == EPI_PARTIAL) return fail(DLM_ERR_ARG, "gemm: row-owned plan has no partial sums");
    if (N != plan.R * plan.splits || plan.R % 2 || plan.R > 32 * kMaxSub)
      return fail(DLM_ERR_SHAPE, "gemm: bad row-owned plan");
    const int ns = (plan.R + 31) / 32;
    // ring depths from sweeps at the 4B shapes (QKV: 8 beat 6, 12, 16 and 20 steps; gate/up
    // with two panels: 4 beat 6 and 8)
    if (mb == 1) {
      if (ns == 1) launch(gemm_owned_kernel<1, 8, 1>);
      else if (ns == 2) launch(gemm_owned_kernel<2, 12, 1>);
      else if (ns == 3) launch(gemm_owned_kernel<3, 8, 1>);
      else launch(gemm_owned_kernel<4, 8, 1>);
    } else {
      if (ns == 1) launch(gemm_owned_kernel<1, 8, 2>);
      else if (ns == 2) launch(gemm_owned_kernel<2, 8, 2>);
      else if (ns == 3) launch(gemm_owned_kernel<3, 4, 2>);
      else launch(gemm_owned_kernel<4, 4, 2>);
    }
    return check_hip(hipGetLastError(), "gemm_bf16 launch");
  }
  if (mb == 2 && ep.kind != EPI_PARTIAL)
    return fail(DLM_ERR_ARG, "gemm: more than 32 rows need a row-owned plan or deferred output");
  if (mb == 1) launch(gemm_bf16_kernel<8, 1>);
  else launch(gemm_bf16_kernel<4, 2>);   // two panels: a 4-unit ring measured faster than 6 or 8
  return check_hip(hipGetLastError(), "gemm_bf16 launch");
}

// ------------------------------------------------------------------ f32 kernel
struct F32P {
  F32Mats W;
  const float* X;
  int N, K, map, units;
  EpiParams ep;
};


__device__ inline float dot_row(const F32P& p, int n, const float* x) {
  int r = n, i = 0;
  while (i < 2 && r >= p.W.rows[i]) { r -= p.W.rows[i]; ++i; }
  const float* w = p.W.w[i] + (size_t)r * p.K;
  float acc = 0.f;
  for (int k = 0; k < p.K; ++k) acc = fmaf(x[k], w[k], acc);
  return acc;
}

__global__ __launch_bounds__(256) void gemm_f32_kernel(F32P p) {
  if (p.ep.cont_dev && *p.ep.cont_dev == 0) return;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  const int m = idx / p.units, u = idx % p.units;
  if (m >= p.ep.M) return;
  const float* x = p.X + (size_t)m * p.K;
  const EpiParams& e = p.ep;
  if (p.map == MAP_QKV) {
    const int Nq = e.hq * e.D, Nk = e.hkv * e.D;
    const int pairs = (Nq + Nk) / 2;
    if (u < pairs) {
      const int part = u < Nq / 2 ? 0 : 1;
      const int rel = u - (part ? Nq / 2 : 0);
      const int head = rel / (e.D / 2), j = rel % (e.D / 2);
      const int first = (part ? Nq : 0) + head * e.D + j;
      epi_qk_rope(e, m, part, head, j, dot_row(p, first, x), dot_row(p, first + e.D / 2, x));
    } else {
      const int rel = u - pairs;
      epi_v(e, m, rel, dot_row(p, Nq + Nk + rel, x));
    }
  } else if (p.map == MAP_GU) {
    epi_swiglu(e, m, u, dot_row(p, u, x), dot_row(p, e.F + u, x));
  } else {
    epi_single(e, m, u, dot_row(p, u, x));
  }
}

int gemm_f32(const F32Mats& W, const float* X, int N, int K, int map_kind, const EpiParams& ep,
             hipStream_t st) {
  F32P p;
  p.W = W;
  p.X = X;
  p.N = N;
  p.K = K;
  p.map = map_kind;
  if (map_kind == MAP_QKV) p.units = (ep.hq * ep.D + ep.hkv * ep.D) / 2 + ep.hkv * ep.D;
  else if (map_kind == MAP_GU) p.units = N / 2;
  else p.units = N;
  p.ep = ep;
  const int total = ep.M * p.units;
  hipLaunchKernelGGL(gemm_f32_kernel, dim3((total + 255) / 256), dim3(256), 0, st, p);
  return check_hip(hipGetLastError(), "gemm_f32 launch");
}

// ------------------------------------------------------------------ packing
struct PackP {
  const uint16_t* src[3];
  int rows[3];
  int n_src, k, KT;
  int ld;              // row stride of the sources in elements (k unless a column slice is packed)
  const int32_t* map;
  uint16_t* dst;
};

__global__ __launch_bounds__(64) void pack_kernel(PackP p) {
  const int t = blockIdx.x / p.KT, kt = blockIdx.x % p.KT, lane = threadIdx.x;
  int row = p.map ? p.map[t * 32 + (lane & 31)] : t * 32 + (lane & 31);
  int i = 0;
  while (i < p.n_src - 1 && row >= p.rows[i]) { row -= p.rows[i]; ++i; }
  const uint16_t* s = p.src[i] + (size_t)row * p.ld + kt * 16 + 8 * (lane >> 5);
  u32x4_t v = *(const u32x4_t*)s;
  *(u32x4_t*)(p.dst + ((size_t)blockIdx.x * 64 + lane) * 8) = v;
}

// Row-owned layout (see gemm_owned_kernel): 16-byte chunk c of the output decodes to
// workgroup g, step kt, sub-tile s, row i, column half h.
__global__ __launch_bounds__(256) void pack_owned_kernel(PackP p, int R, long long chunks) {
  const long long c = (long long)blockIdx.x * 256 + threadIdx.x;
  if (c >= chunks) return;
  const long long per_g = (long long)R * p.k / 8;
  const int g = (int)(c / per_g);
  const int rem = (int)(c % per_g);
  const int kt = rem / (2 * R), w = rem % (2 * R);
  const int s = w / 64, x = w % 64;
  const int rows_s = min(32, R - 32 * s);
  const int i = x % rows_s, h = x / rows_s;
  const int prow = g * R + 32 * s + i;
  int row = p.map ? p.map[prow] : prow;
  int src = 0;
  while (src < p.n_src - 1 && row >= p.rows[src]) { row -= p.rows[src]; ++src; }
  const uint16_t* sp = p.src[src] + (size_t)row * p.ld + kt * 16 + 8 * h;
  *(u32x4_t*)(p.dst + (size_t)c * 8) = *(const u32x4_t*)sp;
}

int pack_bf16_owned(const void* const* srcs, const int* src_rows, int n_src, int n_rows, int k,
                    const int32_t* row_map_dev, int R, void* dst, hipStream_t st, int ld) {
  PackP p;
  for (int i = 0; i < 3; ++i) {
    p.src[i] = i < n_src ? (const uint16_t*)srcs[i] : nullptr;
    p.rows[i] = i < n_src ? src_rows[i] : 0;
  }
  p.n_src = n_src;
  p.k = k;
  p.KT = k / 16;
  p.ld = ld > 0 ? ld : k;
  p.map = row_map_dev;
  p.dst = (uint16_t*)dst;
  if (R <= 0 || n_rows % R || R % 2) return fail(DLM_ERR_SHAPE, "pack: bad row-owned layout");
  const long long chunks = (long long)n_rows * k / 8;
  hipLaunchKernelGGL(pack_owned_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, st, p, R, chunks);
  return check_hip(hipGetLastError(), "pack launch");
}

int pack_bf16(const void* const* srcs, const int* src_rows, int n_src, int n_rows, int k,
              const int32_t* row_map_dev, void* dst, hipStream_t st) {
  PackP p;
  for (int i = 0; i < 3; ++i) {
    p.src[i] = i < n_src ? (const uint16_t*)srcs[i] : nullptr;
    p.rows[i] = i < n_src ? src_rows[i] : 0;
  }
  p.n_src = n_src;
  p.k = k;
  p.KT = k / 16;
  p.ld = k;
  p.map = row_map_dev;
  p.dst = (uint16_t*)dst;
  hipLaunchKernelGGL(pack_kernel, dim3((n_rows / 32) * p.KT), dim3(64), 0, st, p);
  return check_hip(hipGetLastError(), "pack launch");
}

}  // namespace dlm

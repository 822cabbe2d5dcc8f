// Tied-embedding head with fused row statistics and the p.E feedback mix.
//
// For the open rows h_i of the block: l = h_i E^T over the whole vocabulary, then
// lse, entropy, max-prob, argmax and pe_i = sum_v softmax(l)_v E_v, with the logits never
// stored (page "ORL: diffusion LLMs get a learnable 'tokens per forward'", section "What
// shipped": per-round distribution over unresolved tokens, self-conditioning on the tied
// embedding; "QwenDLM-4B-ORL" model card, evaluation pipeline: fused row statistics).
//
// bf16 path: one workgroup of NW waves per (vocabulary chunk, group of 16 open rows).
// Wave w owns the d-slice [w d/NW, (w+1) d/NW): it keeps the rows' slice of h and its
// slice of the p.E accumulator in registers for the whole kernel.  Per tile of 16 vocabulary
// rows: (1) each wave streams its slice of the tile's E rows from HBM (prefetched one tile
// ahead) and forms partial logits with v_mfma_f32_16x16x32_bf16 (A = E rows, B = h rows);
// (2) the NW partials are summed through LDS in a fixed order and 256 threads update the
// online statistics per row (running max, sum of e^(l-m), sum of e^(l-m)(l-m) for the
// entropy, argmax with lowest-id ties; 16-lane reductions by DPP row moves) and publish
// p = e^(l - m_new) in bf16 and the rescale factor; (3) each wave adds P (16 rows x 16
// vocab) times its E slice with v_mfma_f32_16x16x16bf16_1k.  The slice is kept in a
// wave-private LDS copy in its natural [vocab][d] layout (one 16-byte write per k-step) and
// read back transposed, vocabulary-major, by the transpose read ds_read_b64_tr_b16; the
// accumulators are rescaled only when a row's running max moved.  The three steps are
// software-pipelined over tiles: (1) of tile t + 1 and (2) of tile t run between the same two
// barriers, (3) of tile t after them, so a tile costs one barrier.  E is read
// from HBM once per row group; the groups of one chunk run on one XCD, so the second
// group mostly hits L2.  Partial statistics and partial pe (bf16) per chunk go to the workspace
// and a combine kernel merges the chunks in index order (deterministic).
#include "head.h"

namespace dlm {

namespace {

struct HeadP {
  const uint16_t* h;       // [rows, d] bf16 (f32 path: const float*)
  const uint16_t* E;       // [V, d]
  const uint8_t* committed;
  int rows, d, V;
  float* st;               // [CH][rows_max][8] partial stats
  float* pe_part;          // [CH][rows_max][d]: f32 path float, bf16 path bf16 (uint16_t)
  float* logits_dbg;       // [rows, V] or null
  int rows_max, chunks_fixed;
  // outputs (combine)
  float* lse;
  float* ent;
  float* maxp;
  int32_t* amax;
  float* pe;
  const int32_t* cont_dev;
};

// open rows of the block (rows <= 64) as a bit mask: one flag load per lane, then a wave
// ballot (every wave computes the same mask)
__device__ inline unsigned long long open_mask(const uint8_t* committed, int rows) {
  const int lane = threadIdx.x & 63;
  bool open = false;
  if (lane < rows) open = committed == nullptr || committed[lane] == 0;
  return __ballot(open);
}

// open-row compaction shared by all kernels: returns n_open, and fills idx[k] = row of the
// k-th open row (idx in LDS, size >= 64); any multiple of 64 threads.
__device__ inline int compact_open(const uint8_t* committed, int rows, int* idx) {
  const unsigned long long mask = open_mask(committed, rows);
  const int lane = threadIdx.x & 63;
  if (threadIdx.x < 64 && ((mask >> lane) & 1ull)) idx[__popcll(mask & ((1ull << lane) - 1ull))] = lane;
  __syncthreads();
  return __popcll(mask);
}

// bf16 path: 256 workgroups = 8 XCDs x 32 slots; the n_groups row groups of a chunk share
// an XCD slot range, so the chunk count is 8 * floor(32 / n_groups).
__device__ inline int n_chunks_for(int n_groups, int chunks_fixed) {
  return chunks_fixed > 0 ? chunks_fixed : 8 * (32 / n_groups);
}

// statistics layout per (chunk, open row): m, s, T, best value, best index (as float bits)
enum { ST_M = 0, ST_S = 1, ST_T = 2, ST_BV = 3, ST_BI = 4 };

// Reductions over the 16 lanes of a DPP row (lanes 16 r .. 16 r + 15) by DPP moves: swap
// neighbours, swap pairs, mirror each half-row, mirror the row.  After the two quad swaps
// the 4 lanes of a quad hold the same value, so each mirror combines two equal-valued groups
// and every lane of the row ends with the same, order-independent-of-lane result.
enum : int { DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140 };

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<DPP_XOR1>(v));
  v = fmaxf(v, dpp_f<DPP_XOR2>(v));
  v = fmaxf(v, dpp_f<DPP_HALF_MIRROR>(v));
  return fmaxf(v, dpp_f<DPP_MIRROR>(v));
}
// two sums at once (independent chains)
__device__ __forceinline__ void row16_sum2(float& a, float& b) {
  a += dpp_f<DPP_XOR1>(a);
  b += dpp_f<DPP_XOR1>(b);
  a += dpp_f<DPP_XOR2>(a);
  b += dpp_f<DPP_XOR2>(b);
  a += dpp_f<DPP_HALF_MIRROR>(a);
  b += dpp_f<DPP_HALF_MIRROR>(b);
  a += dpp_f<DPP_MIRROR>(a);
  b += dpp_f<DPP_MIRROR>(b);
}
// (value, index) with the larger value, lowest index among equal values
template <int CTRL>
__device__ __forceinline__ void argmax_step(float& v, int& i) {
  const float ov = dpp_f<CTRL>(v);
  const int oi = dpp_i<CTRL>(i);
  if (ov > v || (ov == v && oi < i)) { v = ov; i = oi; }
}
__device__ __forceinline__ void row16_argmax(float& v, int& i) {
  argmax_step<DPP_XOR1>(v, i);
  argmax_step<DPP_XOR2>(v, i);
  argmax_step<DPP_HALF_MIRROR>(v, i);
  argmax_step<DPP_MIRROR>(v, i);
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));
// Transpose read (gfx950): within each 16-lane group, lane i receives element i % 4 of the
// 8-byte loads of lanes 4 j + i / 4 (j = 0..3) of its group.
__device__ __forceinline__ u32x2_t lds_read_tr16(const uint16_t* p) {
  const s16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)p);
  return __builtin_bit_cast(u32x2_t, r);
}

// Loads are branch-free (rows, vocabulary entries and d-steps out of range use out-of-range
// buffer offsets, which read zeros), so the next tile's loads stay in flight while a tile is
// processed.  DBG: also store every logit (tests).
template <int MAXK, int NW, bool DBG>
__global__ __launch_bounds__(NW * 64) void head_bf16_kernel(HeadP p) {
  if (p.cont_dev && *p.cont_dev == 0) return;
  __shared__ int s_idx[DLM_MAX_ROWS];
  // double-buffered by tile parity: a tile's statistics are taken while the next tile's
  // partial logits are written (the 16-wave form has LDS for one buffer and takes its
  // statistics before the next partial logits, behind one more barrier)
  constexpr int NLP = NW == 8 ? 2 : 1;
  __shared__ float lpart[NLP][NW][16][17];       // [parity][wave][v][row]
  __shared__ __attribute__((aligned(16))) uint16_t Pt[2][16][16];   // [parity][row][v] bf16
  __shared__ float alpha_s[2][16];
  // wave-private copy of the wave's E slice, [vocab][d] with rows padded by 16 bytes (the 16
  // rows of a transpose read then cover the 64 banks twice, the rows of a write once per lane
  // group)
  constexpr int EROW = MAXK * 32 + 8;
  __shared__ __attribute__((aligned(16))) uint16_t En[NW][16][EROW];
  const int n_open = compact_open(p.committed, p.rows, s_idx);
  if (n_open == 0) return;
  const int n_groups = (n_open + 15) / 16;
  const int CH = n_chunks_for(n_groups, 0);
  const int b = blockIdx.x;
  int chunk, grp;
  {
    const int xcd = b & 7, j = b >> 3;
    chunk = (j / n_groups) * 8 + xcd;
    grp = j % n_groups;
  }
  if (chunk >= CH) return;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int KST = p.d / 32;
  const int kw0 = (w * KST) / NW, kw1 = ((w + 1) * KST) / NW;
  const int nk = kw1 - kw0;
  const int VT = (p.V + 15) / 16;
  const int t0 = (int)(((long long)chunk * VT) / CH), t1 = (int)(((long long)(chunk + 1) * VT) / CH);

  // h fragments (B operand of the logit MFMA): lane l: row 16grp + l%16, d = 32kt + 8(l/16)..
  u32x4_t hf[MAXK];
  {
    const int k = 16 * grp + (lane & 15);
    const bool ok = k < n_open;
    const int row = ok ? s_idx[k] : 0;
    const __amdgpu_buffer_rsrc_t hr = make_rsrc(p.h, (uint32_t)(p.rows * p.d * 2));
#pragma unroll
    for (int u = 0; u < MAXK; ++u)
      hf[u] = bload16(hr, (ok && u < nk) ? (uint32_t)((row * p.d + (kw0 + u) * 32 + 8 * (lane >> 4)) * 2)
                                         : 0x80000000u);
  }
  f32x4_t acc[MAXK][2];
#pragma unroll
  for (int u = 0; u < MAXK; ++u) acc[u][0] = acc[u][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // running statistics for row (tid / 16) of the group, replicated over 16 lanes
  float rm = -INFINITY, rs = 0.f, rT = 0.f, bv = -INFINITY;
  int bi = 0x7fffffff;
  const int my_row = tid >> 4, my_v = tid & 15;

  // E rows as a buffer (the host keeps V d 2 < 2^31)
  const __amdgpu_buffer_rsrc_t er = make_rsrc(p.E, (uint32_t)((size_t)p.V * p.d * 2));
  auto load_tile = [&](int t, u32x4_t* ef) {
    const int v = t * 16 + (lane & 15);
    const bool ok = v < p.V && t < t1;
    const uint32_t base = ((uint32_t)v * (uint32_t)p.d + (uint32_t)(kw0 * 32 + 8 * (lane >> 4))) * 2u;
#pragma unroll
    for (int u = 0; u < MAXK; ++u) ef[u] = bload16(er, (ok && u < nk) ? base + (uint32_t)u * 64u : 0x80000000u);
  };
  // Software-pipelined over tiles, one barrier per tile.  Between barriers: tile t + 1's
  // partial logits (all waves) and tile t's statistics (threads 0..255, from the partials
  // written before the previous barrier); after the barrier: tile t's P . E (from the LDS copy)
  // and the LDS copy of tile t + 1.  Two register buffers alternate: a buffer's tile is
  // requested two tiles before its partial logits, right after the buffer was copied to LDS.
  // Past t1 the loads read zeros and the extra partial logits and copy are never used.
  auto logits = [&](const u32x4_t* ef, int par) {
    // partial logits over this wave's d-slice: L^T[v][row] (d-steps past nk are zeros)
    f32x4_t lp = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < MAXK; ++u) lp = mfma16x16x32(ef[u], hf[u], lp);
#pragma unroll
    for (int r = 0; r < 4; ++r) lpart[par % NLP][w][4 * (lane >> 4) + r][lane & 15] = lp[r];
  };
  auto stash = [&](const u32x4_t* ef) {
#pragma unroll
    for (int u = 0; u < MAXK; ++u) *(u32x4_t*)&En[w][lane & 15][u * 32 + 8 * (lane >> 4)] = ef[u];
  };
  // reduce tile t's partials and update the statistics of row my_row (threads 0..255)
  auto stats = [&](int t, int par) {
    if (tid >= 256) return;
    float l = 0.f;
#pragma unroll
    for (int q = 0; q < NW; ++q) l += lpart[par % NLP][q][my_v][my_row];
    const int vg = t * 16 + my_v;
    const bool valid = vg < p.V;
    if (!valid) l = -INFINITY;
    const int k = 16 * grp + my_row;
    if (DBG && valid && k < n_open) p.logits_dbg[(size_t)s_idx[k] * p.V + vg] = l;
    const float tm = row16_max(l);
    // tile argmax (lowest id among equal values)
    float cv = l;
    int ci = valid ? vg : 0x7fffffff;
    row16_argmax(cv, ci);
    if (cv > bv || (cv == bv && ci < bi)) { bv = cv; bi = ci; }
    const float mn = fmaxf(rm, tm);
    const float al = rs > 0.f ? expf(rm - mn) : 0.f;
    const float e = valid ? expf(l - mn) : 0.f;
    float se = e, te = valid ? e * (l - mn) : 0.f;
    row16_sum2(se, te);
    rT = rs > 0.f ? al * (rT + (rm - mn) * rs) + te : te;
    rs = al * rs + se;
    rm = mn;
    Pt[par][my_row][my_v] = f2bf(e);
    if (my_v == 0) alpha_s[par][my_row] = al;
  };
  // acc[rows][d-slice] = alpha * acc + P E_slice.  B operand of d-block (u, hb): lane l takes
  // E[vocab 4(l/16) + j][d 32u + 16hb + l%16], j = 0..3, by a transpose read whose lanes address
  // vocabulary row 4(l/16) + (l%16)/4 at d 32u + 16hb + 4(l%4).
  auto pe_step = [&](int par) {
    const u32x2_t pa = *(const u32x2_t*)&Pt[par][lane & 15][4 * (lane >> 4)];
    float al4[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) al4[r] = alpha_s[par][4 * (lane >> 4) + r];
    // rescale only when some row's running max moved (alpha 1 leaves acc unchanged)
    const bool moved = __builtin_amdgcn_ballot_w64(al4[0] != 1.f || al4[1] != 1.f || al4[2] != 1.f ||
                                                   al4[3] != 1.f) != 0;
    const uint16_t* eb0 = &En[w][4 * (lane >> 4) + ((lane & 15) >> 2)][4 * (lane & 3)];
#pragma unroll
    for (int u = 0; u < MAXK; ++u) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const u32x2_t eb = lds_read_tr16(eb0 + u * 32 + 16 * hb);
        f32x4_t a = acc[u][hb];
        if (moved) {
#pragma unroll
          for (int r = 0; r < 4; ++r) a[r] *= al4[r];
        }
        acc[u][hb] = mfma16x16x16(pa, eb, a);
      }
    }
  };
  // one tile: bn holds tile t + 1, bf tile t + 2 (in flight)
  auto iter = [&](int t, int par, u32x4_t* bn) {
    if constexpr (NLP == 2) {
      logits(bn, par ^ 1);
      stats(t, par);
    } else {
      stats(t, par);
      __syncthreads();
      logits(bn, par ^ 1);
    }
    __syncthreads();
    pe_step(par);
    stash(bn);
    load_tile(t + 3, bn);            // past t1: zeros, no traffic
    // keep the requests here (left alone, the scheduler sinks loads below the matrix ops that
    // wait for the tile before, and a tile is then requested only once that one has arrived)
    __builtin_amdgcn_sched_barrier(0);
  };
  u32x4_t b0[MAXK], b1[MAXK];
  load_tile(t0, b0);
  load_tile(t0 + 1, b1);
  __builtin_amdgcn_sched_barrier(0);
  logits(b0, 0);
  stash(b0);
  load_tile(t0 + 2, b0);
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  int t = t0;
  for (; t + 1 < t1; t += 2) {
    iter(t, 0, b1);
    iter(t + 1, 1, b0);
  }
  if (t < t1) iter(t, 0, b1);      // uniform over the workgroup
  // partial outputs for rows k = 16grp + r
  if (tid < 256 && my_v == 0) {
    const int k = 16 * grp + my_row;
    if (k < n_open) {
      float* st = p.st + ((size_t)chunk * p.rows_max + k) * 8;
      st[ST_M] = rm;
      st[ST_S] = rs;
      st[ST_T] = rT;
      st[ST_BV] = bv;
      st[ST_BI] = __int_as_float(bi);
    }
  }
  // acc[u][hb] lane l: row 4(l/16)+r, d = kw0*32 + u*32 + 16hb + l%16; stored in bf16 (the
  // combine reads 256 chunks' partials of every open row, so this halves its bytes; each partial
  // is one term of a positively weighted sum, and the result feeds a bf16 input anyway)
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int k = 16 * grp + 4 * (lane >> 4) + r;
    if (k < n_open) {
      uint16_t* dst = (uint16_t*)p.pe_part + ((size_t)chunk * p.rows_max + k) * p.d + kw0 * 32;
#pragma unroll
      for (int u = 0; u < MAXK; ++u)
        if (u < nk) {
          dst[u * 32 + (lane & 15)] = f2bf(acc[u][0][r]);
          dst[u * 32 + 16 + (lane & 15)] = f2bf(acc[u][1][r]);
        }
    }
  }
}

// f32 path: one 256-thread workgroup per (open row k, chunk of 256 vocabulary rows)
__global__ __launch_bounds__(256) void head_f32_kernel(HeadP p) {
  if (p.cont_dev && *p.cont_dev == 0) return;
  __shared__ int s_idx[DLM_MAX_ROWS];
  __shared__ float ev[256];
  __shared__ float red[4][3];
  __shared__ int redi[4];
  const int n_open = compact_open(p.committed, p.rows, s_idx);
  const int k = blockIdx.x / p.chunks_fixed, chunk = blockIdx.x % p.chunks_fixed;
  if (k >= n_open) return;
  const int row = s_idx[k];
  const float* h = (const float*)p.h + (size_t)row * p.d;
  const float* E = (const float*)p.E;
  const int per = (p.V + p.chunks_fixed - 1) / p.chunks_fixed;
  const int v0 = chunk * per, v1 = min(p.V, v0 + per);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  float rm = -INFINITY, rs = 0.f, rT = 0.f, bv = -INFINITY;
  int bi = 0x7fffffff;
  float pacc = 0.f;   // pe partial for d = tid (the host keeps d <= 256 on this path)
  for (int base = v0; base < v1; base += 256) {
    const int v = base + tid;
    float l = -INFINITY;
    if (v < v1) {
      float a = 0.f;
      for (int t = 0; t < p.d; ++t) a = fmaf(h[t], E[(size_t)v * p.d + t], a);
      l = a;
      if (p.logits_dbg) p.logits_dbg[(size_t)row * p.V + v] = l;
    }
    // block max and argmax
    float mx = l;
    int mi = v < v1 ? v : 0x7fffffff;
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(mx, o, 64);
      const int oi = __shfl_xor(mi, o, 64);
      if (ov > mx || (ov == mx && oi < mi)) { mx = ov; mi = oi; }
    }
    if (lane == 0) { red[w][0] = mx; redi[w] = mi; }
    __syncthreads();
    float tm = red[0][0];
    int ti = redi[0];
    for (int q = 1; q < 4; ++q)
      if (red[q][0] > tm || (red[q][0] == tm && redi[q] < ti)) { tm = red[q][0]; ti = redi[q]; }
    __syncthreads();
    if (tm > bv || (tm == bv && ti < bi)) { bv = tm; bi = ti; }
    const float mn = fmaxf(rm, tm);
    const float al = rs > 0.f ? expf(rm - mn) : 0.f;
    const float e = v < v1 ? expf(l - mn) : 0.f;
    const float te0 = v < v1 ? e * (l - mn) : 0.f;
    const float se = wave_sum(e), te = wave_sum(te0);
    if (lane == 0) { red[w][1] = se; red[w][2] = te; }
    ev[tid] = e;
    __syncthreads();
    const float S = ((red[0][1] + red[1][1]) + red[2][1]) + red[3][1];
    const float T = ((red[0][2] + red[1][2]) + red[2][2]) + red[3][2];
    rT = rs > 0.f ? al * (rT + (rm - mn) * rs) + T : T;
    rs = al * rs + S;
    rm = mn;
    // pe partial: this thread owns d = tid (first pass only; d <= 256 enforced by host)
    if (tid < p.d) {
      float a = pacc * al;
      const int nv = min(256, v1 - base);
      for (int i = 0; i < nv; ++i) a = fmaf(ev[i], E[(size_t)(base + i) * p.d + tid], a);
      pacc = a;
    }
    __syncthreads();
  }
  float* st = p.st + ((size_t)chunk * p.rows_max + k) * 8;
  if (tid == 0) {
    st[ST_M] = rm;
    st[ST_S] = rs;
    st[ST_T] = rT;
    st[ST_BV] = bv;
    st[ST_BI] = __int_as_float(bi);
  }
  if (tid < p.d) p.pe_part[((size_t)chunk * p.rows_max + k) * p.d + tid] = pacc;
}

// combine: one workgroup (256 threads) per (output row, 256-wide d slice).  Thread c loads
// chunk c's statistics; the chunk statistics are merged with fixed-order tree reductions, and
// the pe partials are read 64 chunks at a time so the loads overlap.
__device__ inline float block_max(float v, float* red) {
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const float r = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return r;
}

__device__ inline float block_sum(float v, float* red) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const float r = ((red[0] + red[1]) + red[2]) + red[3];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(256) void head_combine_kernel(HeadP p, int bf16_path) {
  if (p.cont_dev && *p.cont_dev == 0) return;
  __shared__ int s_idx[DLM_MAX_ROWS];
  __shared__ float wts[256];
  __shared__ float red[4];
  __shared__ float redv[4];
  __shared__ int redi[4];
  const int n_open = compact_open(p.committed, p.rows, s_idx);
  const int dblocks = (p.d + 255) / 256;
  const int row = blockIdx.x / dblocks, db = blockIdx.x % dblocks;
  const int tid = threadIdx.x;
  const bool open = p.committed == nullptr || p.committed[row] == 0;
  const int dcol = db * 256 + tid;
  if (!open) {
    if (db == 0 && tid == 0) {
      p.lse[row] = 0.f;
      p.ent[row] = 0.f;
      p.maxp[row] = 0.f;
      p.amax[row] = -1;
    }
    if (p.pe && dcol < p.d) p.pe[(size_t)row * p.d + dcol] = 0.f;
    return;
  }
  const int k = __popcll(open_mask(p.committed, p.rows) & ((1ull << row) - 1ull));   // open rows before row
  const int n_groups = (n_open + 15) / 16;
  const int CH = bf16_path ? n_chunks_for(n_groups, 0) : p.chunks_fixed;
  float cm = -INFINITY, cs = 0.f, ct = 0.f, cbv = -INFINITY;
  int cbi = 0x7fffffff;
  if (tid < CH) {
    const float* st = p.st + ((size_t)tid * p.rows_max + k) * 8;
    cm = st[ST_M];
    cs = st[ST_S];
    ct = st[ST_T];
    cbv = st[ST_BV];
    cbi = __float_as_int(st[ST_BI]);
  }
  const float M = block_max(cm, red);
  const float f = cs > 0.f ? expf(cm - M) : 0.f;
  const float S = block_sum(f * cs, red);
  const float T = block_sum(cs > 0.f ? f * (ct + (cm - M) * cs) : 0.f, red);
  // argmax over chunks: largest value, lowest id on ties
  float bv = cbv;
  int bi = cbi;
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
  }
  if ((tid & 63) == 0) { redv[tid >> 6] = bv; redi[tid >> 6] = bi; }
  __syncthreads();
  if (db == 0 && tid == 0) {
    float fbv = redv[0];
    int fbi = redi[0];
    for (int q = 1; q < 4; ++q)
      if (redv[q] > fbv || (redv[q] == fbv && redi[q] < fbi)) { fbv = redv[q]; fbi = redi[q]; }
    const float lnS = logf(S);
    p.lse[row] = M + lnS;
    p.ent[row] = lnS - T / S;
    p.maxp[row] = 1.0f / S;
    p.amax[row] = (fbi >= 0 && fbi < p.V) ? fbi : 0;   // all-NaN rows still name a valid id
  }
  if (!p.pe) return;
  wts[tid] = tid < CH ? f / S : 0.f;     // 256 threads: every slot, zero past the chunks
  __syncthreads();
  if (dcol < p.d) {
    // branch-free buffer loads (chunks past CH read zeros; the host keeps the partial area
    // below 2^31 bytes)
    const int es = bf16_path ? 2 : 4;                // partial element bytes
    const __amdgpu_buffer_rsrc_t pr = make_rsrc(p.pe_part, (uint32_t)((size_t)CH * p.rows_max * p.d * es));
    const uint32_t off0 = (uint32_t)(((size_t)k * p.d + dcol) * es), cstride = (uint32_t)(p.rows_max * p.d * es);
    float a = 0.f;
    constexpr int NB = 64;     // partial loads in flight per thread
    for (int c0 = 0; c0 < CH; c0 += NB) {
      float v[NB];
      if (bf16_path) {
#pragma unroll
        for (int j = 0; j < NB; ++j)
          v[j] = bf2f(__builtin_amdgcn_raw_buffer_load_b16(
              pr, c0 + j < CH ? (int)(off0 + (uint32_t)(c0 + j) * cstride) : (int)0x80000000, 0, 0));
      } else {
#pragma unroll
        for (int j = 0; j < NB; ++j)
          v[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
              pr, c0 + j < CH ? (int)(off0 + (uint32_t)(c0 + j) * cstride) : (int)0x80000000, 0, 0));
      }
#pragma unroll
      for (int j = 0; j < NB; ++j) a = fmaf(wts[c0 + j], v[j], a);     // c0 + j < 256
    }
    p.pe[(size_t)row * p.d + dcol] = a;
  }
}

}  // namespace

size_t head_ws_bytes(int dtype, int rows, int d, int V) {
  (void)V;
  const int CH = dtype == DLM_BF16 ? 256 : 16;
  return align_up((size_t)CH * rows * 8 * 4, 256) + align_up((size_t)CH * rows * d * 4, 256);
}

int head_launch(int dtype, const void* h, const void* E, const uint8_t* committed, int rows, int d,
                int V, float* lse, float* ent, float* maxp, int32_t* amax, float* pe,
                float* logits_dbg, void* ws, const int32_t* cont_dev, hipStream_t st) {
  HeadP p;
  p.h = (const uint16_t*)h;
  p.E = (const uint16_t*)E;
  p.committed = committed;
  p.rows = rows;
  p.d = d;
  p.V = V;
  p.rows_max = rows;
  const int CH = dtype == DLM_BF16 ? 256 : 16;
  p.st = (float*)ws;
  p.pe_part = (float*)((char*)ws + align_up((size_t)CH * rows * 8 * 4, 256));
  p.logits_dbg = logits_dbg;
  p.chunks_fixed = dtype == DLM_BF16 ? 0 : 16;
  p.lse = lse;
  p.ent = ent;
  p.maxp = maxp;
  p.amax = amax;
  p.pe = pe;
  p.cont_dev = cont_dev;
  if (dtype == DLM_BF16) {
    if ((size_t)V * d * 2 >= (1ull << 31)) return fail(DLM_ERR_SHAPE, "head: embedding of %d x %d too large", V, d);
    if ((size_t)CH * rows * d * 4 >= (1ull << 31)) return fail(DLM_ERR_SHAPE, "head: %d rows of %d too large", rows, d);
    const int grid = 256;   // n_groups * chunks <= 256, extra workgroups exit
    const int k8 = (d / 32 + 7) / 8;     // k-steps per wave with 8 waves
    const bool dbg = logits_dbg != nullptr;
    if (k8 <= 10) {
      switch (k8) {
#define HEAD_CASE(K)                                                                                    \
  case K:                                                                                               \
    if (dbg) hipLaunchKernelGGL((head_bf16_kernel<K, 8, true>), dim3(grid), dim3(512), 0, st, p);       \
    else hipLaunchKernelGGL((head_bf16_kernel<K, 8, false>), dim3(grid), dim3(512), 0, st, p);          \
    break;
        HEAD_CASE(1) HEAD_CASE(2) HEAD_CASE(3) HEAD_CASE(4) HEAD_CASE(5) HEAD_CASE(6) HEAD_CASE(7)
        HEAD_CASE(8) HEAD_CASE(9) HEAD_CASE(10)
#undef HEAD_CASE
        default: break;
      }
    } else {
      const int k16 = (d / 32 + 15) / 16;
      if (k16 > 8) return fail(DLM_ERR_SHAPE, "head: d=%d too large", d);
      if (dbg) hipLaunchKernelGGL((head_bf16_kernel<8, 16, true>), dim3(grid), dim3(1024), 0, st, p);
      else hipLaunchKernelGGL((head_bf16_kernel<8, 16, false>), dim3(grid), dim3(1024), 0, st, p);
    }
  } else {
    hipLaunchKernelGGL(head_f32_kernel, dim3(rows * 16), dim3(256), 0, st, p);
  }
  hipLaunchKernelGGL(head_combine_kernel, dim3(rows * ((d + 255) / 256)), dim3(256), 0, st, p,
                     dtype == DLM_BF16 ? 1 : 0);
  return check_hip(hipGetLastError(), "head launch");
}

}  // namespace dlm

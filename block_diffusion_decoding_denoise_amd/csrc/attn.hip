// Block attention: B block queries attend to the L prefix keys and all B block keys,
// with no mask (a denoising round predicts the block's unresolved positions together,
// page "ORL: diffusion LLMs get a learnable 'tokens per forward'", section "What shipped").
//
// The V cache is stored transposed in 32-key blocks, [kv head][cap/32][D][32], so that 8
// consecutive keys of one value column are one 16-byte load and a 32-key tile of V^T is one
// contiguous run.
//
// bf16 path.  One workgroup per (query head, key split).  Its 4 waves take every 4th 32-key
// tile of the split and run independently, with no LDS in the loop: K and V^T come straight
// from global memory (L2-shared by the query heads of one kv head, whose workgroups are placed
// on one XCD).  Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_16x16x32_bf16;
// the K rows fed to the MFMA are permuted so that lane l ends up owning one query (l % 16) and
// the 8 consecutive keys 8(l/16) .. +7 of each 32-key tile.  The online-softmax statistics
// therefore stay in the lane (two xor shuffles finish a row) and the probabilities are
// already the B operand of O^T = V^T P^T, whose A operand is one 16-byte load of V^T (the
// keys' order inside an MFMA's contraction is a free permutation shared by both operands).  The 4 waves' results
// are merged in LDS in wave order; with one split the normalised output is written directly,
// otherwise each split writes (O, running max, running sum) and a combine kernel merges the
// splits in index order.  Deterministic throughout.
#include "attn.h"

#include <algorithm>
#include <type_traits>

namespace dlm {

namespace {

// Optional per-workgroup timestamps for kernel studies (compiled out unless defined).
#ifndef DLM_TRACE_POINT
#define DLM_TRACE_POINT(i)
#endif

constexpr int TK = 32;          // keys per tile
constexpr int kMaxSplits = 32;  // key splits per kv head

// Query block j (of nqb; j > 0 only with B = 32) holds rows 32 j .. 32 j + B - 1 of q and out,
// sits at positions L + 32 j .. and attends to keys [0, L + 32 j + B): with two blocks, the
// first is a committed block whose keys the second one also sees.
struct AttnP {
  const uint16_t* q;            // [nqb 32, hq, D]
  const uint16_t* k;            // [hkv, cap, D]
  const uint16_t* v;            // V cache, [hkv][cap/32][D][32] (vt_index)
  uint16_t* out;                // [nqb 32, hq, D] (or packed, 32-row panels)
  uint16_t* part_o;             // [nqb][hkv][ns][G][32][D] bf16: each split's normalised output
  float* part_ml;               // [nqb][hkv][ns][G][32][2]
  int hq, hkv, B, nqb, cap, chunk, nsplit_max, out_packed;
  float scale_log2;             // softmax scale * log2(e) (times the key scale of an FP8 cache)
  float v_scale;                // value scale of an FP8 cache
  const int32_t* len_dev;
  int len_host;
  const int32_t* cont_dev;
};

// Keys per split for N keys over at most nsplit_max splits: the smallest multiple of one
// pass (PT tiles of 32 keys) that needs no more splits, so short prefixes use few splits and
// long ones spread over all of them.
constexpr int PT = 2;           // tiles per pass
__device__ inline int split_chunk(int N, int nsplit_max) {
  const int unit = PT * TK;
  return ((N + nsplit_max * unit - 1) / (nsplit_max * unit)) * unit;
}

// One workgroup per (kv head, group of WPG query heads, key split); wave w serves query head
// WPG hg + w of the group.  The split is processed in passes of PT 32-key tiles: the tiles'
// K and V^T are loaded once per workgroup (non-temporal buffer loads into registers, then LDS,
// double-buffered, the next pass in flight while this one is computed) and shared by the
// waves.  Per pass each wave forms the scores of all PT tiles (independent MFMA chains), takes
// one online-softmax step over the pass and adds P V.
// Two waves per SIMD (at most 256 registers per lane): the compiler fits the 4-wave form in
// 228 without spills, so two workgroups share a CU; left to itself it takes 288.
// KV8: the caches hold FP8 e4m3 codes (same layouts, one byte per element).  A pass then
// loads half the bytes, and the codes are widened to bf16 (exactly: every e4m3 value is a
// bf16 value) on their way into LDS, so everything after the LDS write is the bf16 path; the
// key scale is folded into the softmax scale and the value scale into the output.
__device__ inline u32x4_t e4m3x8_to_bf16(u32x2_t x) {
  u32x4_t r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[0], 1.0f, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[0], 1.0f, true));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[1], 1.0f, false));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[1], 1.0f, true));
  return r;
}

template <int D, int WPG, bool KV8 = false>
__global__ __launch_bounds__(64 * WPG) __attribute__((amdgpu_waves_per_eu(2))) void attn_bf16_kernel(AttnP p) {
  DLM_TRACE_POINT(0);
  if (p.cont_dev && *p.cont_dev == 0) return;
  constexpr int DS = D / 32;    // d-steps of the score MFMA
  constexpr int DB = D / 16;    // dv blocks of the output
  constexpr int NT = 64 * WPG;
  // LDS tile: K rows of 2D bytes padded by 16 (the rows a lane group reads land on distinct
  // banks), V^T rows of 32 keys (64 bytes) padded by 16
  constexpr int KROW = 2 * D + 16, VROW = 64 + 16;
  constexpr int KBYTES = TK * KROW, VBYTES = D * VROW, TBYTES = KBYTES + VBYTES;
  constexpr int KC = TK * D / 8 / NT, VC = D * 4 / NT;     // 16-byte chunks per thread and tile
  static_assert(KC >= 1 && VC >= 1 && KC * NT == TK * D / 8 && VC * NT == D * 4, "tile split");
  __shared__ __attribute__((aligned(16))) uint8_t smem[2][PT][TBYTES];
  const int G = p.hq / p.hkv;
  const int HG = G / WPG;
  const int per_qb = p.hkv * HG * p.nsplit_max;
  const int qblk = blockIdx.x / per_qb, bx = blockIdx.x % per_qb;
  const int s = bx % p.nsplit_max, gh = bx / p.nsplit_max;
  const int g = gh / HG, hg = gh % HG;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = WPG * hg + w;                // query head within the kv head's group
  const int head = g * G + hl;
  // Q fragments (B operand): lane l: query 16qb + l%16, d = 32ds + 8(l/16) .. +8; requested
  // before the prefix length is known (queries past B read zeros)
  u32x4_t qf[2][DS];
  {
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(p.q, (uint32_t)(32 * p.nqb * p.hq * D * 2));
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qi = 16 * qb + (lane & 15);
      const uint32_t qo = (uint32_t)((((32 * qblk + qi) * p.hq + head) * D + 8 * (lane >> 4)) * 2);
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) qf[qb][ds] = bload16(qr, qi < p.B ? qo + (uint32_t)ds * 64u : 0x80000000u);
    }
  }
  const int L = (p.len_dev ? *p.len_dev : p.len_host) + 32 * qblk;
  const int N = min(L + p.B, p.cap);
  const int chunk = split_chunk(N, p.nsplit_max);
  const int nsplit = (N + chunk - 1) / chunk;
  if (s >= nsplit) return;
  DLM_TRACE_POINT(1);
  const int c0 = s * chunk, c1 = min(N, c0 + chunk);
  const int npass = (c1 - c0 + PT * TK - 1) / (PT * TK);
  // buffer descriptors: K rows past c1 read as zeros; V^T tiles stay inside this head's
  // [cap/32][D][32] block (a tile wholly past c1 is not loaded; keys past c1 inside a tile are
  // masked after the LDS read)
  constexpr int ES = KV8 ? 1 : 2;                          // cache bytes per element
  const __amdgpu_buffer_rsrc_t kr = make_rsrc((const uint8_t*)p.k + (size_t)g * p.cap * D * ES, (uint32_t)c1 * D * ES);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc((const uint8_t*)p.v + (size_t)g * D * p.cap * ES, (uint32_t)D * p.cap * ES);
  const int lg = lane >> 4;                                // lane group: keys 8lg .. 8lg+7

  // global -> register staging of one pass (PT tiles; KC + VC chunks of 8 elements per thread
  // each: 16 bytes, or 8 for an FP8 cache)
  typedef typename std::conditional<KV8, u32x2_t, u32x4_t>::type chunk_t;
  chunk_t stk[PT][KC], stv[PT][VC];
  auto ld = [&](__amdgpu_buffer_rsrc_t r, uint32_t off) -> chunk_t {
    if constexpr (KV8) return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 2));
    else return bload16_nt(r, off);
  };
  auto widen = [&](chunk_t x) -> u32x4_t {
    if constexpr (KV8) return e4m3x8_to_bf16(x);
    else return x;
  };
  auto fetch = [&](int t0) {
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const int tu = t0 + u * TK;
      const bool in = tu < c1;
#pragma unroll
      for (int j = 0; j < KC; ++j) {
        const int c = tid + NT * j, key = c / (D / 8), col = c % (D / 8);
        stk[u][j] = ld(kr, in ? (uint32_t)(((tu + key) * D + col * 8) * ES) : 0x80000000u);
      }
#pragma unroll
      for (int j = 0; j < VC; ++j) {
        const int c = tid + NT * j, dv = c >> 2, part = c & 3;
        stv[u][j] = ld(vr, in ? (uint32_t)((((tu >> 5) * D + dv) * 32 + part * 8) * ES) : 0x80000000u);
      }
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      uint8_t* sk = smem[buf][u];
      uint8_t* sv = smem[buf][u] + KBYTES;
#pragma unroll
      for (int j = 0; j < KC; ++j) {
        const int c = tid + NT * j, key = c / (D / 8), col = c % (D / 8);
        *(u32x4_t*)(sk + key * KROW + col * 16) = widen(stk[u][j]);
      }
#pragma unroll
      for (int j = 0; j < VC; ++j) {
        const int c = tid + NT * j, dv = c >> 2, part = c & 3;
        *(u32x4_t*)(sv + dv * VROW + part * 16) = widen(stv[u][j]);
      }
    }
  };
  fetch(c0);

  f32x4_t o[DB][2];
#pragma unroll
  for (int b = 0; b < DB; ++b) o[b][0] = o[b][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float mrow[2] = {-INFINITY, -INFINITY}, lrow[2] = {0.f, 0.f};

  stash(0);
  if (npass > 1) fetch(c0 + PT * TK);
  __syncthreads();
  for (int ip = 0; ip < npass; ++ip) {
    const int p0 = c0 + ip * PT * TK;
    // scores of every tile of the pass.  K rows for score block kb: MFMA row i (= lane % 16)
    // takes key 8(i/4) + 4kb + i%4, so the result rows 4(l/16) + r of block kb are keys
    // 8(l/16) + 4kb + r; lane l ends up holding query 16qb + l%16.
    f32x4_t sc[PT][2][2];
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const uint8_t* sk = smem[ip & 1][u];
      u32x4_t kc[2][DS];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int i = lane & 15;
        const int key = 8 * (i >> 2) + 4 * kb + (i & 3);
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) kc[kb][ds] = *(const u32x4_t*)(sk + key * KROW + (32 * ds + 8 * lg) * 2);
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          f32x4_t a = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ds = 0; ds < DS; ++ds) a = mfma16x16x32(kc[kb][ds], qf[qb][ds], a);
          sc[u][kb][qb] = a;
        }
    }
    // one online-softmax step over the pass, per query (lane-resident), in log2 units
    u32x4_t pf[PT][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int u = 0; u < PT; ++u)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = p0 + u * TK + 8 * lg + 4 * kb + r;
            float v = sc[u][kb][qb][r] * p.scale_log2;
            v = key < c1 ? v : -INFINITY;
            sc[u][kb][qb][r] = v;
            mx = fmaxf(mx, v);
          }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mnew = fmaxf(mrow[qb], mx);
      const float alpha = __builtin_amdgcn_exp2f(mrow[qb] - mnew);
      float sum = 0.f;
#pragma unroll
      for (int u = 0; u < PT; ++u) {
        float pv[8];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float e = __builtin_amdgcn_exp2f(sc[u][kb][qb][r] - mnew);
            pv[4 * kb + r] = e;     // k-slot 4kb + r of lane group lg is key 8lg + 4kb + r
            sum += e;
          }
        u32x4_t pk;
#pragma unroll
        for (int i = 0; i < 4; ++i) pk[i] = pack2bf(pv[2 * i], pv[2 * i + 1]);
        pf[u][qb] = pk;
      }
      sum += __shfl_xor(sum, 16, 64);
      sum += __shfl_xor(sum, 32, 64);
      lrow[qb] = lrow[qb] * alpha + sum;
      mrow[qb] = mnew;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[b][qb][r] *= alpha;
    }
    // O^T[b][qb] += V^T[16b.., keys] P^T[keys, q]; V^T fragments (A operand): lane l: column
    // dv = 16b + l%16, keys 8lg .. +8 (keys past c1 zeroed: stale cache contents could be
    // non-finite)
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const uint8_t* sv = smem[ip & 1][u] + KBYTES;
      const int nvalid = min(8, max(0, c1 - (p0 + u * TK + 8 * lg)));
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        u32x4_t vc = *(const u32x4_t*)(sv + (16 * b + (lane & 15)) * VROW + 16 * lg);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          vc[jj] &= (2 * jj < nvalid ? 0x0000ffffu : 0u) | (2 * jj + 1 < nvalid ? 0xffff0000u : 0u);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) o[b][qb] = mfma16x16x32(vc, pf[u][qb], o[b][qb]);
      }
    }
    if (ip == 0) DLM_TRACE_POINT(2);
    // the next pass's registers go to the other buffer (last read in the previous pass, which
    // every wave has finished), then the pass after it is requested
    if (ip + 1 < npass) {
      stash((ip + 1) & 1);
      if (ip + 2 < npass) fetch(p0 + 2 * PT * TK);
    }
    __syncthreads();
  }
  DLM_TRACE_POINT(3);
  // o[b][qb][r] = O^T[dv = 16b + 4(l/16) + r][query 16qb + l%16]
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qi = 16 * qb + (lane & 15);
    if (qi >= p.B) continue;
    const float inv = (KV8 ? p.v_scale : 1.0f) / lrow[qb];
    if (nsplit == 1) {
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        const int dv = 16 * b + 4 * (lane >> 4);
        u32x2_t pk;
        pk[0] = pack2bf(o[b][qb][0] * inv, o[b][qb][1] * inv);
        pk[1] = pack2bf(o[b][qb][2] * inv, o[b][qb][3] * inv);
        // 4 consecutive columns are 8 contiguous bytes in both layouts
        const int qr = 32 * qblk + qi;
        const size_t oi = p.out_packed ? xpk_index_m(qr, head * D + dv, p.hq * D) : ((size_t)qr * p.hq + head) * D + dv;
        *(u32x2_t*)(p.out + oi) = pk;
      }
    } else {
      // the split's normalised output (bf16) and its (max, sum)
      const size_t row = ((((size_t)qblk * p.hkv + g) * p.nsplit_max + s) * G + hl) * 32 + qi;
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        u32x2_t pk;
        pk[0] = pack2bf(o[b][qb][0] * inv, o[b][qb][1] * inv);
        pk[1] = pack2bf(o[b][qb][2] * inv, o[b][qb][3] * inv);
        *(u32x2_t*)(p.part_o + row * D + 16 * b + 4 * (lane >> 4)) = pk;
      }
      if ((lane >> 4) == 0) {
        p.part_ml[row * 2 + 0] = mrow[qb];
        p.part_ml[row * 2 + 1] = lrow[qb];
      }
    }
  }
  DLM_TRACE_POINT(4);
}

// merge the splits of (head, query): D / 4 threads per (query block, head, query), each
// holding 4 output columns (one 8-byte load per split), 256 threads per workgroup; all partial
// loads are issued before the arithmetic (at most kMaxSplits splits); splits added in index order
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnP p) {
  if (p.cont_dev && *p.cont_dev == 0) return;
  constexpr int TPQ = D / 4, PPW = 256 / TPQ;     // threads per (head, query), pairs per workgroup
  const int pair = blockIdx.x * PPW + threadIdx.x / TPQ;
  const int dv = 4 * (threadIdx.x % TPQ);
  const int qblk = pair / (p.hq * p.B), bx = pair % (p.hq * p.B);
  if (qblk >= p.nqb) return;
  const int L = (p.len_dev ? *p.len_dev : p.len_host) + 32 * qblk;
  const int N = min(L + p.B, p.cap);
  const int chunk = split_chunk(N, p.nsplit_max);
  const int nsplit = (N + chunk - 1) / chunk;
  if (nsplit <= 1) return;      // the attention kernel wrote the output itself
  const int head = bx / p.B, qi = bx % p.B;
  const int G = p.hq / p.hkv;
  const int g = head / G, hh = head % G;
  constexpr int MAXS = kMaxSplits;
  // branch-free loads: split slots past nsplit use out-of-range buffer offsets (zeros)
  const size_t nrow = (size_t)p.nqb * p.hkv * p.nsplit_max * G * 32;
  const __amdgpu_buffer_rsrc_t mr = make_rsrc(p.part_ml, (uint32_t)(nrow * 8));
  const __amdgpu_buffer_rsrc_t orr = make_rsrc(p.part_o, (uint32_t)(nrow * D * 2));
  float mv[MAXS], lv[MAXS];
  u32x2_t ov[MAXS];
#pragma unroll
  for (int s = 0; s < MAXS; ++s) {
    const size_t row = ((((size_t)qblk * p.hkv + g) * p.nsplit_max + s) * G + hh) * 32 + qi;
    const bool ok = s < nsplit;
    const u32x2_t mlv = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(mr, ok ? (int)(row * 8) : (int)0x80000000, 0, 0));
    mv[s] = ok ? __uint_as_float(mlv[0]) : -INFINITY;
    lv[s] = __uint_as_float(mlv[1]);
    ov[s] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(orr, ok ? (int)((row * D + dv) * 2) : (int)0x80000000, 0, 0));
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < MAXS; ++s) M = fmaxf(M, mv[s]);
  float num[4] = {0.f, 0.f, 0.f, 0.f}, den = 0.f;
#pragma unroll
  for (int s = 0; s < MAXS; ++s) {
    const float f = mv[s] == -INFINITY ? 0.f : lv[s] * exp2f(mv[s] - M);   // split weight
    num[0] += f * lo_bf(ov[s][0]);
    num[1] += f * hi_bf(ov[s][0]);
    num[2] += f * lo_bf(ov[s][1]);
    num[3] += f * hi_bf(ov[s][1]);
    den += f;
  }
  const int qr = 32 * qblk + qi;
  const size_t o = p.out_packed ? xpk_index_m(qr, head * D + dv, p.hq * D) : ((size_t)qr * p.hq + head) * D + dv;
  // 4 consecutive columns are 8 contiguous bytes in both layouts
  *(u32x2_t*)(p.out + o) = u32x2_t{pack2bf(num[0] / den, num[1] / den), pack2bf(num[2] / den, num[3] / den)};
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

size_t attn_ws_bytes(int hq, int hkv, int D, AttnPlan pl, int nqb) {
  const int G = hq / hkv;
  const size_t po = (size_t)nqb * hkv * pl.nsplit_max * G * 32 * D * 2;
  const size_t pm = (size_t)nqb * hkv * pl.nsplit_max * G * 32 * 2 * 4;
  return align_up(po, 256) + align_up(pm, 256);
}

int attn_bf16(const void* q, const void* k, const void* v, void* out, int hq, int hkv, int D,
              int B, int nqb, int cap, float scale, const int32_t* len_dev, int len_host,
              const int32_t* cont_dev, AttnPlan pl, void* ws, int out_packed, hipStream_t st, AttnKv kvf) {
  if (nqb < 1 || nqb > 2 || (nqb == 2 && B != 32))
    return fail(DLM_ERR_SHAPE, "attention: one query block, or two of 32 rows");
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
  const int WPG = G < 4 ? G : 4;
  if (G % WPG || (WPG != 1 && WPG != 2 && WPG != 4))
    return fail(DLM_ERR_SHAPE, "attention: query heads per kv head must be 1, 2 or a multiple of 4");
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

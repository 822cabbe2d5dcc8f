// Block attention building blocks shared by the attention op (attn.hip) and the fused
// attention sublayer (layer.hip): the split loop of one workgroup and the split combine of
// one output item.  See attn.hip for the design.
#pragma once
#include <type_traits>

#include "common.h"

namespace dlm {

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
// long ones spread over all of them.  The split count is then ceil(N / chunk); the passes are
// dealt to the splits in turn (pass j to split j % nsplit), so a split holds chunk keys or
// fewer, interleaved, and its first pass does not depend on N.
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

// Lane exchanges across 16-lane rows by the gfx950 permlane swaps, in the VALU rather than
// through LDS.  Given one value in both operands, permlane16_swap returns rows (x0, x0, x2, x2)
// and (x1, x1, x3, x3), so combining its two results gives every lane the combination of its
// row pair (lanes l and l ^ 16); permlane32_swap likewise pairs the wave's halves (l ^ 32).
// Both lanes of a pair compute the same combination in the same operand order.
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One split (key range s of query block qblk of kv head g, query-head group hg) by the WPG
// waves of the calling workgroup; smem: LDS of at least attn_smem_bytes<D, WPG>() bytes.
// COH: q and the K/V tiles were written earlier in the same kernel by other compute units of
// this XCD, so they are read with L1-bypassing (sc1) loads, which see the XCD's L2.
template <int D, int WPG>
constexpr int attn_smem_bytes() {
  return 2 * PT * (TK * (2 * D + 16) + D * (64 + 16));
}

// hook: called once by every thread when the split's first two passes are in flight (or, for a
// workgroup without a split, when it knows it has none): loads it issues then queue behind them.
struct NoHook {
  __device__ __forceinline__ void operator()() const {}
};

template <int D, int WPG, bool KV8, bool COH, typename Hook = NoHook>
__device__ __forceinline__ void attn_split_body(const AttnP& p, int qblk, int g, int hg, int s, uint8_t* smem_base,
                                                Hook hook = Hook()) {
  constexpr int DS = D / 32;    // d-steps of the score MFMA
  constexpr int DB = D / 16;    // dv blocks of the output
  constexpr int NT = 64 * WPG;
  // LDS tile: K rows of 2D bytes padded by 16 (the rows a lane group reads land on distinct
  // banks), V^T rows of 32 keys (64 bytes) padded by 16
  constexpr int KROW = 2 * D + 16, VROW = 64 + 16;
  constexpr int KBYTES = TK * KROW, VBYTES = D * VROW, TBYTES = KBYTES + VBYTES;
  constexpr int KC = TK * D / 8 / NT, VC = D * 4 / NT;     // 16-byte chunks per thread and tile
  static_assert(KC >= 1 && VC >= 1 && KC * NT == TK * D / 8 && VC * NT == D * 4, "tile split");
  auto smem = [&](int buf, int u) -> uint8_t* { return smem_base + (buf * PT + u) * TBYTES; };
  const int G = p.hq / p.hkv;
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
      for (int ds = 0; ds < DS; ++ds)
        qf[qb][ds] = __builtin_amdgcn_raw_buffer_load_b128(qr, (int)(qi < p.B ? qo + (uint32_t)ds * 64u : 0x80000000u),
                                                           0, COH ? 16 : 0);
    }
  }
  // buffer descriptors over this head's whole cache (K [cap][D], V^T [cap/32][D][32]); keys
  // past the N visible ones are masked after the LDS read, and tiles wholly past N are not
  // loaded once N is known (kend)
  constexpr int ES = KV8 ? 1 : 2;                          // cache bytes per element
  const __amdgpu_buffer_rsrc_t kr = make_rsrc((const uint8_t*)p.k + (size_t)g * p.cap * D * ES, (uint32_t)p.cap * D * ES);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc((const uint8_t*)p.v + (size_t)g * D * p.cap * ES, (uint32_t)D * p.cap * ES);
  const int lg = lane >> 4;                                // lane group: keys 8lg .. 8lg+7

  // global -> register staging of one pass (PT tiles; KC + VC chunks of 8 elements per thread
  // each: 16 bytes, or 8 for an FP8 cache)
  typedef typename std::conditional<KV8, u32x2_t, u32x4_t>::type chunk_t;
  chunk_t stk[PT][KC], stv[PT][VC];
  auto ld = [&](__amdgpu_buffer_rsrc_t r, uint32_t off) -> chunk_t {
    constexpr int aux = COH ? 18 : 2;      // non-temporal (and L1-bypassing when COH)
    if constexpr (KV8) return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, aux));
    else return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, aux);
  };
  auto widen = [&](chunk_t x) -> u32x4_t {
    if constexpr (KV8) return e4m3x8_to_bf16(x);
    else return x;
  };
  int kend = p.cap;
  auto fetch = [&](int t0) {
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const int tu = t0 + u * TK;
      const bool in = tu < kend;
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
      uint8_t* sk = smem(buf, u);
      uint8_t* sv = smem(buf, u) + KBYTES;
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
  // Pass j (keys [PT TK j, PT TK (j + 1))) of the prefix and block belongs to split j % nsplit,
  // so this split's first pass is pass s whatever the prefix length: it is requested before
  // the length is read.
  fetch(s * PT * TK);
  const int L = (p.len_dev ? *p.len_dev : p.len_host) + 32 * qblk;
  const int N = min(L + p.B, p.cap);
  const int chunk = split_chunk(N, p.nsplit_max);
  const int nsplit = (N + chunk - 1) / chunk;
  if (s >= nsplit) {
    hook();
    return;
  }
  DLM_TRACE_POINT(1);
  kend = N;
  const int P = (N + PT * TK - 1) / (PT * TK);
  const int npass = (P - s + nsplit - 1) / nsplit;        // passes s, s + nsplit, ...

  f32x4_t o[DB][2];
#pragma unroll
  for (int b = 0; b < DB; ++b) o[b][0] = o[b][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float mrow[2] = {-INFINITY, -INFINITY}, lrow[2] = {0.f, 0.f};

  stash(0);
  if (npass > 1) fetch((s + nsplit) * PT * TK);
  hook();
  __syncthreads();
  for (int ip = 0; ip < npass; ++ip) {
    const int p0 = (s + ip * nsplit) * PT * TK;
    // scores of every tile of the pass.  K rows for score block kb: MFMA row i (= lane % 16)
    // takes key 8(i/4) + 4kb + i%4, so the result rows 4(l/16) + r of block kb are keys
    // 8(l/16) + 4kb + r; lane l ends up holding query 16qb + l%16.
    f32x4_t sc[PT][2][2];
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const uint8_t* sk = smem(ip & 1, u);
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
            v = key < N ? v : -INFINITY;
            sc[u][kb][qb][r] = v;
            mx = fmaxf(mx, v);
          }
      mx = max_xor32(max_xor16(mx));
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
      sum = sum_xor32(sum_xor16(sum));
      lrow[qb] = lrow[qb] * alpha + sum;
      mrow[qb] = mnew;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[b][qb][r] *= alpha;
    }
    // O^T[b][qb] += V^T[16b.., keys] P^T[keys, q]; V^T fragments (A operand): lane l: column
    // dv = 16b + l%16, keys 8lg .. +8 (keys past N zeroed: stale cache contents could be
    // non-finite)
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const uint8_t* sv = smem(ip & 1, u) + KBYTES;
      const int nvalid = min(8, max(0, N - (p0 + u * TK + 8 * lg)));
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
      if (ip + 2 < npass) fetch(p0 + 2 * nsplit * PT * TK);
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
// One (query block, head, query, 4 columns) output of the split combine.  COH: the partials
// were written earlier in the same kernel (L1-bypassing loads).
template <int D, bool COH>
__device__ __forceinline__ void attn_combine_item(const AttnP& p, int qblk, int head, int qi, int dv) {
  const int L = (p.len_dev ? *p.len_dev : p.len_host) + 32 * qblk;
  const int N = min(L + p.B, p.cap);
  const int chunk = split_chunk(N, p.nsplit_max);
  const int nsplit = (N + chunk - 1) / chunk;
  if (nsplit <= 1) return;      // the attention kernel wrote the output itself
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
    const u32x2_t mlv = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(mr, ok ? (int)(row * 8) : (int)0x80000000, 0, COH ? 16 : 0));
    mv[s] = ok ? __uint_as_float(mlv[0]) : -INFINITY;
    lv[s] = __uint_as_float(mlv[1]);
    ov[s] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(orr, ok ? (int)((row * D + dv) * 2) : (int)0x80000000, 0, COH ? 16 : 0));
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

}  // namespace dlm

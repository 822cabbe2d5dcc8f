// Block attention: B block queries attend to the L prefix keys and all B block keys,
// with no mask (a denoising round predicts the block's unresolved positions together,
// page "ORL: diffusion LLMs get a learnable 'tokens per forward'", section "What shipped").
//
// The V cache is stored transposed, [kv head, D, cap], so that 8 consecutive keys of one value
// column are one 16-byte load.
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

namespace dlm {

namespace {

constexpr int TK = 32;          // keys per tile

struct AttnP {
  const uint16_t* q;            // [B, hq, D]
  const uint16_t* k;            // [hkv, cap, D]
  const uint16_t* v;            // V^T cache [hkv, D, cap]
  uint16_t* out;                // [B, hq, D]
  float* part_o;                // [hkv][ns][G][32][D]
  float* part_ml;               // [hkv][ns][G][32][2]
  int hq, hkv, B, cap, chunk, nsplit_max, out_packed;
  float scale_log2;             // softmax scale * log2(e)
  const int32_t* len_dev;
  int len_host;
  const int32_t* cont_dev;
};

template <int D>
__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(AttnP p) {
  if (p.cont_dev && *p.cont_dev == 0) return;
  constexpr int DS = D / 32;    // d-steps of the score MFMA
  constexpr int DB = D / 16;    // dv blocks of the output
  __shared__ float red_o[4][D][33];
  __shared__ float wm[4][32], wl[4][32];
  const int L = p.len_dev ? *p.len_dev : p.len_host;
  const int N = min(L + p.B, p.cap);
  const int nsplit = min((N + p.chunk - 1) / p.chunk, p.nsplit_max);
  const int G = p.hq / p.hkv;
  // workgroup -> (kv head g, split s, query head hh in the group); the G query heads of one
  // (g, s) share an XCD (workgroup ids are dealt round-robin to the 8 XCDs)
  int g, s, hh;
  {
    const int b = blockIdx.x, xcd = b & 7, j = b >> 3;
    hh = j % G;
    const int u = (j / G) * 8 + xcd;
    g = u / p.nsplit_max;
    s = u % p.nsplit_max;
    if (g >= p.hkv) return;
  }
  if (s >= nsplit) return;
  const int head = g * G + hh;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c0 = s * p.chunk, c1 = min(N, c0 + p.chunk);
  // buffer descriptors: K rows past c1 read as zeros; V^T reads stay inside this head's
  // [D][cap] block (the keys past c1 inside it are masked after the load)
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(p.k + (size_t)g * p.cap * D, (uint32_t)c1 * D * 2u);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(p.v + (size_t)g * D * p.cap, (uint32_t)D * p.cap * 2u);
  const int lg = lane >> 4;                                // lane group: keys 8lg .. 8lg+7

  // Q fragments (B operand): lane l: query 16qb + l%16, d = 32ds + 8(l/16) .. +8
  u32x4_t qf[2][DS];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qi = 16 * qb + (lane & 15);
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
      qf[qb][ds] = qi < p.B ? ld16(p.q + ((size_t)qi * p.hq + head) * D + 32 * ds + 8 * (lane >> 4))
                            : u32x4_t{0u, 0u, 0u, 0u};
  }
  f32x4_t o[DB][2];
#pragma unroll
  for (int b = 0; b < DB; ++b) o[b][0] = o[b][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float mrow[2] = {-INFINITY, -INFINITY}, lrow[2] = {0.f, 0.f};

  // K rows for score block kb: MFMA row i (= lane % 16) takes key 8(i/4) + 4kb + i%4, so the
  // result rows 4(l/16) + r of block kb are keys 8(l/16) + 4kb + r.  V^T fragments (A operand
  // of O^T = V^T P^T): lane l: column dv = 16b + l%16, keys 8lg .. +8.  The next tile of this
  // wave is loaded while the current one is computed (buffer loads: past the ends they read
  // zeros or in-bounds data that is masked).
  u32x4_t kf[2][DS], vf[DB];
  auto load_tile = [&](int t0, u32x4_t (&kt)[2][DS], u32x4_t (&vt)[DB]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int i = lane & 15;
      const int key = t0 + 8 * (i >> 2) + 4 * kb + (i & 3);
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) kt[kb][ds] = bload16(kr, (uint32_t)(key * D + 32 * ds + 8 * (lane >> 4)) * 2u);
    }
#pragma unroll
    for (int b = 0; b < DB; ++b) vt[b] = bload16(vr, (uint32_t)((16 * b + (lane & 15)) * p.cap + t0 + 8 * lg) * 2u);
  };
  load_tile(c0 + w * TK, kf, vf);
  for (int t0 = c0 + w * TK; t0 < c1; t0 += 4 * TK) {
    u32x4_t kn[2][DS], vn[DB];
    load_tile(t0 + 4 * TK, kn, vn);
    // keys kv0 .. kv0+7 past c1 are zeroed (their probabilities are zero too, but stale cache
    // contents could be non-finite): a per-lane mask of the valid 16-bit halves
    const int kv0 = t0 + 8 * lg;
    const int nvalid = min(8, max(0, c1 - kv0));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t msk = (2 * j < nvalid ? 0x0000ffffu : 0u) | (2 * j + 1 < nvalid ? 0xffff0000u : 0u);
#pragma unroll
      for (int b = 0; b < DB; ++b) vf[b][j] &= msk;
    }
    // scores S^T[kb][qb]: lane l holds keys 8(l/16) + 4kb + r for query 16qb + l%16
    f32x4_t sc[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        f32x4_t a = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) a = mfma16x16x32(kf[kb][ds], qf[qb][ds], a);
        sc[kb][qb] = a;
      }
    // online softmax per query (lane-resident), in log2 units
    u32x4_t pf[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = t0 + 8 * lg + 4 * kb + r;
          float v = sc[kb][qb][r] * p.scale_log2;
          v = key < c1 ? v : -INFINITY;
          sc[kb][qb][r] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mnew = fmaxf(mrow[qb], mx);
      const float alpha = exp2f(mrow[qb] - mnew);
      float pv[8];
      float sum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = exp2f(sc[kb][qb][r] - mnew);
          pv[4 * kb + r] = e;     // k-slot 4kb + r of lane group lg is key 8lg + 4kb + r
          sum += e;
        }
      sum += __shfl_xor(sum, 16, 64);
      sum += __shfl_xor(sum, 32, 64);
      lrow[qb] = lrow[qb] * alpha + sum;
      mrow[qb] = mnew;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[b][qb][r] *= alpha;
      u32x4_t pk;
#pragma unroll
      for (int i = 0; i < 4; ++i) pk[i] = (uint32_t)f2bf(pv[2 * i]) | ((uint32_t)f2bf(pv[2 * i + 1]) << 16);
      pf[qb] = pk;
    }
    // O^T[b][qb] += V^T[16b.., keys] P^T[keys, q]
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) o[b][qb] = mfma16x16x32(vf[b], pf[qb], o[b][qb]);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) kf[kb][ds] = kn[kb][ds];
#pragma unroll
    for (int b = 0; b < DB; ++b) vf[b] = vn[b];
  }
  // merge the 4 waves: common max per query, each wave's O rescaled to it and published in
  // LDS, then every output summed over the waves in wave order
  if (lane < 16) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      wm[w][16 * qb + lane] = mrow[qb];
      wl[w][16 * qb + lane] = lrow[qb];
    }
  }
  __syncthreads();
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qi = 16 * qb + (lane & 15);
    const float M = fmaxf(fmaxf(wm[0][qi], wm[1][qi]), fmaxf(wm[2][qi], wm[3][qi]));
    const float sw = mrow[qb] == -INFINITY ? 0.f : exp2f(mrow[qb] - M);
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) red_o[w][16 * b + 4 * (lane >> 4) + r][qi] = o[b][qb][r] * sw;
  }
  __syncthreads();
  // thread -> (query, 8 consecutive value columns)
  for (int e = tid; e < 32 * (D / 8); e += 256) {
    const int qi = e % 32, dv0 = (e / 32) * 8;
    if (qi >= p.B) continue;
    const float M = fmaxf(fmaxf(wm[0][qi], wm[1][qi]), fmaxf(wm[2][qi], wm[3][qi]));
    float Ls = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) Ls += wm[ww][qi] == -INFINITY ? 0.f : wl[ww][qi] * exp2f(wm[ww][qi] - M);
    float val[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      val[j] = ((red_o[0][dv0 + j][qi] + red_o[1][dv0 + j][qi]) + red_o[2][dv0 + j][qi]) + red_o[3][dv0 + j][qi];
    if (nsplit == 1) {
      const float inv = 1.0f / Ls;
      u32x4_t pk;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        pk[j] = (uint32_t)f2bf(val[2 * j] * inv) | ((uint32_t)f2bf(val[2 * j + 1] * inv) << 16);
      const size_t oi = p.out_packed ? xpk_index(qi, head * D + dv0) : ((size_t)qi * p.hq + head) * D + dv0;
      *(u32x4_t*)(p.out + oi) = pk;   // 8 consecutive columns are 16 contiguous bytes in both layouts
    } else {
      const size_t row = (((size_t)g * p.nsplit_max + s) * G + hh) * 32 + qi;
#pragma unroll
      for (int j = 0; j < 8; ++j) p.part_o[row * D + dv0 + j] = val[j];
      if (dv0 == 0) {
        p.part_ml[row * 2 + 0] = M;
        p.part_ml[row * 2 + 1] = Ls;
      }
    }
  }
}

// merge the splits of (head, query): one workgroup per (head, query), D threads; all partial
// loads are issued before the arithmetic (at most 16 splits)
template <int D>
__global__ __launch_bounds__(D) void attn_combine_kernel(AttnP p) {
  if (p.cont_dev && *p.cont_dev == 0) return;
  const int L = p.len_dev ? *p.len_dev : p.len_host;
  const int N = min(L + p.B, p.cap);
  const int nsplit = min((N + p.chunk - 1) / p.chunk, p.nsplit_max);
  if (nsplit <= 1) return;      // the attention kernel wrote the output itself
  const int head = blockIdx.x / p.B, qi = blockIdx.x % p.B;
  const int G = p.hq / p.hkv;
  const int g = head / G, hh = head % G;
  const int dv = threadIdx.x;
  constexpr int MAXS = 16;
  float mv[MAXS], lv[MAXS], ov[MAXS];
#pragma unroll
  for (int s = 0; s < MAXS; ++s) {
    const size_t row = (((size_t)g * p.nsplit_max + s) * G + hh) * 32 + qi;
    const bool ok = s < nsplit;
    mv[s] = ok ? p.part_ml[row * 2] : -INFINITY;
    lv[s] = ok ? p.part_ml[row * 2 + 1] : 0.f;
    ov[s] = ok ? p.part_o[row * D + dv] : 0.f;
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < MAXS; ++s) M = fmaxf(M, mv[s]);
  float num = 0.f, den = 0.f;
#pragma unroll
  for (int s = 0; s < MAXS; ++s) {
    const float f = mv[s] == -INFINITY ? 0.f : exp2f(mv[s] - M);
    num += f * ov[s];
    den += f * lv[s];
  }
  const size_t o = p.out_packed ? xpk_index(qi, head * D + dv) : ((size_t)qi * p.hq + head) * D + dv;
  p.out[o] = f2bf(num / den);
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
  const float* vb = p.v + (size_t)g * p.D * p.cap;   // V^T: [D][cap]
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
    for (int t = 0; t < p.D; ++t) acc[t] = fmaf(e, vb[(size_t)t * p.cap + j], acc[t]);
  }
  den = wave_sum(den);
  for (int t = 0; t < p.D; ++t) {
    const float num = wave_sum(acc[t]);
    if (lane == 0) p.out[((size_t)qi * p.hq + head) * p.D + t] = num / den;
  }
}

}  // namespace

AttnPlan attn_plan(int hq, int hkv, int D, int B, int max_len) {
  (void)hq; (void)D; (void)B;
  AttnPlan pl;
  const int N = max_len + B;
  // chunk: multiple of 32 keys, at least 256, at most 32 splits per kv head
  // chunk: a multiple of 4 tiles of 32 keys (one tile per wave and round), at most 16 splits
  int chunk = 128;
  while ((N + chunk - 1) / chunk > 16) chunk += 128;
  pl.chunk = chunk;
  pl.nsplit_max = (N + chunk - 1) / chunk;
  (void)hkv;
  return pl;
}

size_t attn_ws_bytes(int hq, int hkv, int D, AttnPlan pl) {
  const int G = hq / hkv;
  const size_t po = (size_t)hkv * pl.nsplit_max * G * 32 * D * 4;
  const size_t pm = (size_t)hkv * pl.nsplit_max * G * 32 * 2 * 4;
  return align_up(po, 256) + align_up(pm, 256);
}

int attn_bf16(const void* q, const void* k, const void* v, void* out, int hq, int hkv, int D,
              int B, int cap, float scale, const int32_t* len_dev, int len_host,
              const int32_t* cont_dev, AttnPlan pl, void* ws, int out_packed, hipStream_t st) {
  AttnP p;
  p.out_packed = out_packed;
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.out = (uint16_t*)out;
  const int G = hq / hkv;
  const size_t po = (size_t)hkv * pl.nsplit_max * G * 32 * D * 4;
  p.part_o = (float*)ws;
  p.part_ml = (float*)((char*)ws + align_up(po, 256));
  p.hq = hq;
  p.hkv = hkv;
  p.B = B;
  p.cap = cap;
  p.chunk = pl.chunk;
  p.nsplit_max = pl.nsplit_max;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.len_dev = len_dev;
  p.len_host = len_host;
  p.cont_dev = cont_dev;
  const int units = hkv * pl.nsplit_max;
  const int grid = ((units + 7) / 8) * 8 * G;
  if (D == 128) {
    hipLaunchKernelGGL(attn_bf16_kernel<128>, dim3(grid), dim3(256), 0, st, p);
    hipLaunchKernelGGL(attn_combine_kernel<128>, dim3(hq * B), dim3(128), 0, st, p);
  } else {
    hipLaunchKernelGGL(attn_bf16_kernel<64>, dim3(grid), dim3(256), 0, st, p);
    hipLaunchKernelGGL(attn_combine_kernel<64>, dim3(hq * B), dim3(64), 0, st, p);
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

// Block attention: B block queries attend to the L prefix keys and all B block keys,
// with no mask (a denoising round predicts the block's unresolved positions together,
// page "ORL: diffusion LLMs get a learnable 'tokens per forward'", section "What shipped").
//
// bf16 path.  One workgroup per (kv head, key split); its 4 waves are the q heads of that
// kv head (grouped-query attention), so every K/V tile is read from HBM once per split and
// shared through LDS.  Scores are computed transposed, S^T = K Q^T, with
// v_mfma_f32_16x16x32_bf16: lane l then owns one query (l % 16) and 8 keys of every
// 32-key tile, so the online-softmax statistics stay in the lane (two xor shuffles finish
// a row) and the probabilities are already the B operand of O^T = V^T P^T (the keys'
// order inside an MFMA's contraction is a free permutation shared by both operands).  V
// is staged transposed in LDS for that product.  Each split writes an unnormalised
// partial (O, running max, running sum); a combine kernel merges the splits in index
// order (deterministic) and rounds to bf16.
#include "attn.h"

namespace dlm {

namespace {

constexpr int TK = 32;          // keys per tile
constexpr int KPAD = 8;         // bf16 padding of a K row in LDS
constexpr int VPAD = 8;         // bf16 padding of a V^T row in LDS

struct AttnP {
  const uint16_t* q;            // [B, hq, D]
  const uint16_t* k;            // [hkv, cap, D]
  const uint16_t* v;
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
__global__ __launch_bounds__(256) void attn_bf16_kernel(AttnP p) {
  if (p.cont_dev && *p.cont_dev == 0) return;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[TK][D + KPAD];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D][TK + VPAD];
  const int L = p.len_dev ? *p.len_dev : p.len_host;
  const int N = min(L + p.B, p.cap);
  const int nsplit = min((N + p.chunk - 1) / p.chunk, p.nsplit_max);
  const int g = blockIdx.x / p.nsplit_max, s = blockIdx.x % p.nsplit_max;
  if (s >= nsplit) return;
  const int G = p.hq / p.hkv;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int c0 = s * p.chunk, c1 = min(N, c0 + p.chunk);
  const uint16_t* kbase = p.k + (size_t)g * p.cap * D;
  const uint16_t* vbase = p.v + (size_t)g * p.cap * D;
  constexpr int DS = D / 32;    // d-steps of the score MFMA
  constexpr int DB = D / 16;    // dv blocks of the output

  for (int hh0 = 0; hh0 < G; hh0 += 4) {
    const int hh = hh0 + w;
    const bool active = hh < G;
    const int head = g * G + (active ? hh : 0);
    // Q fragments (B operand): lane l: query 16qb + l%16, d = 32ds + 8(l/16) .. +8
    u32x4_t qf[2][DS];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qi = 16 * qb + (lane & 15);
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        if (qi < p.B)
          qf[qb][ds] = ld16(p.q + ((size_t)qi * p.hq + head) * D + 32 * ds + 8 * (lane >> 4));
        else
          qf[qb][ds] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
    f32x4_t o[DB][2];
#pragma unroll
    for (int b = 0; b < DB; ++b) o[b][0] = o[b][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float mrow[2] = {-INFINITY, -INFINITY}, lrow[2] = {0.f, 0.f};

    for (int t0 = c0; t0 < c1; t0 += TK) {
      __syncthreads();
      // cooperative tile load: 32 keys x D for K and V
      for (int e = tid; e < TK * D / 8; e += 256) {
        const int key = e / (D / 8), d8 = (e % (D / 8)) * 8;
        const int gk = t0 + key;
        u32x4_t kv = u32x4_t{0u, 0u, 0u, 0u}, vv = u32x4_t{0u, 0u, 0u, 0u};
        if (gk < c1) {
          kv = ld16(kbase + (size_t)gk * D + d8);
          vv = ld16(vbase + (size_t)gk * D + d8);
        }
        *(u32x4_t*)&Ks[key][d8] = kv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          Vt[d8 + 2 * i][key] = (uint16_t)(vv[i] & 0xffffu);
          Vt[d8 + 2 * i + 1][key] = (uint16_t)(vv[i] >> 16);
        }
      }
      __syncthreads();
      if (!active) continue;
      // scores S^T[kb][qb]: lane l holds keys 16kb + 4(l/16) + r for query 16qb + l%16
      f32x4_t sc[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        u32x4_t kf[DS];
#pragma unroll
        for (int ds = 0; ds < DS; ++ds)
          kf[ds] = *(const u32x4_t*)&Ks[16 * kb + (lane & 15)][32 * ds + 8 * (lane >> 4)];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          f32x4_t a = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ds = 0; ds < DS; ++ds) a = mfma16x16x32(kf[ds], qf[qb][ds], a);
          sc[kb][qb] = a;
        }
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
            const int key = t0 + 16 * kb + 4 * (lane >> 4) + r;
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
            pv[4 * kb + r] = e;
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
        for (int i = 0; i < 4; ++i)
          pk[i] = (uint32_t)f2bf(pv[2 * i]) | ((uint32_t)f2bf(pv[2 * i + 1]) << 16);
        pf[qb] = pk;
      }
      // O^T[b][qb] += V^T[16b.., keys] P^T[keys, q]: k-slot (g, e) -> key 4g+e (e<4), 16+4g+e-4
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        const int dv = 16 * b + (lane & 15);
        const int kg = 4 * (lane >> 4);
        const u32x2_t lo = *(const u32x2_t*)&Vt[dv][kg];
        const u32x2_t hi = *(const u32x2_t*)&Vt[dv][16 + kg];
        const u32x4_t vf = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) o[b][qb] = mfma16x16x32(vf, pf[qb], o[b][qb]);
      }
    }
    if (!active) continue;
    // partial out: o[b][qb][r] is dv = 16b + 4(l/16) + r, query 16qb + l%16
    const size_t pbase = (((size_t)g * p.nsplit_max + s) * G + hh) * 32;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qi = 16 * qb + (lane & 15);
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) p.part_o[(pbase + qi) * D + 16 * b + 4 * (lane >> 4) + r] = o[b][qb][r];
      if (lane < 16) {
        p.part_ml[(pbase + qi) * 2 + 0] = mrow[qb];
        p.part_ml[(pbase + qi) * 2 + 1] = lrow[qb];
      }
    }
  }
}

// merge the splits of (head, query): one workgroup per (head, query), D threads
template <int D>
__global__ __launch_bounds__(D) void attn_combine_kernel(AttnP p) {
  if (p.cont_dev && *p.cont_dev == 0) return;
  const int L = p.len_dev ? *p.len_dev : p.len_host;
  const int N = min(L + p.B, p.cap);
  const int nsplit = min((N + p.chunk - 1) / p.chunk, p.nsplit_max);
  const int head = blockIdx.x / p.B, qi = blockIdx.x % p.B;
  const int G = p.hq / p.hkv;
  const int g = head / G, hh = head % G;
  const int dv = threadIdx.x;
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s)
    M = fmaxf(M, p.part_ml[(((((size_t)g * p.nsplit_max + s) * G + hh) * 32) + qi) * 2]);
  float num = 0.f, den = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const size_t row = (((size_t)g * p.nsplit_max + s) * G + hh) * 32 + qi;
    const float f = exp2f(p.part_ml[row * 2] - M);
    num += f * p.part_o[row * D + dv];
    den += f * p.part_ml[row * 2 + 1];
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
  const float* vb = p.v + (size_t)g * p.cap * p.D;
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
    for (int t = 0; t < p.D; ++t) acc[t] = fmaf(e, vb[(size_t)j * p.D + t], acc[t]);
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
  int chunk = 256;
  while ((N + chunk - 1) / chunk > 32) chunk += 32;
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
  const int grid = hkv * pl.nsplit_max;
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

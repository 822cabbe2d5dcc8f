// Epilogue helpers of the skinny GEMMs (shared by the per-op kernels and the fused layer
// kernels): row orders of the fused matrices, RoPE with the K/V cache write, SwiGLU.
#pragma once
#include "gemm.h"

namespace dlm {

// ------------------------------------------------------------------ row maps
__host__ __device__ inline int qkv_logical(int prow, int hq, int hkv, int D) {
  const int Nq = hq * D, Nk = hkv * D;
  if (prow >= Nq + Nk) return prow;
  const int base = prow < Nq ? 0 : Nq;
  const int rel = prow - base;
  const int head = rel / D, within = rel % D;
  const int t = within / 32, r = within % 32;
  return base + head * D + 16 * t + r / 2 + (r % 2) * (D / 2);
}

__host__ __device__ inline int gu_logical(int prow, int F) {
  const int t = prow / 32, r = prow % 32;
  return (r % 2) * F + 16 * t + r / 2;
}

// ------------------------------------------------------------------ epilogues
__device__ inline int prefix_len(const EpiParams& e) {
  return e.len_dev ? *e.len_dev : e.len_host;
}

__device__ inline void store_act(void* base, size_t idx, float v, int bf16) {
  if (bf16) ((uint16_t*)base)[idx] = f2bf(v);
  else ((float*)base)[idx] = v;
}

// a K/V cache element: the stored (bf16 or f32) value, or for an FP8 cache the e4m3 code of
// the bf16 value divided by the cache scale (an IEEE single-precision quotient)
__device__ inline void store_kv(const EpiParams& e, void* base, size_t idx, float v, float scale) {
  if (e.kv8) ((uint8_t*)base)[idx] = (uint8_t)e4m3_code(bf2f(f2bf(v)) / scale);
  else store_act(base, idx, v, e.bf16_out);
}

__device__ inline float load_act(const void* base, size_t idx, int bf16) {
  return bf16 ? bf2f(((const uint16_t*)base)[idx]) : ((const float*)base)[idx];
}

// rotate-half RoPE of the pair (j, j + D/2) of a q (part 0) or k (part 1) head.  The angle
// pos * base^(-2j/D) is formed in double (base^(-2j/D) = r^j with r = base^(-2/D) from the
// host, by repeated squaring) and reduced to [-pi, pi] in double; only the final sine and
// cosine of the reduced angle are single precision.
__device__ inline double ipow(double r, int j) {
  double out = 1.0;
  while (j) {
    if (j & 1) out *= r;
    r *= r;
    j >>= 1;
  }
  return out;
}

__device__ inline void epi_qk_rope(const EpiParams& e, int m, int part, int head, int j, float a,
                                   float b) {
  const int L = prefix_len(e);
  const int pos = L + m;
  const double ang = (double)pos * ipow(e.rope_r, j);
  const double two_pi = 6.283185307179586476925286766559;
  const double red = fma(-rint(ang / two_pi), two_pi, ang);
  float sn, cs;
  __sincosf((float)red, &sn, &cs);
  const float a2 = a * cs - b * sn;
  const float b2 = b * cs + a * sn;
  if (part == 0) {
    const size_t o = (size_t)m * e.hq * e.D + (size_t)head * e.D + j;
    // (q rows are always in range; cache rows are guarded below)
    store_act(e.q_out, o, a2, e.bf16_out);
    store_act(e.q_out, o + e.D / 2, b2, e.bf16_out);
  } else {
    if (L + m >= e.cap) return;   // a prefix length past the cache capacity writes nothing
    const size_t o = ((size_t)head * e.cap + (L + m)) * e.D + j;
    store_kv(e, e.k_cache, o, a2, e.k_scale);
    store_kv(e, e.k_cache, o + e.D / 2, b2, e.k_scale);
  }
}

// the V cache is stored transposed in 32-key blocks (vt_index)
__device__ inline void epi_v(const EpiParams& e, int m, int rel, float v) {
  const int L = prefix_len(e);
  if (L + m >= e.cap) return;
  const int head = rel / e.D, j = rel % e.D;
  store_kv(e, e.v_cache, vt_index(head, e.D, e.cap, L + m, j), v, e.v_scale);
}

__device__ inline void epi_swiglu(const EpiParams& e, int m, int j, float g, float u) {
  const float s = g / (1.0f + expf(-g));
  store_act(e.act_out, e.bf16_out ? xpk_index_m(m, j, e.F) : (size_t)m * e.F + j, s * u, e.bf16_out);
}

}  // namespace dlm

// Internal helpers shared by the library's translation units (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string>

#include "../../include/dlm.h"

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

#define DLM_WAVE 64

// ---------------------------------------------------------------- bf16 <-> f32
__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// round-to-nearest-even (the hardware conversion, v_cvt_pk_bf16_f32); NaN stays NaN
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
// two values, a in the low half
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2bf(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

__device__ __forceinline__ float lo_bf(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ---------------------------------------------------------------- MFMA wrappers
// 16x16x32 bf16 -> f32.  Lane l holds a[e] = A[l%16][8*(l/16)+e], b[e] = B[8*(l/16)+e][l%16];
// result lane l holds D[4*(l/16)+r][l%16] (r = 0..3).
__device__ __forceinline__ f32x4_t mfma16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
// 16x16x16 bf16 -> f32.  Lane l holds a[e] = A[l%16][4*(l/16)+e], b[e] = B[4*(l/16)+e][l%16].
__device__ __forceinline__ f32x4_t mfma16x16x16(u32x2_t a, u32x2_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a),
                                                   __builtin_bit_cast(i16x4_t, b), c, 0, 0, 0);
}

// 32x32x16 bf16 -> f32.  Lane l holds a[e] = A[l%32][8*(l/32)+e], b[e] = B[8*(l/32)+e][l%32];
// result lane l holds D[8*(r/4) + 4*(l/32) + r%4][l%32] (r = 0..15).
__device__ __forceinline__ f32x16_t mfma32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------- FP8 e4m3 (OCP)
// e4m3 code (OCP: bias 7, 3 mantissa bits, largest 448, subnormal step 2^-9) of v rounded to
// nearest, ties to even, saturating at 448; NaN gives the NaN code 0x7F.
__device__ inline uint32_t e4m3_code(float v) {
  if (v != v) return 0x7Fu;
  const uint32_t sign = v < 0.f ? 0x80u : 0u;
  const float a = fabsf(v);
  float q;
  if (a >= 448.f) {
    q = 448.f;
  } else {
    int ex;
    frexpf(a, &ex);
    const int E = a > 0.f ? max(ex - 1, -6) : -6;
    q = rintf(a * ldexpf(1.f, 3 - E)) * ldexpf(1.f, E - 3);    // exact power-of-two scalings
    q = fminf(q, 448.f);
  }
  if (q == 0.f) return sign;
  int ex;
  frexpf(q, &ex);
  const int E = ex - 1;
  if (E < -6) return sign | (uint32_t)(q * 512.f);                                   // subnormal
  return sign | ((uint32_t)(E + 7) << 3) | (uint32_t)(q * ldexpf(1.f, 3 - E) - 8.f);
}

// ---------------------------------------------------------------- buffer loads
// Raw buffer loads: an offset at or beyond num_records returns zeros without touching memory,
// so a prefetch ring can run past the end of a range with no branches.
#define DLM_RSRC_WORD3 0x00020000
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, DLM_RSRC_WORD3);
}
__device__ __forceinline__ u32x4_t bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}
__device__ __forceinline__ u32x4_t bload16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2);
}

// ---------------------------------------------------------------- memory helpers
__device__ __forceinline__ u32x4_t ld16_nt(const void* p) {
  return __builtin_nontemporal_load((const u32x4_t*)p);
}
__device__ __forceinline__ u32x4_t ld16(const void* p) { return *(const u32x4_t*)p; }

// Cross-workgroup hand-off without whole-cache maintenance.  An agent-scope release or
// acquire fence on gfx950 writes back or invalidates the XCD's entire L2, which costs tens of
// microseconds when hundreds of workgroups do it.  Instead the data handed over is stored and
// loaded with agent-scope (coherent, L2-bypassing) accesses, each thread waits for its own
// stores to complete (s_waitcnt 0) before the workgroup barrier, and only then one thread
// bumps the agent-scope counter; the reader loads after observing the counter.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0); }
__device__ __forceinline__ int atomic_add_agent(int* p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// wave-wide reductions (all 64 lanes return the result)
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// ---------------------------------------------------------------- packed activations
// bf16 activations that feed a skinny GEMM (the B operand, 32 rows x K) are stored in the
// matrix-core operand order: for 16-column step kt, lane l's 8 values are
// X[l % 32][16 kt + 8 (l / 32) .. +8], and the 64 lanes' 16 bytes form one contiguous 1 KiB
// run.  Element (m, k) of the 32-row block lives at this index.
__host__ __device__ __forceinline__ size_t xpk_index(int m, int k) {
  return ((size_t)(k >> 4) * 64 + m + 32 * ((k >> 3) & 1)) * 8 + (k & 7);
}
// More than 32 rows (K columns) are stored as consecutive 32-row panels of that order.
__host__ __device__ __forceinline__ size_t xpk_index_m(int m, int k, int K) {
  return (size_t)(m >> 5) * 32 * K + xpk_index(m & 31, k);
}

// ---------------------------------------------------------------- V cache layout
// The V cache of a kv head is stored transposed in 32-key blocks: [cap / 32][D][32], so that
// a 32-key tile of V^T (the A operand of the attention's P V product, keys contiguous) is one
// contiguous D x 64-byte run.  Element (key t, column j) of kv head h:
__host__ __device__ __forceinline__ size_t vt_index(int h, int D, int cap, int t, int j) {
  return (((size_t)h * (cap >> 5) + (t >> 5)) * D + j) * 32 + (t & 31);
}

// ---------------------------------------------------------------- host side
namespace dlm {
void set_error(const char* fmt, ...);
int fail(int code, const char* fmt, ...);
int check_hip(hipError_t e, const char* what);
bool device_ok();
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
}  // namespace dlm

#define DLM_REQUIRE(cond, code, ...) \
  do { if (!(cond)) return dlm::fail((code), __VA_ARGS__); } while (0)
#define DLM_HIP(call) \
  do { hipError_t e_ = (call); if (e_ != hipSuccess) return dlm::check_hip(e_, #call); } while (0)

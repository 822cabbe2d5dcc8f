// XCD-local synchronisation of the workgroups of one launch -- internal interface.
//
// The chip's 256 compute units sit in 8 XCDs of 32, each with its own L2, and the dispatcher
// deals the workgroups of a launch to the XCDs round-robin, so workgroups b and b + 8 share an
// XCD.  Which XCD group b % 8 lands on rotates from launch to launch (the round-robin goes on
// where the previous launch ended), so every launch that relies on the grouping checks it with
// the XCC_ID hardware register.  The workgroups of one group then meet at an L2 atomic counter
// (about 1.2 us), and data one of them stored before the meeting is read by the others with
// L1-bypassing (sc1) loads, which the XCD's L2 serves.
//
// Sync words (err, 9 x 128 bytes, zero before the first use): word 0 holds flags (bit 0: a
// barrier wait gave up; bit 1: a workgroup ran off its group's XCD), word 32 (1 + x) the XCC id
// group x ran on in the last launch.  Barrier counters (bar, 64 words per group, zero before the
// first use) only grow: each of the group's kWgPerXcd workgroups adds one per barrier.
#pragma once
#include "common.h"

namespace dlm {

constexpr int kXcds = 8;
constexpr int kWgPerXcd = 32;
constexpr long kSpinLimit = 1L << 22;    // about 0.4 s of polling: then flag and go on

__device__ __forceinline__ unsigned xcc_id() {
  return __builtin_amdgcn_s_getreg((20) | (0 << 6) | ((4 - 1) << 11)) & 0xfu;   // HW_REG_XCC_ID[3:0]
}

// Workgroup 0 of group x stores its XCC id before the group's first barrier; after it every
// workgroup compares its own (a group split over two XCDs would not pass the barrier, whose
// counter lives in one XCD's L2, and would set bit 0 instead); a mismatch sets bit 1.
__device__ __forceinline__ void publish_placement(int* err, int x, int w) {
  if (threadIdx.x == 0 && w == 0) err[32 * (1 + x)] = (int)xcc_id();
}

__device__ __forceinline__ void check_placement(int* err, int x) {
  if (threadIdx.x == 0) {
    const int pub = (int)__builtin_amdgcn_raw_buffer_load_b32(make_rsrc(err, 9 * 128), 128 * (1 + x), 0, 16);
    if (pub != (int)xcc_id()) __hip_atomic_fetch_or(err, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// L1-bypassing loads of data written earlier in this kernel by another compute unit of the
// same XCD (served by the XCD's L2)
__device__ __forceinline__ u32x4_t ld16_xcd(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 16);
}

// Barrier of the kWgPerXcd workgroups of one group.  At each barrier the counter starts at a
// multiple of kWgPerXcd and the target is the next one.  Every wave waits for its own stores
// to reach L2 before the workgroup arrives; the arrival is an atomic at the XCD's L2 and the
// wait polls it with L1-bypassing loads.  A wait that gives up sets bit 0 of the error word;
// once it is set no barrier waits any more, so a broken placement costs one time-out, not one
// per barrier.
// issue: loads (prefetches of the next step's weights) that every thread issues after its
// own stores are complete and before the barrier wait, so that they stream while the
// workgroups of the XCD meet (vector memory operations complete in issue order, so a
// prefetch issued before the stores would hold up the arrival).
struct NoIssue {
  __device__ __forceinline__ void operator()() const {}
};

template <typename Issue = NoIssue>
__device__ __forceinline__ void xcd_sync(unsigned* ctr, int* err, Issue issue = Issue()) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  issue();
  if (threadIdx.x == 0) {
    const unsigned v = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    const unsigned target = (v & ~(unsigned)(kWgPerXcd - 1)) + (unsigned)kWgPerXcd;
    const bool failed = __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & 1;
    for (long i = 0; !failed; ++i) {
      const unsigned cur = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if ((int)(cur - target) >= 0) break;
      if (i > kSpinLimit) {
        __hip_atomic_fetch_or(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  __syncthreads();
}

}  // namespace dlm

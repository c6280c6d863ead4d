// xcd_sync.hpp -- barrier and data exchange between workgroups that share one XCD.
//
// MI355X has eight XCDs, each with its own L2; the L2s are not coherent with each other for
// ordinary accesses. Workgroups of one launch are dispatched round-robin over the XCDs, so
// workgroup ids w and w + 8k run on the same XCD (checked at run time through the hardware
// XCC id; a mismatch raises an error flag). Within one XCD the L2 is the point of coherence:
//   writer: plain stores, then s_waitcnt vmcnt(0) (stores have reached L2), then arrive;
//   barrier: relaxed device-scope atomic add on a counter in its own 256-byte line, spin with
//            device-scope loads until the target count, bounded by a spin limit;
//   reader: device-scope (sc1) loads, which do not hit in the per-CU L1.
// This avoids the L2 write-back / invalidate that agent-scope release / acquire fences need
// (measured at 16-35 us per barrier against ~1 us for this protocol).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttt {

constexpr int SYNC_LINE = 64;            // uint32 words per counter (256 bytes)
constexpr long SYNC_SPIN_LIMIT = 1l << 26;

__device__ __forceinline__ unsigned hw_xcc_id() {
  return __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 15;  // HW_REG_XCC_ID[3:0]
}

// All prior global stores of the calling thread have reached L2.
__device__ __forceinline__ void drain_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Barrier of `members` workgroups on counter `cnt` (all on one XCD). `target` = members * k
// for the k-th barrier since the counter was zeroed. Returns false on a spin timeout (the
// error word is incremented); callers then continue without the data guarantee.
__device__ inline bool xcd_barrier(unsigned* cnt, unsigned target, unsigned* err) {
  drain_stores();
  __syncthreads();
  __shared__ int ok;
  if (threadIdx.x == 0) {
    ok = 1;
    __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    long spins = 0;
    while (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      if (++spins > SYNC_SPIN_LIMIT) {
        __hip_atomic_fetch_add(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ok = 0;
        break;
      }
    }
  }
  __syncthreads();
  return ok != 0;
}

// Load written by another workgroup of the same XCD (bypasses the per-CU L1).
__device__ __forceinline__ float xcd_load(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace ttt

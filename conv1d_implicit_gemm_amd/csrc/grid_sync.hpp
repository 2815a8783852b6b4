// Waits between the workgroups of one launch whose grid is resident at once.
//
// A group of workgroups (the tiles of one sample, or of one row block) meets
// on a 32-bit arrival counter in the caller's workspace, zeroed before the
// launch by zero_u32_kernel (a fill kernel rather than a memset, so the call
// may be captured in a graph).  What the workgroups exchange is written with
// device-scope atomic stores and read with device-scope atomic loads: those
// reach the point of coherence of all XCDs, so no cache-wide flush is needed.
#pragma once

#include <cstdlib>

#include "common.hpp"

namespace c1g {
namespace {

// Polls before a barrier wait gives up: ~0.1 s, far beyond any legitimate
// wait.  The environment variable C1G_BARRIER_SPINS overrides it (read at each
// launch), which lets a test force the give-up path with every kernel still
// ending normally.
inline unsigned barrier_poll_limit() {
  const char* e = std::getenv("C1G_BARRIER_SPINS");
  if (e && *e) {
    char* end = nullptr;
    const unsigned long v = std::strtoul(e, &end, 10);
    if (end && *end == '\0' && v <= (1ul << 22)) return (unsigned)v;
  }
  return 1u << 22;
}

// sample_barrier: every thread of the workgroup returns once `expect`
// workgroups have arrived on *ctr (this one included).  Waits for this wave's outstanding memory
// operations first, so every store the workgroup issued before the call is
// visible to the others once they see its arrival.  The wait gives up after
// a bound no legitimate wait approaches (every workgroup of such a launch is
// resident), records that in *fault and returns false, so no
// path can hang; the caller then poisons what depended on the others.
// The two halves of the wait, for callers with work to issue in between
// (barrier_arrive, then barrier_wait); sample_barrier is both.
__device__ __forceinline__ void barrier_arrive(unsigned* ctr) {
  // This wave's stores are done: the hardware wait, and (memory clobber) no
  // store the compiler could otherwise sink past it.  Together with the
  // workgroup barrier below, every store of the workgroup has been
  // acknowledged before thread 0 publishes the arrival.  The stores other
  // workgroups read are device-scope atomic stores, acknowledged only once
  // they are at the point of coherence of all XCDs, and those workgroups read
  // them with device-scope atomic loads issued after they observed the count,
  // so no cache flush or invalidation is needed on either side.
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bool barrier_wait(unsigned* ctr, unsigned expect, unsigned* fault,
                                             unsigned max_polls) {
  __shared__ int complete;
  if (threadIdx.x == 0) {
    unsigned spins = 0;
    int ok = 1;
    while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < expect) {
      if (++spins > max_polls) {
        __hip_atomic_store(fault, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    complete = ok;
  }
  __syncthreads();
  return complete != 0;
}

__device__ __forceinline__ bool sample_barrier(unsigned* ctr, unsigned expect, unsigned* fault,
                                               unsigned max_polls) {
  barrier_arrive(ctr);
  return barrier_wait(ctr, expect, fault, max_polls);
}

__global__ void zero_u32_kernel(unsigned* p, int64_t count) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) p[i] = 0u;
}

}  // namespace
}  // namespace c1g

// sk_sync.h -- cross-workgroup hand-over of split partials (library-internal).
//
// A row block computed by several workgroups is finished by the last of them
// to arrive. The partials are the only data that cross workgroups (and XCDs,
// whose L2 caches are not coherent with each other) inside one launch, so only
// they use agent-coherent accesses: stores write through to the coherent
// memory side and loads read from it. No device-scope fence is needed, and
// none is used: on this GPU such a fence writes back and invalidates the
// whole L2 of the XCD, which costs every other workgroup its cached columns.
#pragma once

#include <hip/hip_runtime.h>

namespace sk {

__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// (M, S) pair of a partial, written as two coherent words.
__device__ __forceinline__ void store_coherent(float2* p, float2 v) {
  float* q = reinterpret_cast<float*>(p);
  store_coherent(q, v.x);
  store_coherent(q + 1, v.y);
}

// Arrival of this workgroup at a counter shared by `count` workgroups; true in
// every thread of the last one. The caller's partials must have been written
// with store_coherent: waiting for this thread's stores to complete makes them
// visible at the coherent level before the workgroup counts itself in, and the
// counter's atomic add is coherent across the device.
__device__ inline bool arrive_last(unsigned* counter, int count) {
  __shared__ int s_last;
  __builtin_amdgcn_s_waitcnt(0);  // all of this thread's memory operations complete
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = (__hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              (unsigned)(count - 1));
  __syncthreads();
  return s_last != 0;
}

}  // namespace sk

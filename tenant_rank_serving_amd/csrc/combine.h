// Fixed-order sums of partial results across work items of one launch.
// Included inside namespace dc, anonymous namespace, of the .hip files that
// use it.
//
// Work items that each produce a partial sum of the same outputs store it
// with device-coherent stores, wait until those stores have completed, and
// bump the outputs' arrival counter; the item that arrives last reads every
// partial back with device-coherent loads and adds them in item order, so
// the result does not depend on which item ran first.  Only these accesses
// bypass the per-XCD L2 caches; nothing writes back or invalidates a whole
// L2 (which a device-scope fence would).  Counters start at zero (cleared by
// the kernel before, in stream order).
#pragma once

__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// True in every thread of the block that arrives last of `total` blocks
// sharing `counter`.  Every thread of the block must call it.
__device__ __forceinline__ bool arrive_last(uint32_t* counter, int total, int* flag) {
  __builtin_amdgcn_s_waitcnt(0);   // this thread's partial stores have completed
  __syncthreads();
  if (threadIdx.x == 0)
    *flag = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(total - 1);
  __syncthreads();
  return *flag != 0;
}

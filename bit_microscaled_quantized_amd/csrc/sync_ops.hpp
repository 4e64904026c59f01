// Device-scope atomic operations for the workgroup exchanges of
// grid_sync.hpp, as the quantize kernels run them on gfx950.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// Device-scope atomics for the exchange.  It communicates only through the
// slot's atomics and device-coherent loads and stores, which gfx950 performs
// at the device's coherence point (past the per-XCD L2), so release and
// acquire need no cache maintenance: release waits until this wave's earlier
// memory operations have been performed (s_waitcnt), acquire keeps the
// compiler from moving the following loads above the one that observed the
// flag.  Agent-scope C++ fences would instead write back and invalidate the
// XCD's whole L2 in every workgroup, stalling the loads of the others on that
// XCD (measured: 80 instead of 19 us of load phase on an 84 MB tensor).
struct DeviceOps {
  static __device__ void drain() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
  static __device__ void max_relaxed(uint32_t* p, uint32_t v) {
    __hip_atomic_fetch_max(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  static __device__ uint32_t add_release(uint32_t* p, uint32_t v) {
    drain();
    const uint32_t old = __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    drain();
    return old;
  }
  static __device__ uint32_t load_relaxed(uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  static __device__ void store_relaxed(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  static __device__ void store_release(uint32_t* p, uint32_t v) {
    drain();
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // 64-bit compare-and-swap after this wave's earlier memory operations;
  // true if *p held `expected` (then it holds `desired`), else `expected` = *p
  static __device__ bool cas64(uint64_t* p, uint64_t& expected, uint64_t desired) {
    drain();
    const bool ok = __hip_atomic_compare_exchange_strong(p, &expected, desired, __ATOMIC_RELAXED,
                                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    drain();
    return ok;
  }
  static __device__ uint64_t exchange64(uint64_t* p, uint64_t v) {
    return __hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  static __device__ uint64_t exchange64_release(uint64_t* p, uint64_t v) {
    drain();
    return __hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  static __device__ void store64_relaxed(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  static __device__ uint64_t load64(uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  static __device__ void fence_acquire() { asm volatile("" ::: "memory"); }
  static __device__ void pause() { __builtin_amdgcn_s_sleep(8); }
};

}  // namespace nvfp4

// The barrier of an LDS ring that buffer loads fill directly (the matrix-core
// GEMMs and the router GEMM).
#pragma once
#include <hip/hip_runtime.h>

namespace moe {

// Barrier of an LDS ring filled by buffer loads that write LDS directly:
// vmcnt kVm (expcnt untouched) and lgkmcnt 0, then the workgroup barrier.
// Every wave has then received its own transfers up to the vmcnt and finished
// its LDS reads, so the stage the next transfers overwrite is free and the
// stage read next is complete for every wave.  No workgroup fence: the
// compiler counts LDS transfers as LDS writes and would wait for all of them,
// the ones issued steps ahead included.  The empty asm statements keep the
// compiler from moving memory accesses across the barrier.
template <int kVm>
__device__ __forceinline__ void ring_barrier() {
  static_assert(kVm >= 0 && kVm < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0070 | kVm);  // vmcnt kVm, expcnt 7, lgkmcnt 0
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

}  // namespace moe

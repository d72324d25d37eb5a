// Debug instrumentation, off in the normal build. Compiled with
// -DMODA_POISON_LDS=1 (the library's poisoned-LDS build), every kernel that uses
// LDS first fills it with 0x7fc07fc0, a NaN as fp32 and as each of two bf16
// halves: a read of LDS bytes that no write of the same workgroup preceded then
// turns the results into NaNs or changes them, which a comparison with the
// normal build (the kernels are deterministic) shows.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#ifndef MODA_POISON_LDS
#define MODA_POISON_LDS 0
#endif

namespace moda {

constexpr bool kPoisonLds = MODA_POISON_LDS != 0;

// Called by every thread of the workgroup at the kernel's start, before any
// other LDS access; a no-op in the normal build.
__device__ __forceinline__ void poison_lds(void* lds, int bytes) {
  if constexpr (kPoisonLds) {
    uint32_t* w = static_cast<uint32_t*>(lds);
    for (int i = threadIdx.x; i < bytes / 4; i += blockDim.x) w[i] = 0x7fc07fc0u;
    __syncthreads();
  }
}

}  // namespace moda

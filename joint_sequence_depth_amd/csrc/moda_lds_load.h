// Loads from memory straight into LDS (buffer loads with the LDS flag) and the
// wait immediate that goes with them; shared by the bf16 forward and the
// projection GEMM.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moda {

// s_waitcnt immediate: wait until at most n vector-memory loads are outstanding
// (gfx9 encoding: vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14; expcnt and
// lgkmcnt at their maximum, i.e. not waited for).
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource (raw, no stride): byte range [base, base + nrec); reads past it
// return zeros without touching memory.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t nrec) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = (int)(uint32_t)b;
  r[1] = (int)((uint32_t)(b >> 32) & 0xffffu);
  r[2] = (int)nrec;
  r[3] = 0x00020000;
  return r;
}

// One wave-wide 16-byte-per-lane load from memory straight into LDS: lane l reads
// bytes [voff, voff + 16) of the resource and writes them to LDS bytes
// [lds + 16 l, lds + 16 l + 16) (lds is uniform; the compiler puts it in M0).
// Written as inline assembly so that the compiler's wait insertion does not see
// an LDS write in flight and drain all loads before every later LDS read: the
// kernel waits for these loads itself (vector-memory loads complete in issue
// order, so the compiler's own waits for other loads only become more
// conservative).
__device__ __forceinline__ void load_to_lds16(uint32_t lds, uint32_t voff, i32x4 rsrc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) rsrc[i] = __builtin_amdgcn_readfirstlane(rsrc[i]);  // uniform: no-op when scalar
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds) : "memory");
}

}  // namespace moda

// Row-wise helpers shared by the kernels that lay a key row across a group of
// lanes (decode, the backward's depth and fp32 kernels): LPR = D / 8 lanes hold
// one row, 8 consecutive elements each, and sums over a row run across the group.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moda {
namespace rowops {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of LPR (8 or 16) lanes; every lane of a group ends with
// the same bits: swap neighbours, swap pairs, mirror within 8, mirror within 16.
template <int LPR>
__device__ __forceinline__ float group_sum(float s) {
  static_assert(LPR == 8 || LPR == 16, "groups of 8 or 16 lanes");
  s += dpp_mov<0xB1>(s);
  s += dpp_mov<0x4E>(s);
  s += dpp_mov<0x141>(s);
  if constexpr (LPR == 16) s += dpp_mov<0x140>(s);
  return s;
}

// One 16-byte load with the non-temporal hint: for streams read once (depth slots,
// a decode step's cache rows), so that they do not push data that is read again
// (a sequence's K/V blocks) out of L2.
__device__ __forceinline__ uint4 stream_load16(const void* p) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// 8 consecutive elements at element offset `elem` as fp32 (bf16 or fp32 storage).
template <bool BF16>
__device__ __forceinline__ void load8(const void* base, int64_t elem, float (&x)[8]) {
  if constexpr (BF16) {
    const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem);
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = __uint_as_float(u[j] << 16);
      x[2 * j + 1] = __uint_as_float(u[j] & 0xffff0000u);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem);
    const float4 a = p[0], b = p[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

// Two fp32 values to a bf16 pair (round to nearest even), low element first.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  const f2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// One 16-byte store with the non-temporal hint (for streams written once).
__device__ __forceinline__ void stream_store16(void* p, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = {a, b, c, d};
  __builtin_nontemporal_store(v, static_cast<u32x4*>(p));
}

// Stores n (4 or 8) consecutive fp32 values at element offset `elem`, as bf16 or
// fp32; NT: with the non-temporal hint (N = 8).
template <bool F32, int N, bool NT = false>
__device__ __forceinline__ void store_n(void* base, int64_t elem, const float* x) {
  static_assert(N == 4 || N == 8, "4 or 8 elements");
  static_assert(!NT || N == 8, "streaming stores of whole 16-byte words");
  if constexpr (F32 && NT) {
    float* p = static_cast<float*>(base) + elem;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      stream_store16(p + 4 * j, __float_as_uint(x[4 * j]), __float_as_uint(x[4 * j + 1]), __float_as_uint(x[4 * j + 2]),
                     __float_as_uint(x[4 * j + 3]));
  } else if constexpr (F32) {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(base) + elem);
#pragma unroll
    for (int j = 0; j < N / 4; ++j) p[j] = make_float4(x[4 * j], x[4 * j + 1], x[4 * j + 2], x[4 * j + 3]);
  } else if constexpr (NT) {
    stream_store16(static_cast<uint16_t*>(base) + elem, pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                   pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7]));
  } else if constexpr (N == 8) {
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + elem) =
        make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7]));
  } else {
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(base) + elem) =
        make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
  }
}

}  // namespace rowops
}  // namespace moda

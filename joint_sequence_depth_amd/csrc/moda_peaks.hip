// Attained-peak microbenchmarks: the rates this chip actually reaches on the two
// resources the MoDA forward is bound by, used as the denominators of the
// "fraction of attained peak" figures next to the published peaks.
//
//  * moda_peak_stream_read: every lane streams 16-byte non-temporal loads over a
//    buffer (grid-stride, several loads in flight per lane) and folds them into
//    one XOR per workgroup, the access pattern of the depth-KV stream without its
//    arithmetic.
//  * moda_peak_mfma_bf16: every wave issues back-to-back
//    v_mfma_f32_32x32x16_bf16 on register operands, four independent
//    accumulator chains, no memory traffic: the matrix-core rate the sequence
//    loop's products could reach.
//
// Both only measure rates; neither reads or writes outside the caller's buffers.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moda_peaks.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kReadUnroll = 8;  // 16-byte loads in flight per lane per round

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, int64_t n_vec,
                                                          uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (kReadUnroll - 1) * stride < n_vec; i += kReadUnroll * stride) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u];
  }
  for (; i < n_vec; i += stride) acc ^= __builtin_nontemporal_load(src + i);
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  // one value per workgroup keeps the loads live
  __shared__ uint32_t red[256];
  red[threadIdx.x] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int t = 0; t < (int)blockDim.x; ++t) r ^= red[t];
    sink[blockIdx.x] = r;
  }
}

__global__ __launch_bounds__(256) void mfma_loop_kernel(int32_t iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(0.001f * (float)(lane + j));
    b[j] = (__bf16)(0.002f * (float)(lane - j));
  }
  f32x16 c0, c1, c2, c3;
#pragma unroll
  for (int j = 0; j < 16; ++j) c0[j] = c1[j] = c2[j] = c3[j] = 0.f;
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) s += c0[j] + c1[j] + c2[j] + c3[j];
  if (s == 12345.678f) sink[blockIdx.x] = s;  // practically never: keeps the products live
}

}  // namespace

extern "C" {

int moda_peak_stream_read(const void* buf, int64_t bytes, void* sink, int32_t workgroups, void* stream) {
  if (!buf || !sink || bytes < 16 || (bytes & 15) || workgroups < 1 || (reinterpret_cast<uintptr_t>(buf) & 15))
    return 1;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)workgroups), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(buf), bytes / 16, static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

int moda_peak_mfma_bf16(int32_t iters, void* sink, int32_t workgroups, void* stream) {
  if (!sink || iters < 1 || workgroups < 1) return 1;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3((unsigned)workgroups), dim3(256), 0, static_cast<hipStream_t>(stream),
                     iters, static_cast<float*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

double moda_peak_mfma_flops_per_launch(int32_t iters, int32_t workgroups) {
  // 4 waves per workgroup, 4 products of 32 x 32 x 16 (2 flops per multiply-add) per iteration
  return (double)workgroups * 4.0 * iters * 4.0 * (2.0 * 32 * 32 * 16);
}

}  // extern "C"

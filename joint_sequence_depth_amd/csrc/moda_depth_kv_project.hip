// The FFN input's KV projection, written straight into one depth slot.
//
// MoDA deck, slide "Reuse attention KV; add a projection for FFN inputs" (paper
// Sec. 2.2): a layer keeps its attention KV for later layers and projects its FFN
// input into additional depth KV slots. For every token n:
//   k_depth[n, slot] = x_n W_k^T,  v_depth[n, slot] = x_n W_v^T   ([H_kv, d] each)
// with W = [W_k; W_v] of shape [2 H_kv d, D_model] (the [out, in] layout of a
// linear layer). No intermediate tensor: the product's epilogue stores the rows
// at their place in the [N, S_cap, H_kv, d] cache.
//
// bf16: a dense contraction on the matrix cores. A workgroup computes the
// transposed tile C^T[f, n] = sum_k W[f, k] x[n, k] for 128 output features x 128
// tokens with v_mfma_f32_32x32x16_bf16 (four waves, each 64 x 64 = 2 x 2 MFMA
// tiles): both operands are read along k, so both are MFMA operands as stored. K
// steps of 64 go through two LDS stages (16-byte chunks XOR-swizzled by row, the
// next step's global loads in registers while the current one is multiplied).
// The output lane layout puts 4 consecutive features of one token in a lane, so
// the epilogue writes 8-byte runs of a slot row. Workgroups are renumbered so that
// each XCD takes a contiguous range of tiles: the 32 feature tiles of a token
// tile then share its x rows in one L2.
// fp32: a tiled vector kernel (the full-precision path, not a performance target).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moda_internal.h"

namespace moda {
namespace {

typedef __bf16 pbf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 pbf16x2 __attribute__((ext_vector_type(2)));
typedef float pf32x16 __attribute__((ext_vector_type(16)));
typedef float pf32x2 __attribute__((ext_vector_type(2)));

constexpr int kPF = 128;        // output features per workgroup tile
constexpr int kPT = 128;        // tokens per workgroup tile
constexpr int kPK = 64;         // k per step
constexpr int kCH = kPK / 8;    // 16-byte chunks per tile row
constexpr int kLoads = kPF * kCH / 256;  // 16-byte loads per thread per operand and step

// LDS index (16-byte units) of chunk `c` of tile row `row`: XOR-swizzled so that
// the 32 rows an MFMA operand read touches spread over the banks
__device__ __forceinline__ int pswz(int row, int c) { return row * kCH + (c ^ (row & 7)); }

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  const pf32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, pbf16x2));
}

__device__ __forceinline__ int64_t tile_id(const ProjParams& p) {
  int64_t id = blockIdx.x;
  const int64_t n_tiles = (int64_t)p.n_feat_tiles * p.n_tok_tiles;
  // workgroups go to the 8 XCDs round-robin: give each XCD a contiguous range
  if (n_tiles % 8 == 0) id = (id % 8) * (n_tiles / 8) + id / 8;
  return id;
}

__global__ __launch_bounds__(256, 2) void moda_depth_kv_project_bf16_kernel(const ProjParams p) {
  __shared__ uint4 sw[2][kPF * kCH];
  __shared__ uint4 sx[2][kPT * kCH];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wf = wave >> 1, wt = wave & 1;  // this wave's 64-feature and 64-token quarter
  const int r = lane & 31, hh = lane >> 5;
  const int64_t id = tile_id(p);
  const int f0 = (int)(id % p.n_feat_tiles) * kPF;
  const int64_t t0 = (id / p.n_feat_tiles) * kPT;
  const uint16_t* __restrict__ X = static_cast<const uint16_t*>(p.x);
  const uint16_t* __restrict__ W = static_cast<const uint16_t*>(p.w);
  const int K = p.d_model;
  const int nk = K / kPK;

  uint4 rx[kLoads], rw[kLoads];
  // thread tid loads chunks c = tid + 256 j: row c / 8, 16-byte column c % 8 (eight
  // consecutive threads read one 128-byte row segment); tokens past N read zeros
  auto gload = [&](int kt) {
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int c = tid + 256 * j, row = c >> 3, col = c & 7;
      rw[j] = *reinterpret_cast<const uint4*>(W + (int64_t)(f0 + row) * K + kt * kPK + col * 8);
      const int64_t n = t0 + row;
      rx[j] = n < p.n_tokens ? *reinterpret_cast<const uint4*>(X + n * K + kt * kPK + col * 8)
                             : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int c = tid + 256 * j, row = c >> 3, col = c & 7;
      sw[buf][pswz(row, col)] = rw[j];
      sx[buf][pswz(row, col)] = rx[j];
    }
  };

  pf32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;

  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);  // in flight during this step's products
#pragma unroll
    for (int kk = 0; kk < kPK / 16; ++kk) {
      pbf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[i] = __builtin_bit_cast(pbf16x8, sw[buf][pswz(wf * 64 + i * 32 + r, 2 * kk + hh)]);
        b[i] = __builtin_bit_cast(pbf16x8, sx[buf][pswz(wt * 64 + i * 32 + r, 2 * kk + hh)]);
      }
#pragma unroll
      for (int fi = 0; fi < 2; ++fi)
#pragma unroll
        for (int ti = 0; ti < 2; ++ti)
          acc[fi][ti] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[fi], b[ti], acc[fi][ti], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(buf ^ 1);  // the other stage was released by the last barrier
    __syncthreads();
  }

  // epilogue: lane (r, hh) of tile (fi, ti) holds token t0 + 64 wt + 32 ti + r and
  // features 8 g + 4 hh + {0..3} of its 32-feature block, g = 0..3
  const int HD = p.hd;
  uint16_t* KDo = static_cast<uint16_t*>(p.kd);
  uint16_t* VDo = static_cast<uint16_t*>(p.vd);
#pragma unroll
  for (int ti = 0; ti < 2; ++ti) {
    const int64_t n = t0 + wt * 64 + ti * 32 + r;
    if (n >= p.n_tokens) continue;
    const int64_t row = (n * p.S_cap + p.slot) * (int64_t)HD;
#pragma unroll
    for (int fi = 0; fi < 2; ++fi)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int f = f0 + wf * 64 + fi * 32 + 8 * g + 4 * hh;
        const uint2 val = make_uint2(pack2(acc[fi][ti][4 * g], acc[fi][ti][4 * g + 1]),
                                     pack2(acc[fi][ti][4 * g + 2], acc[fi][ti][4 * g + 3]));
        uint16_t* dst = f < HD ? KDo + row + f : VDo + row + (f - HD);
        *reinterpret_cast<uint2*>(dst) = val;
      }
  }
}

// fp32: 64 features x 64 tokens per workgroup, thread (tx, ty) computes features
// 4 tx .. 4 tx + 3 of tokens 4 ty .. 4 ty + 3, k in steps of 16 through LDS.
__global__ __launch_bounds__(256) void moda_depth_kv_project_f32_kernel(const ProjParams p) {
  __shared__ float sw[16][64 + 1];
  __shared__ float sx[16][64 + 1];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int64_t id = blockIdx.x;
  const int f0 = (int)(id % p.n_feat_tiles) * 64;
  const int64_t t0 = (id / p.n_feat_tiles) * 64;
  const float* __restrict__ X = static_cast<const float*>(p.x);
  const float* __restrict__ W = static_cast<const float*>(p.w);
  const int K = p.d_model;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    // 64 rows x 16 k of each operand: 4 elements per thread
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = tid + 256 * j, row = e >> 4, kk = e & 15;
      sw[kk][row] = W[(int64_t)(f0 + row) * K + k0 + kk];
      const int64_t n = t0 + row;
      sx[kk][row] = n < p.n_tokens ? X[n * K + k0 + kk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk)
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = fmaf(sw[kk][4 * tx + a], sx[kk][4 * ty + b], acc[a][b]);
    __syncthreads();
  }
  const int HD = p.hd;
  float* KDo = static_cast<float*>(p.kd);
  float* VDo = static_cast<float*>(p.vd);
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int64_t n = t0 + 4 * ty + b;
    if (n >= p.n_tokens) continue;
    const int64_t row = (n * p.S_cap + p.slot) * (int64_t)HD;
    const int f = f0 + 4 * tx;  // 4 consecutive features, never across the K/V boundary (HD % 64 == 0)
    float* dst = f < HD ? KDo + row + f : VDo + row + (f - HD);
    *reinterpret_cast<float4*>(dst) = make_float4(acc[0][b], acc[1][b], acc[2][b], acc[3][b]);
  }
}

}  // namespace

hipError_t launch_depth_kv_project(ProjParams p, bool bf16, hipStream_t stream) {
  const int F = 2 * p.hd;
  if (bf16) {
    p.n_feat_tiles = F / kPF;
    p.n_tok_tiles = (p.n_tokens + kPT - 1) / kPT;
    const int64_t n = (int64_t)p.n_feat_tiles * p.n_tok_tiles;
    hipLaunchKernelGGL(moda_depth_kv_project_bf16_kernel, dim3((unsigned)n), dim3(256), 0, stream, p);
  } else {
    p.n_feat_tiles = F / 64;
    p.n_tok_tiles = (p.n_tokens + 63) / 64;
    const int64_t n = (int64_t)p.n_feat_tiles * p.n_tok_tiles;
    hipLaunchKernelGGL(moda_depth_kv_project_f32_kernel, dim3((unsigned)n), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace moda

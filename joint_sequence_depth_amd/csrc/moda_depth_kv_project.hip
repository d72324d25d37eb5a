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
// bf16: a dense contraction on the matrix cores. A workgroup of eight waves
// computes the transposed tile C^T[f, n] = sum_k W[f, k] x[n, k] for 256 output
// features x 256 tokens with v_mfma_f32_32x32x16_bf16, each wave 128 x 64 (4 x 2
// MFMA tiles); both operands are read along k, so both are MFMA operands as
// stored. K steps of 64 go from memory straight into two LDS stages (buffer
// loads with the LDS flag: no register staging), the next step's loads in flight
// while the current one is multiplied; rows past the last token or feature read
// zeros. In LDS each 128-byte row holds its eight 16-byte chunks XOR-swizzled by
// (row / 2) % 8, so the 16 rows that one operand read serves per LDS cycle cover
// every bank once. Operands are read one k sub-step ahead of the products. The
// output lane layout puts 4 consecutive features of one token in a lane, so the
// epilogue stages each wave's outputs through LDS token by token and stores whole
// 256-byte runs of a slot row with the non-temporal hint. Workgroups are renumbered so
// that each XCD takes a contiguous range of tiles: the feature tiles of a token
// tile then share its x rows in one L2.
// fp32: a tiled vector kernel (the full-precision path, not a performance target).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moda_internal.h"
#include "moda_lds_load.h"

namespace moda {
namespace {

typedef __bf16 pbf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 pbf16x2 __attribute__((ext_vector_type(2)));
typedef float pf32x16 __attribute__((ext_vector_type(16)));
typedef float pf32x2 __attribute__((ext_vector_type(2)));

#ifndef MODA_PROJ_PK
#define MODA_PROJ_PK 64
#define MODA_PROJ_NST 2
#endif
#ifndef MODA_PROJ_PW  // 4 (128 x 128 per wave, one wave per SIMD) measured 27 % slower
#define MODA_PROJ_PW 8
#endif
constexpr int kPF = 256;             // output features per workgroup tile
constexpr int kPT = 256;             // tokens per workgroup tile
constexpr int kPK = MODA_PROJ_PK;    // k per step
constexpr int kNST = MODA_PROJ_NST;  // LDS stages (loads run kNST - 1 steps ahead)
constexpr int kPW = MODA_PROJ_PW;    // waves per workgroup: 2 along features x kPW / 2 along tokens
constexpr int kWT = kPT / (kPW / 2); // tokens per wave
constexpr int kNTI = kWT / 32;       // 32-token MFMA tiles per wave
constexpr int kRow = kPK * 2;        // bytes of one tile row per stage
constexpr int kCPR = kPK / 8;        // 16-byte chunks per row
constexpr int kRPR = 1024 / kRow;    // rows per 1 KB run
constexpr int kRuns = kPF / kRPR;    // runs per operand tile and step
constexpr int kRunsW = kRuns / kPW;  // runs of each operand loaded by each wave per step
constexpr int kLoadsW = 2 * kRunsW;  // loads issued by a wave per step
constexpr int kStage = (kPF + kPT) * kRow;  // bytes of one stage (W rows, then x rows)
constexpr int kBankRows = 256 / kRow;       // rows sharing one 256-byte bank line
static_assert(kPF == kPT && kRunsW * kPW == kRuns && kNST >= 2, "tile shape");

// byte offset in a stage of 16-byte chunk c of tile row `row`: the chunks of the
// 16 rows one operand read serves per LDS cycle land on distinct bank slots
__device__ __forceinline__ uint32_t pswz(int row, int c) {
  return (uint32_t)(row * kRow + 16 * (c ^ ((row / kBankRows) % kCPR)));
}

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

__global__ __launch_bounds__(64 * kPW, 1) void moda_depth_kv_project_bf16_kernel(const ProjParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[kNST * kStage];
  poison_lds(smem, kNST * kStage);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wf = wave & 1, wt = wave >> 1;  // this wave's 128-feature half and kWT-token slice
  const int r = lane & 31, hh = lane >> 5;
  const int64_t id = tile_id(p);
  const int f0 = (int)(id % p.n_feat_tiles) * kPF;
  const int64_t t0 = (id / p.n_feat_tiles) * kPT;
  const int K = p.d_model;
  const int nk = K / kPK;
  const int64_t rowb = (int64_t)K * 2;  // bytes from one operand row to the next

  // the tile's rows of W and x as buffer ranges: rows past the last feature or
  // token read zeros
  const int64_t w_left = 2 * (int64_t)p.hd - f0;
  const int64_t x_left = p.n_tokens - t0;
  const int64_t w_bytes = (w_left < kPF ? w_left : kPF) * rowb;
  const int64_t x_bytes = (x_left < kPT ? x_left : kPT) * rowb;
  const i32x4 w_rs = make_rsrc(static_cast<const char*>(p.w) + (int64_t)f0 * rowb, (uint32_t)w_bytes);
  const i32x4 x_rs = make_rsrc(static_cast<const char*>(p.x) + t0 * rowb, (uint32_t)x_bytes);

  // lane l of a 1 KB run fills LDS bytes [16 l, 16 l + 16): row l / kCPR of the run
  // at chunk position l % kCPR, which holds the chunk pswz puts there
  auto issue = [&](int kt, int stage) __attribute__((always_inline)) {
    const uint32_t lds = (uint32_t)(uintptr_t)(smem + stage * kStage);
    const uint32_t kofs = (uint32_t)(kt * kRow);
#pragma unroll
    for (int j = 0; j < kRunsW; ++j) {
      const int run = wave * kRunsW + j;
      const int row = run * kRPR + lane / kCPR;
      const int chunk = (lane % kCPR) ^ ((row / kBankRows) % kCPR);
      const uint32_t voff = (uint32_t)(row * rowb) + 16u * (uint32_t)chunk + kofs;
      load_to_lds16(lds + 1024u * run, voff, w_rs);
      load_to_lds16(lds + kPF * kRow + 1024u * run, voff, x_rs);
    }
  };

  pf32x16 acc[4][kNTI];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < kNTI; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;

  // operands of k sub-step kk (16 k) of a stage: W rows 128 wf + 32 i + r and x
  // rows kWT wt + 32 i + r, chunk 2 kk + hh
  auto read_ops = [&](const unsigned char* st, int kk, pbf16x8(&a)[4], pbf16x8(&b)[kNTI])
      __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a[i] = *reinterpret_cast<const pbf16x8*>(st + pswz(wf * 128 + i * 32 + r, 2 * kk + hh));
#pragma unroll
    for (int i = 0; i < kNTI; ++i)
      b[i] = *reinterpret_cast<const pbf16x8*>(st + kPF * kRow + pswz(wt * kWT + i * 32 + r, 2 * kk + hh));
  };

  // every step issues one load group (past the last k step it reloads that one
  // into a free stage) so that a fixed wait count leaves exactly the later groups
  // in flight
#pragma unroll
  for (int j = 0; j < kNST - 1; ++j) issue(j < nk ? j : nk - 1, j);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(kLoadsW * (kNST - 2)));
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int stage = kt % kNST;
    {  // into the stage step kt - 1 used, released by the last barrier
      const int kn = kt + kNST - 1;
      issue(kn < nk ? kn : nk - 1, kn % kNST);
    }
    const unsigned char* st = smem + stage * kStage;
    pbf16x8 a[2][4], b[2][kNTI];
    read_ops(st, 0, a[0], b[0]);
#pragma unroll
    for (int kk = 0; kk < kPK / 16; ++kk) {
      if (kk + 1 < kPK / 16) read_ops(st, kk + 1, a[(kk + 1) & 1], b[(kk + 1) & 1]);
#pragma unroll
      for (int fi = 0; fi < 4; ++fi)
#pragma unroll
        for (int ti = 0; ti < kNTI; ++ti)
          acc[fi][ti] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kk & 1][fi], b[kk & 1][ti], acc[fi][ti], 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kLoadsW * (kNST - 2)));  // step kt + 1's rows have landed
    __syncthreads();                                               // and every wave is done with this stage
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no load into LDS outlives the loop
  __syncthreads();                           // nor any other wave's: the stages are free

  // epilogue: lane (r, hh) of tile (fi, ti) holds token kWT wt + 32 ti + r of the
  // tile and features 8 g + 4 hh + {0..3} of its 32-feature block, g = 0..3. Each
  // wave stages its 128 features x kWT tokens through LDS, token-major (the
  // 16-byte chunks of a token's 256-byte row XOR-swizzled by token % 16), and
  // stores whole runs: 16 lanes write a token's 256 contiguous bytes.
  constexpr int kOR = 128 * 2;      // bytes of a wave's token row (128 features)
  constexpr int kOC = kOR / 16;     // 16-byte chunks per row
  static_assert(kPW * kWT * kOR <= kNST * kStage, "output staging");
  unsigned char* ob = smem + wave * kWT * kOR;
#pragma unroll
  for (int ti = 0; ti < kNTI; ++ti) {
    const int tt = ti * 32 + r;
#pragma unroll
    for (int fi = 0; fi < 4; ++fi)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<uint2*>(ob + tt * kOR + 16 * ((4 * fi + g) ^ (tt % kOC)) + 8 * hh) =
            make_uint2(pack2(acc[fi][ti][4 * g], acc[fi][ti][4 * g + 1]),
                       pack2(acc[fi][ti][4 * g + 2], acc[fi][ti][4 * g + 3]));
  }
  const int HD = p.hd;
  uint16_t* KDo = static_cast<uint16_t*>(p.kd);
  uint16_t* VDo = static_cast<uint16_t*>(p.vd);
  const int c = lane % kOC;
  const int f = f0 + wf * 128 + 8 * c;  // first of the chunk's 8 features (HD % 64 == 0: one side of HD)
#pragma unroll
  for (int j = 0; j < kWT * kOC / 64; ++j) {
    const int tt = j * (64 / kOC) + lane / kOC;
    typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
    const u32x4v v = *reinterpret_cast<const u32x4v*>(ob + tt * kOR + 16 * (c ^ (tt % kOC)));
    const int64_t n = t0 + wt * kWT + tt;
    if (n < p.n_tokens && f < 2 * HD) {
      const int64_t row = (n * p.S_cap + p.slot) * (int64_t)HD;
      uint16_t* dst = f < HD ? KDo + row + f : VDo + row + (f - HD);
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4v*>(dst));
    }
  }
}

// fp32: 64 features x 64 tokens per workgroup, thread (tx, ty) computes features
// 4 tx .. 4 tx + 3 of tokens 4 ty .. 4 ty + 3, k in steps of 16 through LDS.
__global__ __launch_bounds__(256) void moda_depth_kv_project_f32_kernel(const ProjParams p) {
  __shared__ float sw[16][64 + 1];
  __shared__ float sx[16][64 + 1];
  poison_lds(sw, sizeof(sw));
  poison_lds(sx, sizeof(sx));
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
    p.n_feat_tiles = (F + kPF - 1) / kPF;
    p.n_tok_tiles = (p.n_tokens + kPT - 1) / kPT;
    const int64_t n = (int64_t)p.n_feat_tiles * p.n_tok_tiles;
    hipLaunchKernelGGL(moda_depth_kv_project_bf16_kernel, dim3((unsigned)n), dim3(64 * kPW), 0, stream, p);
  } else {
    p.n_feat_tiles = F / 64;
    p.n_tok_tiles = (p.n_tokens + 63) / 64;
    const int64_t n = (int64_t)p.n_feat_tiles * p.n_tok_tiles;
    hipLaunchKernelGGL(moda_depth_kv_project_f32_kernel, dim3((unsigned)n), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace moda

// Backward of the MoDA joint sequence/depth attention (MoDA, arXiv 2603.15619;
// forward on deck slide "One denominator allocates probability across both
// memories"). The pages give the forward only; this is its exact derivative.
// With P the joint softmax of a row (over its visible sequence keys and its own
// depth slots, recomputed from the forward's lse), dout the upstream gradient:
//
//   delta_t = <dout_t, out_t>        (= sum over the row's keys of P dP)
//   dS_x    = P_x (<dout_t, value_x> - delta_t)
//   dq_t    = scale (sum_j dS_j k_j + sum_i dS_i k_depth_{t,i})
//   dk_j    = scale sum_t dS_tj q_t,     dv_j = sum_t P_tj dout_t
//   dk_depth_{t,i} = scale dS_ti q_t,    dv_depth_{t,i} = P_ti dout_t
//
// summed over the G query heads of a KV head. Three launches on one stream:
//
//  * prep (any dtype): one wave per (token, KV head). Computes delta for the G
//    heads, then the depth part, which is row-local (a depth slot belongs to one
//    token): lanes hold 8-element slices of a slot row (LPR = D / 8 lanes per
//    row), so dk_depth / dv_depth are summed over the heads in registers and
//    written once, and the depth share of dq (summed over slots in LDS) goes to an
//    fp32 workspace.
//  * dq (bf16, matrix cores): a workgroup of 4 waves per (segment, query head,
//    128 tokens), 32 tokens per wave, K/V blocks of 64 keys staged in LDS.
//    S^T = K Q^T and dP^T = V dO^T put one token per lane; dS^T feeds
//    dQ^T += K^T dS^T through transposing LDS reads of K, with the keys of the
//    dS^T registers and of the K^T operand in the same order. The epilogue adds
//    the depth share.
//  * dk/dv (bf16, matrix cores): a workgroup of 8 waves per (segment, KV head,
//    128 keys), two waves per 32-key block splitting each 64-token query tile,
//    looping over the G query heads and the tiles that can see the keys (Q, dO,
//    lse and delta staged in LDS, K and V rows in LDS). S = Q K^T and
//    dP = dO V^T put one key per lane; dV^T += dO^T P and dK^T += Q^T dS read
//    dO^T and Q^T transposed from LDS.
//  * fp32 inputs take row-wise vector kernels for dq and dk/dv instead (lanes over
//    8-element slices, as in prep): the full-precision path.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moda_internal.h"
#include "moda_rowops.h"

namespace moda {
namespace {

using rowops::group_sum;
using rowops::load8;
using rowops::store_n;

typedef __bf16 bbf16x8 __attribute__((ext_vector_type(8)));
typedef float bf32x16 __attribute__((ext_vector_type(16)));
typedef short bi16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kBwdWaves = 4;   // waves per workgroup, all kernels
constexpr int kBlk = 128;      // tokens (dq) or keys (dk/dv) per workgroup
constexpr int kTile = 64;      // keys (dq) or tokens (dk/dv) staged per step
// Bytes of padding per staged LDS row (272-byte rows at d = 128 keep the 16-byte
// row reads conflict-free; 48 bytes, free of conflicts for the transposing reads
// too, measured no faster).
constexpr int kPad = 16;

#define MODA_BWD_TR_READ(a) __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) bi16x4*)(a))

struct Seg {
  int64_t start, len;
};

__device__ __forceinline__ Seg segment(const BwdParams& p, int seg) {
  if (p.cu_seqlens) {
    int64_t a = p.cu_seqlens[seg], b = p.cu_seqlens[seg + 1];
    a = a < 0 ? 0 : (a > p.total_tokens ? p.total_tokens : a);
    b = b < a ? a : (b > p.total_tokens ? p.total_tokens : b);
    return {a, b - a};
  }
  return {(int64_t)seg * p.uniform_len, p.uniform_len};
}

// Segment holding packed token n (the segment whose range contains it).
__device__ __forceinline__ Seg segment_of(const BwdParams& p, int64_t n) {
  if (!p.cu_seqlens) {
    const int64_t s = n / p.uniform_len;
    return {s * p.uniform_len, p.uniform_len};
  }
  int lo = 0, hi = p.n_seg - 1;  // last segment whose clamped start <= n
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (segment(p, mid).start <= n) lo = mid;
    else hi = mid - 1;
  }
  return segment(p, lo);
}

// lse element of packed token n, query head h.
__device__ __forceinline__ int64_t lse_index(const BwdParams& p, int64_t n, int h) {
  if (p.lse_batch_layout) {
    const int64_t b = n / p.lse_head_stride, t = n - b * p.lse_head_stride;
    return (b * p.Hq + h) * p.lse_head_stride + t;
  }
  return (int64_t)h * p.lse_head_stride + n;
}

// ---------------------------------------------------------------- prep + depth
// 8 consecutive elements of a row as stored (bf16: one 16-byte word, fp32: two);
// kept raw while the load is in flight and widened where it is used. NT: with the
// non-temporal hint (the depth slots, read once by the whole backward).
template <bool BF16>
struct Raw8 {
  uint4 w[BF16 ? 1 : 2];
};
template <bool BF16, bool NT = false>
__device__ __forceinline__ Raw8<BF16> load_raw8(const void* base, int64_t elem) {
  Raw8<BF16> r;
  if constexpr (BF16 && NT) {
    r.w[0] = rowops::stream_load16(static_cast<const uint16_t*>(base) + elem);
  } else if constexpr (BF16) {
    r.w[0] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem);
  } else if constexpr (NT) {
    const float* p = static_cast<const float*>(base) + elem;
    r.w[0] = rowops::stream_load16(p);
    r.w[1] = rowops::stream_load16(p + 4);
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(base) + elem);
    r.w[0] = p[0];
    r.w[1] = p[1];
  }
  return r;
}
template <bool BF16>
__device__ __forceinline__ void widen8(const Raw8<BF16>& r, float (&x)[8]) {
  if constexpr (BF16) {
    const uint32_t u[4] = {r.w[0].x, r.w[0].y, r.w[0].z, r.w[0].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = __uint_as_float(u[j] << 16);
      x[2 * j + 1] = __uint_as_float(u[j] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      x[4 * j] = __uint_as_float(r.w[j].x);
      x[4 * j + 1] = __uint_as_float(r.w[j].y);
      x[4 * j + 2] = __uint_as_float(r.w[j].z);
      x[4 * j + 3] = __uint_as_float(r.w[j].w);
    }
  }
}

// Prep and depth: one wave per (token, block of NGRP consecutive KV heads); lane
// group grp (LPR = D / 8 lanes, 8 elements each) owns KV head hb * NGRP + grp and
// its G query heads. A step handles one slot for all the wave's KV heads, so each
// load is NGRP consecutive rows of the slot (one contiguous run of the depth
// cache); kPrepRing slots are in flight. Nothing crosses lane groups: dk_depth and
// dv_depth sum the G heads in registers, and the depth share of dq sums the slots
// in registers (GC = G in {1, 2, 4}) or in the group's own LDS block (GC = 0: any
// G). Lane groups past the last KV head repeat it: they compute the same values
// and store them to the same places, so no store needs a branch. The main loop
// is straight-line (prefetches of slots past the end re-read the last slot), so
// every wait covers exactly the load it needs.
template <int D>
__host__ __device__ constexpr int prep_ngrp() { return 64 / (D / 8); }
// LDS floats per wave for GC = 0: dq share [NGRP][G][D], then lse2 and delta [NGRP][G]
__host__ __device__ constexpr int prep_wave_floats(int G, int D) { return (64 / (D / 8)) * G * (D + 2); }
constexpr int kPrepMaxLds = 64 * 1024;
constexpr int kPrepRing = 4;  // slots in flight per wave

template <int D, bool BF16, bool GF32, int GC>
__global__ __launch_bounds__(256) void moda_bwd_prep_kernel(const BwdParams p) {
  constexpr int LPR = D / 8;
  constexpr int NGRP = prep_ngrp<D>();
  constexpr bool REG = GC > 0;    // the G heads' state in registers
  constexpr int GR = REG ? GC : 1;  // register copies
  extern __shared__ float dyn[];
  if constexpr (GC == 0) poison_lds(dyn, (int)(blockDim.x >> 6) * prep_wave_floats(p.G, D) * 4);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wpb = blockDim.x >> 6;
  const int grp = lane / LPR, cl = lane % LPR;
  const int n_hb = (p.Hkv + NGRP - 1) / NGRP;
  const int64_t item = (int64_t)blockIdx.x * wpb + wave;
  if (item >= p.total_tokens * n_hb) return;  // no workgroup barrier below
  const int64_t n = item / n_hb;
  const int hk_raw = (int)(item % n_hb) * NGRP + grp;
  const int hk = hk_raw < p.Hkv ? hk_raw : p.Hkv - 1;
  const int G = REG ? GC : p.G;
  float* dqd = dyn + (size_t)wave * prep_wave_floats(G, D) + (size_t)grp * G * D;  // [G][D], GC = 0
  float* lse2s = dyn + (size_t)wave * prep_wave_floats(G, D) + (size_t)NGRP * G * D + 2 * grp * G;
  float* dels = lse2s + G;
  const int S = p.n_depth;
  auto slot_elem = [&](int i) __attribute__((always_inline)) {
    i = i < S ? i : S - 1;
    return ((n * p.S_cap + i) * p.Hkv + hk) * D + 8 * cl;
  };
  Raw8<BF16> kr[kPrepRing], vr[kPrepRing];
  if (S > 0) {  // the first slots are in flight while delta is computed
#pragma unroll
    for (int j = 0; j < kPrepRing - 1; ++j) {
      kr[j] = load_raw8<BF16, true>(p.kd, slot_elem(j));
      vr[j] = load_raw8<BF16, true>(p.vd, slot_elem(j));
    }
  }

  Raw8<BF16> qr[GR];
  Raw8<!GF32> dor[GR];
  float dqr[GR][8], lr[GR], dr[GR];
  for (int g = 0; g < G; ++g) {
    const int h = hk * G + g;
    const int64_t e = (n * p.Hq + h) * D + 8 * cl;
    float o8[8], d8[8];
    load8<!GF32>(p.out, e, o8);
    load8<!GF32>(p.dout, e, d8);
    float sdo = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) sdo = fmaf(o8[j], d8[j], sdo);
    sdo = group_sum<LPR>(sdo);
    const float l2 = p.lse[lse_index(p, n, h)] * kLog2e;
    if (cl == 0) p.delta[(int64_t)h * p.total_tokens + n] = sdo;
    if constexpr (REG) {
#pragma unroll
      for (int gg = 0; gg < GR; ++gg)
        if (gg == g) {
          qr[gg] = load_raw8<BF16>(p.q, e);
          dor[gg] = load_raw8<!GF32>(p.dout, e);
          lr[gg] = l2;
          dr[gg] = sdo;
#pragma unroll
          for (int j = 0; j < 8; ++j) dqr[gg][j] = 0.f;
        }
    } else {
      if (cl == 0) {
        lse2s[g] = l2;
        dels[g] = sdo;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) dqd[g * D + 8 * cl + j] = 0.f;
    }
  }
  if (S <= 0) return;
  // LDS accesses of one wave complete in issue order: the values written above
  // are visible to every lane of the wave below.
  __builtin_amdgcn_wave_barrier();

  const float c2 = p.scale_log2, sc = p.scale;
  // one head's contribution of slot (kd8, vd8)
  auto head = [&](const float (&q8)[8], const float (&do8)[8], float l2, float dl, const float (&kd8)[8],
                  const float (&vd8)[8], float (&dk8)[8], float (&dv8)[8], float (&dq8)[8])
                  __attribute__((always_inline)) {
    float b = 0.f, dp = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      b = fmaf(q8[j], kd8[j], b);
      dp = fmaf(do8[j], vd8[j], dp);
    }
    b = group_sum<LPR>(b);
    dp = group_sum<LPR>(dp);
    const float pr = __builtin_amdgcn_exp2f(b * c2 - l2);
    const float ds = pr * (dp - dl) * sc;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      dv8[j] = fmaf(pr, do8[j], dv8[j]);
      dk8[j] = fmaf(ds, q8[j], dk8[j]);
      dq8[j] = fmaf(ds, kd8[j], dq8[j]);
    }
  };
  auto process = [&](int i, const Raw8<BF16>& kraw, const Raw8<BF16>& vraw) __attribute__((always_inline)) {
    float kd8[8], vd8[8], dk8[8], dv8[8];
    widen8<BF16>(kraw, kd8);
    widen8<BF16>(vraw, vd8);
#pragma unroll
    for (int j = 0; j < 8; ++j) dk8[j] = dv8[j] = 0.f;
    if constexpr (REG) {
#pragma unroll
      for (int g = 0; g < GR; ++g) {
        float q8[8], do8[8];
        Raw8<BF16> qx = qr[g];
        Raw8<!GF32> dx = dor[g];
        if constexpr (GR > 1) {  // widen per slot: hoisting every head's widened rows costs occupancy
#pragma unroll
          for (int w = 0; w < (BF16 ? 1 : 2); ++w) asm volatile("" : "+v"(qx.w[w].x), "+v"(qx.w[w].y), "+v"(qx.w[w].z), "+v"(qx.w[w].w));
#pragma unroll
          for (int w = 0; w < (GF32 ? 2 : 1); ++w) asm volatile("" : "+v"(dx.w[w].x), "+v"(dx.w[w].y), "+v"(dx.w[w].z), "+v"(dx.w[w].w));
        }
        widen8<BF16>(qx, q8);
        widen8<!GF32>(dx, do8);
        head(q8, do8, lr[g], dr[g], kd8, vd8, dk8, dv8, dqr[g]);
      }
    } else {
      for (int g = 0; g < G; ++g) {
        const int64_t e = (n * p.Hq + hk * G + g) * D + 8 * cl;
        float q8[8], do8[8], dq8[8];
        load8<BF16>(p.q, e, q8);
        load8<!GF32>(p.dout, e, do8);
#pragma unroll
        for (int j = 0; j < 8; ++j) dq8[j] = dqd[g * D + 8 * cl + j];
        head(q8, do8, lse2s[g], dels[g], kd8, vd8, dk8, dv8, dq8);
#pragma unroll
        for (int j = 0; j < 8; ++j) dqd[g * D + 8 * cl + j] = dq8[j];
      }
    }
    const int64_t de = slot_elem(i);
    store_n<GF32, 8, true>(p.dkd, de, dk8);  // the depth gradients: written once, streamed
    store_n<GF32, 8, true>(p.dvd, de, dv8);
  };
  int i0 = 0;
  for (; i0 + kPrepRing <= S; i0 += kPrepRing) {  // whole rounds: straight-line body
#pragma unroll
    for (int u = 0; u < kPrepRing; ++u) {
      const int r = (u + kPrepRing - 1) % kPrepRing;
      kr[r] = load_raw8<BF16, true>(p.kd, slot_elem(i0 + u + kPrepRing - 1));
      vr[r] = load_raw8<BF16, true>(p.vd, slot_elem(i0 + u + kPrepRing - 1));
      process(i0 + u, kr[u], vr[u]);
    }
  }
#pragma unroll
  for (int u = 0; u < kPrepRing - 1; ++u)  // the last slots (already loaded)
    if (i0 + u < S) process(i0 + u, kr[u], vr[u]);

  if constexpr (REG) {
#pragma unroll
    for (int g = 0; g < GR; ++g) store_n<true, 8>(p.dq_depth, (n * p.Hq + hk * GC + g) * D + 8 * cl, dqr[g]);
  } else {
    for (int g = 0; g < G; ++g)
      store_n<true, 8>(p.dq_depth, (n * p.Hq + hk * G + g) * D + 8 * cl, dqd + g * D + 8 * cl);
  }
}

// ---------------------------------------------------------------- bf16 helpers
// One 16-byte chunk of a row (8 bf16) from global memory, as bf16; fp32 storage is
// rounded to bf16 (nearest even).
template <bool F32>
__device__ __forceinline__ uint4 load_chunk_bf16(const void* base, int64_t elem) {
  if constexpr (F32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem);
    const float4 a = p[0], b = p[1];
    return make_uint4(rowops::pack_bf16x2(a.x, a.y), rowops::pack_bf16x2(a.z, a.w), rowops::pack_bf16x2(b.x, b.y),
                      rowops::pack_bf16x2(b.z, b.w));
  } else {
    return *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem);
  }
}

__device__ __forceinline__ bbf16x8 as_b8(uint4 w) { return __builtin_bit_cast(bbf16x8, w); }

__device__ __forceinline__ bbf16x8 pk_b8(const uint32_t* w) {
  return __builtin_bit_cast(bbf16x8, make_uint4(w[0], w[1], w[2], w[3]));
}

// Transposed operand of rows [r0, r0 + 16) of a row-major LDS tile (pitch PITCH
// bytes), d tile dt: lane 16 g + 4 e + q reads rows r0 + 4 (g / 2) + e and that + 8
// at columns 32 dt + 16 (g % 2) + 4 q .. + 3; after the transpose lane (r, hh)
// holds column 32 dt + r at rows r0 + 4 hh + {0..3, 8..11}, the row order of 8
// consecutive accumulator registers of a 32 x 32 score tile.
template <int PITCH>
__device__ __forceinline__ bbf16x8 tr_operand(const unsigned char* tile, int r0, int dt, int lane) {
  const int g = lane >> 4, e = (lane >> 2) & 3, q = lane & 3;
  const uint32_t a = (uint32_t)(uintptr_t)tile + (uint32_t)((r0 + 4 * (g >> 1) + e) * PITCH) +
                     (uint32_t)(2 * (32 * dt + 16 * (g & 1) + 4 * q));
  const bi16x4 x0 = MODA_BWD_TR_READ(a);
  const bi16x4 x1 = MODA_BWD_TR_READ(a + 8 * PITCH);
  return __builtin_bit_cast(bbf16x8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
}

// ---------------------------------------------------------------- dq (bf16)
// two waves per SIMD: the second wave's vector work overlaps the first one's
// matrix products (with one wave per SIMD the kernel runs ~40 % longer)
#define MODA_BWD_DQ_ATTR __attribute__((amdgpu_waves_per_eu(2, 2)))
template <int D, bool GF32>
__global__ __launch_bounds__(64 * kBwdWaves) MODA_BWD_DQ_ATTR void moda_bwd_dq_kernel(const BwdParams p) {
  constexpr int KC = D / 16, DT = D / 32;
  constexpr int PITCH = D * 2 + kPad;
  constexpr int CPR = D * 2 / 16;                      // 16-byte chunks per row
  constexpr int NLD = kTile * CPR / (64 * kBwdWaves);  // chunks per thread per tile
  // two buffers: the tile after next is stored while the current one is read
  __shared__ __align__(16) unsigned char kbuf[2][kTile * PITCH];
  __shared__ __align__(16) unsigned char vbuf[2][kTile * PITCH];
  poison_lds(kbuf, sizeof(kbuf));
  poison_lds(vbuf, sizeof(vbuf));
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r = lane & 31, hh = lane >> 5;

  // Workgroup order: with xcd_group, consecutive workgroups (which the hardware
  // deals round-robin to the 8 XCDs) are mapped so that each (segment, head) row
  // runs on one XCD, heaviest query block first, and the K/V tiles the row
  // re-reads stay in that XCD's L2; rows go round-robin over the XCDs, so
  // segments of different lengths spread over all of them.
  int64_t rest = blockIdx.x;
  if (p.xcd_group) {
    const int64_t x = rest % 8, j = rest / 8;
    rest = ((j / p.n_qblocks) * 8 + x) * p.n_qblocks + (p.n_qblocks - 1 - j % p.n_qblocks);
  }
  const int qb = (int)(rest % p.n_qblocks);
  rest /= p.n_qblocks;
  const int h = (int)(rest % p.Hq);
  const int seg = (int)(rest / p.Hq);
  const Seg sg = segment(p, seg);
  const int64_t t0 = (int64_t)qb * kBlk;
  if (t0 >= sg.len) return;  // whole workgroup, before any barrier
  const int hk = h / p.G;
  const int64_t tw = t0 + 32 * wave;
  const int64_t t = tw + r;
  const bool row_ok = t < sg.len;
  const int64_t n = sg.start + (row_ok ? t : sg.len - 1);

  bbf16x8 qf[KC], dof[KC];
  {
    const int64_t e = (n * p.Hq + h) * D;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      qf[kc] = as_b8(load_chunk_bf16<false>(p.q, e + 16 * kc + 8 * hh));
      dof[kc] = as_b8(load_chunk_bf16<GF32>(p.dout, e + 16 * kc + 8 * hh));
    }
  }
  const float lse2 = p.lse[lse_index(p, n, h)] * kLog2e;
  const float dl = p.delta[(int64_t)h * p.total_tokens + n];
  const float c2 = p.scale_log2;

  bf32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;

  const int64_t kend = p.causal ? (t0 + kBlk < sg.len ? t0 + kBlk : sg.len) : sg.len;
  const int nkb = (int)((kend + kTile - 1) / kTile);
  // the next tile's rows in flight, as vector values (not arrays, which the
  // compiler would keep in private memory across the loop)
  typedef uint32_t stage_t __attribute__((ext_vector_type(4 * NLD)));
  struct Stage {
    stage_t k, v;
  };
  auto gload = [&](int kb) __attribute__((always_inline)) {
    Stage g;
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int idx = tid + 64 * kBwdWaves * u, row = idx / CPR, ch = idx % CPR;
      int64_t key = (int64_t)kb * kTile + row;
      key = key < sg.len ? key : sg.len - 1;  // rows past the end repeat the last key (masked)
      const int64_t e = ((sg.start + key) * p.Hkv + hk) * D + 8 * ch;
      const uint4 a = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.k) + e);
      const uint4 b = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.v) + e);
      g.k[4 * u] = a.x;
      g.k[4 * u + 1] = a.y;
      g.k[4 * u + 2] = a.z;
      g.k[4 * u + 3] = a.w;
      g.v[4 * u] = b.x;
      g.v[4 * u + 1] = b.y;
      g.v[4 * u + 2] = b.z;
      g.v[4 * u + 3] = b.w;
    }
    return g;
  };
  auto sstore = [&](const Stage& g, int b) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int idx = tid + 64 * kBwdWaves * u, row = idx / CPR, ch = idx % CPR;
      *reinterpret_cast<uint4*>(kbuf[b] + row * PITCH + 16 * ch) =
          make_uint4(g.k[4 * u], g.k[4 * u + 1], g.k[4 * u + 2], g.k[4 * u + 3]);
      *reinterpret_cast<uint4*>(vbuf[b] + row * PITCH + 16 * ch) =
          make_uint4(g.v[4 * u], g.v[4 * u + 1], g.v[4 * u + 2], g.v[4 * u + 3]);
    }
  };

  // Tile kb is read from buffer kb % 2; tile kb + 1 arrives in registers during
  // step kb and is stored into the other buffer, which every wave finished reading
  // before the barrier that ended step kb - 1.
  Stage next = gload(0);
  sstore(next, 0);
  __syncthreads();
  if (nkb > 1) next = gload(1);
  for (int kb = 0; kb < nkb; ++kb) {
    const unsigned char* ks = kbuf[kb & 1];
    const unsigned char* vs = vbuf[kb & 1];
    // S^T = K Q^T and dP^T = V dO^T of sub-tile st (32 keys)
    auto sdp = [&](int st, bf32x16& s, bf32x16& dp) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = dp[i] = 0.f;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const int off = (32 * st + r) * PITCH + 16 * (2 * kc + hh);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_b8(*reinterpret_cast<const uint4*>(ks + off)), qf[kc], s, 0, 0,
                                                    0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_b8(*reinterpret_cast<const uint4*>(vs + off)), dof[kc], dp, 0,
                                                     0, 0);
      }
    };
    // dS^T of sub-tile st as bf16 pairs; register i holds key
    // k0 + 8 (i / 4) + 4 hh + i % 4 of token t
    auto dscore = [&](int st, const bf32x16& s, const bf32x16& dp, uint32_t(&dsp)[8]) __attribute__((always_inline)) {
      const int64_t k0 = (int64_t)kb * kTile + 32 * st;
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        float v2[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int64_t key = k0 + 8 * ((i + u) >> 2) + 4 * hh + ((i + u) & 3);
          const bool vis = row_ok && key < sg.len && (!p.causal || key <= t);
          const float pr = vis ? __builtin_amdgcn_exp2f(s[i + u] * c2 - lse2) : 0.f;
          v2[u] = pr * (dp[i + u] - dl);
        }
        dsp[i >> 1] = rowops::pack_bf16x2(v2[0], v2[1]);
      }
    };
    // dQ^T += K^T dS^T for sub-tile st
    auto accumulate = [&](int st, const uint32_t(&dsp)[8]) __attribute__((always_inline)) {
#pragma unroll
      for (int part = 0; part < 2; ++part)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand<PITCH>(ks, 32 * st + 16 * part, dt, lane),
                                                            pk_b8(dsp + 4 * part), acc[dt], 0, 0, 0);
    };
    auto active = [&](int st) __attribute__((always_inline)) {
      const int64_t k0 = (int64_t)kb * kTile + 32 * st;
      return k0 < sg.len && !(p.causal && k0 > tw + 31);  // wave-uniform
    };
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      if (!active(st)) continue;
      bf32x16 s, dp;
      uint32_t dsp[8];
      sdp(st, s, dp);
      dscore(st, s, dp, dsp);
      accumulate(st, dsp);
    }
    if (kb + 1 < nkb) sstore(next, (kb + 1) & 1);
    __syncthreads();
    if (kb + 2 < nkb) next = gload(kb + 2);
  }

  if (!row_ok) return;
  const int64_t e = (n * p.Hq + h) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = 32 * dt + 8 * j + 4 * hh;
      float x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = acc[dt][4 * j + u] * p.scale;
      if (p.n_depth > 0) {
        const float4 a = *reinterpret_cast<const float4*>(p.dq_depth + e + c);
        x[0] += a.x;
        x[1] += a.y;
        x[2] += a.z;
        x[3] += a.w;
      }
      store_n<GF32, 4>(p.dq, e + c, x);
    }
}

// ---------------------------------------------------------------- dk / dv (bf16)
// A workgroup of 8 waves owns 128 keys of one (segment, KV head) and loops over
// the G query heads and the 64-token query tiles that can see them (Q, dO, lse
// and delta double-buffered in LDS). The two waves of a 32-key block split each
// tile (wave w: keys 32 (w % 4), rows 32 (w / 4) of the tile), so a SIMD runs two
// waves, each holding one 128 x 32 dK^T and one dV^T accumulator in registers;
// the K and V rows of the 128 keys sit in LDS as the products' B operands. At the
// end each pair adds its two partial sums through LDS. (With 4 waves holding all
// of a key block's tiles and K/V in registers, one wave per SIMD fit: 10-22 %
// slower.)
constexpr int kDkv8Waves = 8;

template <int D, bool GF32>
__global__ __launch_bounds__(64 * kDkv8Waves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void moda_bwd_dkv8_kernel(const BwdParams p) {
  constexpr int KC = D / 16, DT = D / 32;
  constexpr int PITCH = D * 2 + kPad;
  constexpr int CPR = D * 2 / 16;
  constexpr int NTH = 64 * kDkv8Waves;
  constexpr int NLD = kTile * CPR / NTH;        // Q (and dO) chunks per thread per tile
  constexpr int NKV = kBlk * CPR / NTH;         // K (and V) chunks per thread, once
  constexpr int KV_BYTES = kBlk * PITCH;        // one of K, V
  constexpr int TILE_BYTES = kTile * PITCH;     // one of Q, dO, per buffer
  constexpr int OFF_Q = 2 * KV_BYTES;
  constexpr int OFF_O = OFF_Q + 2 * TILE_BYTES;
  constexpr int OFF_L = OFF_O + 2 * TILE_BYTES;
  constexpr int OFF_D = OFF_L + 2 * kTile * 4;
  constexpr int LDS_BYTES = OFF_D + 2 * kTile * 4;
  static_assert(4 * 64 * 2 * DT * 16 * 4 <= LDS_BYTES, "partials of four waves fit in the LDS block");
  __shared__ __align__(16) unsigned char sm[LDS_BYTES];
  poison_lds(sm, LDS_BYTES);
  unsigned char* const kt = sm;
  unsigned char* const vt = sm + KV_BYTES;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r = lane & 31, hh = lane >> 5;
  const int kbw = wave & 3, half = wave >> 2;

  int64_t rest = blockIdx.x;
  if (p.xcd_group) {
    const int64_t x = rest % 8, j = rest / 8;
    rest = ((j / p.n_kblocks) * 8 + x) * p.n_kblocks + j % p.n_kblocks;
  }
  const int kbk = (int)(rest % p.n_kblocks);
  rest /= p.n_kblocks;
  const int hk = (int)(rest % p.Hkv);
  const int seg = (int)(rest / p.Hkv);
  const Seg sg = segment(p, seg);
  const int64_t k0 = (int64_t)kbk * kBlk;
  if (k0 >= sg.len) return;  // whole workgroup, before any barrier
  const int64_t kw = k0 + 32 * kbw;
  const int64_t key = kw + r;
  const bool key_ok = key < sg.len;

  // the 128 keys' K and V rows into LDS (rows past the end repeat the last key)
#pragma unroll
  for (int u = 0; u < NKV; ++u) {
    const int idx = tid + NTH * u, row = idx / CPR, ch = idx % CPR;
    int64_t kk = k0 + row;
    kk = kk < sg.len ? kk : sg.len - 1;
    const int64_t e = ((sg.start + kk) * p.Hkv + hk) * D + 8 * ch;
    *reinterpret_cast<uint4*>(kt + row * PITCH + 16 * ch) = load_chunk_bf16<false>(p.k, e);
    *reinterpret_cast<uint4*>(vt + row * PITCH + 16 * ch) = load_chunk_bf16<false>(p.v, e);
  }

  bf32x16 dka[DT], dva[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) dka[dt][i] = dva[dt][i] = 0.f;

  const float c2 = p.scale_log2;
  const int64_t tstart = p.causal ? k0 / kTile * kTile : 0;
  const int ntq = (int)((sg.len - tstart + kTile - 1) / kTile);
  const int nsteps = p.G * ntq;  // (query head, query tile) pairs
  typedef uint32_t stage_t __attribute__((ext_vector_type(4 * NLD)));
  struct Stage {
    stage_t q, o;
    float l, d;
  };
  auto gload = [&](int step) __attribute__((always_inline)) {
    Stage g;
    const int h = hk * p.G + step / ntq;
    const int64_t tq0 = tstart + (int64_t)(step % ntq) * kTile;
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int idx = tid + NTH * u, row = idx / CPR, ch = idx % CPR;
      int64_t tq = tq0 + row;
      tq = tq < sg.len ? tq : sg.len - 1;  // rows past the end repeat the last token (masked)
      const int64_t e = ((sg.start + tq) * p.Hq + h) * D + 8 * ch;
      const uint4 a = load_chunk_bf16<false>(p.q, e), b = load_chunk_bf16<GF32>(p.dout, e);
      g.q[4 * u] = a.x;
      g.q[4 * u + 1] = a.y;
      g.q[4 * u + 2] = a.z;
      g.q[4 * u + 3] = a.w;
      g.o[4 * u] = b.x;
      g.o[4 * u + 1] = b.y;
      g.o[4 * u + 2] = b.z;
      g.o[4 * u + 3] = b.w;
    }
    g.l = g.d = 0.f;
    if (tid < kTile) {
      int64_t tq = tq0 + tid;
      tq = tq < sg.len ? tq : sg.len - 1;
      const int64_t nq = sg.start + tq;
      g.l = p.lse[lse_index(p, nq, h)] * kLog2e;
      g.d = p.delta[(int64_t)h * p.total_tokens + nq];
    }
    return g;
  };
  auto sstore = [&](const Stage& g, int b) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int idx = tid + NTH * u, row = idx / CPR, ch = idx % CPR;
      *reinterpret_cast<uint4*>(sm + OFF_Q + b * TILE_BYTES + row * PITCH + 16 * ch) =
          make_uint4(g.q[4 * u], g.q[4 * u + 1], g.q[4 * u + 2], g.q[4 * u + 3]);
      *reinterpret_cast<uint4*>(sm + OFF_O + b * TILE_BYTES + row * PITCH + 16 * ch) =
          make_uint4(g.o[4 * u], g.o[4 * u + 1], g.o[4 * u + 2], g.o[4 * u + 3]);
    }
    if (tid < kTile) {
      reinterpret_cast<float*>(sm + OFF_L)[b * kTile + tid] = g.l;
      reinterpret_cast<float*>(sm + OFF_D)[b * kTile + tid] = g.d;
    }
  };

  // step i reads buffer i % 2 while step i + 1's tile is stored into the other
  Stage next;
  if (nsteps > 0) {
    next = gload(0);
    sstore(next, 0);
  }
  __syncthreads();  // also publishes the K/V rows
  if (nsteps > 1) next = gload(1);
  for (int step = 0; step < nsteps; ++step) {
    const int b = step & 1;
    const unsigned char* qs = sm + OFF_Q + b * TILE_BYTES;
    const unsigned char* os = sm + OFF_O + b * TILE_BYTES;
    const float* lse2s = reinterpret_cast<const float*>(sm + OFF_L) + b * kTile;
    const float* dels = reinterpret_cast<const float*>(sm + OFF_D) + b * kTile;
    const int64_t q0 = tstart + (int64_t)(step % ntq) * kTile + 32 * half;
    if (q0 < sg.len && !(p.causal && q0 + 31 < kw)) {  // wave-uniform
      bf32x16 sc, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[i] = dp[i] = 0.f;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const int off = (32 * half + r) * PITCH + 16 * (2 * kc + hh);   // this lane's query row
        const int koff = (32 * kbw + r) * PITCH + 16 * (2 * kc + hh);  // this lane's key row
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_b8(*reinterpret_cast<const uint4*>(qs + off)),
                                                     as_b8(*reinterpret_cast<const uint4*>(kt + koff)), sc, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_b8(*reinterpret_cast<const uint4*>(os + off)),
                                                     as_b8(*reinterpret_cast<const uint4*>(vt + koff)), dp, 0, 0, 0);
      }
      // register i holds token q0 + 8 (i / 4) + 4 hh + i % 4 and key `key`
      uint32_t pp[8], dsp[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 l4 = *reinterpret_cast<const float4*>(lse2s + 32 * half + 8 * j + 4 * hh);
        const float4 d4 = *reinterpret_cast<const float4*>(dels + 32 * half + 8 * j + 4 * hh);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dv4[4] = {d4.x, d4.y, d4.z, d4.w};
        float pv[4], dsv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = 4 * j + u;
          const int64_t tq = q0 + 8 * j + 4 * hh + u;
          const bool vis = key_ok && tq < sg.len && (!p.causal || key <= tq);
          const float pr = vis ? __builtin_amdgcn_exp2f(sc[i] * c2 - lv[u]) : 0.f;
          pv[u] = pr;
          dsv[u] = pr * (dp[i] - dv4[u]);
        }
        pp[2 * j] = rowops::pack_bf16x2(pv[0], pv[1]);
        pp[2 * j + 1] = rowops::pack_bf16x2(pv[2], pv[3]);
        dsp[2 * j] = rowops::pack_bf16x2(dsv[0], dsv[1]);
        dsp[2 * j + 1] = rowops::pack_bf16x2(dsv[2], dsv[3]);
      }
#pragma unroll
      for (int part = 0; part < 2; ++part)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          dva[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand<PITCH>(os, 32 * half + 16 * part, dt, lane),
                                                            pk_b8(pp + 4 * part), dva[dt], 0, 0, 0);
          dka[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand<PITCH>(qs, 32 * half + 16 * part, dt, lane),
                                                            pk_b8(dsp + 4 * part), dka[dt], 0, 0, 0);
        }
    }
    if (step + 1 < nsteps) sstore(next, (step + 1) & 1);
    __syncthreads();
    if (step + 2 < nsteps) next = gload(step + 2);
  }

  // the second wave of each key block hands its partial sums to the first
  float* part = reinterpret_cast<float*>(sm) + (size_t)kbw * 64 * 2 * DT * 16 + (size_t)lane * 2 * DT * 16;
  if (half == 1) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; i += 4) {
        *reinterpret_cast<float4*>(part + dt * 16 + i) = make_float4(dka[dt][i], dka[dt][i + 1], dka[dt][i + 2], dka[dt][i + 3]);
        *reinterpret_cast<float4*>(part + (DT + dt) * 16 + i) =
            make_float4(dva[dt][i], dva[dt][i + 1], dva[dt][i + 2], dva[dt][i + 3]);
      }
  }
  __syncthreads();
  if (half == 1 || !key_ok) return;
  const int64_t nk = sg.start + key;
  const int64_t e = (nk * p.Hkv + hk) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = 32 * dt + 8 * j + 4 * hh;
      const float4 pk = *reinterpret_cast<const float4*>(part + dt * 16 + 4 * j);
      const float4 pv = *reinterpret_cast<const float4*>(part + (DT + dt) * 16 + 4 * j);
      const float xk[4] = {(dka[dt][4 * j] + pk.x) * p.scale, (dka[dt][4 * j + 1] + pk.y) * p.scale,
                           (dka[dt][4 * j + 2] + pk.z) * p.scale, (dka[dt][4 * j + 3] + pk.w) * p.scale};
      const float xv[4] = {dva[dt][4 * j] + pv.x, dva[dt][4 * j + 1] + pv.y, dva[dt][4 * j + 2] + pv.z,
                           dva[dt][4 * j + 3] + pv.w};
      store_n<GF32, 4>(p.dk, e + c, xk);
      store_n<GF32, 4>(p.dv, e + c, xv);
    }
}

// ---------------------------------------------------------------- fp32 (vector)
// dq: one wave per (packed token, query head); lane groups take NGRP keys at a time.
template <int D>
__global__ __launch_bounds__(64 * kBwdWaves) void moda_bwd_dq_f32_kernel(const BwdParams p) {
  constexpr int LPR = D / 8, NGRP = 64 / LPR;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane / LPR, cl = lane % LPR;
  const int64_t item = (int64_t)blockIdx.x * kBwdWaves + wave;
  if (item >= p.total_tokens * p.Hq) return;
  const int64_t n = item / p.Hq;
  const int h = (int)(item % p.Hq), hk = h / p.G;
  const Seg sg = segment_of(p, n);
  const int64_t t = n - sg.start;
  float q8[8], do8[8], acc[8];
  load8<false>(p.q, (n * p.Hq + h) * D + 8 * cl, q8);
  load8<false>(p.dout, (n * p.Hq + h) * D + 8 * cl, do8);
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  const float lse2 = p.lse[lse_index(p, n, h)] * kLog2e;
  const float dl = p.delta[(int64_t)h * p.total_tokens + n];
  const int64_t nkeys = p.causal ? t + 1 : sg.len;
  for (int64_t j0 = 0; j0 < nkeys; j0 += NGRP) {
    const int64_t j = j0 + grp;
    const bool vis = j < nkeys;
    const int64_t e = ((sg.start + (vis ? j : nkeys - 1)) * p.Hkv + hk) * D + 8 * cl;
    float k8[8], v8[8];
    load8<false>(p.k, e, k8);
    load8<false>(p.v, e, v8);
    float s = 0.f, dp = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      s = fmaf(q8[c], k8[c], s);
      dp = fmaf(do8[c], v8[c], dp);
    }
    s = group_sum<LPR>(s);
    dp = group_sum<LPR>(dp);
    const float pr = vis ? __builtin_amdgcn_exp2f(s * p.scale_log2 - lse2) : 0.f;
    const float ds = pr * (dp - dl);
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = fmaf(ds, k8[c], acc[c]);
  }
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] += __shfl_xor(acc[c], off);
  if (grp != 0) return;
  const int64_t e = (n * p.Hq + h) * D + 8 * cl;
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] *= p.scale;
  if (p.n_depth > 0) {
    const float4 a = *reinterpret_cast<const float4*>(p.dq_depth + e);
    const float4 b = *reinterpret_cast<const float4*>(p.dq_depth + e + 4);
    acc[0] += a.x; acc[1] += a.y; acc[2] += a.z; acc[3] += a.w;
    acc[4] += b.x; acc[5] += b.y; acc[6] += b.z; acc[7] += b.w;
  }
  store_n<true, 8>(p.dq, e, acc);
}

// dk / dv: one wave per (packed key token, KV head); lane groups take NGRP query
// tokens at a time, for each of the G query heads.
template <int D>
__global__ __launch_bounds__(64 * kBwdWaves) void moda_bwd_dkv_f32_kernel(const BwdParams p) {
  constexpr int LPR = D / 8, NGRP = 64 / LPR;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane / LPR, cl = lane % LPR;
  const int64_t item = (int64_t)blockIdx.x * kBwdWaves + wave;
  if (item >= p.total_tokens * p.Hkv) return;
  const int64_t n = item / p.Hkv;
  const int hk = (int)(item % p.Hkv);
  const Seg sg = segment_of(p, n);
  const int64_t j = n - sg.start;
  float k8[8], v8[8], dk8[8], dv8[8];
  load8<false>(p.k, (n * p.Hkv + hk) * D + 8 * cl, k8);
  load8<false>(p.v, (n * p.Hkv + hk) * D + 8 * cl, v8);
#pragma unroll
  for (int c = 0; c < 8; ++c) dk8[c] = dv8[c] = 0.f;
  const int64_t tbeg = p.causal ? j : 0;
  for (int g = 0; g < p.G; ++g) {
    const int h = hk * p.G + g;
    for (int64_t t0 = tbeg; t0 < sg.len; t0 += NGRP) {
      const int64_t t = t0 + grp;
      const bool vis = t < sg.len;
      const int64_t nq = sg.start + (vis ? t : sg.len - 1);
      const int64_t e = (nq * p.Hq + h) * D + 8 * cl;
      float q8[8], do8[8];
      load8<false>(p.q, e, q8);
      load8<false>(p.dout, e, do8);
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        s = fmaf(q8[c], k8[c], s);
        dp = fmaf(do8[c], v8[c], dp);
      }
      s = group_sum<LPR>(s);
      dp = group_sum<LPR>(dp);
      const float lse2 = p.lse[lse_index(p, nq, h)] * kLog2e;
      const float dl = p.delta[(int64_t)h * p.total_tokens + nq];
      const float pr = vis ? __builtin_amdgcn_exp2f(s * p.scale_log2 - lse2) : 0.f;
      const float ds = pr * (dp - dl);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        dv8[c] = fmaf(pr, do8[c], dv8[c]);
        dk8[c] = fmaf(ds, q8[c], dk8[c]);
      }
    }
  }
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      dk8[c] += __shfl_xor(dk8[c], off);
      dv8[c] += __shfl_xor(dv8[c], off);
    }
  if (grp != 0) return;
#pragma unroll
  for (int c = 0; c < 8; ++c) dk8[c] *= p.scale;
  const int64_t e = (n * p.Hkv + hk) * D + 8 * cl;
  store_n<true, 8>(p.dk, e, dk8);
  store_n<true, 8>(p.dv, e, dv8);
}

template <int D, bool BF16, bool GF32>
void launch_prep(int gc, dim3 grid, dim3 block, size_t lds, hipStream_t stream, const BwdParams& p) {
  switch (gc) {
    case 1: hipLaunchKernelGGL((moda_bwd_prep_kernel<D, BF16, GF32, 1>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((moda_bwd_prep_kernel<D, BF16, GF32, 2>), grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL((moda_bwd_prep_kernel<D, BF16, GF32, 4>), grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL((moda_bwd_prep_kernel<D, BF16, GF32, 0>), grid, block, lds, stream, p); break;
  }
}

template <int D>
hipError_t launch_bwd_d(const BwdParams& p, bool bf16, bool grad_f32, hipStream_t stream) {
  const dim3 block(64 * kBwdWaves);
  // prep: G in {1, 2, 4} keeps the heads' state in registers; other G use LDS,
  // with waves per workgroup chosen so that it stays within 64 KB
  const int gc = (p.G == 1 || p.G == 2 || p.G == 4) ? p.G : 0;
  const size_t wave_lds = gc ? 0 : (size_t)prep_wave_floats(p.G, D) * sizeof(float);
  int wpb = 4;
  while (wpb > 1 && wave_lds * wpb > (size_t)kPrepMaxLds) wpb /= 2;
  const int64_t items = p.total_tokens * ((p.Hkv + prep_ngrp<D>() - 1) / prep_ngrp<D>());
  const dim3 prep_grid((unsigned)((items + wpb - 1) / wpb)), prep_block(64 * wpb);
  const size_t lds = wave_lds * wpb;
  if (bf16 && grad_f32)
    launch_prep<D, true, true>(gc, prep_grid, prep_block, lds, stream, p);
  else if (bf16)
    launch_prep<D, true, false>(gc, prep_grid, prep_block, lds, stream, p);
  else
    launch_prep<D, false, true>(gc, prep_grid, prep_block, lds, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (bf16) {
    const dim3 gq((unsigned)((int64_t)p.n_seg * p.Hq * p.n_qblocks));
    const dim3 gk((unsigned)((int64_t)p.n_seg * p.Hkv * p.n_kblocks));
    const dim3 block8(64 * kDkv8Waves);
    if (grad_f32) {
      hipLaunchKernelGGL((moda_bwd_dq_kernel<D, true>), gq, block, 0, stream, p);
      hipLaunchKernelGGL((moda_bwd_dkv8_kernel<D, true>), gk, block8, 0, stream, p);
    } else {
      hipLaunchKernelGGL((moda_bwd_dq_kernel<D, false>), gq, block, 0, stream, p);
      hipLaunchKernelGGL((moda_bwd_dkv8_kernel<D, false>), gk, block8, 0, stream, p);
    }
  } else {
    const dim3 gq((unsigned)((p.total_tokens * p.Hq + kBwdWaves - 1) / kBwdWaves));
    const dim3 gk((unsigned)((p.total_tokens * p.Hkv + kBwdWaves - 1) / kBwdWaves));
    hipLaunchKernelGGL((moda_bwd_dq_f32_kernel<D>), gq, block, 0, stream, p);
    hipLaunchKernelGGL((moda_bwd_dkv_f32_kernel<D>), gk, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdParams& p, int head_dim, bool bf16, bool grad_f32, hipStream_t stream) {
  if (head_dim == 128) return launch_bwd_d<128>(p, bf16, grad_f32, stream);
  if (head_dim == 64) return launch_bwd_d<64>(p, bf16, grad_f32, stream);
  return hipErrorInvalidValue;
}

}  // namespace moda

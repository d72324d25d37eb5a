// Slot selection for bounded depth reads (top-S, sliding window, hybrid).
//
// The MoDA deck lists a bounded S << L slot buffer (top-S, sliding window or
// hybrid) as future work (slide "The main open cost is retaining and reading
// depth history", paper Sec. 6.1-6.2) without defining it. Reading taken: of a
// query row's slots [0, n_depth), the last `recent` always enter its joint
// softmax; of the others, the `topk` with the largest depth logits
// b_i = scale <q, k_depth_i> enter, ties to the lower slot index.
//
// One wave per (token, KV head): LPR = D / 8 lanes hold a 16-byte slice of a slot
// row, so a wave-wide load covers 64 / LPR slots; all of the token's slot keys
// (n_depth <= 64) stay in registers, as fp32, while the G query heads of the KV
// head are scored against them (fp32 FMA, DPP group sums). Per head,
// lane i then ranks slot i among the older slots by (logit descending, index
// ascending) and a ballot gives the 64-bit mask of the slots that enter, written
// to mask[token * Hq + head]. The fp32 forward reads the mask and leaves the
// other slots out of the softmax (the bf16 forward selects inside its own depth
// pass). The selection only decides membership: the forward recomputes the kept
// logits itself.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moda_internal.h"
#include "moda_rowops.h"

namespace moda {
namespace {

constexpr int kSelWaves = 4;  // (token, KV head) units per workgroup
constexpr float kNegInf = -__builtin_inff();

template <int D, bool BF16>
__global__ __launch_bounds__(64 * kSelWaves) void moda_depth_select_kernel(const SelectParams p) {
  constexpr int LPR = D / 8;          // lanes per slot row
  constexpr int NGRP = 64 / LPR;      // slot rows per wave-wide load
  constexpr int NB = 64 / NGRP;       // loads covering 64 slots
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane / LPR, cl = lane % LPR;
  // every wave runs the same loops (the barriers below need all of them): a wave
  // past the last unit recomputes the last one and writes nothing
  const int64_t n_units = p.n_tokens * p.Hkv;
  const int64_t unit0 = (int64_t)blockIdx.x * kSelWaves + wave;  // token * Hkv + hk
  const bool active = unit0 < n_units;
  const int64_t unit = active ? unit0 : n_units - 1;
  const int64_t n = unit / p.Hkv;
  const int hk = (int)(unit % p.Hkv);
  const int S = p.n_depth;
  __shared__ float logit[kSelWaves][64];
  poison_lds(logit, sizeof(logit));

  // the token's slot keys: slice cl of slot b * NGRP + grp in kx[b]
  float kx[NB][8];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int slot = b * NGRP + grp;
    if (slot < S) {
      rowops::load8<BF16>(p.kd, ((n * p.S_cap + slot) * p.Hkv + hk) * (int64_t)D + 8 * cl, kx[b]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) kx[b][j] = 0.f;
    }
  }
  const int n_old = S - p.recent;  // slots [n_old, S) always enter
  for (int g = 0; g < p.G; ++g) {
    const int h = hk * p.G + g;
    float qx[8];
    rowops::load8<BF16>(p.q, (n * p.Hq + h) * (int64_t)D + 8 * cl, qx);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) s = fmaf(qx[j], kx[b][j], s);
      s = rowops::group_sum<LPR>(s);
      const int slot = b * NGRP + grp;
      if (cl == 0) logit[wave][slot] = slot < S ? s * p.scale : kNegInf;
    }
    __syncthreads();  // the logits of all slots are in LDS
    // lane i: rank of slot i among the older slots
    const float bi = logit[wave][lane];
    int rank = 0;
    for (int j = 0; j < n_old; ++j) {
      const float bj = logit[wave][j];
      rank += (bj > bi || (bj == bi && j < lane)) ? 1 : 0;
    }
    const bool keep = (lane < n_old && rank < p.topk) || (lane >= n_old && lane < S);
    const uint64_t m = __ballot(keep);
    if (lane == 0 && active) p.mask[n * p.Hq + h] = m;
    __syncthreads();  // every lane has read the logits before the next head overwrites them
  }
}

}  // namespace

hipError_t launch_depth_select(const SelectParams& p, int head_dim, bool bf16, hipStream_t stream) {
  const int64_t units = p.n_tokens * p.Hkv;
  const dim3 grid((unsigned)((units + kSelWaves - 1) / kSelWaves)), block(64 * kSelWaves);
  if (head_dim == 128) {
    if (bf16)
      hipLaunchKernelGGL((moda_depth_select_kernel<128, true>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((moda_depth_select_kernel<128, false>), grid, block, 0, stream, p);
  } else if (head_dim == 64) {
    if (bf16)
      hipLaunchKernelGGL((moda_depth_select_kernel<64, true>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((moda_depth_select_kernel<64, false>), grid, block, 0, stream, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moda

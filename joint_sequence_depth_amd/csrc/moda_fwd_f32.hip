// MoDA joint sequence/depth attention forward for fp32 inputs (the full-precision
// path; no rounding below fp32 anywhere).
//
// Same operator as the bf16 kernel (MoDA deck, slide "One denominator allocates
// probability across both memories"): one softmax over the causal sequence keys
// and the token's own depth slots, kept as the running state (m, acc, o) of slide
// "Shared online-softmax states preserve the joint operator", in base 2.
//
// One thread per query row, 64 rows (one wave) per workgroup, one query head per
// workgroup. Every lane of the wave reads the same key row at the same time, so
// the sequence loads are broadcasts; the depth slots are per row.
#include "moda_internal.h"

namespace moda {
namespace {

constexpr float NEG_INF = -__builtin_inff();
constexpr float LN2 = 0.693147180559945309417f;

template <int D>
__device__ __forceinline__ float dot_row(const float (&q)[D], const float* __restrict__ x) {
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
  for (int c = 0; c < D; c += 4) {
    const float4 w = *reinterpret_cast<const float4*>(x + c);
    s0 = fmaf(q[c + 0], w.x, s0);
    s1 = fmaf(q[c + 1], w.y, s1);
    s2 = fmaf(q[c + 2], w.z, s2);
    s3 = fmaf(q[c + 3], w.w, s3);
  }
  return (s0 + s1) + (s2 + s3);
}

template <int D>
__device__ __forceinline__ void update(float x, const float* __restrict__ vrow, float& m, float& l, float (&o)[D]) {
  const float m_new = fmaxf(m, x);
  const float alpha = __builtin_amdgcn_exp2f(m - m_new);  // m = -inf at the first key: alpha = 0
  const float pr = __builtin_amdgcn_exp2f(x - m_new);
  l = fmaf(l, alpha, pr);
#pragma unroll
  for (int c = 0; c < D; c += 4) {
    const float4 w = *reinterpret_cast<const float4*>(vrow + c);
    o[c + 0] = fmaf(o[c + 0], alpha, pr * w.x);
    o[c + 1] = fmaf(o[c + 1], alpha, pr * w.y);
    o[c + 2] = fmaf(o[c + 2], alpha, pr * w.z);
    o[c + 3] = fmaf(o[c + 3], alpha, pr * w.w);
  }
  m = m_new;
}

template <int D>
__global__ __launch_bounds__(64) void moda_fwd_f32_kernel(const Params p) {
  int64_t rest = blockIdx.x;
  const int qb = (int)(rest % p.n_qblocks);
  rest /= p.n_qblocks;
  const int h = (int)(rest % p.Hq);
  const int seg = (int)(rest / p.Hq);

  int64_t seg_start, len;
  if (p.cu_seqlens) {
    int64_t a = p.cu_seqlens[seg], b = p.cu_seqlens[seg + 1];
    a = a < 0 ? 0 : (a > p.total_tokens ? p.total_tokens : a);
    b = b < a ? a : (b > p.total_tokens ? p.total_tokens : b);
    seg_start = a;
    len = b - a;
  } else {
    seg_start = (int64_t)seg * p.uniform_len;
    len = p.uniform_len;
  }
  const int64_t t0 = (int64_t)qb * kF32BlockRows;
  if (t0 >= len) return;
  const int64_t t = t0 + threadIdx.x;
  const bool valid = t < len;
  const int hk = h / p.G;
  const float c2 = p.scale_log2;
  const float* __restrict__ Q = static_cast<const float*>(p.q);
  const float* __restrict__ K = static_cast<const float*>(p.k);
  const float* __restrict__ V = static_cast<const float*>(p.v);

  float q[D], o[D];
  const int64_t n = seg_start + (valid ? t : 0);
  {
    const float* qrow = Q + (n * p.Hq + h) * (int64_t)D;
#pragma unroll
    for (int c = 0; c < D; c += 4) {
      float4 w = valid ? *reinterpret_cast<const float4*>(qrow + c) : make_float4(0.f, 0.f, 0.f, 0.f);
      q[c] = w.x; q[c + 1] = w.y; q[c + 2] = w.z; q[c + 3] = w.w;
    }
  }
#pragma unroll
  for (int c = 0; c < D; ++c) o[c] = 0.f;
  float m = NEG_INF, l = 0.f;

  // depth slots of this token (left out when the launch computes the sequence part alone)
  if (valid && p.n_depth > 0 && (p.phase & kPhaseDepth)) {
    const float* KD = static_cast<const float*>(p.kd);
    const float* VD = static_cast<const float*>(p.vd);
    // bounded depth reads: the slots this row's selection keeps (all without one)
    const uint64_t sel = p.depth_mask ? p.depth_mask[n * p.Hq + h] : ~0ull;
    for (int i = 0; i < p.n_depth; ++i) {
      if (!((sel >> (i & 63)) & 1ull)) continue;  // (a mask exists only for n_depth <= 64)
      const int64_t off = ((n * p.S_cap + i) * p.Hkv + hk) * (int64_t)D;
      update<D>(dot_row<D>(q, KD + off) * c2, VD + off, m, l, o);
    }
  }
  // sequence keys j <= t (all of the segment without the causal mask)
  const int64_t last_row = (t0 + 63 < len - 1) ? t0 + 63 : len - 1;
  // (no keys when the launch computes the depth part alone)
  const int64_t jmax = !(p.phase & kPhaseSeq) ? -1 : p.causal ? last_row : len - 1;
  const int64_t my_jmax = p.causal ? t : len - 1;
  for (int64_t j = 0; j <= jmax; ++j) {
    if (valid && j <= my_jmax) {
      const int64_t off = ((seg_start + j) * p.Hkv + hk) * (int64_t)D;
      update<D>(dot_row<D>(q, K + off) * c2, V + off, m, l, o);
    }
  }
  if (valid) {
    const float inv = 1.f / l;
    float* orow = static_cast<float*>(p.out) + (n * p.Hq + h) * (int64_t)D;
#pragma unroll
    for (int c = 0; c < D; c += 4)
      *reinterpret_cast<float4*>(orow + c) = make_float4(o[c] * inv, o[c + 1] * inv, o[c + 2] * inv, o[c + 3] * inv);
    if (p.lse) {
      const int64_t lbase = p.lse_batch_layout ? (int64_t)seg * p.Hq * p.lse_head_stride : seg_start;
      p.lse[lbase + (int64_t)h * p.lse_head_stride + t] = (m + __log2f(l)) * LN2;
    }
  }
}

}  // namespace

hipError_t launch_fwd_f32(const Params& p, int head_dim, hipStream_t stream) {
  if (head_dim == 128) {
    hipLaunchKernelGGL((moda_fwd_f32_kernel<128>), dim3((unsigned)p.n_tiles), dim3(64), 0, stream, p);
  } else if (head_dim == 64) {
    hipLaunchKernelGGL((moda_fwd_f32_kernel<64>), dim3((unsigned)p.n_tiles), dim3(64), 0, stream, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moda

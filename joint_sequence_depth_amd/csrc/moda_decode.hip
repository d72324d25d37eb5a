// MoDA joint sequence/depth attention for a decode step: one new token per
// sequence attends to its sequence-cache prefix and to its own depth slots
// through ONE softmax (MoDA, arXiv 2603.15619; deck slide "One denominator
// allocates probability across both memories"; the decode caches are those of the
// paper's Table 1 as the deck quotes it).
//
// With one query row per (sequence, head) there is no matrix product to feed the
// matrix cores: each key row is read once and dotted with the GD query heads that
// share its KV head, so the step is bound by HBM (G flops per byte). Two kernels:
//
//  * partial: a workgroup of DW waves per (sequence, KV head, head group, key
//    chunk). LPR = D / 8 lanes hold one 8-element slice of a key row, so one
//    wave-wide load covers NGRP = 64 / LPR rows; each lane group keeps, per head,
//    the running max (base 2), the running sum and its slice of the weighted value
//    sum, loads U rows ahead of the arithmetic in registers, and the lane groups
//    and waves merge by the online-softmax update at the end. The depth slots of
//    the token have the same row stride as the cache (H_kv d elements), so they are
//    one more chunk. Partial states go to the caller's workspace.
//  * merge: per (sequence, query head) the chunks' states merge into the output
//    and the natural-log lse, normalised once.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moda_internal.h"
#include "moda_rowops.h"

namespace moda {
namespace {

typedef __bf16 dbf16x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309417f;
constexpr int kDecWaves = 4;  // waves per partial workgroup (2 and 8 measured slower)
constexpr int kDecU = 4;      // key rows per lane group per load batch (8 costs occupancy)

__device__ __forceinline__ float d_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float d_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float d_dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(dbf16x2, a), __builtin_bit_cast(dbf16x2, b), c, false);
}

// 8 consecutive elements of a row, as stored (bf16: one 16-byte word; fp32: two),
// loaded with the non-temporal hint: a step reads each cache and slot row once.
template <bool BF16>
struct Slice {
  uint4 w[BF16 ? 1 : 2];
};
template <bool BF16>
__device__ __forceinline__ Slice<BF16> load_slice(const void* base, int64_t elem) {
  Slice<BF16> s;
  if constexpr (BF16) {
    s.w[0] = rowops::stream_load16(static_cast<const uint16_t*>(base) + elem);
  } else {
    const float* p = static_cast<const float*>(base) + elem;
    s.w[0] = rowops::stream_load16(p);
    s.w[1] = rowops::stream_load16(p + 4);
  }
  return s;
}
template <bool BF16>
__device__ __forceinline__ float elem(const Slice<BF16>& s, int i) {
  if constexpr (BF16) {
    const uint32_t w = i < 2 ? s.w[0].x : i < 4 ? s.w[0].y : i < 6 ? s.w[0].z : s.w[0].w;
    return (i & 1) ? d_hi(w) : d_lo(w);
  } else {
    const uint4 q = s.w[i >> 2];
    const uint32_t w = (i & 3) == 0 ? q.x : (i & 3) == 1 ? q.y : (i & 3) == 2 ? q.z : q.w;
    return __uint_as_float(w);
  }
}
// <q slice, k slice> in fp32
template <bool BF16>
__device__ __forceinline__ float dot8(const Slice<BF16>& q, const Slice<BF16>& k) {
  if constexpr (BF16) {
    float s = d_dot2(q.w[0].x, k.w[0].x, 0.f);
    s = d_dot2(q.w[0].y, k.w[0].y, s);
    s = d_dot2(q.w[0].z, k.w[0].z, s);
    return d_dot2(q.w[0].w, k.w[0].w, s);
  } else {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s = fmaf(elem<false>(q, i), elem<false>(k, i), s);
    return s;
  }
}

// Merges running state (mb, lb, rb, ob) into (ma, la, ra, oa), base-2 units.
__device__ __forceinline__ void merge_state(float& ma, float& la, float& ra, float (&oa)[8], float mb, float lb,
                                            float rb, const float (&ob)[8]) {
  const float m = fmaxf(ma, mb);
  const float mu = m == kNegInf ? 0.f : m;
  const float fa = __builtin_amdgcn_exp2f(ma - mu), fb = __builtin_amdgcn_exp2f(mb - mu);
  la = la * fa + lb * fb;
  ra = ra * fa + rb * fb;
#pragma unroll
  for (int j = 0; j < 8; ++j) oa[j] = oa[j] * fa + ob[j] * fb;
  ma = m;
}

template <int D, int GD, bool BF16>
__global__ __launch_bounds__(64 * kDecWaves) void moda_decode_partial_kernel(const DecodeParams p) {
  constexpr int LPR = D / 8;
  constexpr int NGRP = 64 / LPR;
  constexpr int U = kDecU;
  constexpr int NBUF = 2;
  constexpr int ROWS_PER_BATCH = NGRP * U;  // key rows one wave consumes per batch
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = lane / LPR, cl = lane % LPR;
  __shared__ float red[kDecWaves][GD][D + 4];  // per wave: o slices, then m, l and r
  poison_lds(red, sizeof(red));

  // workgroup -> (sequence b, KV head hk, head group hg, chunk s)
  int64_t id = blockIdx.x;
  const int s = (int)(id % p.n_chunks);
  id /= p.n_chunks;
  const int hg = (int)(id % p.n_hgroups);
  id /= p.n_hgroups;
  const int hk = (int)(id % p.Hkv);
  const int b = (int)(id / p.Hkv);

  int64_t L = p.cache_seqlens[b];
  L = L < 1 ? 1 : (L > p.T_max ? p.T_max : L);  // the token's own key is always there
  const bool depth_chunk = s == p.n_seq_chunks;
  const int64_t r0 = depth_chunk ? 0 : (int64_t)s * p.chunk;
  const int64_t r1 = depth_chunk ? p.n_depth : (r0 + p.chunk < L ? r0 + p.chunk : L);
  if (r0 >= r1) return;  // chunk past this sequence's cache (the merge does not read it)

  const int64_t row_stride = (int64_t)p.Hkv * D;  // cache and depth rows alike
  const int64_t base_row = depth_chunk ? ((int64_t)b * p.S_cap) * p.Hkv + hk : ((int64_t)b * p.T_max) * p.Hkv + hk;
  const void* KB = depth_chunk ? p.kd : p.kc;
  const void* VB = depth_chunk ? p.vd : p.vc;
  const int h0 = hk * p.G + hg * GD;  // first query head of the group
  const float c2 = p.scale_log2;

  Slice<BF16> qs[GD];
#pragma unroll
  for (int g = 0; g < GD; ++g) qs[g] = load_slice<BF16>(p.q, ((int64_t)b * p.Hq + h0 + g) * D + 8 * cl);

  // per head: running max m (base 2), sum l of the weights, sum r of the weights
  // as rounded to bf16 for the value products (bf16 inputs; = l for fp32), and
  // this lane's slice o of the weighted value sum
  float m[GD], l[GD], rr[GD], o[GD][8];
#pragma unroll
  for (int g = 0; g < GD; ++g) {
    m[g] = kNegInf;
    l[g] = 0.f;
    rr[g] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) o[g][j] = 0.f;
  }

  // this wave's batches: rows r0 + (wave + k DW) ROWS_PER_BATCH + u NGRP + grp
  const int64_t n_rows = r1 - r0;
  const int n_batches = (int)((n_rows + ROWS_PER_BATCH - 1) / ROWS_PER_BATCH);
  const int my_batches = n_batches > wave ? (n_batches - wave + kDecWaves - 1) / kDecWaves : 0;
  auto row_of = [&](int k, int u) { return r0 + (int64_t)(wave + k * kDecWaves) * ROWS_PER_BATCH + u * NGRP + grp; };
  // Loads are unconditional (a fixed count per batch keeps the compiler's waits
  // exact): rows past the chunk re-read its last row and are masked.
  auto issue = [&](int k, Slice<BF16>(&kw)[U], Slice<BF16>(&vw)[U]) {
    k = k < my_batches ? k : my_batches - 1;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int64_t r = row_of(k, u);
      r = r < r1 ? r : r1 - 1;
      const int64_t e = (base_row + r * p.Hkv) * D + 8 * cl;
      kw[u] = load_slice<BF16>(KB, e);
      vw[u] = load_slice<BF16>(VB, e);
    }
  };
  auto process = [&](int k, const Slice<BF16>(&kw)[U], const Slice<BF16>(&vw)[U]) {
    // bf16: the values of row pairs (u, u + 1) interleaved per column, so that one
    // v_dot2 adds both rows' weighted values: vp[u / 2][c] = (v_u[c], v_{u+1}[c])
    uint32_t vp[U / 2][8];
    if constexpr (BF16) {
#pragma unroll
      for (int u = 0; u < U; u += 2) {
        const uint32_t a[4] = {vw[u].w[0].x, vw[u].w[0].y, vw[u].w[0].z, vw[u].w[0].w};
        const uint32_t b[4] = {vw[u + 1].w[0].x, vw[u + 1].w[0].y, vw[u + 1].w[0].z, vw[u + 1].w[0].w};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          vp[u / 2][2 * w] = __builtin_amdgcn_perm(b[w], a[w], 0x05040100u);      // low halves
          vp[u / 2][2 * w + 1] = __builtin_amdgcn_perm(b[w], a[w], 0x07060302u);  // high halves
        }
      }
    }
#pragma unroll
    for (int g = 0; g < GD; ++g) {
      float sc[U];
      float mx = kNegInf;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float t = rowops::group_sum<LPR>(dot8<BF16>(qs[g], kw[u])) * c2;
        t = row_of(k, u) < r1 ? t : kNegInf;
        sc[u] = t;
        mx = fmaxf(mx, t);
      }
      const float mn = fmaxf(m[g], mx);
      const float mu = mn == kNegInf ? 0.f : mn;
      const float alpha = __builtin_amdgcn_exp2f(m[g] - mu);
      l[g] *= alpha;
      rr[g] *= alpha;
#pragma unroll
      for (int j = 0; j < 8; ++j) o[g][j] *= alpha;
      if constexpr (BF16) {
#pragma unroll
        for (int u = 0; u < U; u += 2) {
          const float p0 = __builtin_amdgcn_exp2f(sc[u] - mu), p1 = __builtin_amdgcn_exp2f(sc[u + 1] - mu);
          l[g] += p0 + p1;
          const uint32_t pk = rowops::pack_bf16x2(p0, p1);
          rr[g] = d_dot2(pk, 0x3F803F80u, rr[g]);  // the two rounded weights (bf16 1.0 pair)
#pragma unroll
          for (int j = 0; j < 8; ++j) o[g][j] = d_dot2(pk, vp[u / 2][j], o[g][j]);
        }
      } else {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const float pu = __builtin_amdgcn_exp2f(sc[u] - mu);
          l[g] += pu;
#pragma unroll
          for (int j = 0; j < 8; ++j) o[g][j] = fmaf(pu, elem<BF16>(vw[u], j), o[g][j]);
        }
        rr[g] = l[g];
      }
      m[g] = mn;
    }
  };
  if (my_batches > 0) {
    Slice<BF16> kb[NBUF][U], vb[NBUF][U];
    issue(0, kb[0], vb[0]);
    for (int k = 0; k < my_batches; k += NBUF) {
#pragma unroll
      for (int j = 0; j < NBUF; ++j) {
        issue(k + j + 1, kb[(j + 1) % NBUF], vb[(j + 1) % NBUF]);
        if (k + j < my_batches) process(k + j, kb[j], vb[j]);
      }
    }
  }

  // merge the NGRP lane groups (lanes with the same slice cl), then the waves
#pragma unroll
  for (int g = 0; g < GD; ++g) {
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
      const float mb = __shfl_xor(m[g], off), lb = __shfl_xor(l[g], off), rb = __shfl_xor(rr[g], off);
      float ob[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) ob[j] = __shfl_xor(o[g][j], off);
      merge_state(m[g], l[g], rr[g], o[g], mb, lb, rb, ob);
    }
  }
  if (grp == 0) {
#pragma unroll
    for (int g = 0; g < GD; ++g) {
#pragma unroll
      for (int j = 0; j < 8; ++j) red[wave][g][8 * cl + j] = o[g][j];
      if (cl == 0) {
        red[wave][g][D] = m[g];
        red[wave][g][D + 1] = l[g];
        red[wave][g][D + 2] = rr[g];
      }
    }
  }
  __syncthreads();
  // one thread per (head, 8-element slice) writes the chunk's state
  float* ws = p.workspace;
  for (int t = tid; t < GD * LPR; t += 64 * kDecWaves) {
    const int g = t / LPR, c = t % LPR;
    float ma = kNegInf, la = 0.f, ra = 0.f, oa[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) oa[j] = 0.f;
    for (int w = 0; w < kDecWaves; ++w) {
      float ob[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) ob[j] = red[w][g][8 * c + j];
      merge_state(ma, la, ra, oa, red[w][g][D], red[w][g][D + 1], red[w][g][D + 2], ob);
    }
    // record [b][h][chunk]: o[D], m, l, r (stride D + 4 floats)
    float* rec = ws + (((int64_t)b * p.Hq + h0 + g) * p.n_chunks + s) * (D + 4);
    *reinterpret_cast<float4*>(rec + 8 * c) = make_float4(oa[0], oa[1], oa[2], oa[3]);
    *reinterpret_cast<float4*>(rec + 8 * c + 4) = make_float4(oa[4], oa[5], oa[6], oa[7]);
    if (c == 0) {
      rec[D] = ma;
      rec[D + 1] = la;
      rec[D + 2] = ra;
    }
  }
}

// One wave per (sequence, query head). The chunk states are read side by side,
// not one after another: the maximum first (lanes over chunks), then the weighted
// sums, NG chunks at a time with C4 lanes per chunk (one float4 of o each) and
// four rounds of loads in flight, the groups' partial sums added at the end.
template <int D, bool OUT_F32>
__global__ __launch_bounds__(64) void moda_decode_merge_kernel(const DecodeParams p) {
  constexpr int C4 = D / 4;     // float4 words of a state's o (16 or 32)
  constexpr int NG = 64 / C4;   // chunk states read side by side (4 or 2)
  constexpr int UR = 4;         // rounds of loads issued before they are used
  const int lane = threadIdx.x;
  const int64_t bh = blockIdx.x;  // b * Hq + h
  const int b = (int)(bh / p.Hq);
  int64_t L = p.cache_seqlens[b];
  L = L < 1 ? 1 : (L > p.T_max ? p.T_max : L);
  const int n_used = (int)((L + p.chunk - 1) / p.chunk);
  // the states written for this row: sequence chunks [0, n_used), then the depth chunk
  const int n_rec = n_used + (p.n_depth > 0 ? 1 : 0);
  const float* recs = p.workspace + bh * p.n_chunks * (D + 4);
  auto rec_of = [&](int i) { return recs + (int64_t)(i < n_used ? i : p.n_seq_chunks) * (D + 4); };

  float M = kNegInf;
  for (int i = lane; i < n_rec; i += 64) M = fmaxf(M, rec_of(i)[D]);
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
  const float mu = M == kNegInf ? 0.f : M;

  const int grp = lane / C4, c4 = lane % C4;
  float Z = 0.f, R = 0.f;  // Z: sum of the weights (for lse); R: as applied to the values
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int i0 = 0; i0 < n_rec; i0 += UR * NG) {
    float mi[UR], li[UR], ri[UR];
    float4 oi[UR];
#pragma unroll
    for (int u = 0; u < UR; ++u) {  // loads of all rounds first
      const int i = i0 + u * NG + grp;
      const float* rec = rec_of(i < n_rec ? i : 0);
      mi[u] = i < n_rec ? rec[D] : kNegInf;
      li[u] = rec[D + 1];
      ri[u] = rec[D + 2];
      oi[u] = *reinterpret_cast<const float4*>(rec + 4 * c4);
    }
#pragma unroll
    for (int u = 0; u < UR; ++u) {
      const float f = mi[u] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(mi[u] - mu);
      Z = fmaf(li[u], f, Z);
      R = fmaf(ri[u], f, R);
      acc.x = fmaf(oi[u].x, f, acc.x);
      acc.y = fmaf(oi[u].y, f, acc.y);
      acc.z = fmaf(oi[u].z, f, acc.z);
      acc.w = fmaf(oi[u].w, f, acc.w);
    }
  }
#pragma unroll
  for (int off = C4; off < 64; off <<= 1) {  // add the groups' sums
    Z += __shfl_xor(Z, off);
    R += __shfl_xor(R, off);
    acc.x += __shfl_xor(acc.x, off);
    acc.y += __shfl_xor(acc.y, off);
    acc.z += __shfl_xor(acc.z, off);
    acc.w += __shfl_xor(acc.w, off);
  }
  const float inv = R > 0.f ? 1.f / R : 0.f;
  if (grp == 0) {
    const int64_t e = bh * D + 4 * c4;
    if constexpr (OUT_F32) {
      *reinterpret_cast<float4*>(static_cast<float*>(p.out) + e) =
          make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    } else {
      typedef float f2 __attribute__((ext_vector_type(2)));
      const f2 v0 = {acc.x * inv, acc.y * inv}, v1 = {acc.z * inv, acc.w * inv};
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + e) =
          make_uint2(__builtin_bit_cast(uint32_t, __builtin_convertvector(v0, dbf16x2)),
                     __builtin_bit_cast(uint32_t, __builtin_convertvector(v1, dbf16x2)));
    }
    if (lane == 0 && p.lse) p.lse[bh] = (M + __log2f(Z)) * kLn2;
  }
}

template <int D, bool BF16>
hipError_t launch_partial(const DecodeParams& p, int gd, hipStream_t stream) {
  const dim3 grid((unsigned)p.n_partial_blocks), block(64 * kDecWaves);
  switch (gd) {
    case 1: hipLaunchKernelGGL((moda_decode_partial_kernel<D, 1, BF16>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((moda_decode_partial_kernel<D, 2, BF16>), grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL((moda_decode_partial_kernel<D, 4, BF16>), grid, block, 0, stream, p); break;
    case 8: hipLaunchKernelGGL((moda_decode_partial_kernel<D, 8, BF16>), grid, block, 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_dec(const DecodeParams& p, int gd, bool bf16, bool out_f32, hipStream_t stream) {
  hipError_t e = bf16 ? launch_partial<D, true>(p, gd, stream) : launch_partial<D, false>(p, gd, stream);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)(p.B * p.Hq)), block(64);
  if (out_f32)
    hipLaunchKernelGGL((moda_decode_merge_kernel<D, true>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((moda_decode_merge_kernel<D, false>), grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace

int decode_rows_per_chunk_unit(int head_dim) { return 64 / (head_dim / 8) * kDecU * kDecWaves; }

hipError_t launch_decode(const DecodeParams& p, int head_dim, int heads_per_block, bool bf16, bool out_f32,
                         hipStream_t stream) {
  if (head_dim == 128) return launch_dec<128>(p, heads_per_block, bf16, out_f32, stream);
  if (head_dim == 64) return launch_dec<64>(p, heads_per_block, bf16, out_f32, stream);
  return hipErrorInvalidValue;
}

}  // namespace moda

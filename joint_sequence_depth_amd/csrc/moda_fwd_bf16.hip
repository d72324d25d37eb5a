// Fused MoDA joint sequence/depth attention forward, bf16 storage, fp32 math.
//
// Operator (MoDA, arXiv 2603.15619; deck slide "One denominator allocates
// probability across both memories"): for query row (token t, head h) the causal
// sequence keys j <= t and the depth slots i of token t share ONE softmax:
//   o = (sum_j e^{a_j} v_j + sum_i e^{b_i} vd_i) / (sum_j e^{a_j} + sum_i e^{b_i}).
// The running state (m, acc, o) of slide "Shared online-softmax states preserve
// the joint operator" is carried in base 2: logits are multiplied by
// scale * log2(e) so that exp2 reproduces the natural exponential (deck backup
// slide "pseudocode needs implementation-level checks").
//
// Work unit: one workgroup (4 waves, 256 threads) owns 128 expanded query rows:
// TOK = 128 / GB tokens x GB query heads of one KV head (rows ordered token-major,
// row r -> token r / GB, head r % GB, as in the expanded-row map of the deck's
// backup slide on grouped indexing). Wave w owns rows [32 w, 32 w + 32).
//
// Phase 1, depth (HBM-bound): each wave streams the depth K/V of its tokens.
// LPR = D / 8 lanes hold one 16-byte slice of a slot row, so one 128-bit load per
// lane covers 64 / LPR slot rows (one per token group). A token's slot row is
// read ONCE and dotted with all GB query heads of the group. The per-row depth
// state (m, acc, o) goes through LDS into the MFMA accumulator layout below.
//
// Phase 2, sequence (MFMA-bound): flash-style loop over 64-key blocks of K and
// V^T staged in LDS (double buffered, one barrier per block). S^T = K Q^T on
// v_mfma_f32_32x32x16_bf16 puts one query row per lane (lanes l and l + 32 hold
// the two halves of its 64 keys), so the row max needs one cross-half exchange
// and the rescale by alpha is a per-lane multiply. O^T += V^T P^T reuses the
// probabilities straight from the S^T registers: the contraction index (keys) is
// permuted identically in both operands.
//
// Rounding: QK^T and PV accumulate in fp32; P is rounded to bf16 (RNE) before PV;
// the output is written in fp32, or rounded to bf16 (RNE) once, after the single
// normalisation.
#include "moda_internal.h"

namespace moda {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BN = 64;  // keys per sequence block
constexpr int WAVES = 4;
constexpr int WROWS = 32;  // rows per wave
constexpr float NEG_INF = -__builtin_inff();
constexpr float LN2 = 0.693147180559945309417f;

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const uint32_t x = __builtin_bit_cast(uint16_t, (__bf16)a);
  const uint32_t y = __builtin_bit_cast(uint16_t, (__bf16)b);
  return x | (y << 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint4 ldg16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// Workgroups are handed to the 8 XCDs round-robin (id % 8). Give each XCD one
// contiguous range of logical tiles, so the query blocks of one (segment, KV head)
// run on one XCD and share its L2 for the K/V blocks they all read.
__device__ __forceinline__ int64_t xcd_remap(int64_t id, int64_t n) {
  const int64_t x = id & 7, j = id >> 3;
  const int64_t q = n >> 3, r = n & 7;
  return x * q + (x < r ? x : r) + j;
}

template <int D, int GB>
struct Smem {
  static constexpr int KS = D + 8;   // K tile row stride (bf16): 16 B skew per row
  static constexpr int VS = BN + 4;  // V^T tile row stride (bf16)
  static constexpr int OS = D + 4;   // depth hand-off row stride (fp32)
  static constexpr int K_BYTES = 2 * BN * KS * 2;
  static constexpr int V_BYTES = 2 * D * VS * 2;
  static constexpr int SEQ_BYTES = K_BYTES + V_BYTES;
  static constexpr int DEPTH_BYTES = (WAVES * WROWS * OS + 2 * WAVES * WROWS) * 4;
  static constexpr int BYTES = SEQ_BYTES > DEPTH_BYTES ? SEQ_BYTES : DEPTH_BYTES;
};

template <int D, int GB, bool OUT_F32>
__global__ __launch_bounds__(256, 2) void moda_fwd_bf16_kernel(const Params p) {
  constexpr int TOK = kBlockRows / GB;  // tokens per workgroup
  constexpr int TW = WROWS / GB;        // tokens per wave
  constexpr int LPR = D / 8;            // lanes per 16-byte-sliced row of D
  constexpr int NGRP = 64 / LPR;        // depth token groups per wave
  constexpr int KPT = BN * LPR / 256;   // keys per thread per K/V block load
  constexpr int KC = D / 16;            // k-chunks of Q K^T
  constexpr int DT = D / 32;            // 32-wide d tiles of O^T
  constexpr int U = 4;                  // depth slots per load batch
  using SM = Smem<D, GB>;
  static_assert(KPT >= 1 && (BN * LPR) % 256 == 0, "tile shape");

  __shared__ __attribute__((aligned(16))) unsigned char smem[SM::BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // ---- tile decode ------------------------------------------------------------
  int64_t rest = xcd_remap(blockIdx.x, p.n_tiles);
  const int qb = p.n_qblocks - 1 - (int)(rest % p.n_qblocks);  // heavy (late) blocks first
  rest /= p.n_qblocks;
  const int hg = (int)(rest % p.n_hgroups);
  rest /= p.n_hgroups;
  const int hk = (int)(rest % p.Hkv);
  const int seg = (int)(rest / p.Hkv);

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
  const int64_t t0 = (int64_t)qb * TOK;
  if (t0 >= len) return;  // whole workgroup: this query block lies past the segment

  const int Hq = p.Hq, Hkv = p.Hkv;
  const int hbase = hk * p.G + hg * GB;  // first query head of this workgroup
  const float c2 = p.scale_log2;
  const uint16_t* __restrict__ Q = static_cast<const uint16_t*>(p.q);
  const uint16_t* __restrict__ K = static_cast<const uint16_t*>(p.k);
  const uint16_t* __restrict__ V = static_cast<const uint16_t*>(p.v);

  float* od = reinterpret_cast<float*>(smem);  // [WAVES*WROWS][OS]
  float* md = od + WAVES * WROWS * SM::OS;     // [WAVES*WROWS]
  float* ad = md + WAVES * WROWS;              // [WAVES*WROWS]

  // ---- phase 1: depth slots of each token --------------------------------------
  const int n_depth = p.n_depth;
  if (n_depth > 0) {
    const uint16_t* __restrict__ KD = static_cast<const uint16_t*>(p.kd);
    const uint16_t* __restrict__ VD = static_cast<const uint16_t*>(p.vd);
    const int grp = lane / LPR, cl = lane % LPR;
    const int64_t slot_stride = (int64_t)Hkv * D;
    for (int tb = 0; tb < TW; tb += NGRP) {
      const int tl = tb + grp;  // token index within the wave
      const int64_t t = t0 + (int64_t)wave * TW + tl;
      const bool valid = (tl < TW) && (t < len);
      const int64_t n = seg_start + (valid ? t : 0);
      float qf[GB][8];
#pragma unroll
      for (int g = 0; g < GB; ++g) {
        uint4 w = make_uint4(0, 0, 0, 0);
        if (valid) w = ldg16(Q + ((n * Hq + hbase + g) * D + 8 * cl));
        qf[g][0] = lo_bf16(w.x); qf[g][1] = hi_bf16(w.x);
        qf[g][2] = lo_bf16(w.y); qf[g][3] = hi_bf16(w.y);
        qf[g][4] = lo_bf16(w.z); qf[g][5] = hi_bf16(w.z);
        qf[g][6] = lo_bf16(w.w); qf[g][7] = hi_bf16(w.w);
      }
      float m[GB], a[GB], o[GB][8];
#pragma unroll
      for (int g = 0; g < GB; ++g) {
        m[g] = NEG_INF;
        a[g] = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) o[g][j] = 0.f;
      }
      const int64_t base = ((n * p.S_cap) * Hkv + hk) * (int64_t)D + 8 * cl;
      for (int i0 = 0; i0 < n_depth; i0 += U) {
        uint4 kw[U], vw[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          kw[u] = make_uint4(0, 0, 0, 0);
          vw[u] = make_uint4(0, 0, 0, 0);
          if (valid && i0 + u < n_depth) {
            kw[u] = ldg16(KD + base + (int64_t)(i0 + u) * slot_stride);
            vw[u] = ldg16(VD + base + (int64_t)(i0 + u) * slot_stride);
          }
        }
#pragma unroll
        for (int g = 0; g < GB; ++g) {
          float b[U];
#pragma unroll
          for (int u = 0; u < U; ++u) {
            float s = qf[g][0] * lo_bf16(kw[u].x);
            s = fmaf(qf[g][1], hi_bf16(kw[u].x), s);
            s = fmaf(qf[g][2], lo_bf16(kw[u].y), s);
            s = fmaf(qf[g][3], hi_bf16(kw[u].y), s);
            s = fmaf(qf[g][4], lo_bf16(kw[u].z), s);
            s = fmaf(qf[g][5], hi_bf16(kw[u].z), s);
            s = fmaf(qf[g][6], lo_bf16(kw[u].w), s);
            s = fmaf(qf[g][7], hi_bf16(kw[u].w), s);
#pragma unroll
            for (int off = LPR / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off);
            b[u] = (i0 + u < n_depth) ? s * c2 : NEG_INF;
          }
          float mx = b[0];
#pragma unroll
          for (int u = 1; u < U; ++u) mx = fmaxf(mx, b[u]);
          const float m_new = fmaxf(m[g], mx);
          const float m_use = (m_new == NEG_INF) ? 0.f : m_new;
          const float alpha = fast_exp2(m[g] - m_use);
          a[g] *= alpha;
#pragma unroll
          for (int j = 0; j < 8; ++j) o[g][j] *= alpha;
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const float pu = fast_exp2(b[u] - m_use);
            a[g] += pu;
            o[g][0] = fmaf(pu, lo_bf16(vw[u].x), o[g][0]);
            o[g][1] = fmaf(pu, hi_bf16(vw[u].x), o[g][1]);
            o[g][2] = fmaf(pu, lo_bf16(vw[u].y), o[g][2]);
            o[g][3] = fmaf(pu, hi_bf16(vw[u].y), o[g][3]);
            o[g][4] = fmaf(pu, lo_bf16(vw[u].z), o[g][4]);
            o[g][5] = fmaf(pu, hi_bf16(vw[u].z), o[g][5]);
            o[g][6] = fmaf(pu, lo_bf16(vw[u].w), o[g][6]);
            o[g][7] = fmaf(pu, hi_bf16(vw[u].w), o[g][7]);
          }
          m[g] = m_new;
        }
      }
      if (tl < TW) {
#pragma unroll
        for (int g = 0; g < GB; ++g) {
          const int row = wave * WROWS + tl * GB + g;
          float4* dst = reinterpret_cast<float4*>(od + row * SM::OS + 8 * cl);
          dst[0] = make_float4(o[g][0], o[g][1], o[g][2], o[g][3]);
          dst[1] = make_float4(o[g][4], o[g][5], o[g][6], o[g][7]);
          if (cl == 0) {
            md[row] = m[g];
            ad[row] = a[g];
          }
        }
      }
    }
    __syncthreads();
  }

  // ---- phase 2 set-up: this lane's query row -----------------------------------
  const int r = lane & 31;   // row within the wave (column of the 32x32 tiles)
  const int hh = lane >> 5;  // which half of each 16-wide contraction chunk
  const int rowb = wave * WROWS + r;
  const int64_t tq = t0 + rowb / GB;
  const int hq = hbase + rowb % GB;
  const bool row_valid = tq < len;

  f32x16 acc[DT];
  float m_run, l_run;
  if (n_depth > 0) {
    m_run = md[rowb];
    l_run = hh == 0 ? ad[rowb] : 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 x = *reinterpret_cast<const float4*>(od + rowb * SM::OS + 32 * dt + 8 * q4 + 4 * hh);
        acc[dt][4 * q4 + 0] = x.x;
        acc[dt][4 * q4 + 1] = x.y;
        acc[dt][4 * q4 + 2] = x.z;
        acc[dt][4 * q4 + 3] = x.w;
      }
    __syncthreads();  // the hand-off area is reused for K/V blocks below
  } else {
    m_run = NEG_INF;
    l_run = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;
  }

  bf16x8 qf[KC];
  {
    const int64_t nq = seg_start + (row_valid ? tq : 0);
    const uint16_t* qrow = Q + (nq * Hq + hq) * (int64_t)D + 8 * hh;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      uint4 w = make_uint4(0, 0, 0, 0);
      if (row_valid) w = ldg16(qrow + 16 * kc);
      qf[kc] = as_bf16x8(w);
    }
  }

  uint16_t* Ks = reinterpret_cast<uint16_t*>(smem);                  // [2][BN][KS]
  uint16_t* Vt = reinterpret_cast<uint16_t*>(smem + SM::K_BYTES);    // [2][D][VS]

  const int64_t kend = p.causal ? (len < t0 + TOK ? len : t0 + TOK) : len;
  const int nkb = (int)((kend + BN - 1) / BN);
  const int ld_cl = tid % LPR, ld_kg = tid / LPR;
  uint4 pk[KPT], pv[KPT];

  auto gload = [&](int kb) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int64_t key = (int64_t)kb * BN + ld_kg * KPT + j;
      pk[j] = make_uint4(0, 0, 0, 0);
      pv[j] = make_uint4(0, 0, 0, 0);
      if (key < kend) {
        const int64_t off = ((seg_start + key) * Hkv + hk) * (int64_t)D + 8 * ld_cl;
        pk[j] = ldg16(K + off);
        pv[j] = ldg16(V + off);
      }
    }
  };
  auto swrite = [&](int buf) {
    uint16_t* ks = Ks + buf * BN * SM::KS;
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      *reinterpret_cast<uint4*>(ks + (ld_kg * KPT + j) * SM::KS + 8 * ld_cl) = pk[j];
    uint16_t* vt = Vt + buf * D * SM::VS + ld_kg * KPT;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int word = e >> 1;
      const bool hi = e & 1;
      uint32_t w[KPT];
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const uint32_t x = word == 0 ? pv[j].x : word == 1 ? pv[j].y : word == 2 ? pv[j].z : pv[j].w;
        w[j] = hi ? (x >> 16) : (x & 0xffffu);
      }
      uint16_t* dst = vt + (8 * ld_cl + e) * SM::VS;
      if constexpr (KPT == 4) {
        *reinterpret_cast<uint2*>(dst) = make_uint2(w[0] | (w[1] << 16), w[2] | (w[3] << 16));
      } else if constexpr (KPT == 2) {
        *reinterpret_cast<uint32_t*>(dst) = w[0] | (w[1] << 16);
      } else {
#pragma unroll
        for (int j = 0; j < KPT; ++j) dst[j] = (uint16_t)w[j];
      }
    }
  };

  const int64_t wave_tmin = t0 + (wave * WROWS) / GB;
  const int64_t wave_tmax = t0 + (wave * WROWS + WROWS - 1) / GB;

  gload(0);
  swrite(0);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int cur = kb & 1;
    if (kb + 1 < nkb) gload(kb + 1);
    const int64_t k0 = (int64_t)kb * BN;
    if (!p.causal || k0 <= wave_tmax) {
      const uint16_t* ks = Ks + cur * BN * SM::KS;
      const uint16_t* vt = Vt + cur * D * SM::VS;
      f32x16 s[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s[st][i] = 0.f;
      }
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(ks + (32 * st + r) * SM::KS + 16 * kc + 8 * hh));
          s[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kc], s[st], 0, 0, 0);
        }
      }
      const bool need_mask = (p.causal && k0 + BN - 1 > wave_tmin) || (k0 + BN > len);
      if (need_mask) {
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int64_t key = k0 + 32 * st + 8 * (i >> 2) + 4 * hh + (i & 3);
            const bool vis = key < len && (!p.causal || key <= tq);
            if (!vis) s[st][i] = NEG_INF;
          }
      }
      float mx = NEG_INF;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[st][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx * c2);
      const float m_use = (m_new == NEG_INF) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[dt][i] *= alpha;
      uint32_t pp[2][8];
      float lsum = 0.f;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const float p0 = fast_exp2(fmaf(s[st][i], c2, -m_use));
          const float p1 = fast_exp2(fmaf(s[st][i + 1], c2, -m_use));
          lsum += p0 + p1;
          pp[st][i >> 1] = pack_bf16(p0, p1);
        }
      l_run += lsum;
      m_run = m_new;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int part = 0; part < 2; ++part) {
          const bf16x8 bfrag = as_bf16x8(
              make_uint4(pp[st][4 * part + 0], pp[st][4 * part + 1], pp[st][4 * part + 2], pp[st][4 * part + 3]));
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const uint16_t* vrow = vt + (32 * dt + r) * SM::VS + 32 * st + 16 * part + 4 * hh;
            const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
            const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 8);
            const bf16x8 afrag = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
            acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afrag, bfrag, acc[dt], 0, 0, 0);
          }
        }
    }
    if (kb + 1 < nkb) swrite(cur ^ 1);
    __syncthreads();
  }

  // ---- normalise once and write ------------------------------------------------
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (row_valid) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const int64_t obase = ((seg_start + tq) * Hq + hq) * (int64_t)D + 4 * hh;
    if constexpr (OUT_F32) {
      float* orow = static_cast<float*>(p.out) + obase;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *reinterpret_cast<float4*>(orow + 32 * dt + 8 * q4) =
              make_float4(acc[dt][4 * q4 + 0] * inv, acc[dt][4 * q4 + 1] * inv, acc[dt][4 * q4 + 2] * inv,
                          acc[dt][4 * q4 + 3] * inv);
    } else {
      uint16_t* orow = static_cast<uint16_t*>(p.out) + obase;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const uint32_t w0 = pack_bf16(acc[dt][4 * q4 + 0] * inv, acc[dt][4 * q4 + 1] * inv);
          const uint32_t w1 = pack_bf16(acc[dt][4 * q4 + 2] * inv, acc[dt][4 * q4 + 3] * inv);
          *reinterpret_cast<uint2*>(orow + 32 * dt + 8 * q4) = make_uint2(w0, w1);
        }
    }
    if (hh == 0 && p.lse) {
      const int64_t lbase = p.lse_batch_layout ? (int64_t)seg * Hq * p.lse_head_stride : seg_start;
      p.lse[lbase + (int64_t)hq * p.lse_head_stride + tq] = (m_run + __log2f(l_tot)) * LN2;
    }
  }
}

template <int D, int GB>
hipError_t launch_t(const Params& p, bool out_f32, hipStream_t stream) {
  if (out_f32)
    hipLaunchKernelGGL((moda_fwd_bf16_kernel<D, GB, true>), dim3((unsigned)p.n_tiles), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((moda_fwd_bf16_kernel<D, GB, false>), dim3((unsigned)p.n_tiles), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const Params& p, int head_dim, int heads_per_block, bool out_f32, hipStream_t stream) {
  if (head_dim == 128) {
    switch (heads_per_block) {
      case 1: return launch_t<128, 1>(p, out_f32, stream);
      case 2: return launch_t<128, 2>(p, out_f32, stream);
      case 4: return launch_t<128, 4>(p, out_f32, stream);
      case 8: return launch_t<128, 8>(p, out_f32, stream);
    }
  } else if (head_dim == 64) {
    switch (heads_per_block) {
      case 1: return launch_t<64, 1>(p, out_f32, stream);
      case 2: return launch_t<64, 2>(p, out_f32, stream);
      case 4: return launch_t<64, 4>(p, out_f32, stream);
      case 8: return launch_t<64, 8>(p, out_f32, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace moda

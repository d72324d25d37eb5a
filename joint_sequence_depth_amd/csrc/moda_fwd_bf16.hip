// Fused MoDA joint sequence/depth attention forward, bf16 storage, fp32 math.
//
// Operator (MoDA, arXiv 2603.15619; deck slide "One denominator allocates
// probability across both memories"): for query row (token t, head h) the causal
// sequence keys j <= t and the depth slots i of token t share ONE softmax:
//   o = (sum_j e^{a_j} v_j + sum_i e^{b_i} vd_i) / (sum_j e^{a_j} + sum_i e^{b_i}).
// The running state (m, acc, o) of slide "Shared online-softmax states preserve
// the joint operator" is carried in base 2: logits are multiplied by
// scale * log2(e) so that exp2 reproduces the natural exponential (deck backup
// slide "pseudocode needs implementation-level checks"). The slide processes the
// sequence blocks, then the depth blocks, through one state; here the depth slots
// are folded into a partial state of their own, merged with the sequence state by
// one more application of the same update before the single normalisation: the
// same operator up to the order of rounding.
//
// Work unit: one workgroup owns 32 NW expanded query rows (NW in {2, 4}):
// TOK = 32 NW / GB tokens x GB query heads of one KV head (rows ordered
// token-major, row r -> token r / GB, head r % GB, as in the expanded-row map of
// the deck's backup slide on grouped indexing). Wave w owns rows [32 w, 32 w + 32)
// and runs two parts, one after the other:
//
//  * the depth pass (HBM-bound): the depth K/V rows of the wave's tokens. LPR =
//    D / 8 lanes hold one 16-byte slice of a slot row, so one 128-bit load per lane
//    covers 64 / LPR slot rows (one per token). Each slot row is read ONCE and
//    dotted with all GB query heads of the group (v_dot2_f32_bf16 on the packed
//    operands, DPP group sums). Loads run NBUF - 1 batches of U slots ahead of the
//    arithmetic in register buffers and carry the non-temporal hint (the slots are
//    read once; the sequence K/V blocks are read again by later query blocks and
//    should keep their L2 lines). Finished row states (m, acc, o) go to LDS.
//    With bounded depth reads (mode kSelect) the pass reads and ranks every
//    slot's key first and then reads the values of the kept slots only.
//
//  * the sequence loop (MFMA-bound): a flash-style loop over 64-key blocks.
//    S^T = K Q^T on v_mfma_f32_32x32x16_bf16 puts one query row per lane (lanes l
//    and l + 32 hold the two halves of its 64 keys), so the row max needs one
//    cross-half exchange and the rescale by alpha is a per-lane multiply.
//    O^T += V^T P^T takes the probabilities straight from the S^T registers: the
//    contraction index (keys) is permuted identically in both operands. K and V
//    blocks go from memory straight into LDS (buffer loads with the LDS flag),
//    NST - 1 blocks ahead, and are read back as MFMA operands, V through the
//    gfx950 transposing LDS read.
//
// Workgroups start at different times (a new one takes each freed slot), so while
// one streams its depth rows from HBM its CU neighbour is usually in its sequence
// loop on the matrix cores; each wave then merges its two partial states,
// normalises once and writes.
//
// Rounding: QK^T and PV accumulate in fp32; P enters PV as the sum of two bf16
// values (its rounding and the rounding of the remainder, 16 significant bits);
// the output is written in fp32, or rounded to bf16 (RNE) once, after the single
// normalisation by the fp32 sum of the weights.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "moda_internal.h"
#include "moda_lds_load.h"
#include "moda_rowops.h"

namespace moda {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int BN = 64;     // keys per sequence block
constexpr int WROWS = 32;  // query rows per wave
constexpr float NEG_INF = -__builtin_inff();
constexpr float LN2 = 0.693147180559945309417f;

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// (a, b) -> packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// a.lo * b.lo + a.hi * b.hi + c, bf16 pairs, fp32 accumulation
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// The value of lane l ^ 32 (v_permlane32_swap: no LDS round trip).
__device__ __forceinline__ float other_half(float x, int lane) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, lane < 32 ? sw[1] : sw[0]);
}

__device__ __forceinline__ uint4 ldg16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// The low 32 bits of a generic pointer into __shared__ memory are its LDS byte
// address.
// 8 bytes read with the gfx950 transposing LDS load (ds_read_b64_tr_b16): within
// each group of 16 lanes, lane 4 e + q supplies 4 consecutive 16-bit values, row e
// and columns 4 q .. 4 q + 3 of a 4 x 16 tile, and lane j receives column j.
// The argument is a 32-bit LDS byte address; constant parts added to it in 32-bit
// arithmetic become the instruction's offset field.
#define MODA_TR_READ(a) __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(a))

// Lambdas of the kernel are always inlined: an outlined call would reload its
// captures through memory and spill the live accumulators around the call.
#define MODA_INL __attribute__((always_inline))

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of LPR (8 or 16) lanes with DPP moves. Every step adds
// a lane pair in both orders, so all lanes of a group end with the same bits.
template <int LPR>
__device__ __forceinline__ float group_sum(float s) {
  s += dpp_f<0xB1>(s);   // quad_perm [1,0,3,2]
  s += dpp_f<0x4E>(s);   // quad_perm [2,3,0,1]
  s += dpp_f<0x141>(s);  // row_half_mirror: the other quad of the 8-lane half
  if constexpr (LPR == 16) s += dpp_f<0x140>(s);  // row_mirror: the other half of the row
  return s;
}
template <int LPR>
__device__ __forceinline__ float group_max(float s) {
  s = fmaxf(s, dpp_f<0xB1>(s));
  s = fmaxf(s, dpp_f<0x4E>(s));
  s = fmaxf(s, dpp_f<0x141>(s));
  if constexpr (LPR == 16) s = fmaxf(s, dpp_f<0x140>(s));
  return s;
}

struct Tile {
  int seg, hk, hg, qb;
};

// A pair = (segment, KV head); its tiles are (query block, head group), head group
// fastest, so the workgroups of a KV head's head groups run side by side and share
// that token block's depth rows in L2. Workgroups go to the 8 XCDs round-robin
// (id % 8). Late (heavy causal) query blocks go first. Orders:
//  - xcd_interleave 2 (one head group per KV head, KV heads a multiple of 8):
//    segment-major, then query block, KV head fastest. The KV heads of a token
//    block run at the same time, so the slot rows of a token ([S, H_kv, d], one
//    contiguous run per slot) are read whole rather than head by head at
//    different times, and KV head hk always lands on XCD hk % 8: its K/V blocks,
//    read by every query block, stay in that XCD's L2.
//  - xcd_interleave 1 (a multiple of 8 pairs): pair p runs all of its tiles on XCD
//    p % 8, and every XCD gets an equal share of every segment.
//  - qb_major (used when the grid runs in few rounds): by query block across all
//    pairs, heaviest first, so the first round holds the longest causal tiles.
__device__ __forceinline__ Tile decode_tile(const Params& p) {
  const int64_t id = blockIdx.x;
  const int64_t per_pair = (int64_t)p.n_qblocks * p.n_hgroups;
  int64_t pair, r;
  if (p.qb_major) {
    const int64_t units = (int64_t)p.n_seg * p.Hkv * p.n_hgroups;  // (pair, head group) per query block
    const int64_t qrank = id / units, u = id % units;
    pair = u / p.n_hgroups;
    r = qrank * p.n_hgroups + u % p.n_hgroups;
  } else if (p.xcd_interleave == 2) {
    const int64_t per_seg = (int64_t)p.n_qblocks * p.Hkv;
    const int64_t seg = id / per_seg, rr = id % per_seg;
    pair = seg * p.Hkv + rr % p.Hkv;
    r = rr / p.Hkv;
  } else if (p.xcd_interleave == 1) {
    const int64_t x = id & 7, j = id >> 3;
    pair = (j / per_pair) * 8 + x;
    r = j % per_pair;
  } else {
    pair = id / per_pair;
    r = id % per_pair;
  }
  Tile t;
  t.hg = (int)(r % p.n_hgroups);
  t.qb = p.n_qblocks - 1 - (int)(r / p.n_hgroups);
  t.hk = (int)(pair % p.Hkv);
  t.seg = (int)(pair / p.Hkv);
  return t;
}

enum Mode : int {
  kNoDepth = 0,    // sequence keys only (n_depth == 0, or the sequence phase alone)
  kSerial = 1,     // every wave runs a depth pass and the sequence loop, one after the other
  kDepthOnly = 2,  // depth slots only (the depth phase alone): the sequence loop is skipped
  kSelect = 3,     // as kSerial, with bounded depth reads: each row keeps some of its slots
};

// LDS. Stages hold one K or V block each: BN rows of D bf16 without padding, the
// 16-byte chunks of a row XOR-swizzled (K and V with different patterns, chosen
// for their readers).
//  * Shared tiles (SPLIT false): NST K and NST V stages shared by the NW waves;
//    the depth hand-off reuses the stage bytes between the two parts.
//  * Split tiles (SPLIT true): each wave has its own NST K and V stages; the depth
//    hand-off has its own area; the partial states of waves 1 .. NW - 1 reuse the
//    stage bytes for the final merge.
template <int D, int NW, int MODE, bool SPLIT>
struct Smem {
  static constexpr int NST = SPLIT ? 2 : (D == 64 ? 3 : 2);  // loads run NST - 1 blocks ahead
  static constexpr int STAGE = BN * D * 2;                    // bytes of one K or V block
  static constexpr int SETS = SPLIT ? NW : 1;                 // stage sets
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = SETS * NST * STAGE;
  static constexpr int SEQ_BYTES = 2 * SETS * NST * STAGE;
  static constexpr int ROWS = SPLIT ? WROWS : NW * WROWS;  // query rows of the workgroup
  static constexpr int OS = D + 4;                          // depth hand-off row stride (fp32)
  static constexpr int OD_OFF = SPLIT ? SEQ_BYTES : 0;
  static constexpr int MD_OFF = OD_OFF + ROWS * OS * 4;
  static constexpr int AD_OFF = MD_OFF + ROWS * 4;
  static constexpr int END = AD_OFF + ROWS * 4;
  static constexpr int MG = 16 * (D / 32) + 4;  // merge record per lane (fp32): acc, m, l, r
  static constexpr int MG_BYTES = SPLIT ? (NW - 1) * 64 * MG * 4 : 0;
  static constexpr int BYTES = MODE == kNoDepth ? SEQ_BYTES : (END > SEQ_BYTES ? END : SEQ_BYTES);
  static_assert(MG_BYTES <= SEQ_BYTES, "merge area");
};

// SPLIT: the NW waves of a workgroup share one 32-row tile and split its key
// blocks (wave w takes blocks w, w + NW, ...), each through its own stages and
// without workgroup barriers; their partial states merge at the end. For problems
// with too few tiles to give every SIMD a wave: it shortens the longest chain of
// dependent blocks (the last causal tile) NW times.
template <int D, int GB, int NW, int MODE, bool OUT_F32, bool SPLIT>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW),
                          amdgpu_waves_per_eu(SPLIT ? 1 : 2, SPLIT ? 1 : 2))) void
moda_fwd_bf16_kernel(const Params p) {
  constexpr int TW = WROWS / GB;                 // tokens of a 32-row tile
  constexpr int TOK = SPLIT ? TW : TW * NW;      // tokens per workgroup
  constexpr int TPW = SPLIT ? TW / NW : TW;      // tokens of each wave's depth pass
  constexpr int LPR = D / 8;                     // lanes per 16-byte-sliced row of D
  constexpr int NGRP = 64 / LPR;                 // tokens per wave-wide depth load
  constexpr int NTG = (TPW + NGRP - 1) / NGRP;   // depth token groups per wave
  constexpr int CPR = D / 8;                     // 16-byte chunks per K/V row
  constexpr int RPI = 64 / CPR;                  // K/V rows per wave-wide direct-to-LDS load (1 KB)
  constexpr int KPT = SPLIT ? BN / RPI : BN / (NW * RPI);  // such loads per wave per K (or V) block
  constexpr int KC = D / 16;                   // k-chunks of Q K^T
  constexpr int DT = D / 32;                   // 32-wide d tiles of O^T
  constexpr int U = GB == 1 ? 8 : 4;  // depth slots per load batch
  constexpr bool QPRE = GB <= 2;               // prefetch a token's q rows with its first batch
  constexpr int QBUF = QPRE ? GB : 1;
  // depth load buffers (batches in flight + 1); split tiles run the pass beside
  // the live O^T accumulators, so the count stays small (more batches issued
  // before a split tile's loop only add to the HBM burst at its start). Four
  // heads: four slots with two buffers beat two slots with three (gqa depth-only
  // 345 -> 320 us) and eight slots.
  constexpr int NBUF = GB == 2 ? 3 : 2;
  using SM = Smem<D, NW, MODE, SPLIT>;
  constexpr int NST = SM::NST;
  constexpr int P = NST - 1;                 // load groups in flight ahead of the current block
  constexpr int WAIT_N = (P - 1) * 2 * KPT;  // loads allowed outstanding at the end of a block
  static_assert(KPT >= 1 && KPT * (SPLIT ? 1 : NW) * RPI == BN && RPI % 4 == 0, "tile shape");
  static_assert(!SPLIT || (TW % NW == 0 && NW >= 2), "split tile shape");

  __shared__ __attribute__((aligned(16))) unsigned char smem[SM::BYTES];
  poison_lds(smem, SM::BYTES);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // ---- tile decode (uniform over the workgroup) ---------------------------------
  const Tile tile = decode_tile(p);
  const int qb = tile.qb, hg = tile.hg, hk = tile.hk, seg = tile.seg;
  if (seg >= p.n_seg) return;

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
  const int64_t kend = p.causal ? (len < t0 + TOK ? len : t0 + TOK) : len;
  constexpr bool SEQ = MODE != kDepthOnly;   // the sequence keys enter this launch's softmax
  constexpr bool DEPTH = MODE != kNoDepth;   // the depth slots do
  constexpr bool SELECT = MODE == kSelect;   // bounded depth reads, selected inside the depth pass
  const int nkb = SEQ ? (int)((kend + BN - 1) / BN) : 0;  // sequence key blocks

  float* od = reinterpret_cast<float*>(smem + SM::OD_OFF);  // [ROWS][OS]
  float* md = reinterpret_cast<float*>(smem + SM::MD_OFF);  // [ROWS]
  float* ad = reinterpret_cast<float*>(smem + SM::AD_OFF);  // [ROWS]

  // ================================================================ depth pass
  // Folds the depth slots of the workgroup's tokens [dt0, dt0 + TPW) (its rows
  // [dt0 GB, (dt0 + TPW) GB)) into partial row states (m, acc, o) in LDS.
  // depth_begin issues the first NBUF - 1 load batches, depth_end runs the rest.
  const int dt0 = wave * TPW;
  const int n_depth = p.n_depth;
  const uint16_t* __restrict__ KD = static_cast<const uint16_t*>(p.kd);
  const uint16_t* __restrict__ VD = static_cast<const uint16_t*>(p.vd);
  const int d_grp = lane / LPR, d_cl = lane % LPR;
  const int64_t slot_stride = (int64_t)Hkv * D;
  const int nch = (n_depth + U - 1) / U;  // slot batches per token
  const int n_it = NTG * nch;             // (token group, slot batch) steps
  // depth load buffers: shared by depth_begin and depth_end (always written
  // before they are read)
  uint4 dkb[NBUF][U], dvb[NBUF][U], dqb[NBUF][QBUF];

  // Loads for step `it`: U slot rows of K and V (and the token's q rows at its
  // first batch) into one of the register buffers. The loads are unconditional so
  // the compiler keeps them in flight across the arithmetic: a slot past n_depth
  // re-reads the last slot and a token past the segment re-reads its last token
  // (cache hits); such logits are masked and such rows discarded.
  auto issue = [&](int it, uint4(&kw)[U], uint4(&vw)[U], uint4(&qw)[QBUF]) MODA_INL {
    it = it < n_it ? it : n_it - 1;  // the steps past the end re-load the last one (never processed)
    const int tg = it / nch, ch = it - tg * nch;
    const int tl = tg * NGRP + d_grp;
    int64_t t = t0 + dt0 + (tl < TPW ? tl : TPW - 1);
    t = t < len ? t : len - 1;
    const int64_t n = seg_start + t;
    const int64_t base = (n * p.S_cap * Hkv + hk) * (int64_t)D + 8 * d_cl;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int slot = ch * U + u < n_depth ? ch * U + u : n_depth - 1;
      kw[u] = rowops::stream_load16(KD + base + slot * slot_stride);
      vw[u] = rowops::stream_load16(VD + base + slot * slot_stride);
    }
    if constexpr (QPRE) {  // every step: a fixed load count keeps the wait counts exact
#pragma unroll
      for (int g = 0; g < QBUF; ++g) qw[g] = ldg16(Q + ((n * Hq + hbase + g) * (int64_t)D + 8 * d_cl));
    }
  };
  // One step of the pass on the loaded batch; the row states (qc: q rows of the
  // current token, dm / da / dacc: max, sum and weighted sum per head) belong to
  // one call of depth_end, so none of them lives across the sequence loop.
  auto process = [&](int it, const uint4(&kw)[U], const uint4(&vw)[U], const uint4(&qw)[QBUF], uint4(&qc)[GB],
                     float(&dm)[GB], float(&da)[GB], float(&dacc)[GB][8]) MODA_INL {
    const int tg = it / nch, ch = it - tg * nch;
    const int tl = tg * NGRP + d_grp;
    if (ch == 0) {
      int64_t t = t0 + dt0 + (tl < TPW ? tl : TPW - 1);
      t = t < len ? t : len - 1;
      const int64_t n = seg_start + t;
#pragma unroll
      for (int g = 0; g < GB; ++g) {
        if constexpr (QPRE) {
          qc[g] = qw[g < QBUF ? g : 0];
        } else {
          qc[g] = ldg16(Q + ((n * Hq + hbase + g) * (int64_t)D + 8 * d_cl));
        }
        dm[g] = NEG_INF;
        da[g] = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) dacc[g][j] = 0.f;
      }
    }
#pragma unroll
    for (int g = 0; g < GB; ++g) {
      float b[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float sc = dot2(qc[g].x, kw[u].x, 0.f);
        sc = dot2(qc[g].y, kw[u].y, sc);
        sc = dot2(qc[g].z, kw[u].z, sc);
        sc = dot2(qc[g].w, kw[u].w, sc);
        sc = group_sum<LPR>(sc);
        const int slot = ch * U + u;
        b[u] = slot < n_depth ? sc * c2 : NEG_INF;
      }
      float mx = b[0];
#pragma unroll
      for (int u = 1; u < U; ++u) mx = fmaxf(mx, b[u]);
      const float m_new = fmaxf(dm[g], mx);
      const float m_use = (m_new == NEG_INF) ? 0.f : m_new;
      const float alpha = fast_exp2(dm[g] - m_use);
      da[g] *= alpha;
#pragma unroll
      for (int j = 0; j < 8; ++j) dacc[g][j] *= alpha;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float pu = fast_exp2(b[u] - m_use);
        da[g] += pu;
        dacc[g][0] = fmaf(pu, lo_bf16(vw[u].x), dacc[g][0]);
        dacc[g][1] = fmaf(pu, hi_bf16(vw[u].x), dacc[g][1]);
        dacc[g][2] = fmaf(pu, lo_bf16(vw[u].y), dacc[g][2]);
        dacc[g][3] = fmaf(pu, hi_bf16(vw[u].y), dacc[g][3]);
        dacc[g][4] = fmaf(pu, lo_bf16(vw[u].z), dacc[g][4]);
        dacc[g][5] = fmaf(pu, hi_bf16(vw[u].z), dacc[g][5]);
        dacc[g][6] = fmaf(pu, lo_bf16(vw[u].w), dacc[g][6]);
        dacc[g][7] = fmaf(pu, hi_bf16(vw[u].w), dacc[g][7]);
      }
      dm[g] = m_new;
    }
    if (ch == nch - 1 && tl < TPW) {
#pragma unroll
      for (int g = 0; g < GB; ++g) {
        const int row = (dt0 + tl) * GB + g;
        float4* dst = reinterpret_cast<float4*>(od + row * SM::OS + 8 * d_cl);
        dst[0] = make_float4(dacc[g][0], dacc[g][1], dacc[g][2], dacc[g][3]);
        dst[1] = make_float4(dacc[g][4], dacc[g][5], dacc[g][6], dacc[g][7]);
        if (d_cl == 0) {
          md[row] = dm[g];
          ad[row] = da[g];
        }
      }
    }
  };
  // NBUF register buffers, loads NBUF - 1 steps ahead. Every step issues the same
  // number of loads, so the compiler waits exactly for the buffer it reads and
  // leaves the others in flight.
  auto depth_begin = [&]() MODA_INL {
#pragma unroll
    for (int j = 0; j < NBUF - 1; ++j) issue(j, dkb[j], dvb[j], dqb[j]);
  };
  auto depth_end = [&]() MODA_INL {
    uint4 qc[GB];
    float dm[GB], da[GB], dacc[GB][8];
    for (int it = 0; it < n_it; it += NBUF) {
#pragma unroll
      for (int j = 0; j < NBUF; ++j) {
        issue(it + j + NBUF - 1, dkb[(j + NBUF - 1) % NBUF], dvb[(j + NBUF - 1) % NBUF], dqb[(j + NBUF - 1) % NBUF]);
        if (it + j < n_it) process(it + j, dkb[j], dvb[j], dqb[j], qc, dm, da, dacc);
      }
    }
  };

  // ---------------------------------------------------- bounded depth reads (kSelect)
  // Of a row's slots [0, n_depth), the last sel_recent always enter its softmax and
  // of the older ones the sel_topk with the largest logits, ties to the lower slot
  // (the future-work buffer of the MoDA deck's slide "The main open cost is
  // retaining and reading depth history", read as a per-row selection). The
  // selection runs inside the pass. Per token group, K steps read every slot's
  // key row, score it against the GB heads and keep the raw dot products in the
  // rows' LDS hand-off records; after the last K step each row ranks its older
  // slots and adds its 64-bit keep mask and the max of its kept logits to the
  // record. V steps then read the value rows of the kept slots only (for GB > 1,
  // of the union over the heads, at most n_cand rows per token) and accumulate
  // against the known max: no rescale. Steps run as [K(0)], [K(1), V(0)], ...,
  // [V(last)], so a V step's slots, which follow from its group's masks, are
  // loaded (one step ahead) only after that group's ranking has run; with a
  // single token group the first V step is issued after it instead.
  constexpr int US = GB == 1 ? 16 : (GB == 2 ? 8 : 4);  // slot rows per select step (keys or values)
  constexpr int SPL = 64 / LPR;     // slots each lane ranks
  constexpr int REC_MASK = 64;      // record words: [0, 64) dot products, mask (2 words), max
  constexpr int REC_MAX = 66;
  static_assert(SM::OS > REC_MAX, "selection record");
  const uintptr_t vd_minus_kd = reinterpret_cast<uintptr_t>(p.vd) - reinterpret_cast<uintptr_t>(p.kd);
  const int sel_recent = SELECT ? p.sel_recent : 0;
  const int n_old = n_depth - sel_recent;
  const int n_keep = (p.sel_topk < n_old ? p.sel_topk : n_old) + sel_recent;
  const int n_cand = GB * n_keep < n_depth ? GB * n_keep : n_depth;  // value rows per token (bound)
  const int nck = (n_depth + US - 1) / US;  // K steps per token group
  const int ncv = (n_cand + US - 1) / US;   // V steps per token group
  const int seg_steps = nck + ncv;
  const int n_sel = NTG * seg_steps;
  struct SelStep {
    bool is_k;
    int tg, b;
  };
  auto sel_step = [&](int it) MODA_INL {
    SelStep st;
    if (it < nck) {
      st.is_k = true;
      st.tg = 0;
      st.b = it;
    } else {
      const int j = it - nck, sg = 1 + j / seg_steps, r = j - (sg - 1) * seg_steps;
      st.is_k = sg < NTG && r < nck;
      st.tg = st.is_k ? sg : sg - 1;
      st.b = st.is_k ? r : (sg < NTG ? r - nck : r);
    }
    return st;
  };
  // the record of row (token tl of this wave, head g); tokens past the wave's use
  // its last token's (they compute, but never write)
  auto rec_of = [&](int tl, int g) MODA_INL {
    const int tlc = tl < TPW ? tl : TPW - 1;
    return od + ((dt0 + tlc) * GB + g) * SM::OS;
  };
  auto rec_mask = [&](const float* rec) MODA_INL {
    return (uint64_t)__float_as_uint(rec[REC_MASK]) | ((uint64_t)__float_as_uint(rec[REC_MASK + 1]) << 32);
  };
  // slots of V step b of token tl: set bits b US .. b US + US - 1 of the union of its
  // heads' masks (-1 past the last), every index below n_depth
  auto v_slots = [&](int tl, int b, int(&slot)[US]) MODA_INL {
    uint64_t m = 0;
#pragma unroll
    for (int g = 0; g < GB; ++g) m |= rec_mask(rec_of(tl, g));
    for (int k = 0; k < b * US; ++k) m &= m - 1;
#pragma unroll
    for (int u = 0; u < US; ++u) {
      const int i = m ? (int)__builtin_ctzll(m) : -1;
      slot[u] = i < n_depth ? i : n_depth - 1;
      m &= m - 1;
    }
  };
  auto sel_issue = [&](int it, uint4(&w)[US], uint4(&qw)[QBUF]) MODA_INL {
    it = it < n_sel ? it : n_sel - 1;  // the steps past the end re-load the last one (never processed)
    const SelStep st = sel_step(it);
    const int tl = st.tg * NGRP + d_grp;
    int64_t t = t0 + dt0 + (tl < TPW ? tl : TPW - 1);
    t = t < len ? t : len - 1;
    const int64_t n = seg_start + t;
    const int64_t base = (n * p.S_cap * Hkv + hk) * (int64_t)D + 8 * d_cl;
    int slot[US];
    if (st.is_k) {
#pragma unroll
      for (int u = 0; u < US; ++u) slot[u] = st.b * US + u < n_depth ? st.b * US + u : n_depth - 1;
    } else {
      v_slots(tl, st.b, slot);
#pragma unroll
      for (int u = 0; u < US; ++u) slot[u] = slot[u] < 0 ? 0 : slot[u];
    }
    // key or value rows: KD plus a selected byte offset (a select between the two
    // captured pointers becomes a select of their addresses, which keeps them in
    // scratch memory)
    const uintptr_t src_addr = reinterpret_cast<uintptr_t>(KD) + (st.is_k ? 0 : vd_minus_kd);
    const uint16_t* src = reinterpret_cast<const uint16_t*>(src_addr);
#pragma unroll
    for (int u = 0; u < US; ++u) w[u] = rowops::stream_load16(src + base + slot[u] * slot_stride);
    if constexpr (QPRE) {
#pragma unroll
      for (int g = 0; g < QBUF; ++g) qw[g] = ldg16(Q + ((n * Hq + hbase + g) * (int64_t)D + 8 * d_cl));
    }
  };
  auto sel_process = [&](int it, const uint4(&w)[US], const uint4(&qw)[QBUF], uint4(&qc)[GB], float(&da)[GB],
                         float(&dacc)[GB][8]) MODA_INL {
    const SelStep st = sel_step(it);
    const int tl = st.tg * NGRP + d_grp;
    const bool own = tl < TPW;
    if (st.is_k) {
      if (st.b == 0) {
        int64_t t = t0 + dt0 + (tl < TPW ? tl : TPW - 1);
        t = t < len ? t : len - 1;
        const int64_t n = seg_start + t;
#pragma unroll
        for (int g = 0; g < GB; ++g) {
          if constexpr (QPRE) {
            qc[g] = qw[g < QBUF ? g : 0];
          } else {
            qc[g] = ldg16(Q + ((n * Hq + hbase + g) * (int64_t)D + 8 * d_cl));
          }
        }
      }
#pragma unroll
      for (int g = 0; g < GB; ++g) {
        float* rec = rec_of(tl, g);
#pragma unroll
        for (int u = 0; u < US; ++u) {
          float sc = dot2(qc[g].x, w[u].x, 0.f);
          sc = dot2(qc[g].y, w[u].y, sc);
          sc = dot2(qc[g].z, w[u].z, sc);
          sc = dot2(qc[g].w, w[u].w, sc);
          sc = group_sum<LPR>(sc);
          const int slot = st.b * US + u;
          if (own && slot < n_depth && d_cl == u % LPR) rec[slot] = sc;
        }
      }
      if (st.b == nck - 1) {  // every key scored: rank the older slots of each head's row
#pragma unroll
        for (int g = 0; g < GB; ++g) {
          float* rec = rec_of(tl, g);
          float bj[SPL];
          int rank[SPL];
#pragma unroll
          for (int k = 0; k < SPL; ++k) {
            const int j = d_cl + LPR * k;
            bj[k] = j < n_depth ? rec[j] : NEG_INF;
            rank[k] = 0;
          }
          for (int i = 0; i < n_old; ++i) {
            const float bi = rec[i];
#pragma unroll
            for (int k = 0; k < SPL; ++k) {
              const int j = d_cl + LPR * k;
              rank[k] += (bi > bj[k] || (bi == bj[k] && i < j)) ? 1 : 0;
            }
          }
          uint64_t keep_mask = 0;
          float mx = NEG_INF;
#pragma unroll
          for (int k = 0; k < SPL; ++k) {
            const int j = d_cl + LPR * k;
            const bool keep = j < n_depth && (j >= n_old || rank[k] < p.sel_topk);
            if (keep) mx = fmaxf(mx, bj[k]);
            const uint64_t bal = __ballot(keep);  // bits of this lane group: slots LPR k .. LPR k + LPR - 1
            keep_mask |= ((bal >> (LPR * d_grp)) & ((1ull << LPR) - 1)) << (LPR * k);
          }
          mx = group_max<LPR>(mx);
          if (own && d_cl == 0) {
            rec[REC_MASK] = __uint_as_float((uint32_t)keep_mask);
            rec[REC_MASK + 1] = __uint_as_float((uint32_t)(keep_mask >> 32));
            rec[REC_MAX] = mx * c2;
          }
        }
      }
    } else {
      if (st.b == 0) {
#pragma unroll
        for (int g = 0; g < GB; ++g) {
          da[g] = 0.f;
#pragma unroll
          for (int j = 0; j < 8; ++j) dacc[g][j] = 0.f;
        }
      }
      int slot[US];
      v_slots(tl, st.b, slot);
      float mg[GB];
#pragma unroll
      for (int g = 0; g < GB; ++g) {
        const float* rec = rec_of(tl, g);
        const uint64_t km = rec_mask(rec);
        mg[g] = rec[REC_MAX];
#pragma unroll
        for (int u = 0; u < US; ++u) {
          const bool kept = slot[u] >= 0 && ((km >> (slot[u] & 63)) & 1ull);
          const float pu = kept ? fast_exp2(rec[slot[u] < 0 ? 0 : slot[u]] * c2 - mg[g]) : 0.f;
          da[g] += pu;
          dacc[g][0] = fmaf(pu, lo_bf16(w[u].x), dacc[g][0]);
          dacc[g][1] = fmaf(pu, hi_bf16(w[u].x), dacc[g][1]);
          dacc[g][2] = fmaf(pu, lo_bf16(w[u].y), dacc[g][2]);
          dacc[g][3] = fmaf(pu, hi_bf16(w[u].y), dacc[g][3]);
          dacc[g][4] = fmaf(pu, lo_bf16(w[u].z), dacc[g][4]);
          dacc[g][5] = fmaf(pu, hi_bf16(w[u].z), dacc[g][5]);
          dacc[g][6] = fmaf(pu, lo_bf16(w[u].w), dacc[g][6]);
          dacc[g][7] = fmaf(pu, hi_bf16(w[u].w), dacc[g][7]);
        }
      }
      if (st.b == ncv - 1 && own) {  // the record's words are read: the row state replaces them
#pragma unroll
        for (int g = 0; g < GB; ++g) {
          const int row = (dt0 + tl) * GB + g;
          float4* dst = reinterpret_cast<float4*>(od + row * SM::OS + 8 * d_cl);
          dst[0] = make_float4(dacc[g][0], dacc[g][1], dacc[g][2], dacc[g][3]);
          dst[1] = make_float4(dacc[g][4], dacc[g][5], dacc[g][6], dacc[g][7]);
          if (d_cl == 0) {
            md[row] = mg[g];
            ad[row] = da[g];
          }
        }
      }
    }
  };
  auto sel_pass = [&]() MODA_INL {
    uint4 sw[2][US], sq[2][QBUF];
    uint4 qc[GB];
    float da[GB], dacc[GB][8];
    sel_issue(0, sw[0], sq[0]);
    for (int it = 0; it < n_sel; it += 2) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        // one token group: its first V step's slots come from this step's ranking
        const bool late = NTG == 1 && it + j + 1 == nck;
        if (!late) sel_issue(it + j + 1, sw[j ^ 1], sq[j ^ 1]);
        if (it + j < n_sel) sel_process(it + j, sw[j], sq[j], qc, da, dacc);
        if (late) sel_issue(it + j + 1, sw[j ^ 1], sq[j ^ 1]);
      }
    }
  };

  // ============================================================ sequence state
  const int r = lane & 31;   // row within the wave (column of the 32x32 tiles)
  const int hh = lane >> 5;  // which half of each 16-wide contraction chunk
  const int wrow0 = SPLIT ? 0 : wave * WROWS;  // first row of this wave's 32
  const int rowb = wrow0 + r;
  const int64_t tq = t0 + rowb / GB;
  const int hq = hbase + rowb % GB;
  const bool row_valid = tq < len;

  f32x16 acc[DT];
  // running max (base 2) and denominator (one half of the keys per lane)
  float m_run = NEG_INF, l_run = 0.f;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;

  // Folds this row's depth state (published in LDS) into (m_run, l_run, acc).
  auto depth_fold = [&]() MODA_INL {
    const float m_d = md[rowb];
    const float m_new = fmaxf(m_run, m_d);
    const float m_use = (m_new == NEG_INF) ? 0.f : m_new;
    const float f_seq = fast_exp2(m_run - m_use);
    const float f_dep = fast_exp2(m_d - m_use);
    const float a_d = hh == 0 ? ad[rowb] * f_dep : 0.f;
    l_run = l_run * f_seq + a_d;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 x = *reinterpret_cast<const float4*>(od + rowb * SM::OS + 32 * dt + 8 * q4 + 4 * hh);
        acc[dt][4 * q4 + 0] = fmaf(x.x, f_dep, acc[dt][4 * q4 + 0] * f_seq);
        acc[dt][4 * q4 + 1] = fmaf(x.y, f_dep, acc[dt][4 * q4 + 1] * f_seq);
        acc[dt][4 * q4 + 2] = fmaf(x.z, f_dep, acc[dt][4 * q4 + 2] * f_seq);
        acc[dt][4 * q4 + 3] = fmaf(x.w, f_dep, acc[dt][4 * q4 + 3] * f_seq);
      }
    m_run = m_new;
  };

  // Shared tiles: the depth pass runs first, so the workgroup's HBM phase precedes
  // its matrix-core phase and the staggered starts of the workgroups on a CU
  // overlap the two. With one or two heads per workgroup this is fixed at compile
  // time: the depth buffers are then never live together with the output
  // accumulators, which keeps those D = 128 instances free of register spills.
  // Four-head tiles alternate the order (below); their depth-last path holds both
  // and spills 36 bytes per lane, which the better overlap outweighs. Split tiles
  // at D = 64: the depth loads are issued as the sequence loop starts and
  // consumed after it, which hides their latency (at D = 128 the loop needs those
  // registers; the pass follows the loop).
  constexpr bool EARLY_DEPTH = DEPTH && SPLIT && D == 64 && !SELECT;
  constexpr bool depth_first = DEPTH && !SPLIT;
  // Four-head tiles (few launch rounds: every workgroup of a round would stream
  // its depth rows at the same time) alternate the order: the second 256
  // workgroups of each 512 - one per CU once the first 256 have taken theirs - run
  // the pass after the sequence loop (gqa 1.026 -> 0.986 ms; for one head per
  // workgroup, many rounds desynchronise on their own and the alternation cost
  // 1-2 %).
  const bool pass_first = !(GB == 4 && MODE == kSerial) || ((blockIdx.x >> 8) & 1) == 0;
  if (depth_first && pass_first) {
    if constexpr (SELECT) {
      sel_pass();
    } else {
      depth_begin();
      depth_end();
    }
    __syncthreads();
    depth_fold();
    __syncthreads();  // the hand-off area is the K/V area
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

  // ---- K/V staging ---------------------------------------------------------------
  // K and V rows of this (segment, KV head) are read through buffer resources
  // rebased at every key block, whose range ends with key kend - 1. Each wave-wide
  // load moves RPI whole rows (1 KB) into LDS: lane l fills bytes [16 l, 16 l + 16)
  // of the run, i.e. chunk position l % CPR of row l / CPR, with the chunk of the
  // row that the swizzle puts there. Rows past the last key load the last key's
  // row, so the masked tail of the last block holds finite values (their p is
  // exactly 0). Blocks past the end, issued by the fixed-count pipeline, have an
  // empty range: those loads return zeros and touch no memory; their stages are
  // never read.
  //   K: chunk c of row k sits at position c ^ (k % CPR): the score operand reads
  //      (16 lanes = 16 rows, one chunk) hit 16 different bank groups.
  //   V: chunk c of row k sits at position c ^ sv(k), sv(k) = 4 (k % 4) (D = 128)
  //      or 4 ((k / 2) % 2) (D = 64): the transposing reads of 32 lanes (4 rows x 4
  //      chunks) cover every bank once.
  const int64_t row_bytes = (int64_t)Hkv * D * 2;  // bytes from one key's row to the next
  const char* kbase = static_cast<const char*>(p.k) + ((seg_start * Hkv + hk) * (int64_t)D) * 2;
  const char* vbase = static_cast<const char*>(p.v) + ((seg_start * Hkv + hk) * (int64_t)D) * 2;
  auto sv = [](int k) MODA_INL { return D == 128 ? 4 * (k & 3) : 4 * ((k >> 1) & 1); };
  const int ld_row = lane / CPR, ld_pos = lane % CPR;  // this lane's place in a 1 KB run
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // the wave index as a scalar
  const int run0 = SPLIT ? 0 : wave_u * KPT;  // this wave's first 1 KB run of a block
  const uint32_t row_bytes32 = (uint32_t)Hkv * (uint32_t)(D * 2);  // scalar: a full block's offsets fit 32 bits
  auto stage_of = [](int kb) MODA_INL { return kb - (kb / NST) * NST; };
  // Per-lane parts of the load offsets of a full block (loop-invariant): the LDS
  // row of load j is (run0 + j) RPI + ld_row, whose uniform part is added per
  // load (no multiply in the loop). The K swizzle at D = 128 also depends on that row's bits 2-3,
  // a uniform XOR of bits 6-7 of the chunk offset; row_bytes is then a multiple of
  // 256, so the XOR never meets a carry from the row part.
  const uint32_t k_lane = (uint32_t)(ld_row * row_bytes + 16 * (ld_pos ^ (ld_row % CPR)));
  const uint32_t v_lane = (uint32_t)(ld_row * row_bytes + 16 * (ld_pos ^ sv(ld_row)));
  // one block of K (or V) into `stage`: KPT wave-wide loads by this wave (runs
  // run0 .. run0 + KPT - 1 of the block)
  auto load_block = [&](const char* base, int kb, unsigned char* stage, bool is_v) MODA_INL {
    const int64_t keys_left = kend - (int64_t)kb * BN;
    int64_t nrec = keys_left > 0 ? (keys_left - 1) * row_bytes + D * 2 : 0;
    nrec = nrec < 0x7fffffff ? nrec : 0x7fffffff;
    const i32x4 rs = make_rsrc(base + (int64_t)kb * BN * row_bytes, (uint32_t)nrec);
    const uint32_t lds0 = (uint32_t)(uintptr_t)stage + (uint32_t)run0 * 1024u;
    if (keys_left >= BN) {  // full block: every row in range, no clamp
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const uint32_t rg = (uint32_t)(run0 + j);  // uniform: which RPI-row run
        uint32_t voff = is_v ? v_lane : k_lane;
        if (D == 128 && !is_v) voff ^= 64u * (rg & 3u);
        load_to_lds16(lds0 + 1024u * j, voff + rg * (uint32_t)RPI * row_bytes32, rs);
      }
    } else {  // the segment's last block (or a block past it): clamp rows to the last key
      const int last = keys_left > 0 ? (int)keys_left - 1 : 0;
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const int row = (run0 + j) * RPI + ld_row;  // key within the block = LDS row
        const int src = row < last ? row : last;            // key whose row is loaded there
        const int chunk = ld_pos ^ (is_v ? sv(row) : (row % CPR));
        load_to_lds16(lds0 + 1024u * j, (uint32_t)(src * row_bytes + 16 * chunk), rs);
      }
    }
  };
  unsigned char* const kst = smem + SM::K_OFF + (SPLIT ? wave_u * NST * SM::STAGE : 0);
  unsigned char* const vst = smem + SM::V_OFF + (SPLIT ? wave_u * NST * SM::STAGE : 0);
  // This wave's key blocks: bid(i), i = 0 .. nbw - 1 (all blocks, or every NW-th).
  const int nbw = SPLIT ? (nkb > wave_u ? (nkb - wave_u + NW - 1) / NW : 0) : nkb;
  auto bid = [&](int i) MODA_INL { return SPLIT ? wave_u + i * NW : i; };
  // Load group i: K of block bid(i + 1) and V of block bid(i), both read in step i
  // (the scores run one block ahead). Group i + P is issued at the top of step i,
  // into the stages of K(bid(i)) and V(bid(i - 1)), which step i - 1 released.
  auto issue_group = [&](int i) MODA_INL {
    load_block(kbase, bid(i + 1), kst + stage_of(i + 1) * SM::STAGE, false);
    load_block(vbase, bid(i), vst + stage_of(i) * SM::STAGE, true);
  };
  // the end of a step: load group i + 1 has landed (only later groups may still be
  // in flight); shared tiles: every wave is done with step i's stages
  auto block_end = [&]() MODA_INL {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(WAIT_N));
    if constexpr (!SPLIT) __syncthreads();
  };

  const int64_t wave_tmin = t0 + wrow0 / GB;
  const int64_t wave_tmax = t0 + (wrow0 + WROWS - 1) / GB;
  // a wave's rows see key block kb at all (monotone in kb)
  auto active = [&](int kb) MODA_INL { return !p.causal || (int64_t)kb * BN <= wave_tmax; };

  // Score operand reads: QK MFMA i uses k-chunk i / 2 of key tile i % 2.
  auto kread = [&](const unsigned char* ks, int i) MODA_INL {
    const int kc = i >> 1, row = 32 * (i & 1) + r;
    const int chunk = (2 * kc + hh) ^ (row % CPR);
    return as_bf16x8(*reinterpret_cast<const uint4*>(ks + row * (D * 2) + 16 * chunk));
  };
  // V^T operand reads: PV MFMA i = (key tile st, half part, d tile dt). Lane
  // 16 g + 4 e + q reads keys key0 + e and key0 + 8 + e, key0 = 32 st + 16 part +
  // 4 (g / 2), columns 32 dt + 16 (g % 2) + 4 q .. + 3: after the transpose, lane
  // (r, hh) holds column 32 dt + r at keys 32 st + 16 part + 4 hh + {0..3, 8..11},
  // the key order of the P^T registers.
  const int tr_g = lane >> 4, tr_e = (lane >> 2) & 3, tr_q = lane & 3;
  const int tr_row = 4 * (tr_g >> 1) + tr_e;       // row within a 16-key half; rows + 8 share sv
  const int tr_lo = 2 * (tr_g & 1) + (tr_q >> 1);  // chunk within the 4 of a d tile
  uint32_t tr_off[DT];                             // this lane's byte offset in a stage, per d tile
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
    tr_off[dt] = (uint32_t)(tr_row * (D * 2) + 8 * (tr_q & 1) + 16 * (((4 * dt) ^ sv(tr_row)) + tr_lo));
  auto vread = [&](const unsigned char* vs, int i) MODA_INL {
    const int st = i / (2 * DT), part = (i / DT) % 2, dt = i % DT;
    const uint32_t a = (uint32_t)(uintptr_t)vs + tr_off[dt];
    const i16x4 x0 = MODA_TR_READ(a + (32 * st + 16 * part) * (D * 2));
    const i16x4 x1 = MODA_TR_READ(a + (32 * st + 16 * part + 8) * (D * 2));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // S^T = K Q^T for one key block: two 32-key tiles, fp32.
  auto qk = [&](const unsigned char* ks, f32x16(&s)[2]) MODA_INL {
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[st][i] = 0.f;
#pragma unroll
    for (int i = 0; i < 2 * KC; ++i)
      s[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kread(ks, i), qf[i >> 1], s[i & 1], 0, 0, 0);
  };

  // ---- online softmax of one key block, in pieces ------------------------------
  // Scores of keys past the causal limit of this lane's row or past the segment
  // end become -inf (blocks crossing the diagonal or the segment end only).
  auto mask_block = [&](int kb, f32x16(&s)[2]) MODA_INL {
    const int64_t k0 = (int64_t)kb * BN;
    // key k0 + off is visible iff off <= lim (32-bit offsets within the block)
    const int64_t last = p.causal ? (tq < len - 1 ? tq : len - 1) : len - 1;
    const int lim = (int)(last - k0 < BN ? last - k0 : BN);
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int off = 32 * st + 8 * (i >> 2) + 4 * hh + (i & 3);
        if (off > lim) s[st][i] = NEG_INF;
      }
  };
  // Row max of the block (base-2 units) and the lazy rescale: the reference max
  // m_run only moves (and O, l are rescaled) when some row's block max exceeds it
  // by more than 2^8; otherwise the probabilities, bounded by 2^8, accumulate
  // against the old reference. The final o / l is the same; only the order of
  // roundings differs. Returns the reference to subtract.
  auto max_and_rescale = [&](const f32x16(&s)[2]) MODA_INL {
    float mx = NEG_INF;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[st][i]);
    mx = fmaxf(mx, other_half(mx, lane)) * c2;
    if (__any(mx > m_run + 8.f)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - m_new);  // m_run = -inf at first: alpha = 0
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[dt][i] *= alpha;
      m_run = m_new;
    }
    return (m_run == NEG_INF) ? 0.f : m_run;
  };
  // p = 2^(s c2 - m) as the sum of two bf16 values for the P.V product, pair q of
  // the 16 per lane: ph = bf16(p) and pl = bf16(p - ph), so that ph + pl carries 16
  // significant bits. One bf16 weight alone (8 bits) moves a row that averages few
  // values by up to ~2^-9 of their spread, more than 2e-2 of the RMS of a whole
  // long-context output; with the low part the applied weights equal p to ~2^-17
  // and the output is normalised by the sum of the unrounded p, as lse is.
  auto exp_pair = [&](const f32x16(&s)[2], float m_use, int q, uint32_t(&ph)[2][8], uint32_t(&pl)[2][8],
                      float& lsum) MODA_INL {
    const int se = q >> 3, j = q & 7;
    const float p0 = fast_exp2(fmaf(s[se][2 * j], c2, -m_use));
    const float p1 = fast_exp2(fmaf(s[se][2 * j + 1], c2, -m_use));
    lsum += p0 + p1;
    const uint32_t h = pack_bf16(p0, p1);
    ph[se][j] = h;
    pl[se][j] = pack_bf16(p0 - lo_bf16(h), p1 - hi_bf16(h));
  };
  // fast steps: p of pair q written over its scores and packed as bf16 (the high
  // part); the low part is formed from them later, beside the P.V products
  auto exp_hi = [&](f32x16(&s)[2], float m_use, int q, uint32_t(&ph)[2][8], float& lsum) MODA_INL {
    const int se = q >> 3, j = q & 7;
    const float p0 = fast_exp2(fmaf(s[se][2 * j], c2, -m_use));
    const float p1 = fast_exp2(fmaf(s[se][2 * j + 1], c2, -m_use));
    lsum += p0 + p1;
    s[se][2 * j] = p0;
    s[se][2 * j + 1] = p1;
    ph[se][j] = pack_bf16(p0, p1);
  };
  auto lo_of = [&](const f32x16(&s)[2], int q, const uint32_t(&ph)[2][8], uint32_t(&pl)[2][8]) MODA_INL {
    const int se = q >> 3, j = q & 7;
    const uint32_t h = ph[se][j];
    pl[se][j] = pack_bf16(s[se][2 * j] - lo_bf16(h), s[se][2 * j + 1] - hi_bf16(h));
  };
  // B operand of PV MFMA i: the packed probabilities of key tile st, half part.
  auto pfrag = [](const uint32_t(&pp)[2][8], int i) MODA_INL {
    const int st = i / (2 * DT), part = (i / DT) % 2;
    return as_bf16x8(
        make_uint4(pp[st][4 * part + 0], pp[st][4 * part + 1], pp[st][4 * part + 2], pp[st][4 * part + 3]));
  };
  constexpr int NQK = 2 * KC;  // score MFMAs per block
  constexpr int NPV = 4 * DT;  // P.V MFMAs per block

  // Prologue: K(bid(0)) and load groups 0 .. P - 1, then the scores of block
  // bid(0). Shared tiles: the barrier after them keeps step 0 from reloading
  // K(0)'s stage under a wave that is still reading it (split tiles: the stages are
  // the wave's own, read before it issues the next loads).
  f32x16 sA[2], sB[2];
  if (nbw > 0) {  // shared tiles: always (nkb >= 1); split: waves past the last block skip
    load_block(kbase, bid(0), kst, false);
#pragma unroll
    for (int j = 0; j < P; ++j) issue_group(j);
    block_end();
    qk(kst, sA);  // every wave sees its first block (unconditional: the q loads are waited for here only)
    if constexpr (!SPLIT) __syncthreads();
  }
  if constexpr (EARLY_DEPTH) depth_begin();

  // Blocks [0, n_full) are fully visible to every row of this wave: a
  // straight-line step (no mask, the next block's scores always issued) lets the
  // compiler interleave the matrix-core and vector work. The rest (diagonal,
  // segment end, blocks beyond the wave's rows) take the generic step.
  const int64_t full_keys = p.causal ? (wave_tmin + 1 < len ? wave_tmin + 1 : len) : len;
  const int n_full = (int)(full_keys / BN);

  // Step for a fully visible block, written in issue order: each score MFMA of
  // the next block is followed by the exponentials of pairs of this block's
  // scores (p over the scores, and its bf16 high part); the low parts of P.V
  // fragment f + 1 are formed between the products of fragment f, so the wave's
  // vector work also fills its P.V phase. Operands are read two MFMAs ahead.
  // sched_barrier keeps that order. When kb + 1 == nkb the next scores read a
  // stage that holds no keys and are never used.
  auto fast_step = [&](int i, f32x16(&scur)[2], f32x16(&snext)[2]) MODA_INL {
    issue_group(i + P);
    const float m_use = max_and_rescale(scur);
    const unsigned char* ks = kst + stage_of(i + 1) * SM::STAGE;
    const unsigned char* vs = vst + stage_of(i) * SM::STAGE;
    uint32_t ph[2][8], pl[2][8];
    float lsum = 0.f;
    bf16x8 a0 = kread(ks, 0), a1 = kread(ks, 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      bf16x8 a2 = a1;
      if (i + 2 < NQK) a2 = kread(ks, i + 2);
      const int kc = i >> 1, st = i & 1;
      if (kc == 0) {
        f32x16 zero;
#pragma unroll
        for (int z = 0; z < 16; ++z) zero[z] = 0.f;
        snext[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[kc], zero, 0, 0, 0);
      } else {
        snext[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[kc], snext[st], 0, 0, 0);
      }
#pragma unroll
      for (int q = i * 16 / NQK; q < (i + 1) * 16 / NQK; ++q) exp_hi(scur, m_use, q, ph, lsum);
      if (i >= NQK - 4) lo_of(scur, i - (NQK - 4), ph, pl);  // low parts of the first P.V fragment
      __builtin_amdgcn_sched_barrier(0);
      a0 = a1;
      a1 = a2;
    }
    l_run += lsum;
    bf16x8 b0 = vread(vs, 0), b1 = vread(vs, 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      bf16x8 b2 = b1;
      if (i + 2 < NPV) b2 = vread(vs, i + 2);
      acc[i % DT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b0, pfrag(ph, i), acc[i % DT], 0, 0, 0);
      // fragment f = i / DT (pairs 4 f .. 4 f + 3) is in use: form the next one's low parts
      if (i / DT + 1 < 4) {
#pragma unroll
        for (int k = 0; k < 4 / DT; ++k) lo_of(scur, 4 * (i / DT + 1) + (i % DT) * (4 / DT) + k, ph, pl);
      }
      acc[i % DT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b0, pfrag(pl, i), acc[i % DT], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      b0 = b1;
      b1 = b2;
    }
    block_end();
  };
  // Generic step (the diagonal block, the segment end, blocks beyond some of the
  // wave's rows): the same loads and barriers as the fast step.
  auto step = [&](int i, f32x16(&scur)[2], f32x16(&snext)[2]) MODA_INL {
    const int kb = bid(i);
    if (!SPLIT && kb < n_full) {
      fast_step(i, scur, snext);
      return;
    }
    issue_group(i + P);
    if (i + 1 < nbw && active(bid(i + 1))) qk(kst + stage_of(i + 1) * SM::STAGE, snext);
    if (active(kb)) {
      mask_block(kb, scur);
      const float m_use = max_and_rescale(scur);
      uint32_t ph[2][8], pl[2][8];
      float lsum = 0.f;
#pragma unroll
      for (int q = 0; q < 16; ++q) exp_pair(scur, m_use, q, ph, pl, lsum);
      l_run += lsum;
      const unsigned char* vs = vst + stage_of(i) * SM::STAGE;
#pragma unroll
      for (int j = 0; j < NPV; ++j) {
        const bf16x8 b = vread(vs, j);
        acc[j % DT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, pfrag(ph, j), acc[j % DT], 0, 0, 0);
        acc[j % DT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, pfrag(pl, j), acc[j % DT], 0, 0, 0);
      }
    }
    block_end();
  };
  // Split tiles: the fully visible blocks are a prefix of this wave's blocks, so a
  // loop of fast steps runs first and one of generic steps after it (no path merge
  // inside either loop: at one wave per SIMD the register allocator otherwise
  // copies the score vectors at every merge). Shared tiles choose per step (their
  // register budget is tighter and one loop spills less).
  const int nfw = SPLIT ? (n_full > wave_u ? (n_full - wave_u + NW - 1) / NW : 0) : 0;
  const int n_fast = nfw < nbw ? nfw : nbw;
  int i = 0;
  for (; i + 1 < n_fast; i += 2) {
    fast_step(i, sA, sB);
    fast_step(i + 1, sB, sA);
  }
  if (i < n_fast) {  // odd count: one more fast step, then the generic loop starts from sB
    fast_step(i, sA, sB);
    ++i;
#pragma unroll
    for (int st = 0; st < 2; ++st) sA[st] = sB[st];
  }
  for (; i < nbw; i += 2) {
    step(i, sA, sB);
    if (i + 1 < nbw) step(i + 1, sB, sA);
  }
  // the groups issued past the last block must land before their LDS is reused
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

  // ---- fold in the depth state of this row ------------------------------------
  if constexpr (SPLIT) {
    // finish the depth pass (its own LDS area), then merge the partial states of
    // waves 1 .. NW - 1 into wave 0's through the (now free) stage bytes
    if constexpr (SELECT) {
      sel_pass();
    } else if constexpr (DEPTH) {
      if constexpr (!EARLY_DEPTH) depth_begin();
      depth_end();
    }
    __syncthreads();  // every wave is past its loop: the stages are free, depth rows published
    float* mg = reinterpret_cast<float*>(smem);  // [NW - 1][64][MG]
    if (wave > 0) {
      float* rec = mg + ((wave - 1) * 64 + lane) * SM::MG;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *reinterpret_cast<float4*>(rec + 16 * dt + 4 * q4) =
              make_float4(acc[dt][4 * q4], acc[dt][4 * q4 + 1], acc[dt][4 * q4 + 2], acc[dt][4 * q4 + 3]);
      *reinterpret_cast<float4*>(rec + 16 * DT) = make_float4(m_run, l_run, 0.f, 0.f);
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      const float* rec = mg + ((w - 1) * 64 + lane) * SM::MG;
      const float4 st = *reinterpret_cast<const float4*>(rec + 16 * DT);
      const float m_new = fmaxf(m_run, st.x);
      const float m_use = (m_new == NEG_INF) ? 0.f : m_new;
      const float f_a = fast_exp2(m_run - m_use), f_b = fast_exp2(st.x - m_use);
      l_run = l_run * f_a + st.y * f_b;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 x = *reinterpret_cast<const float4*>(rec + 16 * dt + 4 * q4);
          acc[dt][4 * q4 + 0] = fmaf(x.x, f_b, acc[dt][4 * q4 + 0] * f_a);
          acc[dt][4 * q4 + 1] = fmaf(x.y, f_b, acc[dt][4 * q4 + 1] * f_a);
          acc[dt][4 * q4 + 2] = fmaf(x.z, f_b, acc[dt][4 * q4 + 2] * f_a);
          acc[dt][4 * q4 + 3] = fmaf(x.w, f_b, acc[dt][4 * q4 + 3] * f_a);
        }
      m_run = m_new;
    }
    if constexpr (DEPTH) depth_fold();
  } else if (depth_first && !pass_first) {
    __syncthreads();  // every wave is past its loop: the K/V area is free for the hand-off
    depth_begin();
    depth_end();
    __syncthreads();
    depth_fold();
  }  // the other shared tiles folded their depth state before the loop

  // ---- normalise once and write ------------------------------------------------
  // A lane holds 4 output values of one row, so a direct store would spread each
  // instruction over 32 rows. The wave's 32 rows go through LDS instead (the stage
  // bytes, free once every wave is past its loop) and leave as whole rows: lane l
  // stores 16-byte chunk l % CH of row l / CH. Marking the stores non-temporal
  // takes about a third off what the writes cost the depth stream.
  constexpr int EB = OUT_F32 ? 4 : 2;   // output element bytes
  constexpr int RB = D * EB;            // bytes of one output row
  constexpr int CH = RB / 16;           // 16-byte chunks per row (8 .. 32)
  constexpr int ORI = 64 / CH;          // rows per store instruction
  static_assert(SM::SEQ_BYTES >= (SPLIT ? 1 : NW) * WROWS * RB, "output staging");
  if constexpr (!SPLIT) __syncthreads();  // other waves may still read the stages or the hand-off
  unsigned char* ob = smem + (SPLIT ? 0 : wave * WROWS * RB);
  // The empty asm makes the lane terms opaque here, so the compiler cannot form
  // the staging addresses before the loops and hold (spill) them across them.
  int er = r, ehh = hh;
  asm volatile("" : "+v"(er), "+v"(ehh));
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int off = (32 * dt + 8 * q4 + 4 * ehh) * EB;  // byte offset in the row
      unsigned char* dst = ob + er * RB + 16 * ((off / 16) ^ (er % CH)) + off % 16;
      if constexpr (OUT_F32) {
        *reinterpret_cast<float4*>(dst) = make_float4(acc[dt][4 * q4 + 0] * inv, acc[dt][4 * q4 + 1] * inv,
                                                      acc[dt][4 * q4 + 2] * inv, acc[dt][4 * q4 + 3] * inv);
      } else {
        *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16(acc[dt][4 * q4 + 0] * inv, acc[dt][4 * q4 + 1] * inv),
                                                    pack_bf16(acc[dt][4 * q4 + 2] * inv, acc[dt][4 * q4 + 3] * inv));
      }
    }
  if (row_valid && hh == 0 && p.lse) {
    const int64_t lbase = p.lse_batch_layout ? (int64_t)seg * Hq * p.lse_head_stride : seg_start;
    p.lse[lbase + (int64_t)hq * p.lse_head_stride + tq] = (m_run + __log2f(l_tot)) * LN2;
  }
  const int c = lane % CH;
#pragma unroll
  for (int j = 0; j < WROWS / ORI; ++j) {
    const int rr = j * ORI + lane / CH;  // row within the wave
    const int64_t t = t0 + (wrow0 + rr) / GB;
    const int h = hbase + (wrow0 + rr) % GB;
    const u32x4 v = *reinterpret_cast<const u32x4*>(ob + rr * RB + 16 * (c ^ (rr % CH)));
    if (t < len)  // streaming store: nothing reads the output back here
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(static_cast<unsigned char*>(p.out) +
                                                              ((seg_start + t) * Hq + h) * (int64_t)RB + 16 * c));
  }
}

template <int D, int GB, int NW, int MODE, bool SPLIT>
hipError_t launch_t(const Params& p, bool out_f32, hipStream_t stream) {
  const dim3 grid((unsigned)p.n_tiles), block(64 * NW);
  if (out_f32)
    hipLaunchKernelGGL((moda_fwd_bf16_kernel<D, GB, NW, MODE, true, SPLIT>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((moda_fwd_bf16_kernel<D, GB, NW, MODE, false, SPLIT>), grid, block, 0, stream, p);
  return hipGetLastError();
}

// phase: kPhaseBoth (the operator), kPhaseSeq (sequence keys only) or
// kPhaseDepth (depth slots only, n_depth > 0): the same kernel code with the
// other part compiled out.
template <int D, int GB, int NW, bool SPLIT>
hipError_t launch_d(const Params& p, int phase, bool out_f32, hipStream_t stream) {
  if (phase == kPhaseDepth) return launch_t<D, GB, NW, kDepthOnly, SPLIT>(p, out_f32, stream);
  if (p.n_depth == 0 || phase == kPhaseSeq) return launch_t<D, GB, NW, kNoDepth, SPLIT>(p, out_f32, stream);
  if (p.sel_fused) return launch_t<D, GB, NW, kSelect, SPLIT>(p, out_f32, stream);
  return launch_t<D, GB, NW, kSerial, SPLIT>(p, out_f32, stream);
}

}  // namespace

// Every (head dim, heads per workgroup) pair is instantiated in a compilation
// unit of its own (MODA_FWD_D / MODA_FWD_GB), so the instances build in parallel.
template <int D, int GB>
hipError_t launch_fwd_bf16_dg(const Params& p, int waves, bool split, int phase, bool out_f32, hipStream_t stream) {
  if (split) {
    if (waves == kSplitWaves<D>) return launch_d<D, GB, kSplitWaves<D>, true>(p, phase, out_f32, stream);
    return hipErrorInvalidValue;
  }
  if (waves == 2) return launch_d<D, GB, 2, false>(p, phase, out_f32, stream);
  if (waves == 4) return launch_d<D, GB, 4, false>(p, phase, out_f32, stream);
  return hipErrorInvalidValue;
}

#if defined(MODA_FWD_D) && defined(MODA_FWD_GB)
template hipError_t launch_fwd_bf16_dg<MODA_FWD_D, MODA_FWD_GB>(const Params&, int, bool, int, bool, hipStream_t);
#endif

}  // namespace moda

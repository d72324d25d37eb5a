// Internal interface between the host dispatch (moda_attn.hip) and the kernels.
// Not part of the public C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moda_debug.h"

namespace moda {

// One launch of the fused joint sequence/depth attention forward.
// Token n of segment s is packed token seg_start(s) + t, 0 <= t < seg_len(s).
// Element offsets (in elements of the input dtype, always 64-bit):
//   q, out : (n * Hq + h) * D + c
//   k, v   : (n * Hkv + hk) * D + c
//   depth  : ((n * S_cap + i) * Hkv + hk) * D + c
//   lse    : lse_seg_base(s) + h * lse_head_stride + t
struct Params {
  const void* q;
  const void* k;
  const void* v;
  const void* kd;
  const void* vd;
  void* out;
  float* lse;  // may be null

  const int32_t* cu_seqlens;  // device, n_seg + 1 entries; null = uniform segments
  int64_t uniform_len;        // segment length when cu_seqlens is null
  int64_t total_tokens;       // N: every packed index is clamped below this
  int32_t n_seg;
  int32_t n_qblocks;          // query blocks per (segment, head group)

  int32_t Hq, Hkv, G;
  int32_t n_hgroups;          // G / heads-per-block
  int32_t S_cap, n_depth;
  int32_t causal;
  float scale_log2;           // scale * log2(e): logits go to base 2

  int64_t lse_head_stride;    // T (batch layout) or N (packed layout)
  int32_t lse_batch_layout;   // 1: base = s * Hq * T; 0: base = seg_start
  int32_t xcd_interleave;     // 1: (segment, KV head) pairs go round-robin to the 8 XCDs;
                              // 2: KV head fastest, KV head hk on XCD hk % 8
  int32_t qb_major;           // 1: tiles ordered by query block across all pairs (heaviest first)
  int32_t phase;              // kPhaseBoth, or one part alone (kPhaseSeq / kPhaseDepth)
  int64_t n_tiles;
  // bounded depth reads, fp32 path: bit i of depth_mask[n * Hq + h] says whether
  // slot i enters row (n, h)'s softmax (null = every slot below n_depth)
  const uint64_t* depth_mask;
  // bounded depth reads, bf16 path (sel_fused = 1): selected inside the depth pass;
  // 0 < sel_topk < n_depth - sel_recent, 0 <= sel_recent <= n_depth
  int32_t sel_fused, sel_topk, sel_recent;
};

// Which key sets enter the softmax of a forward launch: both (the operator), or
// one alone (its partial softmax, for measuring and checking the two parts).
constexpr int kPhaseSeq = 1;
constexpr int kPhaseDepth = 2;
constexpr int kPhaseBoth = 3;

// Launchers (return the hipError_t of the launch). The bf16 kernel's instances
// are split by head dim D and query heads per workgroup GB (moda_fwd_bf16.hip).
template <int D, int GB>
hipError_t launch_fwd_bf16_dg(const Params& p, int waves, bool split, int phase, bool out_f32, hipStream_t stream);
hipError_t launch_fwd_f32(const Params& p, int head_dim, hipStream_t stream);

// Expanded query rows (tokens x grouped heads) per bf16 wave; a workgroup has 1,
// 2 or 4 waves.
constexpr int kWaveRows = 32;
// Waves per workgroup of the split bf16 kernel (they share one 32-row tile and
// split its key blocks). Their K/V stages take 2 x 2 x 16 KB per wave at D = 128
// and 2 x 2 x 8 KB at D = 64; two waves keep two workgroups per CU at D = 64, so
// the small grids run in one round.
template <int D>
constexpr int kSplitWaves = 2;
constexpr int kF32BlockRows = 64;

// Backward of the joint forward (see moda_bwd.hip). Offsets as in Params; out,
// dout and every gradient are in the gradient dtype; delta and dq_depth are fp32
// workspace: delta[h * N + n] = <dout, out> of row (n, h); dq_depth[(n * Hq + h) * D + c]
// is the depth slots' share of dq (written only when n_depth > 0).
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* kd;
  const void* vd;
  const void* out;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  void* dkd;
  void* dvd;
  float* delta;
  float* dq_depth;

  const int32_t* cu_seqlens;  // null = uniform segments of uniform_len tokens
  int64_t uniform_len;
  int64_t total_tokens;       // N
  int32_t n_seg;
  int32_t n_qblocks;          // 128-token blocks per segment (bf16 dq kernel)
  int32_t n_kblocks;          // 128-key blocks per segment (bf16 dk/dv kernel)
  int32_t Hq, Hkv, G;
  int32_t S_cap, n_depth;
  int32_t causal;
  float scale;
  float scale_log2;
  int64_t lse_head_stride;    // as in Params
  int32_t lse_batch_layout;
  int32_t xcd_group;          // 1: dq/dk-dv rows grouped per XCD (needs rows % 8 == 0 in both grids)
};

hipError_t launch_bwd(const BwdParams& p, int head_dim, bool bf16, bool grad_f32, hipStream_t stream);

// Slot selection of bounded depth reads (moda_depth_select.hip): per (token n,
// query head h) the 64-bit mask of the slots [0, n_depth) that enter the softmax:
// the last `recent`, and the `topk` largest logits of the others (ties to the
// lower slot). n_depth <= 64.
struct SelectParams {
  const void* q;
  const void* kd;
  uint64_t* mask;  // [N, Hq]
  int64_t n_tokens;
  int32_t Hq, Hkv, G;
  int32_t S_cap, n_depth, topk, recent;
  float scale;
};
constexpr int kMaxSelectSlots = 64;
hipError_t launch_depth_select(const SelectParams& p, int head_dim, bool bf16, hipStream_t stream);

// Depth-KV writer (moda_depth_kv.hip): rows of row_vecs 16-byte vectors per token.
struct DepthWriteParams {
  const void* k_src;
  const void* v_src;
  void* k_depth;
  void* v_depth;
  int64_t n_tokens;
  int64_t row_vecs;  // H_kv * d * element bytes / 16
  int32_t S_cap;
  int32_t slot;
};
hipError_t launch_depth_kv_write(const DepthWriteParams& p, hipStream_t stream);

// The FFN input's KV projection into one depth slot (moda_depth_kv_project.hip):
// x [N, d_model], w [2 hd, d_model] (key rows, then value rows), hd = H_kv d;
// outputs at element ((n S_cap + slot) hd + c) of k_depth / v_depth.
struct ProjParams {
  const void* x;
  const void* w;
  void* kd;
  void* vd;
  int64_t n_tokens;
  int32_t d_model;  // a multiple of 64
  int32_t hd;       // H_kv * d, a multiple of 64
  int32_t S_cap;
  int32_t slot;
  int32_t n_feat_tiles;  // set by the launcher
  int64_t n_tok_tiles;   // set by the launcher
};
hipError_t launch_depth_kv_project(ProjParams p, bool bf16, hipStream_t stream);

// One decode step (one new token per sequence); see moda_decode.hip.
// Element offsets: q, out: (b * Hq + h) * D + c; caches: ((b * T_max + j) * Hkv + hk) * D + c;
// depth: ((b * S_cap + i) * Hkv + hk) * D + c; lse: b * Hq + h.
struct DecodeParams {
  const void* q;
  const void* kc;
  const void* vc;
  const void* kd;
  const void* vd;
  void* out;
  float* lse;                  // may be null
  const int32_t* cache_seqlens;  // device, B entries
  float* workspace;            // [B][Hq][n_chunks][D + 4] fp32 partial states
  int64_t B;
  int64_t T_max;
  int32_t Hq, Hkv, G, n_hgroups;
  int32_t S_cap, n_depth;
  float scale_log2;
  int64_t chunk;               // cache rows per chunk (a multiple of the partial kernel's rows per batch round)
  int32_t n_seq_chunks;        // ceil(T_max / chunk)
  int32_t n_chunks;            // n_seq_chunks + 1 (the last one holds the depth slots)
  int64_t n_partial_blocks;    // B * Hkv * n_hgroups * n_chunks
};

// Rows a decode chunk is a multiple of (one round of load batches of all waves).
int decode_rows_per_chunk_unit(int head_dim);
hipError_t launch_decode(const DecodeParams& p, int head_dim, int heads_per_block, bool bf16, bool out_f32,
                         hipStream_t stream);

// The arguments of one decode step as the C ABI takes them (without workspace).
struct DecodeArgs {
  const void *q, *k_cache, *v_cache, *k_depth, *v_depth;
  void* out;
  float* lse;
  int32_t dtype, out_dtype;
  const int32_t* cache_seqlens;
  int64_t batch;
  int32_t max_cache_len, n_heads_q, n_heads_kv, head_dim, depth_capacity, n_depth;
  float scale;
};
// A checked decode step: kernel parameters (all but the workspace) and the
// workspace it needs.
struct DecodePlan {
  DecodeParams p;
  int head_dim, heads_per_block;
  bool bf16, out_f32;
  int64_t workspace_bytes;
};
constexpr int kNothingToLaunch = -1;  // decode_prepare: a valid empty problem (batch 0)
// Host checks of a decode step (no HIP call): MODA_OK with `plan` filled,
// kNothingToLaunch, or an error status with the per-thread message set.
int decode_prepare(const DecodeArgs& a, DecodePlan& plan);
// Launches both decode kernels with `workspace` (plan.workspace_bytes of device
// memory); MODA_OK or MODA_ERR_HIP.
int decode_launch(DecodePlan& plan, void* workspace, hipStream_t stream);
// Sets the per-thread message moda_last_error() returns; returns `code`.
int set_error(int code, const char* msg);

}  // namespace moda

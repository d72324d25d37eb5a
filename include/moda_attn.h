/*
 * moda_attn.h - C ABI of the MoDA joint sequence/depth attention (forward,
 * backward, decode step and depth-KV writer) on AMD Instinct MI355X (gfx950).
 *
 * Operator: "Mixture-of-Depths Attention" (arXiv 2603.15619), MoDA deck slide
 * "One denominator allocates probability across both memories" (teaching form of
 * paper Sec. 2.2 / Algorithm 1). For query head h and token t of a sequence:
 *
 *   a_j = scale * <q_t, k_j>             sequence keys j <= t (all j if causal == 0)
 *   b_i = scale * <q_t, k_depth_{t,i}>   the token's own depth slots i < n_depth
 *   out_t = (sum_j e^{a_j} v_j + sum_i e^{b_i} v_depth_{t,i})
 *           / (sum_j e^{a_j} + sum_i e^{b_i})
 *   lse_t = ln(sum_j e^{a_j} + sum_i e^{b_i})        (natural log, float32)
 *
 * One numerator and one denominator span both key sets; this is not the sum of
 * two separate softmaxes. Query head h reads key/value head h / G (sequence and
 * depth alike), G = n_heads_q / n_heads_kv, contiguous groups (Table 1 of the
 * paper groups the depth cache by G).
 *
 * Layouts (row-major, last dimension contiguous, no padding):
 *   q, out    [B, T, Hq, d]            varlen: [N, Hq, d]   (out in out_dtype)
 *   k, v      [B, T, Hkv, d]           varlen: [N, Hkv, d]
 *   k_depth,
 *   v_depth   [B, T, S_cap, Hkv, d]    varlen: [N, S_cap, Hkv, d]
 *   lse       [B, Hq, T] float32       varlen: [Hq, N] float32
 * Slots [0, n_depth) of the slot axis are read; n_depth <= S_cap.
 *
 * Ownership: every pointer is device memory owned by the caller; the library
 * allocates nothing, keeps no pointer after returning, and launches
 * asynchronously on `stream` (a hipStream_t; NULL = the default stream). `out`
 * and `lse` are fully overwritten for every valid row; nothing else is written.
 *
 * Errors: all checks run on the host before any device work. On a non-zero
 * return nothing was launched and the outputs are untouched, except MODA_ERR_HIP,
 * which reports a failed launch. moda_last_error() then describes the failure
 * (per calling thread). The device contents of cu_seqlens are not checked on the
 * host: offsets are clamped to [0, N] on the device, so malformed offsets give
 * unspecified values but never an out-of-bounds access. Every entry point refuses
 * (MODA_ERR_SHAPE) sizes under which a tensor it names would hold 2^56 elements
 * or more, and the workspace-size queries return -1 for them, so no size the
 * library computes can overflow.
 */
#ifndef MODA_ATTN_H
#define MODA_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MODA_ABI_VERSION 7

/* status codes */
#define MODA_OK 0
#define MODA_ERR_NULL 1        /* a required pointer is NULL                      */
#define MODA_ERR_SHAPE 2       /* sizes negative, inconsistent or too large       */
#define MODA_ERR_DTYPE 3       /* unknown dtype code or unsupported dtype pair    */
#define MODA_ERR_ALIGN 4       /* a tensor pointer is not 16-byte aligned         */
#define MODA_ERR_UNSUPPORTED 5 /* valid request outside what is built (head_dim)  */
#define MODA_ERR_HIP 6         /* the HIP runtime rejected the launch             */
#define MODA_ERR_VALUE 7       /* scale not finite and positive                   */

/* dtype codes. `dtype` is the storage type of q, k, v, k_depth and v_depth;
 * `out_dtype` that of out. Supported pairs: (F32, F32); (BF16, BF16) and
 * (BF16, F32). bf16 inputs are computed with fp32 accumulation and fp32 softmax
 * state; the probabilities enter the P.V product rounded to bf16. A bf16 `out`
 * is the fp32 result rounded to nearest-even once, after normalisation. */
#define MODA_DTYPE_F32 0
#define MODA_DTYPE_BF16 1

/*
 * Joint sequence/depth attention forward over B equal-length sequences.
 *
 * batch (B) >= 0, seqlen (T) >= 0: B * T == 0 returns MODA_OK with no launch.
 * n_heads_q % n_heads_kv == 0. head_dim (d) in {64, 128}.
 * depth_capacity (S_cap) >= n_depth >= 0; k_depth / v_depth may be NULL only when
 * n_depth == 0. lse may be NULL (not written). scale > 0 and finite (the MoDA
 * operator uses 1/sqrt(d)). causal: 1 = keys j <= t (the MoDA operator), 0 = all
 * keys of the sequence.
 * Returns MODA_OK or an error code above.
 */
int moda_attn_fwd(const void* q, const void* k, const void* v, const void* k_depth, const void* v_depth,
                  void* out, float* lse, int32_t dtype, int32_t out_dtype, int64_t batch, int64_t seqlen,
                  int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim, int32_t depth_capacity,
                  int32_t n_depth, int32_t causal, float scale, void* stream);

/*
 * Same operator over packed variable-length sequences.
 *
 * cu_seqlens: DEVICE pointer to n_seqs + 1 non-decreasing int32 offsets,
 * cu_seqlens[0] == 0, cu_seqlens[n_seqs] == total_tokens (N); sequence s holds
 * packed tokens [cu_seqlens[s], cu_seqlens[s+1]). max_seqlen must be >= every
 * sequence length (rows beyond max_seqlen are not computed). Attention never
 * crosses a sequence boundary, for the sequence keys nor for the depth slots.
 * n_seqs == 0 or total_tokens == 0 returns MODA_OK with no launch.
 */
int moda_attn_fwd_varlen(const void* q, const void* k, const void* v, const void* k_depth,
                         const void* v_depth, void* out, float* lse, int32_t dtype, int32_t out_dtype,
                         const int32_t* cu_seqlens, int32_t n_seqs, int64_t total_tokens, int32_t max_seqlen,
                         int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim, int32_t depth_capacity,
                         int32_t n_depth, int32_t causal, float scale, void* stream);

/*
 * The two parts of the forward, one at a time (for measuring each part and for
 * checking the merge of their partial results; not needed to compute the
 * operator). MoDA deck, slide "Shared online-softmax states preserve the joint
 * operator": the sequence blocks and the depth blocks update one running
 * softmax state, so each part alone is a softmax of its own, and the operator is
 * their merge by log-sum-exp:
 *   phase_mask 1: out = softmax over the sequence keys alone, lse = its log-sum-exp;
 *   phase_mask 2: out = softmax over the token's depth slots alone (n_depth > 0);
 *   phase_mask 3: the operator (identical to moda_attn_fwd / moda_attn_fwd_varlen).
 * With (o_s, l_s) and (o_d, l_d) from phases 1 and 2, l = ln(e^l_s + e^l_d) and
 * out = e^(l_s - l) o_s + e^(l_d - l) o_d. Each phase runs the kernel of the fused
 * call with the other part compiled out. Arguments, checks and errors as for
 * moda_attn_fwd / moda_attn_fwd_varlen; MODA_ERR_VALUE for any other phase_mask
 * and for phase_mask 2 with n_depth == 0.
 */
int moda_attn_fwd_phases(const void* q, const void* k, const void* v, const void* k_depth, const void* v_depth,
                         void* out, float* lse, int32_t dtype, int32_t out_dtype, int64_t batch, int64_t seqlen,
                         int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim, int32_t depth_capacity,
                         int32_t n_depth, int32_t causal, float scale, int32_t phase_mask, void* stream);
int moda_attn_fwd_varlen_phases(const void* q, const void* k, const void* v, const void* k_depth,
                                const void* v_depth, void* out, float* lse, int32_t dtype, int32_t out_dtype,
                                const int32_t* cu_seqlens, int32_t n_seqs, int64_t total_tokens, int32_t max_seqlen,
                                int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim, int32_t depth_capacity,
                                int32_t n_depth, int32_t causal, float scale, int32_t phase_mask, void* stream);

/*
 * Bounded depth reads (top-S, sliding window or hybrid slot buffer): the operator
 * of moda_attn_fwd / moda_attn_fwd_varlen in which each query row (token t, head
 * h) reads only some of its depth slots. The MoDA deck lists such a bounded
 * S << L slot buffer as future work (slide "The main open cost is retaining and
 * reading depth history", paper Sec. 6.1-6.2) without defining it; the reading
 * taken here: of slots [0, n_depth), the last depth_recent always enter the joint
 * softmax; of the others, the depth_topk with the largest depth logits
 * b_i = scale <q_t, k_depth_{t,i}> enter, ties going to the lower slot index; the
 * other slots leave the softmax as if absent. depth_recent = 0 is top-S,
 * depth_topk = 0 a sliding window of the depth_recent most recent slots, both > 0
 * the hybrid. When depth_topk covers every older slot the call is the operator.
 *
 * bf16 inputs: the forward's depth pass makes the selection itself (it reads
 * every slot's key, ranks each row's logits, then reads the values of the kept
 * slots only) and leaves `workspace` untouched. fp32 inputs: a selection kernel
 * scores every slot and writes a 64-bit slot mask per row to `workspace`, which
 * the forward then reads. `workspace`: DEVICE memory of at least
 * moda_attn_fwd_topk_workspace_size(N, Hq) bytes, 16-byte aligned, caller-owned,
 * contents on entry irrelevant; calls that share one workspace must not overlap
 * (required for both dtypes). Every kernel runs on `stream`. The logits that
 * decide the selection are fp32: slots whose logits tie within fp32 rounding may
 * be chosen either way.
 * n_depth <= 64 (MODA_ERR_UNSUPPORTED otherwise); depth_topk, depth_recent >= 0
 * (MODA_ERR_VALUE). Other arguments, checks and errors as for moda_attn_fwd /
 * moda_attn_fwd_varlen; MODA_ERR_SHAPE also for a too small workspace.
 */
int moda_attn_fwd_topk(const void* q, const void* k, const void* v, const void* k_depth, const void* v_depth,
                       void* out, float* lse, int32_t dtype, int32_t out_dtype, int64_t batch, int64_t seqlen,
                       int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim, int32_t depth_capacity,
                       int32_t n_depth, int32_t depth_topk, int32_t depth_recent, int32_t causal, float scale,
                       void* workspace, int64_t workspace_bytes, void* stream);
int moda_attn_fwd_varlen_topk(const void* q, const void* k, const void* v, const void* k_depth, const void* v_depth,
                              void* out, float* lse, int32_t dtype, int32_t out_dtype, const int32_t* cu_seqlens,
                              int32_t n_seqs, int64_t total_tokens, int32_t max_seqlen, int32_t n_heads_q,
                              int32_t n_heads_kv, int32_t head_dim, int32_t depth_capacity, int32_t n_depth,
                              int32_t depth_topk, int32_t depth_recent, int32_t causal, float scale, void* workspace,
                              int64_t workspace_bytes, void* stream);

/* Workspace bytes of the bounded depth reads for N = total tokens (B * T), or -1
 * for invalid sizes. */
int64_t moda_attn_fwd_topk_workspace_size(int64_t total_tokens, int32_t n_heads_q);

/*
 * One decode step: a single new token per sequence attends, through the same
 * joint softmax, to its sequence-cache prefix and to its own depth slots (the
 * decode-time sequence and depth caches of the paper's Table 1, as the MoDA deck
 * quotes it on slide "Depth compute still accumulates quadratically in depth").
 *
 *   q          [B, Hq, d]              the new tokens' queries
 *   k_cache,
 *   v_cache    [B, T_max, Hkv, d]      sequence b reads rows 0 .. cache_seqlens[b] - 1;
 *                                      the last of them is the new token's own key/value
 *   k_depth,
 *   v_depth    [B, S_cap, Hkv, d]      the new token's depth slots; [0, n_depth) are read
 *   out        [B, Hq, d] (out_dtype)  lse [B, Hq] float32 (may be NULL)
 *   cache_seqlens: DEVICE pointer to B int32 lengths in [1, T_max] (T_max =
 *   max_cache_len); values outside are clamped to that range on the device.
 *
 * dtype pairs, head_dim, grouping and scale as for moda_attn_fwd. The causal
 * mask is implied (the cache prefix is the visible set).
 *
 * workspace: DEVICE memory of at least moda_attn_decode_workspace_size(...)
 * bytes, 16-byte aligned, owned by the caller; it holds fp32 partial states of
 * the key chunks between the two kernels of the step, its contents on entry do
 * not matter, and calls that share one workspace must not overlap. The call
 * launches both kernels on `stream` and returns without waiting.
 * Returns MODA_OK or an error code (MODA_ERR_SHAPE also for a too small workspace).
 */
int moda_attn_decode(const void* q, const void* k_cache, const void* v_cache, const void* k_depth,
                     const void* v_depth, void* out, float* lse, int32_t dtype, int32_t out_dtype,
                     const int32_t* cache_seqlens, int64_t batch, int32_t max_cache_len, int32_t n_heads_q,
                     int32_t n_heads_kv, int32_t head_dim, int32_t depth_capacity, int32_t n_depth, float scale,
                     void* workspace, int64_t workspace_bytes, void* stream);

/*
 * moda_attn_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). The same two kernels pass their partial
 * states through a device array the library holds: MODA_DECODE_SCRATCH_BYTES per
 * GPU, set up on the first call on that GPU (the current device; `stream`, if
 * not NULL, must belong to it) and kept until the process ends. The call
 * allocates nothing. Steps whose moda_attn_decode_workspace_size exceeds
 * MODA_DECODE_SCRATCH_BYTES are rejected with MODA_ERR_SHAPE (use
 * moda_attn_decode with a workspace). All calls on one GPU share the array:
 * calls that overlap on one GPU (other streams, other threads) race; calls in
 * order on one stream do not. Arguments, checks, results and errors otherwise
 * as for moda_attn_decode.
 */
#define MODA_DECODE_SCRATCH_BYTES (16ll << 20)
int moda_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, const void* k_depth,
                             const void* v_depth, void* out, float* lse, int32_t dtype, int32_t out_dtype,
                             const int32_t* cache_seqlens, int64_t batch, int32_t max_cache_len, int32_t n_heads_q,
                             int32_t n_heads_kv, int32_t head_dim, int32_t depth_capacity, int32_t n_depth,
                             float scale, void* stream);

/* Workspace bytes moda_attn_decode needs for these sizes, or -1 for invalid sizes. */
int64_t moda_attn_decode_workspace_size(int64_t batch, int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim,
                                        int32_t max_cache_len);

/*
 * Backward of moda_attn_fwd: the gradients of the joint operator for an upstream
 * gradient dout of out. The pages (MoDA deck, slide "One denominator allocates
 * probability across both memories") define the forward; this is its exact
 * derivative. With P the joint softmax of row (t, h) over its visible sequence
 * keys and its own depth slots (recomputed from lse), delta_t = <dout_t, out_t>
 * and dS_x = P_x (<dout_t, value_x> - delta_t):
 *   dq_t = scale (sum_j dS_j k_j + sum_i dS_i k_depth_{t,i})
 *   dk_j = scale sum_t dS_tj q_t,  dv_j = sum_t P_tj dout_t
 *   dk_depth_{t,i} = scale dS_ti q_t,  dv_depth_{t,i} = P_ti dout_t
 * with the sums of the G query heads of a KV head added into it.
 *
 * q, k, v, k_depth, v_depth: the forward's inputs, in `dtype`. out, dout and
 * every gradient (dq, dk, dv, dk_depth, dv_depth) are in `grad_dtype`, laid out
 * like the tensor they belong to; lse is the forward's float32 lse (required).
 * dtype pairs as for the forward: (F32, F32), (BF16, BF16), (BF16, F32). For bf16
 * inputs the matrix products take bf16 operands (dout and the softmax gradient
 * rounded to bf16) with fp32 accumulation.
 * dq, dk, dv are fully overwritten. dk_depth / dv_depth: slots [0, n_depth) are
 * overwritten, slots [n_depth, S_cap) are not written; both may be NULL when
 * n_depth == 0. n_heads_q / n_heads_kv <= 16.
 *
 * workspace: DEVICE memory of at least moda_attn_bwd_workspace_size(...) bytes,
 * 256-byte aligned, owned by the caller (fp32 delta and the depth share of dq);
 * contents on entry do not matter; calls sharing one workspace must not overlap.
 * Launches on `stream` and returns without waiting. Other arguments, checks and
 * errors as for moda_attn_fwd; MODA_ERR_SHAPE also for a too small workspace.
 */
int moda_attn_bwd(const void* q, const void* k, const void* v, const void* k_depth, const void* v_depth,
                  const void* out, const void* dout, const float* lse, void* dq, void* dk, void* dv,
                  void* dk_depth, void* dv_depth, int32_t dtype, int32_t grad_dtype, int64_t batch, int64_t seqlen,
                  int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim, int32_t depth_capacity, int32_t n_depth,
                  int32_t causal, float scale, void* workspace, int64_t workspace_bytes, void* stream);

/* The backward over packed variable-length sequences (layouts and cu_seqlens as
 * for moda_attn_fwd_varlen, lse [Hq, N]). */
int moda_attn_bwd_varlen(const void* q, const void* k, const void* v, const void* k_depth, const void* v_depth,
                         const void* out, const void* dout, const float* lse, void* dq, void* dk, void* dv,
                         void* dk_depth, void* dv_depth, int32_t dtype, int32_t grad_dtype,
                         const int32_t* cu_seqlens, int32_t n_seqs, int64_t total_tokens, int32_t max_seqlen,
                         int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim, int32_t depth_capacity,
                         int32_t n_depth, int32_t causal, float scale, void* workspace, int64_t workspace_bytes,
                         void* stream);

/* Workspace bytes the backward needs for N = total tokens (B * T), or -1 for
 * invalid sizes. */
int64_t moda_attn_bwd_workspace_size(int64_t total_tokens, int32_t n_heads_q, int32_t head_dim, int32_t n_depth);

/*
 * Depth-KV writer: stores one layer's key and value rows of every token into
 * slot `slot` of the depth cache that later layers read (MoDA deck, slide "Reuse
 * attention KV; add a projection for FFN inputs": a layer's attention KV is kept
 * for later layers; the FFN input's KV projection fills further slots, written
 * with the same call from the projection's output).
 *
 *   k_src, v_src       [N, Hkv, d]            (batch layout: N = B * T)
 *   k_depth, v_depth   [N, S_cap, Hkv, d]     slot `slot` of every token is overwritten
 *
 * All in `dtype`; 0 <= slot < depth_capacity (S_cap); Hkv * d * element bytes a
 * multiple of 16; all pointers 16-byte aligned, device memory owned by the
 * caller; sources and destinations must not overlap. Nothing else is written.
 * A bounded slot buffer (the paper's future work, as the deck quotes it on slide
 * "The main open cost is retaining and reading depth history") writes entry w to
 * slot w mod S_cap and reads n_depth = min(w + 1, S_cap) slots: the joint softmax
 * is invariant to the order of its keys, so that is a sliding window over the
 * most recent S_cap entries. A window [o, o + n) of a longer slot axis is read by
 * passing k_depth + o * Hkv * d (and v_depth likewise) with the same
 * depth_capacity and n_depth = n, o + n <= S_cap.
 * n_tokens == 0 returns MODA_OK with no launch.
 */
int moda_depth_kv_write(const void* k_src, const void* v_src, void* k_depth, void* v_depth, int32_t dtype,
                        int64_t n_tokens, int32_t n_heads_kv, int32_t head_dim, int32_t depth_capacity, int32_t slot,
                        void* stream);

/*
 * The FFN input's KV projection, written straight into one depth slot (MoDA
 * deck, slide "Reuse attention KV; add a projection for FFN inputs", paper Sec.
 * 2.2: step 4 projects the FFN input into additional depth KV slots; the default
 * variant reuses the attention KV, stored by moda_depth_kv_write, and adds this
 * projection). For every token n:
 *   k_depth[n, slot] = x_n W_k^T,  v_depth[n, slot] = x_n W_v^T   (each [Hkv, d])
 *
 *   x                  [N, d_model]               the FFN input of N tokens
 *   w_kv               [2 * Hkv * d, d_model]     [W_k; W_v] in the [out, in] layout of
 *                                                 a linear layer (key rows first); no bias
 *   k_depth, v_depth   [N, S_cap, Hkv, d]         slot `slot` of every token is overwritten
 *
 * All in `dtype`; bf16 is multiplied on the matrix cores with fp32 accumulation
 * and rounded to nearest-even once per output; fp32 in fp32. d_model a positive
 * multiple of 64 and head_dim in {64, 128} (MODA_ERR_UNSUPPORTED otherwise);
 * 0 <= slot < depth_capacity; all pointers 16-byte aligned, device memory owned
 * by the caller; x and w_kv must not overlap the cache. Nothing else is written.
 * n_tokens == 0 returns MODA_OK with no launch. Launches on `stream`.
 */
int moda_depth_kv_project(const void* x, const void* w_kv, void* k_depth, void* v_depth, int32_t dtype,
                          int64_t n_tokens, int32_t d_model, int32_t n_heads_kv, int32_t head_dim,
                          int32_t depth_capacity, int32_t slot, void* stream);

/* Description of the last non-OK status returned on the calling thread ("" if none). */
const char* moda_last_error(void);

/* MODA_ABI_VERSION of the loaded library. */
int32_t moda_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MODA_ATTN_H */

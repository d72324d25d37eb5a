// Host side of the C ABI: argument checks, work decomposition, kernel dispatch.
// Every check runs before any HIP call, so a rejected call touches no device state.
#include "moda_attn.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <initializer_list>

#include "moda_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// Every size the host derives from the arguments (element and byte counts,
// offsets, workspace sizes) is a product of a few of them with small constants.
// A call is refused unless each tensor it names holds fewer than 2^56 elements,
// so that none of those products can overflow int64 (checked without overflowing).
constexpr int64_t kMaxElems = int64_t(1) << 56;
bool fits(std::initializer_list<int64_t> factors) {
  int64_t x = 1;
  for (const int64_t f : factors) {
    if (f < 0 || __builtin_mul_overflow(x, f, &x) || x >= kMaxElems) return false;
  }
  return true;
}

// Query heads handled together by one bf16 workgroup: the largest power of two
// (at most 4) dividing the group size. A workgroup's heads share one KV head, so
// its depth slot rows are read once for all of them; the head groups of one KV
// head run side by side and meet in L2.
int heads_per_block(int G) {
  if (G % 4 == 0) return 4;
  if (G % 2 == 0) return 2;
  return 1;
}

struct Common {
  const void *q, *k, *v, *kd, *vd;
  void* out;
  float* lse;
  int32_t dtype, out_dtype, Hq, Hkv, d, S_cap, n_depth, causal;
  float scale;
};

int check_common(const Common& c) {
  if (!c.q || !c.k || !c.v || !c.out) return fail(MODA_ERR_NULL, "q, k, v and out must be non-NULL");
  if (c.dtype != MODA_DTYPE_F32 && c.dtype != MODA_DTYPE_BF16) return fail(MODA_ERR_DTYPE, "unknown dtype code %d", c.dtype);
  if (c.out_dtype != MODA_DTYPE_F32 && c.out_dtype != MODA_DTYPE_BF16)
    return fail(MODA_ERR_DTYPE, "unknown out_dtype code %d", c.out_dtype);
  if (c.dtype == MODA_DTYPE_F32 && c.out_dtype != MODA_DTYPE_F32)
    return fail(MODA_ERR_DTYPE, "fp32 inputs need an fp32 output");
  if (c.Hq < 1 || c.Hkv < 1) return fail(MODA_ERR_SHAPE, "head counts must be >= 1 (got Hq=%d Hkv=%d)", c.Hq, c.Hkv);
  if (c.Hq % c.Hkv != 0) return fail(MODA_ERR_SHAPE, "n_heads_q (%d) must be a multiple of n_heads_kv (%d)", c.Hq, c.Hkv);
  if (c.d != 64 && c.d != 128) return fail(MODA_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", c.d);
  if (c.n_depth < 0 || c.S_cap < c.n_depth)
    return fail(MODA_ERR_SHAPE, "need 0 <= n_depth (%d) <= depth_capacity (%d)", c.n_depth, c.S_cap);
  if (c.n_depth > 0 && (!c.kd || !c.vd)) return fail(MODA_ERR_NULL, "k_depth and v_depth must be non-NULL when n_depth > 0");
  if (!(c.scale > 0.f) || !isfinite(c.scale)) return fail(MODA_ERR_VALUE, "scale must be finite and > 0");
  if (c.causal != 0 && c.causal != 1) return fail(MODA_ERR_VALUE, "causal must be 0 or 1");
  if (!aligned16(c.q) || !aligned16(c.k) || !aligned16(c.v) || !aligned16(c.out))
    return fail(MODA_ERR_ALIGN, "q, k, v and out must be 16-byte aligned");
  if (c.n_depth > 0 && (!aligned16(c.kd) || !aligned16(c.vd)))
    return fail(MODA_ERR_ALIGN, "k_depth and v_depth must be 16-byte aligned");
  if (c.lse && (reinterpret_cast<uintptr_t>(c.lse) & 3u)) return fail(MODA_ERR_ALIGN, "lse must be 4-byte aligned");
  return MODA_OK;
}

moda::Params base_params(const Common& c) {
  moda::Params p{};
  p.q = c.q;
  p.k = c.k;
  p.v = c.v;
  p.kd = c.n_depth > 0 ? c.kd : nullptr;
  p.vd = c.n_depth > 0 ? c.vd : nullptr;
  p.out = c.out;
  p.lse = c.lse;
  p.Hq = c.Hq;
  p.Hkv = c.Hkv;
  p.G = c.Hq / c.Hkv;
  p.S_cap = c.S_cap;
  p.n_depth = c.n_depth;
  p.causal = c.causal;
  p.scale_log2 = c.scale * 1.4426950408889634f;
  p.phase = moda::kPhaseBoth;
  return p;
}

hipError_t launch_fwd_bf16(const moda::Params& p, int d, int gb, int waves, bool split, bool out_f32,
                           hipStream_t stream) {
  const int phase = p.phase;
  if (d == 64) {
    if (gb == 1) return moda::launch_fwd_bf16_dg<64, 1>(p, waves, split, phase, out_f32, stream);
    if (gb == 2) return moda::launch_fwd_bf16_dg<64, 2>(p, waves, split, phase, out_f32, stream);
    if (gb == 4) return moda::launch_fwd_bf16_dg<64, 4>(p, waves, split, phase, out_f32, stream);
  } else if (d == 128) {
    if (gb == 1) return moda::launch_fwd_bf16_dg<128, 1>(p, waves, split, phase, out_f32, stream);
    if (gb == 2) return moda::launch_fwd_bf16_dg<128, 2>(p, waves, split, phase, out_f32, stream);
    if (gb == 4) return moda::launch_fwd_bf16_dg<128, 4>(p, waves, split, phase, out_f32, stream);
  }
  return hipErrorInvalidValue;
}

// Fills the work decomposition and launches. max_len bounds every segment length.
int dispatch(moda::Params& p, const Common& c, int64_t n_seg, int64_t max_len, hipStream_t stream) {
  const int64_t kMaxTiles = 0x7fffffffLL;
  hipError_t err;
  if (c.dtype == MODA_DTYPE_BF16) {
    const int gb = heads_per_block(p.G);
    p.n_hgroups = p.G / gb;
    const int64_t n_pairs = n_seg * p.Hkv;
    // Waves per workgroup: the largest of 4, 2 that still gives every CU two
    // workgroups (fewer rows per workgroup for small problems).
    int waves = 1;
    for (int w = 4; w >= 2; w /= 2) {
      const int tok = moda::kWaveRows * w / gb;
      if (n_pairs * p.n_hgroups * ((max_len + tok - 1) / tok) >= 512) {
        waves = w;
        break;
      }
    }
    // Too few tiles for two waves per CU even with one-wave tiles: split tiles,
    // whose waves share a 32-row tile and divide its key blocks, ordered heaviest
    // first across all pairs.
    const bool split = waves == 1;
    if (split) waves = c.d == 64 ? moda::kSplitWaves<64> : moda::kSplitWaves<128>;  // both 2
    const int tok = split ? moda::kWaveRows / gb : moda::kWaveRows * waves / gb;
    const int64_t nqb = (max_len + tok - 1) / tok;
    p.n_qblocks = (int32_t)nqb;
    p.n_tiles = n_pairs * p.n_hgroups * nqb;
    p.xcd_interleave = split ? 0 : (p.n_hgroups == 1 && p.Hkv % 8 == 0) ? 2 : n_pairs % 8 == 0 ? 1 : 0;
    p.qb_major = split ? 1 : 0;
    if (nqb > kMaxTiles || p.n_tiles > kMaxTiles) return fail(MODA_ERR_SHAPE, "problem too large for one launch");
    err = launch_fwd_bf16(p, c.d, gb, waves, split, c.out_dtype == MODA_DTYPE_F32, stream);
  } else {
    const int64_t nqb = (max_len + moda::kF32BlockRows - 1) / moda::kF32BlockRows;
    p.n_hgroups = 1;
    p.n_qblocks = (int32_t)nqb;
    p.n_tiles = n_seg * p.Hq * nqb;
    if (nqb > kMaxTiles || p.n_tiles > kMaxTiles) return fail(MODA_ERR_SHAPE, "problem too large for one launch");
    err = moda::launch_fwd_f32(p, c.d, stream);
  }
  if (err != hipSuccess) return fail(MODA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
  g_err[0] = '\0';
  return MODA_OK;
}

// ---- decode ---------------------------------------------------------------------
// Workgroups the chunking aims for. Few heads per workgroup stream rows with
// little arithmetic each, and more, shorter chunks hide the tail (measured: MHA
// decode 4.5 -> 4.9 TB/s at 4096); with 4 or 8 heads a row the partial kernel
// is bound by its vector arithmetic and longer chunks amortise its set-up.
int64_t decode_target_blocks(int heads_per_block) { return heads_per_block <= 2 ? 4096 : 1024; }

// Query heads per decode workgroup: the largest of 8, 4, 2, 1 dividing G.
int decode_heads_per_block(int G) {
  for (int g = 8; g > 1; g /= 2)
    if (G % g == 0) return g;
  return 1;
}

// Cache rows per chunk: enough chunks for about decode_target_blocks
// workgroups, each a whole number of the partial kernel's load rounds. Shared by
// the call and the workspace-size query, so both see the same chunk count.
int64_t decode_chunk(int64_t batch, int Hq, int Hkv, int d, int64_t T_max) {
  const int64_t unit = moda::decode_rows_per_chunk_unit(d);
  const int gd = decode_heads_per_block(Hq / Hkv);
  const int64_t target = decode_target_blocks(gd);
  int64_t units = batch * Hkv * (int64_t)((Hq / Hkv) / gd);
  if (units < 1) units = 1;
  int64_t want = units >= target ? 1 : (target + units - 1) / units;
  int64_t chunk = (T_max + want - 1) / want;
  chunk = (chunk + unit - 1) / unit * unit;
  return chunk < unit ? unit : chunk;
}

// -1 when the workspace would not fit the size limit.
int64_t decode_workspace_bytes(int64_t batch, int Hq, int Hkv, int d, int64_t T_max) {
  if (!fits({batch, Hq, T_max, d + 4})) return -1;
  const int64_t chunk = decode_chunk(batch, Hq, Hkv, d, T_max);
  const int64_t n_chunks = (T_max + chunk - 1) / chunk + 1;
  if (!fits({batch, Hq, n_chunks, d + 4})) return -1;
  return batch * Hq * n_chunks * (int64_t)(d + 4) * 4;
}

// ---- backward --------------------------------------------------------------------
constexpr int kBwdMaxGroup = 16;  // query heads per KV head the backward supports

int64_t round256(int64_t x) { return (x + 255) / 256 * 256; }

int64_t bwd_workspace_bytes(int64_t N, int Hq, int d, int n_depth) {
  const int64_t delta = round256(4 * N * (int64_t)Hq);
  return delta + (n_depth > 0 ? round256(4 * N * (int64_t)Hq * d) : 0);
}

struct BwdArgs {
  const void *q, *k, *v, *kd, *vd, *out, *dout;
  const float* lse;
  void *dq, *dk, *dv, *dkd, *dvd;
  int32_t dtype, grad_dtype, Hq, Hkv, d, S_cap, n_depth, causal;
  float scale;
  void* workspace;
  int64_t workspace_bytes;
};

// Checks shared by both backward entry points; fills the fields of p they fix.
int check_bwd(const BwdArgs& a, int64_t N, moda::BwdParams& p) {
  const Common c{a.q,  a.k,   a.v,   a.kd,      a.vd,    a.dq,   nullptr, a.dtype, a.grad_dtype,
                 a.Hq, a.Hkv, a.d,   a.S_cap,   a.n_depth, a.causal, a.scale};
  const int rc = check_common(c);
  if (rc != MODA_OK) return rc;
  if (!a.out || !a.dout || !a.lse || !a.dk || !a.dv)
    return fail(MODA_ERR_NULL, "out, dout, lse, dq, dk and dv must be non-NULL");
  if (a.n_depth > 0 && (!a.dkd || !a.dvd))
    return fail(MODA_ERR_NULL, "dk_depth and dv_depth must be non-NULL when n_depth > 0");
  if (a.Hq / a.Hkv > kBwdMaxGroup)
    return fail(MODA_ERR_UNSUPPORTED, "backward supports up to %d query heads per KV head (got %d)", kBwdMaxGroup,
                a.Hq / a.Hkv);
  if (!aligned16(a.out) || !aligned16(a.dout) || !aligned16(a.dk) || !aligned16(a.dv))
    return fail(MODA_ERR_ALIGN, "out, dout, dq, dk and dv must be 16-byte aligned");
  if (a.n_depth > 0 && (!aligned16(a.dkd) || !aligned16(a.dvd)))
    return fail(MODA_ERR_ALIGN, "dk_depth and dv_depth must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(a.lse) & 3u) return fail(MODA_ERR_ALIGN, "lse must be 4-byte aligned");
  if (!fits({N, a.Hq, a.d}) || !fits({N, a.S_cap, a.Hkv, a.d}))
    return fail(MODA_ERR_SHAPE, "problem too large (a tensor of 2^56 elements or more)");
  if (!a.workspace) return fail(MODA_ERR_NULL, "workspace must be non-NULL");
  if (reinterpret_cast<uintptr_t>(a.workspace) & 255u) return fail(MODA_ERR_ALIGN, "workspace must be 256-byte aligned");
  const int64_t need = bwd_workspace_bytes(N, a.Hq, a.d, a.n_depth);
  if (a.workspace_bytes < need)
    return fail(MODA_ERR_SHAPE, "workspace too small: %lld bytes given, %lld needed", (long long)a.workspace_bytes,
                (long long)need);
  p = moda::BwdParams{};
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.kd = a.n_depth > 0 ? a.kd : nullptr;
  p.vd = a.n_depth > 0 ? a.vd : nullptr;
  p.out = a.out;
  p.dout = a.dout;
  p.lse = a.lse;
  p.dq = a.dq;
  p.dk = a.dk;
  p.dv = a.dv;
  p.dkd = a.n_depth > 0 ? a.dkd : nullptr;
  p.dvd = a.n_depth > 0 ? a.dvd : nullptr;
  unsigned char* ws = static_cast<unsigned char*>(a.workspace);
  p.delta = reinterpret_cast<float*>(ws);
  p.dq_depth = a.n_depth > 0 ? reinterpret_cast<float*>(ws + round256(4 * N * (int64_t)a.Hq)) : nullptr;
  p.total_tokens = N;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.G = a.Hq / a.Hkv;
  p.S_cap = a.S_cap;
  p.n_depth = a.n_depth;
  p.causal = a.causal;
  p.scale = a.scale;
  p.scale_log2 = a.scale * 1.4426950408889634f;
  return MODA_OK;
}

int launch_bwd_checked(moda::BwdParams& p, const BwdArgs& a, int64_t n_seg, int64_t max_len, hipStream_t stream) {
  const int64_t nb = (max_len + 127) / 128;
  p.n_qblocks = (int32_t)nb;
  p.n_kblocks = (int32_t)nb;
  // rows of the dq grid (segment, query head) and the dk/dv grid (segment, KV head)
  p.xcd_group = (n_seg * a.Hkv) % 8 == 0 ? 1 : 0;
  if (n_seg * a.Hq * nb > 0x7fffffffLL || p.total_tokens * a.Hq > 0x7fffffffLL * 4)
    return fail(MODA_ERR_SHAPE, "problem too large for one launch");
  const hipError_t err =
      moda::launch_bwd(p, a.d, a.dtype == MODA_DTYPE_BF16, a.grad_dtype == MODA_DTYPE_F32, stream);
  if (err != hipSuccess) return fail(MODA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
  g_err[0] = '\0';
  return MODA_OK;
}

// phase_mask: kPhaseBoth (the operator), kPhaseSeq or kPhaseDepth (one part's
// own softmax). Checked after the no-op cases, like every other argument.
int check_phase(int32_t phase, int32_t n_depth) {
  if (phase != moda::kPhaseSeq && phase != moda::kPhaseDepth && phase != moda::kPhaseBoth)
    return fail(MODA_ERR_VALUE, "phase_mask must be 1 (sequence), 2 (depth) or 3 (both), got %d", phase);
  if (phase == moda::kPhaseDepth && n_depth == 0)
    return fail(MODA_ERR_VALUE, "the depth phase alone needs n_depth > 0");
  return MODA_OK;
}

// Bounded depth reads (top-S / sliding window / hybrid): which slots of each row
// enter its softmax is decided by the selection kernel into the workspace.
struct Select {
  bool on;
  int32_t topk, recent;
  void* workspace;
  int64_t workspace_bytes;
};
constexpr Select kNoSelect{false, 0, 0, nullptr, 0};

int64_t select_workspace_bytes(int64_t N, int Hq) { return N * (int64_t)Hq * 8; }

// Host checks of a bounded read; on MODA_OK `p` reads only the kept slots: every
// slot (no launch), none (n_depth = 0) or a mask from the selection kernel,
// launched on `stream` before the forward.
int prepare_select(const Select& sel, const Common& c, moda::Params& p, int64_t N, hipStream_t stream) {
  if (!sel.on) return MODA_OK;
  if (sel.topk < 0 || sel.recent < 0) return fail(MODA_ERR_VALUE, "depth_topk and depth_recent must be >= 0");
  if (c.n_depth > moda::kMaxSelectSlots)
    return fail(MODA_ERR_UNSUPPORTED, "bounded depth reads support n_depth <= %d (got %d)", moda::kMaxSelectSlots,
                c.n_depth);
  const int64_t need = select_workspace_bytes(N, c.Hq);
  if (!sel.workspace) return fail(MODA_ERR_NULL, "workspace must be non-NULL");
  if (!aligned16(sel.workspace)) return fail(MODA_ERR_ALIGN, "workspace must be 16-byte aligned");
  if (sel.workspace_bytes < need)
    return fail(MODA_ERR_SHAPE, "workspace too small: %lld bytes given, %lld needed", (long long)sel.workspace_bytes,
                (long long)need);
  const int recent = sel.recent < c.n_depth ? sel.recent : c.n_depth;
  const int n_old = c.n_depth - recent;
  if (sel.topk >= n_old) return MODA_OK;  // every slot stays: the operator itself
  if (sel.topk == 0 && recent == 0) {     // no slot stays
    p.n_depth = 0;
    p.kd = p.vd = nullptr;
    return MODA_OK;
  }
  if (c.dtype == MODA_DTYPE_BF16) {  // selected inside the forward's depth pass
    p.sel_fused = 1;
    p.sel_topk = sel.topk;
    p.sel_recent = recent;
    return MODA_OK;
  }
  moda::SelectParams s{};  // fp32: a selection kernel writes one slot mask per row
  s.q = c.q;
  s.kd = c.kd;
  s.mask = static_cast<uint64_t*>(sel.workspace);
  s.n_tokens = N;
  s.Hq = c.Hq;
  s.Hkv = c.Hkv;
  s.G = c.Hq / c.Hkv;
  s.S_cap = c.S_cap;
  s.n_depth = c.n_depth;
  s.topk = sel.topk;
  s.recent = recent;
  s.scale = c.scale;
  const hipError_t err = moda::launch_depth_select(s, c.d, c.dtype == MODA_DTYPE_BF16, stream);
  if (err != hipSuccess) return fail(MODA_ERR_HIP, "selection kernel launch failed: %s", hipGetErrorString(err));
  p.depth_mask = s.mask;
  return MODA_OK;
}

int fwd_batch(const void* q, const void* k, const void* v, const void* k_depth, const void* v_depth, void* out,
              float* lse, int32_t dtype, int32_t out_dtype, int64_t batch, int64_t seqlen, int32_t n_heads_q,
              int32_t n_heads_kv, int32_t head_dim, int32_t depth_capacity, int32_t n_depth, int32_t causal,
              float scale, int32_t phase, void* stream, const Select& sel = kNoSelect) {
  if (batch < 0 || seqlen < 0) return fail(MODA_ERR_SHAPE, "batch and seqlen must be >= 0");
  const Common c{q,        k,          v,        k_depth,        v_depth, out,     lse,    dtype,
                 out_dtype, n_heads_q, n_heads_kv, head_dim, depth_capacity, n_depth, causal, scale};
  if (batch == 0 || seqlen == 0) {
    g_err[0] = '\0';
    return MODA_OK;
  }
  int rc = check_common(c);
  if (rc != MODA_OK) return rc;
  rc = check_phase(phase, n_depth);
  if (rc != MODA_OK) return rc;
  if (batch > 0x7fffffffLL) return fail(MODA_ERR_SHAPE, "batch too large");
  if (!fits({batch, seqlen, n_heads_q, head_dim}) || !fits({batch, seqlen, depth_capacity, n_heads_kv, head_dim}))
    return fail(MODA_ERR_SHAPE, "problem too large (a tensor of 2^56 elements or more)");
  moda::Params p = base_params(c);
  p.phase = phase;
  p.cu_seqlens = nullptr;
  p.uniform_len = seqlen;
  p.total_tokens = batch * seqlen;
  p.n_seg = (int32_t)batch;
  p.lse_head_stride = seqlen;
  p.lse_batch_layout = 1;
  rc = prepare_select(sel, c, p, batch * seqlen, static_cast<hipStream_t>(stream));
  if (rc != MODA_OK) return rc;
  return dispatch(p, c, batch, seqlen, static_cast<hipStream_t>(stream));
}

int fwd_varlen(const void* q, const void* k, const void* v, const void* k_depth, const void* v_depth, void* out,
               float* lse, int32_t dtype, int32_t out_dtype, const int32_t* cu_seqlens, int32_t n_seqs,
               int64_t total_tokens, int32_t max_seqlen, int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim,
               int32_t depth_capacity, int32_t n_depth, int32_t causal, float scale, int32_t phase, void* stream,
               const Select& sel = kNoSelect) {
  if (n_seqs < 0 || total_tokens < 0 || max_seqlen < 0)
    return fail(MODA_ERR_SHAPE, "n_seqs, total_tokens and max_seqlen must be >= 0");
  const Common c{q,        k,          v,        k_depth,        v_depth, out,     lse,    dtype,
                 out_dtype, n_heads_q, n_heads_kv, head_dim, depth_capacity, n_depth, causal, scale};
  if (n_seqs == 0 || total_tokens == 0 || max_seqlen == 0) {
    g_err[0] = '\0';
    return MODA_OK;
  }
  if (!cu_seqlens) return fail(MODA_ERR_NULL, "cu_seqlens must be non-NULL");
  if ((int64_t)max_seqlen > total_tokens) return fail(MODA_ERR_SHAPE, "max_seqlen exceeds total_tokens");
  int rc = check_common(c);
  if (rc != MODA_OK) return rc;
  rc = check_phase(phase, n_depth);
  if (rc != MODA_OK) return rc;
  if (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) return fail(MODA_ERR_ALIGN, "cu_seqlens must be 4-byte aligned");
  if (!fits({total_tokens, n_heads_q, head_dim}) || !fits({total_tokens, depth_capacity, n_heads_kv, head_dim}) ||
      !fits({n_seqs, n_heads_q, max_seqlen}))  // the tile grid: segments x heads x query blocks
    return fail(MODA_ERR_SHAPE, "problem too large (a tensor of 2^56 elements or more)");
  moda::Params p = base_params(c);
  p.phase = phase;
  p.cu_seqlens = cu_seqlens;
  p.uniform_len = 0;
  p.total_tokens = total_tokens;
  p.n_seg = n_seqs;
  p.lse_head_stride = total_tokens;
  p.lse_batch_layout = 0;
  rc = prepare_select(sel, c, p, total_tokens, static_cast<hipStream_t>(stream));
  if (rc != MODA_OK) return rc;
  return dispatch(p, c, n_seqs, max_seqlen, static_cast<hipStream_t>(stream));
}

}  // namespace

namespace moda {

int set_error(int code, const char* msg) { return fail(code, "%s", msg); }

int decode_prepare(const DecodeArgs& a, DecodePlan& plan) {
  if (a.batch < 0) return fail(MODA_ERR_SHAPE, "batch must be >= 0");
  const Common c{a.q,         a.k_cache,  a.v_cache,  a.k_depth,        a.v_depth, a.out,     a.lse,
                 a.dtype,     a.out_dtype, a.n_heads_q, a.n_heads_kv, a.head_dim, a.depth_capacity,
                 a.n_depth,   1,          a.scale};
  if (a.batch == 0) {
    g_err[0] = '\0';
    return kNothingToLaunch;
  }
  const int rc = check_common(c);
  if (rc != MODA_OK) return rc;
  if (a.max_cache_len < 1) return fail(MODA_ERR_SHAPE, "max_cache_len must be >= 1");
  if (!a.cache_seqlens) return fail(MODA_ERR_NULL, "cache_seqlens must be non-NULL");
  if (reinterpret_cast<uintptr_t>(a.cache_seqlens) & 3u)
    return fail(MODA_ERR_ALIGN, "cache_seqlens must be 4-byte aligned");
  if (a.batch > 0x7fffffffLL) return fail(MODA_ERR_SHAPE, "batch too large");
  if (!fits({a.batch, a.max_cache_len, a.n_heads_kv, a.head_dim}) ||
      !fits({a.batch, a.depth_capacity, a.n_heads_kv, a.head_dim}) ||
      decode_workspace_bytes(a.batch, a.n_heads_q, a.n_heads_kv, a.head_dim, a.max_cache_len) < 0)
    return fail(MODA_ERR_SHAPE, "problem too large (a tensor of 2^56 elements or more)");
  DecodeParams& p = plan.p;
  p = DecodeParams{};
  p.q = a.q;
  p.kc = a.k_cache;
  p.vc = a.v_cache;
  p.kd = a.n_depth > 0 ? a.k_depth : nullptr;
  p.vd = a.n_depth > 0 ? a.v_depth : nullptr;
  p.out = a.out;
  p.lse = a.lse;
  p.cache_seqlens = a.cache_seqlens;
  p.workspace = nullptr;
  p.B = a.batch;
  p.T_max = a.max_cache_len;
  p.Hq = a.n_heads_q;
  p.Hkv = a.n_heads_kv;
  p.G = a.n_heads_q / a.n_heads_kv;
  plan.heads_per_block = decode_heads_per_block(p.G);
  p.n_hgroups = p.G / plan.heads_per_block;
  p.S_cap = a.depth_capacity;
  p.n_depth = a.n_depth;
  p.scale_log2 = a.scale * 1.4426950408889634f;
  p.chunk = decode_chunk(a.batch, a.n_heads_q, a.n_heads_kv, a.head_dim, a.max_cache_len);
  p.n_seq_chunks = (int32_t)((a.max_cache_len + p.chunk - 1) / p.chunk);
  p.n_chunks = p.n_seq_chunks + 1;
  p.n_partial_blocks = a.batch * a.n_heads_kv * p.n_hgroups * p.n_chunks;
  if (p.n_partial_blocks > 0x7fffffffLL || a.batch * a.n_heads_q > 0x7fffffffLL)
    return fail(MODA_ERR_SHAPE, "problem too large for one launch");
  plan.head_dim = a.head_dim;
  plan.bf16 = a.dtype == MODA_DTYPE_BF16;
  plan.out_f32 = a.out_dtype == MODA_DTYPE_F32;
  plan.workspace_bytes = decode_workspace_bytes(a.batch, a.n_heads_q, a.n_heads_kv, a.head_dim, a.max_cache_len);
  return MODA_OK;
}

int decode_launch(DecodePlan& plan, void* workspace, hipStream_t stream) {
  plan.p.workspace = static_cast<float*>(workspace);
  const hipError_t err = launch_decode(plan.p, plan.head_dim, plan.heads_per_block, plan.bf16, plan.out_f32, stream);
  if (err != hipSuccess) return fail(MODA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
  g_err[0] = '\0';
  return MODA_OK;
}

}  // namespace moda

extern "C" {

int moda_attn_fwd(const void* q, const void* k, const void* v, const void* k_depth, const void* v_depth, void* out,
                  float* lse, int32_t dtype, int32_t out_dtype, int64_t batch, int64_t seqlen, int32_t n_heads_q, int32_t n_heads_kv,
                  int32_t head_dim, int32_t depth_capacity, int32_t n_depth, int32_t causal, float scale,
                  void* stream) {
  return fwd_batch(q, k, v, k_depth, v_depth, out, lse, dtype, out_dtype, batch, seqlen, n_heads_q, n_heads_kv,
                   head_dim, depth_capacity, n_depth, causal, scale, moda::kPhaseBoth, stream);
}

int moda_attn_fwd_varlen(const void* q, const void* k, const void* v, const void* k_depth, const void* v_depth,
                         void* out, float* lse, int32_t dtype, int32_t out_dtype, const int32_t* cu_seqlens, int32_t n_seqs,
                         int64_t total_tokens, int32_t max_seqlen, int32_t n_heads_q, int32_t n_heads_kv,
                         int32_t head_dim, int32_t depth_capacity, int32_t n_depth, int32_t causal, float scale,
                         void* stream) {
  return fwd_varlen(q, k, v, k_depth, v_depth, out, lse, dtype, out_dtype, cu_seqlens, n_seqs, total_tokens,
                    max_seqlen, n_heads_q, n_heads_kv, head_dim, depth_capacity, n_depth, causal, scale,
                    moda::kPhaseBoth, stream);
}

int moda_attn_fwd_phases(const void* q, const void* k, const void* v, const void* k_depth, const void* v_depth,
                         void* out, float* lse, int32_t dtype, int32_t out_dtype, int64_t batch, int64_t seqlen,
                         int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim, int32_t depth_capacity,
                         int32_t n_depth, int32_t causal, float scale, int32_t phase_mask, void* stream) {
  return fwd_batch(q, k, v, k_depth, v_depth, out, lse, dtype, out_dtype, batch, seqlen, n_heads_q, n_heads_kv,
                   head_dim, depth_capacity, n_depth, causal, scale, phase_mask, stream);
}

int moda_attn_fwd_varlen_phases(const void* q, const void* k, const void* v, const void* k_depth,
                                const void* v_depth, void* out, float* lse, int32_t dtype, int32_t out_dtype,
                                const int32_t* cu_seqlens, int32_t n_seqs, int64_t total_tokens, int32_t max_seqlen,
                                int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim, int32_t depth_capacity,
                                int32_t n_depth, int32_t causal, float scale, int32_t phase_mask, void* stream) {
  return fwd_varlen(q, k, v, k_depth, v_depth, out, lse, dtype, out_dtype, cu_seqlens, n_seqs, total_tokens,
                    max_seqlen, n_heads_q, n_heads_kv, head_dim, depth_capacity, n_depth, causal, scale, phase_mask,
                    stream);
}

int moda_attn_fwd_topk(const void* q, const void* k, const void* v, const void* k_depth, const void* v_depth,
                       void* out, float* lse, int32_t dtype, int32_t out_dtype, int64_t batch, int64_t seqlen,
                       int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim, int32_t depth_capacity,
                       int32_t n_depth, int32_t depth_topk, int32_t depth_recent, int32_t causal, float scale,
                       void* workspace, int64_t workspace_bytes, void* stream) {
  const Select sel{true, depth_topk, depth_recent, workspace, workspace_bytes};
  return fwd_batch(q, k, v, k_depth, v_depth, out, lse, dtype, out_dtype, batch, seqlen, n_heads_q, n_heads_kv,
                   head_dim, depth_capacity, n_depth, causal, scale, moda::kPhaseBoth, stream, sel);
}

int moda_attn_fwd_varlen_topk(const void* q, const void* k, const void* v, const void* k_depth, const void* v_depth,
                              void* out, float* lse, int32_t dtype, int32_t out_dtype, const int32_t* cu_seqlens,
                              int32_t n_seqs, int64_t total_tokens, int32_t max_seqlen, int32_t n_heads_q,
                              int32_t n_heads_kv, int32_t head_dim, int32_t depth_capacity, int32_t n_depth,
                              int32_t depth_topk, int32_t depth_recent, int32_t causal, float scale, void* workspace,
                              int64_t workspace_bytes, void* stream) {
  const Select sel{true, depth_topk, depth_recent, workspace, workspace_bytes};
  return fwd_varlen(q, k, v, k_depth, v_depth, out, lse, dtype, out_dtype, cu_seqlens, n_seqs, total_tokens,
                    max_seqlen, n_heads_q, n_heads_kv, head_dim, depth_capacity, n_depth, causal, scale,
                    moda::kPhaseBoth, stream, sel);
}

int64_t moda_attn_fwd_topk_workspace_size(int64_t total_tokens, int32_t n_heads_q) {
  if (total_tokens < 0 || n_heads_q < 1 || !fits({total_tokens, n_heads_q})) return -1;
  return select_workspace_bytes(total_tokens, n_heads_q);
}

int64_t moda_attn_decode_workspace_size(int64_t batch, int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim,
                                        int32_t max_cache_len) {
  if (batch < 0 || n_heads_q < 1 || n_heads_kv < 1 || n_heads_q % n_heads_kv != 0 || max_cache_len < 1 ||
      (head_dim != 64 && head_dim != 128))
    return -1;
  return decode_workspace_bytes(batch, n_heads_q, n_heads_kv, head_dim, max_cache_len);
}

int moda_attn_decode(const void* q, const void* k_cache, const void* v_cache, const void* k_depth,
                     const void* v_depth, void* out, float* lse, int32_t dtype, int32_t out_dtype,
                     const int32_t* cache_seqlens, int64_t batch, int32_t max_cache_len, int32_t n_heads_q,
                     int32_t n_heads_kv, int32_t head_dim, int32_t depth_capacity, int32_t n_depth, float scale,
                     void* workspace, int64_t workspace_bytes, void* stream) {
  const moda::DecodeArgs a{q,          k_cache,  v_cache,   k_depth,        v_depth, out,   lse,
                           dtype,      out_dtype, cache_seqlens, batch,     max_cache_len, n_heads_q, n_heads_kv,
                           head_dim,   depth_capacity, n_depth, scale};
  moda::DecodePlan plan;
  int rc = moda::decode_prepare(a, plan);
  if (rc == moda::kNothingToLaunch) return MODA_OK;
  if (rc != MODA_OK) return rc;
  if (!workspace) return fail(MODA_ERR_NULL, "workspace must be non-NULL");
  if (!aligned16(workspace)) return fail(MODA_ERR_ALIGN, "workspace must be 16-byte aligned");
  if (workspace_bytes < plan.workspace_bytes)
    return fail(MODA_ERR_SHAPE, "workspace too small: %lld bytes given, %lld needed", (long long)workspace_bytes,
                (long long)plan.workspace_bytes);
  return moda::decode_launch(plan, workspace, static_cast<hipStream_t>(stream));
}

int64_t moda_attn_bwd_workspace_size(int64_t total_tokens, int32_t n_heads_q, int32_t head_dim, int32_t n_depth) {
  if (total_tokens < 0 || n_heads_q < 1 || n_depth < 0 || (head_dim != 64 && head_dim != 128)) return -1;
  if (!fits({total_tokens, n_heads_q, head_dim})) return -1;
  return bwd_workspace_bytes(total_tokens, n_heads_q, head_dim, n_depth);
}

int moda_attn_bwd(const void* q, const void* k, const void* v, const void* k_depth, const void* v_depth,
                  const void* out, const void* dout, const float* lse, void* dq, void* dk, void* dv,
                  void* dk_depth, void* dv_depth, int32_t dtype, int32_t grad_dtype, int64_t batch, int64_t seqlen,
                  int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim, int32_t depth_capacity, int32_t n_depth,
                  int32_t causal, float scale, void* workspace, int64_t workspace_bytes, void* stream) {
  if (batch < 0 || seqlen < 0) return fail(MODA_ERR_SHAPE, "batch and seqlen must be >= 0");
  if (batch == 0 || seqlen == 0) {
    g_err[0] = '\0';
    return MODA_OK;
  }
  if (batch > 0x7fffffffLL) return fail(MODA_ERR_SHAPE, "batch too large");
  if (!fits({batch, seqlen})) return fail(MODA_ERR_SHAPE, "problem too large (a tensor of 2^56 elements or more)");
  const BwdArgs a{q,  k,  v,  k_depth, v_depth,    out,       dout,       lse,          dq,
                  dk, dv, dk_depth, dv_depth, dtype, grad_dtype, n_heads_q, n_heads_kv, head_dim,
                  depth_capacity, n_depth, causal, scale, workspace, workspace_bytes};
  moda::BwdParams p;
  const int rc = check_bwd(a, batch * seqlen, p);
  if (rc != MODA_OK) return rc;
  p.cu_seqlens = nullptr;
  p.uniform_len = seqlen;
  p.n_seg = (int32_t)batch;
  p.lse_head_stride = seqlen;
  p.lse_batch_layout = 1;
  return launch_bwd_checked(p, a, batch, seqlen, static_cast<hipStream_t>(stream));
}

int moda_attn_bwd_varlen(const void* q, const void* k, const void* v, const void* k_depth, const void* v_depth,
                         const void* out, const void* dout, const float* lse, void* dq, void* dk, void* dv,
                         void* dk_depth, void* dv_depth, int32_t dtype, int32_t grad_dtype,
                         const int32_t* cu_seqlens, int32_t n_seqs, int64_t total_tokens, int32_t max_seqlen,
                         int32_t n_heads_q, int32_t n_heads_kv, int32_t head_dim, int32_t depth_capacity,
                         int32_t n_depth, int32_t causal, float scale, void* workspace, int64_t workspace_bytes,
                         void* stream) {
  if (n_seqs < 0 || total_tokens < 0 || max_seqlen < 0)
    return fail(MODA_ERR_SHAPE, "n_seqs, total_tokens and max_seqlen must be >= 0");
  if (n_seqs == 0 || total_tokens == 0 || max_seqlen == 0) {
    g_err[0] = '\0';
    return MODA_OK;
  }
  if (!cu_seqlens) return fail(MODA_ERR_NULL, "cu_seqlens must be non-NULL");
  if ((int64_t)max_seqlen > total_tokens) return fail(MODA_ERR_SHAPE, "max_seqlen exceeds total_tokens");
  const BwdArgs a{q,  k,  v,  k_depth, v_depth,    out,       dout,       lse,          dq,
                  dk, dv, dk_depth, dv_depth, dtype, grad_dtype, n_heads_q, n_heads_kv, head_dim,
                  depth_capacity, n_depth, causal, scale, workspace, workspace_bytes};
  if (!fits({n_seqs, n_heads_q, max_seqlen}))  // the grids: segments x heads x blocks
    return fail(MODA_ERR_SHAPE, "problem too large (a tensor of 2^56 elements or more)");
  moda::BwdParams p;
  const int rc = check_bwd(a, total_tokens, p);
  if (rc != MODA_OK) return rc;
  if (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) return fail(MODA_ERR_ALIGN, "cu_seqlens must be 4-byte aligned");
  p.cu_seqlens = cu_seqlens;
  p.uniform_len = 0;
  p.n_seg = n_seqs;
  p.lse_head_stride = total_tokens;
  p.lse_batch_layout = 0;
  return launch_bwd_checked(p, a, n_seqs, max_seqlen, static_cast<hipStream_t>(stream));
}

int moda_depth_kv_write(const void* k_src, const void* v_src, void* k_depth, void* v_depth, int32_t dtype,
                        int64_t n_tokens, int32_t n_heads_kv, int32_t head_dim, int32_t depth_capacity, int32_t slot,
                        void* stream) {
  if (n_tokens < 0) return fail(MODA_ERR_SHAPE, "n_tokens must be >= 0");
  if (n_tokens == 0) {
    g_err[0] = '\0';
    return MODA_OK;
  }
  if (!k_src || !v_src || !k_depth || !v_depth) return fail(MODA_ERR_NULL, "all four tensors must be non-NULL");
  if (dtype != MODA_DTYPE_F32 && dtype != MODA_DTYPE_BF16) return fail(MODA_ERR_DTYPE, "unknown dtype code %d", dtype);
  if (n_heads_kv < 1 || head_dim < 1) return fail(MODA_ERR_SHAPE, "n_heads_kv and head_dim must be >= 1");
  if (depth_capacity < 1 || slot < 0 || slot >= depth_capacity)
    return fail(MODA_ERR_SHAPE, "need 0 <= slot (%d) < depth_capacity (%d)", slot, depth_capacity);
  if (!fits({n_tokens, depth_capacity, n_heads_kv, head_dim}))
    return fail(MODA_ERR_SHAPE, "problem too large (a tensor of 2^56 elements or more)");
  const int64_t row_bytes = (int64_t)n_heads_kv * head_dim * (dtype == MODA_DTYPE_BF16 ? 2 : 4);
  if (row_bytes % 16) return fail(MODA_ERR_SHAPE, "n_heads_kv * head_dim * element bytes must be a multiple of 16");
  if (!aligned16(k_src) || !aligned16(v_src) || !aligned16(k_depth) || !aligned16(v_depth))
    return fail(MODA_ERR_ALIGN, "all four tensors must be 16-byte aligned");
  moda::DepthWriteParams p{k_src, v_src, k_depth, v_depth, n_tokens, row_bytes / 16, depth_capacity, slot};
  const hipError_t err = moda::launch_depth_kv_write(p, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(MODA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
  g_err[0] = '\0';
  return MODA_OK;
}

int moda_depth_kv_project(const void* x, const void* w_kv, void* k_depth, void* v_depth, int32_t dtype,
                          int64_t n_tokens, int32_t d_model, int32_t n_heads_kv, int32_t head_dim,
                          int32_t depth_capacity, int32_t slot, void* stream) {
  if (n_tokens < 0) return fail(MODA_ERR_SHAPE, "n_tokens must be >= 0");
  if (n_tokens == 0) {
    g_err[0] = '\0';
    return MODA_OK;
  }
  if (!x || !w_kv || !k_depth || !v_depth) return fail(MODA_ERR_NULL, "x, w_kv, k_depth and v_depth must be non-NULL");
  if (dtype != MODA_DTYPE_F32 && dtype != MODA_DTYPE_BF16) return fail(MODA_ERR_DTYPE, "unknown dtype code %d", dtype);
  if (n_heads_kv < 1) return fail(MODA_ERR_SHAPE, "n_heads_kv must be >= 1");
  if (head_dim != 64 && head_dim != 128) return fail(MODA_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", head_dim);
  if (d_model < 64 || d_model % 64 != 0)
    return fail(MODA_ERR_UNSUPPORTED, "d_model must be a positive multiple of 64 (got %d)", d_model);
  if (depth_capacity < 1 || slot < 0 || slot >= depth_capacity)
    return fail(MODA_ERR_SHAPE, "need 0 <= slot (%d) < depth_capacity (%d)", slot, depth_capacity);
  if (!aligned16(x) || !aligned16(w_kv) || !aligned16(k_depth) || !aligned16(v_depth))
    return fail(MODA_ERR_ALIGN, "x, w_kv, k_depth and v_depth must be 16-byte aligned");
  if ((int64_t)n_heads_kv * head_dim > 0x3fffffffLL) return fail(MODA_ERR_SHAPE, "n_heads_kv * head_dim too large");
  if (!fits({n_tokens, d_model}) || !fits({n_tokens, depth_capacity, n_heads_kv, head_dim}) ||
      !fits({2, n_heads_kv, head_dim, d_model}))
    return fail(MODA_ERR_SHAPE, "problem too large (a tensor of 2^56 elements or more)");
  moda::ProjParams p{};
  p.x = x;
  p.w = w_kv;
  p.kd = k_depth;
  p.vd = v_depth;
  p.n_tokens = n_tokens;
  p.d_model = d_model;
  p.hd = n_heads_kv * head_dim;
  p.S_cap = depth_capacity;
  p.slot = slot;
  const int64_t tiles = (int64_t)(2 * p.hd / 64) * ((n_tokens + 63) / 64);
  if (tiles > 0x7fffffffLL) return fail(MODA_ERR_SHAPE, "problem too large for one launch");
  const hipError_t err = moda::launch_depth_kv_project(p, dtype == MODA_DTYPE_BF16, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(MODA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
  g_err[0] = '\0';
  return MODA_OK;
}

const char* moda_last_error(void) { return g_err; }

int32_t moda_abi_version(void) { return MODA_ABI_VERSION; }

}  // extern "C"

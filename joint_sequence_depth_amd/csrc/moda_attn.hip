// Host side of the C ABI: argument checks, work decomposition, kernel dispatch.
// Every check runs before any HIP call, so a rejected call touches no device state.
#include "moda_attn.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>

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
  return p;
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
    p.xcd_interleave = (!split && n_pairs % 8 == 0) ? 1 : 0;
    p.qb_major = split ? 1 : 0;
#ifdef MODA_FORCE_SERIAL_ORDER
    p.serial_order = MODA_FORCE_SERIAL_ORDER;
#else
    p.serial_order = 0;
#endif
    if (nqb > kMaxTiles || p.n_tiles > kMaxTiles) return fail(MODA_ERR_SHAPE, "problem too large for one launch");
    err = moda::launch_fwd_bf16(p, c.d, gb, waves, split, c.out_dtype == MODA_DTYPE_F32, stream);
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

}  // namespace

extern "C" {

int moda_attn_fwd(const void* q, const void* k, const void* v, const void* k_depth, const void* v_depth, void* out,
                  float* lse, int32_t dtype, int32_t out_dtype, int64_t batch, int64_t seqlen, int32_t n_heads_q, int32_t n_heads_kv,
                  int32_t head_dim, int32_t depth_capacity, int32_t n_depth, int32_t causal, float scale,
                  void* stream) {
  if (batch < 0 || seqlen < 0) return fail(MODA_ERR_SHAPE, "batch and seqlen must be >= 0");
  const Common c{q,        k,          v,        k_depth,        v_depth, out,     lse,    dtype,
                 out_dtype, n_heads_q, n_heads_kv, head_dim, depth_capacity, n_depth, causal, scale};
  if (batch == 0 || seqlen == 0) {
    g_err[0] = '\0';
    return MODA_OK;
  }
  const int rc = check_common(c);
  if (rc != MODA_OK) return rc;
  if (batch > 0x7fffffffLL) return fail(MODA_ERR_SHAPE, "batch too large");
  moda::Params p = base_params(c);
  p.cu_seqlens = nullptr;
  p.uniform_len = seqlen;
  p.total_tokens = batch * seqlen;
  p.n_seg = (int32_t)batch;
  p.lse_head_stride = seqlen;
  p.lse_batch_layout = 1;
  return dispatch(p, c, batch, seqlen, static_cast<hipStream_t>(stream));
}

int moda_attn_fwd_varlen(const void* q, const void* k, const void* v, const void* k_depth, const void* v_depth,
                         void* out, float* lse, int32_t dtype, int32_t out_dtype, const int32_t* cu_seqlens, int32_t n_seqs,
                         int64_t total_tokens, int32_t max_seqlen, int32_t n_heads_q, int32_t n_heads_kv,
                         int32_t head_dim, int32_t depth_capacity, int32_t n_depth, int32_t causal, float scale,
                         void* stream) {
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
  const int rc = check_common(c);
  if (rc != MODA_OK) return rc;
  if (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) return fail(MODA_ERR_ALIGN, "cu_seqlens must be 4-byte aligned");
  moda::Params p = base_params(c);
  p.cu_seqlens = cu_seqlens;
  p.uniform_len = 0;
  p.total_tokens = total_tokens;
  p.n_seg = n_seqs;
  p.lse_head_stride = total_tokens;
  p.lse_batch_layout = 0;
  return dispatch(p, c, n_seqs, max_seqlen, static_cast<hipStream_t>(stream));
}

const char* moda_last_error(void) { return g_err; }

int32_t moda_abi_version(void) { return MODA_ABI_VERSION; }

}  // extern "C"

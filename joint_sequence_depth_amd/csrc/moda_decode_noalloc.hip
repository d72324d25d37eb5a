// Allocation-free decode step, for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid it).
//
// moda_attn_decode passes the fp32 partial states of its key chunks from the
// partial kernel to the merge kernel through a caller-owned workspace. This
// variant uses a fixed device array of the library instead: `scratch` below,
// kScratchBytes per GPU, held from the first call on a GPU until the process
// ends. Its address is looked up once per device (hipGetSymbolAddress, with that
// device current) and kept; the kernels take it as their workspace argument.
// The merge kernel reads only chunk states the partial kernel wrote in the same
// call, so nothing in the array needs clearing between calls. Calls that overlap
// on one GPU (two streams, or two threads) share the array and race.
#include <stdio.h>

#include <mutex>

#include "moda_attn.h"
#include "moda_internal.h"

namespace {

constexpr int64_t kScratchBytes = 16ll << 20;  // MODA_DECODE_SCRATCH_BYTES
static_assert(kScratchBytes == MODA_DECODE_SCRATCH_BYTES, "header and library agree on the scratch size");
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch array's device address on the current device (looked up on the
// first call there). `stream` must belong to that device.
int scratch_of_current_device(hipStream_t stream, void** ptr) {
  char msg[256];
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    snprintf(msg, sizeof(msg), "hipGetDevice failed: %s", hipGetErrorString(e));
    return moda::set_error(MODA_ERR_HIP, msg);
  }
  if (dev < 0 || dev >= kMaxDevices) return moda::set_error(MODA_ERR_UNSUPPORTED, "device ordinal out of range");
  if (stream) {
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) {
      snprintf(msg, sizeof(msg), "hipStreamGetDevice failed: %s", hipGetErrorString(e));
      return moda::set_error(MODA_ERR_HIP, msg);
    }
    if (sdev != dev) {
      snprintf(msg, sizeof(msg), "stream belongs to device %d but device %d is current", (int)sdev, dev);
      return moda::set_error(MODA_ERR_VALUE, msg);
    }
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      snprintf(msg, sizeof(msg), "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
      return moda::set_error(MODA_ERR_HIP, msg);
    }
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MODA_OK;
}

}  // namespace

extern "C" int moda_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                        const void* k_depth, const void* v_depth, void* out, float* lse,
                                        int32_t dtype, int32_t out_dtype, const int32_t* cache_seqlens,
                                        int64_t batch, int32_t max_cache_len, int32_t n_heads_q, int32_t n_heads_kv,
                                        int32_t head_dim, int32_t depth_capacity, int32_t n_depth, float scale,
                                        void* stream) {
  const moda::DecodeArgs a{q,        k_cache,   v_cache,       k_depth, v_depth,       out,       lse,
                           dtype,    out_dtype, cache_seqlens, batch,   max_cache_len, n_heads_q, n_heads_kv,
                           head_dim, depth_capacity, n_depth, scale};
  moda::DecodePlan plan;
  int rc = moda::decode_prepare(a, plan);
  if (rc == moda::kNothingToLaunch) return MODA_OK;
  if (rc != MODA_OK) return rc;
  if (plan.workspace_bytes > kScratchBytes) {
    char msg[256];
    snprintf(msg, sizeof(msg),
             "decode step needs %lld bytes of scratch, the allocation-free call holds %lld: use moda_attn_decode "
             "with a workspace",
             (long long)plan.workspace_bytes, (long long)kScratchBytes);
    return moda::set_error(MODA_ERR_SHAPE, msg);
  }
  void* ws = nullptr;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  rc = scratch_of_current_device(s, &ws);
  if (rc != MODA_OK) return rc;
  return moda::decode_launch(plan, ws, s);
}

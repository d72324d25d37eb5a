// Depth-KV writer: stores one layer's key/value rows of every token into one slot
// of the depth cache that later layers read (MoDA deck, slide "Reuse attention
// KV; add a projection for FFN inputs": the attention KV of a layer is kept for
// later layers, and the FFN input adds further slots). A bounded slot buffer
// (the paper's future work, as the deck quotes it on slide "The main open cost is
// retaining and reading depth history") uses the slot axis as a ring: the w-th entry written goes to slot w mod S_cap, and since the joint
// softmax does not depend on the order of its keys, reading all valid slots is a
// sliding window over the most recent S_cap entries.
//
// Per token the source row (H_kv d elements) and the destination slot row are
// both contiguous, so the copy is a stream of 16-byte vectors: thread i moves
// vector i of the flattened [N, H_kv d] source into the slot row of its token,
// stored with the non-temporal hint.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moda_internal.h"
#include "moda_rowops.h"

namespace moda {
namespace {

constexpr int kWriterThreads = 256;

__global__ __launch_bounds__(kWriterThreads) void moda_depth_kv_write_kernel(const DepthWriteParams p) {
  const int64_t n_vec = p.n_tokens * p.row_vecs;  // 16-byte vectors per source tensor
  const int64_t stride = (int64_t)gridDim.x * kWriterThreads;
  for (int64_t i = (int64_t)blockIdx.x * kWriterThreads + threadIdx.x; i < n_vec; i += stride) {
    const int64_t n = i / p.row_vecs, c = i - n * p.row_vecs;
    const int64_t dst = (n * p.S_cap + p.slot) * p.row_vecs + c;
    const uint4 kv = reinterpret_cast<const uint4*>(p.k_src)[i];
    const uint4 vv = reinterpret_cast<const uint4*>(p.v_src)[i];
    // streaming stores: a later layer reads the slot, not this kernel (16384 tokens
    // x 16 KV heads x 128: 43.1 -> 39.5 us)
    rowops::stream_store16(reinterpret_cast<uint4*>(p.k_depth) + dst, kv.x, kv.y, kv.z, kv.w);
    rowops::stream_store16(reinterpret_cast<uint4*>(p.v_depth) + dst, vv.x, vv.y, vv.z, vv.w);
  }
}

}  // namespace

hipError_t launch_depth_kv_write(const DepthWriteParams& p, hipStream_t stream) {
  const int64_t n_vec = p.n_tokens * p.row_vecs;
  int64_t blocks = (n_vec + kWriterThreads - 1) / kWriterThreads;
  const int64_t cap = 256 * 64;  // 64 workgroups per CU, then grid-stride
  blocks = blocks < cap ? blocks : cap;
  hipLaunchKernelGGL(moda_depth_kv_write_kernel, dim3((unsigned)blocks), dim3(kWriterThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace moda

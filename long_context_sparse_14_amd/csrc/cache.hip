// Cache append: the indexer key cache and the latent cache grow by one token
// per sequence and step.  (DeepSeek-V3.2 model documentation, section
// "DeepSeek Sparse Attention (DSA)": the indexer keeps its own per-token,
// single-head key cache next to the main key/value cache and updates it as
// tokens arrive.)  Static-cache layout: [B, N, width], the new token of
// sequence b goes to row pos[b].
#include "device_common.h"
#include "launch.h"

namespace dsa {
namespace {

// One workgroup per sequence: copies the new indexer key row and the new
// latent row into place, in 2-byte units (every supported row is a whole
// number of them).
__global__ __launch_bounds__(256) void cache_append_kernel(uint16_t* __restrict__ k_idx, uint16_t* __restrict__ kv,
                                                           const uint16_t* __restrict__ new_k_idx,
                                                           const uint16_t* __restrict__ new_kv,
                                                           const int64_t* __restrict__ pos, int64_t N, int64_t wk,
                                                           int64_t wv) {
  const int64_t b = blockIdx.x;
  const int64_t p = pos[b];
  if (p < 0 || p >= N) return;
  if (k_idx != nullptr)
    for (int64_t i = threadIdx.x; i < wk; i += blockDim.x) k_idx[(b * N + p) * wk + i] = new_k_idx[b * wk + i];
  if (kv != nullptr)
    for (int64_t i = threadIdx.x; i < wv; i += blockDim.x) kv[(b * N + p) * wv + i] = new_kv[b * wv + i];
}

}  // namespace

hipError_t launch_cache_append(void* k_idx, void* kv, const void* new_k_idx, const void* new_kv, const int64_t* pos,
                               int64_t B, int64_t N, int D_I, int D, int esize, hipStream_t stream) {
  const int64_t halves = esize / 2;  // 2-byte units per element
  hipLaunchKernelGGL(cache_append_kernel, dim3((unsigned)B), dim3(256), 0, stream, static_cast<uint16_t*>(k_idx),
                     static_cast<uint16_t*>(kv), static_cast<const uint16_t*>(new_k_idx),
                     static_cast<const uint16_t*>(new_kv), pos, N, (int64_t)D_I * halves, (int64_t)D * halves);
  return hipGetLastError();
}

}  // namespace dsa

// Cache append: the indexer key cache and the latent cache grow by one token
// per sequence and step.  (DeepSeek-V3.2 model documentation, section
// "DeepSeek Sparse Attention (DSA)": the indexer keeps its own per-token,
// single-head key cache next to the main key/value cache and updates it as
// tokens arrive.)  Static-cache layout: [B, N, width], the new token of
// sequence b goes to row pos[b].  Paged layout: a pool of blocks of rows with
// one block table per sequence; the new token goes to the pool row that
// holds logical row pos[b].  The paged steps read the top-k's logical
// indices through the same tables (page_translate_kernel).
#include "device_common.h"
#include "launch.h"

namespace dsa {
namespace {

// Pool row of logical row r of sequence b, or -1 when the sequence's table
// entry for that block lies outside [0, num_blocks) (an unset block).
__device__ __forceinline__ int64_t paged_row(const Paged& pg, int64_t b, int64_t r) {
  const int32_t e = pg.table[b * pg.max_blocks + (r >> pg.shift)];
  if ((uint32_t)e >= (uint32_t)pg.num_blocks) return -1;
  return ((int64_t)e << pg.shift) | (r & ((1 << pg.shift) - 1));
}

// One workgroup per sequence: copies the new indexer key row and the new
// latent row into place, in 2-byte units (every supported row is a whole
// number of them).  With PAGED, N is the logical capacity max_blocks << shift
// and the caches are pools; a row whose block is unset is not written.
template <bool PAGED>
__global__ __launch_bounds__(256) void cache_append_kernel(uint16_t* __restrict__ k_idx, uint16_t* __restrict__ kv,
                                                           const uint16_t* __restrict__ new_k_idx,
                                                           const uint16_t* __restrict__ new_kv,
                                                           const int64_t* __restrict__ pos, int64_t N, int64_t wk,
                                                           int64_t wv, Paged pg) {
  const int64_t b = blockIdx.x;
  const int64_t p = pos[b];
  if (p < 0 || p >= N) return;
  const int64_t row = PAGED ? paged_row(pg, b, p) : b * N + p;
  if (row < 0) return;
  if (k_idx != nullptr)
    for (int64_t i = threadIdx.x; i < wk; i += blockDim.x) k_idx[row * wk + i] = new_k_idx[b * wk + i];
  if (kv != nullptr)
    for (int64_t i = threadIdx.x; i < wv; i += blockDim.x) kv[row * wv + i] = new_kv[b * wv + i];
}

// Logical key indices [R, K] (rows of Tq per sequence) -> pool rows; entries
// outside [0, max_blocks << shift), and those whose block is unset, become -1
// (masked by the sparse MLA).
__global__ __launch_bounds__(256) void page_translate_kernel(const int32_t* __restrict__ idx, int32_t* __restrict__ out,
                                                             int64_t total, int64_t Tq, int K, Paged pg) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int64_t b = (i / K) / Tq;
  const int32_t v = idx[i];
  out[i] = (v >= 0 && (int64_t)v < (pg.max_blocks << pg.shift)) ? (int32_t)paged_row(pg, b, v) : -1;
}

}  // namespace

hipError_t launch_cache_append(void* k_idx, void* kv, const void* new_k_idx, const void* new_kv, const int64_t* pos,
                               int64_t B, int64_t N, int D_I, int D, int esize, hipStream_t stream, const Paged* pg) {
  const int64_t halves = esize / 2;  // 2-byte units per element
  if (pg != nullptr)
    hipLaunchKernelGGL(cache_append_kernel<true>, dim3((unsigned)B), dim3(256), 0, stream,
                       static_cast<uint16_t*>(k_idx), static_cast<uint16_t*>(kv),
                       static_cast<const uint16_t*>(new_k_idx), static_cast<const uint16_t*>(new_kv), pos,
                       pg->max_blocks << pg->shift, (int64_t)D_I * halves, (int64_t)D * halves, *pg);
  else
    hipLaunchKernelGGL(cache_append_kernel<false>, dim3((unsigned)B), dim3(256), 0, stream,
                       static_cast<uint16_t*>(k_idx), static_cast<uint16_t*>(kv),
                       static_cast<const uint16_t*>(new_k_idx), static_cast<const uint16_t*>(new_kv), pos, N,
                       (int64_t)D_I * halves, (int64_t)D * halves, Paged{});
  return hipGetLastError();
}

hipError_t launch_page_translate(const int32_t* idx, int32_t* out, int64_t B, int64_t Tq, int K, const Paged& pg,
                                 hipStream_t stream) {
  const int64_t total = B * Tq * K;
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL(page_translate_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, idx, out,
                     total, Tq, K, pg);
  return hipGetLastError();
}

}  // namespace dsa

// Host-side launchers of the gfx950 kernels (one per kernel family).
// Each returns the hipError_t of its launch; shapes are validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

// seq_lens (device, [B], may be null): per-sequence lengths in tokens; when
// given, the queries of sequence b sit at positions seq_lens[b] - Tq + t and
// q_pos0 is ignored.  m: compression rate of the key axis (row w becomes
// visible to the query at position p when w < (p + 1) / m; m = 1: causal).
hipError_t launch_index_scores_bf16(const uint16_t* q_idx, const uint16_t* k_idx, const uint16_t* w,
                                    float* scores, int64_t B, int64_t Tq, int64_t N, int64_t q_pos0,
                                    hipStream_t stream, const int64_t* seq_lens = nullptr, int m = 1);
hipError_t launch_index_scores_f32(const float* q_idx, const float* k_idx, const float* w, float* scores,
                                   int64_t B, int64_t Tq, int64_t N, int64_t q_pos0, int H_I, int D_I,
                                   hipStream_t stream, const int64_t* seq_lens = nullptr, int m = 1);

size_t topk_workspace_bytes(int64_t B, int64_t Tq, int64_t N, int K);
hipError_t launch_topk(const float* scores, int32_t* idx, int64_t B, int64_t Tq, int64_t N, int64_t q_pos0,
                       int K, void* workspace, hipStream_t stream, const int64_t* seq_lens = nullptr,
                       int m = 1);

// Writes row pos[b] of each sequence's caches (rows of D_I and D elements of
// esize bytes); entries of pos outside [0, N) are skipped.  Either cache may
// be null.
hipError_t launch_cache_append(void* k_idx, void* kv, const void* new_k_idx, const void* new_kv, const int64_t* pos,
                               int64_t B, int64_t N, int D_I, int D, int esize, hipStream_t stream);

int mla_num_splits(int64_t rows, int K);
size_t mla_workspace_bytes(int64_t rows, int H, int DV, int K, int is_bf16);
hipError_t launch_sparse_mla_bf16(const uint16_t* q, const uint16_t* kv, const int32_t* idx, uint16_t* out,
                                  float* lse, int64_t B, int64_t Tq, int64_t N, int K, float scale,
                                  void* workspace, hipStream_t stream);
hipError_t launch_sparse_mla_f32(const float* q, const float* kv, const int32_t* idx, float* out, float* lse,
                                 int64_t B, int64_t Tq, int64_t N, int H, int D, int DV, int K, float scale,
                                 hipStream_t stream);

}  // namespace dsa

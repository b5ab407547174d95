// Host-side launchers of the gfx950 kernels (one per kernel family).
// Each returns the hipError_t of its launch; shapes are validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

// A paged cache: rows live in a pool of num_blocks blocks of 2^shift rows;
// row r of sequence b is pool row table[b * max_blocks + (r >> shift)] *
// 2^shift + (r & (2^shift - 1)).  A table entry outside [0, num_blocks) marks
// an unset block: appends skip it, index translation masks it, and the
// indexer reads it as block 0 (a caller error that must not become a wild
// access).
struct Paged {
  const int32_t* table;
  int64_t max_blocks;
  int32_t shift;
  int32_t num_blocks;
};

// Pre-selection lists of the decode indexer (workspace of the top-k): each
// workgroup of the indexer scores one segment of kpw keys of one row, and
// lists, in index order, every key of the segment whose order key is at least
// thr (at most cap entries, about tgt); thr = 0 means the list holds the whole
// segment.
// The top-k then selects among the lists of a row and falls back to the full
// row when some truncated list's thr lies above the row's K-th key.
constexpr int kPreselRowCap = 8192;  // list entries the top-k can hold for one row
constexpr int kPreselMaxCap = 512;   // entries of one segment's list
struct PreselWs {
  uint32_t* count;  // [R][G] entries in each list
  uint32_t* thr;    // [R][G]
  uint2* list;      // [R][G][cap] (order key, key index)
  int64_t kpw;      // keys per segment
  int32_t G;        // segments per row (the indexer's grid)
  int32_t cap;      // entries per list
  int32_t tgt;      // entries a list aims to hold (a few times the segment's expected share)
};
// The pre-selection geometry of a decode problem for the bf16 indexer, or
// with fp8 for the FP8 indexer (whose segments are the FP8 kernel's
// workgroups), or false when it does not apply (then the indexer runs plain
// and the top-k takes its usual methods).
bool presel_geometry(int64_t B, int64_t Tq, int64_t N, int64_t nmax, int K, PreselWs& ps, bool fp8 = false);
// Workspace of the lists: nonzero when either indexer's geometry applies.
size_t presel_workspace_bytes(int64_t B, int64_t Tq, int64_t N, int K);
// Places the lists in `workspace` (presel_workspace_bytes large).
PreselWs presel_ws(void* workspace, int64_t B, int64_t Tq, int64_t N, int64_t nmax, int K, bool fp8 = false);

// seq_lens (device, [B], may be null): per-sequence lengths in tokens; when
// given, the queries of sequence b sit at positions seq_lens[b] - Tq + t and
// q_pos0 is ignored.  m: compression rate of the key axis (row w becomes
// visible to the query at position p when w < (p + 1) / m; m = 1: causal).
// pg (may be null): the key cache is a paged pool (decode shapes, Tq <= 4;
// seq_lens required); N is then the logical capacity max_blocks << shift.
// ps (may be null): also write the pre-selection lists (decode shapes whose
// geometry presel_geometry accepts; ps must come from presel_ws with the same
// B, Tq, N and longest visible row, n entries at rate m).
hipError_t launch_index_scores_bf16(const uint16_t* q_idx, const uint16_t* k_idx, const uint16_t* w,
                                    float* scores, int64_t B, int64_t Tq, int64_t N, int64_t q_pos0,
                                    hipStream_t stream, const int64_t* seq_lens = nullptr, int m = 1,
                                    const Paged* pg = nullptr, const PreselWs* ps = nullptr);
hipError_t launch_index_scores_f32(const float* q_idx, const float* k_idx, const float* w, float* scores,
                                   int64_t B, int64_t Tq, int64_t N, int64_t q_pos0, int H_I, int D_I,
                                   hipStream_t stream, const int64_t* seq_lens = nullptr, int m = 1);

// FP8 indexer: rows of 128 bf16 -> Hadamard-rotated OCP E4M3 codes and one
// power-of-two scale per row; scores from codes and scales (decode kernel,
// any Tq, causal with q_pos0).  ps (may be null, non-paged only): also write the
// pre-selection lists, as for the bf16 indexer (presel_ws with fp8).
hipError_t launch_quantize_fp8(const uint16_t* x, uint8_t* codes, float* scales, int64_t R, hipStream_t stream);
hipError_t launch_index_scores_fp8(const uint8_t* q8, const float* qs, const uint8_t* k8, const float* ks,
                                   const uint16_t* w, float* scores, int64_t B, int64_t Tq, int64_t N,
                                   int64_t q_pos0, hipStream_t stream, const int64_t* seq_lens = nullptr,
                                   const Paged* pg = nullptr, const PreselWs* ps = nullptr);

size_t topk_workspace_bytes(int64_t B, int64_t Tq, int64_t N, int K);
// The top-k from the indexer's pre-selection lists (scores: the full rows,
// read only by rows that fall back).
hipError_t launch_topk_presel(const float* scores, int32_t* idx, int64_t B, int64_t Tq, int64_t N, int64_t q_pos0,
                              int K, const PreselWs& ps, hipStream_t stream, const int64_t* seq_lens = nullptr,
                              int m = 1);
hipError_t launch_topk(const float* scores, int32_t* idx, int64_t B, int64_t Tq, int64_t N, int64_t q_pos0,
                       int K, void* workspace, hipStream_t stream, const int64_t* seq_lens = nullptr,
                       int m = 1);

// Writes row pos[b] of each sequence's caches (rows of D_I and D elements of
// esize bytes); entries of pos outside [0, N) are skipped.  Either cache may
// be null.
// pg (may be null): the caches are pools and pos[b] is a logical row.
hipError_t launch_cache_append(void* k_idx, void* kv, const void* new_k_idx, const void* new_kv, const int64_t* pos,
                               int64_t B, int64_t N, int D_I, int D, int esize, hipStream_t stream,
                               const Paged* pg = nullptr);
// Logical key indices idx [B, Tq, K] -> pool rows in out (same shape).
hipError_t launch_page_translate(const int32_t* idx, int32_t* out, int64_t B, int64_t Tq, int K, const Paged& pg,
                                 hipStream_t stream);

int mla_num_splits(int64_t rows, int K);
size_t mla_workspace_bytes(int64_t rows, int H, int DV, int K, int is_bf16);
hipError_t launch_sparse_mla_bf16(const uint16_t* q, const uint16_t* kv, const int32_t* idx, uint16_t* out,
                                  float* lse, int64_t B, int64_t Tq, int64_t N, int K, float scale,
                                  void* workspace, hipStream_t stream);
hipError_t launch_sparse_mla_f32(const float* q, const float* kv, const int32_t* idx, float* out, float* lse,
                                 int64_t B, int64_t Tq, int64_t N, int H, int D, int DV, int K, float scale,
                                 hipStream_t stream);

// Batched bf16 GEMM: C[z][m, n] = sum_k A[z][m, k] * B[z](k, n) for z < batch,
// fp32 accumulation, bf16 (round to nearest even) output.  A: row m at
// A + z*sA + m*lda, k contiguous.  B: b_nk ? element (k, n) at B + z*sB +
// n*ldb + k : at B + z*sB + k*ldb + n.  C: element (m, n) at C + z*sC + m*ldc +
// n.  Requires K % 32 == 0, 16-byte aligned rows of A and B (lda, ldb, sA, sB
// multiples of 8, and N % 8 == 0 when !b_nk), M <= 65535*64, batch <= 65535.
// When cp_dst is set, the first column block also copies cp_w (a multiple of
// 8) elements of each row m: cp_src + z*cp_ss + m*cp_lds -> cp_dst + z*cp_sd +
// m*cp_ldd (16-byte aligned rows).
struct GemmArgs {
  const uint16_t* A;
  int64_t lda, sA;
  const uint16_t* B;
  int64_t ldb, sB;
  uint16_t* C;
  int64_t ldc, sC;
  int64_t M;
  int N, K;
  const uint16_t* cp_src;
  int64_t cp_lds, cp_ss;
  uint16_t* cp_dst;
  int64_t cp_ldd, cp_sd;
  int cp_w;
};
hipError_t launch_gemm_bf16(const GemmArgs& g, bool b_nk, int64_t batch, hipStream_t stream);

// Streaming read (dst null) or copy of `bytes` (a multiple of 16, 16-byte
// aligned buffers): the bandwidth yardstick.
hipError_t launch_calib_stream(const void* src, void* dst, size_t bytes, hipStream_t stream);

}  // namespace dsa

/*
 * CPU oracle of the DeepSeek Sparse Attention (DSA) forward pass: C interface.
 *
 * TEST INFRASTRUCTURE ONLY.  The test suite, the package smoke check and the
 * CPU-baseline leg of the benchmark load this library (through the ctypes
 * layer in oracle/__init__.py); the product path never does.  This interface
 * and its implementation (dsa_oracle.cpp) share no code, header or constant
 * with the HIP library: the only thing both sides consume is the seeded input
 * generator in synth/.
 *
 * Conventions of every entry point:
 *   * tensors are dense, row-major host arrays;
 *   * a read-only floating-point tensor comes as (pointer, element type):
 *     DSAO_F64 (double), DSAO_F32 (float) or DSAO_BF16 (uint16_t bit patterns
 *     of bfloat16, the upper half of a float32); every value is widened
 *     exactly to double before any arithmetic;
 *   * "rows" lists the queries to compute as n_rows pairs (b, t), flattened:
 *     rows[2r] is the sequence, rows[2r+1] the query within it; outputs are
 *     indexed by r;
 *   * q_pos0[b] is the absolute position of query 0 of sequence b; query t
 *     sits at position q_pos0[b] + t;
 *   * threads <= 0 uses every hardware thread; rows are dealt to threads
 *     round-robin, so any thread count gives the same bits;
 *   * return value 0 = success, 1 = invalid argument (nothing written),
 *     2 = out of memory or no thread could be started.
 */
#ifndef DSA_ORACLE_H
#define DSA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { DSAO_F64 = 0, DSAO_F32 = 1, DSAO_BF16 = 2 };

int dsao_version(void);

/* out[i] = element i of x, widened to double (i < n). */
int dsao_widen(const void* x, int dt, int64_t n, double* out);

/* Visible keys of the query at position q_pos0 + t in a cache of N rows whose
 * key axis is compressed at rate m (m = 1: plain causal rule). */
int64_t dsao_n_valid_keys(int64_t t, int64_t q_pos0, int64_t N, int64_t m);

/* O1, lightning indexer.  q_idx [B,Tq,H_I,D_I], k_idx [B,N,D_I], w [B,Tq,H_I].
 * out [n_rows, N]: for each listed query, entries s < n_valid_keys get
 *   I[s] = sum_h w[h] * ReLU(sum_d q_idx[h,d] * k_idx[s,d])
 * in double; entries past the visible keys are left untouched. */
int dsao_index_scores(const void* q_idx, int q_dt, const void* k_idx, int k_dt, const void* w, int w_dt,
                      int64_t B, int64_t Tq, int64_t N, int32_t H_I, int32_t D_I, const int64_t* q_pos0,
                      int64_t m, const int64_t* rows, int64_t n_rows, double* out, int threads);

/* O2, top-k.  scores [n_rows, row_stride] float32; row r has n_valid[r]
 * visible entries.  out [n_rows, K]: the K best keys under (score desc,
 * index asc), listed ascending, padded with -1 when n_valid[r] < K. */
int dsao_topk(const float* scores, int64_t n_rows, int64_t row_stride, const int64_t* n_valid, int32_t K,
              int32_t* out, int threads);

/* O3, sparse MLA in absorbed latent form.  q [B,Tq,H,D], kv [B,N,D],
 * idx [B,Tq,K] (entries < 0 or >= N are masked).  o [n_rows,H,DV] and
 * lse [n_rows,H] (natural log; -inf for a row with no valid index). */
int dsao_sparse_mla(const void* q, int q_dt, const void* kv, int kv_dt, const int32_t* idx, int64_t B, int64_t Tq,
                    int64_t N, int32_t H, int32_t D, int32_t DV, int32_t K, double scale, const int64_t* rows,
                    int64_t n_rows, double* o, double* lse, int threads);

/* O3', the same attention written as dense causal attention over every
 * visible key plus an additive mask (0 on selected keys, -inf elsewhere). */
int dsao_dense_masked_mla(const void* q, int q_dt, const void* kv, int kv_dt, const int32_t* idx, int64_t B,
                          int64_t Tq, int64_t N, int32_t H, int32_t D, int32_t DV, int32_t K, double scale,
                          const int64_t* q_pos0, const int64_t* rows, int64_t n_rows, double* o, double* lse,
                          int threads);

/* O4, composition: O1 -> (scores rounded to float32) -> O2 -> O3 for each
 * listed query.  scores (nullable) [n_rows, N] as in dsao_index_scores;
 * idx [n_rows, K]; o [n_rows, H, DV]; lse [n_rows, H]. */
int dsao_forward(const void* q_idx, int qi_dt, const void* k_idx, int ki_dt, const void* w, int w_dt,
                 const void* q, int q_dt, const void* kv, int kv_dt, int64_t B, int64_t Tq, int64_t N,
                 const int64_t* q_pos0, int32_t H_I, int32_t D_I, int32_t H, int32_t D, int32_t DV, int32_t K,
                 double scale, const int64_t* rows, int64_t n_rows, double* scores, int32_t* idx, double* o,
                 double* lse, int threads);

/* O5, Sylvester Hadamard matrix H_n (n a power of two), out [n, n]. */
int dsao_sylvester_hadamard(int32_t n, double* out);

/* FP8 indexer helpers (reading of the rotation and format: see oracle/__init__.py). */
int dsao_fwht_f32(float* x, int64_t n_rows, int32_t n);
int dsao_e4m3_decode(const uint8_t* codes, int64_t n, double* out);
int dsao_e4m3_encode_rne(const float* v, int64_t n, uint8_t* out);   /* 1 if some |v| > 448 or NaN */
int dsao_pow2_scale_exp(double amax);
int dsao_quantize_fp8_rows(const void* x, int dt, int64_t n_rows, int32_t D, uint8_t* codes, float* scales);
/* q8 [B,Tq,H_I,D], qs [B,Tq,H_I], k8 [B,N,D], ks [B,N], w [B,Tq,H_I]; out [n_rows, N]. */
int dsao_index_scores_fp8(const uint8_t* q8, const float* qs, const uint8_t* k8, const float* ks, const void* w,
                          int w_dt, int64_t B, int64_t Tq, int64_t N, int32_t H_I, int32_t D, const int64_t* q_pos0,
                          const int64_t* rows, int64_t n_rows, double* out, int threads);

/* Projections on either side of the absorbed MLA, and the naive per-head form. */
int dsao_linear(const void* x, int x_dt, const void* W, int W_dt, int64_t M, int64_t N_out, int64_t K_in, double* y,
                int threads);
int dsao_mla_absorb_query(const void* q, int q_dt, const void* W_UK, int w_dt, int64_t M, int32_t H, int32_t d_nope,
                          int32_t d_rope, int32_t d_c, double* out, int threads);
int dsao_mla_output_projection(const void* o_lat, int o_dt, const void* W_UV, int w_dt, int64_t M, int32_t H,
                               int32_t d_c, int32_t d_v, double* out, int threads);
int dsao_mla_naive_row(const void* q_head, int q_dt, const void* c_kv, int c_dt, const void* k_rope, int r_dt,
                       int64_t N, const int32_t* idx, int32_t K, const void* W_UK, int uk_dt, const void* W_UV,
                       int uv_dt, int32_t H, int32_t d_nope, int32_t d_rope, int32_t d_c, int32_t d_v, double scale,
                       double* o, double* lse, int threads);

/* Paged cache: logical row r of a sequence is pool row
 * table_row[r / block_size] * block_size + r % block_size.  Copies n_rows
 * rows of row_bytes bytes; 1 if an entry the rows need lies outside the pool. */
int dsao_paged_gather(const void* pool, int64_t pool_rows, int64_t row_bytes, const int64_t* table_row,
                      int64_t table_len, int64_t block_size, int64_t n_rows, void* out);

#ifdef __cplusplus
}
#endif

#endif /* DSA_ORACLE_H */

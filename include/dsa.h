/*
 * dsa.h -- C ABI of the MI355X (gfx950) DeepSeek Sparse Attention forward.
 *
 * The library computes the three steps of DeepSeek Sparse Attention (DSA) as
 * described in the DeepSeek-V3.2 model documentation, section "DeepSeek
 * Sparse Attention (DSA)":
 *
 *   1. lightning indexer: a cheap scorer with few heads gives every query an
 *      index score against each key at or before its position, using a
 *      per-token, single-head indexer key cache of width index_head_dim;
 *   2. fine-grained token selection: each query keeps its index_topk
 *      best-scoring keys;
 *   3. the main MLA attention runs over the kept keys only (on the pages this
 *      is an additive mask over dense attention; here it is a gather over the
 *      kept rows, which gives the same result).
 *
 * Shapes follow the DeepseekV32Config section of the same documentation
 * (index_n_heads = 64, index_head_dim = 128, index_topk = 2048,
 * num_attention_heads = 128, kv_lora_rank = 512, qk_rope_head_dim = 64).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor arguments are DEVICE pointers to dense, row-major, contiguous
 *    buffers owned by the caller.  The library never allocates, frees or
 *    keeps a pointer after the call returns, and never synchronises: work is
 *    enqueued on `stream` (a hipStream_t; NULL = the default stream) and the
 *    call returns at once.  Errors raised by the device show up at the
 *    caller's next synchronisation.
 *  - Float tensors of one call share one storage type, `dtype`:
 *    DSA_BF16 (bfloat16) or DSA_F32 (float32).  Scores are always float32,
 *    indices always int32.  Every pointer must be 16-byte aligned.
 *  - B sequences, Tq queries per sequence, N cached keys per sequence.  Query
 *    t of a sequence sits at absolute position q_pos0 + t and sees keys
 *    s = 0 .. min(N, q_pos0 + t + 1) - 1 (its own position included).
 *    Prefill: q_pos0 = 0, Tq = N.  Decode of one new token whose key is the
 *    last cache row: Tq = 1, q_pos0 = N - 1.
 *  - Validation happens on the host before anything is enqueued.  On any
 *    error the call returns a non-zero dsa_status, enqueues nothing and leaves
 *    every output untouched; dsa_last_error() then describes the failure
 *    (thread-local text).  A failed kernel launch returns DSA_ERR_HIP.
 *  - Compiled shapes.  DSA_BF16: indexer H_I = 64, D_I = 128; MLA H = 128,
 *    D = 576, DV = 512.  DSA_F32 (small reference-size problems): indexer
 *    H_I <= 64, D_I <= 256; MLA H <= 128, D <= 1024, DV <= min(D, 512).
 *    Other shapes return DSA_ERR_UNSUPPORTED.
 *  - Sizes: 1 <= B, Tq, N; N < 2^31; 1 <= K <= 65536; q_pos0 >= 0.
 *  - Calls are reentrant; concurrent calls on different streams may share
 *    inputs but not outputs or workspaces.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dsa_status {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = 1, /* null pointer, bad size, misaligned pointer, bad dtype */
  DSA_ERR_UNSUPPORTED = 2, /* valid request for a shape that is not compiled */
  DSA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the size query returns */
  DSA_ERR_HIP = 4          /* the HIP runtime refused a launch */
} dsa_status;

typedef enum dsa_dtype { DSA_BF16 = 0, DSA_F32 = 1 } dsa_dtype;

/* Library version as major*10000 + minor*100 + patch. */
int dsa_version(void);

/* Static text for a status code. */
const char* dsa_status_string(int status);

/* Detail of the last error returned on the calling thread ("" if none). */
const char* dsa_last_error(void);

/*
 * Step 1 -- lightning indexer scores.
 * (DeepSeek-V3.2 documentation, section "DeepSeek Sparse Attention (DSA)",
 *  paragraph on the lightning indexer and paragraph on its key cache.)
 *
 *   scores[b,t,s] = sum_{h < H_I} w[b,t,h] * max(0, sum_{d < D_I} q_idx[b,t,h,d] * k_idx[b,s,d])
 *
 * for s < min(N, q_pos0 + t + 1).  Entries of a row past that bound are not
 * written.  No scale is applied (fold any scale into w).  Products are summed
 * in float32: integer-valued inputs with power-of-two weights, whose sums stay
 * below 2^24 steps, give exactly the real-number scores.
 *
 *   q_idx  [B, Tq, H_I, D_I]  indexer queries                  (dtype)
 *   k_idx  [B, N, D_I]        single-head indexer key cache      (dtype)
 *   w      [B, Tq, H_I]       per-token head weights             (dtype)
 *   scores [B, Tq, N]         output                             (float32)
 */
dsa_status dsa_index_scores(const void* q_idx, const void* k_idx, const void* w, float* scores,
                            int64_t B, int64_t Tq, int64_t N, int64_t q_pos0, int32_t H_I,
                            int32_t D_I, int32_t dtype, void* stream);

/*
 * Step 2 -- per-query top-k.
 * (DeepSeek-V3.2 documentation, section "DeepSeek Sparse Attention (DSA)",
 *  paragraph on fine-grained token selection; the -1 "no selection" entry of
 *  the DeepSeek-V4 documentation, attention mask layout section.)
 *
 * Row (b,t) considers its n = min(N, q_pos0 + t + 1) visible scores.  If
 * n <= K it returns 0, 1, ..., n-1 followed by K-n entries of -1.  Otherwise
 * it returns the K keys ranked first under (score descending, key index
 * ascending) -- equal scores go to the lower index, -0 equals +0 -- listed
 * in ascending key order.  Scores must be finite (NaN gives an unspecified
 * but in-range selection).
 *
 *   scores [B, Tq, N] float32;  idx [B, Tq, K] int32 output.
 *   workspace: dsa_topk_workspace_size(...) bytes of device memory (may be
 *   NULL when that size is 0); contents on entry do not matter.
 */
size_t dsa_topk_workspace_size(int64_t B, int64_t Tq, int64_t N, int32_t K);
dsa_status dsa_topk(const float* scores, int32_t* idx, int64_t B, int64_t Tq, int64_t N,
                    int64_t q_pos0, int32_t K, void* workspace, size_t ws_bytes, void* stream);

/*
 * Steps 1 and 2 as the fused forward runs them at long-context decode shapes.
 * (DeepSeek-V3.2 documentation, section "DeepSeek Sparse Attention (DSA)":
 *  the lightning indexer scores each query against every earlier key, and
 *  fine-grained token selection keeps the index_topk best.)
 *
 * dsa_index_scores_presel: dsa_index_scores (same scores, same rules), and in
 *   `workspace` (dsa_topk_workspace_size(B, Tq, N, K) bytes) a pre-selection
 *   of each query's row: the bf16 decode indexer scores every row in segments
 *   of keys, and each segment also lists, in index order, all of its keys at
 *   or above a threshold it picks from its own scores (a few times the
 *   segment's expected share of the row's K best).
 * dsa_topk_presel: dsa_topk (same indices) for scores and a workspace that
 *   dsa_index_scores_presel filled with the same B, Tq, N, q_pos0, K and
 *   dtype.  It selects among the listed keys; where some list's threshold
 *   lies above the row's K-th key (the listed keys cannot be shown to hold
 *   the row's top K) that row is selected from its full scores instead, so
 *   the result is exact in every case.
 * Where no pre-selection applies (fp32, more than 4 queries per sequence,
 * rows of at most 16384 keys, K > 4096, or too many segments per row for the
 * lists) the pair is exactly dsa_index_scores then dsa_topk.  Arguments,
 * layouts and errors are those of dsa_index_scores and dsa_topk.
 */
dsa_status dsa_index_scores_presel(const void* q_idx, const void* k_idx, const void* w, float* scores,
                                   int64_t B, int64_t Tq, int64_t N, int64_t q_pos0, int32_t H_I,
                                   int32_t D_I, int32_t K, int32_t dtype, void* workspace, size_t ws_bytes,
                                   void* stream);
dsa_status dsa_topk_presel(const float* scores, int32_t* idx, int64_t B, int64_t Tq, int64_t N,
                           int64_t q_pos0, int32_t K, int32_t dtype, void* workspace, size_t ws_bytes,
                           void* stream);

/*
 * Step 3 -- sparse MLA in absorbed latent form over the selected keys.
 * (DeepSeek-V3.2 documentation, section "DeepSeek Sparse Attention (DSA)",
 *  paragraph on fine-grained token selection: attention restricted to the
 *  selected tokens; DeepseekV32Config section for kv_lora_rank = 512 and
 *  qk_rope_head_dim = 64, hence D = 576 and DV = 512.)
 *
 * For every (b, t, h), with S = { idx[b,t,j] : 0 <= idx[b,t,j] < N }:
 *   l_j          = scale * sum_{d < D} q[b,t,h,d] * kv[b,idx_j,d]
 *   out[b,t,h,:] = sum_j softmax(l)_j * kv[b,idx_j,0:DV]
 *   lse[b,t,h]   = ln sum_j exp(l_j)
 * Entries of idx that are negative or >= N are masked (an additive -inf).
 * An index row with no valid entry yields out = 0 and lse = -inf.  idx must
 * not repeat a key within a row (the top-k step never does); causality is not
 * checked here -- idx decides.  bf16 accumulates in float32 (MFMA) and rounds
 * out to bf16 (nearest-even).  When there are fewer query rows than compute
 * units, a row's index list is split over several workgroups; each split's
 * normalised output is then rounded to bf16 in the workspace and the splits
 * are merged in float32 (so such rows are rounded twice).
 *
 *   q   [B, Tq, H, D] (dtype);  kv [B, N, D] latent cache (dtype), value = the
 *   first DV columns;  idx [B, Tq, K] int32;  out [B, Tq, H, DV] (dtype);
 *   lse [B, Tq, H] float32, may be NULL.
 *   workspace: dsa_sparse_mla_workspace_size(...) bytes (split-K partials).
 */
size_t dsa_sparse_mla_workspace_size(int64_t B, int64_t Tq, int32_t H, int32_t DV, int32_t K,
                                     int32_t dtype);
dsa_status dsa_sparse_mla_fwd(const void* q, const void* kv, const int32_t* idx, void* out,
                              float* lse, int64_t B, int64_t Tq, int64_t N, int32_t H, int32_t D,
                              int32_t DV, int32_t K, float scale, int32_t dtype, void* workspace,
                              size_t ws_bytes, void* stream);

/*
 * Steps 1-3 in one call, stream-ordered, with no host synchronisation.
 * (DeepSeek-V3.2 documentation, section "DeepSeek Sparse Attention (DSA)":
 *  each layer runs its own indexer, selection and sparse attention.)
 *
 * Same arguments as the three steps above.  The intermediate scores (and the
 * indices, when idx_out is NULL) live in the workspace; pass idx_out
 * [B, Tq, K] int32 to also receive the selection.  Steps 1 and 2 run as
 * dsa_index_scores_presel and dsa_topk_presel.  The result equals
 * dsa_sparse_mla_fwd(dsa_topk(dsa_index_scores(...))) bit for bit.
 */
size_t dsa_forward_workspace_size(int64_t B, int64_t Tq, int64_t N, int32_t H, int32_t DV,
                                  int32_t K, int32_t dtype);
dsa_status dsa_forward(const void* q_idx, const void* k_idx, const void* w, const void* q,
                       const void* kv, void* out, float* lse, int32_t* idx_out, int64_t B,
                       int64_t Tq, int64_t N, int64_t q_pos0, int32_t H_I, int32_t D_I, int32_t H,
                       int32_t D, int32_t DV, int32_t K, float scale, int32_t dtype,
                       void* workspace, size_t ws_bytes, void* stream);

/*
 * dsa_forward without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops and
 * harnesses that forbid hipMalloc.
 *
 * Arguments, outputs and errors are those of dsa_forward; the result equals
 * dsa_forward's bit for bit.  The workspace is instead a scratch array of
 * DSA_NOALLOC_SCRATCH_BYTES bytes that the library holds in static device
 * memory: one copy per GPU it runs on, set up on the first call on that GPU
 * (the device `stream` belongs to; NULL = the current device) and kept until
 * the process ends.  The call allocates nothing.  A problem whose
 * dsa_forward_workspace_size exceeds DSA_NOALLOC_SCRATCH_BYTES returns
 * DSA_ERR_WORKSPACE and launches nothing (64 MiB holds, for example, the
 * 32-sequence decode at 131072-token context; a 16384-token prefill needs
 * dsa_forward).  Every call on one GPU shares that GPU's scratch, which keeps
 * the last call's contents (nothing in it needs to start at zero): calls
 * that overlap on one GPU (on different streams, or from different threads
 * without ordering) race and give undefined results.
 */
#define DSA_NOALLOC_SCRATCH_BYTES (64u << 20)
dsa_status dsa_forward_noalloc(const void* q_idx, const void* k_idx, const void* w, const void* q,
                               const void* kv, void* out, float* lse, int32_t* idx_out, int64_t B,
                               int64_t Tq, int64_t N, int64_t q_pos0, int32_t H_I, int32_t D_I,
                               int32_t H, int32_t D, int32_t DV, int32_t K, float scale, int32_t dtype,
                               void* stream);

/*
 * Per-sequence cache lengths ("varlen"): the three steps and the fused call
 * for a batch whose sequences hold different numbers of tokens.
 * (DeepSeek-V3.2 documentation, section "DeepSeek Sparse Attention (DSA)":
 * each query is scored against all of its sequence's preceding keys; in a
 * batch those counts differ per sequence.)
 *
 * seq_lens: device memory, int64 [B], 8-byte aligned; sequence b holds
 * seq_lens[b] valid rows of its caches (expected 0 <= seq_lens[b] <= N; the
 * kernels clamp to N).  Its Tq queries are its last Tq tokens: query t sits at
 * position seq_lens[b] - Tq + t and sees keys s < seq_lens[b] - Tq + t + 1 (a
 * query at a negative position sees none: its top-k row is all -1 and its
 * attention output is 0 with lse = -inf).  Everything else, including the
 * workspaces and their sizes (dsa_topk_workspace_size,
 * dsa_forward_workspace_size with the same B, Tq, N), is as for the entry
 * points above with q_pos0 replaced by seq_lens[b] - Tq per sequence.  The
 * host cannot see seq_lens, so no length is validated.
 */
dsa_status dsa_index_scores_varlen(const void* q_idx, const void* k_idx, const void* w, float* scores,
                                   const int64_t* seq_lens, int64_t B, int64_t Tq, int64_t N, int32_t H_I,
                                   int32_t D_I, int32_t dtype, void* stream);
dsa_status dsa_topk_varlen(const float* scores, int32_t* idx, const int64_t* seq_lens, int64_t B, int64_t Tq,
                           int64_t N, int32_t K, void* workspace, size_t ws_bytes, void* stream);
dsa_status dsa_forward_varlen(const void* q_idx, const void* k_idx, const void* w, const void* q, const void* kv,
                              void* out, float* lse, int32_t* idx_out, const int64_t* seq_lens, int64_t B,
                              int64_t Tq, int64_t N, int32_t H_I, int32_t D_I, int32_t H, int32_t D, int32_t DV,
                              int32_t K, float scale, int32_t dtype, void* workspace, size_t ws_bytes,
                              void* stream);

/*
 * Indexer and top-k over a compressed key axis (the DeepSeek-V4 compressed
 * sparse attention layer: the lightning indexer scores each query against
 * compressed cache entries and keeps index_topk of them).
 * (DeepSeek-V4 documentation, hybrid attention section for the compression
 *  rate m of the compressed sparse layer (default 4) and index_topk (default
 *  512); attention mask layout section for the visibility rule: entry w,
 *  which summarises positions m*w .. m*w + m - 1, becomes visible to the query
 *  at position p once that window has closed, i.e. when w < (p + 1) / m, so
 *  queries before the first window closes select nothing and get only -1.)
 *
 * k_idx [B, N, D_I] holds N compressed entries per sequence (the indexer's
 * compressed key cache); query t sits at position p = q_pos0 + t and sees
 * entries w < min(N, (p + 1) / m) (integer division).  m = 1 is
 * dsa_index_scores / dsa_topk.  m < 1 returns DSA_ERR_INVALID_ARG and
 * launches nothing.  Arguments, layouts, workspace and the other errors are
 * those of dsa_index_scores / dsa_topk.  When no query sees an entry the
 * indexer launches nothing and leaves scores untouched.
 *
 * dsa_index_scores_compressed_presel / dsa_topk_compressed_presel: the same
 * two steps with the decode pre-selection of dsa_index_scores_presel and
 * dsa_topk_presel over the visible entries (rows of more than 16384 visible
 * entries, at most 4 queries per sequence, K <= 4096): the indexer also lists
 * each segment's best entries in `workspace` (dsa_topk_workspace_size(B, Tq,
 * N, K) bytes), and the top-k selects among the lists, with the same exact
 * fallback to a row's full scores.  The indices equal dsa_topk_compressed's.
 * Pass both calls the same B, Tq, N, q_pos0, m, K, dtype and workspace; where
 * no pre-selection applies the pair is dsa_index_scores_compressed then
 * dsa_topk_compressed.
 */
dsa_status dsa_index_scores_compressed(const void* q_idx, const void* k_idx, const void* w, float* scores,
                                       int64_t B, int64_t Tq, int64_t N, int64_t q_pos0, int32_t m, int32_t H_I,
                                       int32_t D_I, int32_t dtype, void* stream);
dsa_status dsa_topk_compressed(const float* scores, int32_t* idx, int64_t B, int64_t Tq, int64_t N,
                               int64_t q_pos0, int32_t m, int32_t K, void* workspace, size_t ws_bytes,
                               void* stream);
dsa_status dsa_index_scores_compressed_presel(const void* q_idx, const void* k_idx, const void* w, float* scores,
                                              int64_t B, int64_t Tq, int64_t N, int64_t q_pos0, int32_t m,
                                              int32_t H_I, int32_t D_I, int32_t K, int32_t dtype, void* workspace,
                                              size_t ws_bytes, void* stream);
dsa_status dsa_topk_compressed_presel(const float* scores, int32_t* idx, int64_t B, int64_t Tq, int64_t N,
                                      int64_t q_pos0, int32_t m, int32_t K, int32_t dtype, void* workspace,
                                      size_t ws_bytes, void* stream);

/*
 * Cache append: one new token per sequence.
 * (DeepSeek-V3.2 documentation, section "DeepSeek Sparse Attention (DSA)",
 *  paragraph on the indexer's key cache: a per-token, single-head key cache
 *  kept next to the main key/value cache and updated as tokens arrive.)
 *
 * Static-cache layout (the caches of the entry points above):
 *   k_idx [B, N, D_I] and kv [B, N, D] (dtype), updated in place;
 *   new_k_idx [B, D_I], new_kv [B, D] (dtype): the new token's rows;
 *   pos: device memory, int64 [B], 8-byte aligned.
 * For every b with 0 <= pos[b] < N: k_idx[b, pos[b], :] = new_k_idx[b, :] and
 * kv[b, pos[b], :] = new_kv[b, :]; other entries of pos write nothing (the
 * host cannot see pos).  A cache and its new rows are given together or both
 * NULL (that cache is then left alone); at least one cache is required.
 * Appending then running the steps with seq_lens[b] = pos[b] + 1 equals
 * running them on caches built with that row in place.
 */
dsa_status dsa_cache_append(void* k_idx, void* kv, const void* new_k_idx, const void* new_kv, const int64_t* pos,
                            int64_t B, int64_t N, int32_t D_I, int32_t D, int32_t dtype, void* stream);

/*
 * Projections on either side of the sparse MLA (bf16 only; fp32 accumulation,
 * outputs rounded to nearest even).
 * (DeepSeek-V3 documentation, "DeepseekV3Config": keys and values are
 *  low-rank projections of a kv_lora_rank-wide latent, with qk_nope_head_dim,
 *  qk_rope_head_dim and v_head_dim per head; its limitations note describes the
 *  naive per-head form these projections turn into the absorbed one.
 *  DeepSeek-V3.2 documentation, "DeepSeek Sparse Attention (DSA)": the
 *  indexer's queries come from the low-rank query latent through wq_b.)
 *
 * dsa_mla_absorb_q: folds the key up-projection into the query.
 *   q     [M, H, d_nope + d_rope]  per-head queries, the part without rotary
 *                                  embedding first (M = B*Tq rows);
 *   w_uk  [H, d_nope, d_c]         key up-projection of each head (key_h = w_uk[h] c);
 *   q_lat [M, H, d_c + d_rope]     out: q_lat[m,h,:d_c] = w_uk[h]^T q[m,h,:d_nope],
 *                                  q_lat[m,h,d_c:] = q[m,h,d_nope:] (copied).
 *   q_lat is the query dsa_sparse_mla_fwd takes (d_c = 512, d_rope = 64).
 *   Requires d_nope a positive multiple of 32, d_c a positive multiple of 8,
 *   d_rope a multiple of 8 (0 allowed).
 *
 * dsa_mla_out_proj: applies the value up-projection to the latent output.
 *   o_lat [M, H, d_c]   the output of dsa_sparse_mla_fwd;
 *   w_uv  [H, d_v, d_c] value up-projection of each head (value_h = w_uv[h] c);
 *   o     [M, H, d_v]   out: o[m,h,:] = w_uv[h] o_lat[m,h,:].
 *   Requires d_c a positive multiple of 32, d_v >= 1.
 *
 * dsa_linear: y [M, N] = x [M, K] w^T, w [N, K] (a linear layer's weight, as
 *   the indexer's wq_b [H_I*D_I, q_lora_rank] and its head-weight projection).
 *   Requires K a positive multiple of 32, N >= 1.
 *
 * All tensors are dense, row-major, 16-byte aligned device memory owned by the
 * caller; inputs and outputs must not overlap.  M = 0 launches nothing.
 * M <= 65535*64 and H <= 65535.  Errors: DSA_ERR_INVALID_ARG (null or
 * misaligned pointers, negative sizes, unknown dtype), DSA_ERR_UNSUPPORTED
 * (fp32, or sizes outside the requirements above); nothing is launched then.
 */
dsa_status dsa_mla_absorb_q(const void* q, const void* w_uk, void* q_lat, int64_t M, int32_t H, int32_t d_nope,
                            int32_t d_rope, int32_t d_c, int32_t dtype, void* stream);
dsa_status dsa_mla_out_proj(const void* o_lat, const void* w_uv, void* o, int64_t M, int32_t H, int32_t d_c,
                            int32_t d_v, int32_t dtype, void* stream);
dsa_status dsa_linear(const void* x, const void* w, void* y, int64_t M, int32_t N, int32_t K, int32_t dtype,
                      void* stream);

/*
 * FP8 indexer.
 * (DeepSeek-V3.2 documentation, "DeepSeek Sparse Attention (DSA)": the
 *  reference implementation runs the lightning indexer in FP8 after a
 *  Hadamard rotation of queries and keys; the rotation is orthogonal,
 *  Hq . Hk = q . k, and FP8 is a precision optimisation only.)
 * Format (the pages give none; readings of this library): OCP E4M3 codes
 * (bias 7, largest finite 448), rows of D = 128 rotated by the unnormalised
 * Sylvester Hadamard matrix (entries +-1, H H^T = 128 I; fast Walsh-Hadamard
 * transform in float32, pair distance 1, 2, 4, ...), one power-of-two scale
 * per row: scale = 2^e, the smallest with max|Hx| <= 448 * 2^e (1 for an
 * all-zero row), codes = E4M3 round-to-nearest-even of Hx / scale.
 *
 * dsa_indexer_quantize_fp8: x bf16 [R, D] -> codes uint8 [R, D], scales
 *   float [R].  Used for the indexer key cache (R = B*N rows, or the rows
 *   being appended) and for the indexer queries (R = B*Tq*H_I rows).
 *   dtype must be DSA_BF16 and D = 128.
 *
 * dsa_index_scores_fp8: scores [B, Tq, N] float32 =
 *   ks[b,s] * sum_h (w[b,t,h] * qs[b,t,h] / 128) * max(0, sum_d q8[b,t,h,d] k8[b,s,d])
 *   (codes read as their E4M3 values), for s < min(N, q_pos0 + t + 1); other
 *   entries are not written.  q8 [B, Tq, H_I, D_I], q_scale [B, Tq, H_I],
 *   k8 [B, N, D_I], k_scale [B, N], w bf16 [B, Tq, H_I] (dtype DSA_BF16);
 *   compiled for H_I = 64, D_I = 128.  The key cache is streamed once per
 *   query (the decode shape); prefill works but re-reads the cache per query.
 *
 * dsa_index_scores_fp8_presel / dsa_topk_presel_fp8: steps 1 and 2 as
 *   dsa_forward_fp8 runs them.  The first is dsa_index_scores_fp8 (same
 *   scores) and, at the decode shapes where dsa_index_scores_presel lists
 *   (more than 16384 keys per row, at most 4 queries per sequence, K <= 4096)
 *   and the FP8 kernel's segments leave room for the lists, the same
 *   pre-selection over those segments, kept in `workspace`
 *   (dsa_topk_workspace_size(B, Tq, N, K) bytes).  The second returns
 *   dsa_topk's indices for those scores, from the lists where they apply
 *   (with the same exact fallback as dsa_topk_presel), else by dsa_topk
 *   itself.  Pass both calls the same B, Tq, N, q_pos0, K and workspace.
 *   Arguments, layouts and errors as for dsa_index_scores_fp8 and dsa_topk.
 *
 * dsa_forward_fp8: dsa_forward with the FP8 indexer in place of the bf16 one
 *   (same outputs, workspace size from dsa_forward_workspace_size); steps 1
 *   and 2 run as dsa_index_scores_fp8_presel and dsa_topk_presel_fp8.
 *
 * All pointers: device memory, 16-byte aligned, owned by the caller.  Errors
 * as for dsa_index_scores / dsa_forward; fp32 head weights or other shapes
 * return DSA_ERR_UNSUPPORTED.
 */
dsa_status dsa_indexer_quantize_fp8(const void* x, uint8_t* codes, float* scales, int64_t R, int32_t D,
                                    int32_t dtype, void* stream);
dsa_status dsa_index_scores_fp8(const uint8_t* q8, const float* q_scale, const uint8_t* k8, const float* k_scale,
                                const void* w, float* scores, int64_t B, int64_t Tq, int64_t N, int64_t q_pos0,
                                int32_t H_I, int32_t D_I, int32_t dtype, void* stream);
dsa_status dsa_index_scores_fp8_presel(const uint8_t* q8, const float* q_scale, const uint8_t* k8,
                                       const float* k_scale, const void* w, float* scores, int64_t B, int64_t Tq,
                                       int64_t N, int64_t q_pos0, int32_t H_I, int32_t D_I, int32_t K,
                                       int32_t dtype, void* workspace, size_t ws_bytes, void* stream);
dsa_status dsa_topk_presel_fp8(const float* scores, int32_t* idx, int64_t B, int64_t Tq, int64_t N,
                               int64_t q_pos0, int32_t K, void* workspace, size_t ws_bytes, void* stream);
dsa_status dsa_forward_fp8(const uint8_t* q8, const float* q_scale, const uint8_t* k8, const float* k_scale,
                           const void* w, const void* q, const void* kv, void* out, float* lse, int32_t* idx_out,
                           int64_t B, int64_t Tq, int64_t N, int64_t q_pos0, int32_t H_I, int32_t D_I, int32_t H,
                           int32_t D, int32_t DV, int32_t K, float scale, int32_t dtype, void* workspace,
                           size_t ws_bytes, void* stream);

/*
 * Paged caches (decode shapes, bf16).
 * (DeepSeek-V3.2 documentation, "DeepSeek Sparse Attention (DSA)": the
 *  indexer key cache lives beside the main key/value cache in static or
 *  growing cache layers and is updated as tokens arrive.  Reading of this
 *  library: a paged layer keeps each cache as a pool of fixed-size blocks
 *  with one block table per sequence.)
 *
 * Layout: k_pool [num_blocks * block_size, D_I] (bf16 indexer keys, or E4M3
 * codes with k_scale_pool [num_blocks * block_size] for the FP8 indexer) and
 * kv_pool [num_blocks * block_size, D] (bf16 latent rows); block_table int32
 * [B, max_blocks] (device, 4-byte aligned): logical row r of sequence b is
 * pool row block_table[b, r / block_size] * block_size + r % block_size.
 * block_size is a power of two in [64, 2^20]; max_blocks * block_size and
 * num_blocks * block_size are below 2^31.  seq_lens int64 [B] (device) gives
 * each sequence's length; its Tq queries are its last Tq tokens, exactly as
 * for the varlen entry points, and only table entries of blocks that hold
 * rows < seq_lens[b] are read.  A table entry outside [0, num_blocks) marks
 * an unset block: the paged append writes nothing into it, the paged sparse
 * MLA masks every index that falls into it (as an index of -1), and the paged
 * indexer reads it as block 0 (a caller error there: wrong scores, never an
 * access outside the pool).
 * Every paged call equals the matching static-cache call on the caches
 * gathered through the table (scores over the logical axis of length
 * max_blocks * block_size, indices logical).
 *
 * dsa_index_scores_paged / dsa_index_scores_fp8_paged: scores [B, Tq,
 *   max_blocks * block_size]; Tq <= 4 (DSA_ERR_UNSUPPORTED otherwise).
 *   Select with dsa_topk_varlen.
 * dsa_sparse_mla_fwd_paged: idx [B, Tq, K] logical; the pool is gathered as
 *   one array of num_blocks * block_size rows (any size below 2^31 rows).
 *   Workspace:
 *   dsa_paged_workspace_size(...) bytes (covers this call and the next).
 * dsa_forward_paged: indexer -> top-k -> sparse MLA over paged caches;
 *   workspace dsa_paged_workspace_size(...) bytes; idx_out (optional)
 *   receives the logical indices.
 * dsa_cache_append_paged: as dsa_cache_append, pos[b] logical; entries of pos
 *   outside [0, max_blocks * block_size), or in an unset block, write nothing.
 */
size_t dsa_paged_workspace_size(int64_t B, int64_t Tq, int64_t max_blocks, int32_t block_size, int32_t H,
                                int32_t DV, int32_t K, int32_t dtype);
dsa_status dsa_index_scores_paged(const void* q_idx, const void* k_pool, const void* w, float* scores,
                                  const int64_t* seq_lens, const int32_t* block_table, int64_t B, int64_t Tq,
                                  int64_t max_blocks, int32_t block_size, int64_t num_blocks, int32_t H_I,
                                  int32_t D_I, int32_t dtype, void* stream);
dsa_status dsa_index_scores_fp8_paged(const uint8_t* q8, const float* q_scale, const uint8_t* k8_pool,
                                      const float* k_scale_pool, const void* w, float* scores,
                                      const int64_t* seq_lens, const int32_t* block_table, int64_t B, int64_t Tq,
                                      int64_t max_blocks, int32_t block_size, int64_t num_blocks, int32_t H_I,
                                      int32_t D_I, int32_t dtype, void* stream);
dsa_status dsa_sparse_mla_fwd_paged(const void* q, const void* kv_pool, const int32_t* idx, const int32_t* block_table,
                                    void* out, float* lse, int64_t B, int64_t Tq, int64_t max_blocks,
                                    int32_t block_size, int64_t num_blocks, int32_t H, int32_t D, int32_t DV, int32_t K,
                                    float scale, int32_t dtype, void* workspace, size_t ws_bytes, void* stream);
dsa_status dsa_forward_paged(const void* q_idx, const void* k_pool, const void* w, const void* q, const void* kv_pool,
                             void* out, float* lse, int32_t* idx_out, const int64_t* seq_lens,
                             const int32_t* block_table, int64_t B, int64_t Tq, int64_t max_blocks,
                             int32_t block_size, int64_t num_blocks, int32_t H_I, int32_t D_I, int32_t H, int32_t D,
                             int32_t DV, int32_t K, float scale, int32_t dtype, void* workspace, size_t ws_bytes,
                             void* stream);
dsa_status dsa_cache_append_paged(void* k_pool, void* kv_pool, const void* new_k_idx, const void* new_kv,
                                  const int64_t* pos, const int32_t* block_table, int64_t B, int64_t max_blocks,
                                  int32_t block_size, int64_t num_blocks, int32_t D_I, int32_t D, int32_t dtype,
                                  void* stream);

/*
 * Bandwidth calibration (not a step of the method): streams `bytes` of src
 * through the device once, as a read only (dst NULL) or as a copy into dst,
 * with 16-byte loads and stores, so that the HBM-bound kernels above can be
 * set against what a plain stream reaches on the same device.  src and dst:
 * device, 16-byte aligned, not overlapping; bytes a multiple of 16 (0 is a
 * no-op).  DSA_ERR_INVALID_ARG otherwise.
 */
dsa_status dsa_calib_stream(const void* src, void* dst, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */

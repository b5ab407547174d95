// C-ABI front end of the DSA forward library: argument validation, workspace
// planning and kernel launches.  The contract of every entry point is stated
// in include/dsa.h.  Validation is pure host code and runs before any HIP
// call, so a rejected call never touches the device.
#include "dsa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "launch.h"

namespace {

thread_local char g_last_error[512] = "";

dsa_status fail(dsa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

dsa_status ok() {
  g_last_error[0] = '\0';
  return DSA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kMaxN = 0x7fffffff;
constexpr int32_t kMaxK = 65536;
constexpr int64_t kMaxGrid = 0x7fffffff;

dsa_status check_common(int64_t B, int64_t Tq, int64_t N, int64_t q_pos0, int32_t dtype) {
  if (B < 1 || Tq < 1 || N < 1) return fail(DSA_ERR_INVALID_ARG, "B, Tq and N must be >= 1 (got %lld, %lld, %lld)",
                                            (long long)B, (long long)Tq, (long long)N);
  if (N > kMaxN) return fail(DSA_ERR_INVALID_ARG, "N must be < 2^31 (got %lld)", (long long)N);
  if (q_pos0 < 0) return fail(DSA_ERR_INVALID_ARG, "q_pos0 must be >= 0 (got %lld)", (long long)q_pos0);
  if (q_pos0 > kMaxN) return fail(DSA_ERR_INVALID_ARG, "q_pos0 must be < 2^31");
  if (B > 65535) return fail(DSA_ERR_INVALID_ARG, "B must be <= 65535 (got %lld)", (long long)B);
  if (B * Tq > kMaxGrid) return fail(DSA_ERR_INVALID_ARG, "B*Tq must be < 2^31");
  if (dtype != DSA_BF16 && dtype != DSA_F32) return fail(DSA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  return DSA_OK;
}

// Checks the indexer inputs; `scores` is checked only when check_scores is set
// (the fused entry point keeps its scores in the workspace).
dsa_status check_index_scores(const void* q_idx, const void* k_idx, const void* w, const float* scores, int64_t B,
                              int64_t Tq, int64_t N, int64_t q_pos0, int32_t H_I, int32_t D_I, int32_t dtype,
                              bool check_scores) {
  dsa_status st = check_common(B, Tq, N, q_pos0, dtype);
  if (st != DSA_OK) return st;
  if (!q_idx || !k_idx || !w || (check_scores && !scores)) return fail(DSA_ERR_INVALID_ARG, "null tensor pointer");
  if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned16(w) || (check_scores && !aligned16(scores)))
    return fail(DSA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  if (H_I < 1 || D_I < 1) return fail(DSA_ERR_INVALID_ARG, "H_I and D_I must be >= 1");
  if (dtype == DSA_BF16) {
    if (H_I != 64 || D_I != 128)
      return fail(DSA_ERR_UNSUPPORTED, "bf16 indexer is compiled for H_I=64, D_I=128 (got %d, %d)", H_I, D_I);
  } else {
    if (H_I > 64 || D_I > 256)
      return fail(DSA_ERR_UNSUPPORTED, "fp32 indexer supports H_I <= 64, D_I <= 256 (got %d, %d)", H_I, D_I);
    const int64_t chunks = (std::min<int64_t>(N, q_pos0 + Tq) + 255) / 256;
    if (B * Tq * chunks > kMaxGrid) return fail(DSA_ERR_UNSUPPORTED, "fp32 indexer problem too large");
  }
  return DSA_OK;
}

dsa_status check_topk(const float* scores, const int32_t* idx, int64_t B, int64_t Tq, int64_t N, int64_t q_pos0,
                      int32_t K, const void* workspace, size_t ws_bytes) {
  dsa_status st = check_common(B, Tq, N, q_pos0, DSA_F32);
  if (st != DSA_OK) return st;
  if (!scores || !idx) return fail(DSA_ERR_INVALID_ARG, "null tensor pointer");
  if (!aligned16(scores) || !aligned16(idx)) return fail(DSA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  if (K < 1 || K > kMaxK) return fail(DSA_ERR_INVALID_ARG, "K must be in [1, 65536] (got %d)", K);
  const size_t need = dsa::topk_workspace_bytes(B, Tq, N, K);
  if (need > 0 && (!workspace || ws_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "top-k workspace needs %zu bytes (got %zu)", need, ws_bytes);
  return DSA_OK;
}

// Checks the sparse-MLA arguments; `idx` and the workspace are checked only
// when check_idx_ws is set (the fused entry point produces both itself).
dsa_status check_mla(const void* q, const void* kv, const int32_t* idx, const void* out, const float* lse, int64_t B,
                     int64_t Tq, int64_t N, int32_t H, int32_t D, int32_t DV, int32_t K, float scale, int32_t dtype,
                     const void* workspace, size_t ws_bytes, bool check_idx_ws) {
  dsa_status st = check_common(B, Tq, N, 0, dtype);
  if (st != DSA_OK) return st;
  if (!q || !kv || (check_idx_ws && !idx) || !out) return fail(DSA_ERR_INVALID_ARG, "null tensor pointer");
  if (!aligned16(q) || !aligned16(kv) || (check_idx_ws && !aligned16(idx)) || !aligned16(out) ||
      (lse && !aligned16(lse)))
    return fail(DSA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  if (K < 1 || K > kMaxK) return fail(DSA_ERR_INVALID_ARG, "K must be in [1, 65536] (got %d)", K);
  if (H < 1 || D < 1 || DV < 1 || DV > D) return fail(DSA_ERR_INVALID_ARG, "need H, D >= 1 and 1 <= DV <= D");
  if (!(scale > 0.f) || scale != scale || scale > 3.0e38f)
    return fail(DSA_ERR_INVALID_ARG, "scale must be a finite positive number");
  if (dtype == DSA_BF16) {
    if (H != 128 || D != 576 || DV != 512)
      return fail(DSA_ERR_UNSUPPORTED, "bf16 sparse MLA is compiled for H=128, D=576, DV=512 (got %d, %d, %d)", H, D,
                  DV);
  } else {
    if (H > 128 || D > 1024 || DV > 512)
      return fail(DSA_ERR_UNSUPPORTED, "fp32 sparse MLA supports H <= 128, D <= 1024, DV <= 512");
    if (B * Tq * H > kMaxGrid) return fail(DSA_ERR_UNSUPPORTED, "fp32 sparse MLA problem too large");
  }
  if (check_idx_ws) {
    const size_t need = dsa::mla_workspace_bytes(B * Tq, H, DV, K, dtype == DSA_BF16);
    if (need > 0 && (!workspace || ws_bytes < need))
      return fail(DSA_ERR_WORKSPACE, "sparse MLA workspace needs %zu bytes (got %zu)", need, ws_bytes);
  }
  return DSA_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct ForwardLayout {
  size_t scores, idx, mla, total;
};

ForwardLayout forward_layout(int64_t B, int64_t Tq, int64_t N, int32_t H, int32_t DV, int32_t K, int32_t dtype) {
  ForwardLayout L;
  L.scores = 0;
  L.idx = align256((size_t)B * Tq * N * sizeof(float));
  L.mla = L.idx + align256((size_t)B * Tq * K * sizeof(int32_t));
  L.total = L.mla + align256(dsa::mla_workspace_bytes(B * Tq, H, DV, K, dtype == DSA_BF16));
  const size_t tk = dsa::topk_workspace_bytes(B, Tq, N, K);
  if (tk > 0) L.total += align256(tk);  // top-k scratch follows the MLA partials
  return L;
}

bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }

dsa_status check_seq_lens(const int64_t* seq_lens) {
  if (!seq_lens) return fail(DSA_ERR_INVALID_ARG, "seq_lens must not be null");
  if (!aligned8(seq_lens)) return fail(DSA_ERR_INVALID_ARG, "seq_lens must be 8-byte aligned");
  return DSA_OK;
}

dsa_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Checks the FP8 indexer inputs (codes, scales, bf16 head weights).
dsa_status check_index_scores_fp8(const uint8_t* q8, const float* qs, const uint8_t* k8, const float* ks,
                                  const void* w, const float* scores, int64_t B, int64_t Tq, int64_t N,
                                  int64_t q_pos0, int32_t H_I, int32_t D_I, int32_t dtype, bool check_scores) {
  dsa_status st = check_common(B, Tq, N, q_pos0, dtype);
  if (st != DSA_OK) return st;
  if (dtype != DSA_BF16) return fail(DSA_ERR_UNSUPPORTED, "the FP8 indexer takes bf16 head weights");
  if (!q8 || !qs || !k8 || !ks || !w || (check_scores && !scores)) return fail(DSA_ERR_INVALID_ARG, "null tensor pointer");
  if (!aligned16(q8) || !aligned16(qs) || !aligned16(k8) || !aligned16(ks) || !aligned16(w) ||
      (check_scores && !aligned16(scores)))
    return fail(DSA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  if (H_I != 64 || D_I != 128)
    return fail(DSA_ERR_UNSUPPORTED, "the FP8 indexer is compiled for H_I=64, D_I=128 (got %d, %d)", H_I, D_I);
  if (Tq > 65535) return fail(DSA_ERR_UNSUPPORTED, "the FP8 indexer takes at most 65535 queries per sequence");
  return DSA_OK;
}

// Checks a paged cache description and fills `pg`.
dsa_status check_paged(const int32_t* block_table, int64_t max_blocks, int32_t block_size, int64_t num_blocks,
                       dsa::Paged& pg) {
  if (!block_table) return fail(DSA_ERR_INVALID_ARG, "block_table must not be null");
  if ((reinterpret_cast<uintptr_t>(block_table) & 3u) != 0)
    return fail(DSA_ERR_INVALID_ARG, "block_table must be 4-byte aligned");
  if (block_size < 64 || block_size > (1 << 20) || (block_size & (block_size - 1)) != 0)
    return fail(DSA_ERR_UNSUPPORTED, "block_size must be a power of two in [64, 2^20] (got %d)", block_size);
  if (max_blocks < 1 || num_blocks < 1) return fail(DSA_ERR_INVALID_ARG, "max_blocks and num_blocks must be >= 1");
  if (max_blocks * (int64_t)block_size > kMaxN || num_blocks * (int64_t)block_size > kMaxN)
    return fail(DSA_ERR_INVALID_ARG, "max_blocks*block_size and num_blocks*block_size must be < 2^31");
  int shift = 0;
  while ((1 << shift) < block_size) ++shift;
  pg = dsa::Paged{block_table, max_blocks, shift, (int32_t)num_blocks};
  return DSA_OK;
}

// The paged sparse MLA: logical indices -> pool rows (into `phys`), then the
// gather kernel over the pool as one sequence of num_blocks * block_size rows.
dsa_status run_paged_mla(const void* q, const void* kv_pool, const int32_t* idx, int32_t* phys, void* out, float* lse,
                         int64_t B, int64_t Tq, int32_t K, float scale, const dsa::Paged& pg, void* mla_ws,
                         hipStream_t s) {
  hipError_t e = dsa::launch_page_translate(idx, phys, B, Tq, K, pg, s);
  if (e != hipSuccess) return hip_status(e, "page translate launch");
  e = dsa::launch_sparse_mla_bf16(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kv_pool), phys,
                                  static_cast<uint16_t*>(out), lse, 1, B * Tq, (int64_t)pg.num_blocks << pg.shift, K,
                                  scale, mla_ws, s);
  return hip_status(e, "sparse MLA launch");
}

constexpr int64_t kMaxGemmRows = 65535LL * 64;

dsa_status check_proj_common(const void* a, const void* b, const void* c, int64_t M, int32_t dtype) {
  if (dtype != DSA_BF16 && dtype != DSA_F32) return fail(DSA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (dtype != DSA_BF16) return fail(DSA_ERR_UNSUPPORTED, "the projections are built for bf16 only");
  if (!a || !b || !c) return fail(DSA_ERR_INVALID_ARG, "tensor pointers must not be null");
  if (!aligned16(a) || !aligned16(b) || !aligned16(c))
    return fail(DSA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  if (M < 0) return fail(DSA_ERR_INVALID_ARG, "M must be >= 0 (got %lld)", (long long)M);
  if (M > kMaxGemmRows) return fail(DSA_ERR_UNSUPPORTED, "M must be <= %lld", (long long)kMaxGemmRows);
  return DSA_OK;
}

// Whether the bf16 decode indexer (or with fp8 the FP8 one) leaves a
// pre-selection of each row for the top-k (see PreselWs): decode rows too long
// for the one-workgroup top-k.
bool presel_applies(int64_t B, int64_t Tq, int64_t N, int64_t nmax, int32_t K, int32_t dtype, dsa::PreselWs* ps,
                    bool fp8 = false) {
  if (dtype != DSA_BF16 || dsa::presel_workspace_bytes(B, Tq, N, K) == 0) return false;
  dsa::PreselWs g;
  if (!dsa::presel_geometry(B, Tq, N, nmax, K, g, fp8)) return false;
  if (ps) *ps = g;
  return true;
}

// Steps 1 and 2 of a bf16 forward: the indexer with the pre-selection and its
// top-k where it applies, else the plain indexer and top-k.
hipError_t index_and_topk_bf16(const void* q_idx, const void* k_idx, const void* w, float* scores, int32_t* idx,
                               int64_t B, int64_t Tq, int64_t N, int64_t q_pos0, int32_t K, void* topk_ws,
                               hipStream_t s, const int64_t* seq_lens = nullptr, const dsa::Paged* pg = nullptr) {
  const int64_t nmax = seq_lens != nullptr ? N : std::min(N, q_pos0 + Tq);
  const auto qi = static_cast<const uint16_t*>(q_idx);
  const auto ki = static_cast<const uint16_t*>(k_idx);
  const auto wi = static_cast<const uint16_t*>(w);
  hipError_t e;
  if (presel_applies(B, Tq, N, nmax, K, DSA_BF16, nullptr)) {
    const dsa::PreselWs ps = dsa::presel_ws(topk_ws, B, Tq, N, nmax, K);
    e = dsa::launch_index_scores_bf16(qi, ki, wi, scores, B, Tq, N, q_pos0, s, seq_lens, 1, pg, &ps);
    if (e != hipSuccess) return e;
    return dsa::launch_topk_presel(scores, idx, B, Tq, N, q_pos0, K, ps, s, seq_lens);
  }
  e = dsa::launch_index_scores_bf16(qi, ki, wi, scores, B, Tq, N, q_pos0, s, seq_lens, 1, pg);
  if (e != hipSuccess) return e;
  return dsa::launch_topk(scores, idx, B, Tq, N, q_pos0, K, topk_ws, s, seq_lens);
}

// Validation shared by the fused entry points (everything but the workspace).
dsa_status check_forward(const void* q_idx, const void* k_idx, const void* w, const void* q, const void* kv,
                         const void* out, const float* lse, const int32_t* idx_out, int64_t B, int64_t Tq, int64_t N,
                         int64_t q_pos0, int32_t H_I, int32_t D_I, int32_t H, int32_t D, int32_t DV, int32_t K,
                         float scale, int32_t dtype) {
  dsa_status st = check_index_scores(q_idx, k_idx, w, nullptr, B, Tq, N, q_pos0, H_I, D_I, dtype, false);
  if (st != DSA_OK) return st;
  st = check_mla(q, kv, nullptr, out, lse, B, Tq, N, H, D, DV, K, scale, dtype, nullptr, 0, false);
  if (st != DSA_OK) return st;
  if (idx_out && !aligned16(idx_out)) return fail(DSA_ERR_INVALID_ARG, "idx_out must be 16-byte aligned");
  return DSA_OK;
}

// Indexer -> top-k -> sparse MLA on one stream over a validated problem and a
// workspace of forward_layout(...).total bytes.
dsa_status run_forward(const void* q_idx, const void* k_idx, const void* w, const void* q, const void* kv, void* out,
                       float* lse, int32_t* idx_out, int64_t B, int64_t Tq, int64_t N, int64_t q_pos0, int32_t H_I,
                       int32_t D_I, int32_t H, int32_t D, int32_t DV, int32_t K, float scale, int32_t dtype,
                       void* workspace, hipStream_t s) {
  const ForwardLayout L = forward_layout(B, Tq, N, H, DV, K, dtype);
  char* ws = static_cast<char*>(workspace);
  float* scores = reinterpret_cast<float*>(ws + L.scores);
  int32_t* idx = idx_out ? idx_out : reinterpret_cast<int32_t*>(ws + L.idx);
  void* mla_ws = ws + L.mla;
  void* topk_ws = ws + L.total - align256(dsa::topk_workspace_bytes(B, Tq, N, K));

  hipError_t e;
  if (dtype == DSA_BF16) {
    e = index_and_topk_bf16(q_idx, k_idx, w, scores, idx, B, Tq, N, q_pos0, K, topk_ws, s);
    if (e != hipSuccess) return hip_status(e, "index scores / top-k launch");
  } else {
    e = dsa::launch_index_scores_f32(static_cast<const float*>(q_idx), static_cast<const float*>(k_idx),
                                     static_cast<const float*>(w), scores, B, Tq, N, q_pos0, H_I, D_I, s);
    if (e != hipSuccess) return hip_status(e, "index scores launch");
    e = dsa::launch_topk(scores, idx, B, Tq, N, q_pos0, K, topk_ws, s);
    if (e != hipSuccess) return hip_status(e, "top-k launch");
  }
  if (dtype == DSA_BF16)
    e = dsa::launch_sparse_mla_bf16(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kv), idx,
                                    static_cast<uint16_t*>(out), lse, B, Tq, N, K, scale, mla_ws, s);
  else
    e = dsa::launch_sparse_mla_f32(static_cast<const float*>(q), static_cast<const float*>(kv), idx,
                                   static_cast<float*>(out), lse, B, Tq, N, H, D, DV, K, scale, s);
  return hip_status(e, "sparse MLA launch");
}

}  // namespace

// Scratch of dsa_forward_noalloc: a file-scope device array, one copy per GPU
// the library runs on, held until the process ends.  In host code its name is
// only a stand-in for the symbol; the device address of each GPU's copy comes
// from hipGetSymbolAddress and is the only thing ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[DSA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the scratch copy of the device `stream` runs on, looked
// up once per device with that device current.
dsa_status scratch_of_stream_device(hipStream_t stream, void** ptr) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "finding the stream's device");
  if (dev < 0 || dev >= kMaxDevices) return fail(DSA_ERR_UNSUPPORTED, "device id %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return hip_status(e, "hipGetDevice");
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_status(e, "hipSetDevice");
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess && e2 != hipSuccess) e = e2;
    }
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return DSA_OK;
}

}  // namespace

extern "C" {

int dsa_version(void) { return 10000; }

const char* dsa_status_string(int status) {
  switch (status) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_INVALID_ARG: return "DSA_ERR_INVALID_ARG";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE";
    case DSA_ERR_HIP: return "DSA_ERR_HIP";
    default: return "DSA_ERR_UNKNOWN";
  }
}

const char* dsa_last_error(void) { return g_last_error; }

dsa_status dsa_index_scores(const void* q_idx, const void* k_idx, const void* w, float* scores, int64_t B,
                            int64_t Tq, int64_t N, int64_t q_pos0, int32_t H_I, int32_t D_I, int32_t dtype,
                            void* stream) {
  dsa_status st = check_index_scores(q_idx, k_idx, w, scores, B, Tq, N, q_pos0, H_I, D_I, dtype, true);
  if (st != DSA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (dtype == DSA_BF16)
    e = dsa::launch_index_scores_bf16(static_cast<const uint16_t*>(q_idx), static_cast<const uint16_t*>(k_idx),
                                      static_cast<const uint16_t*>(w), scores, B, Tq, N, q_pos0, s);
  else
    e = dsa::launch_index_scores_f32(static_cast<const float*>(q_idx), static_cast<const float*>(k_idx),
                                     static_cast<const float*>(w), scores, B, Tq, N, q_pos0, H_I, D_I, s);
  return hip_status(e, "index scores launch");
}

size_t dsa_topk_workspace_size(int64_t B, int64_t Tq, int64_t N, int32_t K) {
  if (B < 1 || Tq < 1 || N < 1 || K < 1) return 0;
  return dsa::topk_workspace_bytes(B, Tq, N, K);
}

dsa_status dsa_topk(const float* scores, int32_t* idx, int64_t B, int64_t Tq, int64_t N, int64_t q_pos0, int32_t K,
                    void* workspace, size_t ws_bytes, void* stream) {
  dsa_status st = check_topk(scores, idx, B, Tq, N, q_pos0, K, workspace, ws_bytes);
  if (st != DSA_OK) return st;
  return hip_status(dsa::launch_topk(scores, idx, B, Tq, N, q_pos0, K, workspace, static_cast<hipStream_t>(stream)),
                    "top-k launch");
}

dsa_status dsa_index_scores_presel(const void* q_idx, const void* k_idx, const void* w, float* scores, int64_t B,
                                   int64_t Tq, int64_t N, int64_t q_pos0, int32_t H_I, int32_t D_I, int32_t K,
                                   int32_t dtype, void* workspace, size_t ws_bytes, void* stream) {
  dsa_status st = check_index_scores(q_idx, k_idx, w, scores, B, Tq, N, q_pos0, H_I, D_I, dtype, true);
  if (st != DSA_OK) return st;
  if (K < 1 || K > kMaxK) return fail(DSA_ERR_INVALID_ARG, "K must be in [1, 65536] (got %d)", K);
  const size_t need = dsa::topk_workspace_bytes(B, Tq, N, K);
  if (need > 0 && (!workspace || ws_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "top-k workspace needs %zu bytes (got %zu)", need, ws_bytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t nmax = std::min(N, q_pos0 + Tq);
  hipError_t e;
  if (presel_applies(B, Tq, N, nmax, K, dtype, nullptr)) {
    const dsa::PreselWs ps = dsa::presel_ws(workspace, B, Tq, N, nmax, K);
    e = dsa::launch_index_scores_bf16(static_cast<const uint16_t*>(q_idx), static_cast<const uint16_t*>(k_idx),
                                      static_cast<const uint16_t*>(w), scores, B, Tq, N, q_pos0, s, nullptr, 1,
                                      nullptr, &ps);
  } else if (dtype == DSA_BF16) {
    e = dsa::launch_index_scores_bf16(static_cast<const uint16_t*>(q_idx), static_cast<const uint16_t*>(k_idx),
                                      static_cast<const uint16_t*>(w), scores, B, Tq, N, q_pos0, s);
  } else {
    e = dsa::launch_index_scores_f32(static_cast<const float*>(q_idx), static_cast<const float*>(k_idx),
                                     static_cast<const float*>(w), scores, B, Tq, N, q_pos0, H_I, D_I, s);
  }
  return hip_status(e, "index scores launch");
}

dsa_status dsa_topk_presel(const float* scores, int32_t* idx, int64_t B, int64_t Tq, int64_t N, int64_t q_pos0,
                           int32_t K, int32_t dtype, void* workspace, size_t ws_bytes, void* stream) {
  dsa_status st = check_topk(scores, idx, B, Tq, N, q_pos0, K, workspace, ws_bytes);
  if (st != DSA_OK) return st;
  if (dtype != DSA_BF16 && dtype != DSA_F32) return fail(DSA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t nmax = std::min(N, q_pos0 + Tq);
  if (presel_applies(B, Tq, N, nmax, K, dtype, nullptr))
    return hip_status(dsa::launch_topk_presel(scores, idx, B, Tq, N, q_pos0, K,
                                              dsa::presel_ws(workspace, B, Tq, N, nmax, K), s),
                      "top-k launch");
  return hip_status(dsa::launch_topk(scores, idx, B, Tq, N, q_pos0, K, workspace, s), "top-k launch");
}

size_t dsa_sparse_mla_workspace_size(int64_t B, int64_t Tq, int32_t H, int32_t DV, int32_t K, int32_t dtype) {
  if (B < 1 || Tq < 1 || H < 1 || DV < 1 || K < 1) return 0;
  return dsa::mla_workspace_bytes(B * Tq, H, DV, K, dtype == DSA_BF16);
}

dsa_status dsa_sparse_mla_fwd(const void* q, const void* kv, const int32_t* idx, void* out, float* lse, int64_t B,
                              int64_t Tq, int64_t N, int32_t H, int32_t D, int32_t DV, int32_t K, float scale,
                              int32_t dtype, void* workspace, size_t ws_bytes, void* stream) {
  dsa_status st = check_mla(q, kv, idx, out, lse, B, Tq, N, H, D, DV, K, scale, dtype, workspace, ws_bytes, true);
  if (st != DSA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (dtype == DSA_BF16)
    e = dsa::launch_sparse_mla_bf16(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kv), idx,
                                    static_cast<uint16_t*>(out), lse, B, Tq, N, K, scale, workspace, s);
  else
    e = dsa::launch_sparse_mla_f32(static_cast<const float*>(q), static_cast<const float*>(kv), idx,
                                   static_cast<float*>(out), lse, B, Tq, N, H, D, DV, K, scale, s);
  return hip_status(e, "sparse MLA launch");
}

size_t dsa_forward_workspace_size(int64_t B, int64_t Tq, int64_t N, int32_t H, int32_t DV, int32_t K,
                                  int32_t dtype) {
  if (B < 1 || Tq < 1 || N < 1 || H < 1 || DV < 1 || K < 1) return 0;
  return forward_layout(B, Tq, N, H, DV, K, dtype).total;
}

dsa_status dsa_forward(const void* q_idx, const void* k_idx, const void* w, const void* q, const void* kv, void* out,
                       float* lse, int32_t* idx_out, int64_t B, int64_t Tq, int64_t N, int64_t q_pos0, int32_t H_I,
                       int32_t D_I, int32_t H, int32_t D, int32_t DV, int32_t K, float scale, int32_t dtype,
                       void* workspace, size_t ws_bytes, void* stream) {
  dsa_status st = check_forward(q_idx, k_idx, w, q, kv, out, lse, idx_out, B, Tq, N, q_pos0, H_I, D_I, H, D, DV, K,
                                scale, dtype);
  if (st != DSA_OK) return st;
  const size_t need = forward_layout(B, Tq, N, H, DV, K, dtype).total;
  if (!workspace || ws_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "forward workspace needs %zu bytes (got %zu)", need, ws_bytes);
  if (!aligned16(workspace)) return fail(DSA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  return run_forward(q_idx, k_idx, w, q, kv, out, lse, idx_out, B, Tq, N, q_pos0, H_I, D_I, H, D, DV, K, scale, dtype,
                     workspace, static_cast<hipStream_t>(stream));
}

dsa_status dsa_forward_noalloc(const void* q_idx, const void* k_idx, const void* w, const void* q, const void* kv,
                               void* out, float* lse, int32_t* idx_out, int64_t B, int64_t Tq, int64_t N,
                               int64_t q_pos0, int32_t H_I, int32_t D_I, int32_t H, int32_t D, int32_t DV, int32_t K,
                               float scale, int32_t dtype, void* stream) {
  dsa_status st = check_forward(q_idx, k_idx, w, q, kv, out, lse, idx_out, B, Tq, N, q_pos0, H_I, D_I, H, D, DV, K,
                                scale, dtype);
  if (st != DSA_OK) return st;
  const size_t need = forward_layout(B, Tq, N, H, DV, K, dtype).total;
  if (need > (size_t)DSA_NOALLOC_SCRATCH_BYTES)
    return fail(DSA_ERR_WORKSPACE, "this problem needs %zu bytes of scratch; dsa_forward_noalloc holds at most %zu "
                "(use dsa_forward with a workspace)", need, (size_t)DSA_NOALLOC_SCRATCH_BYTES);
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if ((st = scratch_of_stream_device(s, &ws)) != DSA_OK) return st;
  return run_forward(q_idx, k_idx, w, q, kv, out, lse, idx_out, B, Tq, N, q_pos0, H_I, D_I, H, D, DV, K, scale, dtype,
                     ws, s);
}

dsa_status dsa_index_scores_varlen(const void* q_idx, const void* k_idx, const void* w, float* scores,
                                   const int64_t* seq_lens, int64_t B, int64_t Tq, int64_t N, int32_t H_I,
                                   int32_t D_I, int32_t dtype, void* stream) {
  dsa_status st = check_index_scores(q_idx, k_idx, w, scores, B, Tq, N, 0, H_I, D_I, dtype, true);
  if (st != DSA_OK) return st;
  if ((st = check_seq_lens(seq_lens)) != DSA_OK) return st;
  if (dtype == DSA_F32 && B * Tq * ((N + 255) / 256) > kMaxGrid)
    return fail(DSA_ERR_UNSUPPORTED, "fp32 indexer problem too large");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (dtype == DSA_BF16)
    e = dsa::launch_index_scores_bf16(static_cast<const uint16_t*>(q_idx), static_cast<const uint16_t*>(k_idx),
                                      static_cast<const uint16_t*>(w), scores, B, Tq, N, 0, s, seq_lens);
  else
    e = dsa::launch_index_scores_f32(static_cast<const float*>(q_idx), static_cast<const float*>(k_idx),
                                     static_cast<const float*>(w), scores, B, Tq, N, 0, H_I, D_I, s, seq_lens);
  return hip_status(e, "index scores launch");
}

dsa_status dsa_topk_varlen(const float* scores, int32_t* idx, const int64_t* seq_lens, int64_t B, int64_t Tq,
                           int64_t N, int32_t K, void* workspace, size_t ws_bytes, void* stream) {
  dsa_status st = check_topk(scores, idx, B, Tq, N, 0, K, workspace, ws_bytes);
  if (st != DSA_OK) return st;
  if ((st = check_seq_lens(seq_lens)) != DSA_OK) return st;
  return hip_status(dsa::launch_topk(scores, idx, B, Tq, N, 0, K, workspace, static_cast<hipStream_t>(stream),
                                     seq_lens),
                    "top-k launch");
}

dsa_status dsa_forward_varlen(const void* q_idx, const void* k_idx, const void* w, const void* q, const void* kv,
                              void* out, float* lse, int32_t* idx_out, const int64_t* seq_lens, int64_t B,
                              int64_t Tq, int64_t N, int32_t H_I, int32_t D_I, int32_t H, int32_t D, int32_t DV,
                              int32_t K, float scale, int32_t dtype, void* workspace, size_t ws_bytes,
                              void* stream) {
  dsa_status st = check_index_scores(q_idx, k_idx, w, nullptr, B, Tq, N, 0, H_I, D_I, dtype, false);
  if (st != DSA_OK) return st;
  if (dtype == DSA_F32 && B * Tq * ((N + 255) / 256) > kMaxGrid)
    return fail(DSA_ERR_UNSUPPORTED, "fp32 indexer problem too large");
  st = check_mla(q, kv, nullptr, out, lse, B, Tq, N, H, D, DV, K, scale, dtype, nullptr, 0, false);
  if (st != DSA_OK) return st;
  if ((st = check_seq_lens(seq_lens)) != DSA_OK) return st;
  if (idx_out && !aligned16(idx_out)) return fail(DSA_ERR_INVALID_ARG, "idx_out must be 16-byte aligned");
  const ForwardLayout L = forward_layout(B, Tq, N, H, DV, K, dtype);
  if (!workspace || ws_bytes < L.total)
    return fail(DSA_ERR_WORKSPACE, "forward workspace needs %zu bytes (got %zu)", L.total, ws_bytes);
  if (!aligned16(workspace)) return fail(DSA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");

  char* ws = static_cast<char*>(workspace);
  float* scores = reinterpret_cast<float*>(ws + L.scores);
  int32_t* idx = idx_out ? idx_out : reinterpret_cast<int32_t*>(ws + L.idx);
  void* mla_ws = ws + L.mla;
  void* topk_ws = ws + L.total - align256(dsa::topk_workspace_bytes(B, Tq, N, K));
  hipStream_t s = static_cast<hipStream_t>(stream);

  hipError_t e;
  if (dtype == DSA_BF16) {
    e = index_and_topk_bf16(q_idx, k_idx, w, scores, idx, B, Tq, N, 0, K, topk_ws, s, seq_lens);
    if (e != hipSuccess) return hip_status(e, "index scores / top-k launch");
  } else {
    e = dsa::launch_index_scores_f32(static_cast<const float*>(q_idx), static_cast<const float*>(k_idx),
                                     static_cast<const float*>(w), scores, B, Tq, N, 0, H_I, D_I, s, seq_lens);
    if (e != hipSuccess) return hip_status(e, "index scores launch");
    e = dsa::launch_topk(scores, idx, B, Tq, N, 0, K, topk_ws, s, seq_lens);
    if (e != hipSuccess) return hip_status(e, "top-k launch");
  }
  if (dtype == DSA_BF16)
    e = dsa::launch_sparse_mla_bf16(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kv), idx,
                                    static_cast<uint16_t*>(out), lse, B, Tq, N, K, scale, mla_ws, s);
  else
    e = dsa::launch_sparse_mla_f32(static_cast<const float*>(q), static_cast<const float*>(kv), idx,
                                   static_cast<float*>(out), lse, B, Tq, N, H, D, DV, K, scale, s);
  return hip_status(e, "sparse MLA launch");
}

dsa_status dsa_index_scores_compressed(const void* q_idx, const void* k_idx, const void* w, float* scores,
                                       int64_t B, int64_t Tq, int64_t N, int64_t q_pos0, int32_t m, int32_t H_I,
                                       int32_t D_I, int32_t dtype, void* stream) {
  dsa_status st = check_index_scores(q_idx, k_idx, w, scores, B, Tq, N, q_pos0, H_I, D_I, dtype, true);
  if (st != DSA_OK) return st;
  if (m < 1) return fail(DSA_ERR_INVALID_ARG, "the compression rate m must be >= 1 (got %d)", m);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (dtype == DSA_BF16)
    e = dsa::launch_index_scores_bf16(static_cast<const uint16_t*>(q_idx), static_cast<const uint16_t*>(k_idx),
                                      static_cast<const uint16_t*>(w), scores, B, Tq, N, q_pos0, s, nullptr, m);
  else
    e = dsa::launch_index_scores_f32(static_cast<const float*>(q_idx), static_cast<const float*>(k_idx),
                                     static_cast<const float*>(w), scores, B, Tq, N, q_pos0, H_I, D_I, s, nullptr,
                                     m);
  return hip_status(e, "index scores launch");
}

dsa_status dsa_topk_compressed(const float* scores, int32_t* idx, int64_t B, int64_t Tq, int64_t N,
                               int64_t q_pos0, int32_t m, int32_t K, void* workspace, size_t ws_bytes,
                               void* stream) {
  dsa_status st = check_topk(scores, idx, B, Tq, N, q_pos0, K, workspace, ws_bytes);
  if (st != DSA_OK) return st;
  if (m < 1) return fail(DSA_ERR_INVALID_ARG, "the compression rate m must be >= 1 (got %d)", m);
  return hip_status(dsa::launch_topk(scores, idx, B, Tq, N, q_pos0, K, workspace, static_cast<hipStream_t>(stream),
                                     nullptr, m),
                    "top-k launch");
}

dsa_status dsa_index_scores_compressed_presel(const void* q_idx, const void* k_idx, const void* w, float* scores,
                                              int64_t B, int64_t Tq, int64_t N, int64_t q_pos0, int32_t m,
                                              int32_t H_I, int32_t D_I, int32_t K, int32_t dtype, void* workspace,
                                              size_t ws_bytes, void* stream) {
  dsa_status st = check_index_scores(q_idx, k_idx, w, scores, B, Tq, N, q_pos0, H_I, D_I, dtype, true);
  if (st != DSA_OK) return st;
  if (m < 1) return fail(DSA_ERR_INVALID_ARG, "the compression rate m must be >= 1 (got %d)", m);
  if (K < 1 || K > kMaxK) return fail(DSA_ERR_INVALID_ARG, "K must be in [1, 65536] (got %d)", K);
  const size_t need = dsa::topk_workspace_bytes(B, Tq, N, K);
  if (need > 0 && (!workspace || ws_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "top-k workspace needs %zu bytes (got %zu)", need, ws_bytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t nmax = std::min(N, (q_pos0 + Tq) / m);
  if (presel_applies(B, Tq, N, nmax, K, dtype, nullptr)) {
    const dsa::PreselWs ps = dsa::presel_ws(workspace, B, Tq, N, nmax, K);
    return hip_status(dsa::launch_index_scores_bf16(static_cast<const uint16_t*>(q_idx),
                                                    static_cast<const uint16_t*>(k_idx),
                                                    static_cast<const uint16_t*>(w), scores, B, Tq, N, q_pos0, s,
                                                    nullptr, m, nullptr, &ps),
                      "index scores launch");
  }
  return dsa_index_scores_compressed(q_idx, k_idx, w, scores, B, Tq, N, q_pos0, m, H_I, D_I, dtype, stream);
}

dsa_status dsa_topk_compressed_presel(const float* scores, int32_t* idx, int64_t B, int64_t Tq, int64_t N,
                                      int64_t q_pos0, int32_t m, int32_t K, int32_t dtype, void* workspace,
                                      size_t ws_bytes, void* stream) {
  dsa_status st = check_topk(scores, idx, B, Tq, N, q_pos0, K, workspace, ws_bytes);
  if (st != DSA_OK) return st;
  if (m < 1) return fail(DSA_ERR_INVALID_ARG, "the compression rate m must be >= 1 (got %d)", m);
  if (dtype != DSA_BF16 && dtype != DSA_F32) return fail(DSA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t nmax = std::min(N, (q_pos0 + Tq) / m);
  if (presel_applies(B, Tq, N, nmax, K, dtype, nullptr))
    return hip_status(dsa::launch_topk_presel(scores, idx, B, Tq, N, q_pos0, K,
                                              dsa::presel_ws(workspace, B, Tq, N, nmax, K), s, nullptr, m),
                      "top-k launch");
  return hip_status(dsa::launch_topk(scores, idx, B, Tq, N, q_pos0, K, workspace, s, nullptr, m), "top-k launch");
}

dsa_status dsa_cache_append(void* k_idx, void* kv, const void* new_k_idx, const void* new_kv, const int64_t* pos,
                            int64_t B, int64_t N, int32_t D_I, int32_t D, int32_t dtype, void* stream) {
  if (B < 1 || N < 1) return fail(DSA_ERR_INVALID_ARG, "B and N must be >= 1 (got %lld, %lld)", (long long)B,
                                  (long long)N);
  if (N > kMaxN) return fail(DSA_ERR_INVALID_ARG, "N must be < 2^31 (got %lld)", (long long)N);
  if (B > kMaxGrid) return fail(DSA_ERR_INVALID_ARG, "B must be < 2^31");
  if (dtype != DSA_BF16 && dtype != DSA_F32) return fail(DSA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (!pos) return fail(DSA_ERR_INVALID_ARG, "pos must not be null");
  if (!aligned8(pos)) return fail(DSA_ERR_INVALID_ARG, "pos must be 8-byte aligned");
  if ((k_idx == nullptr) != (new_k_idx == nullptr) || (kv == nullptr) != (new_kv == nullptr))
    return fail(DSA_ERR_INVALID_ARG, "a cache and its new rows must be given together");
  if (!k_idx && !kv) return fail(DSA_ERR_INVALID_ARG, "no cache to append to");
  if ((k_idx && (!aligned16(k_idx) || !aligned16(new_k_idx))) || (kv && (!aligned16(kv) || !aligned16(new_kv))))
    return fail(DSA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  if ((k_idx && D_I < 1) || (kv && D < 1)) return fail(DSA_ERR_INVALID_ARG, "row widths must be >= 1");
  return hip_status(dsa::launch_cache_append(k_idx, kv, new_k_idx, new_kv, pos, B, N, k_idx ? D_I : 0, kv ? D : 0,
                                             dtype == DSA_BF16 ? 2 : 4, static_cast<hipStream_t>(stream)),
                    "cache append launch");
}

dsa_status dsa_mla_absorb_q(const void* q, const void* w_uk, void* q_lat, int64_t M, int32_t H, int32_t d_nope,
                            int32_t d_rope, int32_t d_c, int32_t dtype, void* stream) {
  dsa_status st = check_proj_common(q, w_uk, q_lat, M, dtype);
  if (st != DSA_OK) return st;
  if (H < 1 || H > 65535) return fail(DSA_ERR_INVALID_ARG, "H must be in [1, 65535] (got %d)", H);
  if (d_nope < 32 || d_nope % 32) return fail(DSA_ERR_UNSUPPORTED, "d_nope must be a positive multiple of 32");
  if (d_c < 8 || d_c % 8) return fail(DSA_ERR_UNSUPPORTED, "d_c must be a positive multiple of 8");
  if (d_rope < 0 || d_rope % 8) return fail(DSA_ERR_UNSUPPORTED, "d_rope must be a multiple of 8 (0 allowed)");
  const int64_t dq = (int64_t)d_nope + d_rope, dl = (int64_t)d_c + d_rope;
  const uint16_t* qp = static_cast<const uint16_t*>(q);
  uint16_t* lp = static_cast<uint16_t*>(q_lat);
  dsa::GemmArgs g{qp, H * dq, dq, static_cast<const uint16_t*>(w_uk), d_c, (int64_t)d_nope * d_c, lp, H * dl, dl,
                  M, d_c, d_nope, d_rope ? qp + d_nope : nullptr, H * dq, dq, d_rope ? lp + d_c : nullptr, H * dl,
                  dl, d_rope};
  return hip_status(dsa::launch_gemm_bf16(g, false, H, static_cast<hipStream_t>(stream)), "absorption launch");
}

dsa_status dsa_mla_out_proj(const void* o_lat, const void* w_uv, void* o, int64_t M, int32_t H, int32_t d_c,
                            int32_t d_v, int32_t dtype, void* stream) {
  dsa_status st = check_proj_common(o_lat, w_uv, o, M, dtype);
  if (st != DSA_OK) return st;
  if (H < 1 || H > 65535) return fail(DSA_ERR_INVALID_ARG, "H must be in [1, 65535] (got %d)", H);
  if (d_c < 32 || d_c % 32) return fail(DSA_ERR_UNSUPPORTED, "d_c must be a positive multiple of 32");
  if (d_v < 1) return fail(DSA_ERR_INVALID_ARG, "d_v must be >= 1");
  dsa::GemmArgs g{static_cast<const uint16_t*>(o_lat), (int64_t)H * d_c, d_c, static_cast<const uint16_t*>(w_uv),
                  d_c, (int64_t)d_v * d_c, static_cast<uint16_t*>(o), (int64_t)H * d_v, d_v, M, d_v, d_c,
                  nullptr, 0, 0, nullptr, 0, 0, 0};
  return hip_status(dsa::launch_gemm_bf16(g, true, H, static_cast<hipStream_t>(stream)), "output projection launch");
}

dsa_status dsa_linear(const void* x, const void* w, void* y, int64_t M, int32_t N, int32_t K, int32_t dtype,
                      void* stream) {
  dsa_status st = check_proj_common(x, w, y, M, dtype);
  if (st != DSA_OK) return st;
  if (N < 1) return fail(DSA_ERR_INVALID_ARG, "N must be >= 1");
  if (K < 32 || K % 32) return fail(DSA_ERR_UNSUPPORTED, "K must be a positive multiple of 32");
  dsa::GemmArgs g{static_cast<const uint16_t*>(x), K, 0, static_cast<const uint16_t*>(w), K, 0,
                  static_cast<uint16_t*>(y), N, 0, M, N, K, nullptr, 0, 0, nullptr, 0, 0, 0};
  return hip_status(dsa::launch_gemm_bf16(g, true, 1, static_cast<hipStream_t>(stream)), "linear launch");
}

dsa_status dsa_indexer_quantize_fp8(const void* x, uint8_t* codes, float* scales, int64_t R, int32_t D,
                                    int32_t dtype, void* stream) {
  if (dtype != DSA_BF16 && dtype != DSA_F32) return fail(DSA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (dtype != DSA_BF16) return fail(DSA_ERR_UNSUPPORTED, "FP8 quantisation takes bf16 rows");
  if (D != 128) return fail(DSA_ERR_UNSUPPORTED, "FP8 quantisation is compiled for rows of 128 (got %d)", D);
  if (R < 0) return fail(DSA_ERR_INVALID_ARG, "R must be >= 0 (got %lld)", (long long)R);
  if (!x || !codes || !scales) return fail(DSA_ERR_INVALID_ARG, "null tensor pointer");
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales))
    return fail(DSA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  return hip_status(dsa::launch_quantize_fp8(static_cast<const uint16_t*>(x), codes, scales, R,
                                             static_cast<hipStream_t>(stream)),
                    "FP8 quantisation launch");
}

dsa_status dsa_index_scores_fp8(const uint8_t* q8, const float* q_scale, const uint8_t* k8, const float* k_scale,
                                const void* w, float* scores, int64_t B, int64_t Tq, int64_t N, int64_t q_pos0,
                                int32_t H_I, int32_t D_I, int32_t dtype, void* stream) {
  dsa_status st = check_index_scores_fp8(q8, q_scale, k8, k_scale, w, scores, B, Tq, N, q_pos0, H_I, D_I, dtype, true);
  if (st != DSA_OK) return st;
  return hip_status(dsa::launch_index_scores_fp8(q8, q_scale, k8, k_scale, static_cast<const uint16_t*>(w), scores,
                                                 B, Tq, N, q_pos0, static_cast<hipStream_t>(stream)),
                    "FP8 index scores launch");
}

namespace {

// Steps 1 and 2 with the FP8 indexer, as the fused FP8 forward runs them: the
// indexer also lists each segment's best keys where the FP8 geometry admits a
// pre-selection, and the top-k then selects among the lists; else the plain
// indexer and top-k.  topk_ws: dsa::topk_workspace_bytes(B, Tq, N, K) bytes.
hipError_t index_fp8_presel(const uint8_t* q8, const float* qs, const uint8_t* k8, const float* ks, const void* w,
                            float* scores, int64_t B, int64_t Tq, int64_t N, int64_t q_pos0, int32_t K,
                            void* topk_ws, hipStream_t s) {
  const auto wi = static_cast<const uint16_t*>(w);
  const int64_t nmax = std::min(N, q_pos0 + Tq);
  if (presel_applies(B, Tq, N, nmax, K, DSA_BF16, nullptr, true)) {
    const dsa::PreselWs ps = dsa::presel_ws(topk_ws, B, Tq, N, nmax, K, true);
    return dsa::launch_index_scores_fp8(q8, qs, k8, ks, wi, scores, B, Tq, N, q_pos0, s, nullptr, nullptr, &ps);
  }
  return dsa::launch_index_scores_fp8(q8, qs, k8, ks, wi, scores, B, Tq, N, q_pos0, s);
}
hipError_t topk_fp8_presel(const float* scores, int32_t* idx, int64_t B, int64_t Tq, int64_t N, int64_t q_pos0,
                           int32_t K, void* topk_ws, hipStream_t s) {
  const int64_t nmax = std::min(N, q_pos0 + Tq);
  if (presel_applies(B, Tq, N, nmax, K, DSA_BF16, nullptr, true))
    return dsa::launch_topk_presel(scores, idx, B, Tq, N, q_pos0, K, dsa::presel_ws(topk_ws, B, Tq, N, nmax, K, true),
                                   s);
  return dsa::launch_topk(scores, idx, B, Tq, N, q_pos0, K, topk_ws, s);
}

}  // namespace

dsa_status dsa_index_scores_fp8_presel(const uint8_t* q8, const float* q_scale, const uint8_t* k8,
                                       const float* k_scale, const void* w, float* scores, int64_t B, int64_t Tq,
                                       int64_t N, int64_t q_pos0, int32_t H_I, int32_t D_I, int32_t K, int32_t dtype,
                                       void* workspace, size_t ws_bytes, void* stream) {
  dsa_status st = check_index_scores_fp8(q8, q_scale, k8, k_scale, w, scores, B, Tq, N, q_pos0, H_I, D_I, dtype, true);
  if (st != DSA_OK) return st;
  if (K < 1 || K > kMaxK) return fail(DSA_ERR_INVALID_ARG, "K must be in [1, 65536] (got %d)", K);
  const size_t need = dsa::topk_workspace_bytes(B, Tq, N, K);
  if (need > 0 && (!workspace || ws_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "top-k workspace needs %zu bytes (got %zu)", need, ws_bytes);
  return hip_status(index_fp8_presel(q8, q_scale, k8, k_scale, w, scores, B, Tq, N, q_pos0, K, workspace,
                                     static_cast<hipStream_t>(stream)),
                    "FP8 index scores launch");
}

dsa_status dsa_topk_presel_fp8(const float* scores, int32_t* idx, int64_t B, int64_t Tq, int64_t N, int64_t q_pos0,
                               int32_t K, void* workspace, size_t ws_bytes, void* stream) {
  dsa_status st = check_topk(scores, idx, B, Tq, N, q_pos0, K, workspace, ws_bytes);
  if (st != DSA_OK) return st;
  return hip_status(topk_fp8_presel(scores, idx, B, Tq, N, q_pos0, K, workspace, static_cast<hipStream_t>(stream)),
                    "top-k launch");
}

dsa_status dsa_forward_fp8(const uint8_t* q8, const float* q_scale, const uint8_t* k8, const float* k_scale,
                           const void* w, const void* q, const void* kv, void* out, float* lse, int32_t* idx_out,
                           int64_t B, int64_t Tq, int64_t N, int64_t q_pos0, int32_t H_I, int32_t D_I, int32_t H,
                           int32_t D, int32_t DV, int32_t K, float scale, int32_t dtype, void* workspace,
                           size_t ws_bytes, void* stream) {
  dsa_status st =
      check_index_scores_fp8(q8, q_scale, k8, k_scale, w, nullptr, B, Tq, N, q_pos0, H_I, D_I, dtype, false);
  if (st != DSA_OK) return st;
  st = check_mla(q, kv, nullptr, out, lse, B, Tq, N, H, D, DV, K, scale, dtype, nullptr, 0, false);
  if (st != DSA_OK) return st;
  if (idx_out && !aligned16(idx_out)) return fail(DSA_ERR_INVALID_ARG, "idx_out must be 16-byte aligned");
  const ForwardLayout L = forward_layout(B, Tq, N, H, DV, K, dtype);
  if (!workspace || ws_bytes < L.total)
    return fail(DSA_ERR_WORKSPACE, "forward workspace needs %zu bytes (got %zu)", L.total, ws_bytes);
  if (!aligned16(workspace)) return fail(DSA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  char* ws = static_cast<char*>(workspace);
  float* scores = reinterpret_cast<float*>(ws + L.scores);
  int32_t* idx = idx_out ? idx_out : reinterpret_cast<int32_t*>(ws + L.idx);
  void* topk_ws = ws + L.total - align256(dsa::topk_workspace_bytes(B, Tq, N, K));
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = index_fp8_presel(q8, q_scale, k8, k_scale, w, scores, B, Tq, N, q_pos0, K, topk_ws, s);
  if (e != hipSuccess) return hip_status(e, "FP8 index scores launch");
  e = topk_fp8_presel(scores, idx, B, Tq, N, q_pos0, K, topk_ws, s);
  if (e != hipSuccess) return hip_status(e, "top-k launch");
  e = dsa::launch_sparse_mla_bf16(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kv), idx,
                                  static_cast<uint16_t*>(out), lse, B, Tq, N, K, scale, ws + L.mla, s);
  return hip_status(e, "sparse MLA launch");
}

size_t dsa_paged_workspace_size(int64_t B, int64_t Tq, int64_t max_blocks, int32_t block_size, int32_t H,
                                int32_t DV, int32_t K, int32_t dtype) {
  if (B < 1 || Tq < 1 || max_blocks < 1 || block_size < 1 || H < 1 || DV < 1 || K < 1) return 0;
  return forward_layout(B, Tq, max_blocks * (int64_t)block_size, H, DV, K, dtype).total +
         align256((size_t)B * Tq * K * sizeof(int32_t));
}

dsa_status dsa_index_scores_paged(const void* q_idx, const void* k_pool, const void* w, float* scores,
                                  const int64_t* seq_lens, const int32_t* block_table, int64_t B, int64_t Tq,
                                  int64_t max_blocks, int32_t block_size, int64_t num_blocks, int32_t H_I,
                                  int32_t D_I, int32_t dtype, void* stream) {
  dsa::Paged pg;
  dsa_status st = check_paged(block_table, max_blocks, block_size, num_blocks, pg);
  if (st != DSA_OK) return st;
  const int64_t N = max_blocks * (int64_t)block_size;
  if ((st = check_index_scores(q_idx, k_pool, w, scores, B, Tq, N, 0, H_I, D_I, dtype, true)) != DSA_OK) return st;
  if ((st = check_seq_lens(seq_lens)) != DSA_OK) return st;
  if (dtype != DSA_BF16) return fail(DSA_ERR_UNSUPPORTED, "paged caches are built for bf16 only");
  if (Tq > 4) return fail(DSA_ERR_UNSUPPORTED, "paged caches are built for decode shapes (Tq <= 4, got %lld)",
                          (long long)Tq);
  return hip_status(dsa::launch_index_scores_bf16(static_cast<const uint16_t*>(q_idx),
                                                  static_cast<const uint16_t*>(k_pool), static_cast<const uint16_t*>(w),
                                                  scores, B, Tq, N, 0, static_cast<hipStream_t>(stream), seq_lens, 1,
                                                  &pg),
                    "paged index scores launch");
}

dsa_status dsa_index_scores_fp8_paged(const uint8_t* q8, const float* q_scale, const uint8_t* k8_pool,
                                      const float* k_scale_pool, const void* w, float* scores,
                                      const int64_t* seq_lens, const int32_t* block_table, int64_t B, int64_t Tq,
                                      int64_t max_blocks, int32_t block_size, int64_t num_blocks, int32_t H_I,
                                      int32_t D_I, int32_t dtype, void* stream) {
  dsa::Paged pg;
  dsa_status st = check_paged(block_table, max_blocks, block_size, num_blocks, pg);
  if (st != DSA_OK) return st;
  const int64_t N = max_blocks * (int64_t)block_size;
  st = check_index_scores_fp8(q8, q_scale, k8_pool, k_scale_pool, w, scores, B, Tq, N, 0, H_I, D_I, dtype, true);
  if (st != DSA_OK) return st;
  if ((st = check_seq_lens(seq_lens)) != DSA_OK) return st;
  if (Tq > 4) return fail(DSA_ERR_UNSUPPORTED, "paged caches are built for decode shapes (Tq <= 4, got %lld)",
                          (long long)Tq);
  return hip_status(dsa::launch_index_scores_fp8(q8, q_scale, k8_pool, k_scale_pool, static_cast<const uint16_t*>(w),
                                                 scores, B, Tq, N, 0, static_cast<hipStream_t>(stream), seq_lens, &pg),
                    "paged FP8 index scores launch");
}

dsa_status dsa_sparse_mla_fwd_paged(const void* q, const void* kv_pool, const int32_t* idx, const int32_t* block_table,
                                    void* out, float* lse, int64_t B, int64_t Tq, int64_t max_blocks,
                                    int32_t block_size, int64_t num_blocks, int32_t H, int32_t D, int32_t DV, int32_t K,
                                    float scale, int32_t dtype, void* workspace, size_t ws_bytes, void* stream) {
  dsa::Paged pg;
  dsa_status st = check_paged(block_table, max_blocks, block_size, num_blocks, pg);
  if (st != DSA_OK) return st;
  if (dtype != DSA_BF16) return fail(DSA_ERR_UNSUPPORTED, "paged caches are built for bf16 only");
  // the gather addresses the whole pool as one sequence
  const int64_t pool_rows = num_blocks * (int64_t)block_size;
  st = check_mla(q, kv_pool, idx, out, lse, 1, B * Tq, pool_rows, H, D, DV, K, scale, dtype, nullptr, 0, false);
  if (st != DSA_OK) return st;
  if ((st = check_common(B, Tq, 1, 0, dtype)) != DSA_OK) return st;
  if (!idx || !aligned16(idx)) return fail(DSA_ERR_INVALID_ARG, "idx must be a 16-byte aligned device pointer");
  const size_t mla = align256(dsa::mla_workspace_bytes(B * Tq, H, DV, K, 1));
  const size_t need = mla + align256((size_t)B * Tq * K * sizeof(int32_t));
  if (!workspace || ws_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "paged sparse MLA workspace needs %zu bytes (got %zu)", need, ws_bytes);
  if (!aligned16(workspace)) return fail(DSA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  char* ws = static_cast<char*>(workspace);
  return run_paged_mla(q, kv_pool, idx, reinterpret_cast<int32_t*>(ws + mla), out, lse, B, Tq, K, scale, pg, ws,
                       static_cast<hipStream_t>(stream));
}

dsa_status dsa_forward_paged(const void* q_idx, const void* k_pool, const void* w, const void* q, const void* kv_pool,
                             void* out, float* lse, int32_t* idx_out, const int64_t* seq_lens,
                             const int32_t* block_table, int64_t B, int64_t Tq, int64_t max_blocks,
                             int32_t block_size, int64_t num_blocks, int32_t H_I, int32_t D_I, int32_t H, int32_t D,
                             int32_t DV, int32_t K, float scale, int32_t dtype, void* workspace, size_t ws_bytes,
                             void* stream) {
  dsa::Paged pg;
  dsa_status st = check_paged(block_table, max_blocks, block_size, num_blocks, pg);
  if (st != DSA_OK) return st;
  const int64_t N = max_blocks * (int64_t)block_size;
  if ((st = check_index_scores(q_idx, k_pool, w, nullptr, B, Tq, N, 0, H_I, D_I, dtype, false)) != DSA_OK) return st;
  if (dtype != DSA_BF16) return fail(DSA_ERR_UNSUPPORTED, "paged caches are built for bf16 only");
  if (Tq > 4) return fail(DSA_ERR_UNSUPPORTED, "paged caches are built for decode shapes (Tq <= 4, got %lld)",
                          (long long)Tq);
  st = check_mla(q, kv_pool, nullptr, out, lse, 1, B * Tq, num_blocks * (int64_t)block_size, H, D, DV, K, scale,
                 dtype, nullptr, 0, false);
  if (st != DSA_OK) return st;
  if ((st = check_seq_lens(seq_lens)) != DSA_OK) return st;
  if (idx_out && !aligned16(idx_out)) return fail(DSA_ERR_INVALID_ARG, "idx_out must be 16-byte aligned");
  const ForwardLayout L = forward_layout(B, Tq, N, H, DV, K, dtype);
  const size_t need = L.total + align256((size_t)B * Tq * K * sizeof(int32_t));
  if (!workspace || ws_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "paged forward workspace needs %zu bytes (got %zu)", need, ws_bytes);
  if (!aligned16(workspace)) return fail(DSA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  char* ws = static_cast<char*>(workspace);
  float* scores = reinterpret_cast<float*>(ws + L.scores);
  int32_t* idx = idx_out ? idx_out : reinterpret_cast<int32_t*>(ws + L.idx);
  void* topk_ws = ws + L.total - align256(dsa::topk_workspace_bytes(B, Tq, N, K));
  int32_t* phys = reinterpret_cast<int32_t*>(ws + L.total);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = index_and_topk_bf16(q_idx, k_pool, w, scores, idx, B, Tq, N, 0, K, topk_ws, s, seq_lens, &pg);
  if (e != hipSuccess) return hip_status(e, "paged index scores / top-k launch");
  return run_paged_mla(q, kv_pool, idx, phys, out, lse, B, Tq, K, scale, pg, ws + L.mla, s);
}

dsa_status dsa_cache_append_paged(void* k_pool, void* kv_pool, const void* new_k_idx, const void* new_kv,
                                  const int64_t* pos, const int32_t* block_table, int64_t B, int64_t max_blocks,
                                  int32_t block_size, int64_t num_blocks, int32_t D_I, int32_t D, int32_t dtype,
                                  void* stream) {
  dsa::Paged pg;
  dsa_status st = check_paged(block_table, max_blocks, block_size, num_blocks, pg);
  if (st != DSA_OK) return st;
  if (B < 1) return fail(DSA_ERR_INVALID_ARG, "B must be >= 1 (got %lld)", (long long)B);
  if (B > kMaxGrid) return fail(DSA_ERR_INVALID_ARG, "B must be < 2^31");
  if (dtype != DSA_BF16 && dtype != DSA_F32) return fail(DSA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (!pos) return fail(DSA_ERR_INVALID_ARG, "pos must not be null");
  if (!aligned8(pos)) return fail(DSA_ERR_INVALID_ARG, "pos must be 8-byte aligned");
  if ((k_pool == nullptr) != (new_k_idx == nullptr) || (kv_pool == nullptr) != (new_kv == nullptr))
    return fail(DSA_ERR_INVALID_ARG, "a cache and its new rows must be given together");
  if (!k_pool && !kv_pool) return fail(DSA_ERR_INVALID_ARG, "no cache to append to");
  if ((k_pool && (!aligned16(k_pool) || !aligned16(new_k_idx))) ||
      (kv_pool && (!aligned16(kv_pool) || !aligned16(new_kv))))
    return fail(DSA_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  if ((k_pool && D_I < 1) || (kv_pool && D < 1)) return fail(DSA_ERR_INVALID_ARG, "row widths must be >= 1");
  return hip_status(dsa::launch_cache_append(k_pool, kv_pool, new_k_idx, new_kv, pos, B, 0, k_pool ? D_I : 0,
                                             kv_pool ? D : 0, dtype == DSA_BF16 ? 2 : 4,
                                             static_cast<hipStream_t>(stream), &pg),
                    "paged cache append launch");
}

dsa_status dsa_calib_stream(const void* src, void* dst, size_t bytes, void* stream) {
  if (bytes == 0) return DSA_OK;
  if (src == nullptr) return fail(DSA_ERR_INVALID_ARG, "src must not be NULL");
  if (bytes % 16 != 0) return fail(DSA_ERR_INVALID_ARG, "bytes must be a multiple of 16");
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(dst) % 16 != 0)
    return fail(DSA_ERR_INVALID_ARG, "src and dst must be 16-byte aligned");
  if (dst != nullptr) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
    if (a < b + bytes && b < a + bytes) return fail(DSA_ERR_INVALID_ARG, "src and dst must not overlap");
  }
  return hip_status(dsa::launch_calib_stream(src, dst, bytes, static_cast<hipStream_t>(stream)), "calibration stream launch");
}

}  // extern "C"

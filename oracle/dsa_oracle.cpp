/*
 * CPU oracle of the DeepSeek Sparse Attention (DSA) forward pass.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the test suite, the package smoke check
 * and the CPU-baseline leg of the benchmark, never by the product path.  It
 * shares no code with the HIP library.
 *
 * Plain C++17, double accumulation, scalar loops written straight from the
 * method's definition, one function per step in the order the pages give
 * them.  The only parallelism is across query rows (std::thread); a row is
 * always computed by one thread in one fixed order, so the thread count never
 * changes a bit of the result.
 *
 * What the pages fix (DeepSeek-V3.2 model documentation, section "DeepSeek
 * Sparse Attention (DSA)"):
 *   * the lightning indexer, a light scorer with few heads, scores each query
 *     against every key before it (its paragraph on the lightning indexer);
 *   * it keeps its own single-head key cache of width index_head_dim (the
 *     paragraph on the indexer cache), and per-token head weights come from
 *     weights_proj;
 *   * fine-grained token selection keeps the index_topk best keys per query,
 *     and the main attention runs over those only, applied as an additive
 *     mask (the token-selection paragraph);
 *   * scores computed in FP8 after an orthogonal Hadamard rotation equal those
 *     computed directly.
 * DeepSeek-V3.2 documentation, "DeepseekV32Config": index_n_heads 64,
 * index_head_dim 128, index_topk 2048, kv_lora_rank 512, qk_rope_head_dim 64.
 * DeepSeek-V4 documentation, section on the attention mask layout: an index
 * of -1 means "no selection"; a compressed entry becomes visible once its
 * window of m positions has closed.
 *
 * Readings where the pages are silent (listed with reasons in the repository's
 * design notes): the score is the head-weighted sum of ReLU(per-head q.k) with
 * no further scale; "keys before the query" includes the query's own
 * position; ties in the top-k go to the lower key index; kept indices are
 * listed ascending and padded with -1; the MLA runs in absorbed latent form
 * (one D-wide latent row per key shared by all heads, value = its first DV
 * entries, logits scale * q.kv); an index < 0 or >= N is masked; a row with no
 * valid index gives o = 0 and lse = -inf; lse is the natural-log sum of
 * exp(logits).
 */
#include "dsa_oracle.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <exception>
#include <functional>
#include <limits>
#include <numeric>
#include <thread>
#include <vector>

namespace {

const double kNegInf = -std::numeric_limits<double>::infinity();

// --------------------------------------------------------------------------
// Element access: every input is widened exactly to double before use.
// --------------------------------------------------------------------------

bool dtype_ok(int dt) { return dt == DSAO_F64 || dt == DSAO_F32 || dt == DSAO_BF16; }

// A bfloat16 is the upper 16 bits of a float32.
double bf16_to_double(uint16_t bits) {
  const uint32_t u = static_cast<uint32_t>(bits) << 16;
  float f;
  std::memcpy(&f, &u, sizeof f);
  return f;
}

double element(const void* p, int dt, int64_t i) {
  if (dt == DSAO_F64) return static_cast<const double*>(p)[i];
  if (dt == DSAO_F32) return static_cast<const float*>(p)[i];
  return bf16_to_double(static_cast<const uint16_t*>(p)[i]);
}

// dst[i] = element (first + i) of the tensor, for i < n.
void widen_into(const void* p, int dt, int64_t first, int64_t n, double* dst) {
  for (int64_t i = 0; i < n; ++i) dst[i] = element(p, dt, first + i);
}

// Runs body(r) for r = 0 .. n_rows-1, rows dealt round-robin to the threads.
void for_each_row(int64_t n_rows, int threads, const std::function<void(int64_t)>& body) {
  if (threads <= 0) threads = static_cast<int>(std::max(1u, std::thread::hardware_concurrency()));
  if (threads > n_rows) threads = static_cast<int>(std::max<int64_t>(1, n_rows));
  if (threads == 1) {
    for (int64_t r = 0; r < n_rows; ++r) body(r);
    return;
  }
  std::vector<std::thread> pool;
  std::vector<std::exception_ptr> failed(threads);
  for (int w = 0; w < threads; ++w) {
    pool.emplace_back([&, w] {
      try {
        for (int64_t r = w; r < n_rows; r += threads) body(r);
      } catch (...) {
        failed[w] = std::current_exception();
      }
    });
  }
  for (auto& t : pool) t.join();
  for (auto& e : failed)
    if (e) std::rethrow_exception(e);
}

// Maps the C++ failure modes to the C status codes.
int guarded(const std::function<void()>& fn) {
  try {
    fn();
    return 0;
  } catch (...) {
    return 2;
  }
}

bool rows_ok(const int64_t* rows, int64_t n_rows, int64_t B, int64_t Tq) {
  if (n_rows < 0 || (n_rows > 0 && rows == nullptr)) return false;
  for (int64_t r = 0; r < n_rows; ++r)
    if (rows[2 * r] < 0 || rows[2 * r] >= B || rows[2 * r + 1] < 0 || rows[2 * r + 1] >= Tq) return false;
  return true;
}

// --------------------------------------------------------------------------
// Visibility.  Query at absolute position p sees keys 0..p (own key
// included), capped by the cache length N.  On a key axis compressed at
// rate m, entry e summarises positions m*e .. m*e+m-1 and is visible once
// the last of them has arrived: e < (p + 1) / m.
// --------------------------------------------------------------------------

int64_t n_valid_keys(int64_t t, int64_t q_pos0, int64_t N, int64_t m) {
  const int64_t p1 = q_pos0 + t + 1;   // number of positions 0..p
  if (p1 <= 0) return 0;
  return std::min(N, p1 / m);
}

// --------------------------------------------------------------------------
// O1, lightning indexer score of one query against one key:
//   I = sum_h w[h] * ReLU( sum_d q[h][d] * k[d] )
// --------------------------------------------------------------------------

double relu(double x) { return x > 0.0 ? x : 0.0; }

double index_score(const double* q_t /* [H_I][D_I] */, const double* w_t /* [H_I] */, const double* k_s /* [D_I] */,
                   int32_t H_I, int32_t D_I) {
  double I = 0.0;
  for (int32_t h = 0; h < H_I; ++h) {
    double dot = 0.0;
    for (int32_t d = 0; d < D_I; ++d) dot += q_t[h * D_I + d] * k_s[d];
    I += w_t[h] * relu(dot);
  }
  return I;
}

// Scores of query (b, t) against its n visible keys, into out[0..n).
void index_scores_row(const void* q_idx, int q_dt, const void* k_idx, int k_dt, const void* w, int w_dt,
                      int64_t Tq, int64_t N, int32_t H_I, int32_t D_I, int64_t b, int64_t t, int64_t n,
                      double* out) {
  std::vector<double> q_t(static_cast<size_t>(H_I) * D_I), w_t(H_I), k_s(D_I);
  widen_into(q_idx, q_dt, (b * Tq + t) * H_I * D_I, static_cast<int64_t>(H_I) * D_I, q_t.data());
  widen_into(w, w_dt, (b * Tq + t) * H_I, H_I, w_t.data());
  for (int64_t s = 0; s < n; ++s) {
    widen_into(k_idx, k_dt, (b * N + s) * D_I, D_I, k_s.data());
    out[s] = index_score(q_t.data(), w_t.data(), k_s.data(), H_I, D_I);
  }
}

// --------------------------------------------------------------------------
// O2, top-k of one row of n float32 scores: candidates 0..n-1; if n <= K all
// are kept; otherwise a stable sort by score, descending (equal scores keep
// their index order, so ties go to the lower index), keeps the first K,
// which are then listed in ascending index order.  -1 pads the tail.
// -0 and +0 compare equal, as IEEE comparison has it.
// --------------------------------------------------------------------------

void topk_row(const float* v, int64_t n, int32_t K, int32_t* out) {
  if (n <= K) {
    for (int64_t i = 0; i < K; ++i) out[i] = i < n ? static_cast<int32_t>(i) : -1;
    return;
  }
  std::vector<int64_t> cand(n);
  std::iota(cand.begin(), cand.end(), int64_t{0});
  std::stable_sort(cand.begin(), cand.end(), [v](int64_t a, int64_t b) { return v[a] > v[b]; });
  std::sort(cand.begin(), cand.begin() + K);
  for (int32_t i = 0; i < K; ++i) out[i] = static_cast<int32_t>(cand[i]);
}

// --------------------------------------------------------------------------
// O3, sparse MLA for one query, every head.  With S the valid indices of the
// row, in the order given:
//   l_j = scale * sum_d q[h][d] * kv[S_j][d]
//   m = max_j l_j,  p_j = exp(l_j - m),  l = sum_j p_j
//   o[h][c] = sum_j p_j * kv[S_j][c] / l   (c < DV),   lse[h] = m + ln l
// --------------------------------------------------------------------------

void softmax_attend(const std::vector<double>& logits, const std::vector<const double*>& values, int32_t DV,
                    double* o_h, double* lse_h) {
  const size_t n = logits.size();
  if (n == 0) {
    for (int32_t c = 0; c < DV; ++c) o_h[c] = 0.0;
    *lse_h = kNegInf;
    return;
  }
  double m = kNegInf;
  for (double x : logits) m = std::max(m, x);
  std::vector<double> p(n);
  double l = 0.0;
  for (size_t j = 0; j < n; ++j) {
    p[j] = std::exp(logits[j] - m);
    l += p[j];
  }
  std::vector<double> acc(DV, 0.0);
  for (size_t j = 0; j < n; ++j)
    for (int32_t c = 0; c < DV; ++c) acc[c] += p[j] * values[j][c];
  for (int32_t c = 0; c < DV; ++c) o_h[c] = acc[c] / l;
  *lse_h = m + std::log(l);
}

void sparse_mla_row(const void* q, int q_dt, const void* kv, int kv_dt, const int32_t* idx_row, int64_t Tq,
                    int64_t N, int32_t H, int32_t D, int32_t DV, int32_t K, double scale, int64_t b, int64_t t,
                    double* o /* [H][DV] */, double* lse /* [H] */) {
  std::vector<int64_t> sel;
  for (int32_t j = 0; j < K; ++j) {
    const int64_t i = idx_row[j];
    if (i < 0 || i >= N) continue;   // masked: additive -inf
    sel.push_back(i);
  }
  const size_t n = sel.size();
  std::vector<double> rows(n * D);
  for (size_t j = 0; j < n; ++j) widen_into(kv, kv_dt, (b * N + sel[j]) * D, D, &rows[j * D]);
  std::vector<const double*> values(n);
  for (size_t j = 0; j < n; ++j) values[j] = &rows[j * D];   // value = first DV entries of the row
  std::vector<double> q_h(D), logits(n);
  for (int32_t h = 0; h < H; ++h) {
    widen_into(q, q_dt, ((b * Tq + t) * H + h) * D, D, q_h.data());
    for (size_t j = 0; j < n; ++j) {
      double dot = 0.0;
      for (int32_t d = 0; d < D; ++d) dot += q_h[d] * rows[j * D + d];
      logits[j] = scale * dot;
    }
    softmax_attend(logits, values, DV, o + static_cast<int64_t>(h) * DV, lse + h);
  }
}

// O3', dense form: every visible key s gets logit scale*q.kv[s] plus a mask
// term, 0 if s is selected and -inf otherwise; the softmax runs over all s.
void dense_masked_mla_row(const void* q, int q_dt, const void* kv, int kv_dt, const int32_t* idx_row, int64_t Tq,
                          int64_t N, int32_t H, int32_t D, int32_t DV, int32_t K, double scale, int64_t b,
                          int64_t t, int64_t n_visible, double* o, double* lse) {
  std::vector<double> mask(n_visible, kNegInf);
  for (int32_t j = 0; j < K; ++j)
    if (idx_row[j] >= 0 && idx_row[j] < n_visible) mask[idx_row[j]] = 0.0;
  bool any = false;
  for (double x : mask) any = any || x == 0.0;
  std::vector<double> rows(n_visible * D);
  for (int64_t s = 0; s < n_visible; ++s) widen_into(kv, kv_dt, (b * N + s) * D, D, &rows[s * D]);
  std::vector<double> q_h(D), logits(n_visible), p(n_visible);
  for (int32_t h = 0; h < H; ++h) {
    double* o_h = o + static_cast<int64_t>(h) * DV;
    if (!any) {
      for (int32_t c = 0; c < DV; ++c) o_h[c] = 0.0;
      lse[h] = kNegInf;
      continue;
    }
    widen_into(q, q_dt, ((b * Tq + t) * H + h) * D, D, q_h.data());
    double m = kNegInf;
    for (int64_t s = 0; s < n_visible; ++s) {
      double dot = 0.0;
      for (int32_t d = 0; d < D; ++d) dot += q_h[d] * rows[s * D + d];
      logits[s] = scale * dot + mask[s];
      m = std::max(m, logits[s]);
    }
    double l = 0.0;
    for (int64_t s = 0; s < n_visible; ++s) {
      p[s] = std::exp(logits[s] - m);   // exp(-inf) = 0 for masked keys
      l += p[s];
    }
    std::vector<double> acc(DV, 0.0);
    for (int64_t s = 0; s < n_visible; ++s)
      for (int32_t c = 0; c < DV; ++c) acc[c] += p[s] * rows[s * D + c];
    for (int32_t c = 0; c < DV; ++c) o_h[c] = acc[c] / l;
    lse[h] = m + std::log(l);
  }
}

// --------------------------------------------------------------------------
// FP8 indexer (DeepSeek-V3.2 documentation, "DeepSeek Sparse Attention
// (DSA)": the original indexer runs in FP8 after a Hadamard rotation, which
// is orthogonal and leaves the scores unchanged).  Readings: OCP E4M3 (bias
// 7, largest finite 448, S.1111.111 is NaN); the unnormalised Sylvester
// rotation applied by the fast Walsh-Hadamard transform in float32 with pair
// distance 1, 2, 4, ...; one power-of-two scale per rotated row; codes
// rounded to nearest, ties to even; the factor D of the rotation is divided
// out of the score.
// --------------------------------------------------------------------------

void fwht_row(float* y, int32_t n) {
  for (int32_t dist = 1; dist < n; dist *= 2)
    for (int32_t base = 0; base < n; base += 2 * dist)
      for (int32_t i = 0; i < dist; ++i) {
        const float a = y[base + i], b = y[base + dist + i];
        y[base + i] = a + b;
        y[base + dist + i] = a - b;
      }
}

double e4m3_decode(uint8_t code) {
  const double sign = (code & 0x80) ? -1.0 : 1.0;
  const int E = (code >> 3) & 15;
  const int M = code & 7;
  if ((code & 0x7F) == 0x7F) return std::numeric_limits<double>::quiet_NaN();
  if (E == 0) return sign * M * std::ldexp(1.0, -9);            // subnormal: M * 2^-9
  return sign * (1.0 + M / 8.0) * std::ldexp(1.0, E - 7);
}

// |v| <= 448 assumed (checked by the caller).
uint8_t e4m3_encode_rne(float v) {
  const double a = std::fabs(static_cast<double>(v));
  int code;
  if (a < std::ldexp(1.0, -6)) {
    code = static_cast<int>(std::nearbyint(a * 512.0));           // multiples of 2^-9; 8 is 2^-6, the first normal
  } else {
    int E;
    std::frexp(a, &E);                                            // a = f * 2^E, 0.5 <= f < 1
    int e = E - 1;                                                // 2^e <= a < 2^(e+1)
    int mant = static_cast<int>(std::nearbyint((a / std::ldexp(1.0, e) - 1.0) * 8.0));
    if (mant == 8) {                                              // rounded up into the next binade
      mant = 0;
      e += 1;
    }
    code = ((e + 7) << 3) | mant;
  }
  if (std::signbit(v)) code |= 0x80;
  return static_cast<uint8_t>(code);
}

// Smallest integer e with amax <= 448 * 2^e; 0 for amax == 0.
int pow2_scale_exp(double amax) {
  if (amax == 0.0) return 0;
  int e = std::ilogb(amax) - 9;
  while (amax > std::ldexp(448.0, e)) ++e;
  while (amax <= std::ldexp(448.0, e - 1)) --e;
  return e;
}

void quantize_fp8_row(const void* x, int dt, int64_t row, int32_t D, uint8_t* codes, float* scale) {
  std::vector<float> y(D);
  for (int32_t d = 0; d < D; ++d) y[d] = static_cast<float>(element(x, dt, row * D + d));
  fwht_row(y.data(), D);
  double amax = 0.0;
  for (float v : y) amax = std::max(amax, std::fabs(static_cast<double>(v)));
  const int e = pow2_scale_exp(amax);
  for (int32_t d = 0; d < D; ++d) codes[d] = e4m3_encode_rne(std::ldexp(y[d], -e));   // exact power-of-two scaling
  *scale = std::ldexp(1.0f, e);
}

// I[s] = sum_h w[h] * ReLU( qs[h] * ks[s] / D * sum_d dec(q8[h][d]) * dec(k8[s][d]) )
double index_score_fp8(const double* q_t, const double* qs_t, const double* w_t, const double* k_s, double ks_s,
                       int32_t H_I, int32_t D) {
  double I = 0.0;
  for (int32_t h = 0; h < H_I; ++h) {
    double dot = 0.0;
    for (int32_t d = 0; d < D; ++d) dot += q_t[h * D + d] * k_s[d];
    I += w_t[h] * relu(qs_t[h] * ks_s / D * dot);
  }
  return I;
}

}  // namespace

// ==========================================================================
// C interface
// ==========================================================================

extern "C" {

int dsao_version(void) { return 1; }

int dsao_widen(const void* x, int dt, int64_t n, double* out) {
  if (n < 0 || !dtype_ok(dt) || (n > 0 && (x == nullptr || out == nullptr))) return 1;
  widen_into(x, dt, 0, n, out);
  return 0;
}

int64_t dsao_n_valid_keys(int64_t t, int64_t q_pos0, int64_t N, int64_t m) {
  if (m < 1 || N < 0) return -1;
  return n_valid_keys(t, q_pos0, N, m);
}

int dsao_index_scores(const void* q_idx, int q_dt, const void* k_idx, int k_dt, const void* w, int w_dt,
                      int64_t B, int64_t Tq, int64_t N, int32_t H_I, int32_t D_I, const int64_t* q_pos0,
                      int64_t m, const int64_t* rows, int64_t n_rows, double* out, int threads) {
  if (!q_idx || !k_idx || !w || !q_pos0 || !out || !dtype_ok(q_dt) || !dtype_ok(k_dt) || !dtype_ok(w_dt)) return 1;
  if (B < 1 || Tq < 1 || N < 0 || H_I < 1 || D_I < 1 || m < 1 || !rows_ok(rows, n_rows, B, Tq)) return 1;
  return guarded([&] {
    for_each_row(n_rows, threads, [&](int64_t r) {
      const int64_t b = rows[2 * r], t = rows[2 * r + 1];
      const int64_t n = n_valid_keys(t, q_pos0[b], N, m);
      index_scores_row(q_idx, q_dt, k_idx, k_dt, w, w_dt, Tq, N, H_I, D_I, b, t, n, out + r * N);
    });
  });
}

int dsao_topk(const float* scores, int64_t n_rows, int64_t row_stride, const int64_t* n_valid, int32_t K,
              int32_t* out, int threads) {
  if (n_rows < 0 || K < 1 || row_stride < 0 || (n_rows > 0 && (!scores || !n_valid || !out))) return 1;
  for (int64_t r = 0; r < n_rows; ++r)
    if (n_valid[r] < 0 || n_valid[r] > row_stride) return 1;
  return guarded([&] {
    for_each_row(n_rows, threads,
                 [&](int64_t r) { topk_row(scores + r * row_stride, n_valid[r], K, out + r * K); });
  });
}

int dsao_sparse_mla(const void* q, int q_dt, const void* kv, int kv_dt, const int32_t* idx, int64_t B, int64_t Tq,
                    int64_t N, int32_t H, int32_t D, int32_t DV, int32_t K, double scale, const int64_t* rows,
                    int64_t n_rows, double* o, double* lse, int threads) {
  if (!q || !kv || !idx || !o || !lse || !dtype_ok(q_dt) || !dtype_ok(kv_dt)) return 1;
  if (B < 1 || Tq < 1 || N < 0 || H < 1 || D < 1 || DV < 1 || DV > D || K < 1 || !rows_ok(rows, n_rows, B, Tq))
    return 1;
  return guarded([&] {
    for_each_row(n_rows, threads, [&](int64_t r) {
      const int64_t b = rows[2 * r], t = rows[2 * r + 1];
      sparse_mla_row(q, q_dt, kv, kv_dt, idx + (b * Tq + t) * K, Tq, N, H, D, DV, K, scale, b, t,
                     o + r * H * DV, lse + r * H);
    });
  });
}

int dsao_dense_masked_mla(const void* q, int q_dt, const void* kv, int kv_dt, const int32_t* idx, int64_t B,
                          int64_t Tq, int64_t N, int32_t H, int32_t D, int32_t DV, int32_t K, double scale,
                          const int64_t* q_pos0, const int64_t* rows, int64_t n_rows, double* o, double* lse,
                          int threads) {
  if (!q || !kv || !idx || !q_pos0 || !o || !lse || !dtype_ok(q_dt) || !dtype_ok(kv_dt)) return 1;
  if (B < 1 || Tq < 1 || N < 0 || H < 1 || D < 1 || DV < 1 || DV > D || K < 1 || !rows_ok(rows, n_rows, B, Tq))
    return 1;
  return guarded([&] {
    for_each_row(n_rows, threads, [&](int64_t r) {
      const int64_t b = rows[2 * r], t = rows[2 * r + 1];
      const int64_t n = n_valid_keys(t, q_pos0[b], N, 1);
      dense_masked_mla_row(q, q_dt, kv, kv_dt, idx + (b * Tq + t) * K, Tq, N, H, D, DV, K, scale, b, t, n,
                           o + r * H * DV, lse + r * H);
    });
  });
}

int dsao_forward(const void* q_idx, int qi_dt, const void* k_idx, int ki_dt, const void* w, int w_dt,
                 const void* q, int q_dt, const void* kv, int kv_dt, int64_t B, int64_t Tq, int64_t N,
                 const int64_t* q_pos0, int32_t H_I, int32_t D_I, int32_t H, int32_t D, int32_t DV, int32_t K,
                 double scale, const int64_t* rows, int64_t n_rows, double* scores, int32_t* idx, double* o,
                 double* lse, int threads) {
  if (!q_idx || !k_idx || !w || !q || !kv || !q_pos0 || !idx || !o || !lse) return 1;
  if (!dtype_ok(qi_dt) || !dtype_ok(ki_dt) || !dtype_ok(w_dt) || !dtype_ok(q_dt) || !dtype_ok(kv_dt)) return 1;
  if (B < 1 || Tq < 1 || N < 0 || H_I < 1 || D_I < 1 || H < 1 || D < 1 || DV < 1 || DV > D || K < 1 ||
      !rows_ok(rows, n_rows, B, Tq))
    return 1;
  return guarded([&] {
    for_each_row(n_rows, threads, [&](int64_t r) {
      const int64_t b = rows[2 * r], t = rows[2 * r + 1];
      const int64_t n = n_valid_keys(t, q_pos0[b], N, 1);
      // O1: scores in double
      std::vector<double> s(n);
      index_scores_row(q_idx, qi_dt, k_idx, ki_dt, w, w_dt, Tq, N, H_I, D_I, b, t, n, s.data());
      if (scores)
        for (int64_t i = 0; i < n; ++i) scores[r * N + i] = s[i];
      // O2: the selection is taken on the scores as float32, the precision they are stored in
      std::vector<float> s32(n);
      for (int64_t i = 0; i < n; ++i) s32[i] = static_cast<float>(s[i]);
      topk_row(s32.data(), n, K, idx + r * K);
      // O3: attention over the selected rows; q and kv of this query's sequence
      std::vector<int32_t> row_idx(idx + r * K, idx + r * K + K);
      sparse_mla_row(q, q_dt, kv, kv_dt, row_idx.data(), Tq, N, H, D, DV, K, scale, b, t, o + r * H * DV,
                     lse + r * H);
    });
  });
}

int dsao_sylvester_hadamard(int32_t n, double* out) {
  if (n < 1 || (n & (n - 1)) != 0 || !out) return 1;
  // H_1 = [1];  H_2k = [[H_k, H_k], [H_k, -H_k]]
  out[0] = 1.0;
  for (int32_t k = 1; k < n; k *= 2) {
    for (int32_t i = 0; i < k; ++i)
      for (int32_t j = 0; j < k; ++j) {
        const double h = out[i * n + j];
        out[i * n + (j + k)] = h;
        out[(i + k) * n + j] = h;
        out[(i + k) * n + (j + k)] = -h;
      }
  }
  return 0;
}

int dsao_fwht_f32(float* x, int64_t n_rows, int32_t n) {
  if (n < 1 || (n & (n - 1)) != 0 || n_rows < 0 || (n_rows > 0 && !x)) return 1;
  for (int64_t r = 0; r < n_rows; ++r) fwht_row(x + r * n, n);
  return 0;
}

int dsao_e4m3_decode(const uint8_t* codes, int64_t n, double* out) {
  if (n < 0 || (n > 0 && (!codes || !out))) return 1;
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_decode(codes[i]);
  return 0;
}

int dsao_e4m3_encode_rne(const float* v, int64_t n, uint8_t* out) {
  if (n < 0 || (n > 0 && (!v || !out))) return 1;
  for (int64_t i = 0; i < n; ++i)
    if (!(std::fabs(v[i]) <= 448.0f)) return 1;
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_encode_rne(v[i]);
  return 0;
}

int dsao_pow2_scale_exp(double amax) { return pow2_scale_exp(amax); }

int dsao_quantize_fp8_rows(const void* x, int dt, int64_t n_rows, int32_t D, uint8_t* codes, float* scales) {
  if (!dtype_ok(dt) || D < 1 || (D & (D - 1)) != 0 || n_rows < 0 || (n_rows > 0 && (!x || !codes || !scales)))
    return 1;
  for (int64_t r = 0; r < n_rows; ++r) quantize_fp8_row(x, dt, r, D, codes + r * D, scales + r);
  return 0;
}

int dsao_index_scores_fp8(const uint8_t* q8, const float* qs, const uint8_t* k8, const float* ks, const void* w,
                          int w_dt, int64_t B, int64_t Tq, int64_t N, int32_t H_I, int32_t D, const int64_t* q_pos0,
                          const int64_t* rows, int64_t n_rows, double* out, int threads) {
  if (!q8 || !qs || !k8 || !ks || !w || !q_pos0 || !out || !dtype_ok(w_dt)) return 1;
  if (B < 1 || Tq < 1 || N < 0 || H_I < 1 || D < 1 || !rows_ok(rows, n_rows, B, Tq)) return 1;
  return guarded([&] {
    for_each_row(n_rows, threads, [&](int64_t r) {
      const int64_t b = rows[2 * r], t = rows[2 * r + 1];
      const int64_t n = n_valid_keys(t, q_pos0[b], N, 1);
      std::vector<double> q_t(static_cast<size_t>(H_I) * D), qs_t(H_I), w_t(H_I), k_s(D);
      for (int64_t i = 0; i < static_cast<int64_t>(H_I) * D; ++i) q_t[i] = e4m3_decode(q8[(b * Tq + t) * H_I * D + i]);
      for (int32_t h = 0; h < H_I; ++h) qs_t[h] = qs[(b * Tq + t) * H_I + h];
      widen_into(w, w_dt, (b * Tq + t) * H_I, H_I, w_t.data());
      for (int64_t s = 0; s < n; ++s) {
        for (int32_t d = 0; d < D; ++d) k_s[d] = e4m3_decode(k8[(b * N + s) * D + d]);
        out[r * N + s] = index_score_fp8(q_t.data(), qs_t.data(), w_t.data(), k_s.data(), ks[b * N + s], H_I, D);
      }
    });
  });
}

// y[m][n] = sum_k x[m][k] * W[n][k]   (W stored [out, in])
int dsao_linear(const void* x, int x_dt, const void* W, int W_dt, int64_t M, int64_t N_out, int64_t K_in, double* y,
                int threads) {
  if (!x || !W || !y || !dtype_ok(x_dt) || !dtype_ok(W_dt) || M < 0 || N_out < 1 || K_in < 1) return 1;
  return guarded([&] {
    std::vector<double> w(N_out * K_in);
    widen_into(W, W_dt, 0, N_out * K_in, w.data());
    for_each_row(M, threads, [&](int64_t m) {
      std::vector<double> xm(K_in);
      widen_into(x, x_dt, m * K_in, K_in, xm.data());
      for (int64_t n = 0; n < N_out; ++n) {
        double acc = 0.0;
        for (int64_t k = 0; k < K_in; ++k) acc += xm[k] * w[n * K_in + k];
        y[m * N_out + n] = acc;
      }
    });
  });
}

// q [M, H, d_nope + d_rope] -> out [M, H, d_c + d_rope]:
//   out[m][h][c] = sum_n W_UK[h][n][c] * q[m][h][n]   (c < d_c; W_UK stored [H, d_nope, d_c])
//   out[m][h][d_c + r] = q[m][h][d_nope + r]
int dsao_mla_absorb_query(const void* q, int q_dt, const void* W_UK, int w_dt, int64_t M, int32_t H, int32_t d_nope,
                          int32_t d_rope, int32_t d_c, double* out, int threads) {
  if (!q || !W_UK || !out || !dtype_ok(q_dt) || !dtype_ok(w_dt) || M < 0 || H < 1 || d_nope < 1 || d_rope < 0 ||
      d_c < 1)
    return 1;
  const int64_t qw = d_nope + d_rope, ow = d_c + d_rope;
  return guarded([&] {
    std::vector<double> w_uk(static_cast<int64_t>(H) * d_nope * d_c);
    widen_into(W_UK, w_dt, 0, static_cast<int64_t>(w_uk.size()), w_uk.data());
    for_each_row(M, threads, [&](int64_t m) {
      std::vector<double> qh(qw);
      for (int32_t h = 0; h < H; ++h) {
        const int64_t ob = (m * H + h) * ow;
        widen_into(q, q_dt, (m * H + h) * qw, qw, qh.data());
        for (int32_t c = 0; c < d_c; ++c) {
          double acc = 0.0;
          for (int32_t n = 0; n < d_nope; ++n) acc += w_uk[(static_cast<int64_t>(h) * d_nope + n) * d_c + c] * qh[n];
          out[ob + c] = acc;
        }
        for (int32_t r = 0; r < d_rope; ++r) out[ob + d_c + r] = qh[d_nope + r];
      }
    });
  });
}

// o[m][h][v] = sum_c W_UV[h][v][c] * o_lat[m][h][c]   (W_UV stored [H, d_v, d_c])
int dsao_mla_output_projection(const void* o_lat, int o_dt, const void* W_UV, int w_dt, int64_t M, int32_t H,
                               int32_t d_c, int32_t d_v, double* out, int threads) {
  if (!o_lat || !W_UV || !out || !dtype_ok(o_dt) || !dtype_ok(w_dt) || M < 0 || H < 1 || d_c < 1 || d_v < 1)
    return 1;
  return guarded([&] {
    std::vector<double> w_uv(static_cast<int64_t>(H) * d_v * d_c);
    widen_into(W_UV, w_dt, 0, static_cast<int64_t>(w_uv.size()), w_uv.data());
    for_each_row(M, threads, [&](int64_t m) {
      std::vector<double> oh(d_c);
      for (int32_t h = 0; h < H; ++h) {
        widen_into(o_lat, o_dt, (m * H + h) * d_c, d_c, oh.data());
        for (int32_t v = 0; v < d_v; ++v) {
          double acc = 0.0;
          for (int32_t c = 0; c < d_c; ++c) acc += w_uv[(static_cast<int64_t>(h) * d_v + v) * d_c + c] * oh[c];
          out[(m * H + h) * d_v + v] = acc;
        }
      }
    });
  });
}

// Naive MLA for one query (DeepSeek-V3 documentation: its port computes
// attention per head with explicit keys and values).  Head h builds, for each
// selected token j, the key [W_UK[h] c_j, k_rope_j] and the value W_UV[h] c_j,
// then attends with softmax(scale * q.k).  Heads are split over the threads.
int dsao_mla_naive_row(const void* q_head, int q_dt, const void* c_kv, int c_dt, const void* k_rope, int r_dt,
                       int64_t N, const int32_t* idx, int32_t K, const void* W_UK, int uk_dt, const void* W_UV,
                       int uv_dt, int32_t H, int32_t d_nope, int32_t d_rope, int32_t d_c, int32_t d_v, double scale,
                       double* o, double* lse, int threads) {
  if (!q_head || !c_kv || !k_rope || !idx || !W_UK || !W_UV || !o || !lse) return 1;
  if (!dtype_ok(q_dt) || !dtype_ok(c_dt) || !dtype_ok(r_dt) || !dtype_ok(uk_dt) || !dtype_ok(uv_dt)) return 1;
  if (N < 0 || K < 0 || H < 1 || d_nope < 1 || d_rope < 0 || d_c < 1 || d_v < 1) return 1;
  return guarded([&] {
    std::vector<int64_t> sel;
    for (int32_t j = 0; j < K; ++j)
      if (idx[j] >= 0 && idx[j] < N) sel.push_back(idx[j]);
    const size_t n = sel.size();
    const int32_t kw = d_nope + d_rope;
    std::vector<double> c(n * d_c), kr(n * d_rope);
    for (size_t j = 0; j < n; ++j) {
      widen_into(c_kv, c_dt, sel[j] * d_c, d_c, &c[j * d_c]);
      widen_into(k_rope, r_dt, sel[j] * d_rope, d_rope, &kr[j * d_rope]);
    }
    for_each_row(H, threads, [&](int64_t h) {
      std::vector<double> w_uk(static_cast<int64_t>(d_nope) * d_c), w_uv(static_cast<int64_t>(d_v) * d_c), qh(kw);
      widen_into(W_UK, uk_dt, h * d_nope * d_c, static_cast<int64_t>(w_uk.size()), w_uk.data());
      widen_into(W_UV, uv_dt, h * d_v * d_c, static_cast<int64_t>(w_uv.size()), w_uv.data());
      widen_into(q_head, q_dt, h * kw, kw, qh.data());
      std::vector<double> keys(n * kw), vals(n * d_v), logits(n);
      std::vector<const double*> value_rows(n);
      for (size_t j = 0; j < n; ++j) {
        for (int32_t a = 0; a < d_nope; ++a) {
          double acc = 0.0;
          for (int32_t x = 0; x < d_c; ++x) acc += w_uk[static_cast<int64_t>(a) * d_c + x] * c[j * d_c + x];
          keys[j * kw + a] = acc;
        }
        for (int32_t r = 0; r < d_rope; ++r) keys[j * kw + d_nope + r] = kr[j * d_rope + r];
        for (int32_t v = 0; v < d_v; ++v) {
          double acc = 0.0;
          for (int32_t x = 0; x < d_c; ++x) acc += w_uv[static_cast<int64_t>(v) * d_c + x] * c[j * d_c + x];
          vals[j * d_v + v] = acc;
        }
        value_rows[j] = &vals[j * d_v];
      }
      for (size_t j = 0; j < n; ++j) {
        double dot = 0.0;
        for (int32_t a = 0; a < kw; ++a) dot += qh[a] * keys[j * kw + a];
        logits[j] = scale * dot;
      }
      softmax_attend(logits, value_rows, d_v, o + h * d_v, lse + h);
    });
  });
}

int dsao_paged_gather(const void* pool, int64_t pool_rows, int64_t row_bytes, const int64_t* table_row,
                      int64_t table_len, int64_t block_size, int64_t n_rows, void* out) {
  if (!pool || !table_row || !out || pool_rows < 0 || row_bytes < 1 || block_size < 1 || n_rows < 0) return 1;
  if (n_rows > table_len * block_size) return 1;
  for (int64_t r = 0; r < n_rows; ++r) {
    const int64_t p = table_row[r / block_size] * block_size + r % block_size;
    if (table_row[r / block_size] < 0 || p >= pool_rows) return 1;
  }
  for (int64_t r = 0; r < n_rows; ++r) {
    const int64_t p = table_row[r / block_size] * block_size + r % block_size;
    std::memcpy(static_cast<char*>(out) + r * row_bytes, static_cast<const char*>(pool) + p * row_bytes,
                static_cast<size_t>(row_bytes));
  }
  return 0;
}

}  // extern "C"

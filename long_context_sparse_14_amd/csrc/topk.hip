// Per-query top-k selection on gfx950.
//
// Row (b,t) keeps the K best of its n = min(N, q_pos0 + t + 1) visible
// scores (DeepSeek-V3.2 model documentation, section "DeepSeek Sparse
// Attention (DSA)", paragraph on fine-grained token selection; index_topk =
// 2048 in the DeepseekV32Config section).  The order is score descending, key
// index ascending, so equal scores go to the lower index; the kept keys are
// written in ascending index order and a row with n <= K is 0..n-1 followed by
// -1 entries (the "no selection" value of the DeepSeek-V4 documentation's
// attention mask layout section).
//
// Method: exact radix select on order-preserving 32-bit keys (larger score ->
// larger key, -0 == +0).  With T the K-th largest key and k_eq the number of
// keys equal to T that are kept, key i is kept iff key_i > T, or key_i == T and
// fewer than k_eq equal keys precede it; its output slot is
//   #{j < i : key_j > T} + min(#{j < i : key_j == T}, k_eq).
//
// Two schedules:
//  * rows of up to 16384 keys (prefill): one 1024-thread workgroup per row,
//    the row staged once in LDS, four 8-bit histogram passes, then an
//    in-order compaction with block prefix sums;
//  * long rows (decode at long context): each row is cut into 16384-key
//    segments, one workgroup per segment holds its keys in registers, and
//    four short kernels replace the serial passes:
//      1. per-segment histogram of key bits 31..21 (2048 bins);
//      2. every segment sums the row's bit-31..21 histograms, finds that
//         digit of T, and histograms bits 20..10 of the keys that share it;
//      3. every segment finds bits 31..10 of T and writes, in index order,
//         the keys above that prefix ("definite") and the keys on it
//         ("candidates", low 10 bits + index);
//      4. one workgroup per row resolves the last 10 bits of T among the
//         candidates and merges the two ascending lists into the output.
//    Per-segment histograms are plain stores (no atomics, no zeroing); a row
//    whose candidates overflow their buffers falls back to the one-workgroup
//    method reading the row from global memory.
#include "device_common.h"
#include "launch.h"

namespace dsa {
namespace {

constexpr int TK_THREADS = 1024;
constexpr int TK_WAVES = TK_THREADS / 64;
constexpr int TK_CAP = 16384;         // longest row staged in LDS by the one-workgroup method
constexpr int SEG = 16384;            // segment length of the long-row method
constexpr int SEG_PER_T = SEG / TK_THREADS;
constexpr int HB = 2048;              // bins of an 11-bit digit
constexpr int CAND_CAP = 1024;        // candidates a segment may hand over
constexpr int ROW_CAND_CAP = 8192;    // candidates the final step can hold for one row
constexpr int LONG_MAX_K = 4096;      // largest K of the long-row method
constexpr int64_t LONG_MAX_SEGS = 4096;  // bound on rows x segments (workspace size)

__device__ __forceinline__ int64_t n_visible(int64_t row, int64_t Tq, int64_t N, int64_t q_pos0) {
  return min(N, q_pos0 + row % Tq + 1);
}

// Exclusive block-wide prefix sum of v; `total` receives the block sum.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t& total, uint32_t* sbuf) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) sbuf[wave] = x;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < TK_WAVES; ++w) {
    const uint32_t s = sbuf[w];
    tot += s;
    before += (w < wave) ? s : 0u;
  }
  __syncthreads();
  total = tot;
  return before + x - v;
}

// Given a histogram `h` of `nb` bins (nb <= 2*TK_THREADS) over the keys that
// share the prefix found so far, find the digit holding the kk-th largest key.
// Returns the digit; `above` receives how many counted keys lie in higher bins.
__device__ __forceinline__ uint32_t find_digit(const uint32_t* h, int nb, uint32_t kk, uint32_t& above,
                                               uint32_t* sbuf, uint32_t* s_res) {
  const int tid = threadIdx.x;
  // thread t owns bins nb-1-2t and nb-2-2t (descending order)
  const int b0 = nb - 1 - 2 * tid, b1 = b0 - 1;
  const uint32_t c0 = b0 >= 0 ? h[b0] : 0u, c1 = b1 >= 0 ? h[b1] : 0u;
  uint32_t tot;
  const uint32_t ex = block_excl_scan(c0 + c1, tot, sbuf);
  if (b0 >= 0 && ex < kk && kk <= ex + c0) {
    s_res[0] = (uint32_t)b0;
    s_res[1] = ex;
  } else if (b1 >= 0 && ex + c0 < kk && kk <= ex + c0 + c1) {
    s_res[0] = (uint32_t)b1;
    s_res[1] = ex + c0;
  }
  __syncthreads();
  above = s_res[1];
  const uint32_t d = s_res[0];
  __syncthreads();
  return d;
}

// The one-workgroup method for one row.  skey: LDS stage of TK_CAP keys, or
// nullptr to read the row from global memory on every pass.
__device__ void select_row(const float* __restrict__ src, int64_t n, int K, int32_t* __restrict__ out,
                           uint32_t* skey, uint32_t* hist, uint32_t* sbuf, uint32_t* s_res) {
  const int tid = threadIdx.x;
  if (n <= K) {
    for (int64_t i = tid; i < K; i += TK_THREADS) out[i] = i < n ? (int32_t)i : -1;
    return;
  }
  if (skey != nullptr) {
    for (int64_t i = tid; i < n; i += TK_THREADS) skey[i] = float_order_key(src[i]);
    __syncthreads();
  }
  auto key_at = [&](int64_t i) -> uint32_t { return skey != nullptr ? skey[i] : float_order_key(src[i]); };

  uint32_t prefix = 0, mask = 0, kk = (uint32_t)K;
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int64_t base = tid; base < n; base += 8 * TK_THREADS) {
      uint32_t k[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t i = base + (int64_t)u * TK_THREADS;
        k[u] = i < n ? key_at(i) : 0u;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t i = base + (int64_t)u * TK_THREADS;
        if (i < n && (k[u] & mask) == prefix) atomicAdd(&hist[(k[u] >> shift) & 255u], 1u);
      }
    }
    __syncthreads();
    uint32_t above;
    const uint32_t d = find_digit(hist, 256, kk, above, sbuf, s_res);
    prefix |= d << shift;
    mask |= 255u << shift;
    kk -= above;
  }
  const uint32_t T = prefix, keq = kk;

  uint32_t run_gt = 0, run_eq = 0;
  for (int64_t base = 0; base < n; base += TK_THREADS) {
    const int64_t i = base + tid;
    uint32_t gt = 0, eq = 0;
    if (i < n) {
      const uint32_t k = key_at(i);
      gt = k > T;
      eq = k == T;
    }
    uint32_t tot;
    const uint32_t ex = block_excl_scan((eq << 16) | gt, tot, sbuf);
    const uint32_t gb = run_gt + (ex & 0xffffu), eb = run_eq + (ex >> 16);
    if (gt) out[gb + min(eb, keq)] = (int32_t)i;
    else if (eq && eb < keq) out[gb + eb] = (int32_t)i;
    run_gt += tot & 0xffffu;
    run_eq += tot >> 16;
  }
}

__global__ __launch_bounds__(TK_THREADS) void topk_rows_kernel(const float* __restrict__ scores,
                                                               int32_t* __restrict__ idx, int64_t Tq,
                                                               int64_t N, int64_t q_pos0, int K) {
  __shared__ uint32_t skey[TK_CAP];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sbuf[TK_WAVES];
  __shared__ uint32_t s_res[2];
  const int64_t row = blockIdx.x;
  const int64_t n = n_visible(row, Tq, N, q_pos0);
  select_row(scores + row * N, n, K, idx + row * K, n <= TK_CAP ? skey : nullptr, hist, sbuf, s_res);
}

// ---------------------------------------------------------------- long rows

struct LongWs {
  uint32_t* hist1;  // [R][G][HB]
  uint32_t* hist2;  // [R][G][HB]
  uint32_t* defc;   // [R][G] definite keys per segment
  uint32_t* candc;  // [R][G] candidates per segment (may exceed CAND_CAP: overflow)
  int32_t* defi;    // [R][G][K] definite key indices, ascending within a segment
  uint2* cand;      // [R][G][CAND_CAP] (low 10 key bits, index)
};

__host__ __device__ inline size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

__host__ __device__ inline LongWs long_ws(void* base, int64_t R, int G, int K) {
  char* p = static_cast<char*>(base);
  LongWs w;
  const size_t hs = align_up((size_t)R * G * HB * 4);
  w.hist1 = reinterpret_cast<uint32_t*>(p);
  w.hist2 = reinterpret_cast<uint32_t*>(p + hs);
  w.defc = reinterpret_cast<uint32_t*>(p + 2 * hs);
  w.candc = w.defc + (size_t)R * G;
  const size_t cs = align_up((size_t)R * G * 8);
  w.defi = reinterpret_cast<int32_t*>(p + 2 * hs + cs);
  w.cand = reinterpret_cast<uint2*>(p + 2 * hs + cs + align_up((size_t)R * G * K * 4));
  return w;
}

size_t long_ws_bytes(int64_t R, int G, int K) {
  return 2 * align_up((size_t)R * G * HB * 4) + align_up((size_t)R * G * 8) + align_up((size_t)R * G * K * 4) +
         align_up((size_t)R * G * CAND_CAP * 8);
}

// Keys of this workgroup's segment, SEG_PER_T per thread (index seg0 + tid + 1024*u).
__device__ __forceinline__ void load_segment(const float* __restrict__ src, int64_t seg0, int64_t n,
                                             uint32_t (&k)[SEG_PER_T]) {
#pragma unroll
  for (int u = 0; u < SEG_PER_T; ++u) {
    const int64_t i = seg0 + threadIdx.x + (int64_t)u * TK_THREADS;
    k[u] = i < n ? float_order_key(src[i]) : 0u;
  }
}

// hs[b] = sum over the row's nseg segment histograms h[seg][b].
__device__ __forceinline__ void sum_hist(const uint32_t* __restrict__ h, int nseg, uint32_t* hs) {
  for (int b = threadIdx.x; b < HB; b += TK_THREADS) {
    uint32_t s = 0;
    for (int g = 0; g < nseg; ++g) s += h[(size_t)g * HB + b];
    hs[b] = s;
  }
  __syncthreads();
}

__global__ __launch_bounds__(TK_THREADS) void topk_seg_hist1(const float* __restrict__ scores, LongWs ws,
                                                             int64_t Tq, int64_t N, int64_t q_pos0, int K, int G) {
  __shared__ uint32_t h[HB];
  const int64_t row = blockIdx.y;
  const int g = blockIdx.x;
  const int64_t n = n_visible(row, Tq, N, q_pos0);
  const int64_t seg0 = (int64_t)g * SEG;
  if (n <= K || seg0 >= n) return;
  for (int b = threadIdx.x; b < HB; b += TK_THREADS) h[b] = 0;
  uint32_t k[SEG_PER_T];
  load_segment(scores + row * N, seg0, n, k);
  __syncthreads();
#pragma unroll
  for (int u = 0; u < SEG_PER_T; ++u)
    if (seg0 + threadIdx.x + (int64_t)u * TK_THREADS < n) atomicAdd(&h[k[u] >> 21], 1u);
  __syncthreads();
  uint32_t* dst = ws.hist1 + ((size_t)row * G + g) * HB;
  for (int b = threadIdx.x; b < HB; b += TK_THREADS) dst[b] = h[b];
}

__global__ __launch_bounds__(TK_THREADS) void topk_seg_hist2(const float* __restrict__ scores, LongWs ws,
                                                             int64_t Tq, int64_t N, int64_t q_pos0, int K, int G) {
  __shared__ uint32_t h[HB];
  __shared__ uint32_t hs[HB];
  __shared__ uint32_t sbuf[TK_WAVES];
  __shared__ uint32_t s_res[2];
  const int64_t row = blockIdx.y;
  const int g = blockIdx.x;
  const int64_t n = n_visible(row, Tq, N, q_pos0);
  const int64_t seg0 = (int64_t)g * SEG;
  if (n <= K || seg0 >= n) return;
  const int nseg = (int)((n + SEG - 1) / SEG);
  uint32_t k[SEG_PER_T];
  load_segment(scores + row * N, seg0, n, k);
  for (int b = threadIdx.x; b < HB; b += TK_THREADS) h[b] = 0;
  sum_hist(ws.hist1 + (size_t)row * G * HB, nseg, hs);
  uint32_t above;
  const uint32_t d1 = find_digit(hs, HB, (uint32_t)K, above, sbuf, s_res);
#pragma unroll
  for (int u = 0; u < SEG_PER_T; ++u)
    if (seg0 + threadIdx.x + (int64_t)u * TK_THREADS < n && (k[u] >> 21) == d1)
      atomicAdd(&h[(k[u] >> 10) & (HB - 1)], 1u);
  __syncthreads();
  uint32_t* dst = ws.hist2 + ((size_t)row * G + g) * HB;
  for (int b = threadIdx.x; b < HB; b += TK_THREADS) dst[b] = h[b];
}

__global__ __launch_bounds__(TK_THREADS) void topk_seg_classify(const float* __restrict__ scores, LongWs ws,
                                                                int64_t Tq, int64_t N, int64_t q_pos0, int K,
                                                                int G) {
  __shared__ uint32_t hs[HB];
  __shared__ uint32_t sbuf[TK_WAVES];
  __shared__ uint32_t s_res[2];
  const int64_t row = blockIdx.y;
  const int g = blockIdx.x;
  const int64_t n = n_visible(row, Tq, N, q_pos0);
  const int64_t seg0 = (int64_t)g * SEG;
  if (n <= K || seg0 >= n) return;
  const int nseg = (int)((n + SEG - 1) / SEG);
  uint32_t k[SEG_PER_T];
  load_segment(scores + row * N, seg0, n, k);
  uint32_t above;
  sum_hist(ws.hist1 + (size_t)row * G * HB, nseg, hs);
  const uint32_t d1 = find_digit(hs, HB, (uint32_t)K, above, sbuf, s_res);
  const uint32_t kk1 = (uint32_t)K - above;
  sum_hist(ws.hist2 + (size_t)row * G * HB, nseg, hs);
  const uint32_t d2 = find_digit(hs, HB, kk1, above, sbuf, s_res);
  const uint32_t p22 = (d1 << 11) | d2;

  const size_t sidx = (size_t)row * G + g;
  int32_t* defi = ws.defi + sidx * K;
  uint2* cand = ws.cand + sidx * CAND_CAP;
  uint32_t run_def = 0, run_cand = 0;
#pragma unroll
  for (int u = 0; u < SEG_PER_T; ++u) {
    const int64_t i = seg0 + threadIdx.x + (int64_t)u * TK_THREADS;
    const bool valid = i < n;
    const uint32_t top = k[u] >> 10;
    const uint32_t isdef = valid && top > p22, iscand = valid && top == p22;
    uint32_t tot;
    const uint32_t ex = block_excl_scan((iscand << 16) | isdef, tot, sbuf);
    if (isdef) defi[run_def + (ex & 0xffffu)] = (int32_t)i;
    if (iscand) {
      const uint32_t pos = run_cand + (ex >> 16);
      if (pos < CAND_CAP) cand[pos] = make_uint2(k[u] & 1023u, (uint32_t)i);
    }
    run_def += tot & 0xffffu;
    run_cand += tot >> 16;
  }
  if (threadIdx.x == 0) {
    ws.defc[sidx] = run_def;
    ws.candc[sidx] = run_cand;
  }
}

__global__ __launch_bounds__(TK_THREADS) void topk_seg_final(const float* __restrict__ scores, LongWs ws,
                                                             int32_t* __restrict__ idx, int64_t Tq, int64_t N,
                                                             int64_t q_pos0, int K, int G) {
  __shared__ uint32_t ck[ROW_CAND_CAP];   // candidate low key bits, index order
  __shared__ int32_t ci[ROW_CAND_CAP];    // candidate indices
  __shared__ int32_t dl[LONG_MAX_K];      // definite indices, ascending
  __shared__ int32_t sl[LONG_MAX_K];      // kept candidate indices, ascending
  __shared__ uint32_t h[1024];
  __shared__ uint32_t sbuf[TK_WAVES];
  __shared__ uint32_t s_res[2];
  __shared__ uint32_t s_off[2];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int64_t n = n_visible(row, Tq, N, q_pos0);
  int32_t* out = idx + row * K;
  if (n <= K) {
    for (int64_t i = tid; i < K; i += TK_THREADS) out[i] = i < n ? (int32_t)i : -1;
    return;
  }
  const int nseg = (int)((n + SEG - 1) / SEG);
  const size_t s0 = (size_t)row * G;
  uint32_t ndef = 0, ncand = 0;
  bool overflow = false;
  for (int g = 0; g < nseg; ++g) {
    const uint32_t c = ws.candc[s0 + g];
    overflow |= c > CAND_CAP;
    ndef += ws.defc[s0 + g];
    ncand += c;
  }
  if (overflow || ncand > ROW_CAND_CAP) {
    // many equal keys at the boundary: exact one-workgroup method over the whole row
    select_row(scores + row * N, n, K, out, nullptr, h, sbuf, s_res);
    return;
  }
  // gather both lists in segment order (ascending index)
  uint32_t doff = 0, coff = 0;
  for (int g = 0; g < nseg; ++g) {
    const uint32_t dc = ws.defc[s0 + g], cc = ws.candc[s0 + g];
    for (uint32_t j = tid; j < dc; j += TK_THREADS) dl[doff + j] = ws.defi[(s0 + g) * K + j];
    for (uint32_t j = tid; j < cc; j += TK_THREADS) {
      const uint2 v = ws.cand[(s0 + g) * CAND_CAP + j];
      ck[coff + j] = v.x;
      ci[coff + j] = (int32_t)v.y;
    }
    doff += dc;
    coff += cc;
  }
  for (int b = tid; b < 1024; b += TK_THREADS) h[b] = 0;
  __syncthreads();
  for (uint32_t j = tid; j < ncand; j += TK_THREADS) atomicAdd(&h[ck[j]], 1u);
  __syncthreads();
  const uint32_t kk = (uint32_t)K - ndef;  // candidates to keep (1 <= kk <= ncand)
  uint32_t above;
  const uint32_t d3 = find_digit(h, 1024, kk, above, sbuf, s_res);
  const uint32_t keq = kk - above;
  // kept candidates, in index order
  uint32_t run_sel = 0, run_eq = 0;
  for (uint32_t base = 0; base < ncand; base += TK_THREADS) {
    const uint32_t j = base + tid;
    uint32_t gt = 0, eq = 0;
    if (j < ncand) {
      gt = ck[j] > d3;
      eq = ck[j] == d3;
    }
    uint32_t tot;
    const uint32_t ex = block_excl_scan((eq << 16) | gt, tot, sbuf);
    const uint32_t gb = run_sel + (ex & 0xffffu), eb = run_eq + (ex >> 16);
    if (gt) sl[gb + min(eb, keq)] = ci[j];
    else if (eq && eb < keq) sl[gb + eb] = ci[j];
    run_sel += tot & 0xffffu;
    run_eq += tot >> 16;
  }
  __syncthreads();
  // merge two ascending, disjoint lists: slot = own rank + rank in the other list
  auto lower = [](const int32_t* a, uint32_t len, int32_t v) {
    uint32_t lo = 0, hi = len;
    while (lo < hi) {
      const uint32_t mid = (lo + hi) >> 1;
      if (a[mid] < v) lo = mid + 1;
      else hi = mid;
    }
    return lo;
  };
  for (uint32_t j = tid; j < ndef; j += TK_THREADS) out[j + lower(sl, kk, dl[j])] = dl[j];
  for (uint32_t j = tid; j < kk; j += TK_THREADS) out[j + lower(dl, ndef, sl[j])] = sl[j];
  (void)s_off;
}

int long_segments(int64_t N) { return (int)((N + SEG - 1) / SEG); }

bool use_long_path(int64_t B, int64_t Tq, int64_t N, int K) {
  return N > TK_CAP && K <= LONG_MAX_K && B * Tq * long_segments(N) <= LONG_MAX_SEGS;
}

}  // namespace

size_t topk_workspace_bytes(int64_t B, int64_t Tq, int64_t N, int K) {
  if (!use_long_path(B, Tq, N, K)) return 0;
  return long_ws_bytes(B * Tq, long_segments(N), K);
}

hipError_t launch_topk(const float* scores, int32_t* idx, int64_t B, int64_t Tq, int64_t N, int64_t q_pos0,
                       int K, void* workspace, hipStream_t stream) {
  const int64_t R = B * Tq;
  const int64_t nmax = min(N, q_pos0 + Tq);
  if (nmax <= TK_CAP || !use_long_path(B, Tq, N, K)) {
    hipLaunchKernelGGL(topk_rows_kernel, dim3((unsigned)R), dim3(TK_THREADS), 0, stream, scores, idx, Tq, N, q_pos0,
                       K);
    return hipGetLastError();
  }
  const int G = long_segments(N);
  const LongWs ws = long_ws(workspace, R, G, K);
  const dim3 grid((unsigned)G, (unsigned)R);
  hipLaunchKernelGGL(topk_seg_hist1, grid, dim3(TK_THREADS), 0, stream, scores, ws, Tq, N, q_pos0, K, G);
  hipLaunchKernelGGL(topk_seg_hist2, grid, dim3(TK_THREADS), 0, stream, scores, ws, Tq, N, q_pos0, K, G);
  hipLaunchKernelGGL(topk_seg_classify, grid, dim3(TK_THREADS), 0, stream, scores, ws, Tq, N, q_pos0, K, G);
  hipLaunchKernelGGL(topk_seg_final, dim3((unsigned)R), dim3(TK_THREADS), 0, stream, scores, ws, idx, Tq, N,
                     q_pos0, K, G);
  return hipGetLastError();
}

}  // namespace dsa

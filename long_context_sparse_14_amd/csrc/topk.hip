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
//    the row staged once in LDS, three histogram passes (11, 11 and 10 bits),
//    then an in-order compaction with one block prefix sum per 16384 keys;
//  * long rows (decode at long context): each row is cut into 16384-key
//    segments, one workgroup per segment holds its keys in registers, and
//    four short kernels replace the serial passes:
//      1. per-segment histogram of key bits 31..21 (2048 bins);
//      2. every segment sums the row's bit-31..21 histograms, finds that
//         digit of T, and histograms bits 20..10 of the keys that share it;
//      3. every segment finds bits 31..10 of T (the top digit recorded by
//         step 2) and writes, in index order,
//         the keys above that prefix ("definite") and the keys on it
//         ("candidates", low 10 bits + index);
//      4. one workgroup per row resolves the last 10 bits of T among the
//         candidates and merges the two ascending lists into the output.
//    Per-segment histograms are plain stores (no atomics, no zeroing); a row
//    whose candidates overflow their buffers falls back to the one-workgroup
//    method reading the row from global memory.
// Histograms use plain LDS atomics: even for rows whose scores crowd into a
// few top-bit bins this measured faster than combining equal bins across a
// wave first.  Each thread owns a run of consecutive keys, so one block-wide
// prefix sum orders a whole chunk.
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
constexpr int ROW_CAND_CAP = 2048;    // candidates the final step can hold for one row
constexpr int LONG_MAX_K = 4096;      // largest K of the long-row method
constexpr int64_t LONG_MAX_SEGS = 4096;  // bound on rows x segments (workspace size)
constexpr int LONG_MAX_G = TK_THREADS;   // bound on segments per row (one thread per segment)
constexpr int RUN = 16;                  // consecutive keys per thread in a chunk
constexpr int CHUNK = RUN * TK_THREADS;  // keys ordered by one block prefix sum

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

// Writes the kept keys of the run [i0, i0 + RUN) (clipped to n) of one chunk:
// gt/eq are the per-thread counts before this thread within the whole row.
template <typename KeyAt>
__device__ __forceinline__ void emit_run(KeyAt key_at, int64_t i0, int64_t n, uint32_t T, uint32_t keq,
                                         uint32_t gt, uint32_t eq, int32_t* __restrict__ out) {
  for (int u = 0; u < RUN; ++u) {
    const int64_t i = i0 + u;
    if (i >= n) break;
    const uint32_t k = key_at(i);
    if (k > T) {
      out[gt + min(eq, keq)] = (int32_t)i;
      ++gt;
    } else if (k == T) {
      if (eq < keq) out[gt + eq] = (int32_t)i;
      ++eq;
    }
  }
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

  // three passes: key bits 31..21, 20..10, 9..0
  uint32_t prefix = 0, mask = 0, kk = (uint32_t)K;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nb = pass == 2 ? 1024 : HB;
    for (int b = tid; b < nb; b += TK_THREADS) hist[b] = 0;
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
        const bool hit = i < n && (k[u] & mask) == prefix;
        const uint32_t bin = (k[u] >> shift) & (uint32_t)(nb - 1);
        if (hit) atomicAdd(&hist[bin], 1u);
      }
    }
    __syncthreads();
    uint32_t above;
    const uint32_t d = find_digit(hist, nb, kk, above, sbuf, s_res);
    prefix |= d << shift;
    mask |= (uint32_t)(nb - 1) << shift;
    kk -= above;
  }
  const uint32_t T = prefix, keq = kk;

  // in-order compaction: thread t owns keys [base + RUN*t, base + RUN*t + RUN)
  uint32_t run_gt = 0, run_eq = 0;
  for (int64_t base = 0; base < n; base += CHUNK) {
    const int64_t i0 = base + (int64_t)RUN * tid;
    uint32_t gt = 0, eq = 0;
    for (int u = 0; u < RUN; ++u) {
      const int64_t i = i0 + u;
      if (i >= n) break;
      const uint32_t k = key_at(i);
      gt += k > T;
      eq += k == T;
    }
    uint32_t tot;
    const uint32_t ex = block_excl_scan((eq << 16) | gt, tot, sbuf);
    emit_run(key_at, i0, n, T, keq, run_gt + (ex & 0xffffu), run_eq + (ex >> 16), out);
    run_gt += tot & 0xffffu;
    run_eq += tot >> 16;
  }
}

__global__ __launch_bounds__(TK_THREADS) void topk_rows_kernel(const float* __restrict__ scores,
                                                               int32_t* __restrict__ idx, int64_t Tq,
                                                               int64_t N, int64_t q_pos0, int K) {
  __shared__ uint32_t skey[TK_CAP];
  __shared__ uint32_t hist[HB];
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
  uint32_t* rowd1;  // [R][2] digit 31..21 of the row's threshold and the count of keys above it
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
  w.rowd1 = w.candc + (size_t)R * G;
  const size_t cs = align_up((size_t)R * G * 8 + (size_t)R * 8);
  w.defi = reinterpret_cast<int32_t*>(p + 2 * hs + cs);
  w.cand = reinterpret_cast<uint2*>(p + 2 * hs + cs + align_up((size_t)R * G * K * 4));
  return w;
}

size_t long_ws_bytes(int64_t R, int G, int K) {
  return 2 * align_up((size_t)R * G * HB * 4) + align_up((size_t)R * G * 8 + (size_t)R * 8) +
         align_up((size_t)R * G * K * 4) +
         align_up((size_t)R * G * CAND_CAP * 8);
}

// Keys of this workgroup's segment: thread t holds the run
// [seg0 + RUN*t, seg0 + RUN*t + RUN), 16-byte loads when the row allows.
__device__ __forceinline__ void load_segment(const float* __restrict__ src, int64_t seg0, int64_t n,
                                             uint32_t (&k)[SEG_PER_T]) {
  const int64_t i0 = seg0 + (int64_t)RUN * threadIdx.x;
  if ((reinterpret_cast<uintptr_t>(src) & 15) == 0 && i0 + RUN <= n) {
#pragma unroll
    for (int u = 0; u < SEG_PER_T / 4; ++u) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(src + i0 + 4 * u);
      k[4 * u + 0] = float_order_key(v.x);
      k[4 * u + 1] = float_order_key(v.y);
      k[4 * u + 2] = float_order_key(v.z);
      k[4 * u + 3] = float_order_key(v.w);
    }
  } else {
#pragma unroll
    for (int u = 0; u < SEG_PER_T; ++u) k[u] = i0 + u < n ? float_order_key(src[i0 + u]) : 0u;
  }
}

// hs[b] = sum over the row's nseg segment histograms h[seg][b]; loads are
// issued eight segments at a time so their latencies overlap.
__device__ __forceinline__ void sum_hist(const uint32_t* __restrict__ h, int nseg, uint32_t* hs) {
  for (int b = threadIdx.x; b < HB; b += TK_THREADS) {
    uint32_t s = 0;
    for (int g0 = 0; g0 < nseg; g0 += 8) {
      uint32_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = g0 + u < nseg ? h[(size_t)(g0 + u) * HB + b] : 0u;
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    hs[b] = s;
  }
  __syncthreads();
}

// Shared memory of the three segment steps.
struct SegSmem {
  uint32_t h[HB];
  uint32_t hs[HB];
  uint32_t sbuf[TK_WAVES];
  uint32_t s_res[2];
};

// Step 1: histogram of key bits 31..21 of this segment.
__device__ void seg_hist1(const uint32_t (&k)[SEG_PER_T], int64_t seg0, int64_t n, uint32_t* __restrict__ dst,
                          SegSmem& sm) {
  for (int b = threadIdx.x; b < HB; b += TK_THREADS) sm.h[b] = 0;
  __syncthreads();
  const int64_t i0 = seg0 + (int64_t)RUN * threadIdx.x;
#pragma unroll
  for (int u = 0; u < SEG_PER_T; ++u)
    if (i0 + u < n) atomicAdd(&sm.h[k[u] >> 21], 1u);
  __syncthreads();
  for (int b = threadIdx.x; b < HB; b += TK_THREADS) dst[b] = sm.h[b];
}

// Step 2: digit 31..21 of T from the row's step-1 histograms, then a
// histogram of bits 20..10 of this segment's keys that share it.
__device__ void seg_hist2(const uint32_t (&k)[SEG_PER_T], int64_t seg0, int64_t n, int K, int nseg,
                          const uint32_t* __restrict__ row_hist1, uint32_t* __restrict__ dst,
                          uint32_t* __restrict__ row_d1, bool first, SegSmem& sm) {
  for (int b = threadIdx.x; b < HB; b += TK_THREADS) sm.h[b] = 0;
  sum_hist(row_hist1, nseg, sm.hs);
  uint32_t above;
  const uint32_t d1 = find_digit(sm.hs, HB, (uint32_t)K, above, sm.sbuf, sm.s_res);
  if (first && threadIdx.x == 0) {  // every segment finds the same digit; the first records it for step 3
    row_d1[0] = d1;
    row_d1[1] = above;
  }
  const int64_t i0 = seg0 + (int64_t)RUN * threadIdx.x;
#pragma unroll
  for (int u = 0; u < SEG_PER_T; ++u)
    if (i0 + u < n && (k[u] >> 21) == d1) atomicAdd(&sm.h[(k[u] >> 10) & (HB - 1)], 1u);
  __syncthreads();
  for (int b = threadIdx.x; b < HB; b += TK_THREADS) dst[b] = sm.h[b];
}

// Step 3: bits 31..10 of T, then this segment's keys above that prefix
// (definite) and on it (candidates), in index order.
__device__ void seg_classify(const uint32_t (&k)[SEG_PER_T], int64_t seg0, int64_t n, int K, int nseg,
                             const uint32_t* __restrict__ row_d1, const uint32_t* __restrict__ row_hist2,
                             const LongWs& ws, size_t sidx, SegSmem& sm) {
  uint32_t above;
  const uint32_t d1 = row_d1[0];
  const uint32_t kk1 = (uint32_t)K - row_d1[1];
  sum_hist(row_hist2, nseg, sm.hs);
  const uint32_t d2 = find_digit(sm.hs, HB, kk1, above, sm.sbuf, sm.s_res);
  const uint32_t p22 = (d1 << 11) | d2;

  int32_t* defi = ws.defi + sidx * K;
  uint2* cand = ws.cand + sidx * CAND_CAP;
  const int64_t i0 = seg0 + (int64_t)RUN * threadIdx.x;
  uint32_t nd = 0, nc = 0;
#pragma unroll
  for (int u = 0; u < SEG_PER_T; ++u) {
    const bool valid = i0 + u < n;
    nd += valid && (k[u] >> 10) > p22;
    nc += valid && (k[u] >> 10) == p22;
  }
  uint32_t tot;
  const uint32_t ex = block_excl_scan((nc << 16) | nd, tot, sm.sbuf);
  uint32_t pd = ex & 0xffffu, pc = ex >> 16;
#pragma unroll
  for (int u = 0; u < SEG_PER_T; ++u) {
    if (i0 + u >= n) break;
    const uint32_t top = k[u] >> 10;
    if (top > p22) defi[pd++] = (int32_t)(i0 + u);
    else if (top == p22) {
      if (pc < CAND_CAP) cand[pc] = make_uint2(k[u] & 1023u, (uint32_t)(i0 + u));
      ++pc;
    }
  }
  if (threadIdx.x == 0) {
    ws.defc[sidx] = tot & 0xffffu;
    ws.candc[sidx] = tot >> 16;
  }
}

__global__ __launch_bounds__(TK_THREADS) void topk_seg_hist1(const float* __restrict__ scores, LongWs ws,
                                                             int64_t Tq, int64_t N, int64_t q_pos0, int K, int G) {
  __shared__ SegSmem sm;
  const int64_t row = blockIdx.y;
  const int g = blockIdx.x;
  const int64_t n = n_visible(row, Tq, N, q_pos0);
  const int64_t seg0 = (int64_t)g * SEG;
  if (n <= K || seg0 >= n) return;
  uint32_t k[SEG_PER_T];
  load_segment(scores + row * N, seg0, n, k);
  seg_hist1(k, seg0, n, ws.hist1 + ((size_t)row * G + g) * HB, sm);
}

__global__ __launch_bounds__(TK_THREADS) void topk_seg_hist2(const float* __restrict__ scores, LongWs ws,
                                                             int64_t Tq, int64_t N, int64_t q_pos0, int K, int G) {
  __shared__ SegSmem sm;
  const int64_t row = blockIdx.y;
  const int g = blockIdx.x;
  const int64_t n = n_visible(row, Tq, N, q_pos0);
  const int64_t seg0 = (int64_t)g * SEG;
  if (n <= K || seg0 >= n) return;
  uint32_t k[SEG_PER_T];
  load_segment(scores + row * N, seg0, n, k);
  seg_hist2(k, seg0, n, K, (int)((n + SEG - 1) / SEG), ws.hist1 + (size_t)row * G * HB,
            ws.hist2 + ((size_t)row * G + g) * HB, ws.rowd1 + 2 * row, g == 0, sm);
}

__global__ __launch_bounds__(TK_THREADS) void topk_seg_classify(const float* __restrict__ scores, LongWs ws,
                                                                int64_t Tq, int64_t N, int64_t q_pos0, int K,
                                                                int G) {
  __shared__ SegSmem sm;
  const int64_t row = blockIdx.y;
  const int g = blockIdx.x;
  const int64_t n = n_visible(row, Tq, N, q_pos0);
  const int64_t seg0 = (int64_t)g * SEG;
  if (n <= K || seg0 >= n) return;
  uint32_t k[SEG_PER_T];
  load_segment(scores + row * N, seg0, n, k);
  seg_classify(k, seg0, n, K, (int)((n + SEG - 1) / SEG), ws.rowd1 + 2 * row,
               ws.hist2 + (size_t)row * G * HB, ws, (size_t)row * G + g, sm);
}

// Shared memory of the final step.
struct FinalSmem {
  uint32_t ck[ROW_CAND_CAP];   // candidate low key bits, index order
  int32_t ci[ROW_CAND_CAP];    // candidate indices
  int32_t dl[LONG_MAX_K];      // definite indices, ascending
  int32_t sl[LONG_MAX_K];      // kept candidate indices, ascending
  uint32_t h[HB];              // 1024 bins here; 2048 in the fallback
  uint32_t sbuf[TK_WAVES];
  uint32_t s_res[2];
  uint32_t s_doff[LONG_MAX_G + 1];
  uint32_t s_coff[LONG_MAX_G + 1];
};

__device__ void seg_final_row(const float* __restrict__ scores, const LongWs& ws, int32_t* __restrict__ idx,
                              int64_t row, int64_t Tq, int64_t N, int64_t q_pos0, int K, int G, FinalSmem& sm) {
  uint32_t* ck = sm.ck;
  int32_t* ci = sm.ci;
  int32_t* dl = sm.dl;
  int32_t* sl = sm.sl;
  uint32_t* h = sm.h;
  uint32_t* sbuf = sm.sbuf;
  uint32_t* s_res = sm.s_res;
  uint32_t* s_doff = sm.s_doff;
  uint32_t* s_coff = sm.s_coff;
  const int tid = threadIdx.x;
  const int64_t n = n_visible(row, Tq, N, q_pos0);
  int32_t* out = idx + row * K;
  if (n <= K) {
    for (int64_t i = tid; i < K; i += TK_THREADS) out[i] = i < n ? (int32_t)i : -1;
    return;
  }
  const int nseg = (int)((n + SEG - 1) / SEG);
  const size_t s0 = (size_t)row * G;
  // per-segment list offsets: exclusive prefix sums of the counts (nseg <= TK_THREADS)
  {
    const uint32_t dc = tid < nseg ? ws.defc[s0 + tid] : 0u;
    const uint32_t cc = tid < nseg ? ws.candc[s0 + tid] : 0u;
    uint32_t dtot, ctot, otot;
    const uint32_t dex = block_excl_scan(dc, dtot, sbuf);
    const uint32_t cex = block_excl_scan(cc, ctot, sbuf);
    block_excl_scan(cc > CAND_CAP ? 1u : 0u, otot, sbuf);
    if (tid < nseg) {
      s_doff[tid] = dex;
      s_coff[tid] = cex;
    }
    if (tid == 0) {
      s_doff[nseg] = dtot;
      s_coff[nseg] = otot ? 0xffffffffu : ctot;
    }
    __syncthreads();
  }
  const uint32_t ndef = s_doff[nseg], ncand = s_coff[nseg];
  if (ncand > ROW_CAND_CAP) {
    // many equal keys at the boundary: exact one-workgroup method over the whole row
    select_row(scores + row * N, n, K, out, nullptr, h, sbuf, s_res);
    return;
  }
  // gather both lists in segment order (ascending index); every load independent
  auto seg_of = [&](const uint32_t* off, uint32_t j) {
    int lo = 0, hi = nseg;  // largest g with off[g] <= j
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (off[mid] <= j) lo = mid;
      else hi = mid;
    }
    return lo;
  };
  for (uint32_t j = tid; j < ndef; j += TK_THREADS) {
    const int g = seg_of(s_doff, j);
    dl[j] = ws.defi[(s0 + g) * K + (j - s_doff[g])];
  }
  for (uint32_t j = tid; j < ncand; j += TK_THREADS) {
    const int g = seg_of(s_coff, j);
    const uint2 v = ws.cand[(s0 + g) * CAND_CAP + (j - s_coff[g])];
    ck[j] = v.x;
    ci[j] = (int32_t)v.y;
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
}

__global__ __launch_bounds__(TK_THREADS) void topk_seg_final(const float* __restrict__ scores, LongWs ws,
                                                             int32_t* __restrict__ idx, int64_t Tq, int64_t N,
                                                             int64_t q_pos0, int K, int G) {
  __shared__ FinalSmem sm;
  seg_final_row(scores, ws, idx, blockIdx.x, Tq, N, q_pos0, K, G, sm);
}

int long_segments(int64_t N) { return (int)((N + SEG - 1) / SEG); }

bool use_long_path(int64_t B, int64_t Tq, int64_t N, int K) {
  return N > TK_CAP && K <= LONG_MAX_K && long_segments(N) <= LONG_MAX_G && B * Tq * long_segments(N) <= LONG_MAX_SEGS;
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

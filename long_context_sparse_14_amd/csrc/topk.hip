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
//    the row staged once in LDS with its key range, then exact select rounds
//    that each split the remaining range into 2048 bins (ceil(bits / 11)
//    rounds for a range of that many bits), then an in-order compaction with
//    one block prefix sum per 16384 keys;
//  * long rows (decode at long context): each row is cut into 16384-key
//    segments, and two kernels replace the serial passes:
//      1. one workgroup per segment holds its keys in registers, finds bounds
//         t_lo <= t_hi on T from a 4096-key sample of the row (exact selects
//         at two sample ranks around the one expected to hold T; every
//         segment of a row derives the same bounds), and writes, in index
//         order, key and index of its keys at or above t_lo: those above
//         t_hi are "definite", those in [t_lo, t_hi] "candidates";
//      2. one workgroup per row checks that at most K keys are definite and
//         at least K are definite or candidates, holds the row's list in
//         registers, selects the K - #definite best candidates exactly, and
//         compacts the kept entries, already in index order, into the
//         output with one block prefix sum.
//    The scores are read once (plus the sample).  A row whose bounds miss or
//    whose candidates overflow their buffers (scores ordered by position, a
//    large block of equal keys at the cut) falls back to the one-workgroup
//    method reading the row from global memory.
// Histograms use plain LDS atomics; where the keys crowd into a narrow range
// (a sample, a candidate list) each thread first counts its own repeated bins
// in registers.  Each thread owns a run of consecutive keys, so one
// block-wide prefix sum orders a whole chunk.
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
constexpr int ROW_CAND_CAP = 4096;    // candidates the final step can hold for one row
constexpr int LONG_MAX_K = 4096;      // largest K of the long-row method
constexpr int64_t LONG_MAX_SEGS = 4096;  // bound on rows x segments (workspace size)
constexpr int LONG_MAX_G = TK_THREADS;   // bound on segments per row (one thread per segment)
constexpr int RUN = 16;                  // consecutive keys per thread in a chunk
constexpr int CHUNK = RUN * TK_THREADS;  // keys ordered by one block prefix sum

__device__ __forceinline__ int64_t n_visible(int64_t row, int64_t Tq, int64_t N, int64_t q_pos0, const Vis& vis) {
  return visible_keys(vis, seq_q0(vis, row / Tq, Tq, q_pos0), row % Tq, N);
}

// Exclusive block-wide prefix sum of v; `total` receives the block sum.
// Without TRAIL the closing barrier is left out, and the caller must pass
// another barrier before sbuf[0 .. TK_WAVES) is written again.
template <bool TRAIL = true>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t& total, uint32_t* sbuf) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t x = wave_incl_scan(v);
  if (lane == 63) sbuf[wave] = x;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < TK_WAVES; ++w) {
    const uint32_t s = sbuf[w];
    tot += s;
    before += (w < wave) ? s : 0u;
  }
  if (TRAIL) __syncthreads();
  total = tot;
  return before + x - v;
}

// ------------------------------------------------- range-adaptive select

// Histogram insertion for crowded bins (a row's keys, a sample or a candidate
// list often sit in a narrow range, so a whole wave's plain LDS atomics would
// queue on one address): a thread counts its first two distinct bins in
// registers and sends only other bins to LDS; each register count then goes
// out with one atomic, or with one atomic per wave when every lane of the
// wave holds the same bin.  flush() must be called by all 64 lanes of a wave.
struct HotBins {
  uint32_t b0 = 0u, c0 = 0u, b1 = 0u, c1 = 0u;
  __device__ __forceinline__ void add(uint32_t bin, uint32_t* h) {
    if (c0 != 0u && bin == b0) {
      ++c0;
    } else if (c1 != 0u && bin == b1) {
      ++c1;
    } else if (c0 == 0u) {
      b0 = bin;
      c0 = 1u;
    } else if (c1 == 0u) {
      b1 = bin;
      c1 = 1u;
    } else {
      atomicAdd(&h[bin], 1u);
    }
  }
  __device__ __forceinline__ static void flush_one(uint32_t b, uint32_t c, uint32_t* h) {
    const uint32_t bl = __builtin_amdgcn_readfirstlane(b);
    if (__ballot(c == 0u || b == bl) == ~0ull) {
      const uint32_t t = wave_sum(c);
      if ((threadIdx.x & 63) == 0 && t != 0u) atomicAdd(&h[bl], t);
    } else if (c != 0u) {
      atomicAdd(&h[b], c);
    }
  }
  __device__ __forceinline__ void flush(uint32_t* h) const {
    flush_one(b0, c0, h);
    flush_one(b1, c1, h);
  }
};

// Number of bits needed for x (0 for x == 0).
__device__ __forceinline__ int bit_width(uint32_t x) { return x == 0u ? 0 : 32 - __clz(x); }

// Given a histogram h of 2^FBITS bins, find for each of two descending ranks
// ra, rb (1-based, at most the histogram total) the bin that holds it;
// *_above receives how many counted keys lie in higher bins, count_a how many
// lie in bin ba.  s_res: 8 words; words 0..4 stay valid until the next call
// (whose own barriers precede its writes).  With ZERO each thread clears the
// bins it read, and the closing barrier publishes the cleared histogram.
template <int FBITS, bool ZERO = false>
__device__ __forceinline__ void find_two_bins(uint32_t* h, uint32_t ra, uint32_t rb, uint32_t& ba,
                                              uint32_t& above_a, uint32_t& bb, uint32_t& above_b,
                                              uint32_t& count_a, uint32_t* sbuf, uint32_t* s_res) {
  constexpr int NB = 1 << FBITS, PER_T = NB / TK_THREADS;
  static_assert(PER_T * TK_THREADS == NB, "whole bins per thread");
  const int tid = threadIdx.x;
  uint32_t c[PER_T], t = 0;
#pragma unroll
  for (int u = 0; u < PER_T; ++u) {  // thread t owns bins NB-1-PER_T*t-u, descending
    c[u] = h[NB - 1 - PER_T * tid - u];
    t += c[u];
  }
  if (ZERO)
#pragma unroll
    for (int u = 0; u < PER_T; ++u) h[NB - 1 - PER_T * tid - u] = 0u;
  uint32_t tot;
  uint32_t run = block_excl_scan<false>(t, tot, sbuf);  // the s_res barrier below closes it
#pragma unroll
  for (int u = 0; u < PER_T; ++u) {
    const uint32_t b = (uint32_t)(NB - 1 - PER_T * tid - u);
    if (run < ra && ra <= run + c[u]) {
      s_res[0] = b;
      s_res[1] = run;
      s_res[4] = c[u];
    }
    if (run < rb && rb <= run + c[u]) {
      s_res[2] = b;
      s_res[3] = run;
    }
    run += c[u];
  }
  __syncthreads();
  ba = s_res[0];
  above_a = s_res[1];
  bb = s_res[2];
  above_b = s_res[3];
  count_a = s_res[4];
}

// Block-wide smallest and largest of per-thread values (mn, mx).
// sbuf2: 2 * TK_WAVES words, written once per workgroup (no closing barrier).
__device__ __forceinline__ void block_min_max(uint32_t mn, uint32_t mx, uint32_t& kmin, uint32_t& kmax,
                                              uint32_t* sbuf2) {
  mn = wave_min(mn);
  mx = wave_max(mx);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    sbuf2[2 * wave] = mn;
    sbuf2[2 * wave + 1] = mx;
  }
  __syncthreads();
  mn = 0xffffffffu;
  mx = 0u;
#pragma unroll
  for (int w = 0; w < TK_WAVES; ++w) {
    mn = min(mn, sbuf2[2 * w]);
    mx = max(mx, sbuf2[2 * w + 1]);
  }
  kmin = mn;
  kmax = mx;
}

// Exact select among the keys in [lo, hi] of a key set: the key value at
// descending rank r (1 <= r <= their number), and in `above` how many of them
// exceed it.  Each round splits the remaining key range into 2^FBITS bins of
// (key - lo) >> shift and keeps the bin holding rank r, so a range of b bits
// takes at most ceil(b / FBITS) rounds.  add_keys(hb, lo, hi, shift) must pass
// every key of the set in [lo, hi] to hb.add((key - lo) >> shift, h), and
// each_key(lo, hi, fn) must call fn(key) for the same keys.  Once the kept bin
// holds at most 64 keys they are copied to `small` (65 words) and one wave
// ranks them directly, in place of further histogram rounds.  On entry all
// 2^FBITS bins of h and the counter small[64] must be zero, made visible by a
// barrier; each round's bin search clears the histogram for the next one.
template <int FBITS, typename AddKeys, typename EachKey>
__device__ uint32_t select_rank(AddKeys add_keys, EachKey each_key, uint32_t lo, uint32_t hi, uint32_t r,
                                uint32_t& above, uint32_t* h, uint32_t* sbuf, uint32_t* s_res, uint32_t* small) {
  above = 0;
#pragma unroll 1
  while (true) {
    const int shift = max(0, bit_width(hi - lo) - FBITS);
    HotBins hb;
    add_keys(hb, lo, hi, shift);
    hb.flush(h);
    __syncthreads();
    uint32_t b, ab, b2, ab2, cnt;
    find_two_bins<FBITS, true>(h, r, r, b, ab, b2, ab2, cnt, sbuf, s_res);
    above += ab;
    r -= ab;
    const uint32_t nlo = lo + (b << shift);
    const uint32_t nhi = (uint32_t)min((uint64_t)hi, (uint64_t)nlo + ((uint64_t)1 << shift) - 1);
    lo = nlo;
    hi = nhi;
    if (shift == 0) return lo;
    if (cnt <= 64u) {
      each_key(lo, hi, [&](uint32_t k) {
        const uint32_t s = atomicAdd(&small[64], 1u);
        if (s < 64u) small[s] = k;
      });
      __syncthreads();
      if (threadIdx.x < 64) {  // lane i: how many of the bin's keys exceed / equal its own
        const uint32_t i = threadIdx.x;
        const uint32_t ki = i < cnt ? small[i] : 0u;
        uint32_t gt = 0, eq = 0;
        for (uint32_t j = 0; j < cnt; ++j) {
          const uint32_t kj = small[j];
          gt += kj > ki;
          eq += kj == ki;
        }
        if (i < cnt && gt < r && r <= gt + eq) {  // lanes holding the key at rank r agree
          s_res[5] = ki;
          s_res[6] = gt;
        }
        if (i == 0) small[64] = 0u;  // every append is done: reset the counter
      }
      __syncthreads();
      above += s_res[6];
      return s_res[5];
    }
  }
}

// Writes the kept keys of the run [i0, i0 + RUN) (clipped to n) of one chunk:
// gt/eq are the per-thread counts before this thread within the whole row.
template <typename KeyAt>
__device__ __forceinline__ void emit_run(KeyAt key_at, int i0, int n, uint32_t T, uint32_t keq,
                                         uint32_t gt, uint32_t eq, int32_t* __restrict__ out) {
  for (int u = 0; u < RUN; ++u) {
    const int i = i0 + u;
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
// nullptr to read the row from global memory on every pass.  hist: 2048 bins;
// sbuf: 3 * TK_WAVES words; s_res: 8 words; small: 65 words.
__device__ __forceinline__ void select_row(const float* __restrict__ src, int64_t n, int K, int32_t* __restrict__ out,
                           uint32_t* skey, uint32_t* hist, uint32_t* sbuf, uint32_t* s_res, uint32_t* small) {
  const int tid = threadIdx.x;
  if (n <= K) {
    for (int64_t i = tid; i < K; i += TK_THREADS) out[i] = i < n ? (int32_t)i : -1;
    return;
  }
  // keys (staged in LDS when skey is given) and their range; eight loads in
  // flight per thread
  // (row offsets fit 32 bits: N < 2^31)
  const int n32 = (int)n;
  uint32_t mn = 0xffffffffu, mx = 0u;
  for (int base = tid; base < n32; base += 8 * TK_THREADS) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = base + u * TK_THREADS;
      v[u] = i < n32 ? src[i] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = base + u * TK_THREADS;
      if (i < n32) {
        const uint32_t k = float_order_key(v[u]);
        if (skey != nullptr) skey[i] = k;
        mn = min(mn, k);
        mx = max(mx, k);
      }
    }
  }
  for (int b = tid; b < HB; b += TK_THREADS) hist[b] = 0u;  // the select starts from empty bins
  if (tid == 0) small[64] = 0u;
  uint32_t kmin, kmax;
  block_min_max(mn, mx, kmin, kmax, sbuf + TK_WAVES);  // its barrier also publishes skey and the bins
  auto key_at = [&](int i) -> uint32_t { return skey != nullptr ? skey[i] : float_order_key(src[i]); };
  // (the bins span the keys' own range, so plain atomics rarely collide)
  auto add_row = [&](HotBins&, uint32_t lo, uint32_t hi, int shift) {
    for (int base = tid; base < n32; base += 8 * TK_THREADS) {
      uint32_t k[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = base + u * TK_THREADS;
        k[u] = i < n32 ? key_at(i) : 0u;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = base + u * TK_THREADS;
        if (i < n32 && k[u] >= lo && k[u] <= hi) atomicAdd(&hist[(k[u] - lo) >> shift], 1u);
      }
    }
  };
  auto each_row = [&](uint32_t lo, uint32_t hi, auto fn) {
    for (int base = tid; base < n32; base += 8 * TK_THREADS) {
      uint32_t k[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = base + u * TK_THREADS;
        k[u] = i < n32 ? key_at(i) : 0u;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = base + u * TK_THREADS;
        if (i < n32 && k[u] >= lo && k[u] <= hi) fn(k[u]);
      }
    }
  };
  uint32_t above;
  const uint32_t T = select_rank<11>(add_row, each_row, kmin, kmax, (uint32_t)K, above, hist, sbuf, s_res, small);
  const uint32_t keq = (uint32_t)K - above;

  // in-order compaction: thread t owns keys [base + RUN*t, base + RUN*t + RUN)
  uint32_t run_gt = 0, run_eq = 0;
  for (int base = 0; base < n32; base += CHUNK) {
    const int i0 = base + RUN * tid;
    uint32_t gt = 0, eq = 0;
    for (int u = 0; u < RUN; ++u) {
      const int i = i0 + u;
      if (i >= n32) break;
      const uint32_t k = key_at(i);
      gt += k > T;
      eq += k == T;
    }
    uint32_t tot;
    const uint32_t ex = block_excl_scan((eq << 16) | gt, tot, sbuf);
    emit_run(key_at, i0, n32, T, keq, run_gt + (ex & 0xffffu), run_eq + (ex >> 16), out);
    run_gt += tot & 0xffffu;
    run_eq += tot >> 16;
  }
}

__global__ __launch_bounds__(TK_THREADS) void topk_rows_kernel(const float* __restrict__ scores,
                                                               int32_t* __restrict__ idx, int64_t Tq,
                                                               int64_t N, int64_t q_pos0, Vis vis, int K) {
  __shared__ uint32_t skey[TK_CAP];
  __shared__ uint32_t hist[HB];
  __shared__ uint32_t sbuf[3 * TK_WAVES];
  __shared__ uint32_t s_res[8];
  __shared__ uint32_t small[65];
  const int64_t row = blockIdx.x;
  const int64_t n = n_visible(row, Tq, N, q_pos0, vis);
  select_row(scores + row * N, n, K, idx + row * K, n <= TK_CAP ? skey : nullptr, hist, sbuf, s_res, small);
}

// ---------------------------------------------------------------- long rows

constexpr int SAMPLE_BLOCKS = 64;                        // runs of consecutive keys in a row's sample
constexpr int SAMPLE_RUN = 64;                           // keys per run
constexpr int SAMPLES = SAMPLE_BLOCKS * SAMPLE_RUN;      // 4096
constexpr int SAMPLE_PER_T = SAMPLES / TK_THREADS;       // 4
static_assert(SAMPLE_PER_T * TK_THREADS == SAMPLES && SAMPLE_RUN % SAMPLE_PER_T == 0, "sample geometry");

constexpr int FB_BITS = 12;               // bins of the long-row histograms: 4096
constexpr int FB = 1 << FB_BITS;

// A segment's list holds its keys at or above t_lo in index order, definite
// and candidate keys together: at most K + CAND_CAP entries whenever the
// final step's checks pass.
struct LongWs {
  uint32_t* defc;   // [R][G] definite keys per segment (may exceed K: the bounds missed)
  uint32_t* candc;  // [R][G] candidates per segment (may exceed CAND_CAP: overflow)
  uint2* bounds;    // [R] (t_lo, t_hi), written by segment 0 of the row
  uint2* list;      // [R][G][cap] (key, index) of keys >= t_lo, ascending index
  int cap;          // K + CAND_CAP
};

__host__ __device__ inline size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

__host__ __device__ inline LongWs long_ws(void* base, int64_t R, int G, int K) {
  char* p = static_cast<char*>(base);
  LongWs w;
  const size_t cs = align_up((size_t)R * G * 8);
  w.defc = reinterpret_cast<uint32_t*>(p);
  w.candc = w.defc + (size_t)R * G;
  w.bounds = reinterpret_cast<uint2*>(p + cs);
  w.list = reinterpret_cast<uint2*>(p + cs + align_up((size_t)R * 8));
  w.cap = K + CAND_CAP;
  return w;
}

size_t long_ws_bytes(int64_t R, int G, int K) {
  return align_up((size_t)R * G * 8) + align_up((size_t)R * 8) + align_up((size_t)R * G * (K + CAND_CAP) * 8);
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

// Bounds on the row's threshold from a sample of its keys: SAMPLE_BLOCKS runs
// of SAMPLE_RUN consecutive keys spread evenly over the row (the whole row
// when it has at most SAMPLES keys).  With e = K * S / n the expected sample
// rank of the K-th largest key, r_hi ~ e - 4 sqrt(e) and r_lo ~ e + 4 sqrt(e);
// one histogram over the sample's key range gives the bins holding those
// ranks, and t_hi is the top of the first, t_lo the bottom of the second (at
// most r_hi - 1 sample keys lie above t_hi, at least r_lo lie at or above
// t_lo).  Any two keys would keep the method exact (the final step checks
// them); these make the checks pass with overwhelming probability unless the
// scores are strongly ordered by position, and keep the candidate list short.
__device__ __forceinline__ void sample_bounds(const float* __restrict__ src, int64_t n, int K, uint32_t& t_hi, uint32_t& t_lo,
                              uint32_t* h, uint32_t* sbuf, uint32_t* s_res) {
  uint32_t k[SAMPLE_PER_T];
  bool valid[SAMPLE_PER_T];
  int S;
  if (n <= SAMPLES) {
    S = (int)n;
#pragma unroll
    for (int u = 0; u < SAMPLE_PER_T; ++u) {
      const int j = (int)threadIdx.x + TK_THREADS * u;
      valid[u] = j < S;
      k[u] = valid[u] ? float_order_key(src[j]) : 0u;
    }
  } else {
    S = SAMPLES;
    const int j0 = SAMPLE_PER_T * (int)threadIdx.x;  // a thread's samples lie in one run
    const int64_t blk = j0 / SAMPLE_RUN;
    const int64_t start = blk * (n - SAMPLE_RUN) / (SAMPLE_BLOCKS - 1);
#pragma unroll
    for (int u = 0; u < SAMPLE_PER_T; ++u) {
      valid[u] = true;
      k[u] = float_order_key(src[start + (j0 % SAMPLE_RUN) + u]);
    }
  }
  const float e = (float)K * (float)S / (float)n;
  const float sd = 4.f * sqrtf(e) + 2.f;
  int r_hi = (int)floorf(e - sd), r_lo = (int)ceilf(e + sd);
  r_hi = max(1, min(r_hi, S));
  r_lo = max(r_hi, min(r_lo, S));
  uint32_t mn = 0xffffffffu, mx = 0u, kmin, kmax;
#pragma unroll
  for (int u = 0; u < SAMPLE_PER_T; ++u)
    if (valid[u]) {
      mn = min(mn, k[u]);
      mx = max(mx, k[u]);
    }
  for (int b = threadIdx.x; b < FB; b += TK_THREADS) h[b] = 0u;
  block_min_max(mn, mx, kmin, kmax, sbuf + TK_WAVES);  // its barrier also publishes the cleared bins
  const int shift = max(0, bit_width(kmax - kmin) - FB_BITS);
  {
    HotBins hb;
#pragma unroll
    for (int u = 0; u < SAMPLE_PER_T; ++u)
      if (valid[u]) hb.add((k[u] - kmin) >> shift, h);
    hb.flush(h);
  }
  __syncthreads();
  uint32_t b_hi, ab_hi, b_lo, ab_lo, c_hi;
  find_two_bins<FB_BITS>(h, (uint32_t)r_hi, (uint32_t)r_lo, b_hi, ab_hi, b_lo, ab_lo, c_hi, sbuf, s_res);
  t_hi = (uint32_t)min((uint64_t)kmax, (uint64_t)kmin + ((uint64_t)(b_hi + 1) << shift) - 1);
  t_lo = kmin + (b_lo << shift);
}

// Shared memory of the segment step.
struct SegSmem {
  uint32_t h[FB];
  uint32_t sbuf[3 * TK_WAVES];
  uint32_t s_res[8];
};

// Step 1, one workgroup per segment: the row's bounds t_lo <= t_hi from its
// sample (every segment of a row computes the same ones), then this
// segment's keys at or above t_lo, key and index, in index order: those above
// t_hi are "definite", those in [t_lo, t_hi] "candidates"; both are counted.
__global__ __launch_bounds__(TK_THREADS) void topk_seg_classify(const float* __restrict__ scores, LongWs ws,
                                                                int64_t Tq, int64_t N, int64_t q_pos0, Vis vis,
                                                                int K,
                                                                int G) {
  __shared__ SegSmem sm;
  const int64_t row = blockIdx.y;
  const int g = blockIdx.x;
  const int64_t n = n_visible(row, Tq, N, q_pos0, vis);
  const int64_t seg0 = (int64_t)g * SEG;
  if (n <= K || seg0 >= n) return;
  const float* src = scores + row * N;
  uint32_t k[SEG_PER_T];
  load_segment(src, seg0, n, k);
  uint32_t t_hi, t_lo;
  sample_bounds(src, n, K, t_hi, t_lo, sm.h, sm.sbuf, sm.s_res);

  const size_t sidx = (size_t)row * G + g;
  uint2* list = ws.list + sidx * ws.cap;
  const uint32_t cap = (uint32_t)ws.cap;
  const int64_t i0 = seg0 + (int64_t)RUN * threadIdx.x;
  uint32_t nd = 0, nc = 0;
#pragma unroll
  for (int u = 0; u < SEG_PER_T; ++u) {
    const bool v = i0 + u < n;
    nd += v && k[u] > t_hi;
    nc += v && k[u] >= t_lo && k[u] <= t_hi;
  }
  uint32_t tot;
  const uint32_t ex = block_excl_scan((nc << 16) | nd, tot, sm.sbuf);
  uint32_t pos = (ex & 0xffffu) + (ex >> 16);  // keys >= t_lo before this thread's run
#pragma unroll
  for (int u = 0; u < SEG_PER_T; ++u) {
    if (i0 + u >= n) break;
    if (k[u] >= t_lo) {
      if (pos < cap) list[pos] = make_uint2(k[u], (uint32_t)(i0 + u));
      ++pos;
    }
  }
  if (threadIdx.x == 0) {
    ws.defc[sidx] = tot & 0xffffu;
    ws.candc[sidx] = tot >> 16;
    if (g == 0) ws.bounds[row] = make_uint2(t_lo, t_hi);
  }
}

// Shared memory of the final step.
struct FinalSmem {
  uint32_t h[FB];               // FB >= HB: also the fallback's histogram
  uint32_t sbuf[3 * TK_WAVES];
  uint32_t s_res[8];
  uint32_t small[65];
  uint32_t s_loff[LONG_MAX_G + 1];  // list offsets of the segments in the row's list
};

// Step 2, one workgroup per row: check the bounds (the definite keys are at
// most K and, with the candidates, at least K; no segment's candidates
// overflowed), then treat the segments' lists, concatenated, as one list in
// index order.  Thread t holds entries [LPT*t, LPT*t + LPT) in registers.  The
// K - #definite best candidates are found by an exact select over the
// candidates' keys (the range [t_lo, t_hi] holds every candidate and no
// definite key), and one block prefix sum over the kept entries writes them,
// in index order, straight to the output.  If a check fails, the exact
// one-workgroup method runs over the row from global memory instead.
constexpr int LPT = (LONG_MAX_K + ROW_CAND_CAP) / TK_THREADS;  // list entries per thread
static_assert(LPT * TK_THREADS == LONG_MAX_K + ROW_CAND_CAP, "whole list entries per thread");

__device__ __forceinline__ void seg_final_row(const float* __restrict__ scores, const LongWs& ws, int32_t* __restrict__ idx,
                              int64_t row, int64_t Tq, int64_t N, int64_t q_pos0, const Vis& vis, int K, int G,
                              FinalSmem& sm) {
  const int tid = threadIdx.x;
  const int64_t n = n_visible(row, Tq, N, q_pos0, vis);
  int32_t* out = idx + row * K;
  if (n <= K) {
    for (int64_t i = tid; i < K; i += TK_THREADS) out[i] = i < n ? (int32_t)i : -1;
    return;
  }
  const int nseg = (int)((n + SEG - 1) / SEG);
  const size_t s0 = (size_t)row * G;
  // the select's histogram and small-bin counter start empty (published by
  // the barriers of the count scan below)
  for (int b = tid; b < FB; b += TK_THREADS) sm.h[b] = 0u;
  if (tid == 0) sm.small[64] = 0u;
  // per-segment list offsets: exclusive prefix sums of the list lengths
  // (nseg <= TK_THREADS); up to 64 segments (rows up to 2^20 keys) one wave
  // scans them without barriers
  bool ok;
  uint32_t ndef, ncand;
  if (nseg <= 64) {
    if (tid < 64) {
      const uint32_t dc = tid < nseg ? ws.defc[s0 + tid] : 0u;
      const uint32_t cc = tid < nseg ? ws.candc[s0 + tid] : 0u;
      const uint32_t ov = cc > CAND_CAP ? 1u : 0u;
      const uint32_t di = wave_incl_scan(dc), ci = wave_incl_scan(cc), oi = wave_incl_scan(ov);
      if (tid < nseg) sm.s_loff[tid] = di - dc + ci - cc;
      if (tid == 63) {  // lanes past nseg add nothing: lane 63 holds the totals
        sm.s_loff[nseg] = di + ci;
        sm.s_res[0] = oi;
        sm.s_res[1] = di;
        sm.s_res[2] = ci;
      }
    }
    __syncthreads();
    ok = sm.s_res[0] == 0;
    ndef = sm.s_res[1];
    ncand = sm.s_res[2];
  } else {
    const uint32_t dc = tid < nseg ? ws.defc[s0 + tid] : 0u;
    const uint32_t cc = tid < nseg ? ws.candc[s0 + tid] : 0u;
    uint32_t otot;
    const uint32_t dex = block_excl_scan(dc, ndef, sm.sbuf);
    const uint32_t cex = block_excl_scan(cc, ncand, sm.sbuf);
    block_excl_scan(cc > CAND_CAP ? 1u : 0u, otot, sm.sbuf);
    if (tid < nseg) sm.s_loff[tid] = dex + cex;
    if (tid == 0) sm.s_loff[nseg] = ndef + ncand;
    ok = otot == 0;
    __syncthreads();
  }
  ok = ok && ndef <= (uint32_t)K && ncand <= (uint32_t)ROW_CAND_CAP && ndef + ncand >= (uint32_t)K;
  if (!ok) {
    select_row(scores + row * N, n, K, out, nullptr, sm.h, sm.sbuf, sm.s_res, sm.small);
    return;
  }
  // this thread's entries of the row's list (every load independent)
  const uint32_t len = ndef + ncand;
  const uint32_t j0 = (uint32_t)LPT * (uint32_t)tid;
  uint32_t ck[LPT];
  int32_t ci[LPT];
  {
    int g = 0;  // segment of entry j0: the largest g with s_loff[g] <= j0
    if (j0 < len) {
      int lo = 0, hi = nseg;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (sm.s_loff[mid] <= j0) lo = mid;
        else hi = mid;
      }
      g = lo;
    }
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const uint32_t j = j0 + u;
      ck[u] = 0u;
      ci[u] = -1;
      if (j < len) {
        while (sm.s_loff[g + 1] <= j) ++g;
        const uint2 v = ws.list[(s0 + g) * ws.cap + (j - sm.s_loff[g])];
        ck[u] = v.x;
        ci[u] = (int32_t)v.y;
      }
    }
  }
  const uint2 bnd = ws.bounds[row];
  const uint32_t kk = (uint32_t)K - ndef;  // candidates to keep (0 <= kk <= ncand)
  uint32_t T = bnd.y, keq = 0;             // kk == 0: exactly the definite keys (> t_hi)
  if (kk > 0) {
    auto add_cand = [&](HotBins& hb, uint32_t lo, uint32_t hi, int shift) {
#pragma unroll
      for (int u = 0; u < LPT; ++u)
        if (ci[u] >= 0 && ck[u] >= lo && ck[u] <= hi) hb.add((ck[u] - lo) >> shift, sm.h);
    };
    auto each_cand = [&](uint32_t lo, uint32_t hi, auto fn) {
#pragma unroll
      for (int u = 0; u < LPT; ++u)
        if (ci[u] >= 0 && ck[u] >= lo && ck[u] <= hi) fn(ck[u]);
    };
    uint32_t above;
    T = select_rank<FB_BITS>(add_cand, each_cand, bnd.x, bnd.y, kk, above, sm.h, sm.sbuf, sm.s_res, sm.small);
    keq = kk - above;
  }
  // kept entries in index order: key > T, or key == T among the first keq
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int u = 0; u < LPT; ++u) {
    gt += ci[u] >= 0 && ck[u] > T;
    eq += ci[u] >= 0 && ck[u] == T;
  }
  uint32_t tot;
  const uint32_t ex = block_excl_scan((eq << 16) | gt, tot, sm.sbuf);
  gt = ex & 0xffffu;
  eq = ex >> 16;
#pragma unroll
  for (int u = 0; u < LPT; ++u) {
    if (ci[u] < 0) continue;
    if (ck[u] > T) {
      out[gt + min(eq, keq)] = ci[u];
      ++gt;
    } else if (ck[u] == T) {
      if (eq < keq) out[gt + eq] = ci[u];
      ++eq;
    }
  }
}

__global__ __launch_bounds__(TK_THREADS) void topk_seg_final(const float* __restrict__ scores, LongWs ws,
                                                             int32_t* __restrict__ idx, int64_t Tq, int64_t N,
                                                             int64_t q_pos0, Vis vis, int K, int G) {
  __shared__ FinalSmem sm;
  seg_final_row(scores, ws, idx, blockIdx.x, Tq, N, q_pos0, vis, K, G, sm);
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
                       int K, void* workspace, hipStream_t stream, const int64_t* seq_lens, int m) {
  const Vis vis{seq_lens, m};
  const int64_t R = B * Tq;
  // longest visible row: with per-sequence lengths only N is known on the host
  const int64_t nmax = seq_lens != nullptr ? N : min(N, (q_pos0 + Tq) / m);
  if (nmax <= TK_CAP || !use_long_path(B, Tq, N, K)) {
    hipLaunchKernelGGL(topk_rows_kernel, dim3((unsigned)R), dim3(TK_THREADS), 0, stream, scores, idx, Tq, N, q_pos0,
                       vis, K);
    return hipGetLastError();
  }
  const int G = long_segments(N);
  const LongWs ws = long_ws(workspace, R, G, K);
  const dim3 grid((unsigned)G, (unsigned)R);
  hipLaunchKernelGGL(topk_seg_classify, grid, dim3(TK_THREADS), 0, stream, scores, ws, Tq, N, q_pos0, vis, K, G);
  hipLaunchKernelGGL(topk_seg_final, dim3((unsigned)R), dim3(TK_THREADS), 0, stream, scores, ws, idx, Tq, N,
                     q_pos0, vis, K, G);
  return hipGetLastError();
}

}  // namespace dsa

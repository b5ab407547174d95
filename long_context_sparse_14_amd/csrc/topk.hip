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
// Three schedules:
//  * rows of up to 16384 keys (prefill): one workgroup per row, the row held
//    on chip with its key range, then exact select rounds that each split the
//    remaining range into 2^HBITS bins, then an in-order compaction with one
//    block prefix sum per chunk.  Rows of at most 8192 keys are staged in LDS
//    by 512 threads; rows of up to 16384 keep their first 8192 keys in LDS and
//    the rest in registers on 512 threads (four workgroups per compute unit
//    either way); longer rows that the long-row method below does not take
//    run on 1024 threads from global memory;
//  * decode rows that the indexer pre-selected (topk_presel_final): one
//    workgroup per row selects among the indexer's per-segment lists and
//    falls back to the row's full scores when a list cannot be shown to hold
//    the row's top K;
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
// in registers.  The compactions give each wave (one-workgroup method) or
// each thread (lists held in registers) a run of consecutive keys, so one
// block-wide prefix sum orders a whole chunk.
#include "launch.h"
#include "select_common.h"

namespace dsa {
namespace {

constexpr int TK_THREADS = 1024;
constexpr int TK_WAVES = TK_THREADS / 64;
constexpr int TK_CAP = 16384;         // longest row the one-workgroup method holds on chip
constexpr int SEG = 16384;            // segment length of the long-row method
constexpr int SEG_PER_T = SEG / TK_THREADS;
constexpr int HB = 2048;              // bins of an 11-bit digit
constexpr int CAND_CAP = 1024;        // candidates a segment may hand over
constexpr int ROW_CAND_CAP = 4096;    // candidates the final step can hold for one row
constexpr int LONG_MAX_K = 4096;      // largest K of the long-row method
constexpr int64_t LONG_MAX_SEGS = 4096;  // bound on rows x segments (workspace size)
constexpr int LONG_MAX_G = TK_THREADS;   // bound on segments per row (one thread per segment)
constexpr int RUN = 16;                  // keys per lane in a chunk of the compaction
constexpr int WRUN = RUN * 64;           // consecutive keys of one wave in a chunk

__device__ __forceinline__ int64_t n_visible(int64_t row, int64_t Tq, int64_t N, int64_t q_pos0, const Vis& vis) {
  return visible_keys(vis, seq_q0(vis, row / Tq, Tq, q_pos0), row % Tq, N);
}

// Set bits of a wave-uniform lane mask below this lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Exclusive block-wide prefix sum of v; `total` receives the block sum.
// Without TRAIL the closing barrier is left out, and the caller must pass
// another barrier before sbuf[0 .. TK_WAVES) is written again.
template <bool TRAIL = true, int NTH = TK_THREADS>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t& total, uint32_t* sbuf) {
  return block_excl_scan_w<NTH / 64, TRAIL, true>(v, total, sbuf);
}

// ------------------------------------------------- range-adaptive select

// Given a histogram h of 2^FBITS bins, find for each of two descending ranks
// ra, rb (1-based, at most the histogram total) the bin that holds it;
// *_above receives how many counted keys lie in higher bins, count_a how many
// lie in bin ba.  s_res: 8 words; words 0..4 stay valid until the next call
// (whose own barriers precede its writes).  With ZERO each thread clears the
// bins it read, and the closing barrier publishes the cleared histogram.
template <int FBITS, bool ZERO = false, int NTH = TK_THREADS>
__device__ __forceinline__ void find_two_bins(uint32_t* h, uint32_t ra, uint32_t rb, uint32_t& ba,
                                              uint32_t& above_a, uint32_t& bb, uint32_t& above_b,
                                              uint32_t& count_a, uint32_t* sbuf, uint32_t* s_res) {
  constexpr int NB = 1 << FBITS, PER_T = NB / NTH;
  static_assert(PER_T * NTH == NB, "whole bins per thread");
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
  uint32_t run = block_excl_scan<false, NTH>(t, tot, sbuf);  // the s_res barrier below closes it
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
  lds_barrier();
  ba = s_res[0];
  above_a = s_res[1];
  bb = s_res[2];
  above_b = s_res[3];
  count_a = s_res[4];
}

// Block-wide smallest and largest of per-thread values (mn, mx) over NTH
// threads.  sbuf2: 2 * NTH / 64 words, written once per workgroup (no closing
// barrier).
template <int NTH = TK_THREADS>
__device__ __forceinline__ void block_min_max(uint32_t mn, uint32_t mx, uint32_t& kmin, uint32_t& kmax,
                                              uint32_t* sbuf2) {
  mn = wave_min(mn);
  mx = wave_max(mx);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    sbuf2[2 * wave] = mn;
    sbuf2[2 * wave + 1] = mx;
  }
  lds_barrier();
  mn = 0xffffffffu;
  mx = 0u;
#pragma unroll
  for (int w = 0; w < NTH / 64; ++w) {
    mn = min(mn, sbuf2[2 * w]);
    mx = max(mx, sbuf2[2 * w + 1]);
  }
  kmin = mn;
  kmax = mx;
}

// Block-wide smallest and largest of per-thread values (mn, mx) and the sum
// of per-thread counts c.  sbuf3: 3 * TK_WAVES words, written once per
// workgroup (no closing barrier).
__device__ __forceinline__ void block_min_max_sum(uint32_t mn, uint32_t mx, uint32_t c, uint32_t& kmin,
                                                  uint32_t& kmax, uint32_t& sum, uint32_t* sbuf3) {
  mn = wave_min(mn);
  mx = wave_max(mx);
  c = wave_sum(c);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    sbuf3[3 * wave] = mn;
    sbuf3[3 * wave + 1] = mx;
    sbuf3[3 * wave + 2] = c;
  }
  lds_barrier();
  mn = 0xffffffffu;
  mx = 0u;
  c = 0u;
#pragma unroll
  for (int w = 0; w < TK_WAVES; ++w) {
    mn = min(mn, sbuf3[3 * w]);
    mx = max(mx, sbuf3[3 * w + 1]);
    c += sbuf3[3 * w + 2];
  }
  kmin = mn;
  kmax = mx;
  sum = c;
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
template <int FBITS, int NTH = TK_THREADS, typename AddKeys, typename EachKey>
__device__ uint32_t select_rank(AddKeys add_keys, EachKey each_key, uint32_t lo, uint32_t hi, uint32_t r,
                                uint32_t& above, uint32_t* h, uint32_t* sbuf, uint32_t* s_res, uint32_t* small) {
  above = 0;
#pragma unroll 1
  while (true) {
    const int shift = max(0, bit_width(hi - lo) - FBITS);
    HotBins hb;
    add_keys(hb, lo, hi, shift);
    hb.flush(h);
    lds_barrier();
    uint32_t b, ab, b2, ab2, cnt;
    find_two_bins<FBITS, true, NTH>(h, r, r, b, ab, b2, ab2, cnt, sbuf, s_res);
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
      lds_barrier();
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
      lds_barrier();
      above += s_res[6];
      return s_res[5];
    }
  }
}

// Writes a row with n <= K: 0..n-1, then -1.
template <int NTH = TK_THREADS>
__device__ __forceinline__ void write_whole_row(int64_t n, int K, int32_t* __restrict__ out) {
  for (int64_t i = threadIdx.x; i < K; i += NTH) out[i] = i < n ? (int32_t)i : -1;
}

// The K-th largest key T of a row of n32 > K keys whose range is [kmin,
// kmax], by histogram rounds of 2^HBITS bins over the whole row (NTH
// threads); `above` receives how many keys exceed T.  key_at(i) returns key
// i.  hist (all bins zero) and small[64] (zero) must have been published by a
// barrier.
template <int NTH = TK_THREADS, int HBITS = 11, typename KeyAt>
__device__ __forceinline__ uint32_t select_full(KeyAt key_at, int n32, int K, uint32_t kmin, uint32_t kmax,
                                                uint32_t& above, uint32_t* hist, uint32_t* sbuf, uint32_t* s_res,
                                                uint32_t* small) {
  const int tid = threadIdx.x;
  // (the bins span the keys' own range, so plain atomics rarely collide)
  auto add_row = [&](HotBins&, uint32_t lo, uint32_t hi, int shift) {
    for (int base = tid; base < n32; base += 8 * NTH) {
      uint32_t k[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = base + u * NTH;
        k[u] = i < n32 ? key_at(i) : 0u;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = base + u * NTH;
        if (i < n32 && k[u] >= lo && k[u] <= hi) atomicAdd(&hist[(k[u] - lo) >> shift], 1u);
      }
    }
  };
  auto each_row = [&](uint32_t lo, uint32_t hi, auto fn) {
    for (int base = tid; base < n32; base += 8 * NTH) {
      uint32_t k[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = base + u * NTH;
        k[u] = i < n32 ? key_at(i) : 0u;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = base + u * NTH;
        if (i < n32 && k[u] >= lo && k[u] <= hi) fn(k[u]);
      }
    }
  };
  return select_rank<HBITS, NTH>(add_row, each_row, kmin, kmax, (uint32_t)K, above, hist, sbuf, s_res, small);
}

// In-order compaction of a row of n32 keys with threshold T, keeping keq of
// the keys equal to T (NTH threads).
template <int NTH = TK_THREADS, typename KeyAt>
__device__ __forceinline__ void compact_row(KeyAt key_at, int n32, uint32_t T, uint32_t keq,
                                            int32_t* __restrict__ out, uint32_t* sbuf) {
  constexpr int CHUNK = RUN * NTH;  // keys ordered by one block prefix sum
  const int tid = threadIdx.x;
  // In-order compaction, CHUNK keys at a time: wave w owns the run of WRUN
  // consecutive keys starting at base + WRUN*w and reads it lane by lane (step
  // u: key base + WRUN*w + 64u + lane), so every LDS read is conflict-free.
  // Ballots give each step's keys above / equal to T; one block prefix sum
  // over the per-wave totals orders the waves, and a kept key's slot is its
  // wave's base plus the kept keys before it in the wave's run.
  const int lane = tid & 63, wave = tid >> 6;
  uint32_t run_gt = 0, run_eq = 0;
  for (int base = 0; base < n32; base += CHUNK) {
    const int w0 = base + WRUN * wave;
    uint32_t bits = 0;  // bit u: this lane's key of step u is above T; bit RUN + u: equal to T
    uint32_t cgt = 0, ceq = 0;
#pragma unroll
    for (int u = 0; u < RUN; ++u) {
      const int i = w0 + 64 * u + lane;
      const bool ok = i < n32;
      const uint32_t k = ok ? key_at(i) : 0u;
      bits |= (uint32_t)(ok && k > T) << u;
      bits |= (uint32_t)(ok && k == T) << (RUN + u);
    }
    cgt = wave_sum((uint32_t)__popc(bits & ((1u << RUN) - 1u)));
    ceq = wave_sum((uint32_t)__popc(bits >> RUN));
    uint32_t tot;
    const uint32_t ex = block_excl_scan<true, NTH>(lane == 0 ? (ceq << 16) | cgt : 0u, tot, sbuf);
    const uint32_t wex = __builtin_amdgcn_readfirstlane(ex);  // lane 0's prefix: the keys of earlier waves
    uint32_t g = run_gt + (wex & 0xffffu), e = run_eq + (wex >> 16);
#pragma unroll
    for (int u = 0; u < RUN; ++u) {
      const bool is_gt = (bits >> u) & 1u, is_eq = (bits >> (RUN + u)) & 1u;
      const uint64_t mg = __ballot(is_gt), me = __ballot(is_eq);
      const uint32_t bg = g + lanes_below(mg), be = e + lanes_below(me);
      const int32_t i = w0 + 64 * u + lane;
      if (is_gt) out[bg + min(be, keq)] = i;
      else if (is_eq && be < keq) out[bg + be] = i;
      g += (uint32_t)__popcll(mg);
      e += (uint32_t)__popcll(me);
    }
    run_gt += tot & 0xffffu;
    run_eq += tot >> 16;
  }
}


// The one-workgroup method for one row, NTH threads.  skey: LDS stage of CAP
// keys, or nullptr to read the row from global memory on every pass.  hist:
// 2^HBITS bins; sbuf: 3 * NTH / 64 words; s_res: 8 words; small: 65 words.
template <int NTH = TK_THREADS, int CAP = TK_CAP, int HBITS = 11>
__device__ __forceinline__ void select_row(const float* __restrict__ src, int64_t n, int K, int32_t* __restrict__ out,
                           uint32_t* skey, uint32_t* hist, uint32_t* sbuf, uint32_t* s_res, uint32_t* small) {
  constexpr int PTN = CAP / NTH;  // keys per thread of a row staged in LDS
  static_assert(PTN * NTH == CAP, "whole keys per thread");
  const int tid = threadIdx.x;
  if (n <= K) {
    write_whole_row<NTH>(n, K, out);
    return;
  }
  // keys (staged in LDS when skey is given: the whole row's loads in flight at
  // once) and their range; a longer row, eight loads in flight per thread
  // (row offsets fit 32 bits: N < 2^31)
  const int n32 = (int)n;
  uint32_t mn = 0xffffffffu, mx = 0u;
  if (skey != nullptr) {
    float v[PTN];
#pragma unroll
    for (int u = 0; u < PTN; ++u) {
      const int i = tid + u * NTH;
      v[u] = i < n32 ? src[i] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < PTN; ++u) {
      const int i = tid + u * NTH;
      if (i < n32) {
        const uint32_t k = float_order_key(v[u]);
        skey[i] = k;
        mn = min(mn, k);
        mx = max(mx, k);
      }
    }
  }
  for (int base = tid; skey == nullptr && base < n32; base += 8 * NTH) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = base + u * NTH;
      v[u] = i < n32 ? src[i] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = base + u * NTH;
      if (i < n32) {
        const uint32_t k = float_order_key(v[u]);
        mn = min(mn, k);
        mx = max(mx, k);
      }
    }
  }
  for (int b = tid; b < (1 << HBITS); b += NTH) hist[b] = 0u;  // the select starts from empty bins
  if (tid == 0) small[64] = 0u;
  uint32_t kmin, kmax;
  block_min_max<NTH>(mn, mx, kmin, kmax, sbuf + NTH / 64);  // its barrier also publishes skey and the bins
  auto key_at = [&](int i) -> uint32_t { return skey != nullptr ? skey[i] : float_order_key(src[i]); };
  uint32_t above;
  const uint32_t T = select_full<NTH, HBITS>(key_at, n32, K, kmin, kmax, above, hist, sbuf, s_res, small);
  compact_row<NTH>(key_at, n32, T, (uint32_t)K - above, out, sbuf);
}

// Rows of at most SHORT_KEYS keys run on 512-thread workgroups with a 32 KiB
// stage and 10-bit histogram rounds (36 KiB of LDS, four workgroups per
// compute unit); rows of up to 2 * SHORT_KEYS keys on the same workgroups
// with their second half in registers (select_row_split); longer rows on
// 1024-thread workgroups that read the row from global memory on every pass.
// A row's time is mostly fixed latency (its load, the select's barriers, the
// compaction's stores), so four rows in flight per compute unit, where a
// 64 KiB stage allowed two, serve rows faster.
constexpr int SHORT_KEYS = 8192;
constexpr int SPLIT_NTH = 512;

// One row of SHORT_KEYS < n <= 2 * SHORT_KEYS keys (n > K) on SPLIT_NTH
// threads: keys [0, SHORT_KEYS) staged in LDS (thread t: keys t + 512u), the
// rest in registers in the order the compaction reads them (thread of wave w,
// lane l: key SHORT_KEYS + WRUN*w + 64u + l, u < RUN), so that the second
// compaction chunk is each thread's own registers.
__device__ __forceinline__ void select_row_split(const float* __restrict__ src, int64_t n, int K,
                                                 int32_t* __restrict__ out, uint32_t* skey, uint32_t* hist,
                                                 uint32_t* sbuf, uint32_t* s_res, uint32_t* small) {
  constexpr int NTH = SPLIT_NTH, HBITS = 10, PTN = SHORT_KEYS / NTH;
  static_assert(PTN == RUN && WRUN * (NTH / 64) == SHORT_KEYS, "the register half is one compaction chunk");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n32 = (int)n;
  // every load issued at once (the register half clamped to the row's last key)
  float v[PTN], w[PTN];
#pragma unroll
  for (int u = 0; u < PTN; ++u) v[u] = src[tid + u * NTH];
#pragma unroll
  for (int u = 0; u < PTN; ++u) w[u] = src[min(SHORT_KEYS + WRUN * wave + 64 * u + lane, n32 - 1)];
  uint32_t mn = 0xffffffffu, mx = 0u, rk[PTN], rvm = 0u;  // rvm bit u: register key u lies in the row
#pragma unroll
  for (int u = 0; u < PTN; ++u) {
    const uint32_t k = float_order_key(v[u]);
    skey[tid + u * NTH] = k;
    mn = min(mn, k);
    mx = max(mx, k);
  }
#pragma unroll
  for (int u = 0; u < PTN; ++u) {
    const bool in = SHORT_KEYS + WRUN * wave + 64 * u + lane < n32;
    rk[u] = in ? float_order_key(w[u]) : 0u;
    rvm |= (uint32_t)in << u;
    if (in) {
      mn = min(mn, rk[u]);
      mx = max(mx, rk[u]);
    }
  }
  for (int b = tid; b < (1 << HBITS); b += NTH) hist[b] = 0u;  // the select starts from empty bins
  if (tid == 0) small[64] = 0u;
  uint32_t kmin, kmax;
  block_min_max<NTH>(mn, mx, kmin, kmax, sbuf + NTH / 64);  // its barrier also publishes skey and the bins
  auto add_row = [&](HotBins&, uint32_t lo, uint32_t hi, int shift) {
#pragma unroll
    for (int u = 0; u < PTN; ++u) {
      const uint32_t k = skey[tid + u * NTH];
      if (k >= lo && k <= hi) atomicAdd(&hist[(k - lo) >> shift], 1u);
    }
#pragma unroll
    for (int u = 0; u < PTN; ++u)
      if (((rvm >> u) & 1u) && rk[u] >= lo && rk[u] <= hi) atomicAdd(&hist[(rk[u] - lo) >> shift], 1u);
  };
  auto each_row = [&](uint32_t lo, uint32_t hi, auto fn) {
#pragma unroll
    for (int u = 0; u < PTN; ++u) {
      const uint32_t k = skey[tid + u * NTH];
      if (k >= lo && k <= hi) fn(k);
    }
#pragma unroll
    for (int u = 0; u < PTN; ++u)
      if (((rvm >> u) & 1u) && rk[u] >= lo && rk[u] <= hi) fn(rk[u]);
  };
  uint32_t above;
  const uint32_t T = select_rank<HBITS, NTH>(add_row, each_row, kmin, kmax, (uint32_t)K, above, hist, sbuf, s_res,
                                             small);
  const uint32_t keq = (uint32_t)K - above;
  // In-order compaction in two chunks of SHORT_KEYS keys, as in compact_row:
  // wave w owns keys c0 + WRUN*w + 64u + lane (u < RUN) of chunk c0.
  uint32_t run_gt = 0, run_eq = 0;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int w0 = SHORT_KEYS * c + WRUN * wave;
    uint32_t bits = 0;  // bit u: key u above T; bit RUN + u: equal to T
#pragma unroll
    for (int u = 0; u < RUN; ++u) {
      const bool ok = c == 0 || ((rvm >> u) & 1u);
      const uint32_t k = c == 0 ? skey[w0 + 64 * u + lane] : rk[u];
      bits |= (uint32_t)(ok && k > T) << u;
      bits |= (uint32_t)(ok && k == T) << (RUN + u);
    }
    const uint32_t cgt = wave_sum((uint32_t)__popc(bits & ((1u << RUN) - 1u)));
    const uint32_t ceq = wave_sum((uint32_t)__popc(bits >> RUN));
    uint32_t tot;
    const uint32_t ex = block_excl_scan<true, NTH>(lane == 0 ? (ceq << 16) | cgt : 0u, tot, sbuf);
    const uint32_t wex = __builtin_amdgcn_readfirstlane(ex);  // lane 0's prefix: the keys of earlier waves
    uint32_t g = run_gt + (wex & 0xffffu), e = run_eq + (wex >> 16);
#pragma unroll
    for (int u = 0; u < RUN; ++u) {
      const bool is_gt = (bits >> u) & 1u, is_eq = (bits >> (RUN + u)) & 1u;
      const uint64_t mg = __ballot(is_gt), me = __ballot(is_eq);
      const uint32_t bg = g + lanes_below(mg), be = e + lanes_below(me);
      const int32_t i = w0 + 64 * u + lane;
      if (is_gt) out[bg + min(be, keq)] = i;
      else if (is_eq && be < keq) out[bg + be] = i;
      g += (uint32_t)__popcll(mg);
      e += (uint32_t)__popcll(me);
    }
    run_gt += tot & 0xffffu;
    run_eq += tot >> 16;
  }
}

// Grid: (row index within the sequence from t_begin, sequence).  MODE 0:
// rows of at most SHORT_KEYS keys; 1: rows of up to 2 * SHORT_KEYS; 2: longer
// rows (read from global memory on every pass).  Each instance takes only its
// own rows.
template <int MODE>
__global__ __launch_bounds__(MODE == 2 ? TK_THREADS : SPLIT_NTH, 8) void topk_rows_kernel(
    const float* __restrict__ scores, int32_t* __restrict__ idx, int64_t Tq, int64_t N, int64_t q_pos0, Vis vis, int K,
    int64_t t_begin) {
  constexpr int NTH = MODE == 2 ? TK_THREADS : SPLIT_NTH, HBITS = MODE == 2 ? 11 : 10;
  constexpr int CAP = MODE == 2 ? TK_THREADS : SHORT_KEYS;  // MODE 2 stages nothing (a one-key-per-thread stub)
  __shared__ uint32_t skey[CAP];
  __shared__ uint32_t hist[1 << HBITS];
  __shared__ uint32_t sbuf[3 * NTH / 64];
  __shared__ uint32_t s_res[8];
  __shared__ uint32_t small[65];
  const int64_t t = t_begin + blockIdx.x;
  if (t >= Tq) return;
  const int64_t row = (int64_t)blockIdx.y * Tq + t;
  const int64_t n = n_visible(row, Tq, N, q_pos0, vis);
  const int mode = n <= SHORT_KEYS ? 0 : (n <= 2 * SHORT_KEYS ? 1 : 2);
  if (mode != MODE) return;  // another instance's row (whole workgroup)
  if constexpr (MODE == 1) {
    if (n <= K) write_whole_row<NTH>(n, K, idx + row * K);
    else select_row_split(scores + row * N, n, K, idx + row * K, skey, hist, sbuf, s_res, small);
  } else {
    select_row<NTH, CAP, HBITS>(scores + row * N, n, K, idx + row * K, MODE == 0 ? skey : nullptr, hist, sbuf, s_res,
                                small);
  }
}

// ---------------------------------------------------------------- long rows

constexpr int SAMPLE_BLOCKS = 64;                        // runs of consecutive keys in a row's sample
constexpr int SAMPLE_RUN = 64;                           // keys per run
constexpr int SAMPLES = SAMPLE_BLOCKS * SAMPLE_RUN;      // 4096
constexpr int SAMPLE_PER_T = SAMPLES / TK_THREADS;       // 4
static_assert(SAMPLE_PER_T * TK_THREADS == SAMPLES && SAMPLE_RUN % SAMPLE_PER_T == 0, "sample geometry");

constexpr int FB_BITS = 12;               // bins of the long-row histograms: 4096
constexpr int FB = 1 << FB_BITS;
static_assert(FB >= HB, "a long-row histogram also serves the one-workgroup fallback's 11-bit rounds");

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
    // every load issued (clamped to the row's last key), then the keys past
    // the row dropped: loads under a condition each waited for the previous one
    float v[SEG_PER_T];
#pragma unroll
    for (int u = 0; u < SEG_PER_T; ++u) v[u] = src[min(i0 + u, n - 1)];
#pragma unroll
    for (int u = 0; u < SEG_PER_T; ++u) k[u] = i0 + u < n ? float_order_key(v[u]) : 0u;
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
    float v[SAMPLE_PER_T];
#pragma unroll
    for (int u = 0; u < SAMPLE_PER_T; ++u) v[u] = src[min((int)threadIdx.x + TK_THREADS * u, S - 1)];
#pragma unroll
    for (int u = 0; u < SAMPLE_PER_T; ++u) {
      const int j = (int)threadIdx.x + TK_THREADS * u;
      valid[u] = j < S;
      k[u] = valid[u] ? float_order_key(v[u]) : 0u;
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
  uint32_t h[FB];               // also the fallback's histogram
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
  // this thread's entries of the row's list: where each sits, then all of
  // their loads at once (an entry past the list reads the row's first list
  // slot, workspace memory, and is dropped)
  const uint32_t len = ndef + ncand;
  const uint32_t j0 = (uint32_t)LPT * (uint32_t)tid;
  uint32_t ck[LPT];
  int32_t ci[LPT];
  {
    size_t off[LPT];
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
      off[u] = s0 * ws.cap;
      if (j < len) {
        while (sm.s_loff[g + 1] <= j) ++g;
        off[u] = (s0 + g) * ws.cap + (j - sm.s_loff[g]);
      }
    }
    uint2 lv[LPT];
#pragma unroll
    for (int u = 0; u < LPT; ++u) lv[u] = ws.list[off[u]];
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const bool in = j0 + u < len;
      ck[u] = in ? lv[u].x : 0u;
      ci[u] = in ? (int32_t)lv[u].y : -1;
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

// ------------------------------------------- rows pre-selected by the indexer

// Shared memory of the pre-selected final step.
struct PreselSmem {
  uint32_t h[FB];               // also the fallback's histogram
  uint32_t sbuf[3 * TK_WAVES];
  uint32_t s_res[8];
  uint32_t small[65];
};
constexpr int PLPT = kPreselRowCap / TK_THREADS;  // list entries per thread
static_assert(PLPT * TK_THREADS == kPreselRowCap, "whole list entries per thread");

// One workgroup per row.  The row's segment lists, concatenated, are one list
// in index order holding, for every segment, all of its keys at or above its
// threshold.  With L the largest threshold of a truncated list, every key >= L
// of the row is listed; if at least K listed keys are >= L, the K-th largest
// of them, T, found by an exact select among those alone, is the row's K-th
// key, and the kept keys (> T, and the first keq equal to T) are exactly the
// row's top K; one block prefix sum writes them in index order.  Otherwise
// the row runs the one-workgroup method over its scores in global memory.
__global__ __launch_bounds__(TK_THREADS) void topk_presel_final(const float* __restrict__ scores, PreselWs ps,
                                                                int32_t* __restrict__ idx, int64_t Tq, int64_t N,
                                                                int64_t q_pos0, Vis vis, int K) {
  __shared__ PreselSmem sm;
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int64_t n = n_visible(row, Tq, N, q_pos0, vis);
  int32_t* out = idx + row * K;
  if (n <= K) {
    for (int64_t i = tid; i < K; i += TK_THREADS) out[i] = i < n ? (int32_t)i : -1;
    return;
  }
  const int nseg = (int)((n + ps.kpw - 1) / ps.kpw);  // segments the indexer ran for this row
  const size_t s0 = (size_t)row * ps.G;
  const int cap = ps.cap;
  for (int b = tid; b < FB; b += TK_THREADS) sm.h[b] = 0u;
  if (tid == 0) sm.small[64] = 0u;
  // The row's lists as the workspace holds them, each at its full capacity:
  // slot p is entry p % cap of segment p / cap, at list + s0 * cap + p (the
  // G * cap <= kPreselRowCap slots of a row lie inside the workspace).
  // Thread t takes slots PLPT*t .. PLPT*t + PLPT - 1, which span at most two
  // segments (cap >= 16), and loads them together with those segments' counts
  // and, in every wave, the segments' thresholds: one round trip.  A slot is
  // an entry iff its segment ran and its position is below that segment's
  // count; thread order is then index order.
  const int p0 = PLPT * tid;
  const int ga = p0 / cap, gb = (p0 + PLPT - 1) / cap;
  const uint32_t cnt_a = ps.count[s0 + min(ga, nseg - 1)], cnt_b = ps.count[s0 + min(gb, nseg - 1)];
  // (the first threshold load's address is clamped rather than the load
  // skipped, so that it goes out with the list loads)
  const uint32_t thr0 = ps.thr[s0 + min(tid & 63, nseg - 1)];
  uint2 lv[PLPT];
#pragma unroll
  for (int u = 0; u < PLPT; ++u) lv[u] = ps.list[s0 * cap + p0 + u];
  uint32_t tl = (tid & 63) < nseg ? thr0 : 0u;
  for (int g = (tid & 63) + 64; g < nseg; g += 64) tl = max(tl, ps.thr[s0 + g]);  // rows of more than 64 segments
  // L: the largest threshold of a truncated list (0 when every list holds its
  // whole segment).  Every key of the row at or above L is listed, so when at
  // least K listed keys are >= L, the row's K-th key T is the K-th of those,
  // T >= L, and the keys of the row equal to T are all listed: only entries
  // >= L take part.  With fewer, T < L, and a truncated list may hide keys of
  // the row's top K: the row falls back.  (A list with no room for any of its
  // candidate thresholds has thr all ones, so its row always falls back.)
  const uint32_t L = wave_max(tl);
  uint32_t ck[PLPT];
  int32_t ci[PLPT];
  uint32_t mn = 0xffffffffu, mx = 0u, own = 0u;
#pragma unroll
  for (int u = 0; u < PLPT; ++u) {
    const int p = p0 + u;
    const int g = p / cap;
    const bool in = g < nseg && (uint32_t)(p - g * cap) < (g == ga ? cnt_a : cnt_b) && lv[u].x >= L;
    ck[u] = in ? lv[u].x : 0u;
    ci[u] = in ? (int32_t)lv[u].y : -1;
    if (in) {
      mn = min(mn, lv[u].x);
      mx = max(mx, lv[u].x);
      ++own;
    }
  }
  uint32_t kmin, kmax, total;
  block_min_max_sum(mn, mx, own, kmin, kmax, total, sm.sbuf);  // its barrier also publishes the cleared bins
  const bool ok = total >= (uint32_t)K;
  uint32_t T = 0u, keq = 0u;
  if (ok) {
    auto add_cand = [&](HotBins& hb, uint32_t lo, uint32_t hi, int shift) {
#pragma unroll
      for (int u = 0; u < PLPT; ++u)
        if (ci[u] >= 0 && ck[u] >= lo && ck[u] <= hi) hb.add((ck[u] - lo) >> shift, sm.h);
    };
    auto each_cand = [&](uint32_t lo, uint32_t hi, auto fn) {
#pragma unroll
      for (int u = 0; u < PLPT; ++u)
        if (ci[u] >= 0 && ck[u] >= lo && ck[u] <= hi) fn(ck[u]);
    };
    uint32_t above;
    T = select_rank<FB_BITS>(add_cand, each_cand, kmin, kmax, (uint32_t)K, above, sm.h, sm.sbuf, sm.s_res,
                             sm.small);
    keq = (uint32_t)K - above;
  }
  if (!ok) {
    lds_barrier();  // every wave has read the reduction's words in sbuf before the fallback reuses them
    select_row(scores + row * N, n, K, out, nullptr, sm.h, sm.sbuf, sm.s_res, sm.small);
    return;
  }
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int u = 0; u < PLPT; ++u) {
    gt += ci[u] >= 0 && ck[u] > T;
    eq += ci[u] >= 0 && ck[u] == T;
  }
  uint32_t tot;
  const uint32_t ex = block_excl_scan((eq << 16) | gt, tot, sm.sbuf);
  gt = ex & 0xffffu;
  eq = ex >> 16;
#pragma unroll
  for (int u = 0; u < PLPT; ++u) {
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

int long_segments(int64_t N) { return (int)((N + SEG - 1) / SEG); }

bool use_long_path(int64_t B, int64_t Tq, int64_t N, int K) {
  return N > TK_CAP && K <= LONG_MAX_K && long_segments(N) <= LONG_MAX_G && B * Tq * long_segments(N) <= LONG_MAX_SEGS;
}

}  // namespace

size_t topk_workspace_bytes(int64_t B, int64_t Tq, int64_t N, int K) {
  const size_t pre = presel_workspace_bytes(B, Tq, N, K);
  if (!use_long_path(B, Tq, N, K)) return pre;
  const size_t lw = long_ws_bytes(B * Tq, long_segments(N), K);
  return lw > pre ? lw : pre;
}

hipError_t launch_topk_presel(const float* scores, int32_t* idx, int64_t B, int64_t Tq, int64_t N, int64_t q_pos0,
                              int K, const PreselWs& ps, hipStream_t stream, const int64_t* seq_lens, int m) {
  const Vis vis{seq_lens, m};
  hipLaunchKernelGGL(topk_presel_final, dim3((unsigned)(B * Tq)), dim3(TK_THREADS), 0, stream, scores, ps, idx, Tq, N,
                     q_pos0, vis, K);
  return hipGetLastError();
}

hipError_t launch_topk(const float* scores, int32_t* idx, int64_t B, int64_t Tq, int64_t N, int64_t q_pos0,
                       int K, void* workspace, hipStream_t stream, const int64_t* seq_lens, int m) {
  const Vis vis{seq_lens, m};
  const int64_t R = B * Tq;
  // longest visible row: with per-sequence lengths only N is known on the host
  const int64_t nmax = seq_lens != nullptr ? N : min(N, (q_pos0 + Tq) / m);
  if (nmax <= TK_CAP || !use_long_path(B, Tq, N, K)) {
    // Without per-sequence lengths a row's key count grows with t, the same
    // in every sequence: rows [0, t1) have at most SHORT_KEYS keys, rows
    // [t1, t2) at most 2 * SHORT_KEYS.  With them, every instance runs over
    // every row and each keeps its own.
    int64_t t1 = 0, t2 = 0;
    if (seq_lens == nullptr) {
      auto n_at = [&](int64_t t) {
        const int64_t p1 = q_pos0 + t + 1;
        return p1 <= 0 ? (int64_t)0 : min(N, p1 / m);
      };
      auto first_above = [&](int64_t keys) {  // first t in [0, Tq) with more than `keys` keys, or Tq
        int64_t lo = 0, hi = Tq;
        while (lo < hi) {
          const int64_t mid = (lo + hi) / 2;
          if (n_at(mid) > keys) hi = mid;
          else lo = mid + 1;
        }
        return lo;
      };
      t1 = first_above(SHORT_KEYS);
      t2 = first_above(2 * SHORT_KEYS);
    }
    const int64_t b0[3] = {0, t1, t2}, b1[3] = {seq_lens == nullptr ? t1 : Tq, seq_lens == nullptr ? t2 : Tq, Tq};
    if (b1[0] > b0[0])
      hipLaunchKernelGGL(topk_rows_kernel<0>, dim3((unsigned)(b1[0] - b0[0]), (unsigned)B), dim3(SPLIT_NTH), 0,
                         stream, scores, idx, Tq, N, q_pos0, vis, K, b0[0]);
    if (b1[1] > b0[1])
      hipLaunchKernelGGL(topk_rows_kernel<1>, dim3((unsigned)(b1[1] - b0[1]), (unsigned)B), dim3(SPLIT_NTH), 0,
                         stream, scores, idx, Tq, N, q_pos0, vis, K, b0[1]);
    if (b1[2] > b0[2])
      hipLaunchKernelGGL(topk_rows_kernel<2>, dim3((unsigned)(b1[2] - b0[2]), (unsigned)B), dim3(TK_THREADS), 0,
                         stream, scores, idx, Tq, N, q_pos0, vis, K, b0[2]);
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

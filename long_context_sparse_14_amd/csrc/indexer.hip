// Lightning-indexer scores on gfx950.
//
// Computes, for query t of sequence b and every key s it may see,
//   scores[b,t,s] = sum_h w[b,t,h] * max(0, sum_d q_idx[b,t,h,d] * k_idx[b,s,d])
// (DeepSeek-V3.2 model documentation, section "DeepSeek Sparse Attention
// (DSA)": a light scorer with few heads against every earlier key, over the
// indexer's own single-head key cache; head count and width from the
// DeepseekV32Config section: 64 heads of width 128.)
//
// bf16 path, matrix cores.  One 32x32x16 MFMA block has the 32 heads of a
// query as rows (A = q) and 32 keys as columns (B = k), so after the
// contraction each lane owns one key and 16 of the 32 heads: the ReLU and the
// head-weighted sum are plain per-lane FMAs, and one exchange between lane j
// and lane j+32 completes the 64-head sum.  The contraction order over the
// 128 channels is free, so lane half h takes channels [64h, 64h+64): every
// lane then reads 128 contiguous bytes of its key row, for q and k alike.
//
//  * decode kernel (few queries per sequence): the key cache is read once
//    from HBM into per-wave LDS rings with direct-to-LDS loads of 1 KiB of
//    consecutive bytes each, three 8 KiB tiles of 32 keys in flight per wave,
//    and the scores leave in one burst per workgroup;
//  * tiled kernel (prefill): 8 queries per workgroup (one per wave) share
//    128-key tiles staged in LDS, double-buffered; within a tile each wave
//    overlaps the MFMAs of one 32-key block with the epilogue of the previous
//    one; the causal triangle is walked longest query block first.
#include "launch.h"
#include "select_common.h"

namespace dsa {
namespace {

constexpr int IH = 64;   // indexer heads
constexpr int ID = 128;  // indexer head width

struct QFrags {
  bf16x8 a0[8], a1[8];  // heads [0,32) and [32,64); channels 64*half + 8*s + [0,8)
  float w0[16], w1[16]; // weights of the accumulator rows this lane holds
};

__device__ __forceinline__ void load_query(QFrags& f, const uint16_t* __restrict__ q_idx,
                                           const uint16_t* __restrict__ w, int64_t row, int half, int col) {
  const uint16_t* qr = q_idx + row * (IH * ID) + 64 * half;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    f.a0[s] = load_bf16x8(qr + col * ID + 8 * s);
    f.a1[s] = load_bf16x8(qr + (32 + col) * ID + 8 * s);
  }
  const uint16_t* wr = w + row * IH;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    f.w0[i] = bf16_bits_to_float(wr[mfma_row(i, half)]);
    f.w1[i] = bf16_bits_to_float(wr[32 + mfma_row(i, half)]);
  }
}

// Score of this lane's key (valid in lanes 0..31) from the two head blocks.
// ReLU is a median of three (one instruction for finite scores; fmaxf would
// add a NaN-quieting instruction), and the two halves of the wave are added
// with a lane swap.
__device__ __forceinline__ float weighted_relu_sum(const QFrags& f, const f32x16& c0, const f32x16& c1) {
  float part = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    part = fmaf(f.w0[i], __builtin_amdgcn_fmed3f(c0[i], 0.f, 3.0e38f), part);
    part = fmaf(f.w1[i], __builtin_amdgcn_fmed3f(c1[i], 0.f, 3.0e38f), part);
  }
  return sum_halves(part);
}

// Block-table entries of one workgroup's key range for a paged cache: lane j
// holds entries j, j + 64 and j + 128 (at most 192: the host admits blocks of
// at least 64 keys and at most 8192 keys per workgroup).  page_row() maps a
// wave-uniform key to its pool row.
template <bool PAGED>
struct PageRows {
  int32_t tbl[3] = {0, 0, 0};
  int64_t blk0 = 0;
  int32_t shift = 0;
  __device__ __forceinline__ void load(const Paged& pg, int64_t b, int64_t k_begin, int64_t k_end, int lane) {
    if (!PAGED) return;
    shift = pg.shift;
    blk0 = k_begin >> shift;
    const int64_t nent = ((k_end - 1) >> shift) - blk0 + 1;
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      const int64_t j = lane + 64 * u;
      if (j < nent) {
        const int32_t v = pg.table[b * pg.max_blocks + blk0 + j];
        tbl[u] = (uint32_t)v < (uint32_t)pg.num_blocks ? v : 0;
      }
    }
  }
  __device__ __forceinline__ int64_t row(int64_t key) const {
    if (!PAGED) return key;
    const int64_t j = (key >> shift) - blk0;
    const int32_t v = j < 64 ? tbl[0] : (j < 128 ? tbl[1] : tbl[2]);
    const int32_t e = __builtin_amdgcn_readlane(v, (int)(j & 63));
    return ((int64_t)e << shift) | (key & ((1 << shift) - 1));
  }
  // per-lane form (any key of the range; all lanes of the wave take part)
  __device__ __forceinline__ int64_t row_any(int64_t key) const {
    if (!PAGED) return key;
    const int64_t j = (key >> shift) - blk0;
    const int l = (int)(j & 63);
    const int32_t v0 = __shfl(tbl[0], l), v1 = __shfl(tbl[1], l), v2 = __shfl(tbl[2], l);
    const int32_t e = j < 64 ? v0 : (j < 128 ? v1 : v2);
    return ((int64_t)e << shift) | (key & ((1 << shift) - 1));
  }
};

// Order key -> the float it stands for (inverse of float_order_key; keys
// between those of two finite floats stand for finite floats).
__device__ __forceinline__ float order_key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Pre-selection epilogue of a decode workgroup (WAVES waves), run once its
// n <= SCAP scores sit in LDS (sl) and before any of them is stored: its
// barriers settle LDS only, so nothing waits for global stores, and its own
// global stores come at its end.  It picks a threshold c such that at most
// cap scores of the segment are >= c and about PRE_M * tgt are (tgt: a few
// times the segment's expected share of the row's K best), then lists every
// score >= c (order key and key index) in index order.  Thread t owns the
// run of scores [PER*t, PER*t + PER); scores 0, 8, 16 and 24 of every run form
// a systematic sample, and one histogram of the sample over its own key range
// gives candidate thresholds: the lower edges of the bins holding the sample
// ranks expected to leave PRE_M[j] * tgt scores at or above them.  The first
// candidate whose exact count fits in cap is taken (each count is one pass
// of compares into a per-thread bit mask); if none fits, nothing is listed
// and thr is all ones, so the row falls back.  thr = c's order key, or 0 when
// every score of the segment is listed.  The list is staged in LDS and leaves
// in whole consecutive entries.  The epilogue is short because every pass
// over a thread's PER scores is one compare per score.
// lds: 2048 + 2 * kPreselMaxCap + 4 * WAVES + 8 words of free LDS.
template <int WAVES, int SCAP>
__device__ __forceinline__ void presel_segment(const float* sl, int n, int64_t k_begin, int64_t row, int g,
                                               const PreselWs& ps, uint32_t* lds) {
  constexpr int NTH = WAVES * 64, PER = SCAP / NTH;  // scores per thread, consecutive
  constexpr int HBITS = 11, NBINS = 1 << HBITS, BPT = NBINS / NTH;
  static_assert(PER >= 8 && PER <= 32 && PER % 4 == 0 && BPT * NTH == NBINS,
                "presel geometry: one 32-bit mask per thread");
  constexpr int NC = 3;
  constexpr float PRE_M[NC] = {1.5f, 1.0f, 0.6f};
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i0 = PER * tid;
  const int nv = max(0, min(PER, n - i0));  // scores of this thread's run
  float v[PER];
#pragma unroll
  for (int q = 0; q < PER / 4; ++q) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(&sl[i0 + 4 * q]);  // slots past n hold stale values
    v[4 * q + 0] = x.x;
    v[4 * q + 1] = x.y;
    v[4 * q + 2] = x.z;
    v[4 * q + 3] = x.w;
  }
  uint32_t* h = lds;                                      // NBINS words
  uint2* s_list = reinterpret_cast<uint2*>(lds + NBINS);  // kPreselMaxCap entries
  uint32_t* s_red = lds + NBINS + 2 * kPreselMaxCap;      // 4 * WAVES words
  uint32_t* s_cand = s_red + 4 * WAVES;                   // NC words
  const int cap = ps.cap;
  const uint32_t valid_mask = nv >= 32 ? 0xffffffffu : ((1u << nv) - 1u);
  uint32_t m = valid_mask;  // scores to list
  uint32_t thr = 0u;
  if (n > cap) {
    // the sample: scores 0, 8, 16 and 24 of every run
    constexpr int SPT = 4, SSTEP = PER / SPT;
    uint32_t skey[SPT];
    uint32_t smn = 0xffffffffu, smx = 0u;
#pragma unroll
    for (int e = 0; e < SPT; ++e) {
      skey[e] = float_order_key(v[SSTEP * e]);
      if (SSTEP * e < nv) {
        smn = min(smn, skey[e]);
        smx = max(smx, skey[e]);
      }
    }
    const uint32_t smin = wave_min(smn), smax = wave_max(smx);
    if (lane == 0) {
      s_red[wave] = smin;
      s_red[WAVES + wave] = smax;
    }
#pragma unroll
    for (int u = 0; u < BPT; ++u) h[BPT * tid + u] = 0u;
    lds_barrier();
    uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      lo = min(lo, s_red[w]);
      hi = max(hi, s_red[WAVES + w]);
    }
    const int shift = max(0, bit_width(hi - lo) - HBITS);
#pragma unroll
    for (int e = 0; e < SPT; ++e)
      if (SSTEP * e < nv) atomicAdd(&h[(skey[e] - lo) >> shift], 1u);
    lds_barrier();
    // thread t owns bins NBINS-1-BPT*t-u, descending
    uint32_t cnt[BPT], tsum = 0u;
#pragma unroll
    for (int u = 0; u < BPT; ++u) {
      cnt[u] = h[NBINS - 1 - BPT * tid - u];
      tsum += cnt[u];
    }
    uint32_t ns;  // the sample's size
    uint32_t run = block_excl_scan_w<WAVES, false, true>(tsum, ns, s_red + 2 * WAVES);
    // candidate j: the bin holding sample rank R_j (1-based, from the top)
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int R = max(1, min((int)ns, (int)(PRE_M[j] * (float)ps.tgt * (float)ns / (float)n + 0.5f)));
      uint32_t r2 = run;
#pragma unroll
      for (int u = 0; u < BPT; ++u) {
        if (r2 < (uint32_t)R && (uint32_t)R <= r2 + cnt[u]) s_cand[j] = lo + ((uint32_t)(NBINS - 1 - BPT * tid - u) << shift);
        r2 += cnt[u];
      }
    }
    lds_barrier();
    uint32_t ck[NC];
#pragma unroll
    for (int j = 0; j < NC; ++j) ck[j] = s_cand[j];
    m = 0u;
    thr = 0xffffffffu;  // no candidate fits: list nothing
#pragma unroll 1
    for (int j = 0; j < NC; ++j) {
      const float c = order_key_float(ck[j]);
      uint32_t mj = 0u;
#pragma unroll
      for (int u = 0; u < PER; ++u) mj |= (v[u] >= c ? 1u : 0u) << u;
      mj &= valid_mask;
      const uint32_t t = wave_sum((uint32_t)__popc(mj));
      if (lane == 0) s_red[NC * wave + j] = t;
      lds_barrier();
      uint32_t tot = 0u;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) tot += s_red[NC * w + j];
      if (tot <= (uint32_t)cap) {
        m = mj;
        thr = ck[j];
        break;
      }
    }
    lds_barrier();  // s_red is reused by the scan below
  }
  // the listed scores, in index order: staged in LDS, then copied out whole
  uint32_t listed;
  uint32_t pos = block_excl_scan_w<WAVES, false, true>((uint32_t)__popc(m), listed, s_red);
  while (m != 0u) {
    const int u = __builtin_ctz(m);
    m &= m - 1u;
    s_list[pos++] = make_uint2(float_order_key(sl[i0 + u]), (uint32_t)(k_begin + i0 + u));
  }
  lds_barrier();
  const size_t seg = (size_t)row * ps.G + g;
  uint2* list = ps.list + seg * ps.cap;
  for (int i = tid; i < (int)listed; i += NTH) list[i] = s_list[i];
  if (tid == 0) {
    ps.count[seg] = listed;
    ps.thr[seg] = thr;
  }
}

// Decode kernel with the key tiles staged through LDS.  A wave owns a ring
// of NBUF tiles of 32 keys (8 KiB) in LDS and keeps NBUF-1 of them in flight
// with direct-to-LDS loads.  Each load instruction fetches 1 KiB of
// consecutive cache bytes (four key rows), which the memory system serves at
// the full streaming rate; loading the MFMA operands straight from global
// memory would touch a different 128-byte line in every lane.  No other wave
// touches a wave's ring, so the key loop has no barriers.  The workgroup's
// scores (at most SCAP) collect in LDS and leave in one contiguous burst at
// the end: small score writes spread through the key stream cost the read
// stream far more than their own bytes.
//
// Tile layout: lane L of load u (0..7) of a tile fetches 16-byte chunk
// c = (L & 15) ^ (key & 15) of key 4u + L/16 and lands at slot 64u + L, i.e.
// chunk c of tile key r sits at slot 16r + (c ^ (r & 15)).  The operand read
// of k-step s (chunk 8*half + s of key col) then spreads every 16 lanes over
// all 64 banks.
template <int WAVES, int NBUF, int SCAP, bool PAGED = false, bool PRESEL = false>
__global__ __launch_bounds__(WAVES * 64, 1) void indexer_dma_bf16(
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ k_idx, const uint16_t* __restrict__ w,
    float* __restrict__ scores, int64_t Tq, int64_t N, int64_t q_pos0, Vis vis, int64_t keys_per_wg, Paged pg,
    PreselWs ps) {
  constexpr int TILE_BYTES = 32 * ID * 2;
  static_assert(NBUF >= 2 && NBUF <= 5, "the vmcnt waits below cover up to four tiles in flight");
  static_assert(WAVES * NBUF * TILE_BYTES + SCAP * 4 <= 160 * 1024, "LDS budget");
  __shared__ __align__(16) uint16_t kt[WAVES][NBUF][32 * ID];
  __shared__ __align__(16) float sl[SCAP];  // this workgroup's scores; keys_per_wg <= SCAP
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5, col = lane & 31;
  const int64_t t = blockIdx.y, b = blockIdx.z;
  const int64_t row = b * Tq + t;
  const int64_t n_valid = visible_keys(vis, seq_q0(vis, b, Tq, q_pos0), t, N);
  const int64_t k_begin = (int64_t)blockIdx.x * keys_per_wg;  // a multiple of 32
  const int64_t k_end = min(n_valid, k_begin + keys_per_wg);
  if (k_begin >= k_end) return;
  const int total_tiles = (int)((k_end - k_begin + 31) / 32);
  const int nt = total_tiles > wave ? (total_tiles - wave + WAVES - 1) / WAVES : 0;

  // a paged cache: tiles of 32 keys never cross a block (blocks hold a multiple of 32 keys)
  const uint8_t* kb = reinterpret_cast<const uint8_t*>(k_idx + (PAGED ? 0 : b * N * ID));
  PageRows<PAGED> pr;
  pr.load(pg, b, k_begin, k_end, lane);
  const uint32_t ring = lds_address(&kt[wave][0][0]);
  // per-lane part of the source offset of load u, for u & 3 (the XOR term repeats every 4 loads)
  const int kk = lane >> 4, jj = lane & 15;
  uint32_t voff[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) voff[v] = 256u * kk + 16u * (uint32_t)(jj ^ (4 * v + kk));
  auto key0_of = [&](int it) { return k_begin + 32 * (int64_t)(it * WAVES + wave); };
  auto dma_tile = [&](int it) {
    const int64_t key0 = key0_of(it);
    const uint32_t dst = ring + (uint32_t)((it % NBUF) * TILE_BYTES);
    if (PAGED) {
      const int64_t r0 = pr.row(key0);
#pragma unroll
      for (int u = 0; u < 8; ++u) dma16_stream(kb + (r0 + 4 * u) * (ID * 2), voff[u & 3], dst + 1024u * u);
    } else if (key0 + 32 <= N) {
#pragma unroll
      for (int u = 0; u < 8; ++u) dma16_stream(kb + (key0 + 4 * u) * (ID * 2), voff[u & 3], dst + 1024u * u);
    } else {
      // last rows of the cache: clamp to a real row (those keys are never scored)
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t kbase = min(key0 + 4 * u, N - 1);
        const int64_t key = min(key0 + 4 * u + kk, N - 1);
        const uint32_t off = (uint32_t)(key - kbase) * 256u + (voff[u & 3] & 255u);
        dma16_stream(kb + kbase * (ID * 2), off, dst + 1024u * u);
      }
    }
  };
  QFrags f;
  load_query(f, q_idx, w, row, half, col);
  __builtin_amdgcn_sched_barrier(0);  // query loads first, so one wait covers them and the first tiles
#pragma unroll
  for (int p = 0; p < NBUF - 1; ++p)
    if (p < nt) dma_tile(p);
  // queries in registers and the first tiles in LDS; the compiler now sees no load in flight
  __builtin_amdgcn_s_waitcnt(0);

  // operand read of k-step s: chunk 8*half + s of key col
  const uint32_t rbase = 256u * col;
  const int x = (8 * half) ^ (col & 15);
  float* sr = scores + row * N;
  for (int it = 0; it < nt; ++it) {
    if (it + NBUF - 1 < nt) dma_tile(it + NBUF - 1);
    // loads issued after tile it's: those of the next min(NBUF-1, nt-1-it) tiles
    // (score stores in between only make the wait longer)
    const int after = min(NBUF - 1, nt - 1 - it);
    if (after >= 4) asm volatile("s_waitcnt vmcnt(32)" ::: "memory");
    else if (after == 3) asm volatile("s_waitcnt vmcnt(24)" ::: "memory");
    else if (after == 2) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    else if (after == 1) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const uint16_t* tile = &kt[wave][it % NBUF][0];
    f32x16 c0 = {}, c1 = {};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8 bv = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const uint8_t*>(tile) + rbase +
                                                         16u * (uint32_t)(x ^ s));
      c0 = mfma32x32x16(f.a0[s], bv, c0);
      c1 = mfma32x32x16(f.a1[s], bv, c1);
    }
    const float sc = weighted_relu_sum(f, c0, c1);
    if (half == 0) sl[key0_of(it) - k_begin + col] = sc;  // slots past k_end are never copied out
  }
  __syncthreads();
  const int n = (int)(k_end - k_begin);
  if constexpr (PRESEL) {
    // the key rings are idle: every wave awaited its last tile before the barrier above
    presel_segment<WAVES, SCAP>(sl, n, k_begin, row, (int)blockIdx.x, ps, reinterpret_cast<uint32_t*>(&kt[0][0][0]));
  }
  float* dst = sr + k_begin;
  if (((row * N) & 3) == 0) {  // 16-byte aligned row segment (k_begin is a multiple of 32)
    for (int i = 4 * (int)threadIdx.x; i < n; i += 4 * WAVES * 64) {
      // streaming stores: the scores are read back once, by the top-k
      if (i + 4 <= n) __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(&sl[i]), reinterpret_cast<f32x4*>(dst + i));
      else
        for (int e = i; e < n; ++e) dst[e] = sl[e];
    }
  } else {
    for (int i = (int)threadIdx.x; i < n; i += WAVES * 64) dst[i] = sl[i];
  }
}

// PRIO: a wave raises its issue priority while it issues a block's MFMAs, so
// the two waves sharing a SIMD drift into alternating MFMA and vector phases.
template <int WAVES, int TK, int PRIO>
__global__ __launch_bounds__(WAVES * 64) void indexer_tiled_bf16(
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ k_idx, const uint16_t* __restrict__ w,
    float* __restrict__ scores, int64_t Tq, int64_t N, int64_t q_pos0, Vis vis, int64_t nqb) {
  // TK keys per LDS tile
  constexpr int PITCH = ID + 8;   // bf16 per LDS row (272 B): spreads rows over the banks
  constexpr int CHUNKS = TK * ID / 8;
  constexpr int PER_T = CHUNKS / (WAVES * 64);
  static_assert(PER_T * WAVES * 64 == CHUNKS, "tile chunks must divide evenly");
  __shared__ __align__(16) uint16_t ks[2][TK * PITCH];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int64_t qb = nqb - 1 - (int64_t)blockIdx.x;  // longest rows first
  const int64_t b = blockIdx.y;
  const int64_t t0 = qb * WAVES;
  const int64_t t_last = min(Tq, t0 + WAVES) - 1;
  const int64_t t = t0 + wave;
  const bool active = t < Tq;
  const int64_t q0 = seq_q0(vis, b, Tq, q_pos0);
  const int64_t n_valid = active ? visible_keys(vis, q0, t, N) : 0;
  const int64_t n_blk = visible_keys(vis, q0, t_last, N);
  const int64_t row = b * Tq + (active ? t : t_last);

  QFrags f;
  load_query(f, q_idx, w, row, half, col);
  const uint16_t* kb = k_idx + b * N * ID;
  float* sr = scores + row * N;

  u32x4 pre[PER_T];
  auto gload = [&](int64_t k0) {
#pragma unroll
    for (int u = 0; u < PER_T; ++u) {
      const int c = tid + u * WAVES * 64;
      const int64_t key = min(k0 + (c >> 4), N - 1);
      pre[u] = *reinterpret_cast<const u32x4*>(kb + key * ID + 8 * (c & 15));
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int u = 0; u < PER_T; ++u) {
      const int c = tid + u * WAVES * 64;
      *reinterpret_cast<u32x4*>(&ks[buf][(c >> 4) * PITCH + 8 * (c & 15)]) = pre[u];
    }
  };

  const int ntiles = (int)((n_blk + TK - 1) / TK);
  gload(0);
  lstore(0);
  __syncthreads();
  // The query fragments' first use is inside the tile loop.  Consuming them
  // here makes their loads complete before it, so the compiler puts no wait
  // on them inside the loop; otherwise it waited, in every tile, for every
  // load in flight, including the prefetch of the next tile.
#pragma unroll
  for (int s = 0; s < 8; ++s) asm volatile("" ::"v"(f.a0[s]), "v"(f.a1[s]));
  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    const int64_t k0 = (int64_t)it * TK;
    // Unconditional, like the LDS store below (past the last tile the keys are
    // clamped to a real row and land in the idle buffer): with both under one
    // condition the compiler assumed a path where the loads are never waited
    // for, and waited for them at the top of every tile.
    gload(k0 + TK);
    // Blocks of 32 keys, software-pipelined: the MFMAs of block nb are issued
    // before the ReLU / weighted-sum epilogue of block nb-1, so the vector
    // units work while the matrix cores run.  Blocks past this query's last
    // key are skipped (only on the diagonal tiles).
    constexpr int NBK = TK / 32;
    const int64_t left = n_valid - k0;
    const int nbv = left <= 0 ? 0 : (left >= TK ? NBK : (int)((left + 31) / 32));
    f32x16 c[2][2];
    auto mma_block = [&](int nb, f32x16 (&cc)[2]) {
      const uint16_t* lp = &ks[buf][(32 * nb + col) * PITCH + 64 * half];
      bf16x8 bv[8];  // all eight key operands of the block in flight before the first MFMA
#pragma unroll
      for (int s = 0; s < 8; ++s) bv[s] = *reinterpret_cast<const bf16x8*>(lp + 8 * s);
      __builtin_amdgcn_sched_barrier(0);
      cc[0] = f32x16{};
      cc[1] = f32x16{};
      if (PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        cc[0] = mfma32x32x16(f.a0[s], bv[s], cc[0]);
        cc[1] = mfma32x32x16(f.a1[s], bv[s], cc[1]);
      }
      if (PRIO) __builtin_amdgcn_s_setprio(0);
    };
    auto epi_block = [&](int nb, const f32x16 (&cc)[2]) {
      const int64_t kk0 = k0 + 32 * nb;
      const float sc = weighted_relu_sum(f, cc[0], cc[1]);
      if (half == 0 && kk0 + col < n_valid) sr[kk0 + col] = sc;
    };
    const bool full = left >= TK;
    float scv[NBK];
    if (full) {
      // Full tile (every key visible), branch-free: the scheduler is told to
      // put four vector instructions of block nb-1's epilogue after each of
      // block nb's MFMAs, so they issue while the matrix core runs instead of
      // after it.  The scores leave after the next tile's LDS store (below).
      mma_block(0, c[0]);
#pragma unroll
      for (int nb = 1; nb < NBK; ++nb) {
        const uint16_t* lp = &ks[buf][(32 * nb + col) * PITCH + 64 * half];
        bf16x8 bv[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) bv[s] = *reinterpret_cast<const bf16x8*>(lp + 8 * s);
        __builtin_amdgcn_sched_barrier(0);
        f32x16(&cc)[2] = c[nb & 1];
        cc[0] = f32x16{};
        cc[1] = f32x16{};
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          cc[0] = mfma32x32x16(f.a0[s], bv[s], cc[0]);
          cc[1] = mfma32x32x16(f.a1[s], bv[s], cc[1]);
        }
        scv[nb - 1] = weighted_relu_sum(f, c[(nb - 1) & 1][0], c[(nb - 1) & 1][1]);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // four vector instructions
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      scv[NBK - 1] = weighted_relu_sum(f, c[(NBK - 1) & 1][0], c[(NBK - 1) & 1][1]);
    } else {
      if (nbv > 0) mma_block(0, c[0]);
#pragma unroll
      for (int nb = 1; nb < NBK; ++nb) {
        if (nb < nbv) mma_block(nb, c[nb & 1]);
        __builtin_amdgcn_sched_barrier(0);
        if (nb - 1 < nbv) epi_block(nb - 1, c[(nb - 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (NBK - 1 < nbv) epi_block(NBK - 1, c[(NBK - 1) & 1]);
    }
    lstore(buf ^ 1);
    // The score stores come after the next tile's loads have been waited for,
    // and the barrier settles LDS only: no wave waits for its score stores.
    // (Buffer buf ^ 1 was last read before the previous barrier.)
    if (full && half == 0)
#pragma unroll
      for (int nb = 0; nb < NBK; ++nb) sr[k0 + 32 * nb + col] = scv[nb];
    lds_barrier();
  }
}

__global__ __launch_bounds__(256) void indexer_f32(const float* __restrict__ q, const float* __restrict__ k,
                                                   const float* __restrict__ w, float* __restrict__ scores,
                                                   int64_t Tq, int64_t N, int64_t q_pos0, Vis vis, int H_I,
                                                   int D_I, int64_t chunks) {
  const int64_t blk = blockIdx.x;
  const int64_t rowi = blk / chunks;
  const int64_t s = (blk % chunks) * 256 + threadIdx.x;
  const int64_t t = rowi % Tq, b = rowi / Tq;
  const int64_t n_valid = visible_keys(vis, seq_q0(vis, b, Tq, q_pos0), t, N);
  if (s >= n_valid) return;
  const float* qr = q + rowi * H_I * D_I;
  const float* kr = k + (b * N + s) * D_I;
  const float* wr = w + rowi * H_I;
  float acc = 0.f;
  for (int h = 0; h < H_I; ++h) {
    float dot = 0.f;
    for (int d = 0; d < D_I; ++d) dot = fmaf(qr[h * D_I + d], kr[d], dot);
    acc = fmaf(wr[h], fmaxf(dot, 0.f), acc);
  }
  scores[rowi * N + s] = acc;
}

// ---------------------------------------------------------------------------
// FP8 indexer (DeepSeek-V3.2 documentation, "DeepSeek Sparse Attention (DSA)":
// the reference indexer runs in FP8 after a Hadamard rotation of queries and
// keys; the rotation is orthogonal, so the scores are those of the bf16 path
// up to the quantisation).  Rows of 128 are rotated by the unnormalised
// Sylvester matrix (fast Walsh-Hadamard transform in float32, pair distance
// 1, 2, 4, ...), scaled by one power of two per row (the smallest 2^e with
// max|y| <= 448 * 2^e, so the scaling is exact) and rounded to OCP E4M3,
// nearest even.  The score divides by 128, the squared norm of the rotation:
//   I[t,s] = ks[s] * sum_h (w[t,h] * qs[t,h] / 128) * max(0, q8[t,h] . k8[s]).
// The key cache is read as codes, half the bytes of bf16.  The codes are
// widened to bf16 in registers (exact: E4M3 values have four significant
// bits) for the bf16 MFMA, whose products and sums of such values were exact
// when measured, whereas the fp8 MFMA rounded its dot products to about
// 2^-13 of the largest product.
// ---------------------------------------------------------------------------

// OCP E4M3 code of v (|v| <= 448), round to nearest even.
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = fabsf(v);
  if (a < 0.015625f) return sign | (uint32_t)__builtin_rintf(a * 512.0f);  // multiples of 2^-9; 8 is 0x08
  const uint32_t au = __float_as_uint(a);
  int e = (int)(au >> 23) - 127;
  uint32_t q = (au >> 20) & 7u;
  const uint32_t rem = au & 0xfffffu;
  if (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) ++q;
  if (q == 8u) {
    q = 0u;
    ++e;
  }
  return sign | ((uint32_t)(e + 7) << 3) | q;
}

// One wave per row of 128: lane l holds elements 2l and 2l+1.
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const uint16_t* __restrict__ x, uint8_t* __restrict__ codes,
                                                           float* __restrict__ scales, int64_t R) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * 4;
  for (int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); r < R; r += nw) {
    const uint32_t pair = *reinterpret_cast<const uint32_t*>(x + r * ID + 2 * lane);
    const float a = bf16_bits_to_float(pair & 0xffffu), b = bf16_bits_to_float(pair >> 16);
    float y0 = a + b, y1 = a - b;  // pair distance 1, inside the lane
    // distance 2m: the partner element sits in lane l ^ m; the lane with bit m
    // clear holds the lower element (sum), the other the upper (difference)
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const float p0 = __shfl_xor(y0, m), p1 = __shfl_xor(y1, m);
      const bool upper = (lane & m) != 0;
      y0 = upper ? p0 - y0 : y0 + p0;
      y1 = upper ? p1 - y1 : y1 + p1;
    }
    const uint32_t ab = wave_max(max(__float_as_uint(fabsf(y0)), __float_as_uint(fabsf(y1))));
    int e = 0;
    if (ab != 0u) {
      int E;
      const float m = frexpf(__uint_as_float(ab), &E);  // amax = m * 2^E, 0.5 <= m < 1; 448 = 0.875 * 2^9
      e = m <= 0.875f ? E - 9 : E - 8;
    }
    const uint32_t c0 = e4m3_rne(ldexpf(y0, -e)), c1 = e4m3_rne(ldexpf(y1, -e));
    *reinterpret_cast<uint16_t*>(codes + r * ID + 2 * lane) = (uint16_t)(c0 | (c1 << 8));
    if (lane == 0) scales[r] = ldexpf(1.0f, e);
  }
}

// Eight E4M3 codes (bytes of lo, then hi) -> eight bf16 values (exact: every
// E4M3 value, subnormals included, is a bf16 value).  The gfx950 scaled
// conversion turns two codes into two bf16 values in one instruction; with
// scale 1 it reproduced the exact decoding of all 256 codes in every byte
// position on the hardware, NaN codes giving NaN.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  const b2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const b2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const b2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const b2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Query codes of one row as bf16 MFMA operands (same layout as load_query),
// with each head's weight folded with its scale and the rotation's 1/128.
__device__ __forceinline__ void load_query_fp8(QFrags& f, const uint8_t* __restrict__ q8, const float* __restrict__ qs,
                                               const uint16_t* __restrict__ w, int64_t row, int half, int col) {
  const uint8_t* qr = q8 + row * (IH * ID) + 64 * half;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const u32x4 x0 = *reinterpret_cast<const u32x4*>(qr + col * ID + 16 * v);
    const u32x4 x1 = *reinterpret_cast<const u32x4*>(qr + (32 + col) * ID + 16 * v);
    f.a0[2 * v] = fp8x8_to_bf16(x0[0], x0[1]);
    f.a0[2 * v + 1] = fp8x8_to_bf16(x0[2], x0[3]);
    f.a1[2 * v] = fp8x8_to_bf16(x1[0], x1[1]);
    f.a1[2 * v + 1] = fp8x8_to_bf16(x1[2], x1[3]);
  }
  const uint16_t* wr = w + row * IH;
  const float* sr = qs + row * IH;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int h0 = mfma_row(i, half), h1 = 32 + h0;
    f.w0[i] = bf16_bits_to_float(wr[h0]) * sr[h0] * 0.0078125f;
    f.w1[i] = bf16_bits_to_float(wr[h1]) * sr[h1] * 0.0078125f;
  }
}

// Decode kernel over an FP8 key cache: the bf16 decode kernel's structure
// with 128-byte key rows.  A tile of 32 keys is 4 KiB, fetched by four
// direct-to-LDS loads of eight keys each; lane L of a load fetches chunk
// (L & 7) ^ (L >> 3) of key L >> 3 and lands at slot L, so chunk c of tile key
// r sits at slot 8r + (c ^ (r & 7)).  The key scales are applied when the
// workgroup's scores leave LDS; with PRESEL they are applied in LDS first, and
// the segment's pre-selection list (presel_segment) is drawn from the scaled
// scores before they leave.
template <int WAVES, int NBUF, int SCAP, bool PAGED = false, bool PRESEL = false>
__global__ __launch_bounds__(WAVES * 64, 1) void indexer_dma_fp8(
    const uint8_t* __restrict__ q8, const float* __restrict__ qs, const uint8_t* __restrict__ k8,
    const float* __restrict__ ks, const uint16_t* __restrict__ w, float* __restrict__ scores, int64_t Tq, int64_t N,
    int64_t q_pos0, Vis vis, int64_t keys_per_wg, Paged pg, PreselWs ps) {
  static_assert(!(PAGED && PRESEL), "the pre-selecting FP8 kernel reads a contiguous cache");
  constexpr int TILE_BYTES = 32 * ID;
  static_assert(NBUF >= 2 && NBUF <= 8, "the vmcnt waits below cover up to seven tiles in flight");
  static_assert(WAVES * NBUF * TILE_BYTES + SCAP * 4 <= 160 * 1024, "LDS budget");
  __shared__ __align__(16) uint8_t kt[WAVES][NBUF][TILE_BYTES];
  __shared__ __align__(16) float sl[SCAP];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5, col = lane & 31;
  const int64_t t = blockIdx.y, b = blockIdx.z;
  const int64_t row = b * Tq + t;
  const int64_t n_valid = visible_keys(vis, seq_q0(vis, b, Tq, q_pos0), t, N);
  const int64_t k_begin = (int64_t)blockIdx.x * keys_per_wg;  // a multiple of 32
  const int64_t k_end = min(n_valid, k_begin + keys_per_wg);
  if (k_begin >= k_end) return;
  const int total_tiles = (int)((k_end - k_begin + 31) / 32);
  const int nt = total_tiles > wave ? (total_tiles - wave + WAVES - 1) / WAVES : 0;

  const uint8_t* kb = k8 + (PAGED ? 0 : b * N * ID);
  PageRows<PAGED> pr;
  pr.load(pg, b, k_begin, k_end, lane);
  const uint32_t ring = lds_address(&kt[wave][0][0]);
  const uint32_t voff = 128u * (uint32_t)(lane >> 3) + 16u * (uint32_t)((lane & 7) ^ (lane >> 3));
  auto key0_of = [&](int it) { return k_begin + 32 * (int64_t)(it * WAVES + wave); };
  auto dma_tile = [&](int it) {
    const int64_t key0 = key0_of(it);
    const uint32_t dst = ring + (uint32_t)((it % NBUF) * TILE_BYTES);
    if (PAGED) {
      const int64_t r0 = pr.row(key0);
#pragma unroll
      for (int u = 0; u < 4; ++u) dma16_stream(kb + (r0 + 8 * u) * ID, voff, dst + 1024u * u);
    } else if (key0 + 32 <= N) {
#pragma unroll
      for (int u = 0; u < 4; ++u) dma16_stream(kb + (key0 + 8 * u) * ID, voff, dst + 1024u * u);
    } else {
      // last rows of the cache: clamp to a real row (those keys are never scored)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t kbase = min(key0 + 8 * u, N - 1);
        const int64_t key = min(key0 + 8 * u + (lane >> 3), N - 1);
        const uint32_t off = (uint32_t)(key - kbase) * 128u + (voff & 127u);
        dma16_stream(kb + kbase * ID, off, dst + 1024u * u);
      }
    }
  };
  QFrags f;
  load_query_fp8(f, q8, qs, w, row, half, col);
  // With the pre-selection the key scales are applied to the scores in LDS
  // before the lists are drawn: each thread's scales (keys k_begin + t +
  // 64*WAVES*j) are loaded here, with the queries, so that the epilogue does
  // not wait for them.
  constexpr int KSPT = PRESEL ? SCAP / (WAVES * 64) : 1;
  float ksv[KSPT];
  if constexpr (PRESEL) {
    const int nk = (int)(k_end - k_begin);
    const float* ksr = ks + b * N + k_begin;
#pragma unroll
    for (int j = 0; j < KSPT; ++j) ksv[j] = ksr[min((int)threadIdx.x + WAVES * 64 * j, nk - 1)];
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int p = 0; p < NBUF - 1; ++p)
    if (p < nt) dma_tile(p);
  __builtin_amdgcn_s_waitcnt(0);

  // operand of k-step s: channels 64*half + 8s .. +7 = chunk 4*half + s/2, bytes 8*(s&1)
  const uint32_t rbase = 128u * col;
  for (int it = 0; it < nt; ++it) {
    if (it + NBUF - 1 < nt) dma_tile(it + NBUF - 1);
    const int after = min(NBUF - 1, nt - 1 - it);
    switch (after) {
      case 7: asm volatile("s_waitcnt vmcnt(28)" ::: "memory"); break;
      case 6: asm volatile("s_waitcnt vmcnt(24)" ::: "memory"); break;
      case 5: asm volatile("s_waitcnt vmcnt(20)" ::: "memory"); break;
      case 4: asm volatile("s_waitcnt vmcnt(16)" ::: "memory"); break;
      case 3: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
      case 2: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
      case 1: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
      default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    }
    const uint8_t* tile = &kt[wave][it % NBUF][0];
    f32x16 c0 = {}, c1 = {};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int c = 4 * half + (s >> 1);
      const u32x2 kv = *reinterpret_cast<const u32x2*>(tile + rbase + 16u * (uint32_t)(c ^ (col & 7)) + 8u * (s & 1));
      const bf16x8 bv = fp8x8_to_bf16(kv[0], kv[1]);
      c0 = mfma32x32x16(f.a0[s], bv, c0);
      c1 = mfma32x32x16(f.a1[s], bv, c1);
    }
    const float sc = weighted_relu_sum(f, c0, c1);
    if (half == 0) sl[key0_of(it) - k_begin + col] = sc;
  }
  __syncthreads();
  const int n = (int)(k_end - k_begin);
  float* dst = scores + row * N + k_begin;
  if (PAGED) {
    // key scales through the block table: four consecutive keys share a block
    for (int i0 = 0; i0 < n; i0 += 4 * WAVES * 64) {
      const int i = i0 + 4 * (int)threadIdx.x;
      const int64_t r = pr.row_any(k_begin + min(i, n - 1));  // every lane takes part in the exchange
      for (int e = 0; e < 4; ++e)
        if (i + e < n) dst[i + e] = sl[i + e] * ks[r + e];
    }
    return;
  }
  const float* ksr = ks + b * N + k_begin;
  if constexpr (PRESEL) {
    // the key scales applied in LDS, so that the lists hold the final scores
    // (the same products the store pass below would form)
#pragma unroll
    for (int j = 0; j < KSPT; ++j) {
      const int i = (int)threadIdx.x + WAVES * 64 * j;
      if (i < n) sl[i] *= ksv[j];
    }
    lds_barrier();
    // the key rings are idle: every wave awaited its last tile before the first barrier
    presel_segment<WAVES, SCAP>(sl, n, k_begin, row, (int)blockIdx.x, ps, reinterpret_cast<uint32_t*>(&kt[0][0][0]));
    if (((row * N) & 3) == 0) {
      for (int i = 4 * (int)threadIdx.x; i < n; i += 4 * WAVES * 64) {
        if (i + 4 <= n)
          __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(&sl[i]), reinterpret_cast<f32x4*>(dst + i));
        else
          for (int e = i; e < n; ++e) dst[e] = sl[e];
      }
    } else {
      for (int i = (int)threadIdx.x; i < n; i += WAVES * 64) dst[i] = sl[i];
    }
    return;
  }
  if (((row * N) & 3) == 0 && ((b * N) & 3) == 0) {
    for (int i = 4 * (int)threadIdx.x; i < n; i += 4 * WAVES * 64) {
      if (i + 4 <= n) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(&sl[i]) * *reinterpret_cast<const f32x4*>(ksr + i);
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(dst + i));
      } else {
        for (int e = i; e < n; ++e) dst[e] = sl[e] * ksr[e];
      }
    }
  } else {
    for (int i = (int)threadIdx.x; i < n; i += WAVES * 64) dst[i] = sl[i] * ksr[i];
  }
}

}  // namespace

namespace {

// Launch shape of the bf16 decode kernel.  One workgroup per compute unit at
// a time (each holds all of LDS).  One round of 256 workgroups, split evenly
// over the rows, when the rows fit in at most SCAP keys per workgroup, else
// two rounds (at most 512), so that no partly filled round appears; whole
// tiles for every wave.  A second round costs a second workgroup start: at
// one or four queries of 128K keys one round was 27% and 11% faster.
constexpr int DEC_WAVES = 4, DEC_NBUF = 4, DEC_SCAP = 8192;
constexpr int DEC_ROUND = 256;  // workgroups resident at once (one per compute unit)
struct DecodeGeom {
  int64_t kpw, G;  // keys per workgroup, workgroups per row
};
DecodeGeom decode_geometry(int64_t rows, int64_t nmax) {
  int64_t per_row = DEC_ROUND / rows > 1 ? DEC_ROUND / rows : 1;
  if ((nmax + per_row - 1) / per_row > DEC_SCAP) per_row = 2 * DEC_ROUND / rows > 1 ? 2 * DEC_ROUND / rows : 1;
  int64_t kpw = (nmax + per_row - 1) / per_row;
  kpw = (kpw + 32 * DEC_WAVES - 1) / (32 * DEC_WAVES) * (32 * DEC_WAVES);
  if (kpw > DEC_SCAP) kpw = DEC_SCAP;
  if (kpw < 32 * DEC_WAVES) kpw = 32 * DEC_WAVES;
  return {kpw, (nmax + kpw - 1) / kpw};
}

// Launch shape of the FP8 decode kernel.  Two workgroups resident per compute
// unit (72 KiB of LDS each), three 4 KiB tiles in flight per wave.  One round
// of 512 workgroups when the rows fit in at most FP8_SCAP keys per workgroup
// (at one and four queries of 128K keys, 31% and 32% faster than four
// rounds), else about eight workgroups per compute unit over the launch, in
// whole rounds: the best of a sweep over waves (2, 4, 8), ring depth (2..8)
// and keys per workgroup (1024..8192) at the 128K decode batch.
//
// The pre-selecting instance runs one list epilogue per workgroup, so it takes
// fewer, longer segments: up to FP8P_SCAP = 8192 keys with a ring of three
// tiles (two tiles in flight per wave; 80 KiB of LDS, two per compute unit),
// 512 workgroups at the 128K decode batch.  There, against 2048-key segments
// and four rounds, the fused FP8 forward took 146 rather than 155 us (4096-key
// segments: 150 us; one workgroup per unit with a ring of 4, 6 or 8 tiles, or
// of 8 waves with 4 tiles each: 152-167 us).
constexpr int FP8_WAVES = 4, FP8_NBUF = 4, FP8_SCAP = 2048;
constexpr int FP8P_WAVES = 4, FP8P_NBUF = 3, FP8P_SCAP = 8192;
DecodeGeom fp8_decode_geometry(int64_t rows, int64_t nmax, bool presel = false) {
  const int64_t scap = presel ? FP8P_SCAP : FP8_SCAP, tile_keys = 32 * (presel ? FP8P_WAVES : FP8_WAVES);
  int64_t per_row = 512 / rows > 1 ? 512 / rows : 1;
  if (!presel && (nmax + per_row - 1) / per_row > scap) per_row = 2048 / rows > 1 ? 2048 / rows : 1;
  int64_t kpw = (nmax + per_row - 1) / per_row;
  kpw = (kpw + tile_keys - 1) / tile_keys * tile_keys;  // whole tiles for every wave
  if (kpw > scap) kpw = scap;
  if (kpw < tile_keys) kpw = tile_keys;
  return {kpw, (nmax + kpw - 1) / kpw};
}

}  // namespace

// Pre-selection applies to decode rows too long for the one-workgroup top-k
// (more than 16384 keys, K <= 4096) whose segments can each list several times
// their expected share K * kpw / nmax of the row's K best keys within the
// row's list budget.
bool presel_geometry(int64_t B, int64_t Tq, int64_t N, int64_t nmax, int K, PreselWs& ps, bool fp8) {
  if (Tq > 4 || nmax <= 16384 || N > 0x7fffffff || K > 4096 || nmax < K) return false;
  const DecodeGeom g = fp8 ? fp8_decode_geometry(B * Tq, nmax, true) : decode_geometry(B * Tq, nmax);
  if (g.G > 512) return false;
  const int64_t cap = min((int64_t)kPreselMaxCap, (int64_t)kPreselRowCap / g.G);
  const double share = (double)K * (double)g.kpw / (double)nmax;
  if ((double)cap < 1.4 * (share + 6.0 * sqrt(share) + 8.0)) return false;
  ps.kpw = g.kpw;
  ps.G = (int32_t)g.G;
  ps.cap = (int32_t)cap;
  // list target: the expected share plus six standard deviations of it (keys i.i.d. over the row)
  ps.tgt = (int32_t)min((double)cap, share + 6.0 * sqrt(share) + 8.0);
  return true;
}

static size_t presel_align(size_t x) { return (x + 255) & ~size_t(255); }

size_t presel_workspace_bytes(int64_t B, int64_t Tq, int64_t N, int K) {
  PreselWs ps;
  if (!presel_geometry(B, Tq, N, N, K, ps) && !presel_geometry(B, Tq, N, N, K, ps, true)) return 0;
  // any longest row <= N: G <= 512 segments and G * cap <= kPreselRowCap entries per row
  const size_t R = (size_t)(B * Tq);
  return 2 * presel_align(R * 512 * sizeof(uint32_t)) + presel_align(R * kPreselRowCap * sizeof(uint2));
}

PreselWs presel_ws(void* workspace, int64_t B, int64_t Tq, int64_t N, int64_t nmax, int K, bool fp8) {
  PreselWs ps{};
  presel_geometry(B, Tq, N, nmax, K, ps, fp8);
  const size_t R = (size_t)(B * Tq);
  char* p = static_cast<char*>(workspace);
  ps.count = reinterpret_cast<uint32_t*>(p);
  ps.thr = reinterpret_cast<uint32_t*>(p + presel_align(R * 512 * sizeof(uint32_t)));
  ps.list = reinterpret_cast<uint2*>(p + 2 * presel_align(R * 512 * sizeof(uint32_t)));
  return ps;
}

hipError_t launch_index_scores_bf16(const uint16_t* q_idx, const uint16_t* k_idx, const uint16_t* w,
                                    float* scores, int64_t B, int64_t Tq, int64_t N, int64_t q_pos0,
                                    hipStream_t stream, const int64_t* seq_lens, int m, const Paged* pg,
                                    const PreselWs* ps) {
  const Vis vis{seq_lens, m};
  // longest visible row: with per-sequence lengths only N is known on the host
  const int64_t nmax = seq_lens != nullptr ? N : min(N, (q_pos0 + Tq) / m);
  if (nmax <= 0) return hipSuccess;  // no query sees a row
  if (Tq <= 4) {
    constexpr int WAVES = DEC_WAVES, NBUF = DEC_NBUF, SCAP = DEC_SCAP;
    const DecodeGeom geo = decode_geometry(B * Tq, nmax);
    const int64_t kpw = geo.kpw;
    if (ps != nullptr && (ps->kpw != kpw || ps->G != geo.G)) return hipErrorInvalidValue;
    dim3 grid((unsigned)geo.G, (unsigned)Tq, (unsigned)B);
    const PreselWs none{};
    if (pg != nullptr) {
      if (ps != nullptr)
        hipLaunchKernelGGL((indexer_dma_bf16<WAVES, NBUF, SCAP, true, true>), grid, dim3(WAVES * 64), 0, stream,
                           q_idx, k_idx, w, scores, Tq, N, q_pos0, vis, kpw, *pg, *ps);
      else
        hipLaunchKernelGGL((indexer_dma_bf16<WAVES, NBUF, SCAP, true>), grid, dim3(WAVES * 64), 0, stream, q_idx,
                           k_idx, w, scores, Tq, N, q_pos0, vis, kpw, *pg, none);
    } else {
      if (ps != nullptr)
        hipLaunchKernelGGL((indexer_dma_bf16<WAVES, NBUF, SCAP, false, true>), grid, dim3(WAVES * 64), 0, stream,
                           q_idx, k_idx, w, scores, Tq, N, q_pos0, vis, kpw, Paged{}, *ps);
      else
        hipLaunchKernelGGL((indexer_dma_bf16<WAVES, NBUF, SCAP>), grid, dim3(WAVES * 64), 0, stream, q_idx, k_idx, w,
                           scores, Tq, N, q_pos0, vis, kpw, Paged{}, none);
    }
  } else {
    if (pg != nullptr) return hipErrorInvalidValue;  // paged caches: decode shapes only
    constexpr int WAVES = 8;
    const int64_t nqb = (Tq + WAVES - 1) / WAVES;
    dim3 grid((unsigned)nqb, (unsigned)B);
    hipLaunchKernelGGL((indexer_tiled_bf16<WAVES, 128, 1>), grid, dim3(WAVES * 64), 0, stream, q_idx, k_idx, w, scores,
                       Tq, N, q_pos0, vis, nqb);
  }
  return hipGetLastError();
}

hipError_t launch_index_scores_f32(const float* q_idx, const float* k_idx, const float* w, float* scores,
                                   int64_t B, int64_t Tq, int64_t N, int64_t q_pos0, int H_I, int D_I,
                                   hipStream_t stream, const int64_t* seq_lens, int m) {
  const Vis vis{seq_lens, m};
  const int64_t chunks = ((seq_lens != nullptr ? N : min(N, (q_pos0 + Tq) / m)) + 255) / 256;
  dim3 grid((unsigned)(B * Tq * chunks));
  if (chunks == 0) return hipSuccess;  // no query sees a row
  hipLaunchKernelGGL(indexer_f32, grid, dim3(256), 0, stream, q_idx, k_idx, w, scores, Tq, N, q_pos0, vis, H_I, D_I,
                     chunks);
  return hipGetLastError();
}

hipError_t launch_quantize_fp8(const uint16_t* x, uint8_t* codes, float* scales, int64_t R, hipStream_t stream) {
  if (R <= 0) return hipSuccess;
  const int64_t blocks = (R + 3) / 4 < 16384 ? (R + 3) / 4 : 16384;
  hipLaunchKernelGGL(quantize_fp8_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, codes, scales, R);
  return hipGetLastError();
}

hipError_t launch_index_scores_fp8(const uint8_t* q8, const float* qs, const uint8_t* k8, const float* ks,
                                   const uint16_t* w, float* scores, int64_t B, int64_t Tq, int64_t N,
                                   int64_t q_pos0, hipStream_t stream, const int64_t* seq_lens, const Paged* pg,
                                   const PreselWs* ps) {
  const Vis vis{seq_lens, 1};
  const int64_t nmax = seq_lens != nullptr ? N : min(N, q_pos0 + Tq);
  if (nmax <= 0) return hipSuccess;  // no query sees a key
  constexpr int WAVES = FP8_WAVES, NBUF = FP8_NBUF, SCAP = FP8_SCAP;
  const DecodeGeom geo = fp8_decode_geometry(B * Tq, nmax, ps != nullptr);
  const int64_t kpw = geo.kpw;
  if (ps != nullptr && (pg != nullptr || ps->kpw != kpw || ps->G != geo.G)) return hipErrorInvalidValue;
  dim3 grid((unsigned)geo.G, (unsigned)Tq, (unsigned)B);
  const PreselWs none{};
  if (pg != nullptr)
    hipLaunchKernelGGL((indexer_dma_fp8<WAVES, NBUF, SCAP, true>), grid, dim3(WAVES * 64), 0, stream, q8, qs, k8, ks, w,
                       scores, Tq, N, q_pos0, vis, kpw, *pg, none);
  else if (ps != nullptr)
    hipLaunchKernelGGL((indexer_dma_fp8<FP8P_WAVES, FP8P_NBUF, FP8P_SCAP, false, true>), grid, dim3(FP8P_WAVES * 64),
                       0, stream, q8, qs, k8, ks, w, scores, Tq, N, q_pos0, vis, kpw, Paged{}, *ps);
  else
    hipLaunchKernelGGL((indexer_dma_fp8<WAVES, NBUF, SCAP>), grid, dim3(WAVES * 64), 0, stream, q8, qs, k8, ks, w,
                       scores, Tq, N, q_pos0, vis, kpw, Paged{}, none);
  return hipGetLastError();
}

}  // namespace dsa

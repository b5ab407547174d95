// Device helpers of the top-k selection, shared by the top-k kernels and the
// decode indexer's pre-selection epilogue.
#pragma once

#include "device_common.h"

namespace dsa {

// Number of bits needed for x (0 for x == 0).
__device__ __forceinline__ int bit_width(uint32_t x) { return x == 0u ? 0 : 32 - __clz(x); }

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

// Workgroup barrier that settles LDS only.  __syncthreads() also waits for
// the wave's outstanding global stores (its release fence), which a barrier
// that only exchanges LDS data need not do.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Exclusive prefix sum of v over a workgroup of WAVES waves; `total`
// receives the sum.  sbuf: WAVES words.  Without TRAIL the closing barrier is
// left out, and the caller must pass another barrier before sbuf is written
// again.  LDS_ONLY: the barriers settle LDS only (see lds_barrier).
template <int WAVES, bool TRAIL = true, bool LDS_ONLY = false>
__device__ __forceinline__ uint32_t block_excl_scan_w(uint32_t v, uint32_t& total, uint32_t* sbuf) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t x = wave_incl_scan(v);
  if (lane == 63) sbuf[wave] = x;
  if (LDS_ONLY) lds_barrier();
  else __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < WAVES; ++w) {
    const uint32_t s = sbuf[w];
    tot += s;
    before += (w < wave) ? s : 0u;
  }
  if (TRAIL) {
    if (LDS_ONLY) lds_barrier();
    else __syncthreads();
  }
  total = tot;
  return before + x - v;
}

}  // namespace dsa

/*
 * Seeded synthetic input generator (counter-based, thread-parallel).
 *
 * This file holds no arithmetic of the attention method: it only draws the
 * random tensors that both the CPU oracle and the GPU path consume, so the
 * two sides see byte-identical inputs.
 *
 * Random source: SplitMix64 (Steele, Lea, Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014).  The i-th output of a
 * SplitMix64 stream seeded with `key` is mix(key + (i + 1) * GAMMA); using
 * that closed form makes every element a pure function of (key, i), so any
 * slice of a tensor can be regenerated on its own and the result does not
 * depend on the thread count.
 *
 * Distributions:
 *   normal    Box-Muller (1958): sqrt(-2 ln u1) * cos(2 pi u2), u1/u2 from
 *             outputs 2i and 2i+1 of the stream; computed in double, then
 *             rounded to fp32 and, for bf16 storage, to bf16 (nearest-even).
 *   int       uniform integer in [lo, hi] by a 32x32->64 multiply-high of
 *             the top 32 bits (bias below (hi-lo+1)/2^32, negligible).
 *   pow2      2^e with e a uniform integer in [lo, hi].
 *   choice    uniform over a small set of values passed by the caller.
 *   floyd     per row, k distinct integers of [0, n) by R. W. Floyd's
 *             sampling algorithm (Bentley & Floyd, CACM 30(9), 1987),
 *             emitted in draw order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SM64_GAMMA 0x9e3779b97f4a7c15ULL

static inline uint64_t sm64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
  return z ^ (z >> 31);
}

/* i-th output of the SplitMix64 stream seeded with key */
static inline uint64_t sm64_at(uint64_t key, uint64_t i) {
  return sm64_mix(key + (i + 1) * SM64_GAMMA);
}

uint64_t synth_stream_key(uint64_t seed, uint64_t workload_id, uint64_t tensor_id) {
  uint64_t k = sm64_mix(seed + SM64_GAMMA);
  k = sm64_mix(k ^ (workload_id * 0xd1b54a32d192ed03ULL));
  k = sm64_mix(k ^ (tensor_id * 0x8cb92ba72f3d8dd7ULL));
  return k;
}

/* open interval (0,1) from the top 53 bits */
static inline double u01(uint64_t x) { return ((double)(x >> 11) + 0.5) * (1.0 / 9007199254740992.0); }

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

static inline uint32_t uniform_below(uint64_t x, uint32_t m) {
  return (uint32_t)(((x >> 32) * (uint64_t)m) >> 32);
}

enum { SYN_NORMAL = 0, SYN_INT = 1, SYN_POW2 = 2, SYN_CHOICE = 3 };
enum { SYN_F32 = 0, SYN_BF16 = 1 };

static inline double draw_value(uint64_t key, uint64_t i, int kind, int lo, int hi,
                                const double* set, int nset) {
  switch (kind) {
    case SYN_NORMAL: {
      double u1 = u01(sm64_at(key, 2 * i));
      double u2 = u01(sm64_at(key, 2 * i + 1));
      return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925 * u2);
    }
    case SYN_INT:
      return (double)(lo + (int)uniform_below(sm64_at(key, i), (uint32_t)(hi - lo + 1)));
    case SYN_POW2:
      return ldexp(1.0, lo + (int)uniform_below(sm64_at(key, i), (uint32_t)(hi - lo + 1)));
    case SYN_CHOICE:
      return set[uniform_below(sm64_at(key, i), (uint32_t)nset)];
  }
  return 0.0;
}

/* Fill out[0..count) with elements start..start+count of the stream. */
int synth_fill(uint64_t key, uint64_t start, uint64_t count, int kind, int lo, int hi,
               const double* set, int nset, int dtype, void* out) {
  if (kind < SYN_NORMAL || kind > SYN_CHOICE) return 1;
  if ((kind == SYN_INT || kind == SYN_POW2) && hi < lo) return 1;
  if (kind == SYN_CHOICE && (set == NULL || nset <= 0)) return 1;
  if (dtype == SYN_F32) {
    float* o = (float*)out;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < (int64_t)count; ++j)
      o[j] = (float)draw_value(key, start + (uint64_t)j, kind, lo, hi, set, nset);
  } else if (dtype == SYN_BF16) {
    uint16_t* o = (uint16_t*)out;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < (int64_t)count; ++j)
      o[j] = f32_to_bf16_rne((float)draw_value(key, start + (uint64_t)j, kind, lo, hi, set, nset));
  } else {
    return 1;
  }
  return 0;
}

/* rows x k distinct integers of [0, n), Floyd's algorithm, draw order. */
int synth_floyd(uint64_t key, int64_t rows, int64_t n, int64_t k, int32_t* out) {
  if (k > n || k < 0 || n <= 0 || n > 0x7fffffff) return 1;
  int err = 0;
#pragma omp parallel
  {
    uint8_t* seen = (uint8_t*)calloc((size_t)n, 1);
    if (!seen) {
#pragma omp atomic write
      err = 1;
    } else {
#pragma omp for schedule(static)
      for (int64_t r = 0; r < rows; ++r) {
        uint64_t rk = sm64_mix(key ^ ((uint64_t)(r + 1) * 0xa0761d6478bd642fULL));
        int32_t* o = out + r * k;
        int64_t m = 0;
        for (int64_t j = n - k; j < n; ++j) {
          int64_t t = (int64_t)uniform_below(sm64_at(rk, (uint64_t)m), (uint32_t)(j + 1));
          int64_t pick = seen[t] ? j : t;
          seen[pick] = 1;
          o[m++] = (int32_t)pick;
        }
        for (int64_t i = 0; i < k; ++i) seen[o[i]] = 0;
      }
      free(seen);
    }
  }
  return err;
}

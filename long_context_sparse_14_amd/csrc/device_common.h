// Device helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 16-byte global load of eight bf16 values.
__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits) {
  return __uint_as_float(bits << 16);
}

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t float_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// One 32x32x16 bf16 matrix-core step: c += a * b (fp32 accumulate).
// Operand layout (wave64): lane j supplies row (j % 32) of A and column
// (j % 32) of B, each with eight consecutive k-slots chosen by j / 32.
// Result layout: lane j holds column (j % 32), rows 8*(i/4) + 4*(j/32) + i%4
// for register i = 0..15.
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Two floats -> packed bf16 pair (lo in bits 0..15), round to nearest even,
// with the gfx950 conversion instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// Max / sum of the values of lanes j and j ^ 32.  v_permlane32_swap with both
// operands equal to v leaves the lower half's values in one result register
// and the upper half's in the other, in every lane, so a symmetric combination
// of the two is the same in lane j and lane j ^ 32.
__device__ __forceinline__ float max_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ int mfma_row(int i, int half) { return 8 * (i >> 2) + 4 * half + (i & 3); }

// Order-preserving map of a float32 to uint32 (larger float -> larger key);
// -0 and +0 map to the same key.
__device__ __forceinline__ uint32_t float_order_key(float v) {
  uint32_t u = __float_as_uint(v);
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// 16-byte direct-to-LDS load: every lane reads 16 B at base + voff and the
// wave writes them to LDS bytes [lds_addr + 16*lane, +16).  base is
// wave-uniform (scalar registers), voff a 32-bit per-lane byte offset; the
// instruction offset stays 0 because it would move the LDS destination too.
// Written as inline asm so that the compiler does not track it: otherwise it
// cannot tell that reads of one LDS buffer do not alias loads into another and
// waits for them before every read.  The instruction has no register result;
// its completion is awaited explicitly with vmcnt, which counts it like any
// other vector memory load of the wave.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %2" ::"v"(voff), "s"(lds_addr), "s"(base)
               : "memory", "m0");
}

// The same load with the nontemporal hint, for data read exactly once (the
// decode indexers' key streams): the lines are not kept in the caches, which
// raised the decode indexer's stream from about 5.8 to 6.5 TB/s.
__device__ __forceinline__ void dma16_stream(const void* base, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %2 nt" ::"v"(voff), "s"(lds_addr), "s"(base)
               : "memory", "m0");
}

// The same direct-to-LDS load from a full 64-bit per-lane address (no scalar
// base), for sources whose per-lane offsets do not fit 32 bits.
__device__ __forceinline__ void dma16_addr(const void* addr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(addr), "s"(lds_addr)
               : "memory", "m0");
}

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  typedef const __attribute__((address_space(3))) char* lds_ptr;
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr)p));
}

// Which cache rows a query sees.  seq_lens (device, [B], may be null):
// per-sequence lengths in tokens; with them the queries of sequence b are its
// last Tq tokens, else query t sits at position q_pos0 + t.  m: compression
// rate of the key axis: row w summarises positions m*w .. m*w + m - 1 and
// becomes visible once that window has closed (m = 1: row w is position w).
struct Vis {
  const int64_t* seq_lens;
  int32_t m;
};

// Position of query 0 of sequence b.
__device__ __forceinline__ int64_t seq_q0(const Vis& v, int64_t b, int64_t Tq, int64_t q_pos0) {
  return v.seq_lens != nullptr ? v.seq_lens[b] - Tq : q_pos0;
}

// Rows query t of a sequence may see: w < (q0 + t + 1) / m, at most N (none
// for a query at a negative position).
__device__ __forceinline__ int64_t visible_keys(const Vis& v, int64_t q0, int64_t t, int64_t N) {
  const int64_t p1 = q0 + t + 1;
  return p1 <= 0 ? 0 : min(N, p1 / v.m);
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP lane moves
// (row shifts within each row of 16 lanes, then the row broadcasts of lanes
// 15 and 31): six vector adds, no LDS traffic.  All 64 lanes must be active.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return x;
}

// Smallest / largest value over the 64 lanes of a wave (wave-uniform
// results), with the same lane moves as the scan (lanes without a source
// take the identity of the operation).
__device__ __forceinline__ uint32_t wave_min(uint32_t x) {
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)x, 0x111, 0xf, 0xf, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)x, 0x112, 0xf, 0xf, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)x, 0x114, 0xf, 0xf, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)x, 0x118, 0xf, 0xf, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)x, 0x142, 0xa, 0xf, false));
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)x, 0x143, 0xc, 0xf, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}
__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// Sum over the 64 lanes of a wave (wave-uniform result).
__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(x), 63);
}

// Largest value and sum of a float over the 64 lanes of a wave (wave-uniform
// results), with the same lane moves.  The sum adds in the scan's order, so
// it rounds as that order does.
__device__ __forceinline__ float wave_fmax(float x) {
  const int id = __float_as_int(-INFINITY);
#define DSA_FMAX_STEP(ctrl, rows) \
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(id, __float_as_int(x), ctrl, rows, 0xf, false)))
  DSA_FMAX_STEP(0x111, 0xf);
  DSA_FMAX_STEP(0x112, 0xf);
  DSA_FMAX_STEP(0x114, 0xf);
  DSA_FMAX_STEP(0x118, 0xf);
  DSA_FMAX_STEP(0x142, 0xa);
  DSA_FMAX_STEP(0x143, 0xc);
#undef DSA_FMAX_STEP
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}
__device__ __forceinline__ float wave_fsum(float x) {
#define DSA_FSUM_STEP(ctrl, rows) \
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), ctrl, rows, 0xf, false))
  DSA_FSUM_STEP(0x111, 0xf);
  DSA_FSUM_STEP(0x112, 0xf);
  DSA_FSUM_STEP(0x114, 0xf);
  DSA_FSUM_STEP(0x118, 0xf);
  DSA_FSUM_STEP(0x142, 0xa);
  DSA_FSUM_STEP(0x143, 0xc);
#undef DSA_FSUM_STEP
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

}  // namespace dsa

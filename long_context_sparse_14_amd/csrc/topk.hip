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
// Method: exact radix select on order-preserving 32-bit keys.  Four passes of
// 8 bits build a 256-bin LDS histogram of the keys that still match the
// prefix found so far and pick the digit where the running count from the top
// reaches K; after the last pass the K-th key T is known exactly, with
// k_eq = how many keys equal to T must be kept.  A final pass in index order
// computes each kept key's slot with a block-wide prefix sum:
//   slot(i) = #{j < i : key_j > T} + min(#{j < i : key_j == T}, k_eq).
// One 1024-thread workgroup per row; rows of up to 16384 keys are staged once
// in LDS, longer rows are re-read from the L2/MALL-resident score buffer.
#include "device_common.h"
#include "launch.h"

namespace dsa {
namespace {

constexpr int TK_THREADS = 1024;
constexpr int TK_WAVES = TK_THREADS / 64;
constexpr int TK_CAP = 16384;

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

__global__ __launch_bounds__(TK_THREADS) void topk_rows_kernel(const float* __restrict__ scores,
                                                               int32_t* __restrict__ idx, int64_t Tq,
                                                               int64_t N, int64_t q_pos0, int K) {
  __shared__ uint32_t skey[TK_CAP];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sbuf[TK_WAVES];
  __shared__ uint32_t s_digit, s_above;

  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int64_t t = row % Tq;
  const int64_t n = min(N, q_pos0 + t + 1);
  int32_t* out = idx + row * K;
  if (n <= K) {
    for (int64_t i = tid; i < K; i += TK_THREADS) out[i] = i < n ? (int32_t)i : -1;
    return;
  }
  const float* src = scores + row * N;
  const bool in_lds = n <= TK_CAP;
  if (in_lds) {
    for (int64_t i = tid; i < n; i += TK_THREADS) skey[i] = float_order_key(src[i]);
    __syncthreads();
  }
  auto key_at = [&](int64_t i) -> uint32_t { return in_lds ? skey[i] : float_order_key(src[i]); };

  uint32_t prefix = 0, mask = 0, kk = (uint32_t)K;
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int64_t i = tid; i < n; i += TK_THREADS) {
      const uint32_t k = key_at(i);
      if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    const uint32_t c = tid < 256 ? hist[255 - tid] : 0u;
    uint32_t tot;
    const uint32_t ex = block_excl_scan(c, tot, sbuf);
    if (tid < 256 && ex < kk && kk <= ex + c) {
      s_digit = 255u - (uint32_t)tid;
      s_above = ex;
    }
    __syncthreads();
    prefix |= s_digit << shift;
    mask |= 255u << shift;
    kk -= s_above;
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

}  // namespace

size_t topk_workspace_bytes(int64_t, int64_t, int64_t, int) { return 0; }

hipError_t launch_topk(const float* scores, int32_t* idx, int64_t B, int64_t Tq, int64_t N, int64_t q_pos0,
                       int K, void*, hipStream_t stream) {
  hipLaunchKernelGGL(topk_rows_kernel, dim3((unsigned)(B * Tq)), dim3(TK_THREADS), 0, stream, scores, idx, Tq, N,
                     q_pos0, K);
  return hipGetLastError();
}

}  // namespace dsa

// Sparse MLA (absorbed latent form) over the selected keys, on gfx950.
//
// For each query (b,t) and head h, over the selected rows S of the latent
// cache: logits l_j = scale * q[h] . kv[j] (576 wide), out[h] = softmax(l) .
// kv[S, 0:512], lse[h] = ln sum exp(l).  (DeepSeek-V3.2 model documentation,
// section "DeepSeek Sparse Attention (DSA)": the main MLA attention runs over
// the selected tokens only; DeepseekV32Config section: 128 heads,
// kv_lora_rank 512 + qk_rope_head_dim 64.)
//
// bf16 kernel: one workgroup (8 waves, two per SIMD) per (query, split of
// the index list, at most 2048 indices, staged once in LDS).  Each step
// gathers 32 selected latent rows (1152 B each) straight into LDS with
// direct-to-LDS 16-byte loads (no staging registers) into one of three tile
// buffers, so two tiles' gathers (72 KiB) are in flight during the current
// tile's math, and shares the rows across all 128 heads:
//   * S^T = KV_tile . Q^T on 16x16x32 MFMAs: wave w owns heads [16w, 16w+16)
//     and keeps their queries in registers (18 k-steps of 32 channels);
//   * online softmax in fp32 with exp2 on log2e-prescaled logits; the four
//     lanes that share a head reduce with two lane exchanges;
//   * P (bf16) and the per-head rescale factors go through LDS, then
//     O^T = V^T . P^T on 32x32x16 MFMAs: wave w owns value columns
//     [64w, 64w+64) for all 128 heads (128 fp32 accumulators per lane), so
//     every V element is read from LDS once per tile; rescaling is skipped when
//     no head of a block changed its running max.
// The LDS tile is chunk-major: 16-byte chunk p (channels 8p..8p+7) of tile
// row r sits at slot 32*p + (r ^ 4*(p & 3)).  A gather instruction fills 64
// slots = two chunk columns, so every lane always fetches from the same latent
// row (one index per lane per tile); every operand read below is a per-lane
// base plus a compile-time offset; the XOR keeps the reads at the minimum of
// two passes per 512 bytes.  The PV operand (eight keys of one value column
// per lane) comes from the gfx950 transposing LDS read ds_read_b64_tr_b16:
// within each 16-lane group, lane i receives element (i & 3) of the 8 bytes
// addressed by lane 4c + (i >> 2), c = 0..3 -- so lanes that address four
// consecutive value columns of four consecutive keys hand every lane four
// keys of its own column.
// With more than one split, each split writes its normalised partial output
// and its log2-sum-exp to the workspace and a combine kernel merges them.
#include "device_common.h"
#include "launch.h"

namespace dsa {
namespace {

constexpr int MH = 128, MD = 576, MDV = 512, NT = 32;
constexpr int ROW_CHUNKS = MD / 8;          // 72 chunks of 16 B per latent row
constexpr int TILE_CHUNKS = NT * ROW_CHUNKS; // 2304
constexpr int PP = NT + 8;                   // bf16 per LDS probability row
constexpr int MLA_WAVES = 8;
constexpr int NBUF = 3;                      // latent tile buffers (two gathers in flight)
constexpr int MAX_SPLIT_KEYS = 2048;         // indices handled by one workgroup
constexpr int MLA_THREADS = MLA_WAVES * 64;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ s16x4 lds_read_tr16(const uint16_t* p) {
  typedef __attribute__((address_space(3))) s16x4* lds_s16x4_ptr;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)p);
}

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16-byte direct-to-LDS load: every lane reads 16 B at base + voff and the
// wave writes them to LDS bytes [lds_addr + 16*lane, +16).  base is
// wave-uniform (scalar registers), voff a 32-bit per-lane byte offset; the
// instruction offset stays 0 because it would move the LDS destination too.
// Written as inline asm so that the compiler does not track it: otherwise it
// cannot tell that reads of the current tile buffer do not alias the gathers
// into the other buffers and waits for them before every read.  The
// instruction has no register result; completion is awaited explicitly
// (vmcnt) before the barrier that hands the buffer to the readers.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %2" ::"v"(voff), "s"(lds_addr), "s"(base)
               : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_address(const void* p) {
  typedef const __attribute__((address_space(3))) char* lds_ptr;
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr)p));
}

// Barrier without the memory fence that __syncthreads() adds: the fence would
// also wait for the in-flight direct-to-LDS gathers of the next tiles.
__device__ __forceinline__ void sync_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }


__global__ __launch_bounds__(MLA_THREADS, 1) void sparse_mla_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ idx,
    uint16_t* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o, float* __restrict__ part_lse,
    int64_t R, int64_t Tq, int64_t N, int K, int splits, int keys_per_split, float scale_log2) {
  __shared__ __align__(16) uint16_t kvs[NBUF][NT * MD];  // latent tiles, chunk-major (see above)
  __shared__ __align__(16) int32_t vflag[NBUF][NT];      // row valid flags per buffer
  __shared__ __align__(16) int32_t sidx[MAX_SPLIT_KEYS];  // this split's index list
  __shared__ __align__(16) uint16_t ps[MH * PP];
  __shared__ float alpha_s[MH];
  __shared__ float m_s[MH], l_s[MH];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: lives in a scalar register
  const int half = lane >> 5, col = lane & 31;   // 32x32 operand/result roles
  const int g16 = lane >> 4, c16 = lane & 15;    // 16x16 operand/result roles

  // Work item.  When the rows split evenly over the 8 XCDs (workgroups are
  // dealt round-robin to them), all splits of a query run on one XCD so its
  // 144 KiB query block is fetched once into that XCD's L2.
  int64_t r;
  int sp;
  {
    const int64_t i = blockIdx.x;
    if (splits > 1 && (R & 7) == 0) {
      const int64_t x = i & 7, j = i >> 3;
      r = x + 8 * (j / splits);
      sp = (int)(j % splits);
    } else {
      r = i / splits;
      sp = (int)(i % splits);
    }
  }
  const int64_t b = r / Tq;
  const int kb = sp * keys_per_split;
  const int ke = min(K, kb + keys_per_split);
  const int nkeys = max(ke - kb, 0);
  const int ntiles = (nkeys + NT - 1) / NT;

  // Queries of heads 16*wave + c16, channels 32*s + 8*g16 + [0, 8).
  bf16x8 qf[MD / 32];
  {
    const uint16_t* qp = q + (r * MH + 16 * wave + c16) * (int64_t)MD + 8 * g16;
#pragma unroll
    for (int s = 0; s < MD / 32; ++s) qf[s] = load_bf16x8(qp + 32 * s);
  }
  {
    const int32_t* ip = idx + r * K + kb;
    for (int j = tid; j < ntiles * NT; j += MLA_THREADS) sidx[j] = j < nkeys ? ip[j] : -1;
  }
  f32x16 o[2][4];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) o[mb][nb] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const uint16_t* kvb = kv + b * N * (int64_t)MD;
  // Queries and indices are in place; from here on the only memory loads in
  // flight are the gathers below, which the compiler does not see.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // Gather of tile `it`: instruction u of wave w fills slots [64*ii, 64*ii+64)
  // of the tile, ii = w + 8u (36 instructions in all): chunk columns 2*ii and
  // 2*ii+1, rows 0..31.  Lane l always fetches row l%32, chunk 2*ii + l/32.
  // Waves 0-3 issue 5 instructions per tile, waves 4-7 issue 4.
  constexpr int GU = (TILE_CHUNKS / 64 + MLA_WAVES - 1) / MLA_WAVES;  // 5
  // Slot 32*p + s of the tile holds row s ^ 4*(p & 3); for this wave's
  // instructions p = 2*ii + lane/32 with ii = wave + 8u, so p & 3 is fixed.
  const int grow = (lane & 31) ^ (4 * ((2 * (wave & 1) + (lane >> 5)) & 3));
  // byte address of chunk 2*ii + lane/32 of row v: kvw + [v*1152 + 16*(lane/32)] + 256*u,
  // with kvw = this sequence's cache + 32*wave (scalar) and ii = wave + 8u
  const uint8_t* kvw = reinterpret_cast<const uint8_t*>(kvb) + 32 * wave;
  auto gather = [&](int it) {
    const int buf = it % NBUF;
    const int32_t v = sidx[it * NT + grow];
    const bool ok = v >= 0 && (int64_t)v < N;
    const uint32_t voff = (uint32_t)(ok ? v : 0) * (uint32_t)(MD * 2) + 16u * (uint32_t)(lane >> 5);
    const uint32_t lds0 = lds_address(&kvs[buf][512 * wave]);
    dma16(kvw, voff, lds0);
    dma16(kvw + 256, voff, lds0 + 8192);
    dma16(kvw + 512, voff, lds0 + 16384);
    dma16(kvw + 768, voff, lds0 + 24576);
    if (wave + 4 * MLA_WAVES < TILE_CHUNKS / 64) dma16(kvw + 1024, voff, lds0 + 32768);
    if (wave == 0 && lane < 32) vflag[buf][grow] = ok;  // wave 0, lanes 0..31: row == lane
  };
  // Wait until this wave's gathers of all but the most recently issued tile
  // are complete (vmcnt counts this wave's loads, oldest first).
  auto wait_all_but_newest = [&](bool newest_in_flight) {
    if (!newest_in_flight) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else if (wave < TILE_CHUNKS / 64 - (GU - 1) * MLA_WAVES) asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  };
  static_assert(GU == 5 && TILE_CHUNKS / 64 - (GU - 1) * MLA_WAVES == 4, "per-wave gather counts");

  // QK^T operand: key row 16*kb2 + c16, chunk p = 4*s + g16 (p & 3 == g16)
  //   -> slot 32*p + 16*kb2 + (c16 ^ 4*g16)   [bf16 element = 8 * slot]
  const int abase = 256 * g16 + 8 * (c16 ^ (4 * g16));
  // PV operand, read rd (keys 4rd..4rd+3 of this lane half) of block (ks, mb):
  // 16-lane group G = lane/16, source lane j = lane%16 addresses key
  // 16*ks + 8*half + 4*rd + j/4, value columns 64*wave + 32*mb + 16*(G&1) + 4*(j&3) + [0,4),
  // i.e. chunk p = 8*wave + 4*mb + 2*(G&1) + (j&3)/2, byte 8*(j&1) of it.
  int vbase[2];
  {
    const int G = lane >> 4, j = lane & 15, b = (j & 3) >> 1;
    const int pl = 2 * (G & 1) + b;  // chunk offset within the 4-chunk group (p & 3)
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
      const int key = 8 * half + 4 * rd + (j >> 2);              // + 16*ks (compile-time)
      vbase[rd] = 256 * (8 * wave + pl) + 8 * (key ^ (4 * pl)) + 4 * (j & 1);
    }
  }

  if (ntiles > 0) gather(0);
  if (ntiles > 1) gather(1);
  wait_all_but_newest(ntiles > 1);
  sync_lds();
  for (int it = 0; it < ntiles; ++it) {
    const uint16_t* cur = kvs[it % NBUF];
    const int32_t* vcur = vflag[it % NBUF];
    if (it + 2 < ntiles) gather(it + 2);

    // S^T[key][head] for this wave's 16 heads, keys in two blocks of 16.
    f32x4 sacc[2] = {f32x4{}, f32x4{}};
#pragma unroll
    for (int s = 0; s < MD / 32; ++s) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(cur + abase + 1024 * s + 128 * kb2);  // p = 4s + g16
        sacc[kb2] = mfma16x16x32(av, qf[s], sacc[kb2]);
      }
      if ((s & 1) == 1) __builtin_amdgcn_sched_barrier(0);
    }

    // Online softmax; this lane holds head 16*wave+c16, keys 16*kb2 + 4*g16 + i.
    float x[8];
    float mt = -INFINITY;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      const int4 vf = *reinterpret_cast<const int4*>(&vcur[16 * kb2 + 4 * g16]);
      const int fl[4] = {vf.x, vf.y, vf.z, vf.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[4 * kb2 + i] = fl[i] ? sacc[kb2][i] * scale_log2 : -INFINITY;
        mt = fmaxf(mt, x[4 * kb2 + i]);
      }
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    float alpha = 1.f, lsum = 0.f;
    if (m_new == -INFINITY) {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = 0.f;
    } else {
      alpha = exp2f(m_run - m_new);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        x[i] = exp2f(x[i] - m_new);
        lsum += x[i];
      }
    }
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    l_run = l_run * alpha + lsum;
    m_run = m_new;
    {
      uint16_t* pp = &ps[(16 * wave + c16) * PP + 4 * g16];
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        u32x2 pk;
        pk.x = float_to_bf16_bits(x[4 * kb2 + 0]) | (float_to_bf16_bits(x[4 * kb2 + 1]) << 16);
        pk.y = float_to_bf16_bits(x[4 * kb2 + 2]) | (float_to_bf16_bits(x[4 * kb2 + 3]) << 16);
        *reinterpret_cast<u32x2*>(pp + 16 * kb2) = pk;
      }
      if (g16 == 0) alpha_s[16 * wave + c16] = alpha;
    }
    sync_lds();

    // O^T[dv][head] += V^T . P^T for dv in [64*wave, 64*wave+64), all heads.
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const float an = alpha_s[32 * nb + col];
      if (__any(an != 1.f)) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) o[mb][nb] *= an;
      }
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 av[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        // 16*ks rows and 4*mb chunks: slot += 16*ks + 128*mb (the XOR term is unchanged)
        const s16x4 lo = lds_read_tr16(cur + vbase[0] + 1024 * mb + 128 * ks);
        const s16x4 hi = lds_read_tr16(cur + vbase[1] + 1024 * mb + 128 * ks);
        av[mb] = __builtin_bit_cast(bf16x8, s16x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w});
      }
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const bf16x8 pb = *reinterpret_cast<const bf16x8*>(&ps[(32 * nb + col) * PP + 16 * ks + 8 * half]);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) o[mb][nb] = mfma32x32x16(av[mb], pb, o[mb][nb]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // tile it+1 must have landed; tile it+2 may stay in flight
    wait_all_but_newest(it + 2 < ntiles);
    sync_lds();
  }

  if (g16 == 0) {
    l_s[16 * wave + c16] = l_run;
    m_s[16 * wave + c16] = m_run;
  }
  sync_lds();
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int h = 32 * nb + col;
    const float l = l_s[h], m = m_s[h];
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const float lse2 = l > 0.f ? m + log2f(l) : -INFINITY;
    if (splits == 1) {
      uint16_t* op = out + (r * MH + h) * (int64_t)MDV + 64 * wave + 4 * half;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const f32x16& v = o[mb][nb];
          u32x2 pk;
          pk.x = float_to_bf16_bits(v[4 * a + 0] * inv) | (float_to_bf16_bits(v[4 * a + 1] * inv) << 16);
          pk.y = float_to_bf16_bits(v[4 * a + 2] * inv) | (float_to_bf16_bits(v[4 * a + 3] * inv) << 16);
          *reinterpret_cast<u32x2*>(op + 32 * mb + 8 * a) = pk;
        }
      if (lse != nullptr && wave == 0 && half == 0) lse[r * MH + h] = lse2 * LN2;
    } else {
      float* po = part_o + (((int64_t)sp * R + r) * MH + h) * MDV + 64 * wave + 4 * half;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const f32x16& v = o[mb][nb];
          f32x4 st = {v[4 * a + 0] * inv, v[4 * a + 1] * inv, v[4 * a + 2] * inv, v[4 * a + 3] * inv};
          *reinterpret_cast<f32x4*>(po + 32 * mb + 8 * a) = st;
        }
      if (wave == 0 && half == 0) part_lse[((int64_t)sp * R + r) * MH + h] = lse2;
    }
  }
}

// Merge the split partials of one (query, head): weights 2^(lse_s - lse_max).
__global__ __launch_bounds__(128) void mla_combine_kernel(const float* __restrict__ part_o,
                                                         const float* __restrict__ part_lse,
                                                         uint16_t* __restrict__ out, float* __restrict__ lse,
                                                         int64_t R, int splits) {
  const int64_t rh = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t stride = R * MH;
  float M = -INFINITY;
  for (int s = 0; s < splits; ++s) M = fmaxf(M, part_lse[s * stride + rh]);
  float den = 0.f;
  if (M != -INFINITY)
    for (int s = 0; s < splits; ++s) den += exp2f(part_lse[s * stride + rh] - M);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (M != -INFINITY) {
    const float inv = 1.f / den;
    for (int s = 0; s < splits; ++s) {
      const float wgt = exp2f(part_lse[s * stride + rh] - M) * inv;
      if (wgt != 0.f) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(part_o + (s * stride + rh) * MDV + 4 * tid);
        acc += wgt * v;
      }
    }
  }
  u32x2 pk;
  pk.x = float_to_bf16_bits(acc.x) | (float_to_bf16_bits(acc.y) << 16);
  pk.y = float_to_bf16_bits(acc.z) | (float_to_bf16_bits(acc.w) << 16);
  *reinterpret_cast<u32x2*>(out + rh * MDV + 4 * tid) = pk;
  if (lse != nullptr && tid == 0) lse[rh] = M == -INFINITY ? -INFINITY : (M + log2f(den)) * LN2;
}

// Generic fp32 kernel for small problems: one wave per (query, head), keys in
// index order with an online softmax.
__global__ __launch_bounds__(64) void sparse_mla_f32_kernel(const float* __restrict__ q,
                                                            const float* __restrict__ kv,
                                                            const int32_t* __restrict__ idx, float* __restrict__ out,
                                                            float* __restrict__ lse, int64_t Tq, int64_t N, int H,
                                                            int D, int DV, int K, float scale) {
  const int64_t rh = blockIdx.x;
  const int64_t r = rh / H, b = r / Tq;
  const int lane = threadIdx.x;
  float qr[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    const int d = lane + 64 * c;
    qr[c] = d < D ? q[rh * D + d] : 0.f;
  }
  float o[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) o[c] = 0.f;
  float m = -INFINITY, l = 0.f;
  const int32_t* ip = idx + r * K;
  for (int j = 0; j < K; ++j) {
    const int32_t v = ip[j];
    if (v < 0 || (int64_t)v >= N) continue;
    const float* row = kv + (b * N + v) * D;
    float dot = 0.f;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const int d = lane + 64 * c;
      if (d < D) dot = fmaf(qr[c], row[d], dot);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) dot += __shfl_xor(dot, off);
    const float xl = dot * scale;
    const float mn = fmaxf(m, xl);
    const float al = expf(m - mn);
    const float p = expf(xl - mn);
    l = l * al + p;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int dv = lane + 64 * c;
      if (dv < DV) o[c] = fmaf(p, row[dv], o[c] * al);
    }
    m = mn;
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int dv = lane + 64 * c;
    if (dv < DV) out[rh * DV + dv] = o[c] * inv;
  }
  if (lse != nullptr && lane == 0) lse[rh] = l > 0.f ? m + logf(l) : -INFINITY;
}

}  // namespace

int mla_num_splits(int64_t rows, int K) {
  const int tiles = (K + NT - 1) / NT;
  int64_t want = (256 + rows - 1) / rows;  // about one workgroup per compute unit
  if (want > 32) want = 32;
  if (want > tiles) want = tiles;
  // one workgroup stages at most MAX_SPLIT_KEYS indices
  const int64_t need = (K + MAX_SPLIT_KEYS - 1) / MAX_SPLIT_KEYS;
  if (want < need) want = need;
  return want < 1 ? 1 : (int)want;
}

static int mla_keys_per_split(int K, int splits) {
  const int tiles = (K + NT - 1) / NT;
  return ((tiles + splits - 1) / splits) * NT;
}

size_t mla_workspace_bytes(int64_t rows, int H, int DV, int K, int is_bf16) {
  if (!is_bf16) return 0;
  const int s = mla_num_splits(rows, K);
  if (s <= 1) return 0;
  return (size_t)s * rows * H * DV * sizeof(float) + (size_t)s * rows * H * sizeof(float);
}

hipError_t launch_sparse_mla_bf16(const uint16_t* q, const uint16_t* kv, const int32_t* idx, uint16_t* out,
                                  float* lse, int64_t B, int64_t Tq, int64_t N, int K, float scale,
                                  void* workspace, hipStream_t stream) {
  const int64_t R = B * Tq;
  const int splits = mla_num_splits(R, K);
  const int kps = mla_keys_per_split(K, splits);
  float* part_o = nullptr;
  float* part_lse = nullptr;
  if (splits > 1) {
    part_o = static_cast<float*>(workspace);
    part_lse = part_o + (size_t)splits * R * MH * MDV;
  }
  hipLaunchKernelGGL(sparse_mla_bf16_kernel, dim3((unsigned)(R * splits)), dim3(MLA_THREADS), 0, stream, q, kv,
                     idx, out, lse, part_o, part_lse, R, Tq, N, K, splits, kps, scale * LOG2E);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  hipLaunchKernelGGL(mla_combine_kernel, dim3((unsigned)(R * MH)), dim3(128), 0, stream, part_o, part_lse, out, lse,
                     R, splits);
  return hipGetLastError();
}

hipError_t launch_sparse_mla_f32(const float* q, const float* kv, const int32_t* idx, float* out, float* lse,
                                 int64_t B, int64_t Tq, int64_t N, int H, int D, int DV, int K, float scale,
                                 hipStream_t stream) {
  hipLaunchKernelGGL(sparse_mla_f32_kernel, dim3((unsigned)(B * Tq * H)), dim3(64), 0, stream, q, kv, idx, out,
                     lse, Tq, N, H, D, DV, K, scale);
  return hipGetLastError();
}

}  // namespace dsa

// Sparse MLA (absorbed latent form) over the selected keys, on gfx950.
//
// For each query (b,t) and head h, over the selected rows S of the latent
// cache: logits l_j = scale * q[h] . kv[j] (576 wide), out[h] = softmax(l) .
// kv[S, 0:512], lse[h] = ln sum exp(l).  (DeepSeek-V3.2 model documentation,
// section "DeepSeek Sparse Attention (DSA)": the main MLA attention runs over
// the selected tokens only; DeepseekV32Config section: 128 heads,
// kv_lora_rank 512 + qk_rope_head_dim 64.)
//
// bf16 kernel: one workgroup (4 waves, one per SIMD, 512 registers each) per
// (query, split of the index list, at most 2048 indices, staged once in
// LDS).  Each step gathers 32 selected latent rows (1152 B each) straight into
// LDS with direct-to-LDS 16-byte loads (no staging registers) into one of
// three tile buffers, so two tiles' gathers (72 KiB) are in flight during the
// current tile's math, and shares the rows across all 128 heads:
//   * S^T = KV_tile . Q^T on 32x32x16 MFMAs: wave w owns heads [32w, 32w+32)
//     and keeps their queries in registers (36 k-steps of 16 channels);
//   * softmax in fp32 with exp2 on log2e-prescaled logits against a fixed
//     per-head reference: the first non-empty tile's maximum.  The
//     accumulators are therefore never rescaled (that would need all 256 of
//     them in vector registers at once); should a later logit exceed the
//     reference by more than 64 (log2 units), the split is recomputed with
//     the true maximum as reference, so exp2 stays far below the fp32/bf16
//     range in every case.  A lane owns one head (16 of its keys, the other
//     16 in lane j^32);
//   * P (bf16) goes through LDS, then O^T = V^T . P^T on 32x32x16 MFMAs:
//     wave w owns value columns [128w, 128w+128) for all 128 heads (256 fp32
//     accumulators per lane), so every V element is read from LDS once per
//     tile.
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
// (bf16) and its log2-sum-exp (fp32) to the workspace and a combine kernel
// merges them in fp32.
#include "device_common.h"
#include "launch.h"

namespace dsa {
namespace {

constexpr int MH = 128, MD = 576, MDV = 512, NT = 32;
constexpr int ROW_CHUNKS = MD / 8;          // 72 chunks of 16 B per latent row
constexpr int TILE_CHUNKS = NT * ROW_CHUNKS; // 2304
constexpr int PP = NT + 8;                   // bf16 per LDS probability row
constexpr int MLA_WAVES = 4;
constexpr int NBUF = 3;                      // latent tile buffers (two gathers in flight)
constexpr int SLOOK = 6;                     // QK^T key-operand reads in flight
constexpr int PVLOOK = 2;                    // PV value-operand reads in flight
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

// QK^T MFMAs with their accumulators in ordinary vector registers.  The
// 256 output accumulators of a wave fill the accumulation registers, so the
// logits must live in vector registers; builtin MFMAs would place them in
// accumulation registers and force copies.  The compiler does not look into
// these statements, so each one carries the wait states it needs: two before
// the MFMA (a vector write of an operand just before it), and, after the last
// MFMA of the chain, more than the 19 that any read of an MFMA result needs.
// Between MFMAs of one chain (source C = destination, same shape) the
// hardware forwards the accumulator and needs none.
__device__ __forceinline__ f32x16 mfma_s_first(bf16x8 a, bf16x8 b) {
  f32x16 c;
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
  return c;
}
__device__ __forceinline__ void mfma_s(f32x16& c, bf16x8 a, bf16x8 b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_s_last2(f32x16& c0, bf16x8 a0, bf16x8 b0, f32x16& c1, bf16x8 a1, bf16x8 b1) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %2, %3, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %1, %4, %5, %1\n\t"
      "s_nop 7\n\ts_nop 7\n\ts_nop 7"
      : "+v"(c0), "+v"(c1)
      : "v"(a0), "v"(b0), "v"(a1), "v"(b1));
}

// Barrier without the memory fence that __syncthreads() adds: the fence would
// also wait for the in-flight direct-to-LDS gathers of the next tiles.
__device__ __forceinline__ void sync_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }


__global__ __launch_bounds__(MLA_THREADS, 1) void sparse_mla_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ idx,
    uint16_t* __restrict__ out, float* __restrict__ lse, uint16_t* __restrict__ part_o, float* __restrict__ part_lse,
    int64_t R, int64_t Tq, int64_t N, int K, int splits, int keys_per_split, float scale_log2) {
  __shared__ __align__(16) uint16_t kvs[NBUF][NT * MD];  // latent tiles, chunk-major (see above)
  __shared__ __align__(16) int32_t vflag[NBUF][NT];      // row valid flags per buffer
  __shared__ int32_t tfull[NBUF];                          // 1 if every row of the buffer is valid
  __shared__ __align__(16) int32_t sidx[MAX_SPLIT_KEYS];  // this split's index list
  __shared__ __align__(16) uint16_t ps[MH * PP];
  __shared__ float m_s[MH], l_s[MH];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: lives in a scalar register
  const int half = lane >> 5, col = lane & 31;

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

  // Prologue: this split's indices into LDS, then the gathers of the first
  // two tiles, then the queries, so the query loads overlap the gathers.
  {
    const int32_t* ip = idx + r * K + kb;
    for (int j = tid; j < ntiles * NT; j += MLA_THREADS) sidx[j] = j < nkeys ? ip[j] : -1;
  }
  f32x16 o[4][4];
  float m_ref = -INFINITY;  // exponent reference of this lane's head (log2 units)
  float m_max = -INFINITY;  // largest logit seen
  float l_run = 0.f;
  const uint16_t* kvb = kv + b * N * (int64_t)MD;
  __syncthreads();

  // Gather of tile `it`: instruction u of wave w fills slots [64*ii, 64*ii+64)
  // of the tile, ii = w + 4u (36 instructions, 9 per wave): chunk columns 2*ii
  // and 2*ii+1.  Slot 32*p + s holds row s ^ 4*(p & 3); for this wave's
  // instructions p = 2*ii + lane/32 and p & 3 is fixed.
  constexpr int GU = TILE_CHUNKS / 64 / MLA_WAVES;  // 9
  static_assert(GU * 64 * MLA_WAVES == TILE_CHUNKS && GU == 9, "gather instructions per wave");
  const int grow = (lane & 31) ^ (4 * ((2 * (wave & 1) + (lane >> 5)) & 3));
  // byte address of chunk 2*ii + lane/32 of row v: kvw + [v*1152 + 16*(lane/32)] + 128*u,
  // with kvw = this sequence's cache + 32*wave (scalar) and ii = wave + 4u
  const uint8_t* kvw = reinterpret_cast<const uint8_t*>(kvb) + 32 * wave;
  auto gather = [&](int it) {
    const int buf = it % NBUF;
    const int32_t v = sidx[it * NT + grow];
    const bool ok = v >= 0 && (int64_t)v < N;
    const uint32_t voff = (uint32_t)(ok ? v : 0) * (uint32_t)(MD * 2) + 16u * (uint32_t)(lane >> 5);
    const uint32_t lds0 = lds_address(&kvs[buf][512 * wave]);
#pragma unroll
    for (int u = 0; u < GU; ++u) dma16(kvw + 128 * u, voff, lds0 + 4096 * u);
    if (wave == 0) {
      if (lane < 32) vflag[buf][grow] = ok;  // lanes 0..31: row == lane
      const bool full = __ballot(ok) == ~0ull;  // lanes 32..63 cover the 32 rows again
      if (lane == 0) tfull[buf] = full;
    }
  };
  // Wait until this wave's gathers of all but the most recently issued tile
  // are complete (vmcnt counts this wave's loads, oldest first).
  auto wait_all_but_newest = [&](bool newest_in_flight) {
    if (newest_in_flight) asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };

  // QK^T operand (A): key row col, channels 16*s + 8*half + e, i.e. chunk
  // p = 2s + half, p & 3 = 2*(s & 1) + half  ->  slot 32p + (col ^ 4*(p & 3)).
  int abase[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) abase[par] = 256 * half + 8 * (col ^ (4 * ((2 * par + half) & 3)));
  // PV operand, read rd (keys 4rd..4rd+3 of this lane half) of block (ks, mb):
  // 16-lane group G = lane/16, source lane j = lane%16 addresses key
  // 16*ks + 8*half + 4*rd + j/4, value columns 128*wave + 32*mb + 16*(G&1) + 4*(j&3) + [0,4),
  // i.e. chunk p = 16*wave + 4*mb + 2*(G&1) + (j&3)/2, byte 8*(j&1) of it.
  int vbase[2];
  {
    const int G = lane >> 4, j = lane & 15, bq = (j & 3) >> 1;
    const int pl = 2 * (G & 1) + bq;  // p & 3
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
      const int key = 8 * half + 4 * rd + (j >> 2);  // + 16*ks (compile-time)
      vbase[rd] = 256 * (16 * wave + pl) + 8 * (key ^ (4 * pl)) + 4 * (j & 1);
    }
  }

  if (ntiles > 0) gather(0);
  if (ntiles > 1) gather(1);
  // Queries of heads 32*wave + col, channels 16*s + 8*half + [0, 8).
  bf16x8 qf[MD / 16];
  {
    const uint16_t* qp = q + (r * MH + 32 * wave + col) * (int64_t)MD + 8 * half;
#pragma unroll
    for (int s = 0; s < MD / 16; ++s) qf[s] = load_bf16x8(qp + 16 * s);
  }

  for (int pass = 0; pass < 2; ++pass) {
  if (pass == 1) {
    // a logit ran more than 64 above its reference in some head: redo the
    // split with the true maximum as reference (never the case for ordinary data)
    m_ref = m_max;
    l_run = 0.f;
    if (ntiles > 0) gather(0);
    if (ntiles > 1) gather(1);
  }
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) o[mb][nb] = f32x16{};
  bool overflow = false;
  // queries and tiles 0 (and 1) in place; the compiler now sees no load in flight
  __builtin_amdgcn_s_waitcnt(0);
  sync_lds();
  for (int it = 0; it < ntiles; ++it) {
    const uint16_t* cur = kvs[it % NBUF];
    const int32_t* vcur = vflag[it % NBUF];
    if (it + 2 < ntiles) gather(it + 2);

    // S^T[key][head] for this wave's 32 heads: two independent accumulation
    // chains (even and odd k-steps) so that consecutive MFMAs do not wait for
    // each other.
    // The key operands stream through a ring of SLOOK registers, each read
    // issued SLOOK k-steps ahead of its MFMA; the scheduling barriers keep the
    // compiler from collapsing the ring.
    f32x16 sacc;
    {
      constexpr int KS = MD / 16;
      auto aop = [&](int s) { return *reinterpret_cast<const bf16x8*>(cur + abase[s & 1] + 512 * s); };
      bf16x8 ring[SLOOK];
#pragma unroll
      for (int s = 0; s < SLOOK; ++s) ring[s] = aop(s);
      f32x16 s0, s1;
#pragma unroll
      for (int s = 0; s < KS; s += 2) {
        const bf16x8 a0 = ring[s % SLOOK], a1 = ring[(s + 1) % SLOOK];
        if (s + SLOOK < KS) ring[s % SLOOK] = aop(s + SLOOK);
        if (s + 1 + SLOOK < KS) ring[(s + 1) % SLOOK] = aop(s + 1 + SLOOK);
        if (s == 0) {
          s0 = mfma_s_first(a0, qf[0]);
          s1 = mfma_s_first(a1, qf[1]);
        } else if (s + 2 < KS) {
          mfma_s(s0, a0, qf[s]);
          mfma_s(s1, a1, qf[s + 1]);
        } else {
          mfma_s_last2(s0, a0, qf[s], s1, a1, qf[s + 1]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      sacc = s0 + s1;
    }

    // Online softmax in log2 units.  This lane holds head 32*wave+col for keys
    // mfma_row(i, half); lane j^32 holds the other 16 keys of the tile.  The
    // scale is positive, so the scaled maximum is the maximum of the scaled
    // logits, and each weight is one fused multiply-add and one exp2.
    if (!__builtin_amdgcn_readfirstlane(tfull[it % NBUF])) {
      // some row of this tile is masked: its logit is -inf (weight 0)
      const int32_t* vcur = vflag[it % NBUF];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int4 vf = *reinterpret_cast<const int4*>(&vcur[8 * a + 4 * half]);
        const int fl[4] = {vf.x, vf.y, vf.z, vf.w};
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (!fl[c]) sacc[4 * a + c] = -INFINITY;
      }
    }
    float mh = sacc[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mh = fmaxf(mh, sacc[i]);
    const float mt = max_halves(mh * scale_log2);  // this head's largest scaled logit in the tile
    m_max = fmaxf(m_max, mt);
    if (m_ref == -INFINITY) m_ref = mt;  // nothing accumulated yet: start the reference here
    overflow |= mt > m_ref + 64.f;
    float x[16];
    float lsum = 0.f;
    if (m_ref == -INFINITY) {
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = 0.f;
    } else {
      // arguments are at most 64 here (else the split is redone); exp2(-inf) = 0
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        x[i] = __builtin_amdgcn_exp2f(fmaf(sacc[i], scale_log2, -m_ref));
        lsum += x[i];
      }
    }
    l_run += lsum;  // this half's keys; the halves are added at the end
    {
      uint16_t* pp = &ps[(32 * wave + col) * PP + 4 * half];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        u32x2 pk;
        pk.x = pack_bf16x2(x[4 * a + 0], x[4 * a + 1]);
        pk.y = pack_bf16x2(x[4 * a + 2], x[4 * a + 3]);
        *reinterpret_cast<u32x2*>(pp + 8 * a) = pk;
      }
    }
    sync_lds();

    // O^T[dv][head] += V^T . P^T for dv in [128*wave, 128*wave+128), all heads.
    // Eight steps (ks, mb); the value operand of step st+PVLOOK is read
    // while step st runs its four MFMAs.
    {
      bf16x8 pb[2][4];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          pb[ks][nb] = *reinterpret_cast<const bf16x8*>(&ps[(32 * nb + col) * PP + 16 * ks + 8 * half]);
      auto vop = [&](int st) {
        // 16*ks rows and 4*mb chunks: slot += 16*ks + 128*mb (the XOR term is unchanged)
        const int ks = st >> 2, mb = st & 3;
        const s16x4 lo = lds_read_tr16(cur + vbase[0] + 1024 * mb + 128 * ks);
        const s16x4 hi = lds_read_tr16(cur + vbase[1] + 1024 * mb + 128 * ks);
        return __builtin_bit_cast(bf16x8, s16x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w});
      };
      bf16x8 vring[PVLOOK];
#pragma unroll
      for (int st = 0; st < PVLOOK; ++st) vring[st] = vop(st);
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const int ks = st >> 2, mb = st & 3;
        const bf16x8 av = vring[st % PVLOOK];
        if (st + PVLOOK < 8) vring[st % PVLOOK] = vop(st + PVLOOK);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) o[mb][nb] = mfma32x32x16(av, pb[ks][nb], o[mb][nb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // tile it+1 must have landed; tile it+2 may stay in flight
    wait_all_but_newest(it + 2 < ntiles);
    sync_lds();
  }
  if (!__syncthreads_or(overflow)) break;
  }

  l_run = sum_halves(l_run);
  if (half == 0) {
    l_s[32 * wave + col] = l_run;
    m_s[32 * wave + col] = m_ref;
  }
  sync_lds();
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int h = 32 * nb + col;
    const float l = l_s[h], m = m_s[h];
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const float lse2 = l > 0.f ? m + log2f(l) : -INFINITY;
    // one accumulator block at a time (keeps the vector registers this needs small)
    if (splits == 1) {
      uint16_t* op = out + (r * MH + h) * (int64_t)MDV + 128 * wave + 4 * half;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const f32x16& v = o[mb][nb];
          u32x2 pk;
          pk.x = pack_bf16x2(v[4 * a + 0] * inv, v[4 * a + 1] * inv);
          pk.y = pack_bf16x2(v[4 * a + 2] * inv, v[4 * a + 3] * inv);
          *reinterpret_cast<u32x2*>(op + 32 * mb + 8 * a) = pk;
        }
      }
      if (lse != nullptr && wave == 0 && half == 0) lse[r * MH + h] = lse2 * LN2;
    } else {
      uint16_t* po = part_o + (((int64_t)sp * R + r) * MH + h) * MDV + 128 * wave + 4 * half;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const f32x16& v = o[mb][nb];
          u32x2 pk;
          pk.x = pack_bf16x2(v[4 * a + 0] * inv, v[4 * a + 1] * inv);
          pk.y = pack_bf16x2(v[4 * a + 2] * inv, v[4 * a + 3] * inv);
          *reinterpret_cast<u32x2*>(po + 32 * mb + 8 * a) = pk;
        }
      }
      if (wave == 0 && half == 0) part_lse[((int64_t)sp * R + r) * MH + h] = lse2;
    }
  }
}

// Merge the split partials of one (query, head): weights 2^(lse_s - lse_max).
__global__ __launch_bounds__(128) void mla_combine_kernel(const uint16_t* __restrict__ part_o,
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
        const u32x2 pk = *reinterpret_cast<const u32x2*>(part_o + (s * stride + rh) * MDV + 4 * tid);
        const f32x4 v = {bf16_bits_to_float(pk.x & 0xffffu), bf16_bits_to_float(pk.x >> 16),
                         bf16_bits_to_float(pk.y & 0xffffu), bf16_bits_to_float(pk.y >> 16)};
        acc += wgt * v;
      }
    }
  }
  u32x2 pk;
  pk.x = pack_bf16x2(acc.x, acc.y);
  pk.y = pack_bf16x2(acc.z, acc.w);
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
  // bf16 normalised partial outputs, then fp32 log2-sum-exps
  return (size_t)s * rows * H * DV * sizeof(uint16_t) + (size_t)s * rows * H * sizeof(float);
}

hipError_t launch_sparse_mla_bf16(const uint16_t* q, const uint16_t* kv, const int32_t* idx, uint16_t* out,
                                  float* lse, int64_t B, int64_t Tq, int64_t N, int K, float scale,
                                  void* workspace, hipStream_t stream) {
  const int64_t R = B * Tq;
  const int splits = mla_num_splits(R, K);
  const int kps = mla_keys_per_split(K, splits);
  uint16_t* part_o = nullptr;
  float* part_lse = nullptr;
  if (splits > 1) {
    part_o = static_cast<uint16_t*>(workspace);
    part_lse = reinterpret_cast<float*>(part_o + (size_t)splits * R * MH * MDV);
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

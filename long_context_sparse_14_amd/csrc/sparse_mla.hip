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
// LDS tile layout: row r of the tile (0..31) is 72 chunks of 16 bytes; chunk c
// sits at slot 64*(9*(r/8) + c/8) + 8*(r%8) + ((c%8) ^ f(r)), with
// f(r) = 2*((r>>1)&3) + ((r>>3)&1).  One gather instruction therefore fills a
// 1 KiB block of 64 slots from 8 whole 128-byte cache lines (8 rows), and the
// XOR term spreads both operand reads below over all banks.  Every operand
// read is a per-lane base plus a compile-time offset.  The PV operand (eight
// keys of one value column per lane) comes from the gfx950 transposing LDS
// read ds_read_b64_tr_b16: within each 16-lane group, lane i receives element
// (i & 3) of the 8 bytes addressed by lane 4c + (i >> 2), c = 0..3 -- so lanes
// that address four consecutive value columns of four consecutive keys hand
// every lane four keys of its own column.
// With more than one split, each split writes its normalised partial output
// (bf16) and its log2-sum-exp (fp32) to the workspace and a combine kernel
// merges them in fp32.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace dsa {
namespace {

constexpr int MH = 128, MD = 576, MDV = 512, NT = 32;
constexpr int ROW_CHUNKS = MD / 8;          // 72 chunks of 16 B per latent row
constexpr int TILE_CHUNKS = NT * ROW_CHUNKS; // 2304
constexpr int PP = NT + 8;                   // bf16 per LDS probability row
constexpr int MLA_WAVES = 4;
constexpr int NBUF = 3;                      // latent tile buffers
constexpr int SLOOK = 4;                     // QK^T key-operand reads in flight
constexpr int PVLOOK = 2;                    // PV value-operand reads in flight
constexpr int MAX_SPLIT_KEYS = 2048;         // indices handled by one workgroup
constexpr int MLA_THREADS = MLA_WAVES * 64;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

// XOR swizzle of tile row r (see the layout note above).
__device__ __forceinline__ int row_swizzle(int r) { return 2 * ((r >> 1) & 3) + ((r >> 3) & 1); }

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
__device__ __forceinline__ void mfma_s_last(f32x16& c, bf16x8 a, bf16x8 b) {
  asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\t"
      "s_nop 7\n\ts_nop 7\n\ts_nop 7"
      : "+v"(c)
      : "v"(a), "v"(b));
}

// Barrier without the memory fence that __syncthreads() adds: the fence would
// also wait for the in-flight direct-to-LDS gathers of the next tiles.
__device__ __forceinline__ void sync_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }


// ADDR64: the gathered rows' byte offsets within the sequence need 64 bits
// (a latent cache of 4 GiB or more, e.g. a large paged pool); the gathers then
// take full per-lane addresses.
template <bool ADDR64>
__global__ __launch_bounds__(MLA_THREADS, 1) void sparse_mla_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ idx,
    uint16_t* __restrict__ out, float* __restrict__ lse, uint16_t* __restrict__ part_o, float* __restrict__ part_lse,
    int64_t R, int64_t Tq, int64_t N, int K, int splits, int keys_per_split, float scale_log2) {
  __shared__ __align__(16) uint16_t kvs[NBUF][NT * MD];  // latent tiles, chunk-major (see above)
  __shared__ __align__(16) int32_t vflag[NBUF][NT];      // row valid flags per buffer
  __shared__ __align__(16) int32_t tfull[NBUF][MLA_WAVES]; // per wave: 1 if its 8 rows of the buffer are valid
  __shared__ __align__(16) int32_t sidx[MAX_SPLIT_KEYS];  // this split's index list
  __shared__ __align__(16) uint16_t ps[2][MH * PP];       // bf16 P of two consecutive tiles
  __shared__ float m_s[MH], l_s[MH];
  __shared__ __align__(16) int32_t ovf_s[MLA_WAVES];

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

  // Prologue: this split's index loads, then the query loads (issued while
  // the indices are in flight), then, once the indices are in LDS, the
  // gathers of the first two tiles.
  constexpr int IPT = MAX_SPLIT_KEYS / MLA_THREADS;  // index entries per thread
  int32_t iv[IPT];
  {
    const int32_t* ip = idx + r * K + kb;
#pragma unroll
    for (int k = 0; k < IPT; ++k) {
      const int j = tid + MLA_THREADS * k;
      iv[k] = -1;
      if (j < nkeys) iv[k] = ip[j];
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // Queries of heads 32*wave + col, channels 16*s + 8*half + [0, 8).
  bf16x8 qf[MD / 16];
  {
    const uint16_t* qp = q + (r * MH + 32 * wave + col) * (int64_t)MD + 8 * half;
#pragma unroll
    for (int s = 0; s < MD / 16; ++s) qf[s] = load_bf16x8(qp + 16 * s);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int k = 0; k < IPT; ++k) {
    const int j = tid + MLA_THREADS * k;
    if (j < ntiles * NT) sidx[j] = iv[k];
  }
  f32x16 o[4][4];
  float m_ref = -INFINITY;  // exponent reference of this lane's head (log2 units)
  float m_max = -INFINITY;  // largest logit seen
  float l_run = 0.f;
  const uint16_t* kvb = kv + b * N * (int64_t)MD;
  const uint8_t* kvb8 = reinterpret_cast<const uint8_t*>(kvb);
  sync_lds();  // indices visible (the query loads stay in flight)

  // Gather of tile `it`: wave w fetches rows 8w..8w+7, one 128-byte line of
  // each per instruction (instruction u: bytes [128u, 128u+128) of every row,
  // u = 0..8), so an instruction touches 8 cache lines and a tile 288.  Lane L
  // takes row 8w + L/8 and, within the line, 16-byte chunk (L % 8) ^ f(row);
  // it lands at slot 64*(9w + u) + L (see the layout note at the top).
  constexpr int GU = ROW_CHUNKS / 8;  // 9 lines per row
  static_assert(GU * 8 == ROW_CHUNKS && NT == 8 * MLA_WAVES, "gather geometry");
  const int grow = 8 * wave + (lane >> 3);
  const uint32_t gsw = (uint32_t)((lane & 7) ^ row_swizzle(grow));
  // gather_begin records the rows' validity and returns the per-lane source
  // offset; gather_line(u) then issues instruction u.
  typedef typename std::conditional<ADDR64, uint64_t, uint32_t>::type GOff;
  auto gather_begin = [&](int it, uint32_t& lds0) {
    const int buf = it % NBUF;
    const int32_t v = sidx[it * NT + grow];
    const bool ok = v >= 0 && (int64_t)v < N;
    lds0 = lds_address(&kvs[buf][512 * GU * wave]);
    if ((lane & 7) == 0) vflag[buf][grow] = ok;
    const bool full = __ballot(ok) == ~0ull;
    if (lane == 0) tfull[buf][wave] = full;
    return (GOff)(ok ? v : 0) * (GOff)(MD * 2) + (GOff)(16u * gsw);
  };
  auto gather_line = [&](GOff voff, uint32_t lds0, int u) {
    if constexpr (ADDR64) dma16_addr(kvb8 + voff + 128 * u, lds0 + 1024 * u);
    else dma16(kvb8 + 128 * u, voff, lds0 + 1024 * u);
  };
  auto gather = [&](int it) {
    uint32_t lds0;
    const GOff voff = gather_begin(it, lds0);
#pragma unroll
    for (int u = 0; u < GU; ++u) gather_line(voff, lds0, u);
  };

  // QK^T operand (A) of k-step s: key row col, channels 16s + 8*half + e,
  // i.e. chunk p = 2s + half: slot 64*(9*(col/8) + s/4) + 8*(col%8) + ((2*(s%4) + half) ^ f(col)).
  int abase[4];
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4)
    abase[s4] = 8 * (576 * (col >> 3) + 8 * (col & 7) + ((2 * s4 + half) ^ row_swizzle(col)));
  // PV operand, read rd (keys 4rd..4rd+3 of this lane half) of step (ks, mb):
  // 16-lane group G = lane/16, source lane j = lane%16 addresses key
  // k = 16*ks + 8*half + 4*rd + j/4 and value columns
  // 128*wave + 32*mb + 16*(G&1) + 4*(j&3) + [0,4), i.e. byte 8*(j&1) of chunk
  // p = 16*wave + 4*mb + 2*(G&1) + (j&3)/2.  With f(k) = 4rd + 2(j>>3) + half,
  // its slot is 64*(9*(2ks + half) + 2*wave + mb/2) + 8*(k%8) + ((p%8) ^ f(k))
  //   = vlane + 64*(18ks + mb/2) + 32rd + 4*((mb&1) ^ rd),
  // vlane = 64*(9*half + 2*wave) + 8*(j>>2) + ((2*(G&1) + (j&3)/2) ^ (2*(j>>3) + half)).
  int vlane;
  {
    const int G = lane >> 4, j = lane & 15;
    const int y = (2 * (G & 1) + ((j & 3) >> 1)) ^ (2 * (j >> 3) + half);
    vlane = 8 * (64 * (9 * half + 2 * wave) + 8 * (j >> 2) + y) + 4 * (j & 1);
  }

  if (ntiles > 0) gather(0);
  if (ntiles > 1) gather(1);

  // ---- pieces of one tile ----
  constexpr int KS = MD / 16;  // QK^T k-steps (16 channels each)
  auto aop = [&](const uint16_t* t, int s) {
    return *reinterpret_cast<const bf16x8*>(t + abase[s & 3] + 512 * (s >> 2));
  };
  auto vop = [&](const uint16_t* t, int st) {
    const int ks = st >> 2, mb = st & 3;
    const s16x4 lo = lds_read_tr16(t + vlane + 8 * (64 * (18 * ks + (mb >> 1)) + 4 * (mb & 1)));
    const s16x4 hi = lds_read_tr16(t + vlane + 8 * (64 * (18 * ks + (mb >> 1)) + 32 + 4 * ((mb & 1) ^ 1)));
    return __builtin_bit_cast(bf16x8, s16x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w});
  };
  auto pbop = [&](const uint16_t* pbuf, int ks, int nb) {
    return *reinterpret_cast<const bf16x8*>(&pbuf[(32 * nb + col) * PP + 16 * ks + 8 * half]);
  };
  // k-steps s and s+1 of S^T[key][head] = KV_tile . Q^T for this wave's 32
  // heads, accumulated in sacc; the key operands stream through a ring of
  // SLOOK registers read SLOOK k-steps ahead of their MFMA.
  auto s_pair = [&](const uint16_t* t, int s, bf16x8 (&ring)[SLOOK], f32x16& sacc) {
    const bf16x8 a0 = ring[s % SLOOK], a1 = ring[(s + 1) % SLOOK];
    if (s + SLOOK < KS) ring[s % SLOOK] = aop(t, s + SLOOK);
    if (s + 1 + SLOOK < KS) ring[(s + 1) % SLOOK] = aop(t, s + 1 + SLOOK);
    if (s == 0) sacc = mfma_s_first(a0, qf[0]);
    else mfma_s(sacc, a0, qf[s]);
    if (s + 2 < KS) mfma_s(sacc, a1, qf[s + 1]);
    else mfma_s_last(sacc, a1, qf[s + 1]);
  };
  // step st = (ks, mb) of O^T[dv][head] += V^T . P^T for dv in
  // [128*wave, 128*wave+128) and all 128 heads; the value operand of step
  // st+PVLOOK is read while step st runs.
  auto pv_step = [&](const uint16_t* t, int st, bf16x8 (&vring)[PVLOOK], const bf16x8 (&pb)[4]) {
    const int mb = st & 3;
    const bf16x8 av = vring[st % PVLOOK];
    if (st + PVLOOK < 8) vring[st % PVLOOK] = vop(t, st + PVLOOK);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) o[mb][nb] = mfma32x32x16(av, pb[nb], o[mb][nb]);
  };
  // QK^T of tile tS alone (the first tile of a pass).
  auto tile_s = [&](const uint16_t* tS) {
    bf16x8 ring[SLOOK];
#pragma unroll
    for (int s = 0; s < SLOOK; ++s) ring[s] = aop(tS, s);
    f32x16 sacc;
#pragma unroll
    for (int g = 0; g < KS / 2; ++g) {
      s_pair(tS, 2 * g, ring, sacc);
      __builtin_amdgcn_sched_barrier(0);  // keep the ring
    }
    return sacc;
  };
  // PV of tile tV alone (the last tile of a pass).
  auto tile_pv = [&](const uint16_t* tV, const uint16_t* pbuf) {
    bf16x8 pb[4], vring[PVLOOK];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) pb[nb] = pbop(pbuf, 0, nb);
#pragma unroll
    for (int st = 0; st < PVLOOK; ++st) vring[st] = vop(tV, st);
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      pv_step(tV, st, vring, pb);
      if (st == 3)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) pb[nb] = pbop(pbuf, 1, nb);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  bool overflow = false;
  // Online softmax of tile `t` in log2 units; writes its bf16 P to pbuf.  This
  // lane holds head 32*wave+col for keys mfma_row(i, half); lane j^32 holds
  // the other 16 keys of the tile.  The scale is positive, so the scaled
  // maximum is the maximum of the scaled logits, and each weight is one fused
  // multiply-add and one exp2.
  auto softmax_p = [&](f32x16 sacc, int t, uint16_t* pbuf) {
    const int4 tf = *reinterpret_cast<const int4*>(&tfull[t % NBUF][0]);
    if (!__builtin_amdgcn_readfirstlane(tf.x && tf.y && tf.z && tf.w)) {
      // some row of this tile is masked: its logit is -inf (weight 0)
      const int32_t* vcur = vflag[t % NBUF];
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
    uint16_t* pp = &pbuf[(32 * wave + col) * PP + 4 * half];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      u32x2 pk;
      pk.x = pack_bf16x2(x[4 * a + 0], x[4 * a + 1]);
      pk.y = pack_bf16x2(x[4 * a + 2], x[4 * a + 3]);
      *reinterpret_cast<u32x2*>(pp + 8 * a) = pk;
    }
  };

  // PV of tile tV, QK^T of tile tS (= tile ts) and the softmax of tile ts,
  // with the softmax's vector work spread between the matrix instructions:
  // the 36 QK^T k-steps run in the first three PV steps (six pairs each), so
  // the logits are complete with 20 PV MFMAs still to issue, and the 16
  // softmax pieces go one after each of the middle 16 of those (a wave
  // issues vector instructions while its own MFMA runs only when they sit
  // right behind it).  The gather of tile gt
  // (if gt >= 0) rides on the first nine k-step pairs.  Writes P of tile ts to
  // pout.
  auto tile_fused = [&](const uint16_t* tV, const uint16_t* pbuf, const uint16_t* tS, int ts, uint16_t* pout,
                        int gt) {
    uint32_t g_lds0 = 0;
    GOff g_voff = 0;
    if (gt >= 0) g_voff = gather_begin(gt, g_lds0);
    bf16x8 ring[SLOOK], pb[4], vring[PVLOOK];
#pragma unroll
    for (int s = 0; s < SLOOK; ++s) ring[s] = aop(tS, s);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) pb[nb] = pbop(pbuf, 0, nb);
#pragma unroll
    for (int st = 0; st < PVLOOK; ++st) vring[st] = vop(tV, st);
    const int4 tf = *reinterpret_cast<const int4*>(&tfull[ts % NBUF][0]);
    f32x16 sacc;
    constexpr int PAIRS_AT[4] = {0, 6, 12, 18};  // k-step pairs before PV step st = 0..3
    int g = 0;
#pragma unroll
    for (int st = 0; st < 3; ++st) {
#pragma unroll
      for (int q2 = PAIRS_AT[st]; q2 < PAIRS_AT[st + 1]; ++q2) {
        s_pair(tS, 2 * q2, ring, sacc);
        if (g < GU && gt >= 0) gather_line(g_voff, g_lds0, g);
        ++g;
        __builtin_amdgcn_sched_barrier(0);  // keep the ring
      }
      pv_step(tV, st, vring, pb);
      if (st == 3)  // second half of the tile's keys: the P operands of ks = 1
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) pb[nb] = pbop(pbuf, 1, nb);
      __builtin_amdgcn_sched_barrier(0);
    }
    // softmax pieces (same arithmetic as softmax_p), one after each PV MFMA
    float mh = 0.f, mt = 0.f, lsum = 0.f;
    float x[16];
    uint16_t* pp = &pout[(32 * wave + col) * PP + 4 * half];
    auto piece = [&](int k) {
      if (k == 0) {
        if (!__builtin_amdgcn_readfirstlane(tf.x && tf.y && tf.z && tf.w)) {
          const int32_t* vcur = vflag[ts % NBUF];
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const int4 vf = *reinterpret_cast<const int4*>(&vcur[8 * a + 4 * half]);
            const int fl[4] = {vf.x, vf.y, vf.z, vf.w};
#pragma unroll
            for (int c = 0; c < 4; ++c)
              if (!fl[c]) sacc[4 * a + c] = -INFINITY;
          }
        }
        mh = sacc[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) mh = fmaxf(mh, sacc[i]);
      } else if (k == 1) {
#pragma unroll
        for (int i = 8; i < 16; ++i) mh = fmaxf(mh, sacc[i]);
      } else if (k == 2) {
        mt = max_halves(mh * scale_log2);  // this head's largest scaled logit in the tile
      } else if (k == 3) {
        m_max = fmaxf(m_max, mt);
        if (m_ref == -INFINITY) m_ref = mt;  // nothing accumulated yet: start the reference here
        overflow |= mt > m_ref + 64.f;
      } else if (k >= 4 && k < 12) {
        // arguments are at most 64 here (else the split is redone); exp2(-inf) = 0;
        // no reference yet (every logit so far masked): weight 0
        const int i0 = 2 * (k - 4);
#pragma unroll
        for (int i = i0; i < i0 + 2; ++i) {
          const float e = __builtin_amdgcn_exp2f(fmaf(sacc[i], scale_log2, -m_ref));
          x[i] = m_ref == -INFINITY ? 0.f : e;
          lsum += x[i];
        }
      } else if (k >= 12 && k < 16) {
        const int a = k - 12;
        u32x2 pk;
        pk.x = pack_bf16x2(x[4 * a + 0], x[4 * a + 1]);
        pk.y = pack_bf16x2(x[4 * a + 2], x[4 * a + 3]);
        *reinterpret_cast<u32x2*>(pp + 8 * a) = pk;
        if (k == 15) l_run += lsum;  // this half's keys; the halves are added at the end
      }
    };
    bf16x8 av;
#pragma unroll
    for (int st = 3; st < 8; ++st) {
      const int mb = st & 3;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        if (nb == 0) {
          av = vring[st % PVLOOK];
          if (st + PVLOOK < 8) vring[st % PVLOOK] = vop(tV, st + PVLOOK);
        }
        o[mb][nb] = mfma32x32x16(av, pb[nb], o[mb][nb]);
        __builtin_amdgcn_sched_barrier(0);
        const int slot = 4 * (st - 3) + nb;  // 20 slots for 16 pieces
        if (slot >= 2 && slot < 18) piece(slot - 2);
        if (st == 3 && nb == 3)
#pragma unroll
          for (int b2 = 0; b2 < 4; ++b2) pb[b2] = pbop(pbuf, 1, b2);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // ---- the tile pipeline ----
  // Iteration it runs PV(it) together with QK^T(it+1), the softmax of tile
  // it+1 and the gather of tile it+2, then one barrier.  Tile it+2 goes into
  // the buffer of tile it-1, which every wave finished before that barrier; P
  // alternates between two LDS buffers.
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
    overflow = false;
    // Tile 0 (and, in the first pass, the queries issued before it) must
    // have landed.  Loads complete in issue order, so the wait lets tile 1's
    // nine gather instructions stay in flight.
    if (ntiles > 1) asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    sync_lds();
    if (ntiles > 0) {
      softmax_p(tile_s(kvs[0]), 0, ps[0]);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // tile 1 landed
      sync_lds();  // P(0) and tile 1 visible
    }
    // (the iteration without a gather is peeled, so the loop body has no branch)
    for (int it = 0; it + 2 < ntiles; ++it) {
      tile_fused(kvs[it % NBUF], ps[it & 1], kvs[(it + 1) % NBUF], it + 1, ps[(it + 1) & 1], it + 2);
      // tile it+2 (the only gather in flight) must have landed
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      sync_lds();  // P(it+1) and tile it+2 visible; every wave is done with tile it and P(it)
    }
    if (ntiles > 1) {
      const int it = ntiles - 2;
      tile_fused(kvs[it % NBUF], ps[it & 1], kvs[(it + 1) % NBUF], it + 1, ps[(it + 1) & 1], -1);
      sync_lds();
    }
    if (ntiles > 0) tile_pv(kvs[(ntiles - 1) % NBUF], ps[(ntiles - 1) & 1]);  // the last tile has no successor
    // any overflow in the workgroup?  (one flag per wave; each pass rewrites all four before the barrier)
    const bool wave_ovf = __ballot(overflow) != 0ull;
    if (lane == 0) ovf_s[wave] = wave_ovf;
    sync_lds();  // also: every wave is done with the tile buffers
    const int4 of = *reinterpret_cast<const int4*>(ovf_s);
    if (!__builtin_amdgcn_readfirstlane(of.x | of.y | of.z | of.w)) break;
  }

  l_run = sum_halves(l_run);
  if (half == 0) {
    l_s[32 * wave + col] = l_run;
    m_s[32 * wave + col] = m_ref;
  }
  sync_lds();
  // Output rows (normalised; bf16).  splits == 1: out[r]; else this split's
  // partial row block in the workspace, plus its log2-sum-exp.
  float inv[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int h = 32 * nb + col;
    const float l = l_s[h], m = m_s[h];
    inv[nb] = l > 0.f ? 1.f / l : 0.f;
    const float lse2 = l > 0.f ? m + log2f(l) : -INFINITY;
    if (wave == 0 && half == 0) {
      if (splits == 1) {
        if (lse != nullptr) lse[r * MH + h] = lse2 * LN2;
      } else {
        part_lse[((int64_t)sp * R + r) * MH + h] = lse2;
      }
    }
  }
  uint16_t* const dst = splits == 1 ? out + r * (int64_t)(MH * MDV) : part_o + ((int64_t)sp * R + r) * (MH * MDV);
  // Two rounds of 64 heads staged in the (now idle) tile buffers, rows of
  // EPITCH bf16: each wave writes its 128 value columns of every head, then
  // copies 16 whole rows (1 KiB each, one store instruction per row) out.
  // The lane index is taken afresh from the execution mask here, so that no
  // lane-dependent value has to stay live (or be spilled) across the tiles.
  constexpr int EPITCH = MDV + 8;
  static_assert(64 * EPITCH <= NBUF * NT * MD, "output staging fits the tile buffers");
  uint16_t* const stage = &kvs[0][0];
  const int elane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int wbase = (elane & 31) * EPITCH + 128 * wave + 4 * (elane >> 5);
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    if (q == 1) sync_lds();  // every wave has copied out round 0
#pragma unroll
    for (int n2 = 0; n2 < 2; ++n2) {
      const int nb = 2 * q + n2;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const f32x16& v = o[mb][nb];
          u32x2 pk;
          pk.x = pack_bf16x2(v[4 * a + 0] * inv[nb], v[4 * a + 1] * inv[nb]);
          pk.y = pack_bf16x2(v[4 * a + 2] * inv[nb], v[4 * a + 3] * inv[nb]);
          *reinterpret_cast<u32x2*>(stage + wbase + 32 * n2 * EPITCH + 32 * mb + 8 * a) = pk;
        }
    }
    sync_lds();
#pragma unroll
    for (int g = 0; g < 4; ++g) {  // four row reads in flight, then their four stores
      const uint16_t* sp4 = stage + (16 * wave + 4 * g) * EPITCH + 8 * elane;
      const u32x4 v0 = *reinterpret_cast<const u32x4*>(sp4);
      const u32x4 v1 = *reinterpret_cast<const u32x4*>(sp4 + EPITCH);
      const u32x4 v2 = *reinterpret_cast<const u32x4*>(sp4 + 2 * EPITCH);
      const u32x4 v3 = *reinterpret_cast<const u32x4*>(sp4 + 3 * EPITCH);
      __builtin_amdgcn_sched_barrier(0);
      uint16_t* dp4 = dst + (64 * q + 16 * wave + 4 * g) * MDV + 8 * elane;
      if (splits == 1) {  // the output: streaming stores
        __builtin_nontemporal_store(v0, reinterpret_cast<u32x4*>(dp4));
        __builtin_nontemporal_store(v1, reinterpret_cast<u32x4*>(dp4 + MDV));
        __builtin_nontemporal_store(v2, reinterpret_cast<u32x4*>(dp4 + 2 * MDV));
        __builtin_nontemporal_store(v3, reinterpret_cast<u32x4*>(dp4 + 3 * MDV));
      } else {  // a split partial: kept in this XCD's cache for the combine, which runs on the same XCD
        *reinterpret_cast<u32x4*>(dp4) = v0;
        *reinterpret_cast<u32x4*>(dp4 + MDV) = v1;
        *reinterpret_cast<u32x4*>(dp4 + 2 * MDV) = v2;
        *reinterpret_cast<u32x4*>(dp4 + 3 * MDV) = v3;
      }
    }
  }
}

// Merge the split partials of one (query, head): weights 2^(lse_s - lse_max).
// One wave per (query, head); lane l owns value columns 8l..8l+7, so every
// partial row is one 1 KiB load, and the splits' loads are independent.
constexpr int COMBINE_WAVES = 4;
constexpr int COMBINE_CHUNK = 8;  // partial rows in flight per lane
// part_o is not declared restrict, so that the compiler barrier below keeps
// its loads ahead of the reductions.
__global__ __launch_bounds__(64 * COMBINE_WAVES) void mla_combine_kernel(const uint16_t* part_o,
                                                                        const float* __restrict__ part_lse,
                                                                        uint16_t* __restrict__ out,
                                                                        float* __restrict__ lse, int64_t R,
                                                                        int splits) {
  const int lane = threadIdx.x & 63;
  // (query, head) of this wave.  When the rows split evenly over the 8 XCDs,
  // the MLA kernel ran every split of query r on XCD r & 7 (workgroups are
  // dealt round-robin to the XCDs), and its partials are read on that XCD too.
  int64_t rh;
  if ((R & 7) == 0) {
    constexpr int PER = MH / COMBINE_WAVES;  // workgroups per query
    const int64_t c = blockIdx.x, x = c & 7, j = c >> 3;
    rh = (x + 8 * (j / PER)) * MH + (j % PER) * COMBINE_WAVES + (threadIdx.x >> 6);
  } else {
    rh = (int64_t)blockIdx.x * COMBINE_WAVES + (threadIdx.x >> 6);
  }
  const int64_t stride = R * MH;
  if (rh >= stride) return;  // whole waves only
  // Lane s < splits holds split s's log2-sum-exp (2 <= splits <= 64, checked at
  // launch).  Its load goes out first and the first chunk's partial rows right
  // behind it, so the weights' reductions wait for the log-sums alone and run
  // while the rows arrive: one memory round trip rather than two in a row.
  const float ls_raw = part_lse[min(lane, splits - 1) * stride + rh];
  const uint16_t* base = part_o + rh * MDV + 8 * lane;
  uint4 v[COMBINE_CHUNK];
#pragma unroll
  for (int c = 0; c < COMBINE_CHUNK; ++c)  // past the last split: reread it with weight 0
    v[c] = *reinterpret_cast<const uint4*>(base + min(c, splits - 1) * stride * MDV);
  asm volatile("" ::: "memory");  // keeps the loads here, ahead of the reductions
  const float ls = lane < splits ? ls_raw : -INFINITY;
  const float M = wave_fmax(ls);
  const float e = M == -INFINITY ? 0.f : exp2f(ls - M);  // exp2(-inf) = 0 for empty splits
  const float den = wave_fsum(e);
  const float inv = den > 0.f ? 1.f / den : 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < splits; s0 += COMBINE_CHUNK) {
    if (s0 > 0)
#pragma unroll
      for (int c = 0; c < COMBINE_CHUNK; ++c)
        v[c] = *reinterpret_cast<const uint4*>(base + min(s0 + c, splits - 1) * stride * MDV);
#pragma unroll
    for (int c = 0; c < COMBINE_CHUNK; ++c) {
      // lane s0 + c <= 63 (splits <= 64, chunks of 8); lanes at or past splits hold e = 0
      const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(e), s0 + c)) * inv;
      const uint32_t wd[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        acc[2 * k] += w * bf16_bits_to_float(wd[k] & 0xffffu);
        acc[2 * k + 1] += w * bf16_bits_to_float(wd[k] >> 16);
      }
    }
  }
  u32x4 pk;
  pk.x = pack_bf16x2(acc[0], acc[1]);
  pk.y = pack_bf16x2(acc[2], acc[3]);
  pk.z = pack_bf16x2(acc[4], acc[5]);
  pk.w = pack_bf16x2(acc[6], acc[7]);
  __builtin_nontemporal_store(pk, reinterpret_cast<u32x4*>(out + rh * MDV + 8 * lane));
  if (lse != nullptr && lane == 0) lse[rh] = M == -INFINITY ? -INFINITY : (M + log2f(den)) * LN2;
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
  // At most one workgroup per compute unit (256) over the launch: a second,
  // partly filled round of workgroups would cost as much as the first.
  int64_t want = 256 / rows;
  if (want < 1) want = 1;
  if (want > 32) want = 32;
  if (want > tiles) want = tiles;
  // one workgroup stages at most MAX_SPLIT_KEYS indices
  const int64_t need = (K + MAX_SPLIT_KEYS - 1) / MAX_SPLIT_KEYS;
  if (want < need) want = need;
  // drop splits that whole-tile shares would leave empty
  const int64_t per = (tiles + want - 1) / want;
  want = (tiles + per - 1) / per;
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
  if (N * (int64_t)MD * 2 > (int64_t)0xffffffffLL)
    hipLaunchKernelGGL(sparse_mla_bf16_kernel<true>, dim3((unsigned)(R * splits)), dim3(MLA_THREADS), 0, stream, q,
                       kv, idx, out, lse, part_o, part_lse, R, Tq, N, K, splits, kps, scale * LOG2E);
  else
    hipLaunchKernelGGL(sparse_mla_bf16_kernel<false>, dim3((unsigned)(R * splits)), dim3(MLA_THREADS), 0, stream, q,
                       kv, idx, out, lse, part_o, part_lse, R, Tq, N, K, splits, kps, scale * LOG2E);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  if (splits > 64) return hipErrorInvalidValue;  // the combine holds one split per lane
  const int64_t cwg = (R * MH + COMBINE_WAVES - 1) / COMBINE_WAVES;
  hipLaunchKernelGGL(mla_combine_kernel, dim3((unsigned)cwg), dim3(64 * COMBINE_WAVES), 0, stream, part_o, part_lse,
                     out, lse, R, splits);
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

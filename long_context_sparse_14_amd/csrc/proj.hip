// Projections on either side of the sparse MLA, as one batched bf16 GEMM on
// the matrix cores:
//   * query absorption: q_lat[m, h, :d_c] = W_UK[h]^T q[m, h, :d_nope], with the
//     rope part q[m, h, d_nope:] copied behind it (the key up-projection folded
//     into the query, so that the attention runs over the shared latent rows);
//   * output projection: o[m, h, :] = W_UV[h] o_lat[m, h, :] (the value
//     up-projection applied to the latent attention output);
//   * a plain linear layer y = x W^T (the indexer's query projection wq_b from
//     the query latent, and its per-head weight projection).
// DeepSeek-V3 documentation, "DeepseekV3Config" (kv_lora_rank, qk_nope_head_dim,
// qk_rope_head_dim, v_head_dim: keys and values are low-rank projections of one
// latent); DeepSeek-V3.2 documentation, "DeepSeek Sparse Attention (DSA)" (the
// indexer's queries come from the low-rank query latent through wq_b).
//
// C[z][m, n] = sum_k A[z][m, k] * B[z](k, n), fp32 accumulation, bf16 output
// rounded to nearest even.  A is row-major with k contiguous.  B is either
// [N][K] (k contiguous, as a linear layer's weight) or [K][N] (n contiguous,
// as W_UK[h] [d_nope, d_c] is read by the absorption).
//
// Tiling for many rows: a 256-thread workgroup (4 waves) owns a 128 x 128
// tile of C; each wave a 64 x 64 block, four 32x32x16 MFMA chains fed by two A
// and two B operand reads per k-step (few rows take the split-K kernel below).
// K advances 32 at a time (64 for a [N][K] B when K allows it) through
// double-buffered LDS tiles,
// and global loads run two tiles ahead through registers.  A and a [N][K] B
// sit in LDS row-major with k contiguous (80- or 144-byte pitch), so an operand is
// one 16-byte read.  A [K][N] B keeps its global layout in LDS (n contiguous,
// 288-byte pitch) and reaches the MFMA through the gfx950 transposing read
// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element
// (i & 3) of the 8 bytes addressed by lane 4c + (i >> 2), c = 0..3, so lanes
// that address four consecutive k-rows of four consecutive columns hand every
// lane four k-values of its own column.

#include "device_common.h"
#include "launch.h"
#include "select_common.h"

namespace dsa {
namespace {

constexpr int GN = 128;           // columns of C per workgroup
constexpr int KNPITCH = GN + 16;  // bf16 per LDS k-row of a [K][N] B

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ s16x4 lds_read_tr16(const uint16_t* p) {
  typedef __attribute__((address_space(3))) s16x4* lds_s16x4_ptr;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)p);
}

// WM x WN MFMA tiles per wave, WAVES_M x WAVES_N waves (4 in all); GK k per
// LDS tile (32, or 64 when K allows it: each tile's loads are a round trip
// that the two tiles of prefetch do not fully hide, so fewer, larger tiles
// expose fewer of them).
template <int WM, int WN, int WAVES_M, bool B_NK, int GK>
__global__ __launch_bounds__(256, GK == 32 ? 3 : 2) void gemm_bf16_kernel(GemmArgs g) {
  constexpr int APITCH = GK + 8;    // bf16 per LDS row of A and of a [N][K] B
  constexpr int CPR = GK / 8;       // 16-byte chunks per row of an A tile
  constexpr int WAVES_N = 4 / WAVES_M;
  constexpr int BM = 32 * WM * WAVES_M;
  static_assert(32 * WN * WAVES_N == GN, "a workgroup covers 128 columns");
  constexpr int A_CHUNKS = BM * GK / 8;                   // 16-byte chunks of an A tile
  constexpr int A_PER = (A_CHUNKS + 255) / 256;
  constexpr int B_PER = GN * GK / 8 / 256;                // 2 or 4
  constexpr int B_LDS = B_NK ? GN * APITCH : GK * KNPITCH;
  constexpr int CPITCH = GN + 8;                          // bf16 per staged output row
  constexpr int LDS_ELEMS = 2 * BM * APITCH + 2 * B_LDS;
  static_assert(BM * CPITCH <= LDS_ELEMS, "the output tile is staged in the operand buffers");
  __shared__ __align__(16) uint16_t lds[LDS_ELEMS];
  uint16_t(*As)[BM * APITCH] = reinterpret_cast<uint16_t(*)[BM * APITCH]>(lds);
  uint16_t(*Bs)[B_LDS] = reinterpret_cast<uint16_t(*)[B_LDS]>(lds + 2 * BM * APITCH);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WAVES_M, wn = wave / WAVES_M;
  const int half = lane >> 5, col = lane & 31;
  // Workgroups are dealt to the 8 XCDs round-robin by launch order; renumber
  // them so that each XCD runs a contiguous range of tiles.  Within a batch
  // entry the tiles go in groups of up to GROUP_M row blocks, the column
  // index advancing once per group's sweep down its rows, so that the
  // workgroups resident on one XCD at a time share both their rows of A and
  // their columns of B in its L2 (row block after row block, every row block
  // streamed all of B through it).
  constexpr int64_t GROUP_M = 8;
  const int64_t gx = gridDim.x, gy = gridDim.y;
  const int64_t total = gx * gy * gridDim.z;
  int64_t P = blockIdx.x + gx * (blockIdx.y + gy * (int64_t)blockIdx.z);
  if ((total & 7) == 0) P = (P & 7) * (total >> 3) + (P >> 3);
  const int64_t z = P / (gx * gy);
  const int64_t local = P % (gx * gy);
  const int64_t first_m = local / (GROUP_M * gx) * GROUP_M;
  const int64_t gsz = min(gy - first_m, GROUP_M);
  const int64_t in_group = local % (GROUP_M * gx);
  const int64_t m0 = (first_m + in_group % gsz) * BM;
  const int n0 = (int)(in_group / gsz) * GN;
  const uint16_t* A = g.A + z * g.sA;
  const uint16_t* B = g.B + z * g.sB;
  uint16_t* C = g.C + z * g.sC;

  // Chunk c of an A tile: row c / CPR, k-chunk c % CPR.  Of a [N][K] B tile:
  // the same with n for the row.  Of a [K][N] B tile: k-row c >> 4, n-chunk c & 15.
  typedef u32x4 Stage[A_PER + B_PER];
  auto gload = [&](Stage& r, int k0) {
#pragma unroll
    for (int u = 0; u < A_PER; ++u) {
      const int c = tid + 256 * u;
      const int64_t m = m0 + c / CPR;
      r[u] = (c < A_CHUNKS && m < g.M) ? *reinterpret_cast<const u32x4*>(A + m * g.lda + k0 + 8 * (c % CPR))
                                       : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < B_PER; ++u) {
      const int c = tid + 256 * u;
      if (B_NK) {
        const int n = n0 + c / CPR;
        r[A_PER + u] = n < g.N ? *reinterpret_cast<const u32x4*>(B + (int64_t)n * g.ldb + k0 + 8 * (c % CPR))
                               : u32x4{0, 0, 0, 0};
      } else {
        const int n = n0 + 8 * (c & 15);
        r[A_PER + u] = n < g.N ? *reinterpret_cast<const u32x4*>(B + (int64_t)(k0 + (c >> 4)) * g.ldb + n)
                               : u32x4{0, 0, 0, 0};
      }
    }
  };
  auto lstore = [&](const Stage& r, int buf) {
#pragma unroll
    for (int u = 0; u < A_PER; ++u) {
      const int c = tid + 256 * u;
      if (c < A_CHUNKS) *reinterpret_cast<u32x4*>(&As[buf][(c / CPR) * APITCH + 8 * (c % CPR)]) = r[u];
    }
#pragma unroll
    for (int u = 0; u < B_PER; ++u) {
      const int c = tid + 256 * u;
      if (B_NK)
        *reinterpret_cast<u32x4*>(&Bs[buf][(c / CPR) * APITCH + 8 * (c % CPR)]) = r[A_PER + u];
      else
        *reinterpret_cast<u32x4*>(&Bs[buf][(c >> 4) * KNPITCH + 8 * (c & 15)]) = r[A_PER + u];
    }
  };
  // B operand of MFMA column block j (32 columns) at k-step ks.
  const int g16 = lane >> 4, i16 = lane & 15;
  auto bop = [&](int buf, int j, int ks) -> bf16x8 {
    const int nb = 32 * (WN * wn + j);
    if (B_NK) return *reinterpret_cast<const bf16x8*>(&Bs[buf][(nb + col) * APITCH + 16 * ks + 8 * half]);
    // lane (group g16, c = i16 >> 2, r = i16 & 3) addresses k-row 8*(g16>>1) + c (+4 for the upper four)
    // at columns nb + 16*(g16&1) + 4r .. +3
    const uint16_t* p = &Bs[buf][(16 * ks + 8 * (g16 >> 1) + (i16 >> 2)) * KNPITCH + nb + 16 * (g16 & 1) +
                                 4 * (i16 & 3)];
    const s16x4 lo = lds_read_tr16(p);
    const s16x4 hi = lds_read_tr16(p + 4 * KNPITCH);
    return __builtin_bit_cast(bf16x8, s16x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w});
  };

  f32x16 acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = f32x16{};

  auto compute = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < GK / 16; ++ks) {
      bf16x8 a[WM], b[WN];
#pragma unroll
      for (int i = 0; i < WM; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(&As[buf][(32 * (WM * wm + i) + col) * APITCH + 16 * ks + 8 * half]);
#pragma unroll
      for (int j = 0; j < WN; ++j) b[j] = bop(buf, j, ks);
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j) acc[i][j] = mfma32x32x16(a[i], b[j], acc[i][j]);
    }
  };

  // Global loads run two tiles ahead: r0 and r1 alternate between tiles.
  const int nt = g.K / GK;
  Stage r0, r1;
  gload(r0, 0);
  if (nt > 1) gload(r1, GK);
  lstore(r0, 0);
  __syncthreads();
  for (int it = 0; it < nt; it += 2) {
    if (it + 2 < nt) gload(r0, (it + 2) * GK);
    compute(0);
    if (it + 1 < nt) lstore(r1, 1);
    __syncthreads();
    if (it + 1 >= nt) break;
    if (it + 3 < nt) gload(r1, (it + 3) * GK);
    compute(1);
    if (it + 2 < nt) lstore(r0, 0);
    __syncthreads();
  }

  // Epilogue: the tile is staged in LDS as bf16 (the loop's last barrier has
  // freed the operand buffers), then leaves in 16-byte row chunks.
#pragma unroll
  for (int j = 0; j < WN; ++j)
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        lds[(32 * (WM * wm + i) + mfma_row(e, half)) * CPITCH + 32 * (WN * wn + j) + col] =
            (uint16_t)float_to_bf16_bits(acc[i][j][e]);
  __syncthreads();
  const bool vec = ((reinterpret_cast<uintptr_t>(C) & 15) == 0) && (g.ldc % 8) == 0;
  for (int c = tid; c < BM * (GN / 8); c += 256) {
    const int r = c / (GN / 8), ch = c % (GN / 8);
    const int64_t m = m0 + r;
    const int n = n0 + 8 * ch;
    if (m >= g.M || n >= g.N) continue;
    const uint16_t* src = &lds[r * CPITCH + 8 * ch];
    if (vec && n + 8 <= g.N) {
      *reinterpret_cast<u32x4*>(C + m * g.ldc + n) = *reinterpret_cast<const u32x4*>(src);
    } else {
      for (int e = 0; e < 8 && n + e < g.N; ++e) C[m * g.ldc + n + e] = src[e];
    }
  }

  // Optional row copy riding on the first column block (the rope part of an
  // absorbed query): cp_w bf16 per row, in 16-byte chunks.
  if (g.cp_dst != nullptr && n0 == 0) {
    const int chunks = g.cp_w / 8;
    for (int c = tid; c < BM * chunks; c += 256) {
      const int64_t m = m0 + c / chunks;
      if (m >= g.M) break;
      const int off = 8 * (c % chunks);
      *reinterpret_cast<u32x4*>(g.cp_dst + z * g.cp_sd + m * g.cp_ldd + off) =
          *reinterpret_cast<const u32x4*>(g.cp_src + z * g.cp_ss + m * g.cp_lds + off);
    }
  }
}

// The [K][N] weight with short K (K <= KMAX, the absorption's d_nope) and many
// rows.  With K = 128 a 128 x 128 tile is only eight k-steps of work, so the
// tiled kernel above spends most of each workgroup on its own start and
// epilogue, and fetches each block of A once per column block.  Here a
// 256-thread workgroup owns 128 rows of one batch entry and walks all of N,
// BN columns at a time:
//   * A [128 x K] is staged once through LDS into registers (the MFMA A
//     operands of the wave's rows for every k-step);
//   * B column blocks [K x BN] alternate between two LDS buffers, the next
//     one's global loads in flight while the current one is multiplied, and
//     reach the MFMA through the transposing read as above;
//   * each 128 x BN output block is staged as bf16 in the buffer just
//     consumed and leaves in 16-byte row chunks;
//   * the row copy (the absorbed query's rope part) rides along at the end.
// BN = 64 with each wave on 32 rows (120 registers, 40 KiB of LDS: four
// workgroups per compute unit) ran the absorption at M = 16384 in 0.69-0.70
// ms against 0.75-0.76 with BN = 128 and 64-row waves (242 registers, 72 KiB,
// two per unit): each block's wait for the next B block also waits for the
// previous block's output stores (loads and stores share one counter), and
// more resident workgroups cover it.  The barriers inside the walk settle LDS
// only.  Workgroups are renumbered so that each XCD runs a contiguous range,
// in groups of WALK_HG batch entries with the entry advancing fastest: the
// workgroups resident together write neighbouring pieces of the same output
// rows and share those entries' B in L2.  Requires 16-byte aligned A, B, C
// and row pitches that are multiples of 8 elements.
constexpr int64_t WALK_HG = 16;
template <int KMAX, int BN>
__global__ __launch_bounds__(256, BN == 128 ? 2 : 4) void gemm_kn_walk_kernel(GemmArgs g) {
  constexpr int BM = 128, KS = KMAX / 16;
  constexpr int WAVES_M = BN == 128 ? 2 : 4, WAVES_N = 4 / WAVES_M;
  constexpr int WM = BM / 32 / WAVES_M, WN = BN / 32 / WAVES_N;
  constexpr int BPITCH = BN + 16;          // bf16 per LDS k-row of a B block
  constexpr int APITCH = KMAX + 8;         // bf16 per staged A row
  constexpr int B_LDS = KMAX * BPITCH;     // one [KMAX][BN] column block of B
  constexpr int CPITCH = BN + 8;           // bf16 per staged output row
  constexpr int BCH = BN / 8;              // 16-byte chunks per k-row of a B block
  constexpr int PER_A = BM * KMAX / 8 / 256, PER_B = KMAX * BCH / 256;
  static_assert(BM * APITCH <= 2 * B_LDS && BM * CPITCH <= B_LDS, "A and the output block stage in the B buffers");
  static_assert(KMAX % 32 == 0 && PER_A * 256 * 8 == BM * KMAX && PER_B * 256 == KMAX * BCH, "walk geometry");
  static_assert(WM * 32 * WAVES_M == BM && WN * 32 * WAVES_N == BN, "waves cover the block");
  __shared__ __align__(16) uint16_t lds[2 * B_LDS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WAVES_M, wn = wave / WAVES_M;
  const int half = lane >> 5, col = lane & 31;
  const int64_t gy = (g.M + BM - 1) / BM;
  const int64_t total = gridDim.x, nz = total / gy;
  int64_t P = blockIdx.x;
  if ((total & 7) == 0) P = (P & 7) * (total >> 3) + (P >> 3);
  const int64_t first_z = P / (WALK_HG * gy) * WALK_HG;
  const int64_t zsz = min(nz - first_z, WALK_HG);
  const int64_t in_group = P - first_z * gy;
  const int64_t z = first_z + in_group % zsz;
  const int64_t m0 = in_group / zsz * BM;
  const uint16_t* A = g.A + z * g.sA;
  const uint16_t* B = g.B + z * g.sB;
  uint16_t* C = g.C + z * g.sC;
  const int K = g.K, N = g.N, kc = K / 8;  // K: a multiple of 32, at most KMAX; N: a multiple of 8
  const int nblk = (N + BN - 1) / BN;

  // chunk c of A: row c / kc, k-chunk c % kc; of B block n0: k-row c / BCH, columns n0 + 8 * (c % BCH)
  auto gload_b = [&](u32x4 (&r)[PER_B], int n0) {
#pragma unroll
    for (int u = 0; u < PER_B; ++u) {
      const int c = tid + 256 * u;
      const int n = n0 + 8 * (c % BCH);
      r[u] = (c < K * BCH && n < N) ? *reinterpret_cast<const u32x4*>(B + (int64_t)(c / BCH) * g.ldb + n)
                                    : u32x4{0, 0, 0, 0};
    }
  };
  auto lstore_b = [&](const u32x4 (&r)[PER_B], int buf) {
#pragma unroll
    for (int u = 0; u < PER_B; ++u) {
      const int c = tid + 256 * u;
      if (c < K * BCH) *reinterpret_cast<u32x4*>(&lds[buf * B_LDS + (c / BCH) * BPITCH + 8 * (c % BCH)]) = r[u];
    }
  };

  // A staged at the start of LDS (through registers) while B block 0 is fetched
  u32x4 ra[PER_A], rb[PER_B];
#pragma unroll
  for (int u = 0; u < PER_A; ++u) {
    const int c = tid + 256 * u;
    const int64_t m = m0 + c / kc;
    ra[u] = (c < BM * kc && m < g.M) ? *reinterpret_cast<const u32x4*>(A + m * g.lda + 8 * (c % kc))
                                     : u32x4{0, 0, 0, 0};
  }
  gload_b(rb, 0);
#pragma unroll
  for (int u = 0; u < PER_A; ++u) {
    const int c = tid + 256 * u;
    if (c < BM * kc) *reinterpret_cast<u32x4*>(&lds[(c / kc) * APITCH + 8 * (c % kc)]) = ra[u];
  }
  __syncthreads();
  bf16x8 a[WM][KS];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      if (16 * ks < K)
        a[i][ks] = *reinterpret_cast<const bf16x8*>(&lds[(32 * (WM * wm + i) + col) * APITCH + 16 * ks + 8 * half]);
  lds_barrier();  // A is in registers: the buffers are free
  lstore_b(rb, 0);
  lds_barrier();

  const int g16 = lane >> 4, i16 = lane & 15;
  for (int nb = 0; nb < nblk; ++nb) {
    const int buf = nb & 1, n0 = nb * BN;
    if (nb + 1 < nblk) gload_b(rb, n0 + BN);
    f32x16 acc[WM][WN];
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int j = 0; j < WN; ++j) acc[i][j] = f32x16{};
    const uint16_t* Bs = &lds[buf * B_LDS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (16 * ks >= K) break;
      bf16x8 b[WN];
#pragma unroll
      for (int j = 0; j < WN; ++j) {
        const int nc = 32 * (WN * wn + j);
        const uint16_t* p = Bs + (16 * ks + 8 * (g16 >> 1) + (i16 >> 2)) * BPITCH + nc + 16 * (g16 & 1) + 4 * (i16 & 3);
        const s16x4 lo = lds_read_tr16(p);
        const s16x4 hi = lds_read_tr16(p + 4 * BPITCH);
        b[j] = __builtin_bit_cast(bf16x8, s16x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w});
      }
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j) acc[i][j] = mfma32x32x16(a[i][ks], b[j], acc[i][j]);
    }
    lds_barrier();  // every wave has read this B block and copied the previous output block out of LDS
    uint16_t* Cs = &lds[buf * B_LDS];
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          Cs[(32 * (WM * wm + i) + mfma_row(e, half)) * CPITCH + 32 * (WN * wn + j) + col] =
              (uint16_t)float_to_bf16_bits(acc[i][j][e]);
    if (nb + 1 < nblk) lstore_b(rb, buf ^ 1);
    lds_barrier();
    for (int c = tid; c < BM * BCH; c += 256) {
      const int r = c / BCH, ch = c % BCH;
      const int64_t m = m0 + r;
      const int n = n0 + 8 * ch;
      if (m < g.M && n < N)
        *reinterpret_cast<u32x4*>(C + m * g.ldc + n) = *reinterpret_cast<const u32x4*>(&Cs[r * CPITCH + 8 * ch]);
    }
  }

  // Optional row copy (the rope part of an absorbed query): cp_w bf16 per row,
  // in 16-byte chunks, four per thread at a time with every load issued before
  // the stores (source and destination may alias, so the compiler otherwise
  // keeps each load behind the previous store: four round trips in a row).
  if (g.cp_dst != nullptr) {
    const int chunks = g.cp_w / 8, tot = BM * chunks;
    for (int c0 = 0; c0 < tot; c0 += 4 * 256) {
      u32x4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = c0 + tid + 256 * u;
        const int64_t m = m0 + c / chunks;
        v[u] = (c < tot && m < g.M)
                   ? *reinterpret_cast<const u32x4*>(g.cp_src + z * g.cp_ss + m * g.cp_lds + 8 * (c % chunks))
                   : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = c0 + tid + 256 * u;
        const int64_t m = m0 + c / chunks;
        if (c < tot && m < g.M)
          *reinterpret_cast<u32x4*>(g.cp_dst + z * g.cp_sd + m * g.cp_ldd + 8 * (c % chunks)) = v[u];
      }
    }
  }
}

constexpr int WALK_BN = 64;

// Few rows (M <= 64), where the weights' bytes bound the time.  A workgroup
// of WK x WN waves owns a 32 x 32*WN tile of C over the whole of K: wave
// (wk, wn) computes columns 32*wn .. +32 from every WK-th k-step of 16
// (starting at wk), keeping U k-steps of operand loads in flight.  A and a
// [N][K] B go from global memory straight into the MFMA operand registers
// (lane j: row or column j % 32, eight k from 8 * (j / 32)).  A [K][N] B is
// staged per wave through LDS ([16 k][32 n] per k-step) and read back with the
// transposing read.  With WK > 1 the partial tiles are summed in LDS in a
// fixed order, so the result does not depend on timing.
template <bool B_NK, int WK, int WN, int U>
__global__ __launch_bounds__(64 * WK * WN) void gemm_skinny_kernel(GemmArgs g) {
  constexpr int WAVES = WK * WN;
  constexpr int KP = 48;          // bf16 per staging row (96 B: four rows fall on distinct banks)
  constexpr int STAGE = B_NK ? 1 : WAVES * U * 16 * KP;
  constexpr int RED = WK > 1 ? WAVES * 16 * 64 : 1;
  __shared__ __align__(16) uint16_t stage[STAGE];
  __shared__ float red[RED];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wk = wave % WK, wn = wave / WK;
  const int half = lane >> 5, col = lane & 31;
  const int g16 = lane >> 4, i16 = lane & 15;
  const int64_t z = blockIdx.z;
  const int64_t m0 = (int64_t)blockIdx.y * 32;
  const int n0 = blockIdx.x * 32 * WN + 32 * wn;
  const uint16_t* A = g.A + z * g.sA;
  const uint16_t* B = g.B + z * g.sB;
  uint16_t* C = g.C + z * g.sC;

  const int64_t m = m0 + col;
  const bool m_ok = m < g.M;
  const uint16_t* a_ptr = A + (m_ok ? m : 0) * g.lda + 8 * half;
  // [N][K]: column n0 + col, k from 8 * half.  [K][N]: k-row lane >> 2 of the
  // step, columns n0 + 8 * (lane & 3) .. +7.
  const int n_nk = n0 + col;
  const int n_kn = n0 + 8 * (lane & 3);
  const bool b_ok = B_NK ? n_nk < g.N : n_kn < g.N;
  const uint16_t* b_ptr = B_NK ? B + (int64_t)(b_ok ? n_nk : 0) * g.ldb + 8 * half
                               : B + (int64_t)(lane >> 2) * g.ldb + (b_ok ? n_kn : 0);
  const int64_t b_step = B_NK ? 16 : 16 * g.ldb;

  f32x16 acc{};
  const int S = g.K / 16;
  for (int s0 = wk; s0 < S; s0 += WK * U) {
    u32x4 ra[U], rb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + WK * u;
      if (s < S) {
        ra[u] = m_ok ? *reinterpret_cast<const u32x4*>(a_ptr + 16 * s) : u32x4{0, 0, 0, 0};
        rb[u] = b_ok ? *reinterpret_cast<const u32x4*>(b_ptr + b_step * s) : u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + WK * u;
      if (s >= S) break;
      bf16x8 bv;
      if (B_NK) {
        bv = __builtin_bit_cast(bf16x8, rb[u]);
      } else {
        uint16_t* st = &stage[(wave * U + u) * 16 * KP];
        *reinterpret_cast<u32x4*>(&st[(lane >> 2) * KP + 8 * (lane & 3)]) = rb[u];
        // the wave's own LDS writes are performed before its later reads
        __builtin_amdgcn_wave_barrier();
        const uint16_t* p = &st[(8 * (g16 >> 1) + (i16 >> 2)) * KP + 16 * (g16 & 1) + 4 * (i16 & 3)];
        const s16x4 lo = lds_read_tr16(p);
        const s16x4 hi = lds_read_tr16(p + 4 * KP);
        bv = __builtin_bit_cast(bf16x8, s16x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w});
      }
      acc = mfma32x32x16(__builtin_bit_cast(bf16x8, ra[u]), bv, acc);
    }
  }

  const int nn = n0 + col;
  if (WK == 1) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t mm = m0 + mfma_row(e, half);
      if (mm < g.M && nn < g.N) C[mm * g.ldc + nn] = (uint16_t)float_to_bf16_bits(acc[e]);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e) red[(wave * 16 + e) * 64 + lane] = acc[e];
    __syncthreads();
    constexpr int PER = 16 / WK;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int e = PER * wk + q;
      float v = red[((WK * wn) * 16 + e) * 64 + lane];
#pragma unroll
      for (int w = 1; w < WK; ++w) v += red[((WK * wn + w) * 16 + e) * 64 + lane];
      const int64_t mm = m0 + mfma_row(e, half);
      if (mm < g.M && nn < g.N) C[mm * g.ldc + nn] = (uint16_t)float_to_bf16_bits(v);
    }
  }

  if (g.cp_dst != nullptr && blockIdx.x == 0) {
    const int chunks = g.cp_w / 8;
    for (int c = tid; c < 32 * chunks; c += 64 * WAVES) {
      const int64_t mr = m0 + c / chunks;
      if (mr >= g.M) break;
      const int off = 8 * (c % chunks);
      *reinterpret_cast<u32x4*>(g.cp_dst + z * g.cp_sd + mr * g.cp_ldd + off) =
          *reinterpret_cast<const u32x4*>(g.cp_src + z * g.cp_ss + mr * g.cp_lds + off);
    }
  }
}

template <bool B_NK, int WK, int WN, int U>
hipError_t launch_skinny(const GemmArgs& g, int64_t batch, hipStream_t stream) {
  const dim3 grid((unsigned)((g.N + 32 * WN - 1) / (32 * WN)), (unsigned)((g.M + 31) / 32), (unsigned)batch);
  hipLaunchKernelGGL((gemm_skinny_kernel<B_NK, WK, WN, U>), grid, dim3(64 * WK * WN), 0, stream, g);
  return hipGetLastError();
}

template <int WM, int WN, int WAVES_M>
hipError_t launch_tiles(const GemmArgs& g, bool b_nk, int64_t batch, hipStream_t stream) {
  constexpr int BM = 32 * WM * WAVES_M;
  const dim3 grid((unsigned)((g.N + GN - 1) / GN), (unsigned)((g.M + BM - 1) / BM), (unsigned)batch);
  // 64-wide k tiles for [N][K] weights when K allows it (the output
  // projection at M = 16384: 713 -> 649 us; the linear layer unchanged); the
  // [K][N] absorption weight keeps 32 (with K = 128, the larger tiles' two
  // workgroups per compute unit ran it 17% slower than three).
  if (b_nk && g.K % 64 == 0)  // K is a multiple of 32 (checked on entry)
    hipLaunchKernelGGL((gemm_bf16_kernel<WM, WN, WAVES_M, true, 64>), grid, dim3(256), 0, stream, g);
  else if (b_nk)
    hipLaunchKernelGGL((gemm_bf16_kernel<WM, WN, WAVES_M, true, 32>), grid, dim3(256), 0, stream, g);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<WM, WN, WAVES_M, false, 32>), grid, dim3(256), 0, stream, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs& g, bool b_nk, int64_t batch, hipStream_t stream) {
  if (g.M <= 0 || g.N <= 0 || batch <= 0) return hipSuccess;
  if (g.M <= 64) {
    // Shapes from a sweep at the decode batch (M = 32): [N][K] weights take 8
    // waves over K per 32 columns (16 when the grid alone would leave most
    // compute units idle); the [K][N] absorption weight takes 2 waves over K
    // times 4 over N per 128 columns (6.5 us for 128 heads, against 10.4 us
    // with 4 waves over K per 32 columns).
    const bool few = (int64_t)((g.N + 31) / 32) * ((g.M + 31) / 32) * batch < 256;
    if (b_nk && few) return launch_skinny<true, 16, 1, 4>(g, batch, stream);
    if (b_nk) return launch_skinny<true, 8, 1, 4>(g, batch, stream);
    return launch_skinny<false, 2, 4, 4>(g, batch, stream);
  }
  const bool aligned = ((reinterpret_cast<uintptr_t>(g.A) | reinterpret_cast<uintptr_t>(g.B) |
                         reinterpret_cast<uintptr_t>(g.C)) & 15) == 0 &&
                       (g.lda | g.ldb | g.ldc | g.sA | g.sB | g.sC) % 8 == 0 && g.N % 8 == 0 &&
                       (g.cp_dst == nullptr || ((reinterpret_cast<uintptr_t>(g.cp_src) |
                                                 reinterpret_cast<uintptr_t>(g.cp_dst)) & 15) == 0);
  if (!b_nk && g.K <= 128 && aligned) {
    // the absorption's short K: one workgroup per 128 rows of a batch entry, walking all of N
    const int64_t wgs = (g.M + 127) / 128 * batch;
    hipLaunchKernelGGL((gemm_kn_walk_kernel<128, WALK_BN>), dim3((unsigned)wgs), dim3(256), 0, stream, g);
    return hipGetLastError();
  }
  return launch_tiles<2, 2, 2>(g, b_nk, batch, stream);                  // 128 x 128 tiles
}

}  // namespace dsa

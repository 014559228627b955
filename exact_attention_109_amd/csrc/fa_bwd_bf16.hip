// Attention backward for bf16 inputs on gfx950 (MI355X), by recomputation.
//
// "Flash-Attention" (Awesome System Papers Wiki), core-idea section: the
// backward pass does not keep the N x N probability matrix; it rebuilds the
// probabilities from Q, K, V and per-row statistics saved by the forward
// pass, trading extra arithmetic for memory and HBM traffic. With
// P_ij = exp(scale * q_i.k_j - lse_i) over the allowed keys:
//     dV = P^T dO,   dP = dO V^T,   dS = P o (dP - D),   D_i = <dO_i, O_i>
//     dQ = scale * dS K,   dK = scale * dS^T Q
// (textbook derivatives of the forward definition; the pages give none).
//
// Three kernels on one stream, no atomics (deterministic):
//  * pre:  D_i and lse_i*log2(e) for every query row (HBM-bound pass over O, dO).
//  * dkdv: one workgroup of 8 waves per (batch, key/value head, 128-key
//          tile); the two waves of each SIMD share 32 keys: one keeps K as
//          its MFMA operand and forms S = Q K^T, P and dV^T += dO^T P, the
//          other keeps V and forms dP = dO V^T, dS = P (dP - D) and
//          dK^T += Q^T dS, with P handed over through LDS, so that one's
//          exponentials run beside the other's MFMAs. The query blocks of
//          every query head of the group stream past through LDS (dO and Q
//          read transposed with ds_read_b64_tr_b16 for dV and dK).
//  * dq:   one workgroup of 8 waves per (batch, query head, 256-query tile);
//          each wave owns 32 queries (Q and dO as register operands) while
//          the K/V blocks stream through a 3-deep LDS ring by LDS-DMA:
//          S^T = K Q^T, dP^T = V dO^T, dS^T, then dQ^T += K^T dS^T with K
//          read transposed. Two groups of four waves run in opposite phases
//          (one barrier at each phase boundary), so one group's MFMAs run
//          beside the other group's vector work on every SIMD.
// The accumulator layouts are arranged so that P and dS leave the MFMA
// accumulators already in the k-layout of the next contraction's B operand
// (see row_of_lane), and every LDS tile uses one XOR swizzle that is free of
// bank conflicts for both its row reads and its transposed reads.

#include <climits>
#include <type_traits>

#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kThreads = 256;

// 16-byte chunk swizzle shared by the row reads (16 lanes read the rows
// row_of_lane(0..15) at one logical chunk) and the transposed reads (a phase
// reads 4 consecutive rows x 64 bytes) of a bf16 tile.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 1) | ((row >> 3) & 2);
  else return (((row >> 1) & 1) << 2) | (((row >> 2) & 1) << 1) | ((row >> 4) & 1);
}

template <int D, int BLOCK = 64>
struct BwdCfg {
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int CPR = D / 8;          // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;       // rows per 1 KiB LDS-DMA instruction
  static constexpr int KST = D / 16;         // MFMA k-steps over the head dimension
  static constexpr int DSUB = D / 32;        // 32-column output subtiles
  static constexpr int BLK = BLOCK;          // rows (queries or keys) per streamed block: 32 or 64
  static constexpr int NSUB = BLK / 32;      // 32-row subtiles of a block
  static constexpr int STEPS = BLK / 16;     // MFMA k-steps over a block
  static constexpr int TILE_BYTES = BLK * D * 2;
  static constexpr int DMA_PER_WAVE = TILE_BYTES / 1024 / 4;
};

// Per-lane offsets for the row reads (A operand with rows row_of_lane(col),
// chunk (D/16)*half + t; subtile n adds 32 rows) and the transposed reads
// (rows 16*half + j/4 + 4r, columns 32s + 16*((lane%32)/16) + 4*(j%4),
// j = lane%16; block step u adds 32*(u/2) + 8*(u%2) rows).
template <int D>
struct ReadOffsets {
  int row[BwdCfg<D>::KST];
  int tr[BwdCfg<D>::DSUB][2];
  __device__ __forceinline__ void init(int lane) {
    using C = BwdCfg<D>;
    const int col = lane & 31, half = lane >> 5;
    const int r = row_of_lane(col);
#pragma unroll
    for (int t = 0; t < C::KST; ++t) row[t] = r * C::ROW_BYTES + ((((D / 16) * half + t) ^ swz<D>(r)) * 16);
    const int j16 = lane & 15, vgrp = (lane & 31) >> 4;
#pragma unroll
    for (int s = 0; s < C::DSUB; ++s)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int tr_row = 16 * half + (j16 >> 2) + 4 * q;
        const int cc = 32 * s + 16 * vgrp + 4 * (j16 & 3);
        tr[s][q] = tr_row * C::ROW_BYTES + (((cc >> 3) ^ swz<D>(tr_row)) * 16) + (cc & 7) * 2;
      }
  }
};

// ---------------------------------------------------------------------------
// pre: D_i = <dO_i, O_i>, L2_i = lse_i * log2(e)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_pre_kernel(const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO,
                                                           const float* __restrict__ LSE, float* __restrict__ Dl,
                                                           float* __restrict__ L2, long long rows) {
  constexpr int TPR = D / 8;                // threads per row, 8 elements (16 bytes) each
  constexpr int RPB = kThreads / TPR;       // rows per workgroup
  const int tid = threadIdx.x;
  const long long row = (long long)blockIdx.x * RPB + tid / TPR;
  const int part = tid % TPR;
  const long long rc = row < rows ? row : rows - 1;
  const u32x4 o = ld_global16(O + rc * D + part * 8);
  const u32x4 g = ld_global16(dO + rc * D + part * 8);
  float acc = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    acc = fmaf(__uint_as_float(o[w] << 16), __uint_as_float(g[w] << 16), acc);
    acc = fmaf(__uint_as_float(o[w] & 0xffff0000u), __uint_as_float(g[w] & 0xffff0000u), acc);
  }
#pragma unroll
  for (int m = 1; m < TPR; m <<= 1) acc += __shfl_xor(acc, m);
  if (row < rows && part == 0) {
    Dl[row] = acc;
    L2[row] = LSE[row] * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// Shared pieces of the two main kernels
// ---------------------------------------------------------------------------
// sched_group_barrier instruction classes
constexpr int kSgMfma = 0x008;
constexpr int kSgDsRead = 0x100;

// MFMA-phase schedule: `ahead` LDS reads first, then one read behind each
// MFMA (so each operand arrives several MFMAs before it is used).
template <int NMFMA, int READS_PER_MFMA, int AHEAD>
__device__ __forceinline__ void schedule_mfma_reads() {
  __builtin_amdgcn_sched_group_barrier(kSgDsRead, AHEAD, 0);
#pragma unroll
  for (int i = 0; i < NMFMA; ++i) {
    __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSgDsRead, READS_PER_MFMA, 0);
  }
}
constexpr int kKeysPerWg = 128;  // keys per dK/dV workgroup: 4 wave pairs x 32 keys

// ---------------------------------------------------------------------------
// dK, dV with wave pairs (two waves per SIMD)
// ---------------------------------------------------------------------------
// One workgroup of 8 waves per (batch, key/value head, 128-key tile). Waves w
// and w + 4 (w = 0..3) run on the same SIMD and own the same 32 keys:
//   P wave  (w):     S = Q K^T, P = exp2(S c - L2) (masked), dV^T += dO^T P
//   dS wave (w + 4): dP = dO V^T, dS = P (dP - D), dK^T += Q^T dS
// P goes from the P wave to its dS wave through LDS lane for lane (both waves
// compute their scores in the same accumulator layout, so lane l register i of
// one is lane l register i of the other), as the bf16 pairs the dV product
// takes: half the LDS bytes of float32, and dS = P (dP - D) is rounded to bf16
// for its own product anyway, so the extra rounding of P is of the same order.
// Two ticks per query block j, each ended by a workgroup barrier:
//   tick 1: P wave:  S(j), then P(j) and its hand-over (vector work);
//           dS wave: dK += Q(j-1)^T dS(j-1), then dP(j)          (MFMA)
//   tick 2: P wave:  dV += dO(j)^T P(j)                            (MFMA);
//           dS wave: dS(j) (vector work), LDS-DMA of block j+2, wait for j+1
// so on each SIMD one wave's contractions run while the other does its
// vector work, with the four contractions per block of the textbook
// backward. Each wave keeps one 32-key operand and one accumulator set, about
// half the registers of a wave that owns both, which is what lets two waves
// share a SIMD. Query blocks are streamed from the last one down, so the
// workgroups of all key tiles of a head start on the same block (shared
// through L2) instead of each at its own diagonal.
constexpr int kPairThreads = 512;
constexpr int kPairRing = 3;  // Q / dO / vector buffers: blocks j-1 (dK of the dS wave), j, j+1; j+2 loads into j-1's

// s_waitcnt lgkmcnt(0) (vmcnt and expcnt left at their maxima): this wave's
// LDS writes are complete.
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kPairThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dkdv_pair_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ L2, const float* __restrict__ Dl,
    float* __restrict__ dK, float* __restrict__ dV, int H_q, int H_kv, int N_q, int N_kv, int n_ktiles,
    int xcd_remap, float c, float scale, int paired) {
  using C = BwdCfg<D>;
  constexpr int BQ = C::BLK;
  constexpr int DPW = C::DMA_PER_WAVE;   // 1 KiB pieces of a tile per loading (dS) wave
  __shared__ __attribute__((aligned(1024))) uint8_t qs[kPairRing][C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t os[kPairRing][C::TILE_BYTES];
  __shared__ __attribute__((aligned(256))) float vecs[kPairRing][2][BQ];  // [buffer][L2, D][query]
  __shared__ __attribute__((aligned(1024))) u32x4 pex[4][C::STEPS][64];   // [pair][packed P register][lane], bf16

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pw = wave & 3;         // pair index = 32-key sub-tile = SIMD
  const bool is_ds = wave >= 4;    // wave-uniform role
  const int G = H_q / H_kv;

  // Causal: a workgroup takes key tiles r and n-1-r of one head (tile r has
  // the most query blocks to visit), so that every workgroup costs the same.
  const int n_units = paired ? (n_ktiles + 1) / 2 : n_ktiles;
  const TileAssign ta = assign_tile(blockIdx.x, n_units, 1, xcd_remap);
  const int b = ta.kvidx / H_kv;
  const int hk = ta.kvidx % H_kv;
  const int rank2 = n_ktiles - 1 - ta.tile_rank;
  // The tile body is inlined twice rather than looped: a loop around it kept
  // values of the first tile alive through the second and spilled registers.
  auto do_tile = [&](const int tile_rank) __attribute__((always_inline)) {
  int lane_t = tid & 63;
  asm volatile("" : "+v"(lane_t));  // per-lane values are recomputed per tile, not kept across both
  const int lane = lane_t;
  const int col = lane & 31;
  const int half = lane >> 5;
  const int k0 = tile_rank * kKeysPerWg;
  const int kw = k0 + 32 * pw;     // first key of this pair
  const int key = kw + col;        // this lane's key (MFMA column)
  const size_t kvbase = (size_t(b) * H_kv + hk) * size_t(N_kv) * D;

  // This wave's B operand over the head dimension: K (P wave) or V (dS
  // wave) of its 32 keys.
  bf16x8 kv[C::KST];
  {
    const uint16_t* src = is_ds ? V : K;
    const size_t off = kvbase + size_t(min(key, N_kv - 1)) * D + half * (D / 2);
#pragma unroll
    for (int t = 0; t < C::KST; ++t) kv[t] = as_bf16x8(ld_global16(src + off + 8 * t));
  }
  // (no wait here: these loads stay in flight with the prologue's LDS-DMA.
  // Vector-memory operations retire in order, so the compiler's own waits
  // for kv, which do not count the DMA, are only ever stricter than needed,
  // and the prologue's barrier waits for everything.)

  const int qstart = CAUSAL ? (k0 / BQ) * BQ : 0;
  const int nqb = qstart < N_q ? (N_q - qstart + BQ - 1) / BQ : 0;
  const int nblk = G * nqb;

  // A head's query blocks from the last one down; the lighter key tile of a
  // causal pair, which runs second, from its diagonal up, so that the
  // workgroups of a head read each block at the same step (5 % fewer HBM
  // reads than restarting at the last block, at the same speed).
  const bool asc = paired && 2 * tile_rank > n_ktiles - 1;
  auto block_head = [&](int jb, int& h, int& qb0) __attribute__((always_inline)) {
    const int g = jb / nqb;
    h = hk * G + g;
    qb0 = qstart + (asc ? jb % nqb : nqb - 1 - jb % nqb) * BQ;
  };

  // LDS-DMA of a block by the 4 dS waves: each loads DPW 1 KiB pieces of the
  // Q and of the dO tile; dS waves 0 and 1 also load the 64 L2 and D values.
  // The partial last block of a head reads row N_q - 1 for the rows past it.
  const int tail_q0 = (N_q % BQ) ? N_q - N_q % BQ : -1;
  const int tail_lim = (N_q - 1) % BQ;
  uint32_t doff[DPW], doff_t[DPW];
#pragma unroll
  for (int i = 0; i < DPW; ++i) {
    const int ig = pw * DPW + i;
    const int row = C::RPI * ig + lane / C::CPR;
    const int pch = lane % C::CPR;
    doff[i] = row * C::ROW_BYTES + (pch ^ swz<D>(row)) * 16;
    doff_t[i] = doff[i] - (row - min(row, tail_lim)) * C::ROW_BYTES;
  }
  const uint32_t voff = lane * 4, voff_t = min(lane, tail_lim) * 4;
  const float* vsrc = pw == 0 ? L2 : Dl;
  auto dma_slot = [&](int i, int jb, int bf) __attribute__((always_inline)) {
    int h, qb0;
    block_head(jb, h, qb0);
    const size_t rbase = (size_t(b) * H_q + h) * size_t(N_q);
    const bool tail = qb0 == tail_q0;
    if (i < 2 * DPW) {
      const bool is_q = i < DPW;
      const int ii = is_q ? i : i - DPW;
      const uint8_t* src = reinterpret_cast<const uint8_t*>((is_q ? Q : dO) + (rbase + qb0) * D);
      lds_dma16_sbase_nc(src, tail ? doff_t[ii] : doff[ii],
                         lds_address(is_q ? qs[bf] : os[bf]) + 1024 * (pw * DPW + ii));
    } else {
      lds_dma4_sbase_nc(vsrc + rbase + qb0, tail ? voff_t : voff, lds_address(&vecs[bf][pw][0]));
    }
  };
  // DMA instructions per dS wave and block: waves 0 and 1 add a vector load
  const int n_slots = 2 * DPW + (pw < 2 ? 1 : 0);
  auto dma_block = [&](int jb, int bf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2 * DPW; ++i) dma_slot(i, jb, bf);
    if (pw < 2) dma_slot(2 * DPW, jb, bf);
  };

  ReadOffsets<D> ro;
  ro.init(lane);

  auto need_mask = [&](int jb) __attribute__((always_inline)) {
    int h, qb0;
    block_head(jb, h, qb0);
    (void)h;
    return (CAUSAL && qb0 < kw + 31) || (qb0 + BQ > N_q);
  };
  // Scores of block jb that no query may attend (query before this lane's
  // key, or past N_q) become -inf, so that P, and with it dS, are exactly 0.
  auto mask_scores = [&](int jb, f32x16 (&sx)[C::NSUB]) __attribute__((always_inline)) {
    int h, qb0;
    block_head(jb, h, qb0);
    (void)h;
    const int lo = CAUSAL ? key - qb0 - 16 * half : INT_MIN;
    const int hi = N_q - 1 - qb0 - 16 * half;
#pragma unroll
    for (int n = 0; n < C::NSUB; ++n)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (32 * n + i < lo || 32 * n + i > hi) sx[n][i] = -INFINITY;
  };
  // 16 MFMAs: acc[n] = rows of tile t_rows (Q or dO, rows from LDS) times kv
  auto rows_times_kv = [&](const uint8_t* tile, f32x16 (&acc)[C::NSUB]) __attribute__((always_inline)) {
#pragma unroll
    for (int n = 0; n < C::NSUB; ++n) acc[n] = f32x16{};
#pragma unroll
    for (int t = 0; t < C::KST; ++t)
#pragma unroll
      for (int n = 0; n < C::NSUB; ++n)
        acc[n] = mfma32x32x16(as_bf16x8(*reinterpret_cast<const u32x4*>(tile + ro.row[t] + n * 32 * C::ROW_BYTES)),
                              kv[t], acc[n]);
  };
  // 16 MFMAs: out[s] += tile^T (transposed reads) times the packed block operand
  auto tileT_times = [&](const uint8_t* tile, const u32x4 (&pk)[C::STEPS], f32x16 (&out)[C::DSUB])
      __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < C::STEPS; ++u) {
      const int rb = (32 * (u >> 1) + 8 * (u & 1)) * C::ROW_BYTES;
#pragma unroll
      for (int s = 0; s < C::DSUB; ++s)
        out[s] = mfma32x32x16(lds_read_tr8(tile + ro.tr[s][0] + rb, tile + ro.tr[s][1] + rb), as_bf16x8(pk[u]), out[s]);
    }
  };
  constexpr int NX = C::KST * C::NSUB;   // MFMAs of one rows_times_kv
  constexpr int NZ = C::STEPS * C::DSUB; // MFMAs of one tileT_times

  f32x16 acc[C::DSUB];  // dV^T (P wave) or dK^T (dS wave): lane = key, registers = head-dimension columns
#pragma unroll
  for (int s = 0; s < C::DSUB; ++s) acc[s] = f32x16{};

  // ---- prologue: blocks 0 and 1 into buffers 0 and 1
  if (is_ds && nblk > 0) {
    dma_block(0, 0);
    dma_block(min(1, nblk - 1), 1);
    wait_vmem();
  }
  __syncthreads();

  if (!is_ds) {
    // ------------------------------------------------------------ P wave
    f32x16 sx[C::NSUB];
    u32x4 pk[C::STEPS];
    // block j in ring buffer BF (a compile-time constant, so that every LDS
    // address is a per-lane offset plus an immediate)
    auto p_block = [&](int j, auto bfc) __attribute__((always_inline)) {
      constexpr int BF = decltype(bfc)::value;
      // tick 1: S(j), P(j), hand-over
      __builtin_amdgcn_s_setprio(1);  // S(j) first: the vector work after it is this tick's longer side
      __builtin_amdgcn_sched_barrier(0);
      rows_times_kv(qs[BF], sx);
      schedule_mfma_reads<NX - 4, 1, 4>();
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
      if (need_mask(j)) mask_scores(j, sx);
      const float* lt = vecs[BF][0];
#pragma unroll
      for (int n = 0; n < C::NSUB; ++n) {
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          const f32x4 a = *reinterpret_cast<const f32x4*>(lt + 32 * n + 16 * half + 4 * v4);
          f32x4 pv;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pv[e] = fast_exp2(fmaf(sx[n][4 * v4 + e], c, -a[e]));
            sx[n][4 * v4 + e] = pv[e];
          }
        }
#pragma unroll
        for (int w = 0; w < 2; ++w) {
#pragma unroll
          for (int e = 0; e < 4; ++e) pk[2 * n + w][e] = cvt_pk_bf16(sx[n][8 * w + 2 * e], sx[n][8 * w + 2 * e + 1]);
          pex[pw][2 * n + w][lane] = pk[2 * n + w];  // the hand-over: P in bf16, as the dV product uses it
        }
      }
      // P(j) is packed in this tick: left alone, the compiler sinks the
      // packing past the barrier into the dV MFMAs of the next one
#pragma unroll
      for (int u = 0; u < C::STEPS; ++u) asm volatile("" : "+v"(pk[u]));
      wait_lds();          // P(j) is in LDS before the barrier hands it over
      barrier_nofence();
      // tick 2: dV += dO(j)^T P(j)
      tileT_times(os[BF], pk, acc);
      schedule_mfma_reads<NZ - 4, 2, 8>();
      barrier_nofence();
    };
    for (int j = 0; j < nblk; j += kPairRing) {
      p_block(j, std::integral_constant<int, 0>{});
      if (j + 1 < nblk) p_block(j + 1, std::integral_constant<int, 1>{});
      if (j + 2 < nblk) p_block(j + 2, std::integral_constant<int, 2>{});
    }
    if (key < N_kv) {
      float* dvp = dV + kvbase + size_t(key) * D;
#pragma unroll
      for (int s = 0; s < C::DSUB; ++s)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          f32x4 vv;
#pragma unroll
          for (int e = 0; e < 4; ++e) vv[e] = acc[s][4 * a + e];
          *reinterpret_cast<f32x4*>(dvp + 32 * s + 8 * a + 4 * half) = vv;
        }
    }
  } else {
    // ----------------------------------------------------------- dS wave
    f32x16 px[C::NSUB];
    u32x4 sk[C::STEPS];
    auto ds_block = [&](int j, auto bfc) __attribute__((always_inline)) {
      constexpr int BF = decltype(bfc)::value;
      constexpr int BFP = (BF + kPairRing - 1) % kPairRing;  // block j-1, and j+2's DMA target
      // tick 1: dK += Q(j-1)^T dS(j-1), dP(j)
      if (j >= 1) {
        tileT_times(qs[BFP], sk, acc);
        schedule_mfma_reads<NZ - 4, 2, 8>();
        __builtin_amdgcn_sched_barrier(0);
      }
      rows_times_kv(os[BF], px);
      schedule_mfma_reads<NX - 4, 1, 4>();
      barrier_nofence();
      // tick 2: dS(j) = P(j) (dP(j) - D), DMA of block j+2, wait for block j+1
      const int jd = min(j + 2, nblk - 1);  // past the end: a harmless reload into a free buffer
      const float* dt = vecs[BF][1];
#pragma unroll
      for (int n = 0; n < C::NSUB; ++n) {
        const u32x4 pb[2] = {pex[pw][2 * n][lane], pex[pw][2 * n + 1][lane]};
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(dt + 32 * n + 16 * half + 4 * v4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // score 4 v4 + e of the subtile: packed register v4/2, pair 2 (v4%2) + e/2, half e%2
            const uint32_t w2 = pb[v4 >> 1][2 * (v4 & 1) + (e >> 1)];
            const float pv = __uint_as_float((e & 1) ? (w2 & 0xffff0000u) : (w2 << 16));
            px[n][4 * v4 + e] = pv * (px[n][4 * v4 + e] - d4[e]);
          }
          const int slot = 4 * n + v4;
          if (slot < 2 * DPW) dma_slot(slot, jd, BFP);
        }
#pragma unroll
        for (int w = 0; w < 2; ++w)
#pragma unroll
          for (int e = 0; e < 4; ++e) sk[2 * n + w][e] = cvt_pk_bf16(px[n][8 * w + 2 * e], px[n][8 * w + 2 * e + 1]);
      }
      // dS(j) is formed in this tick, beside the partner's dV MFMAs
#pragma unroll
      for (int u = 0; u < C::STEPS; ++u) asm volatile("" : "+v"(sk[u]));
#pragma unroll
      for (int slot = 4 * C::NSUB; slot < 2 * DPW; ++slot) dma_slot(slot, jd, BFP);
      if (pw < 2) {
        dma_slot(2 * DPW, jd, BFP);
        wait_vmem_keep<2 * DPW + 1>();   // block j+1 (loaded during block j-1) is in LDS
      } else {
        wait_vmem_keep<2 * DPW>();
      }
      barrier_nofence();
    };
    int j = 0;
    for (; j + kPairRing <= nblk; j += kPairRing) {
      ds_block(j, std::integral_constant<int, 0>{});
      ds_block(j + 1, std::integral_constant<int, 1>{});
      ds_block(j + 2, std::integral_constant<int, 2>{});
    }
    // the remaining 0-2 blocks, then dK of the last block
    if (j < nblk) ds_block(j, std::integral_constant<int, 0>{});
    if (j + 1 < nblk) ds_block(j + 1, std::integral_constant<int, 1>{});
    if (nblk > 0) {
      const int bl = (nblk - 1) % kPairRing;
      if (bl == 0) tileT_times(qs[0], sk, acc);
      else if (bl == 1) tileT_times(qs[1], sk, acc);
      else tileT_times(qs[2], sk, acc);
    }
    wait_vmem();  // the reloads past the end land before the workgroup's LDS is released
    if (key < N_kv) {
      float* dkp = dK + kvbase + size_t(key) * D;
#pragma unroll
      for (int s = 0; s < C::DSUB; ++s)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          f32x4 vk;
#pragma unroll
          for (int e = 0; e < 4; ++e) vk[e] = acc[s][4 * a + e] * scale;
          *reinterpret_cast<f32x4*>(dkp + 32 * s + 8 * a + 4 * half) = vk;
        }
    }
  }
  (void)n_slots;
  };
  do_tile(ta.tile_rank);
  if (paired && rank2 != ta.tile_rank) {
    barrier_nofence();  // every wave is done with the first tile's LDS
    do_tile(rank2);
  }
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
// dQ with two wave groups per workgroup in opposite phases (as the forward):
// 8 waves, 256 queries (32 per wave); waves w and w + 4 share a SIMD. Per key
// block j each wave runs an MFMA phase -- Z(j-1): dQ^T += K_{j-1}^T dS^T_{j-1},
// then X(j): S^T = K_j Q^T, dP^T = V_j dO^T -- and a vector phase Y(j): P,
// dS^T = P (dP - D), packed. Group B runs one phase behind group A, with a
// workgroup barrier at every phase boundary, so on each SIMD one wave drives
// the matrix core while the other does its vector work. Group B also loads
// the K/V block j+1 during its vector phase of block j into a 3-deep ring
// (block j-1 is still read by Z in block j) and waits for it at the end of
// its MFMA phase. (Two independent 4-wave workgroups per compute unit, whose
// phases drift freely, measured 1-3 % slower.)
constexpr int kDqWaves = 8;
constexpr int kDqThreads = 64 * kDqWaves;
constexpr int kDqRows = 32 * kDqWaves;  // queries per workgroup
constexpr int kDqRing = 3;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kDqThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ L2, const float* __restrict__ Dl,
    float* __restrict__ dQ, int H_q, int H_kv, int N_q, int N_kv, int n_qtiles, int xcd_remap, int B_heads,
    float c, float scale) {
  using C = BwdCfg<D>;
  constexpr int BK = C::BLK;
  constexpr int DPW = C::DMA_PER_WAVE;  // 1 KiB pieces per loader wave (4 loaders) and tile
  __shared__ __attribute__((aligned(1024))) uint8_t ks[kDqRing][C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vs[kDqRing][C::TILE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;  // 0: group A (leads), 1: group B (one phase behind, loads K/V)
  const int gw = wave & 3;
  const int col = lane & 31;
  const int half = lane >> 5;
  const int G = H_q / H_kv;

  const TileAssign ta = assign_tile(blockIdx.x, n_qtiles, G, xcd_remap, B_heads, true);
  const int b = ta.kvidx / H_kv;
  const int hk = ta.kvidx % H_kv;
  const int h = hk * G + ta.gq;
  const int tile = CAUSAL ? (n_qtiles - 1 - ta.tile_rank) : ta.tile_rank;  // heaviest first
  const int q0 = tile * kDqRows;
  const int wq0 = q0 + 32 * wave;
  const int query = wq0 + col;  // this lane's query (MFMA column)

  const size_t rbase = (size_t(b) * H_q + h) * size_t(N_q);
  const size_t kvbase = (size_t(b) * H_kv + hk) * size_t(N_kv) * D;
  const int qc = min(query, N_q - 1);
  bf16x8 qreg[C::KST], oreg[C::KST];
  {
    const size_t off = (rbase + qc) * D + half * (D / 2);
#pragma unroll
    for (int t = 0; t < C::KST; ++t) {
      qreg[t] = as_bf16x8(ld_global16(Q + off + 8 * t));
      oreg[t] = as_bf16x8(ld_global16(dO + off + 8 * t));
    }
  }
  const float l2 = L2[rbase + qc];
  const float dl = Dl[rbase + qc];
  // (no wait here: these loads stay in flight with the prologue's LDS-DMA;
  // see bwd_dkdv_pair_kernel)

  // key blocks of the workgroup; every wave runs all of them (blocks past a
  // wave's queries are masked to zero)
  const int nblk_all = (N_kv + BK - 1) / BK;
  int nblk = nblk_all;
  if (CAUSAL) nblk = min(nblk_all, (min(q0 + kDqRows, N_q) - 1) / BK + 1);

  const int tail_blk = (N_kv % BK) ? N_kv / BK : -1;
  const int tail_lim = (N_kv - 1) % BK;
  uint32_t doff[DPW], doff_t[DPW];
#pragma unroll
  for (int i = 0; i < DPW; ++i) {
    const int ig = gw * DPW + i;
    const int row = C::RPI * ig + lane / C::CPR;
    const int pch = lane % C::CPR;
    doff[i] = row * C::ROW_BYTES + (pch ^ swz<D>(row)) * 16;
    doff_t[i] = doff[i] - (row - min(row, tail_lim)) * C::ROW_BYTES;
  }
  const uint8_t* Kb = reinterpret_cast<const uint8_t*>(K + kvbase);
  const uint8_t* Vb = reinterpret_cast<const uint8_t*>(V + kvbase);
  constexpr int kSlots = 2 * DPW;
  auto dma_slot = [&](int i, int j, uint8_t* kdst, uint8_t* vdst) __attribute__((always_inline)) {
    const bool is_k = i < DPW;
    const int ii = is_k ? i : i - DPW;
    const uint8_t* src = (is_k ? Kb : Vb) + size_t(j) * BK * C::ROW_BYTES;
    lds_dma16_sbase_nc(src, j == tail_blk ? doff_t[ii] : doff[ii],
                       lds_address(is_k ? kdst : vdst) + 1024 * (gw * DPW + ii));
  };

  ReadOffsets<D> ro;
  ro.init(lane);

  f32x16 dq[C::DSUB];
#pragma unroll
  for (int s = 0; s < C::DSUB; ++s) dq[s] = f32x16{};
  f32x16 sA[C::NSUB], pA[C::NSUB];  // S^T, dP^T of the current block
  u32x4 sk[C::STEPS];                // dS^T (bf16)
  constexpr int NX = 2 * C::KST * C::NSUB;  // MFMAs of X
  constexpr int NZ = C::STEPS * C::DSUB;    // MFMAs of Z
  auto X = [&](const uint8_t* kt, const uint8_t* vt) __attribute__((always_inline)) {
#pragma unroll
    for (int n = 0; n < C::NSUB; ++n) {
      sA[n] = f32x16{};
      pA[n] = f32x16{};
    }
#pragma unroll
    for (int t = 0; t < C::KST; ++t) {
#pragma unroll
      for (int n = 0; n < C::NSUB; ++n) {
        const int o = ro.row[t] + n * 32 * C::ROW_BYTES;
        sA[n] = mfma32x32x16(as_bf16x8(*reinterpret_cast<const u32x4*>(kt + o)), qreg[t], sA[n]);
        pA[n] = mfma32x32x16(as_bf16x8(*reinterpret_cast<const u32x4*>(vt + o)), oreg[t], pA[n]);
      }
    }
    schedule_mfma_reads<NX - 4, 1, 4>();
  };
  // vector phase of block j; the loading group issues its DMA slots between
  // the exponentials (a burst would stall the wave for the whole transfer)
  auto Y = [&](int j, auto&& issue) __attribute__((always_inline)) {
    const int kv0 = j * BK;
    if ((CAUSAL && kv0 + BK - 1 > wq0) || (kv0 + BK > N_kv)) {
      const int last_key = CAUSAL ? min(query, N_kv - 1) : N_kv - 1;
      const int lim = last_key - j * BK - 16 * half;
#pragma unroll
      for (int n = 0; n < C::NSUB; ++n)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (32 * n + i > lim) sA[n][i] = -INFINITY;
    }
#pragma unroll
    for (int n = 0; n < C::NSUB; ++n) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = fast_exp2(fmaf(sA[n][i], c, -l2));
        pA[n][i] = pv * (pA[n][i] - dl);
        const int e = 16 * n + i;
        if (e % 3 == 1 && e / 3 < kSlots) issue(e / 3);
      }
#pragma unroll
      for (int w = 0; w < 2; ++w)
#pragma unroll
        for (int e = 0; e < 4; ++e) sk[2 * n + w][e] = cvt_pk_bf16(pA[n][8 * w + 2 * e], pA[n][8 * w + 2 * e + 1]);
    }
#pragma unroll
    for (int e = 32 * C::NSUB / 3 + 1; e < kSlots; ++e) issue(e);
    // dS is packed in this phase: left alone, the compiler sinks the packing
    // past the barrier into the MFMAs of the next one
#pragma unroll
    for (int u = 0; u < C::STEPS; ++u) asm volatile("" : "+v"(sk[u]));
  };
  auto Z = [&](const uint8_t* kt) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < C::STEPS; ++u) {
      const int rb = (32 * (u >> 1) + 8 * (u & 1)) * C::ROW_BYTES;
#pragma unroll
      for (int s = 0; s < C::DSUB; ++s) {
        const bf16x8 a = lds_read_tr8(kt + ro.tr[s][0] + rb, kt + ro.tr[s][1] + rb);
        dq[s] = mfma32x32x16(a, as_bf16x8(sk[u]), dq[s]);
      }
    }
    schedule_mfma_reads<NZ - 4, 2, 8>();
  };
  // MFMA phase of block j: Z(j-1) then X(j); block j lives in ring buffer BF
  // (a compile-time constant, so that LDS addresses are offsets plus
  // immediates)
  auto mfma_phase = [&](int j, auto bfc) __attribute__((always_inline)) {
    constexpr int BF = decltype(bfc)::value;
    constexpr int BFP = (BF + kDqRing - 1) % kDqRing;
    if (j >= 1) Z(ks[BFP]);
    __builtin_amdgcn_sched_barrier(0);
    if (j < nblk) X(ks[BF], vs[BF]);
  };
  auto no_dma = [](int) __attribute__((always_inline)) {};

  // prologue: block 0 into buffer 0
  if (grp == 1) {
#pragma unroll
    for (int i = 0; i < kSlots; ++i) dma_slot(i, 0, ks[0], vs[0]);
    wait_vmem();
  }
  __syncthreads();

  if (grp == 0) {
    auto a_block = [&](int j, auto bfc) __attribute__((always_inline)) {
      mfma_phase(j, bfc);
      barrier_nofence();
      if (j < nblk) Y(j, no_dma);
      barrier_nofence();
    };
    for (int j = 0; j <= nblk; j += kDqRing) {
      a_block(j, std::integral_constant<int, 0>{});
      if (j + 1 <= nblk) a_block(j + 1, std::integral_constant<int, 1>{});
      if (j + 2 <= nblk) a_block(j + 2, std::integral_constant<int, 2>{});
    }
  } else {
    // block 0: the load of block 1, then X(0)
    {
      const int jn = min(1, nblk - 1);
#pragma unroll
      for (int i = 0; i < kSlots; ++i) dma_slot(i, jn, ks[1], vs[1]);
      barrier_nofence();
      mfma_phase(0, std::integral_constant<int, 0>{});
      wait_vmem();
      barrier_nofence();
    }
    auto b_block = [&](int j, auto bfc) __attribute__((always_inline)) {
      constexpr int BF = decltype(bfc)::value;
      constexpr int BFN = (BF + 1) % kDqRing;  // block j+1 (the buffer of block j-2)
      const int jn = min(j + 1, nblk - 1);     // past the end: a harmless reload into a free buffer
      Y(j - 1, [&](int i) __attribute__((always_inline)) { dma_slot(i, jn, ks[BFN], vs[BFN]); });
      barrier_nofence();  // the DMA stays in flight through the next phase
      mfma_phase(j, bfc);
      wait_vmem();        // block j+1 is in LDS before the barrier publishes it
      barrier_nofence();
    };
    for (int j = 1; j <= nblk; j += kDqRing) {
      b_block(j, std::integral_constant<int, 1>{});
      if (j + 1 <= nblk) b_block(j + 1, std::integral_constant<int, 2>{});
      if (j + 2 <= nblk) b_block(j + 2, std::integral_constant<int, 0>{});
    }
  }

  if (query < N_q) {
    float* dqp = dQ + (rbase + query) * D;
#pragma unroll
    for (int s = 0; s < C::DSUB; ++s)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = dq[s][4 * a + e] * scale;
        *reinterpret_cast<f32x4*>(dqp + 32 * s + 8 * a + 4 * half) = v;
      }
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const BwdParams& p, hipStream_t stream) {
  const long long rows = (long long)p.B * p.H_q * p.N_q;
  float* Dl = p.delta;
  float* L2 = p.delta + rows;
  constexpr int RPB = kThreads / (D / 8);
  hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(p.o), static_cast<const uint16_t*>(p.dO), p.lse, Dl, L2, rows);
  // c > 0 keeps exp2(-inf)-style masking well defined; scale == 0 gives 1/count weights via the LSE
  const float c = fmaxf(p.scale * kLog2e, 1.17549435e-38f);
  const int xcd_remap = ((p.B * p.H_kv) % 8 == 0) ? 1 : 0;
  const int n_ktiles = (p.N_kv + kKeysPerWg - 1) / kKeysPerWg;
  const int paired = CAUSAL ? 1 : 0;
  const int n_units = paired ? (n_ktiles + 1) / 2 : n_ktiles;
  hipLaunchKernelGGL((bwd_dkdv_pair_kernel<D, CAUSAL>), dim3((unsigned)((long long)n_units * p.B * p.H_kv)),
                     dim3(kPairThreads), 0, stream, static_cast<const uint16_t*>(p.q), static_cast<const uint16_t*>(p.k),
                     static_cast<const uint16_t*>(p.v), static_cast<const uint16_t*>(p.dO), L2, Dl, p.dk, p.dv,
                     p.H_q, p.H_kv, p.N_q, p.N_kv, n_ktiles, xcd_remap, c, p.scale, paired);
  const int n_qtiles = (p.N_q + kDqRows - 1) / kDqRows;
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)((long long)n_qtiles * p.B * p.H_q)), dim3(kDqThreads),
                     0, stream, static_cast<const uint16_t*>(p.q), static_cast<const uint16_t*>(p.k),
                     static_cast<const uint16_t*>(p.v), static_cast<const uint16_t*>(p.dO), L2, Dl, p.dq, p.H_q,
                     p.H_kv, p.N_q, p.N_kv, n_qtiles, xcd_remap, p.B * p.H_q, c, p.scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t stream) {
  if (p.d == 128) return p.causal ? launch<128, true>(p, stream) : launch<128, false>(p, stream);
  return p.causal ? launch<64, true>(p, stream) : launch<64, false>(p, stream);
}

}  // namespace fa

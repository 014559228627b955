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
//  * dkdv: one workgroup per (batch, key/value head, 128-key tile); each wave
//          owns 32 keys and keeps their K and V as MFMA operands in
//          registers, while the query blocks of every query head of the
//          group stream past through LDS. Per 64-query block and wave:
//          S = Q K^T and dP = dO V^T (queries x keys, Q/dO rows read from LDS),
//          P and dS on the VALU, then dV^T += dO^T P and dK^T += Q^T dS with the
//          dO/Q operands read transposed (ds_read_b64_tr_b16). Software-
//          pipelined like dq below.
//  * dq:   one workgroup per (batch, query head, 128-query tile); each wave
//          owns 32 queries (Q and dO as register operands) while the K/V
//          blocks stream through LDS: S^T = K Q^T, dP^T = V dO^T, dS^T, then
//          dQ^T += K^T dS^T with K read transposed. Two workgroups share a
//          compute unit (240 registers per wave, 64 KiB of LDS each), so the
//          MFMAs of one wave run beside the vector work of the other wave on
//          its SIMD; K/V of block j+1 arrive by LDS-DMA while block j is
//          processed.
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
constexpr int kNBuf = 4;  // LDS buffers of the dK/dV kernel's streamed blocks: two in use, two loading

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
// ---------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------
constexpr int kKeysPerWg = 128;  // 4 waves x 32 keys

// Per wave (32 keys, K and V as register operands) and streamed query block
// jb (64 queries of one query head):
//   X(jb): S = Q K^T, dP = dO V^T                      (MFMA, Q/dO rows from LDS)
//   Y(jb): P = exp2(S c - L2), dS = P (dP - D), packed  (VALU)
//   Z(jb): dV^T += dO^T P, dK^T += Q^T dS               (MFMA, Q/dO read transposed)
// Iteration jb runs Y(jb) interleaved with X(jb+1) (S/dP double-buffered),
// then Z(jb); the LDS-DMA of block jb+3 is issued between the vector work.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ L2, const float* __restrict__ Dl,
    float* __restrict__ dK, float* __restrict__ dV, int H_q, int H_kv, int N_q, int N_kv, int n_ktiles,
    int xcd_remap, float c, float scale) {
  using C = BwdCfg<D>;
  constexpr int BQ = C::BLK;
  constexpr int DPW = C::DMA_PER_WAVE;
  __shared__ __attribute__((aligned(1024))) uint8_t qs[kNBuf][C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t os[kNBuf][C::TILE_BYTES];
  __shared__ __attribute__((aligned(256))) float vecs[kNBuf][2][BQ];  // [buffer][L2, D][query]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int half = lane >> 5;
  const int G = H_q / H_kv;

  // key tiles: the first ones see the most queries when causal, so they go first
  const TileAssign ta = assign_tile(blockIdx.x, n_ktiles, 1, xcd_remap);
  const int b = ta.kvidx / H_kv;
  const int hk = ta.kvidx % H_kv;
  const int k0 = ta.tile_rank * kKeysPerWg;
  const int kw = k0 + 32 * wave;   // first key of this wave
  const int key = kw + col;        // this lane's key (MFMA column)

  const size_t kvbase = (size_t(b) * H_kv + hk) * size_t(N_kv) * D;
  // K and V of this wave's 32 keys as B operands (k = head dimension)
  bf16x8 kreg[C::KST], vreg[C::KST];
  {
    const size_t off = kvbase + size_t(min(key, N_kv - 1)) * D + half * (D / 2);
#pragma unroll
    for (int t = 0; t < C::KST; ++t) {
      kreg[t] = as_bf16x8(ld_global16(K + off + 8 * t));
      vreg[t] = as_bf16x8(ld_global16(V + off + 8 * t));
    }
    // only MFMAs read these: keep them in AGPRs, out of the vector work's way
#pragma unroll
    for (int t = 0; t < C::KST; ++t) asm volatile("" : "+a"(kreg[t]), "+a"(vreg[t]));
  }
  wait_vmem();  // the LDS-DMA below is not tracked by the compiler's waits

  // query blocks: for each of the G query heads, blocks from qstart to N_q.
  // Every wave runs every block of the workgroup (blocks before a wave's keys
  // are masked to zero).
  const int qstart = CAUSAL ? (k0 / BQ) * BQ : 0;
  const int nqb = qstart < N_q ? (N_q - qstart + BQ - 1) / BQ : 0;
  const int nblk = G * nqb;

  // LDS-DMA of a block: per-lane offsets within a tile, and clamped ones for
  // the partial last block of a head (rows past N_q repeat row N_q - 1).
  const int tail_q0 = (N_q % BQ) ? N_q - N_q % BQ : -1;
  const int tail_lim = (N_q - 1) % BQ;
  uint32_t doff[DPW], doff_t[DPW];
#pragma unroll
  for (int i = 0; i < DPW; ++i) {
    const int ig = wave * DPW + i;
    const int row = C::RPI * ig + lane / C::CPR;
    const int pch = lane % C::CPR;
    doff[i] = row * C::ROW_BYTES + (pch ^ swz<D>(row)) * 16;
    doff_t[i] = doff[i] - (row - min(row, tail_lim)) * C::ROW_BYTES;
  }
  const uint32_t voff = lane * 4, voff_t = min(lane, tail_lim) * 4;
  const float* vsrc = (wave & 1) ? Dl : L2;  // waves 0, 2: L2; waves 1, 3: D (same bytes twice)

  auto block_head = [&](int jb, int& h, int& qb0) __attribute__((always_inline)) {
    const int g = jb / nqb;
    h = hk * G + g;
    qb0 = qstart + (jb % nqb) * BQ;
  };
  // DMA slot i of block jb into buffer bf: Q pieces, dO pieces, then the vector.
  constexpr int kSlots = 2 * DPW + 1;
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
                         lds_address(is_q ? qs[bf] : os[bf]) + 1024 * (wave * DPW + ii));
    } else {
      lds_dma4_sbase_nc(vsrc + rbase + qb0, tail ? voff_t : voff, lds_address(&vecs[bf][wave & 1][0]));
    }
  };

  ReadOffsets<D> ro;
  ro.init(lane);

  f32x16 dk[C::DSUB], dv[C::DSUB];
#pragma unroll
  for (int s = 0; s < C::DSUB; ++s) {
    dk[s] = f32x16{};
    dv[s] = f32x16{};
  }
  f32x16 sA[C::NSUB], pA[C::NSUB], sB[C::NSUB], pB[C::NSUB];  // S, dP of two blocks
  u32x4 pk[C::STEPS], sk[C::STEPS];                            // P, dS (bf16) of the current block

  constexpr int NX = 2 * C::KST * C::NSUB;    // MFMAs of X
  constexpr int NZ = 2 * C::STEPS * C::DSUB;  // MFMAs of Z
  auto X = [&](int bf, f32x16 (&sx)[C::NSUB], f32x16 (&px)[C::NSUB]) __attribute__((always_inline)) {
    const uint8_t* qt = qs[bf];
    const uint8_t* ot = os[bf];
#pragma unroll
    for (int n = 0; n < C::NSUB; ++n) {
      sx[n] = f32x16{};
      px[n] = f32x16{};
    }
#pragma unroll
    for (int t = 0; t < C::KST; ++t) {
#pragma unroll
      for (int n = 0; n < C::NSUB; ++n) {
        const int o = ro.row[t] + n * 32 * C::ROW_BYTES;
        sx[n] = mfma32x32x16(as_bf16x8(*reinterpret_cast<const u32x4*>(qt + o)), kreg[t], sx[n]);
        px[n] = mfma32x32x16(as_bf16x8(*reinterpret_cast<const u32x4*>(ot + o)), vreg[t], px[n]);
      }
    }
  };
  // Scores of block jb that no query may attend (query before this lane's
  // key, or past N_q) become -inf, so that P and dS are exactly 0 there.
  auto mask_scores = [&](int jb, f32x16 (&sx)[C::NSUB]) __attribute__((always_inline)) {
    int h, qb0;
    block_head(jb, h, qb0);
    (void)h;
    // query 32n + 16*half + i of the block is visible iff lo <= 32n + i <= hi
    const int lo = CAUSAL ? key - qb0 - 16 * half : INT_MIN;
    const int hi = N_q - 1 - qb0 - 16 * half;
#pragma unroll
    for (int n = 0; n < C::NSUB; ++n)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (32 * n + i < lo || 32 * n + i > hi) sx[n][i] = -INFINITY;
  };
  // Y(jb) on (s, p) from buffer bfy -> (pk, sk); with WITH_X also X(jb+1)
  // from buffer bfx into (sx, px) and the DMA of block jd into buffer bfd.
  auto YX = [&](auto with_x, int bfy, f32x16 (&s)[C::NSUB], f32x16 (&p)[C::NSUB], int bfx,
                f32x16 (&sx)[C::NSUB], f32x16 (&px)[C::NSUB], int jd, int bfd) __attribute__((always_inline)) {
    constexpr bool WITH_X = decltype(with_x)::value;
    if constexpr (WITH_X) X(bfx, sx, px);
    const float* lt = vecs[bfy][0];
    const float* dt = vecs[bfy][1];
#pragma unroll
    for (int n = 0; n < C::NSUB; ++n) {
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(lt + 32 * n + 16 * half + 4 * v4);
        const f32x4 d = *reinterpret_cast<const f32x4*>(dt + 32 * n + 16 * half + 4 * v4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * v4 + e;
          const float pv = fast_exp2(fmaf(s[n][i], c, -a[e]));
          s[n][i] = pv;
          p[n][i] = pv * (p[n][i] - d[e]);
          if constexpr (WITH_X) {
            const int el = 16 * n + i;
            if (el % 3 == 1 && el / 3 < kSlots) dma_slot(el / 3, jd, bfd);
          }
        }
      }
#pragma unroll
      for (int w = 0; w < 2; ++w)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pk[2 * n + w][e] = cvt_pk_bf16(s[n][8 * w + 2 * e], s[n][8 * w + 2 * e + 1]);
          sk[2 * n + w][e] = cvt_pk_bf16(p[n][8 * w + 2 * e], p[n][8 * w + 2 * e + 1]);
        }
    }
    if constexpr (WITH_X) {
#pragma unroll
      for (int e = 16 * C::NSUB / 3 + 1; e < kSlots; ++e) dma_slot(e, jd, bfd);
    }
  };
  auto Z = [&](int bf) __attribute__((always_inline)) {
    const uint8_t* qt = qs[bf];
    const uint8_t* ot = os[bf];
#pragma unroll
    for (int u = 0; u < C::STEPS; ++u) {
      const int rb = (32 * (u >> 1) + 8 * (u & 1)) * C::ROW_BYTES;
#pragma unroll
      for (int s = 0; s < C::DSUB; ++s) {
        const bf16x8 ao = lds_read_tr8(ot + ro.tr[s][0] + rb, ot + ro.tr[s][1] + rb);
        dv[s] = mfma32x32x16(ao, as_bf16x8(pk[u]), dv[s]);
        const bf16x8 aq = lds_read_tr8(qt + ro.tr[s][0] + rb, qt + ro.tr[s][1] + rb);
        dk[s] = mfma32x32x16(aq, as_bf16x8(sk[u]), dk[s]);
      }
    }
    schedule_mfma_reads<NZ - 4, 2, 8>();
  };
  auto need_mask = [&](int jb) __attribute__((always_inline)) {
    int h, qb0;
    block_head(jb, h, qb0);
    (void)h;
    return (CAUSAL && qb0 < kw + 31) || (qb0 + BQ > N_q);
  };
  // iteration jb (< nblk - 1): Y(jb) on (s, p) with X(jb+1) into (sx, px), then Z(jb)
  auto iteration = [&](int jb, f32x16 (&s)[C::NSUB], f32x16 (&p)[C::NSUB], f32x16 (&sx)[C::NSUB],
                       f32x16 (&px)[C::NSUB]) __attribute__((always_inline)) {
    const int jd = min(jb + 3, nblk - 1);  // past the end: a harmless reload into a free buffer
    if (need_mask(jb)) mask_scores(jb, s);
    __builtin_amdgcn_sched_barrier(0);
    YX(std::true_type{}, jb % kNBuf, s, p, (jb + 1) % kNBuf, sx, px, jd, (jb + 3) % kNBuf);
    __builtin_amdgcn_sched_barrier(0);
    Z(jb % kNBuf);
    wait_vmem_keep<kSlots>();  // block jb+2 (loaded since the last iteration) is in LDS
    barrier_nofence();
  };
  auto last = [&](int jb, f32x16 (&s)[C::NSUB], f32x16 (&p)[C::NSUB]) __attribute__((always_inline)) {
    if (need_mask(jb)) mask_scores(jb, s);
    __builtin_amdgcn_sched_barrier(0);
    YX(std::false_type{}, jb % kNBuf, s, p, 0, sB, pB, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    Z(jb % kNBuf);
  };

  if (nblk > 0) {
    // blocks 0, 1, 2 into buffers 0, 1, 2, X(0), then the pipeline
#pragma unroll
    for (int i = 0; i < kSlots; ++i) dma_slot(i, 0, 0);
#pragma unroll
    for (int i = 0; i < kSlots; ++i) dma_slot(i, min(1, nblk - 1), 1);
#pragma unroll
    for (int i = 0; i < kSlots; ++i) dma_slot(i, min(2, nblk - 1), 2);
    wait_vmem();
    __syncthreads();
    X(0, sA, pA);
    schedule_mfma_reads<NX - 4, 1, 4>();
    __builtin_amdgcn_sched_barrier(0);
    int jb = 0;
    for (; jb + 2 < nblk; jb += 2) {
      iteration(jb, sA, pA, sB, pB);
      iteration(jb + 1, sB, pB, sA, pA);
    }
    if (jb + 1 < nblk) {
      iteration(jb, sA, pA, sB, pB);
      last(jb + 1, sB, pB);
    } else {
      last(jb, sA, pA);
    }
  }

  // dK^T / dV^T accumulators: lane = key, register 4a+b of subtile s = column 32s + 8a + 4*half + b
  if (key < N_kv) {
    float* dkp = dK + kvbase + size_t(key) * D;
    float* dvp = dV + kvbase + size_t(key) * D;
#pragma unroll
    for (int s = 0; s < C::DSUB; ++s)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        f32x4 vk, vv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vk[e] = dk[s][4 * a + e] * scale;
          vv[e] = dv[s][4 * a + e];
        }
        *reinterpret_cast<f32x4*>(dkp + 32 * s + 8 * a + 4 * half) = vk;
        *reinterpret_cast<f32x4*>(dvp + 32 * s + 8 * a + 4 * half) = vv;
      }
  }
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
constexpr int kQueriesPerWg = 128;  // 4 waves x 32 queries

// Per wave (32 queries) and streamed key block j (64 keys):
//   X(j): S^T = K Q^T, dP^T = V dO^T          (MFMA, K/V rows from LDS)
//   Y(j): P, dS^T = P (dP - D), packed         (VALU)
//   Z(j): dQ^T += K^T dS^T                     (MFMA, K read transposed)
// in that order, with the LDS-DMA of block j+1 into the other buffer issued
// between the vector work of Y(j). Overlap of MFMA and vector work comes from
// the second workgroup on the compute unit (two waves per SIMD): within one
// wave the two barely overlap on this hardware, and the software-pipelined
// form that needs S/dP twice (420 registers, one wave per SIMD) measured
// 2-3 % slower.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ L2, const float* __restrict__ Dl,
    float* __restrict__ dQ, int H_q, int H_kv, int N_q, int N_kv, int n_qtiles, int xcd_remap, float c,
    float scale) {
  using C = BwdCfg<D>;
  constexpr int BK = C::BLK;
  constexpr int DPW = C::DMA_PER_WAVE;
  constexpr int kNB = 2;  // two workgroups per CU: 64 KiB of LDS each
  __shared__ __attribute__((aligned(1024))) uint8_t ks[kNB][C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vs[kNB][C::TILE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int half = lane >> 5;
  const int G = H_q / H_kv;

  const TileAssign ta = assign_tile(blockIdx.x, n_qtiles, G, xcd_remap);
  const int b = ta.kvidx / H_kv;
  const int hk = ta.kvidx % H_kv;
  const int h = hk * G + ta.gq;
  const int tile = CAUSAL ? (n_qtiles - 1 - ta.tile_rank) : ta.tile_rank;  // heaviest first
  const int q0 = tile * kQueriesPerWg;
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
  wait_vmem();  // the LDS-DMA below is not tracked by the compiler's waits

  // key blocks of the workgroup; every wave runs all of them (blocks past a
  // wave's queries are masked to zero).
  const int nblk_all = (N_kv + BK - 1) / BK;
  int nblk = nblk_all;
  if (CAUSAL) nblk = min(nblk_all, (min(q0 + kQueriesPerWg, N_q) - 1) / BK + 1);

  const int tail_blk = (N_kv % BK) ? N_kv / BK : -1;
  const int tail_lim = (N_kv - 1) % BK;
  uint32_t doff[DPW], doff_t[DPW];
#pragma unroll
  for (int i = 0; i < DPW; ++i) {
    const int ig = wave * DPW + i;
    const int row = C::RPI * ig + lane / C::CPR;
    const int pch = lane % C::CPR;
    doff[i] = row * C::ROW_BYTES + (pch ^ swz<D>(row)) * 16;
    doff_t[i] = doff[i] - (row - min(row, tail_lim)) * C::ROW_BYTES;
  }
  const uint8_t* Kb = reinterpret_cast<const uint8_t*>(K + kvbase);
  const uint8_t* Vb = reinterpret_cast<const uint8_t*>(V + kvbase);
  constexpr int kSlots = 2 * DPW;
  auto dma_slot = [&](int i, int j, int bf) __attribute__((always_inline)) {
    const bool is_k = i < DPW;
    const int ii = is_k ? i : i - DPW;
    const uint8_t* src = (is_k ? Kb : Vb) + size_t(j) * BK * C::ROW_BYTES;
    lds_dma16_sbase_nc(src, j == tail_blk ? doff_t[ii] : doff[ii],
                       lds_address(is_k ? ks[bf] : vs[bf]) + 1024 * (wave * DPW + ii));
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
  auto X = [&](int bf) __attribute__((always_inline)) {
    const uint8_t* kt = ks[bf];
    const uint8_t* vt = vs[bf];
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
  auto Y = [&](int j, int jd, int bfd) __attribute__((always_inline)) {
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
        if (e % 3 == 1 && e / 3 < kSlots) dma_slot(e / 3, jd, bfd);
      }
#pragma unroll
      for (int w = 0; w < 2; ++w)
#pragma unroll
        for (int e = 0; e < 4; ++e) sk[2 * n + w][e] = cvt_pk_bf16(pA[n][8 * w + 2 * e], pA[n][8 * w + 2 * e + 1]);
    }
#pragma unroll
    for (int e = 32 * C::NSUB / 3 + 1; e < kSlots; ++e) dma_slot(e, jd, bfd);
  };
  auto Z = [&](int bf) __attribute__((always_inline)) {
    const uint8_t* kt = ks[bf];
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

  // block 0 into buffer 0; block j+1 is loaded into the other buffer while
  // block j is processed (the buffer's previous block was finished before
  // the last barrier)
#pragma unroll
  for (int i = 0; i < kSlots; ++i) dma_slot(i, 0, 0);
  wait_vmem();
  __syncthreads();
  for (int j = 0; j < nblk; ++j) {
    const int bf = j & 1;
    const int jd = min(j + 1, nblk - 1);  // past the end: a harmless reload
    X(bf);
    __builtin_amdgcn_sched_barrier(0);
    Y(j, jd, bf ^ 1);
    __builtin_amdgcn_sched_barrier(0);
    Z(bf);
    wait_vmem();
    barrier_nofence();
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
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)((long long)n_ktiles * p.B * p.H_kv)),
                     dim3(kThreads), 0, stream, static_cast<const uint16_t*>(p.q), static_cast<const uint16_t*>(p.k),
                     static_cast<const uint16_t*>(p.v), static_cast<const uint16_t*>(p.dO), L2, Dl, p.dk, p.dv,
                     p.H_q, p.H_kv, p.N_q, p.N_kv, n_ktiles, xcd_remap, c, p.scale);
  const int n_qtiles = (p.N_q + kQueriesPerWg - 1) / kQueriesPerWg;
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)((long long)n_qtiles * p.B * p.H_q)), dim3(kThreads),
                     0, stream, static_cast<const uint16_t*>(p.q), static_cast<const uint16_t*>(p.k),
                     static_cast<const uint16_t*>(p.v), static_cast<const uint16_t*>(p.dO), L2, Dl, p.dq, p.H_q,
                     p.H_kv, p.N_q, p.N_kv, n_qtiles, xcd_remap, c, p.scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t stream) {
  if (p.d == 128) return p.causal ? launch<128, true>(p, stream) : launch<128, false>(p, stream);
  return p.causal ? launch<64, true>(p, stream) : launch<64, false>(p, stream);
}

}  // namespace fa

// Attention forward for bf16 inputs on gfx950 (MI355X).
//
// Method: the Q-stationary blockwise online softmax of "深度学习进阶（三十一）
// FlashAttention：IO 感知的精确注意力" (rkmt.cn blog) §2.2 -- a block of query
// rows stays on chip while every K/V block streams past it; each row keeps a
// running max m, a normalizer l and an output accumulator O, rescaled by
// exp(m_prev - m_new) when the max grows. Scores and probabilities live only
// in registers; O and the per-row logsumexp are the only outputs ("FlashAttention",
// LLM Inference Handbook: tiling plus kernel fusion, no N x N matrix in HBM).
//
// gfx950 mapping
// --------------
//  * Workgroup = 8 wave64s, 256 query rows (32 per wave), one workgroup per
//    CU (2 waves per SIMD). All tiles of one key/value head go to one XCD.
//    Causal calls at d = 128 (dense, or packed with n counted per sequence):
//    a workgroup takes two tiles of one head, r and n-1-r, one after the
//    other, so that every workgroup of a head costs the same
//    (the dispatcher starts an XCD's workgroups a few at a time and in order,
//    so unequal neighbours leave compute units idle) while one head's tiles
//    stay neighbours in the grid (their K/V is shared through L2). The
//    lighter tile runs second and visits its key blocks from the diagonal
//    down, so that all workgroups of a head read the same K/V block at each
//    step of both tiles. Non-causal calls take one workgroup per (batch,
//    query head, 256-row tile). (d = 64 runs the rotation kernel below.)
//  * Contractions on v_mfma_f32_32x32x16_bf16 with fp32 accumulation. The
//    scores are computed transposed, S^T = K Q^T (K as the A operand, Q as B),
//    so that a lane owns one query column; P^T then feeds O^T = V^T P^T as the
//    B operand straight from registers, and every per-row quantity (max, sum,
//    rescale factor) is lane-local. The two halves of a wave hold disjoint
//    keys of the same query and meet through one v_permlane32_swap.
//  * Ping-pong between the two waves of each SIMD: waves 0-3 (group A) and
//    4-7 (group B) run the same per-block sequence -- an MFMA phase
//    (PV of block j-1, then QK^T of block j) and a vector phase (mask, max,
//    exponentials, row sums, bf16 packing of block j) -- with B one phase
//    behind A, and one workgroup barrier per block. A block starts with A's
//    MFMA phase beside B's vector phase; the MFMA phases run at wave priority
//    2 and B's vector phase at 1, so that the wave that finishes first goes
//    on to its next phase on the issue slots its partner leaves.
//  * K and V blocks stream from HBM straight into LDS with 16-byte
//    global_load_lds_dwordx4 (no register staging, double-buffered), issued
//    by group B one at a time between the exponentials of its vector phase:
//    a wave stalls at a vector-memory instruction until the CU's load path
//    accepts it, so a burst would cost the whole transfer time. The block
//    barriers carry no memory fence, so the loads stay in flight through B's
//    MFMA phase and are waited for only before the barrier that publishes
//    them. Tiles are row-major with XOR-swizzled 16-byte chunks chosen so
//    that every LDS read is free of bank conflicts. The V^T operand is read with ds_read_b64_tr_b16, which
//    transposes 16-bit elements across lanes.
//  * Softmax in base 2: scores are multiplied by scale*log2(e) inside one FMA
//    and exponentiated with v_exp_f32; LSE is converted back with ln 2. The
//    running max may be stale by up to 2^8 (exact: the final division and
//    the LSE use the same max). A block's exponentials are taken against the
//    running max first and the block max is formed only if some row's block
//    sum exceeds 2^8 (then the max is raised, O and l rescaled, and the
//    exponentials taken again); after a block that moved the max, the next
//    one forms its max first. This takes the max off most blocks' vector
//    phase, one of the loop's two bounds (the other is the MFMA phase's
//    operand reads from LDS).
//  * Causal: K/V blocks past the tile's last row are never loaded; masking
//    runs only on blocks that cross a wave's diagonal or the end of the keys.
//  * d = 64 runs fwd_bf16_rot_kernel (below): four waves per SIMD in a
//    four-group rotation, for the vector work that outweighs the matrix work
//    about twice at that head size.

#include <type_traits>

#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBR = 32 * kWaves;       // query rows per workgroup
constexpr float kRescaleSlack = 8.0f;  // log2 units: skip the rescale while max grows by <= 2^8


// sched_group_barrier instruction classes
constexpr int kSgValu = 0x402;   // VALU (non-MFMA) and transcendental
constexpr int kSgMfma = 0x008;
constexpr int kSgVmem = 0x010;
constexpr int kSgDsRead = 0x100;

template <int D>
struct FwdCfg {
  static constexpr int BC = 8192 / D;              // keys per block: 64 at d=128 (d=64 calls run the rotation kernel)
  static constexpr int NSUB = BC / 32;             // 32-key subtiles of S^T
  static constexpr int DSUB = D / 32;              // 32-column subtiles of O^T
  static constexpr int QK_STEPS = D / 16;          // MFMA k-steps over the head dimension
  static constexpr int PV_STEPS = BC / 16;         // MFMA k-steps over keys
  static constexpr int CPR = D / 8;                // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;             // rows per 1 KiB LDS-DMA instruction
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int TILE_BYTES = BC * D * 2;    // 16 KiB
  static constexpr int DMA_PER_WAVE = TILE_BYTES / 1024 / 4;  // per tile, 4 loader waves
};

// Chunk swizzles (16-byte chunk index XOR f(row)).
//  K: the 16 lanes of an S^T A-operand read phase touch 16 distinct rows at one
//     logical chunk; f_k spreads them over all 16 (d=128) or 8 x 2-row (d=64)
//     bank groups.
//  V: a ds_read_b64_tr_b16 phase reads 4 consecutive rows x 64 bytes; f_v
//     moves each of the 4 rows to a different 64-byte bank group.
template <int D>
__device__ __forceinline__ int swz_k(int row) {
  if constexpr (D == 128) return (row & 7) | ((row >> 1) & 8);
  else return ((row >> 1) & 3) | ((row >> 2) & 4);
}
template <int D>
__device__ __forceinline__ int swz_v(int row) {
  if constexpr (D == 128) return (row & 3) << 2;
  else return ((row >> 1) & 1) << 2;
}


template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE,
    int H_q, int H_kv, int N_q_arg, int N_kv_arg, int n_qtiles, int xcd_remap, float c,
    const int* __restrict__ cu_q, const int* __restrict__ cu_k, int total_q, int total_k, int paired) {
  using C = FwdCfg<D>;
  constexpr int BC = C::BC;
  constexpr int NSUB = C::NSUB;
  // Four separate LDS objects (K and V, two buffers each) so that the compiler
  // can tell the tiles being read from the ones the in-flight LDS DMA writes,
  // and does not wait for the prefetch before every LDS read.
  __shared__ __attribute__((aligned(1024))) uint8_t kb0[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t kb1[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vb0[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vb1[C::TILE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;    // 0: group A (leads), 1: group B (one phase behind, loads K/V)
  const int gw = wave & 3;      // index within the group (= SIMD)
  const int col = lane & 31;    // query column of this lane (and MFMA row for A operands)
  const int half = lane >> 5;   // lane half: key half for S^T, d half for the Q/K operands
  const int G = H_q / H_kv;

  // ---- schedule: workgroup -> (batch, head, query tile or pair of tiles)
  // Causal tiles differ in cost. Paired, every workgroup costs the same, and
  // a pair rank is dealt over the G query heads of one key/value head, so
  // that the workgroups running side by side read the same K/V blocks at the
  // same steps (with G = 1, a head's pairs one after the other). Packed
  // sequences pair the tiles of each sequence by its own tile count; pair
  // ranks past a short sequence end at once. Unpaired (d = 64), causal tiles
  // are dealt rank by rank over groups of four heads, so that consecutive
  // workgroups still cost about the same.
  const int n_units = paired ? (n_qtiles + 1) / 2 : n_qtiles;
  const TileAssign ta = assign_tile(blockIdx.x, n_units, G, xcd_remap, (int)(gridDim.x / n_units), false,
                                    (CAUSAL && !paired) ? 4 : (paired ? G : 1));
  const int kvidx = ta.kvidx, gq = ta.gq, tile_rank = ta.tile_rank;
  const int b = kvidx / H_kv;
  const int hk = kvidx % H_kv;
  const int h = hk * G + gq;

  // Dense: q, o [B][H_q][N_q][D], k, v [B][H_kv][N_kv][D], lse [B][H_q][N_q].
  // Packed sequences (cu_q != null): b is a sequence, q, o [H_q][total_q][D],
  // k, v [H_kv][total_k][D], lse [H_q][total_q]; sequence b owns rows
  // cu_q[b] .. cu_q[b+1]-1 of q and cu_k[b] .. cu_k[b+1]-1 of k. The offsets
  // are clamped to [0, total], so inconsistent ones give wrong rows, never an
  // access outside the tensors; N_q_arg is then the longest query sequence
  // the grid covers.
  int N_q = N_q_arg, N_kv = N_kv_arg;
  size_t qbase, kvbase, lbase;
  if (cu_q != nullptr) {
    const int qs = min(max(cu_q[b], 0), total_q);
    const int qe = min(max(cu_q[b + 1], qs), total_q);
    const int ks = min(max(cu_k[b], 0), total_k);
    const int ke = min(max(cu_k[b + 1], ks), total_k);
    N_q = min(qe - qs, N_q_arg);
    N_kv = ke - ks;
    qbase = (size_t(h) * total_q + qs) * D;
    kvbase = (size_t(hk) * total_k + ks) * D;
    lbase = size_t(h) * total_q + qs;
  } else {
    qbase = (size_t(b) * H_q + h) * size_t(N_q) * D;
    kvbase = (size_t(b) * H_kv + hk) * size_t(N_kv) * D;
    lbase = (size_t(b) * H_q + h) * size_t(N_q);
  }
  // tiles of this workgroup: the heavier one first, then (paired) its mirror,
  // counted in the sequence's own tiles
  const int n_seq = paired ? (N_q + kBR - 1) / kBR : n_qtiles;
  if (paired && tile_rank >= (n_seq + 1) / 2) return;  // (whole workgroup) past a short sequence
  const int tile_hi = CAUSAL ? (n_seq - 1 - tile_rank) : tile_rank;  // heaviest first
  const int n_it = (D == 128 && paired && tile_rank != tile_hi) ? 2 : 1;  // (launch sets paired only at d = 128)
  for (int it = 0; it < n_it; ++it) {
    const int tile = it == 0 ? tile_hi : tile_rank;
    const int q0 = tile * kBR;
    if (it > 0) barrier_nofence();  // every wave is done with the previous tile's LDS
    if (q0 >= N_q) return;  // (whole workgroup) a tile past a short sequence
    if (N_kv == 0) {
      // a sequence without keys: softmax over nothing; its rows get O = 0 and
      // LSE = -inf (packed sequences only, dense calls reject N_kv = 0)
      const int row = q0 + wave * 32 + col;
      if (row < N_q) {
        uint16_t* op = O + qbase + size_t(row) * D + half * (D / 2);
#pragma unroll
        for (int j = 0; j < D / 2; j += 4) st_global8(op + j, u32x2{0u, 0u});
        if (half == 0) LSE[lbase + row] = -INFINITY;
      }
      continue;
    }
    const uint8_t* __restrict__ Kbytes = reinterpret_cast<const uint8_t*>(K + kvbase);
    const uint8_t* __restrict__ Vbytes = reinterpret_cast<const uint8_t*>(V + kvbase);

    // ---- Q tile into registers: B operand of S^T = K Q^T (read once)
    const int wrow0 = q0 + wave * 32;
    const int qrow = wrow0 + col;
    bf16x8 qreg[C::QK_STEPS];
    {
      const uint16_t* qp = Q + qbase + size_t(min(qrow, N_q - 1)) * D + half * (D / 2);
#pragma unroll
      for (int t = 0; t < C::QK_STEPS; ++t) qreg[t] = as_bf16x8(ld_global16(qp + 8 * t));
    }

    // ---- key blocks visited by the workgroup. Every wave computes all of them:
    // the block barriers make a block cost the same time whether or not a wave
    // skips it, and a block entirely past a wave's rows is masked to exact
    // zeros (every row sees key 0 in block 0, so its running max is finite
    // from then on and exp2 of a masked score is 0).
    const int nblk_all = (N_kv + BC - 1) / BC;
    int nblk = nblk_all;
    if (CAUSAL) {
      const int last_row = min(q0 + kBR, N_q) - 1;
      nblk = min(nblk_all, last_row / BC + 1);
    }
    // Order of the key blocks. Causal, the lighter tile of a mirror pair (t
    // and n-1-t, n the sequence's tile count) takes its diagonal blocks first
    // and then the others from the diagonal down to block 0; every other tile
    // goes from block 0 up. A workgroup runs its heavier tile first, so the
    // workgroups of a head, running side by side, all read key block b at the
    // same step: step b while ascending, step 4n+3-b while descending. Each
    // block is fetched from HBM once for all of them. Had the lighter tile
    // restarted at block 0, the workgroups would reach each block at staggered
    // steps and L2 would have evicted it in between. The first block visited
    // shows every row at least one key (its own diagonal block or, with no
    // diagonal block, one wholly below the tile).
    const int n_own = (N_q + kBR - 1) / kBR;
    const int dlo = (CAUSAL && tile < n_own - 1 - tile) ? min(q0 / BC, nblk) : 0;
    const int n_asc = nblk - dlo;
    auto blk = [&](int j) __attribute__((always_inline)) { return j < n_asc ? dlo + j : nblk - 1 - j; };
    auto need_mask = [&](int jb) __attribute__((always_inline)) {
      const int kv0 = jb * BC;
      return (CAUSAL && kv0 + BC - 1 > wrow0) || (kv0 + BC > N_kv);
    };

    // ---- LDS-DMA staging by the 4 waves of group B: each fills DMA_PER_WAVE
    // KiB of a tile. Instruction i writes bytes [1024*ig, 1024*ig + 1024) of the
    // tile, lane l the 16 bytes at 16*l: row RPI*ig + l/CPR, physical chunk
    // l%CPR, which holds logical chunk (l%CPR) ^ swz(row).
    // The *_t offsets serve the last key block when N_kv is not a multiple of
    // BC: they read row min(row, last valid row) instead (finite data for the
    // masked keys, and no access past the end of K and V).
    const int tail_blk = (N_kv % BC) ? N_kv / BC : -1;
    const int tail_lim = N_kv - 1 - (N_kv / BC) * BC;
    uint32_t dma_koff[C::DMA_PER_WAVE], dma_voff[C::DMA_PER_WAVE];
    uint32_t dma_koff_t[C::DMA_PER_WAVE], dma_voff_t[C::DMA_PER_WAVE];
#pragma unroll
    for (int i = 0; i < C::DMA_PER_WAVE; ++i) {
      const int ig = gw * C::DMA_PER_WAVE + i;
      const int row = C::RPI * ig + lane / C::CPR;
      const int p = lane % C::CPR;
      const int cut = (row - min(row, tail_lim)) * C::ROW_BYTES;
      dma_koff[i] = row * C::ROW_BYTES + (p ^ swz_k<D>(row)) * 16;
      dma_voff[i] = row * C::ROW_BYTES + (p ^ swz_v<D>(row)) * 16;
      dma_koff_t[i] = dma_koff[i] - cut;
      dma_voff_t[i] = dma_voff[i] - cut;
    }
    // DMA slot i of a vector phase of group B: slots 0 .. DMA_PER_WAVE-1 stage
    // 1 KiB pieces of the K tile at key block jk, the others pieces of the V
    // tile at block jv, each from a uniform base plus a per-lane 32-bit offset
    // (the clamped one for block tail_blk, picked by a uniform select).
    auto dma_slot = [&](int i, int jk, int jv, uint8_t* kdst, uint8_t* vdst)
        __attribute__((always_inline)) {
      const bool is_k = i < C::DMA_PER_WAVE;
      const int ii = is_k ? i : i - C::DMA_PER_WAVE;
      const int jb = is_k ? jk : jv;
      const uint8_t* src = (is_k ? Kbytes : Vbytes) + size_t(jb) * BC * C::ROW_BYTES;
      uint32_t off = is_k ? dma_koff[ii] : dma_voff[ii];
      if (jb == tail_blk) off = is_k ? dma_koff_t[ii] : dma_voff_t[ii];
      lds_dma16_sbase(src, off, lds_address(is_k ? kdst : vdst) + 1024 * (gw * C::DMA_PER_WAVE + ii));
    };
    // K_0 for the prologue (only group B calls it)
    auto dma_k0 = [&](uint8_t* kdst) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < C::DMA_PER_WAVE; ++i) dma_slot(i, blk(0), blk(0), kdst, kdst);
    };

    // ---- per-lane LDS read offsets (bytes within a tile)
    // K (S^T A operand): row row_of_lane(col) of subtile n (n adds 32 rows), chunk (D/16)*half + t.
    const int krow = row_of_lane(col);
    int koff[C::QK_STEPS];
#pragma unroll
    for (int t = 0; t < C::QK_STEPS; ++t)
      koff[t] = krow * C::ROW_BYTES + ((((D / 16) * half + t) ^ swz_k<D>(krow)) * 16);
    // V (O^T A operand via transposed reads): a 16-lane group j = lane%16 reads
    // rows r0 + j/4 (r0 = 32n + 16*half + 8w + 4r) at columns c0 + 4*(j%4),
    // c0 = 32*s + 16*((lane%32)/16).
    const int j16 = lane & 15;
    const int vgrp = (lane & 31) >> 4;
    int voff[C::DSUB];
#pragma unroll
    for (int s = 0; s < C::DSUB; ++s) {
      const int row = 16 * half + (j16 >> 2);
      const int cc = 32 * s + 16 * vgrp + 4 * (j16 & 3);
      voff[s] = row * C::ROW_BYTES + (((cc >> 3) ^ swz_v<D>(row)) * 16) + (cc & 7) * 2;
    }

    // ---- online-softmax state (per query column; l is per lane half)
    float m_run = -INFINITY;
    float l_run = 0.f;
    bool eager = true;  // form the block max before the exponentials
    f32x16 oacc[C::DSUB];
#pragma unroll
    for (int s = 0; s < C::DSUB; ++s) oacc[s] = f32x16{};
    f32x16 sacc[NSUB];          // scores of the current block
    u32x4 pk[C::PV_STEPS];      // its probabilities, bf16-packed as PV B operands

    // MFMA phase for block j: O^T += V_{j-1}^T P_{j-1}^T, then S^T_j = K_j Q^T.
    auto pv_part = [&](const uint8_t* vt) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < C::PV_STEPS; ++u) {
        const int rbase = (32 * (u >> 1) + 8 * (u & 1)) * C::ROW_BYTES;  // + 4 rows for the second read
#pragma unroll
        for (int s = 0; s < C::DSUB; ++s) {
          LDS_AS i16x4* p0 = (LDS_AS i16x4*)(vt + voff[s] + rbase);
          LDS_AS i16x4* p1 = (LDS_AS i16x4*)(vt + voff[s] + rbase + 4 * C::ROW_BYTES);
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p0);
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p1);
          u32x4 av;
          av[0] = __builtin_bit_cast(u32x2, lo)[0];
          av[1] = __builtin_bit_cast(u32x2, lo)[1];
          av[2] = __builtin_bit_cast(u32x2, hi)[0];
          av[3] = __builtin_bit_cast(u32x2, hi)[1];
          oacc[s] = mfma32x32x16(as_bf16x8(av), as_bf16x8(pk[u]), oacc[s]);
        }
      }
    };
    auto qk_part = [&](const uint8_t* kt) __attribute__((always_inline)) {
#pragma unroll
      for (int n = 0; n < NSUB; ++n) sacc[n] = f32x16{};
#pragma unroll
      for (int t = 0; t < C::QK_STEPS; ++t) {
#pragma unroll
        for (int n = 0; n < NSUB; ++n) {
          const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(kt + koff[t] + n * 32 * C::ROW_BYTES));
          sacc[n] = mfma32x32x16(a, qreg[t], sacc[n]);
        }
      }
    };
    // Operand reads run ahead of the MFMAs that consume them: 8 V reads up
    // front, then 2 reads behind every PV MFMA and 1 behind every QK^T MFMA
    // (the K reads of the QK^T part start while the last PV MFMAs run).
    auto pv_schedule = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 6; ++i) __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
#pragma unroll
      for (int i = 0; i < C::PV_STEPS * C::DSUB; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSgDsRead, 2, 0);
      }
    };
    auto qk_schedule = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < C::QK_STEPS * NSUB; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
      }
    };
    auto mfma_phase = [&](int j, const uint8_t* kt, const uint8_t* vt) __attribute__((always_inline)) {
      const bool do_pv = j >= 1;
      const bool do_qk = j < nblk;
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(2);
      __builtin_amdgcn_sched_barrier(0);
      if (do_pv) {
        pv_part(vt);
        pv_schedule();
      }
      if (do_qk) {
        qk_part(kt);
#pragma unroll
        for (int i = 0; i < 3; ++i) __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
        qk_schedule();
      }
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
    };

    // Vector phase for block j: mask, block max, (rare) rescale, exponentials,
    // row sums and bf16 packing. `issue(i)`, i = 0 .. kDmaSlots-1, issues the
    // LDS-DMA instructions of the loading group; they are spread through the
    // exponential loop (a wave that issues a vector-memory instruction stalls
    // until the CU's load pipeline accepts it, so a burst of them would stall
    // the wave for the whole transfer instead of overlapping it).
    constexpr int kDmaSlots = 2 * C::DMA_PER_WAVE;
    auto no_dma = [](int) __attribute__((always_inline)) {};
    constexpr int kSlotsPerStep = kDmaSlots / C::PV_STEPS;
    static_assert(kSlotsPerStep * C::PV_STEPS == kDmaSlots, "DMA slots per exponential step");
    auto valu_phase = [&](int j, auto&& issue, auto has_dma) __attribute__((always_inline)) {
      constexpr bool kDma = decltype(has_dma)::value;
      if constexpr (!kDma) {
        if (j >= nblk) return;  // the step that only finishes PV of the last block
      }
      const int jb = blk(j);
      if (need_mask(jb)) {
        // key kv0 + 32n + 16*half + i is visible iff it is <= last_key (the
        // row itself when causal, and < N_kv); one compare against the
        // register's constant key offset per score.
        const int last_key = CAUSAL ? min(qrow, N_kv - 1) : N_kv - 1;
        const int lim = last_key - jb * BC - 16 * half;
#pragma unroll
        for (int n = 0; n < NSUB; ++n)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (32 * n + i > lim) sacc[n][i] = -INFINITY;
      }
      // Exponentials against the running max. A row's block sum above 2^8
      // (or inf / NaN: the max was never set) means a probability may exceed
      // 2^8: the block max is formed, the running max raised and the block's
      // exponentials taken again. A sum within 2^8 bounds every probability.
      float psum = 0.f;
      auto exps = [&](auto&& issue, auto dma_here) __attribute__((always_inline)) {
        constexpr bool kD = decltype(dma_here)::value;
        psum = 0.f;
#pragma unroll
        for (int u = 0; u < C::PV_STEPS; ++u) {
          const int n = u >> 1;
          const int w8 = (u & 1) * 8;
          float p[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            p[e] = fast_exp2(fmaf(sacc[n][w8 + e], c, -m_run));
            psum += p[e];
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) pk[u][e] = cvt_pk_bf16(p[2 * e], p[2 * e + 1]);
          if constexpr (kD) {
#pragma unroll
            for (int r = 0; r < kSlotsPerStep; ++r) issue(u * kSlotsPerStep + r);
          }
        }
        if constexpr (kD) {
#pragma unroll
          for (int i = 0; i < kDmaSlots; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSgValu, 28 / kSlotsPerStep, 0);
            __builtin_amdgcn_sched_group_barrier(kSgVmem, 1, 0);
          }
        }
      };
      auto block_max = [&]() __attribute__((always_inline)) {
        float mx = sacc[0][0];
#pragma unroll
        for (int n = 0; n < NSUB; ++n)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[n][i]);
        return max_xor32(mx) * c;
      };
      auto rescale_to = [&](float m_new) __attribute__((always_inline)) {
        const float alpha = fast_exp2(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int s = 0; s < C::DSUB; ++s)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[s][i] *= alpha;
        m_run = m_new;
      };
      bool moved = false;
      if (eager) {
        // the previous block moved the max: form this block's max first
        const float m_blk = block_max();
        if (__any(m_blk > m_run + kRescaleSlack)) {
          rescale_to(fmaxf(m_run, m_blk));
          moved = true;
        }
      }
      exps(issue, has_dma);
      if (__any(!(psum <= 256.0f))) {
        const float m_new = fmaxf(m_run, block_max());
        // (a sum above 2^8 implies some row's max rose; only NaN inputs can
        // leave every max unchanged, and then the block stands as computed)
        if (__any(m_new > m_run)) {
          rescale_to(m_new);
          exps(no_dma, std::false_type{});
          moved = true;
        }
      }
      eager = moved;
      l_run += psum;
    };

    // One barrier per block j. Group A: MFMA(j), VALU(j). Group B: VALU(j-1)
    // + DMA of K_{j+1}, V_j, MFMA(j), then wait for the DMA. The DMA of block
    // j overwrites the buffers of K_{j-1} and V_{j-2}, which both groups last
    // read in their MFMA phases of block j-1, before the barrier that starts
    // block j. The barriers carry no memory fence: every LDS read of a phase
    // is consumed by an MFMA of the same phase, and DMA data is waited for
    // explicitly before the barrier that publishes it. Wave priorities (MFMA
    // phases 2, B's vector phase 1, A's 0) keep the block's order: A's MFMA
    // beside B's softmax, then B's MFMA beside A's softmax, with the wave that
    // finishes early running ahead on the issue slots the other leaves.
    // Buffers: step j's K and V blocks in kb[j%2], vb[j%2]. Each group runs its own loop
    // (the group test is outside the loop, so the compiler never has to keep
    // both groups' register state alive across the barriers); both loops pass
    // the same nblk+1 barriers.
    auto block_a = [&](int j, const uint8_t* k_cur, const uint8_t* v_prev) __attribute__((always_inline)) {
      mfma_phase(j, k_cur, v_prev);
      valu_phase(j, no_dma, std::false_type{});
      barrier_nofence();
    };
    auto block_b = [&](int j, const uint8_t* k_cur, const uint8_t* v_prev, uint8_t* k_dma, uint8_t* v_dma)
        __attribute__((always_inline)) {
      // K_{j+1} and V_j; past the last block the last one is loaded again into
      // a buffer nobody reads any more, which keeps the issue slots unconditional.
      const int jk = blk(min(j + 1, nblk - 1));
      const int jv = blk(min(j, nblk - 1));
      // B's vector phase, which the block waits for, takes issue precedence
      // over A's, which starts as soon as A's MFMA phase ends
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(1);
      __builtin_amdgcn_sched_barrier(0);
      valu_phase(j - 1, [&](int i) __attribute__((always_inline)) {
        dma_slot(i, jk, jv, k_dma, v_dma); }, std::true_type{});
      mfma_phase(j, k_cur, v_prev);
      wait_vmem();        // K_{j+1} and V_j are in LDS before the barrier publishes them
      barrier_nofence();
    };

    // ---- prologue: K_0 into kb0
    if (grp == 1) {
      dma_k0(kb0);
      wait_vmem();
    }
    __syncthreads();

    // Blocks 0..nblk: the extra step j = nblk finishes PV of the last block.
    if (grp == 0) {
      for (int j = 0; j <= nblk; j += 2) {
        block_a(j, kb0, vb1);
        if (j + 1 <= nblk) block_a(j + 1, kb1, vb0);
      }
    } else {
      // Step 0 has no softmax yet: only the loads of K_1 and V_0, then QK^T of
      // block 0 (peeled, so that every vector phase in the loop has work).
      {
        const int jk = blk(min(1, nblk - 1));
#pragma unroll
        for (int i = 0; i < kDmaSlots; ++i) dma_slot(i, jk, blk(0), kb1, vb0);
        mfma_phase(0, kb0, vb1);
        wait_vmem();
        barrier_nofence();
      }
      for (int j = 1; j <= nblk; j += 2) {
        block_b(j, kb1, vb0, kb0, vb1);
        if (j + 1 <= nblk) block_b(j + 1, kb0, vb1, kb1, vb0);
      }
    }

    // ---- epilogue: O = O_acc / l, LSE = ln2 * (m + log2 l)
    const float l_tot = sum_xor32(l_run);
    if (qrow < N_q) {
      const float inv = 1.0f / l_tot;
      uint16_t* op = O + qbase + size_t(qrow) * D;
#pragma unroll
      for (int s = 0; s < C::DSUB; ++s) {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          u32x2 w;
          w[0] = cvt_pk_bf16(oacc[s][4 * a + 0] * inv, oacc[s][4 * a + 1] * inv);
          w[1] = cvt_pk_bf16(oacc[s][4 * a + 2] * inv, oacc[s][4 * a + 3] * inv);
          st_global8(op + 32 * s + 8 * a + 4 * half, w);
        }
      }
      if (half == 0) LSE[lbase + qrow] = (m_run + __log2f(l_tot)) * kLn2;
    }
  }
}

// Dense when vl is null; packed sequences otherwise (p.B sequences, p.N_q the
// longest query sequence).
template <int D, bool CAUSAL>
hipError_t launch(const FwdParams& p, const VarlenParams* vl, hipStream_t stream) {
  const int n_qtiles = (p.N_q + kBR - 1) / kBR;
  const int paired = (D == 128 && CAUSAL) ? 1 : 0;
  const long long nwg = (long long)(paired ? (n_qtiles + 1) / 2 : n_qtiles) * p.B * p.H_q;
  const int xcd_remap = ((p.B * p.H_kv) % 8 == 0) ? 1 : 0;
  // Masked scores are -inf and exp2(-inf * c) must be 0, so c stays positive:
  // for scale == 0 the smallest normal float gives exactly the uniform weights
  // (every unmasked exponent rounds to exp2(0) = 1).
  const float c = fmaxf(p.scale * kLog2e, 1.17549435e-38f);
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL>), dim3((unsigned)nwg), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(p.q), static_cast<const uint16_t*>(p.k),
                     static_cast<const uint16_t*>(p.v), static_cast<uint16_t*>(p.o), p.lse,
                     p.H_q, p.H_kv, p.N_q, p.N_kv, n_qtiles, xcd_remap, c,
                     vl ? vl->cu_q : nullptr, vl ? vl->cu_k : nullptr, vl ? vl->total_q : 0,
                     vl ? vl->total_k : 0, paired);
  return hipGetLastError();
}


// ---------------------------------------------------------------------------
// d = 64: four-group rotation.
//
// At d = 64 a key block costs the vector ALU about twice what it costs the
// matrix cores (the softmax work per score is the same as at d = 128, the
// MFMA work half). With two waves per SIMD in ping-pong, one softmax wave
// runs beside one MFMA wave and the matrix cores idle half the time. A
// single wave also issues vector instructions well below the SIMD's rate;
// two or three softmax waves on one SIMD together get 1.35-1.6x the
// throughput of one, while an MFMA wave beside them keeps its rate.
//
// So this kernel runs 16 waves (four per SIMD) in four groups of four, 512
// query rows per workgroup. Time is cut into ticks, one workgroup barrier
// each. Group g runs the MFMA phase of key block j (PV of block j-1, QK^T of
// block j) in tick 4j + g, and the softmax of block j in the three ticks
// after it, a third of the scores per tick. So in every tick one wave of each
// SIMD drives the matrix core and three share the vector ALU (the scores
// are split 12 / 8 / 12 over the three ticks; the middle one also issues the
// DMA, which stalls the issuing wave until the load path takes it).
//
// K and V blocks (64 keys) stream through three-buffer LDS rings. In the
// second softmax tick of block j (tick 4j+g+2), every wave issues one 1 KiB
// LDS-DMA piece: groups 0-1 of K_{j+2}, groups 2-3 of V_{j+1}. K_b is read
// in ticks 4b .. 4b+3 and V_b (for PV of block b) in ticks 4b+4 .. 4b+7, so
// each target buffer was last read at tick 4j-1, before the first issue at
// 4j+2. Each wave waits for its piece at the end of its next MFMA phase
// (tick 4j+4+g), whose barrier publishes it before its first reader (tick
// 4j+8).
// ---------------------------------------------------------------------------
constexpr int kRotGroups = 4;
constexpr int kRotWaves = 4 * kRotGroups;
constexpr int kRotThreads = 64 * kRotWaves;
constexpr int kRotBR = 32 * kRotWaves;  // query rows per workgroup

template <bool CAUSAL>
__global__ __launch_bounds__(kRotThreads) __attribute__((amdgpu_waves_per_eu(4, 4))) void fwd_bf16_rot_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE,
    int H_q, int H_kv, int N_q_arg, int N_kv_arg, int n_qtiles, int xcd_remap, float c,
    const int* __restrict__ cu_q, const int* __restrict__ cu_k, int total_q, int total_k) {
  constexpr int D = 64;
  constexpr int BC = 64;                 // keys per block
  constexpr int NSUB = BC / 32;          // 32-key subtiles of S^T
  constexpr int DSUB = D / 32;           // 32-column subtiles of O^T
  constexpr int QK_STEPS = D / 16;
  constexpr int PV_STEPS = BC / 16;
  constexpr int CPR = D / 8;             // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;          // rows per 1 KiB DMA piece
  constexpr int ROW_BYTES = D * 2;
  constexpr int TILE_BYTES = BC * ROW_BYTES;    // 8 KiB: 8 pieces
  constexpr int PIECES = TILE_BYTES / 1024;
  static_assert(2 * PIECES == kRotWaves, "one DMA piece per wave and block");
  __shared__ __attribute__((aligned(1024))) uint8_t kb0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t kb1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t kb2[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vb0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vb1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vb2[TILE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;    // rotation group
  const int col = lane & 31;
  const int half = lane >> 5;
  const int G = H_q / H_kv;

  const TileAssign ta = assign_tile(blockIdx.x, n_qtiles, G, xcd_remap, (int)(gridDim.x / n_qtiles), false,
                                    CAUSAL ? 4 : 1);
  const int kvidx = ta.kvidx, gq = ta.gq;
  const int b = kvidx / H_kv;
  const int hk = kvidx % H_kv;
  const int h = hk * G + gq;
  const int tile = CAUSAL ? (n_qtiles - 1 - ta.tile_rank) : ta.tile_rank;  // heaviest first

  // layouts as in fwd_bf16_kernel (dense, or packed sequences with clamped offsets)
  int N_q = N_q_arg, N_kv = N_kv_arg;
  size_t qbase, kvbase, lbase;
  if (cu_q != nullptr) {
    const int qs = min(max(cu_q[b], 0), total_q);
    const int qe = min(max(cu_q[b + 1], qs), total_q);
    const int ks = min(max(cu_k[b], 0), total_k);
    const int ke = min(max(cu_k[b + 1], ks), total_k);
    N_q = min(qe - qs, N_q_arg);
    N_kv = ke - ks;
    qbase = (size_t(h) * total_q + qs) * D;
    kvbase = (size_t(hk) * total_k + ks) * D;
    lbase = size_t(h) * total_q + qs;
  } else {
    qbase = (size_t(b) * H_q + h) * size_t(N_q) * D;
    kvbase = (size_t(b) * H_kv + hk) * size_t(N_kv) * D;
    lbase = (size_t(b) * H_q + h) * size_t(N_q);
  }
  const int q0 = tile * kRotBR;
  if (q0 >= N_q) return;  // (whole workgroup) a tile past a short sequence
  if (N_kv == 0) {
    const int row = q0 + wave * 32 + col;
    if (row < N_q) {
      uint16_t* op = O + qbase + size_t(row) * D + half * (D / 2);
#pragma unroll
      for (int j = 0; j < D / 2; j += 4) st_global8(op + j, u32x2{0u, 0u});
      if (half == 0) LSE[lbase + row] = -INFINITY;
    }
    return;
  }
  const uint8_t* __restrict__ Kbytes = reinterpret_cast<const uint8_t*>(K + kvbase);
  const uint8_t* __restrict__ Vbytes = reinterpret_cast<const uint8_t*>(V + kvbase);

  const int wrow0 = q0 + wave * 32;
  const int qrow = wrow0 + col;
  bf16x8 qreg[QK_STEPS];
  {
    const uint16_t* qp = Q + qbase + size_t(min(qrow, N_q - 1)) * D + half * (D / 2);
#pragma unroll
    for (int t = 0; t < QK_STEPS; ++t) qreg[t] = as_bf16x8(ld_global16(qp + 8 * t));
  }
  const int nblk_all = (N_kv + BC - 1) / BC;
  int nblk = nblk_all;
  if (CAUSAL) nblk = min(nblk_all, (min(q0 + kRotBR, N_q) - 1) / BC + 1);
  auto need_mask = [&](int j) __attribute__((always_inline)) {
    const int kv0 = j * BC;
    return (CAUSAL && kv0 + BC - 1 > wrow0) || (kv0 + BC > N_kv);
  };

  // ---- LDS-DMA pieces. Piece p (0..7) of a tile covers rows RPI*p ..
  // RPI*p + RPI-1; lane l writes 16 bytes of row RPI*p + l/CPR (physical
  // chunk l%CPR, holding logical chunk (l%CPR) ^ swz(row)). The tail block
  // reads clamped rows (finite data for masked keys, nothing past the end).
  const int tail_blk = (N_kv % BC) ? N_kv / BC : -1;
  const int tail_lim = N_kv - 1 - (N_kv / BC) * BC;
  auto piece_off = [&](int p, bool is_k, int jb) __attribute__((always_inline)) {
    const int row = RPI * p + lane / CPR;
    const int ch = lane % CPR;
    const int r = (jb == tail_blk) ? min(row, tail_lim) : row;
    return uint32_t(r * ROW_BYTES + ((ch ^ (is_k ? swz_k<D>(row) : swz_v<D>(row))) * 16));
  };
  auto dma_piece = [&](int p, bool is_k, int jb, uint8_t* dst) __attribute__((always_inline)) {
    const uint8_t* src = (is_k ? Kbytes : Vbytes) + size_t(jb) * BC * ROW_BYTES;
    lds_dma16_sbase(src, piece_off(p, is_k, jb), lds_address(dst) + 1024 * p);
  };
  // this wave's piece in the loop: groups 0-1 stage K, groups 2-3 stage V
  const int my_piece = wave & (PIECES - 1);
  const bool my_k = wave < PIECES;

  // ---- LDS read offsets (as fwd_bf16_kernel at d = 64)
  const int krow = row_of_lane(col);
  int koff[QK_STEPS];
#pragma unroll
  for (int t = 0; t < QK_STEPS; ++t) koff[t] = krow * ROW_BYTES + ((((D / 16) * half + t) ^ swz_k<D>(krow)) * 16);
  const int j16 = lane & 15;
  const int vgrp = (lane & 31) >> 4;
  int voff[DSUB];
#pragma unroll
  for (int s = 0; s < DSUB; ++s) {
    const int row = 16 * half + (j16 >> 2);
    const int cc = 32 * s + 16 * vgrp + 4 * (j16 & 3);
    voff[s] = row * ROW_BYTES + (((cc >> 3) ^ swz_v<D>(row)) * 16) + (cc & 7) * 2;
  }

  float m_run = -INFINITY;
  float l_run = 0.f;
  float psum = 0.f;
  bool eager = true;
  bool moved = false;
  f32x16 oacc[DSUB];
#pragma unroll
  for (int s = 0; s < DSUB; ++s) oacc[s] = f32x16{};
  f32x16 sacc[NSUB];
  u32x4 pk[PV_STEPS];

  auto mfma_phase = [&](int j, const uint8_t* kt, const uint8_t* vt) __attribute__((always_inline)) {
    if (j >= 1) {
#pragma unroll
      for (int u = 0; u < PV_STEPS; ++u) {
        const int rbase = (32 * (u >> 1) + 8 * (u & 1)) * ROW_BYTES;
#pragma unroll
        for (int s = 0; s < DSUB; ++s)
          oacc[s] = mfma32x32x16(lds_read_tr8(vt + voff[s] + rbase, vt + voff[s] + rbase + 4 * ROW_BYTES),
                                 as_bf16x8(pk[u]), oacc[s]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
#pragma unroll
      for (int i = 0; i < PV_STEPS * DSUB; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSgDsRead, 2, 0);
      }
    }
    if (j < nblk) {
#pragma unroll
      for (int n = 0; n < NSUB; ++n) sacc[n] = f32x16{};
#pragma unroll
      for (int t = 0; t < QK_STEPS; ++t)
#pragma unroll
        for (int n = 0; n < NSUB; ++n)
          sacc[n] = mfma32x32x16(as_bf16x8(*reinterpret_cast<const u32x4*>(kt + koff[t] + n * 32 * ROW_BYTES)),
                                 qreg[t], sacc[n]);
#pragma unroll
      for (int i = 0; i < 2; ++i) __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
#pragma unroll
      for (int i = 0; i < QK_STEPS * NSUB; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
      }
    }
  };

  // Softmax of a block in three parts. Quad q (0..7) = scores
  // sacc[q/4][4(q%4) .. 4(q%4)+3], packed into pk[q/2][2(q%2)], [2(q%2)+1].
  auto exp_quad = [&](int q) __attribute__((always_inline)) {
    const int n = q >> 2, w4 = (q & 3) * 4;
    float p[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      p[e] = fast_exp2(fmaf(sacc[n][w4 + e], c, -m_run));
      psum += p[e];
    }
    pk[q >> 1][2 * (q & 1)] = cvt_pk_bf16(p[0], p[1]);
    pk[q >> 1][2 * (q & 1) + 1] = cvt_pk_bf16(p[2], p[3]);
  };
  auto block_max = [&]() __attribute__((always_inline)) {
    float mx = sacc[0][0];
#pragma unroll
    for (int n = 0; n < NSUB; ++n)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[n][i]);
    return max_xor32(mx) * c;
  };
  auto rescale_to = [&](float m_new) __attribute__((always_inline)) {
    const float alpha = fast_exp2(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int s = 0; s < DSUB; ++s)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[s][i] *= alpha;
    m_run = m_new;
  };
  auto soft1 = [&](int j) __attribute__((always_inline)) {
    if (j >= nblk) return;
    if (need_mask(j)) {
      const int last_key = CAUSAL ? min(qrow, N_kv - 1) : N_kv - 1;
      const int lim = last_key - j * BC - 16 * half;
#pragma unroll
      for (int n = 0; n < NSUB; ++n)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (32 * n + i > lim) sacc[n][i] = -INFINITY;
    }
    moved = false;
    if (eager) {
      const float m_blk = block_max();
      if (__any(m_blk > m_run + kRescaleSlack)) {
        rescale_to(fmaxf(m_run, m_blk));
        moved = true;
      }
    }
    psum = 0.f;
#pragma unroll
    for (int q = 0; q < 3; ++q) exp_quad(q);
  };
  auto soft2 = [&](int j, uint8_t* kd, uint8_t* vd) __attribute__((always_inline)) {
    if (j >= nblk) return;
    // the DMA pieces of K_{j+2} / V_{j+1} (past the end, a block again into a free buffer)
    if (my_k) dma_piece(my_piece, true, min(j + 2, nblk - 1), kd);
    else dma_piece(my_piece, false, min(j + 1, nblk - 1), vd);
#pragma unroll
    for (int q = 3; q < 5; ++q) exp_quad(q);
  };
  auto soft3 = [&](int j) __attribute__((always_inline)) {
    if (j >= nblk) return;
#pragma unroll
    for (int q = 5; q < 8; ++q) exp_quad(q);
    // a row's block sum above 2^8 (or inf / NaN): form the block max, rescale
    // and take the block's exponentials again
    if (__any(!(psum <= 256.0f))) {
      const float m_new = fmaxf(m_run, block_max());
      if (__any(m_new > m_run)) {
        rescale_to(m_new);
        psum = 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q) exp_quad(q);
        moved = true;
      }
    }
    eager = moved;
    l_run += psum;
    // keep the row sum and the packed operands in this tick
    asm volatile("" : "+v"(l_run));
#pragma unroll
    for (int u = 0; u < PV_STEPS; ++u) asm volatile("" : "+v"(pk[u]));
  };

  // ---- prologue: K_0, K_1 and V_0 (24 pieces over 16 waves)
  dma_piece(wave & 7, true, wave < 8 ? 0 : min(1, nblk - 1), wave < 8 ? kb0 : kb1);
  if (wave < 8) dma_piece(wave, false, 0, vb0);
  wait_vmem();
  __syncthreads();

  // ---- the rotation: group g waits g ticks, runs 4 ticks per block for
  // blocks 0..nblk (the extra block only finishes PV), then waits 3-g ticks;
  // every wave passes 4 (nblk + 1) + 3 barriers. Blocks are taken three at a
  // time so that every ring buffer is a compile-time choice:
  // K_j in kb[j%3], V_{j-1} in vb[(j-1)%3], DMA into kb[(j+2)%3], vb[(j+1)%3].
  for (int i = 0; i < grp; ++i) barrier_nofence();
  auto step = [&](int j, const uint8_t* kc, const uint8_t* vp, uint8_t* kd, uint8_t* vd)
      __attribute__((always_inline)) {
    mfma_phase(j, kc, vp);
    wait_vmem();  // this wave's DMA piece from the previous block
    barrier_nofence();
    soft1(j);
    barrier_nofence();
    soft2(j, kd, vd);
    barrier_nofence();
    soft3(j);
    barrier_nofence();
  };
  for (int j = 0; j <= nblk; j += 3) {
    step(j, kb0, vb2, kb2, vb1);
    if (j + 1 <= nblk) step(j + 1, kb1, vb0, kb0, vb2);
    if (j + 2 <= nblk) step(j + 2, kb2, vb1, kb1, vb0);
  }
  for (int i = grp; i < kRotGroups - 1; ++i) barrier_nofence();

  // ---- epilogue: O = O_acc / l, LSE = ln2 * (m + log2 l)
  const float l_tot = sum_xor32(l_run);
  if (qrow < N_q) {
    const float inv = 1.0f / l_tot;
    uint16_t* op = O + qbase + size_t(qrow) * D;
#pragma unroll
    for (int s = 0; s < DSUB; ++s) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        u32x2 w;
        w[0] = cvt_pk_bf16(oacc[s][4 * a + 0] * inv, oacc[s][4 * a + 1] * inv);
        w[1] = cvt_pk_bf16(oacc[s][4 * a + 2] * inv, oacc[s][4 * a + 3] * inv);
        st_global8(op + 32 * s + 8 * a + 4 * half, w);
      }
    }
    if (half == 0) LSE[lbase + qrow] = (m_run + __log2f(l_tot)) * kLn2;
  }
}

template <bool CAUSAL>
hipError_t launch_rot(const FwdParams& p, const VarlenParams* vl, hipStream_t stream) {
  const int n_qtiles = (p.N_q + kRotBR - 1) / kRotBR;
  const long long nwg = (long long)n_qtiles * p.B * p.H_q;
  const int xcd_remap = ((p.B * p.H_kv) % 8 == 0) ? 1 : 0;
  const float c = fmaxf(p.scale * kLog2e, 1.17549435e-38f);
  hipLaunchKernelGGL((fwd_bf16_rot_kernel<CAUSAL>), dim3((unsigned)nwg), dim3(kRotThreads), 0, stream,
                     static_cast<const uint16_t*>(p.q), static_cast<const uint16_t*>(p.k),
                     static_cast<const uint16_t*>(p.v), static_cast<uint16_t*>(p.o), p.lse,
                     p.H_q, p.H_kv, p.N_q, p.N_kv, n_qtiles, xcd_remap, c,
                     vl ? vl->cu_q : nullptr, vl ? vl->cu_k : nullptr, vl ? vl->total_q : 0,
                     vl ? vl->total_k : 0);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t stream) {
  if (p.d == 128) return p.causal ? launch<128, true>(p, nullptr, stream) : launch<128, false>(p, nullptr, stream);
  return p.causal ? launch_rot<true>(p, nullptr, stream) : launch_rot<false>(p, nullptr, stream);
}

hipError_t launch_fwd_varlen_bf16(const FwdParams& p, const VarlenParams& vl, hipStream_t stream) {
  if (p.d == 128) return p.causal ? launch<128, true>(p, &vl, stream) : launch<128, false>(p, &vl, stream);
  return p.causal ? launch_rot<true>(p, &vl, stream) : launch_rot<false>(p, &vl, stream);
}

}  // namespace fa

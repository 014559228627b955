// Attention forward for FP8 (OCP e4m3) inputs with one scale per block of 128
// rows, on the gfx950 FP8 matrix instruction (v_mfma_*_32x32x64_f8f6f4, twice
// the bf16 rate). Output O in bf16 and the float32 logsumexp, as the bf16 path.
//
// Method: the same Q-stationary blockwise online softmax as the bf16 forward
// ("深度学习进阶（三十一）FlashAttention：IO 感知的精确注意力" (rkmt.cn blog)
// §2.2). Low precision is one of the design axes the overview page lists,
// with the warning that scales and errors must be checked ("Flash-Attention"
// (Awesome System Papers Wiki), 设计空间与取舍 / design space); FP8 support
// is one of FlashAttention-3's additions (the version comparison tables of
// the rkmt.cn blog and of "FlashAttention" (LLM Inference Handbook)).
//
// Inputs (codes as produced by fa_quantize_fp8):
//   q8 [B][H_q][N_q][D], k8 and v8 [B][H_kv][N_kv][D]  row-major e4m3 codes
//   *_descale [B][H][ceil(N/128)] float32              value = code * descale of its row block
//
// Arithmetic:
//  * S^T = K Q^T on the FP8 MFMA (exact products, float32 sums); the block's
//    scalar factor c_j = qd * kd_j * scale * log2(e) (one Q block per wave,
//    one K block per 64-key block) is applied inside the exponent's FMA.
//  * P is rounded to e4m3 for the PV product. The V block scale rides on P:
//    x = p * cv_j with cv_j = 8 * vd_j / vd_max, folded into the exponent as
//    + log2(cv_j), so that the raw V codes feed the MFMA and the whole output
//    is multiplied by vd_max / 8 once at the end. The row sums l use the
//    float32 x before rounding (divided by cv_j per block), so the LSE is as
//    accurate as the bf16 path's; only the numerator sees the rounding of P.
//  * The block max is formed only when needed (as in the bf16 forward): a
//    block whose lane sums of x stay within 2^8 keeps the running max, since
//    then every x <= 256 is inside the e4m3 range (448). With cv_j <= 8 the 32
//    values of a lane sum to at most 2^8 against an exact max, so only a max
//    that rose makes a block take its exponentials twice. The running max
//    never exceeds the row's final max, so x is never smaller than against the
//    exact max. Error of one output element:
//    |dO| <= 2^-4 * sum_j max(w_j, 2^-6 / (cv_j * L)) * |v_j| with w the exact
//    probabilities and L the sum of exp(s - max) (rounding to nearest of x
//    costs at most 2^-4 * x for normal x and 2^-10 below 2^-6).
//
// gfx950 mapping: as the bf16 forward (8 waves in two ping-pong groups of 4,
// 256 query rows per workgroup, LDS-DMA double buffering issued between the
// exponentials of group B, one fence-free barrier per block, MFMA phases at
// wave priority 2 and group B's vector phase at 1), with:
//  * the FP8 MFMA operand: lane l holds row l%32 and k = 32*(l/32) + byte;
//    S^T tile n (keys 32n .. 32n+31, A-row permutation row_of_lane) leaves
//    keys 32n + 16g + i in register i of lane half g, so the 32 P bytes of a
//    lane half for a 64-key PV step are keys {16g .. 16g+15, 32+16g .. 32+16g+15};
//  * V row-major like K (contiguous tile loads): the V^T operand of lane
//    (d row r, half g) is four ds_read_b64_tr_b8, each handing the lane 8
//    consecutive keys of its column (in each 16-lane group, output lane i
//    byte k is byte i % 8 of the 8 bytes addressed by lane 2k + i / 8).

#include <type_traits>

#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBR = 32 * kWaves;        // query rows per workgroup
constexpr int kQuantRows = 128;         // rows per scale block
constexpr float kRescaleSlack = 2.0f;   // log2 units: x <= 2^2 * cv <= 32 after a rescale
constexpr float kCvMax = 8.0f;          // cv_j = 8 * vd_j / vd_max: 32 x values of an exact max sum to <= 2^8
constexpr float kCvMin = 9.5367431640625e-07f;  // 2^-20: zero V blocks keep l finite

constexpr int kSgValu = 0x402;
constexpr int kSgMfma = 0x008;
constexpr int kSgVmem = 0x010;
constexpr int kSgDsRead = 0x100;

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  // e4m3 x e4m3 -> f32, unit block scales (E8M0 127 = 2^0)
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Four floats -> four e4m3 codes (round to nearest even, no saturation),
// first value in the lowest byte.
__device__ __forceinline__ int cvt_fp8x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// Maximum over all 64 lanes of a wave (every lane gets the result).
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return max_xor32(x);
}

template <int D>
struct Fp8Cfg {
  static constexpr int BC = 64;                  // keys per block
  static constexpr int NSUB = BC / 32;           // 32-key subtiles of S^T
  static constexpr int DSUB = D / 32;            // 32-row subtiles of O^T
  static constexpr int QK_STEPS = D / 64;        // MFMA k-steps over the head dimension
  static constexpr int PV_STEPS = BC / 64;       // MFMA k-steps over keys
  static constexpr int K_CPR = D / 16;           // 16-byte chunks per K row
  static constexpr int K_RPI = 64 / K_CPR;       // K rows per 1 KiB DMA instruction
  static constexpr int TILE_BYTES = BC * D;      // K tile and V^T tile
  static constexpr int DMA_PER_WAVE = TILE_BYTES / 1024 / 4;
};

// Chunk swizzles, chosen so that the 16 lanes of one ds_read_b128 phase hit
// 16 distinct 16-byte bank groups.
//  K (rows of D bytes): a phase reads rows row_of_lane(0..15) or (16..31) at
//  one logical chunk.
template <int D>
__device__ __forceinline__ int swz_k8(int row) {
  if constexpr (D == 128) return ((row >> 1) & 3) | ((row >> 2) & 4);
  else return ((row >> 2) & 1) | ((row >> 3) & 2);
}
//  V (rows of D bytes) for ds_read_b64_tr_b8: a 32-lane phase reads 8
//  consecutive key rows x 2 logical chunks.
template <int D>
__device__ __forceinline__ int swz_vr8(int row) {
  if constexpr (D == 128) return ((row >> 1) & 3) << 1;
  else return ((row >> 2) & 1) << 1;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_fp8_kernel(
    const uint8_t* __restrict__ Q, const float* __restrict__ QD, const uint8_t* __restrict__ K,
    const float* __restrict__ KD, const uint8_t* __restrict__ V, const float* __restrict__ VD,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int H_q, int H_kv, int N_q, int N_kv,
    int n_qtiles, int xcd_remap, float scale_log2) {
  using C = Fp8Cfg<D>;
  constexpr int BC = C::BC;
  constexpr int NSUB = C::NSUB;
  __shared__ __attribute__((aligned(1024))) uint8_t kb0[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t kb1[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vb0[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vb1[C::TILE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int gw = wave & 3;
  const int col = lane & 31;
  const int half = lane >> 5;
  const int G = H_q / H_kv;

  // causal tiles differ in cost: deal them rank by rank over groups of four
  // heads so that consecutive workgroups cost the same
  const TileAssign ta = assign_tile(blockIdx.x, n_qtiles, G, xcd_remap, (int)(gridDim.x / n_qtiles), false,
                                    CAUSAL ? 4 : 1);
  const int kvidx = ta.kvidx, gq = ta.gq, tile_rank = ta.tile_rank;
  const int b = kvidx / H_kv;
  const int hk = kvidx % H_kv;
  const int h = hk * G + gq;
  const int tile = CAUSAL ? (n_qtiles - 1 - tile_rank) : tile_rank;
  const int q0 = tile * kBR;

  const size_t qhead = size_t(b) * H_q + h;
  const size_t kvhead = size_t(b) * H_kv + hk;
  const int nbq = (N_q + kQuantRows - 1) / kQuantRows;
  const int nbk = (N_kv + kQuantRows - 1) / kQuantRows;
  const uint8_t* __restrict__ Kh = K + kvhead * size_t(N_kv) * D;
  const uint8_t* __restrict__ Vh = V + kvhead * size_t(N_kv) * D;
  const float* __restrict__ kd = KD + kvhead * nbk;
  const float* __restrict__ vd = VD + kvhead * nbk;

  // ---- Q tile into registers (B operand of S^T = K Q^T): lane (column q,
  // half g) holds bytes 64t + 32g .. 64t + 32g + 31 of its query row.
  const int wrow0 = q0 + wave * 32;
  const int qrow = wrow0 + col;
  i32x8 qreg[C::QK_STEPS];
  {
    const uint8_t* qp = Q + (qhead * N_q + size_t(min(qrow, N_q - 1))) * D + 32 * half;
#pragma unroll
    for (int t = 0; t < C::QK_STEPS; ++t) {
      const u32x4 lo = ld_global16(qp + 64 * t);
      const u32x4 hi = ld_global16(qp + 64 * t + 16);
      qreg[t] = i32x8{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]), int(hi[0]), int(hi[1]), int(hi[2]),
                      int(hi[3])};
    }
  }
  const float qd = QD[qhead * nbq + min(wrow0, N_q - 1) / kQuantRows];

  // ---- largest V block scale of the head (every lane of every wave)
  float vmax = 0.f;
  for (int i = lane; i < nbk; i += 64) vmax = fmaxf(vmax, vd[i]);
  vmax = wave_max(vmax);
  // (floor 2^-100: keeps kCvMax / vmax finite when every V block is zero)
  const float vmax_safe = fmaxf(vmax, 7.88860905e-31f);
  const float inv_vmax = kCvMax / vmax_safe;

  const int nblk_all = (N_kv + BC - 1) / BC;
  int nblk = nblk_all;
  if (CAUSAL) {
    const int last_row = min(q0 + kBR, N_q) - 1;
    nblk = min(nblk_all, last_row / BC + 1);
  }
  auto need_mask = [&](int j) __attribute__((always_inline)) {
    const int kv0 = j * BC;
    return (CAUSAL && kv0 + BC - 1 > wrow0) || (kv0 + BC > N_kv);
  };

  // ---- LDS-DMA staging by the 4 waves of group B: K and V tiles of BC rows
  // of D bytes (rows past N_kv read the last key instead), each with its own
  // chunk swizzle.
  const int tail_blk = (N_kv % BC) ? N_kv / BC : -1;
  const int tail_lim = N_kv - 1 - (N_kv / BC) * BC;
  uint32_t dma_koff[C::DMA_PER_WAVE], dma_voff[C::DMA_PER_WAVE], dma_cut[C::DMA_PER_WAVE];
#pragma unroll
  for (int i = 0; i < C::DMA_PER_WAVE; ++i) {
    const int ig = gw * C::DMA_PER_WAVE + i;
    const int row = C::K_RPI * ig + lane / C::K_CPR;
    const int pch = lane % C::K_CPR;
    dma_koff[i] = row * D + (pch ^ swz_k8<D>(row)) * 16;
    dma_voff[i] = row * D + (pch ^ swz_vr8<D>(row)) * 16;
    dma_cut[i] = (row - min(row, tail_lim)) * D;
  }
  auto dma_slot = [&](int i, int jk, int jv, uint8_t* kdst, uint8_t* vdst) __attribute__((always_inline)) {
    const bool is_k = i < C::DMA_PER_WAVE;
    const int ii = is_k ? i : i - C::DMA_PER_WAVE;
    const int jb = is_k ? jk : jv;
    const uint8_t* src = (is_k ? Kh : Vh) + size_t(jb) * BC * D;
    uint32_t off = is_k ? dma_koff[ii] : dma_voff[ii];
    if (jb == tail_blk) off -= dma_cut[ii];
    lds_dma16_sbase(src, off, lds_address(is_k ? kdst : vdst) + 1024 * (gw * C::DMA_PER_WAVE + ii));
  };
  auto dma_k0 = [&](uint8_t* kdst) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < C::DMA_PER_WAVE; ++i) dma_slot(i, 0, 0, kdst, kdst);
  };

  // ---- per-lane LDS read offsets
  // K: row row_of_lane(col) (+32 per subtile n), logical chunks 4t + 2*half + {0,1}.
  const int krow = row_of_lane(col);
  int koff[C::QK_STEPS][2];
#pragma unroll
  for (int t = 0; t < C::QK_STEPS; ++t)
#pragma unroll
    for (int e = 0; e < 2; ++e) koff[t][e] = krow * D + (((4 * t + 2 * half + e) ^ swz_k8<D>(krow)) * 16);
  // V^T of subtile s: read m (m = 0..3) covers the keys 32 (m/2) + 16 half +
  // 8 (m%2) + k, k = 0..7; this lane addresses key row (that run's start) +
  // j/2 and column 32 s + 16 ((lane/16) % 2) + 8 (j % 2), j = lane % 16. The
  // swizzle depends only on j/2 (runs start at multiples of 8), so the run
  // start is a constant offset.
  int voff[C::DSUB];
  {
    const int j = lane & 15;
    const int qh = (lane >> 4) & 1;
    const int r8 = j >> 1;
#pragma unroll
    for (int s = 0; s < C::DSUB; ++s) {
      const int cc = 32 * s + 16 * qh + 8 * (j & 1);
      voff[s] = (16 * half + r8) * D + (((cc >> 4) ^ swz_vr8<D>(r8)) * 16) + (cc & 15);
    }
  }

  float m_run = -INFINITY;
  float l_run = 0.f;
  f32x16 oacc[C::DSUB];
#pragma unroll
  for (int s = 0; s < C::DSUB; ++s) oacc[s] = f32x16{};
  f32x16 sacc[NSUB];
  i32x8 pk[C::PV_STEPS];

  auto pv_part = [&](const uint8_t* vt) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < C::PV_STEPS; ++u) {
#pragma unroll
      for (int s = 0; s < C::DSUB; ++s) {
        i32x2 r[4];
#pragma unroll
        for (int m = 0; m < 4; ++m)
          r[m] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (LDS_AS i32x2*)(vt + voff[s] + (64 * u + 32 * (m >> 1) + 8 * (m & 1)) * D));
        const i32x8 a = i32x8{r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
        oacc[s] = mfma_fp8(a, pk[u], oacc[s]);
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
        const u32x4 lo = *reinterpret_cast<const u32x4*>(kt + koff[t][0] + n * 32 * D);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(kt + koff[t][1] + n * 32 * D);
        const i32x8 a = i32x8{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]),
                              int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
        sacc[n] = mfma_fp8(a, qreg[t], sacc[n]);
      }
    }
  };
  // The MFMA phase runs at raised wave priority, so that its LDS reads and
  // MFMAs win issue arbitration against the vector phases on the same SIMD
  // (the vector phase is the longer one; the matrix core should not wait for
  // it).
  auto mfma_phase = [&](int j, const uint8_t* kt, const uint8_t* vt) __attribute__((always_inline)) {
    const bool do_pv = j >= 1;
    const bool do_qk = j < nblk;
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(2);
    __builtin_amdgcn_sched_barrier(0);
    if (do_pv) {
      pv_part(vt);
#pragma unroll
      for (int i = 0; i < 8; ++i) __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
#pragma unroll
      for (int i = 0; i < C::PV_STEPS * C::DSUB; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSgDsRead, 2, 0);
      }
    }
    if (do_qk) {
      qk_part(kt);
#pragma unroll
      for (int i = 0; i < 4; ++i) __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
#pragma unroll
      for (int i = 0; i < C::QK_STEPS * NSUB; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSgDsRead, 2, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
  };

  // Vector phase of block j: mask, block max and rescale when needed,
  // exponentials with the V scale folded in, float32 row sums, e4m3 packing.
  // The block max is formed first only after a block that moved the running
  // max (and for the first block). Otherwise the exponentials run against the
  // running max: a lane's sum of x = p * cv within 2^8 bounds every x by 2^8,
  // inside the e4m3 range (448), and the block stands. A larger sum (a max
  // that rose) forms the block max, rescales, and takes the block again.
  constexpr int kGroups = NSUB * 4;                // groups of 4 scores per lane
  constexpr int kDmaSlots = 2 * C::DMA_PER_WAVE;
  constexpr int kGroupsPerSlot = kGroups / kDmaSlots;
  static_assert(kGroupsPerSlot * kDmaSlots == kGroups, "DMA slots per exponential group");
  auto no_dma = [](int) __attribute__((always_inline)) {};
  bool eager = true;
  // factors of the current 128-key scale block (two key blocks share one)
  int f_kblk = -1;
  float f_c = 0.f, f_cv = 1.f, f_lcv = 0.f, f_rcv = 1.f;
  auto valu_phase = [&](int j, auto&& issue, auto has_dma) __attribute__((always_inline)) {
    constexpr bool kDma = decltype(has_dma)::value;
    if constexpr (!kDma) {
      if (j >= nblk) return;
    }
    const int kblk = (j * BC) / kQuantRows;
    if (kblk != f_kblk) {
      f_kblk = kblk;
      f_c = fmaxf(qd * kd[kblk] * scale_log2, 1.17549435e-38f);
      f_cv = fmaxf(vd[kblk] * inv_vmax, kCvMin);
      f_lcv = __log2f(f_cv);
      f_rcv = __builtin_amdgcn_rcpf(f_cv);  // v_rcp_f32: 1 ulp
    }
    const float c = f_c;
    const float lcv = f_lcv;
    if (need_mask(j)) {
      const int last_key = CAUSAL ? min(qrow, N_kv - 1) : N_kv - 1;
      const int lim = last_key - j * BC - 16 * half;
#pragma unroll
      for (int n = 0; n < NSUB; ++n)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (32 * n + i > lim) sacc[n][i] = -INFINITY;
    }
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
    float psum = 0.f;
    auto exps = [&](auto&& iss, auto dma_here) __attribute__((always_inline)) {
      constexpr bool kD = decltype(dma_here)::value;
      const float bias = lcv - m_run;
      psum = 0.f;
#pragma unroll
      for (int gi = 0; gi < kGroups; ++gi) {
        const int n = gi >> 2;
        const int v4 = gi & 3;
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[e] = fast_exp2(fmaf(sacc[n][4 * v4 + e], c, bias));
          psum += x[e];
        }
        pk[n >> 1][4 * (n & 1) + v4] = cvt_fp8x4(x[0], x[1], x[2], x[3]);
        if constexpr (kD) {
          if ((gi % kGroupsPerSlot) == kGroupsPerSlot - 1) iss(gi / kGroupsPerSlot);
        }
      }
      if constexpr (kD) {
#pragma unroll
        for (int i = 0; i < kDmaSlots; ++i) {
          __builtin_amdgcn_sched_group_barrier(kSgValu, 14 * kGroupsPerSlot, 0);
          __builtin_amdgcn_sched_group_barrier(kSgVmem, 1, 0);
        }
      }
    };
    bool moved = false;
    if (eager) {
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
    l_run += psum * f_rcv;
    // keep the row sum in this phase: left alone, the compiler sinks the
    // 32 dependent adds past the end of the phase into the next MFMA phase
    asm volatile("" : "+v"(l_run));
  };

  auto block_a = [&](int j, const uint8_t* k_cur, const uint8_t* v_prev) __attribute__((always_inline)) {
    mfma_phase(j, k_cur, v_prev);
    valu_phase(j, no_dma, std::false_type{});
    barrier_nofence();
  };
  auto block_b = [&](int j, const uint8_t* k_cur, const uint8_t* v_prev, uint8_t* k_dma, uint8_t* v_dma)
      __attribute__((always_inline)) {
    const int jk = min(j + 1, nblk - 1);
    const int jv = min(j, nblk - 1);
    // B's vector phase, which the block waits for, takes issue precedence
    // over A's, which starts as soon as A's MFMA phase ends
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
    __builtin_amdgcn_sched_barrier(0);
    valu_phase(j - 1, [&](int i) __attribute__((always_inline)) {
      dma_slot(i, jk, jv, k_dma, v_dma); }, std::true_type{});
    mfma_phase(j, k_cur, v_prev);
    wait_vmem();
    barrier_nofence();
  };

  if (grp == 1) {
    dma_k0(kb0);
    wait_vmem();
  }
  __syncthreads();

  if (grp == 0) {
    for (int j = 0; j <= nblk; j += 2) {
      block_a(j, kb0, vb1);
      if (j + 1 <= nblk) block_a(j + 1, kb1, vb0);
    }
  } else {
    {
      const int jk = min(1, nblk - 1);
#pragma unroll
      for (int i = 0; i < kDmaSlots; ++i) dma_slot(i, jk, 0, kb1, vb0);
      mfma_phase(0, kb0, vb1);
      wait_vmem();
      barrier_nofence();
    }
    for (int j = 1; j <= nblk; j += 2) {
      block_b(j, kb1, vb0, kb0, vb1);
      if (j + 1 <= nblk) block_b(j + 1, kb0, vb1, kb1, vb0);
    }
  }

  // ---- epilogue: O = O_acc * (vd_max / kCvMax) / l, LSE = ln2 * (m + log2 l)
  const float l_tot = sum_xor32(l_run);
  if (qrow < N_q) {
    const float f = (vmax_safe / kCvMax) / l_tot;
    uint16_t* op = O + (qhead * N_q + size_t(qrow)) * D;
#pragma unroll
    for (int s = 0; s < C::DSUB; ++s) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        u32x2 w;
        w[0] = cvt_pk_bf16(oacc[s][4 * a + 0] * f, oacc[s][4 * a + 1] * f);
        w[1] = cvt_pk_bf16(oacc[s][4 * a + 2] * f, oacc[s][4 * a + 3] * f);
        st_global8(op + 32 * s + 8 * a + 4 * half, w);
      }
    }
    if (half == 0) LSE[qhead * N_q + qrow] = (m_run + __log2f(l_tot)) * kLn2;
  }
}

// ---- block quantizer: one workgroup per (batch, head, 128-row block)
constexpr int kQThreads = 256;

template <int D, bool DMAJOR>
__global__ __launch_bounds__(kQThreads) void quantize_fp8_kernel(const uint16_t* __restrict__ X,
                                                                 uint8_t* __restrict__ codes,
                                                                 float* __restrict__ descale, int N, int n_pad) {
  __shared__ float red[kQThreads / 64];
  __shared__ __attribute__((aligned(16))) uint8_t tile[DMAJOR ? kQuantRows * D : 16];
  const int nb = (N + kQuantRows - 1) / kQuantRows;
  const int blk = blockIdx.x % nb;
  const size_t head = blockIdx.x / nb;
  const int r0 = blk * kQuantRows;
  const int rows = min(kQuantRows, N - r0);
  const uint16_t* xb = X + (head * N + r0) * D;
  constexpr int kPer = kQuantRows * D / kQThreads;  // elements per thread (64 or 32)
  constexpr int kVec = 8;                           // bf16 per 16-byte load
  // thread t handles elements e = (t + kQThreads * i) * 8 .. +7 of the block
  float xv[kPer];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < kPer / kVec; ++i) {
    const int e = (threadIdx.x + kQThreads * i) * kVec;
    const int r = e / D;
    u32x4 w = u32x4{0u, 0u, 0u, 0u};
    if (r < rows) w = ld_global16(xb + e);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      xv[i * kVec + 2 * k] = __uint_as_float(w[k] << 16);
      xv[i * kVec + 2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
#pragma unroll
    for (int k = 0; k < kVec; ++k) amax = fmaxf(amax, fabsf(xv[i * kVec + k]));
  }
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float inv = 448.0f / amax;  // correctly rounded float32 division
  const bool zero = !(fabsf(inv) <= 3.40282347e+38f);  // amax = 0 or too small: all codes 0
  if (threadIdx.x == 0) descale[head * nb + blk] = amax / 448.0f;
#pragma unroll
  for (int i = 0; i < kPer / kVec; ++i) {
    const int e = (threadIdx.x + kQThreads * i) * kVec;
    const int r = e / D;
    uint32_t w[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      float y[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float t = zero ? 0.f : xv[i * kVec + 4 * k + q] * inv;
        y[q] = fminf(fmaxf(t, -448.0f), 448.0f);  // the conversion does not saturate
      }
      w[k] = uint32_t(cvt_fp8x4(y[0], y[1], y[2], y[3]));
    }
    if constexpr (!DMAJOR) {
      if (r < rows) st_global8(codes + (head * N + r0) * D + e, u32x2{w[0], w[1]});
    } else {
      *reinterpret_cast<u32x2*>(tile + e) = u32x2{w[0], w[1]};  // rows past N hold zero codes
    }
  }
  if constexpr (DMAJOR) {
    __syncthreads();
    // codes^T: output row c (head dimension), keys r0 .. r0 + 127 (inside n_pad)
    constexpr int kSeg = kQuantRows / 16;  // 16-byte segments per output row
    uint8_t* ob = codes + head * size_t(D) * n_pad + r0;
    for (int it = threadIdx.x; it < D * kSeg; it += kQThreads) {
      const int c = it / kSeg;
      const int seg = it % kSeg;
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t v = 0;
#pragma unroll
        for (int bsh = 0; bsh < 4; ++bsh) v |= uint32_t(tile[(16 * seg + 4 * q + bsh) * D + c]) << (8 * bsh);
        w[q] = v;
      }
      *reinterpret_cast<u32x4*>(ob + size_t(c) * n_pad + 16 * seg) = u32x4{w[0], w[1], w[2], w[3]};
    }
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const Fp8FwdParams& p, hipStream_t stream) {
  const int n_qtiles = (p.N_q + kBR - 1) / kBR;
  const long long nwg = (long long)n_qtiles * p.B * p.H_q;
  const int xcd_remap = ((p.B * p.H_kv) % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL>), dim3((unsigned)nwg), dim3(kThreads), 0, stream,
                     static_cast<const uint8_t*>(p.q), p.q_descale, static_cast<const uint8_t*>(p.k), p.k_descale,
                     static_cast<const uint8_t*>(p.v), p.v_descale, static_cast<uint16_t*>(p.o), p.lse, p.H_q,
                     p.H_kv, p.N_q, p.N_kv, n_qtiles, xcd_remap, p.scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp8(const Fp8FwdParams& p, hipStream_t stream) {
  if (p.d == 128) return p.causal ? launch<128, true>(p, stream) : launch<128, false>(p, stream);
  return p.causal ? launch<64, true>(p, stream) : launch<64, false>(p, stream);
}

hipError_t launch_quantize_fp8(const void* x, void* codes, float* descale, int B, int H, int N, int d, int d_major,
                               hipStream_t stream) {
  const int nb = (N + kQuantRows - 1) / kQuantRows;
  const long long nwg = (long long)B * H * nb;
  const uint16_t* xs = static_cast<const uint16_t*>(x);
  uint8_t* cs = static_cast<uint8_t*>(codes);
  const int n_pad = fp8_v_pad(N);
  if (d == 128) {
    if (d_major)
      hipLaunchKernelGGL((quantize_fp8_kernel<128, true>), dim3((unsigned)nwg), dim3(kQThreads), 0, stream, xs, cs,
                         descale, N, n_pad);
    else
      hipLaunchKernelGGL((quantize_fp8_kernel<128, false>), dim3((unsigned)nwg), dim3(kQThreads), 0, stream, xs, cs,
                         descale, N, n_pad);
  } else {
    if (d_major)
      hipLaunchKernelGGL((quantize_fp8_kernel<64, true>), dim3((unsigned)nwg), dim3(kQThreads), 0, stream, xs, cs,
                         descale, N, n_pad);
    else
      hipLaunchKernelGGL((quantize_fp8_kernel<64, false>), dim3((unsigned)nwg), dim3(kQThreads), 0, stream, xs, cs,
                         descale, N, n_pad);
  }
  return hipGetLastError();
}

}  // namespace fa

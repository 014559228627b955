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
//  * Workgroup = 4 wave64s, 128 query rows (32 per wave). One workgroup per
//    (batch, query head, 128-row tile); grid order puts the heaviest causal
//    tiles first and keeps all tiles of one key/value head on one XCD.
//  * Contractions on v_mfma_f32_32x32x16_bf16 with fp32 accumulation. The
//    scores are computed transposed, S^T = K Q^T (K as the A operand, Q as B),
//    so that a lane owns one query column; P^T then feeds O^T = V^T P^T as the
//    B operand straight from the accumulator registers, and every per-row
//    quantity (max, sum, rescale factor) is lane-local. The two halves of a
//    wave hold disjoint keys of the same query and meet through one
//    v_permlane32_swap.
//  * K and V blocks come from HBM in 16-byte loads (prefetched one block
//    ahead into registers) and are written to a double-buffered LDS: K as
//    rows with XOR-swizzled 16-byte chunks, V transposed (4x8 register
//    transpose) so that the V^T operand is one 16-byte LDS read per MFMA.
//  * Softmax in base 2: scores are multiplied by scale*log2(e) inside one FMA
//    and exponentiated with v_exp_f32; LSE is converted back with ln 2.
//  * Causal: K/V blocks past the tile's last row are never loaded; waves whose
//    rows all precede a block skip it; masking runs only on blocks that cross
//    the diagonal or the end of the keys.

#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kBR = 128;     // query rows per workgroup
constexpr int kThreads = 256;

template <int D>
struct FwdCfg {
  static constexpr int BC = 8192 / D;             // keys per block: 64 (d=128), 128 (d=64)
  static constexpr int NSUB = BC / 32;            // 32-key subtiles of S^T
  static constexpr int DSUB = D / 32;             // 32-column subtiles of O^T
  static constexpr int QK_STEPS = D / 16;         // MFMA k-steps over the head dimension
  static constexpr int PV_STEPS = BC / 16;        // MFMA k-steps over keys
  static constexpr int KCHUNKS = D / 8;           // 16-byte chunks per K row
  static constexpr int K_LOADS = BC * D / 8 / kThreads;  // K chunks per thread per block
  static constexpr int TILE = BC * D;             // elements in one K or V^T buffer
};

// K row r keeps chunk c at c ^ swz_k(r): the 8 rows read together by lanes
// 8a..8a+7 of the S^T A operand get 8 distinct bank groups.
__device__ __forceinline__ int swz_k(int r) { return (r & 3) | ((r >> 2) & 4); }
// V^T row r (a head-dimension column of V) keeps key chunk c at c ^ swz_v(r).
__device__ __forceinline__ int swz_v(int r) { return (r ^ (r >> 3)) & 7; }

// Key held by A-operand row m of a 32-key subtile. With this order the S^T
// accumulator register i of lane half g holds key 16*g + i, so each lane's
// probabilities come out as runs of 8 consecutive keys -- the layout of the
// B operand of the P V contraction.
__device__ __forceinline__ int key_of_row(int m) { return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3); }

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE,
    int H_q, int H_kv, int N_q, int N_kv, int n_qtiles, int xcd_remap, float c) {
  using C = FwdCfg<D>;
  constexpr int BC = C::BC;
  __shared__ __attribute__((aligned(16))) uint16_t ks[2][C::TILE];
  __shared__ __attribute__((aligned(16))) uint16_t vts[2][C::TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;   // query column of this lane (and MFMA row for A operands)
  const int half = lane >> 5;  // lane half: key half for S^T, d half for the Q/K operands
  const int G = H_q / H_kv;

  // ---- schedule: workgroup -> (batch, head, query tile)
  const int L = blockIdx.x;
  int tile_rank, kvidx, gq;
  if (xcd_remap) {
    // Workgroups are dealt to the 8 XCDs round-robin; give each XCD whole
    // key/value heads (with all their query heads and tiles) so K/V is shared
    // through that XCD's L2.
    const int xcd = L & 7;
    const int s = L >> 3;
    tile_rank = s % n_qtiles;
    const int head_local = s / n_qtiles;
    kvidx = xcd + 8 * (head_local / G);
    gq = head_local % G;
  } else {
    tile_rank = L % n_qtiles;
    const int hi = L / n_qtiles;
    kvidx = hi / G;
    gq = hi % G;
  }
  const int b = kvidx / H_kv;
  const int hk = kvidx % H_kv;
  const int h = hk * G + gq;
  const int tile = CAUSAL ? (n_qtiles - 1 - tile_rank) : tile_rank;  // heaviest first
  const int q0 = tile * kBR;

  const size_t qbase = (size_t(b) * H_q + h) * size_t(N_q) * D;
  const size_t kvbase = (size_t(b) * H_kv + hk) * size_t(N_kv) * D;
  const uint16_t* __restrict__ Kh = K + kvbase;
  const uint16_t* __restrict__ Vh = V + kvbase;

  // ---- Q tile into registers: B operand of S^T = K Q^T (read once)
  const int wrow0 = q0 + wave * 32;
  const int qrow = wrow0 + col;
  bf16x8 qreg[C::QK_STEPS];
  {
    const uint16_t* qp = Q + qbase + size_t(min(qrow, N_q - 1)) * D + half * (D / 2);
#pragma unroll
    for (int t = 0; t < C::QK_STEPS; ++t) qreg[t] = as_bf16x8(ld_global16(qp + 8 * t));
  }

  // ---- number of K/V blocks this workgroup visits
  const int nblk_all = (N_kv + BC - 1) / BC;
  int nblk = nblk_all;
  if (CAUSAL) {
    const int last_row = min(q0 + kBR, N_q) - 1;
    nblk = min(nblk_all, last_row / BC + 1);
  }
  const int wlast = min(wrow0 + 31, N_q - 1);  // last valid row of this wave (< wrow0 if none)

  // ---- staging of one K/V block: HBM -> registers -> LDS
  u32x4 kpre[C::K_LOADS];
  u32x4 vpre[4];
  const int vkg = tid / (D / 8);  // V: 4-key group
  const int vdg = tid % (D / 8);  // V: 8-column group

  auto load_block = [&](int j) {
    const int kv0 = j * BC;
#pragma unroll
    for (int r = 0; r < C::K_LOADS; ++r) {
      const int ci = tid + kThreads * r;
      const int row = ci / C::KCHUNKS;
      const int ch = ci % C::KCHUNKS;
      const int krow = min(kv0 + row, N_kv - 1);
      kpre[r] = ld_global16(Kh + size_t(krow) * D + ch * 8);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int vrow = min(kv0 + 4 * vkg + r, N_kv - 1);
      vpre[r] = ld_global16(Vh + size_t(vrow) * D + vdg * 8);
    }
  };

  auto store_block = [&](int buf) {
#pragma unroll
    for (int r = 0; r < C::K_LOADS; ++r) {
      const int ci = tid + kThreads * r;
      const int row = ci / C::KCHUNKS;
      const int ch = ci % C::KCHUNKS;
      st_lds16(ks[buf], row * D + ((ch ^ swz_k(row)) * 8), kpre[r]);
    }
    // 4 keys x 8 columns -> 8 columns x 4 keys
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int w = e >> 1;
      const int sh = (e & 1) * 16;
      const uint32_t x0 = (vpre[0][w] >> sh) & 0xffffu;
      const uint32_t x1 = (vpre[1][w] >> sh) & 0xffffu;
      const uint32_t x2 = (vpre[2][w] >> sh) & 0xffffu;
      const uint32_t x3 = (vpre[3][w] >> sh) & 0xffffu;
      u32x2 packed;
      packed[0] = x0 | (x1 << 16);
      packed[1] = x2 | (x3 << 16);
      const int row = 8 * vdg + e;
      st_lds8(vts[buf], row * BC + (((vkg >> 1) ^ swz_v(row)) * 8) + (vkg & 1) * 4, packed);
    }
  };

  // ---- online-softmax state (per query column, identical in both lane halves
  // except l, which each half accumulates over its own keys)
  float m_run = -INFINITY;
  float l_run = 0.f;
  f32x16 oacc[C::DSUB];
#pragma unroll
  for (int s = 0; s < C::DSUB; ++s) oacc[s] = f32x16{};

  const int krow_a = key_of_row(col);

  load_block(0);
  store_block(0);
  __syncthreads();

  for (int j = 0; j < nblk; ++j) {
    const int buf = j & 1;
    if (j + 1 < nblk) load_block(j + 1);
    const int kv0 = j * BC;
    const bool active = (wrow0 < N_q) && (!CAUSAL || kv0 <= wlast);
    if (active) {
      // S^T = K_j Q^T
      f32x16 sacc[C::NSUB];
#pragma unroll
      for (int n = 0; n < C::NSUB; ++n) sacc[n] = f32x16{};
#pragma unroll
      for (int t = 0; t < C::QK_STEPS; ++t) {
#pragma unroll
        for (int n = 0; n < C::NSUB; ++n) {
          const int row = 32 * n + krow_a;
          const int ch = half * (D / 16) + t;
          const bf16x8 a = as_bf16x8(ld_lds16(ks[buf], row * D + ((ch ^ swz_k(row)) * 8)));
          sacc[n] = mfma32x32x16(a, qreg[t], sacc[n]);
        }
      }
      // mask: causal diagonal and the end of the keys. Masked scores become
      // -inf for the max and their probabilities are forced to 0 below (an
      // exp2 of -inf * c would be NaN for scale == 0).
      const bool need_mask = (CAUSAL && kv0 + BC - 1 > wrow0) || (kv0 + BC > N_kv);
      uint32_t mbits[C::NSUB];
      if (need_mask) {
#pragma unroll
        for (int n = 0; n < C::NSUB; ++n) {
          mbits[n] = 0;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kv0 + 32 * n + 16 * half + i;
            const bool masked = (CAUSAL && key > qrow) || key >= N_kv;
            if (masked) {
              sacc[n][i] = -INFINITY;
              mbits[n] |= 1u << i;
            }
          }
        }
      }
      // row max over the block (in-lane, then across the two halves)
      float mx = sacc[0][0];
#pragma unroll
      for (int n = 0; n < C::NSUB; ++n)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[n][i]);
      mx = max_xor32(mx);
      const float m_new = fmaxf(m_run, mx * c);
      const float alpha = fast_exp2(m_run - m_new);
      float psum = 0.f;
#pragma unroll
      for (int n = 0; n < C::NSUB; ++n) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fast_exp2(fmaf(sacc[n][i], c, -m_new));
          sacc[n][i] = p;
          psum += p;
        }
      }
      if (need_mask) {
        psum = 0.f;
#pragma unroll
        for (int n = 0; n < C::NSUB; ++n)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            if (mbits[n] & (1u << i)) sacc[n][i] = 0.f;
            psum += sacc[n][i];
          }
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int s = 0; s < C::DSUB; ++s)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[s][i] *= alpha;
      // O^T += V_j^T P^T
#pragma unroll
      for (int u = 0; u < C::PV_STEPS; ++u) {
        const int n = u >> 1;
        const int w8 = (u & 1) * 8;
        u32x4 pk;
        pk[0] = pack_bf16x2(sacc[n][w8 + 0], sacc[n][w8 + 1]);
        pk[1] = pack_bf16x2(sacc[n][w8 + 2], sacc[n][w8 + 3]);
        pk[2] = pack_bf16x2(sacc[n][w8 + 4], sacc[n][w8 + 5]);
        pk[3] = pack_bf16x2(sacc[n][w8 + 6], sacc[n][w8 + 7]);
        const bf16x8 pb = as_bf16x8(pk);
        const int ch = 4 * n + 2 * half + (u & 1);
#pragma unroll
        for (int s = 0; s < C::DSUB; ++s) {
          const int row = 32 * s + col;
          const bf16x8 a = as_bf16x8(ld_lds16(vts[buf], row * BC + ((ch ^ swz_v(row)) * 8)));
          oacc[s] = mfma32x32x16(a, pb, oacc[s]);
        }
      }
    }
    if (j + 1 < nblk) store_block(buf ^ 1);
    __syncthreads();
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
        w[0] = pack_bf16x2(oacc[s][4 * a + 0] * inv, oacc[s][4 * a + 1] * inv);
        w[1] = pack_bf16x2(oacc[s][4 * a + 2] * inv, oacc[s][4 * a + 3] * inv);
        st_global8(op + 32 * s + 8 * a + 4 * half, w);
      }
    }
    if (half == 0) LSE[(size_t(b) * H_q + h) * size_t(N_q) + qrow] = (m_run + __log2f(l_tot)) * kLn2;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdParams& p, hipStream_t stream) {
  const int n_qtiles = (p.N_q + kBR - 1) / kBR;
  const long long nwg = (long long)n_qtiles * p.B * p.H_q;
  const int xcd_remap = ((p.B * p.H_kv) % 8 == 0) ? 1 : 0;
  const float c = p.scale * kLog2e;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL>), dim3((unsigned)nwg), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(p.q), static_cast<const uint16_t*>(p.k),
                     static_cast<const uint16_t*>(p.v), static_cast<uint16_t*>(p.o), p.lse,
                     p.H_q, p.H_kv, p.N_q, p.N_kv, n_qtiles, xcd_remap, c);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t stream) {
  if (p.d == 128) return p.causal ? launch<128, true>(p, stream) : launch<128, false>(p, stream);
  return p.causal ? launch<64, true>(p, stream) : launch<64, false>(p, stream);
}

}  // namespace fa

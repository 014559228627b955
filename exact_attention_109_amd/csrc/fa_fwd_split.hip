// Split-KV attention forward for few queries against many keys (decode-like
// shapes: a handful of new query rows per sequence, a long key/value cache).
//
// Method: the same exact attention as fa_fwd, but the keys of each sequence
// are cut into `num_splits` ranges that run in parallel. Each range produces a
// partial output normalised by its own sum and a partial logsumexp; the
// partials are merged with the blockwise rescaling rule of the Q-stationary
// algorithm ("深度学习进阶（三十一）FlashAttention：IO 感知的精确注意力" (rkmt.cn
// blog) §2.2: when two parts of a row are combined, each is rescaled by the
// exponential of its statistic minus the combined one). The split-KV idea for
// decoding is named in the FlashDecoding paragraph of that blog's §3.
//
// gfx950 mapping
// --------------
//  * One workgroup (4 wave64s) per (batch, key/value head, key range). Its
//    rows are the G = H_q/H_kv query heads of the group times the N_q queries
//    (at most 32 rows, one MFMA column block): K and V are read once for all
//    heads that share them.
//  * The 4 waves take turns over 32-key tiles of the range and keep separate
//    running (max, sum, O) states, merged through LDS at the end: no barrier
//    inside the key loop. K and V go through LDS by LDS-DMA (fully coalesced
//    1 KiB pieces); K is read by rows as the A operand of S^T = K Q^T
//    (lane = row), V transposed (ds_read_b64_tr_b16) as the A operand of
//    O^T += V^T P^T.
//  * The work is HBM-bound: each key's K and V rows (512 bytes at d = 128)
//    serve at most 32 rows. Many waves with a tile in flight each keep the
//    memory system busy.
//  * A second kernel merges the key ranges of every row in a fixed order
//    (deterministic): LSE = ln sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s.

#include <atomic>
#include <mutex>

#include "fa.h"
#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kSplitWaves = 4;
constexpr int kSplitThreads = 64 * kSplitWaves;
constexpr int kSplitBK = 32;  // keys per tile
constexpr float kSplitRescaleSlack = 8.0f;  // log2 units

template <int D>
struct SplitCfg {
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int CPR = D / 8;                          // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;                       // rows per 1 KiB LDS-DMA instruction
  static constexpr int TILE_BYTES = kSplitBK * ROW_BYTES;    // 8 KiB (d=128), 4 KiB (d=64)
  static constexpr int NDMA = TILE_BYTES / 1024;             // DMA instructions per tile
  static constexpr int KST = D / 16;                         // MFMA k-steps over d
  static constexpr int DSUB = D / 32;                        // 32-column subtiles of O^T
};

// Tile chunk swizzles (16-byte chunk index XOR f(row)).
//  K: the 16 lanes of an A-operand read phase read 16 distinct rows at one
//     logical chunk; f_k spreads them over the bank groups.
//  V: a transposed-read phase reads 4 consecutive rows x 64 bytes; f_v puts
//     the 4 rows in different 64-byte bank groups.
template <int D>
__device__ __forceinline__ int swz_split_k(int row) {
  if constexpr (D == 128) return (row & 7) | ((row >> 1) & 8);
  else return ((row >> 1) & 3) | ((row >> 2) & 4);
}
template <int D>
__device__ __forceinline__ int swz_split_v(int row) {
  if constexpr (D == 128) return (row & 3) << 2;
  else return ((row >> 1) & 1) << 2;
}

// Partial results of one key range: O_s normalised by the range's own sum
// (float32, [row][D]) and LSE_s (natural log; -inf when the range has no key
// visible to the row). With num_splits == 1 the final O (bf16) and LSE are
// written instead.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kSplitThreads) void fwd_split_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, float* __restrict__ Opart, float* __restrict__ Lpart,
    int H_q, int H_kv, int N_q, int N_kv, int S, int keys_per_split, float c) {
  using C = SplitCfg<D>;
  // per wave: one K and one V tile; reused at the end for the merge of the 4 waves
  constexpr int kVBytes = kSplitWaves * 2 * C::TILE_BYTES;
  constexpr int kMergeBytes = kSplitWaves * D * 32 * 4;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kVBytes > kMergeBytes ? kVBytes : kMergeBytes];
  __shared__ float ms[kSplitWaves][32], ls[kSplitWaves][32];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;   // this lane's row (MFMA column)
  const int half = lane >> 5;
  const int G = H_q / H_kv;
  const int R = G * N_q;       // rows of the workgroup (<= 32, checked by the host)

  const int s = blockIdx.x % S;
  const int bk = blockIdx.x / S;
  const int b = bk / H_kv;
  const int hk = bk % H_kv;

  // this lane's row: query head hk*G + g, query i (lanes past R repeat row R-1)
  const int r = min(col, R - 1);
  const int g = r / N_q;
  const int qi = r % N_q;
  const int h = hk * G + g;
  const size_t qrow_base = ((size_t(b) * H_q + h) * N_q + qi) * D;
  bf16x8 qreg[C::KST];
  {
    const uint16_t* qp = Q + qrow_base + half * (D / 2);
#pragma unroll
    for (int t = 0; t < C::KST; ++t) qreg[t] = as_bf16x8(ld_global16(qp + 8 * t));
  }

  // key range of this split; keys past the last visible one are never read
  const int kb = s * keys_per_split;
  int ke = min(N_kv, kb + keys_per_split);
  if (CAUSAL) ke = min(ke, N_q);  // row i sees keys 0..i, and i < N_q
  const int ntiles = ke > kb ? (ke - kb + kSplitBK - 1) / kSplitBK : 0;
  // last key this lane's row may attend within the range
  const int last_key = min(CAUSAL ? qi : N_kv - 1, ke - 1);

  const size_t kvbase = (size_t(b) * H_kv + hk) * size_t(N_kv) * D;
  const uint16_t* Kh = K + kvbase;
  const uint8_t* Vh = reinterpret_cast<const uint8_t*>(V + kvbase);
  uint8_t* kt = lds + wave * 2 * C::TILE_BYTES;
  uint8_t* vt = kt + C::TILE_BYTES;

  // transposed-read offsets of V (as in the main forward kernel)
  const int j16 = lane & 15;
  const int vgrp = (lane & 31) >> 4;
  int voff[C::DSUB];
#pragma unroll
  for (int sb = 0; sb < C::DSUB; ++sb) {
    const int row = 16 * half + (j16 >> 2);
    const int cc = 32 * sb + 16 * vgrp + 4 * (j16 & 3);
    voff[sb] = row * C::ROW_BYTES + (((cc >> 3) ^ swz_split_v<D>(row)) * 16) + (cc & 7) * 2;
  }
  // K A-operand reads: row row_of_lane(col) (accumulator register i of lane
  // half g then holds key 16g + i), logical chunk (D/16)*half + t
  const int krow_lane = row_of_lane(col);
  int koff[C::KST];
#pragma unroll
  for (int t = 0; t < C::KST; ++t)
    koff[t] = krow_lane * C::ROW_BYTES + ((((D / 16) * half + t) ^ swz_split_k<D>(krow_lane)) * 16);

  float m_run = -INFINITY;
  float l_run = 0.f;
  f32x16 oacc[C::DSUB];
#pragma unroll
  for (int sb = 0; sb < C::DSUB; ++sb) oacc[sb] = f32x16{};

  for (int tt = wave; tt < ntiles; tt += kSplitWaves) {
    const int k0 = kb + tt * kSplitBK;
    // K and V tiles into this wave's LDS buffers by LDS-DMA (each instruction
    // moves 1 KiB of consecutive rows; swizzled 16-byte chunks); rows past the
    // end repeat the last key
#pragma unroll
    for (int ig = 0; ig < C::NDMA; ++ig) {
      const int row = C::RPI * ig + lane / C::CPR;
      const int pch = lane % C::CPR;
      const size_t grow = size_t(min(k0 + row, N_kv - 1)) * C::ROW_BYTES;
      lds_dma16(reinterpret_cast<const uint8_t*>(Kh) + grow + ((pch ^ swz_split_k<D>(row)) * 16),
                (LDS_AS void*)(kt + 1024 * ig));
      lds_dma16(Vh + grow + ((pch ^ swz_split_v<D>(row)) * 16), (LDS_AS void*)(vt + 1024 * ig));
    }
    wait_vmem();

    // S^T = K Q^T (keys x rows; lane = row), K rows read from LDS
    f32x16 sacc = f32x16{};
#pragma unroll
    for (int t = 0; t < C::KST; ++t)
      sacc = mfma32x32x16(as_bf16x8(*reinterpret_cast<const u32x4*>(kt + koff[t])), qreg[t], sacc);
    // key k0 + 16*half + i is visible iff i <= lim
    const int lim = last_key - k0 - 16 * half;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (i > lim) sacc[i] = -INFINITY;

    float mx = sacc[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sacc[i]);
    const float m_blk = max_xor32(mx) * c;
    // The running max is raised (and O, l rescaled) only when the tile's max
    // exceeds it by more than 2^8; exact, since the final division and the
    // logsumexp use the same, possibly stale, reference.
    if (__any(m_blk > m_run + kSplitRescaleSlack)) {
      const float m_new = fmaxf(m_run, m_blk);
      // rows that have seen no visible key yet keep m = -inf (alpha = 1 then,
      // nothing has been accumulated)
      const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int sb = 0; sb < C::DSUB; ++sb)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[sb][i] *= alpha;
      m_run = m_new;
    }
    // reference 0 for a row with no visible key so far: every exponential
    // below is then exp2(-inf) = 0
    const float m_ref = m_run == -INFINITY ? 0.f : m_run;

    u32x4 pk[2];
    float psum = 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = fast_exp2(fmaf(sacc[8 * u + e], c, -m_ref));
        psum += p[e];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) pk[u][e] = cvt_pk_bf16(p[2 * e], p[2 * e + 1]);
    }
    l_run += psum;

    // O^T += V^T P^T (V read transposed from LDS)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int rb = 8 * u * C::ROW_BYTES;
#pragma unroll
      for (int sb = 0; sb < C::DSUB; ++sb) {
        const bf16x8 av = lds_read_tr8(vt + voff[sb] + rb, vt + voff[sb] + rb + 4 * C::ROW_BYTES);
        oacc[sb] = mfma32x32x16(av, as_bf16x8(pk[u]), oacc[sb]);
      }
    }
  }

  // ---- merge the 4 waves: (m, l) per row and O^T (float32) through LDS
  const float l_tot = sum_xor32(l_run);
  __syncthreads();  // every wave is done with its V tile
  float* om = reinterpret_cast<float*>(lds);  // [wave][d][row]
  if (half == 0) {
    ms[wave][col] = m_run;
    ls[wave][col] = l_tot;
  }
  // accumulator register 4a+e of subtile sb holds d = 32 sb + 8a + 4 half + e
#pragma unroll
  for (int sb = 0; sb < C::DSUB; ++sb)
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        om[(wave * D + 32 * sb + 8 * a + 4 * half + e) * 32 + col] = oacc[sb][4 * a + e];
  __syncthreads();

  // each thread: one row and D/8 consecutive columns
  constexpr int kColsPerThread = D * 32 / kSplitThreads;
  const int mr = tid % 32;
  const int d0 = (tid / 32) * kColsPerThread;
  if (mr < R) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kSplitWaves; ++w) M = fmaxf(M, ms[w][mr]);
    float wgt[kSplitWaves];
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < kSplitWaves; ++w) {
      wgt[w] = M == -INFINITY ? 0.f : fast_exp2(ms[w][mr] - M);
      L += wgt[w] * ls[w][mr];
    }
    const float inv = L > 0.f ? 1.0f / L : 0.f;
    float ov[kColsPerThread];
#pragma unroll
    for (int j = 0; j < kColsPerThread; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < kSplitWaves; ++w) acc = fmaf(wgt[w], om[(w * D + d0 + j) * 32 + mr], acc);
      ov[j] = acc * inv;
    }
    const float lse = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
    const int gg = mr / N_q;
    const int ii = mr % N_q;
    const size_t row = (size_t(b) * H_q + hk * G + gg) * N_q + ii;
    if (S == 1) {
#pragma unroll
      for (int j = 0; j < kColsPerThread; j += 4) {
        u32x2 w2;
        w2[0] = cvt_pk_bf16(ov[j], ov[j + 1]);
        w2[1] = cvt_pk_bf16(ov[j + 2], ov[j + 3]);
        st_global8(O + row * D + d0 + j, w2);
      }
      if (d0 == 0) LSE[row] = lse;
    } else {
      float* op = Opart + (row * S + s) * D + d0;
#pragma unroll
      for (int j = 0; j < kColsPerThread; j += 4) {
        f32x4 v4;
        v4[0] = ov[j];
        v4[1] = ov[j + 1];
        v4[2] = ov[j + 2];
        v4[3] = ov[j + 3];
        *reinterpret_cast<f32x4*>(op + j) = v4;
      }
      if (d0 == 0) Lpart[row * S + s] = lse;
    }
  }
}

// ---- FP8 key/value cache (e4m3 codes with one scale per 128-key block,
// K and V row-major [B][H_kv][N_kv][D] like a bf16 cache, so that appending a
// token writes one row), bf16 queries. The codes are widened to bf16 in
// registers (exact: every e4m3 value is a bf16 value) and the contractions
// run on the bf16 MFMA, so the result is the bf16 path's arithmetic on the
// dequantized K and V: the K block scale multiplies the scores of a tile, the
// V block scale relative to the head's largest one multiplies P before its
// bf16 rounding, and the output is multiplied by the largest V scale once.
// HBM traffic per key: 2 x D bytes instead of 4 x D. The V^T operand comes
// from ds_read_b64_tr_b8: in each 16-lane group, output lane i byte k is byte
// (i % 8) of the 8 bytes addressed by lane 2k + i/8, so 16 lanes addressing
// 8 key rows x 16 columns receive 8 consecutive keys of one column each.
typedef int i32x2 __attribute__((ext_vector_type(2)));

template <int D>
struct SplitFp8Cfg {
  static constexpr int K_TILE = kSplitBK * D;                // 32 keys x D bytes
  static constexpr int V_TILE = kSplitBK * D;
  static constexpr int K_CPR = D / 16;                       // 16-byte chunks per row
  static constexpr int K_RPI = 64 / K_CPR;                   // rows per 1 KiB DMA instruction
  static constexpr int K_NDMA = K_TILE / 1024;
  static constexpr int V_NDMA = V_TILE / 1024;
  static constexpr int KST = D / 16;                         // bf16 MFMA k-steps over d
  static constexpr int DSUB = D / 32;
};
// K rows of D bytes: the 16 lanes of a read phase take rows row_of_lane(0..15)
// (or 16..31) at one logical chunk.
template <int D>
__device__ __forceinline__ int swz_split8_k(int row) {
  if constexpr (D == 128) return ((row >> 1) & 3) | ((row >> 2) & 4);
  else return ((row >> 2) & 1) | ((row >> 3) & 2);
}
// V rows of D bytes read by ds_read_b64_tr_b8: a 32-lane phase reads 8 key
// rows x 2 logical chunks; these spread them over all 16 bank groups.
template <int D>
__device__ __forceinline__ int swz_split8_v(int row) {
  if constexpr (D == 128) return ((row >> 1) & 3) << 1;
  else return ((row >> 2) & 1) << 1;
}

// 8 e4m3 codes (two dwords) -> 8 bf16 (four dwords), element order kept.
__device__ __forceinline__ u32x4 widen_fp8x8(uint32_t lo, uint32_t hi) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true));
  return r;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kSplitThreads) void fwd_split_fp8_kernel(
    const uint16_t* __restrict__ Q, const uint8_t* __restrict__ K, const float* __restrict__ KD,
    const uint8_t* __restrict__ V, const float* __restrict__ VD, uint16_t* __restrict__ O,
    float* __restrict__ LSE, float* __restrict__ Opart, float* __restrict__ Lpart, int H_q, int H_kv, int N_q,
    int N_kv, int S, int keys_per_split, float c0) {
  using C = SplitFp8Cfg<D>;
  constexpr int kTileBytes = C::K_TILE + C::V_TILE;
  constexpr int kVBytes = kSplitWaves * 2 * kTileBytes;  // two tiles per wave: one loading, one in use
  constexpr int kMergeBytes = kSplitWaves * D * 32 * 4;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kVBytes > kMergeBytes ? kVBytes : kMergeBytes];
  __shared__ float ms[kSplitWaves][32], ls[kSplitWaves][32];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int half = lane >> 5;
  const int G = H_q / H_kv;
  const int R = G * N_q;

  const int s = blockIdx.x % S;
  const int bk = blockIdx.x / S;
  const int b = bk / H_kv;
  const int hk = bk % H_kv;

  const int r = min(col, R - 1);
  const int g = r / N_q;
  const int qi = r % N_q;
  const int h = hk * G + g;
  const size_t qrow_base = ((size_t(b) * H_q + h) * N_q + qi) * D;
  bf16x8 qreg[C::KST];
  {
    const uint16_t* qp = Q + qrow_base + half * (D / 2);
#pragma unroll
    for (int t = 0; t < C::KST; ++t) qreg[t] = as_bf16x8(ld_global16(qp + 8 * t));
  }

  const int kb = s * keys_per_split;
  int ke = min(N_kv, kb + keys_per_split);
  if (CAUSAL) ke = min(ke, N_q);
  const int ntiles = ke > kb ? (ke - kb + kSplitBK - 1) / kSplitBK : 0;
  const int last_key = min(CAUSAL ? qi : N_kv - 1, ke - 1);

  const size_t kvhead = size_t(b) * H_kv + hk;
  const uint8_t* Kh = K + kvhead * size_t(N_kv) * D;
  const uint8_t* Vh = V + kvhead * size_t(N_kv) * D;
  const int nbk = (N_kv + 127) / 128;
  const float* kd = KD + kvhead * nbk;
  const float* vd = VD + kvhead * nbk;
  // the head's largest V scale (the same in every key range, so that the
  // partial outputs of all ranges are in the same units)
  float vmax = 0.f;
  for (int i = lane; i < nbk; i += 64) vmax = fmaxf(vmax, vd[i]);
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) vmax = fmaxf(vmax, __shfl_xor(vmax, o, 64));
  vmax = fmaxf(max_xor32(vmax), 1.17549435e-38f);
  const float inv_vmax = 1.0f / vmax;

  uint8_t* buf0 = lds + wave * 2 * kTileBytes;
  uint8_t* buf1 = buf0 + kTileBytes;
  // DMA of the tile at key k0 into a buffer: K and V rows of D bytes (rows
  // past the end repeat the last key). Uniform bases plus per-lane 32-bit
  // offsets; the waits are explicit.
  auto issue_tile = [&](int k0, uint8_t* dst) __attribute__((always_inline)) {
    const uint32_t kdst = lds_address(dst);
#pragma unroll
    for (int ig = 0; ig < C::K_NDMA; ++ig) {
      const int row = C::K_RPI * ig + lane / C::K_CPR;
      const int pch = lane % C::K_CPR;
      const uint32_t off = uint32_t(min(k0 + row, N_kv - 1)) * D + ((pch ^ swz_split8_k<D>(row)) * 16);
      lds_dma16_sbase_nc(Kh, off, kdst + 1024 * ig);
    }
#pragma unroll
    for (int ig = 0; ig < C::V_NDMA; ++ig) {
      const int row = C::K_RPI * ig + lane / C::K_CPR;
      const int pch = lane % C::K_CPR;
      const uint32_t off = uint32_t(min(k0 + row, N_kv - 1)) * D + ((pch ^ swz_split8_v<D>(row)) * 16);
      lds_dma16_sbase_nc(Vh, off, kdst + C::K_TILE + 1024 * ig);
    }
  };

  // K A-operand: row row_of_lane(col), bytes (D/2)*half + 8t .. +7 for k-step t,
  // read 16 bytes (two k-steps) at a time
  const int krow_lane = row_of_lane(col);
  int koff[C::KST / 2];
#pragma unroll
  for (int t2 = 0; t2 < C::KST / 2; ++t2)
    koff[t2] = krow_lane * D + ((((D / 32) * half + t2) ^ swz_split8_k<D>(krow_lane)) * 16);
  // V^T A-operand of subtile sb, k-step u (keys 16 half + 8u + e): this lane
  // addresses key row 16 half + 8u + j/2, columns 32 sb + 16 ((lane/16) % 2) + 8 (j % 2)
  // (j = lane % 16); the transposed read hands each lane 8 keys of its column.
  int voff[C::DSUB][2];
  {
    const int j = lane & 15;
    const int qh = (lane >> 4) & 1;
#pragma unroll
    for (int sb = 0; sb < C::DSUB; ++sb)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int row = 16 * half + 8 * u + (j >> 1);
        const int cc = 32 * sb + 16 * qh + 8 * (j & 1);
        voff[sb][u] = row * D + (((cc >> 4) ^ swz_split8_v<D>(row)) * 16) + (cc & 15);
      }
  }

  float m_run = -INFINITY;
  float l_run = 0.f;
  f32x16 oacc[C::DSUB];
#pragma unroll
  for (int sb = 0; sb < C::DSUB; ++sb) oacc[sb] = f32x16{};

  // the query rows and scales are in registers before the first tile DMA, so
  // that no wait for them inside the loop also waits for a prefetch
  wait_vmem();
  if (wave < ntiles) issue_tile(kb + wave * kSplitBK, buf0);
  int it = 0;
  for (int tt = wave; tt < ntiles; tt += kSplitWaves, ++it) {
    const int k0 = kb + tt * kSplitBK;
    uint8_t* kt = (it & 1) ? buf1 : buf0;
    uint8_t* vt = kt + C::K_TILE;
    // the next tile of this wave streams in while this one is used
    if (tt + kSplitWaves < ntiles) {
      issue_tile(k0 + kSplitWaves * kSplitBK, (it & 1) ? buf0 : buf1);
      wait_vmem_keep<C::K_NDMA + C::V_NDMA>();
    } else {
      wait_vmem();
    }
    const int blk = k0 / 128;
    const float c = fmaxf(c0 * kd[blk], 1.17549435e-38f);
    const float rv = vd[blk] * inv_vmax;

    // S^T = K Q^T on bf16 MFMAs, K widened from e4m3
    f32x16 sacc = f32x16{};
#pragma unroll
    for (int t2 = 0; t2 < C::KST / 2; ++t2) {
      const u32x4 raw = *reinterpret_cast<const u32x4*>(kt + koff[t2]);
      sacc = mfma32x32x16(as_bf16x8(widen_fp8x8(raw[0], raw[1])), qreg[2 * t2], sacc);
      sacc = mfma32x32x16(as_bf16x8(widen_fp8x8(raw[2], raw[3])), qreg[2 * t2 + 1], sacc);
    }
    const int lim = last_key - k0 - 16 * half;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (i > lim) sacc[i] = -INFINITY;

    float mx = sacc[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sacc[i]);
    const float m_blk = max_xor32(mx) * c;
    if (__any(m_blk > m_run + kSplitRescaleSlack)) {
      const float m_new = fmaxf(m_run, m_blk);
      const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int sb = 0; sb < C::DSUB; ++sb)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[sb][i] *= alpha;
      m_run = m_new;
    }
    const float m_ref = m_run == -INFINITY ? 0.f : m_run;

    u32x4 pk[2];
    float psum = 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = fast_exp2(fmaf(sacc[8 * u + e], c, -m_ref));
        psum += p[e];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) pk[u][e] = cvt_pk_bf16(p[2 * e] * rv, p[2 * e + 1] * rv);
    }
    l_run += psum;

    // O^T += V^T P^T: 8 keys of one column per lane by a transposed read,
    // widened from e4m3
#pragma unroll
    for (int sb = 0; sb < C::DSUB; ++sb)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const i32x2 raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS i32x2*)(vt + voff[sb][u]));
        oacc[sb] = mfma32x32x16(as_bf16x8(widen_fp8x8(uint32_t(raw[0]), uint32_t(raw[1]))),
                                as_bf16x8(pk[u]), oacc[sb]);
      }
  }

  // ---- merge the 4 waves (as in the bf16 kernel); the output is in units of
  // the largest V scale
  const float l_tot = sum_xor32(l_run);
  __syncthreads();
  float* om = reinterpret_cast<float*>(lds);
  if (half == 0) {
    ms[wave][col] = m_run;
    ls[wave][col] = l_tot;
  }
#pragma unroll
  for (int sb = 0; sb < C::DSUB; ++sb)
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        om[(wave * D + 32 * sb + 8 * a + 4 * half + e) * 32 + col] = oacc[sb][4 * a + e];
  __syncthreads();

  constexpr int kColsPerThread = D * 32 / kSplitThreads;
  const int mr = tid % 32;
  const int d0 = (tid / 32) * kColsPerThread;
  if (mr < R) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kSplitWaves; ++w) M = fmaxf(M, ms[w][mr]);
    float wgt[kSplitWaves];
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < kSplitWaves; ++w) {
      wgt[w] = M == -INFINITY ? 0.f : fast_exp2(ms[w][mr] - M);
      L += wgt[w] * ls[w][mr];
    }
    const float inv = L > 0.f ? vmax / L : 0.f;
    float ov[kColsPerThread];
#pragma unroll
    for (int j = 0; j < kColsPerThread; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < kSplitWaves; ++w) acc = fmaf(wgt[w], om[(w * D + d0 + j) * 32 + mr], acc);
      ov[j] = acc * inv;
    }
    const float lse = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
    const int gg = mr / N_q;
    const int ii = mr % N_q;
    const size_t row = (size_t(b) * H_q + hk * G + gg) * N_q + ii;
    if (S == 1) {
#pragma unroll
      for (int j = 0; j < kColsPerThread; j += 4) {
        u32x2 w2;
        w2[0] = cvt_pk_bf16(ov[j], ov[j + 1]);
        w2[1] = cvt_pk_bf16(ov[j + 2], ov[j + 3]);
        st_global8(O + row * D + d0 + j, w2);
      }
      if (d0 == 0) LSE[row] = lse;
    } else {
      float* op = Opart + (row * S + s) * D + d0;
#pragma unroll
      for (int j = 0; j < kColsPerThread; j += 4) {
        f32x4 v4;
        v4[0] = ov[j];
        v4[1] = ov[j + 1];
        v4[2] = ov[j + 2];
        v4[3] = ov[j + 3];
        *reinterpret_cast<f32x4*>(op + j) = v4;
      }
      if (d0 == 0) Lpart[row * S + s] = lse;
    }
  }
}

// Merge of the key ranges of each row, in split order: one workgroup of D
// threads per row, thread = output column.
template <int D>
__global__ __launch_bounds__(D) void fwd_split_combine_kernel(const float* __restrict__ Opart,
                                                              const float* __restrict__ Lpart,
                                                              uint16_t* __restrict__ O, float* __restrict__ LSE,
                                                              int S) {
  const size_t row = blockIdx.x;
  const int d = threadIdx.x;
  const float* lp = Lpart + row * S;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, lp[s]);
  // every row sees key 0, so some range has a finite LSE_s and M is finite
  float wsum = 0.f, acc = 0.f;
  const float* op = Opart + row * S * D + d;
  for (int s = 0; s < S; ++s) {
    const float w = __expf(lp[s] - M);  // exp(-inf) = 0 for ranges without visible keys
    wsum += w;
    acc = fmaf(w, op[size_t(s) * D], acc);
  }
  const float o = acc / wsum;
  // round to nearest even bf16 (one column per thread)
  const uint32_t u = __float_as_uint(o);
  O[row * D + d] = static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
  if (d == 0) LSE[row] = M + __logf(wsum);
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdParams& p, int S, float* ws, hipStream_t stream) {
  const int keys_per_split = ((p.N_kv + S - 1) / S + kSplitBK - 1) / kSplitBK * kSplitBK;
  const long long rows = (long long)p.B * p.H_q * p.N_q;
  float* Opart = ws;
  float* Lpart = S > 1 ? ws + rows * S * D : nullptr;
  const float c = fmaxf(p.scale * kLog2e, 1.17549435e-38f);
  const long long nwg = (long long)p.B * p.H_kv * S;
  hipLaunchKernelGGL((fwd_split_kernel<D, CAUSAL>), dim3((unsigned)nwg), dim3(kSplitThreads), 0, stream,
                     static_cast<const uint16_t*>(p.q), static_cast<const uint16_t*>(p.k),
                     static_cast<const uint16_t*>(p.v), static_cast<uint16_t*>(p.o), p.lse, Opart, Lpart,
                     p.H_q, p.H_kv, p.N_q, p.N_kv, S, keys_per_split, c);
  if (S > 1)
    hipLaunchKernelGGL((fwd_split_combine_kernel<D>), dim3((unsigned)rows), dim3(D), 0, stream, Opart, Lpart,
                       static_cast<uint16_t*>(p.o), p.lse, S);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_fp8kv(const SplitFp8Params& p, int S, float* ws, hipStream_t stream) {
  const int keys_per_split = ((p.N_kv + S - 1) / S + kSplitBK - 1) / kSplitBK * kSplitBK;
  const long long rows = (long long)p.B * p.H_q * p.N_q;
  float* Opart = ws;
  float* Lpart = S > 1 ? ws + rows * S * D : nullptr;
  const long long nwg = (long long)p.B * p.H_kv * S;
  hipLaunchKernelGGL((fwd_split_fp8_kernel<D, CAUSAL>), dim3((unsigned)nwg), dim3(kSplitThreads), 0, stream,
                     static_cast<const uint16_t*>(p.q), static_cast<const uint8_t*>(p.k), p.k_descale,
                     static_cast<const uint8_t*>(p.v), p.v_descale, static_cast<uint16_t*>(p.o), p.lse, Opart,
                     Lpart, p.H_q, p.H_kv, p.N_q, p.N_kv, S, keys_per_split, p.scale * kLog2e);
  if (S > 1)
    hipLaunchKernelGGL((fwd_split_combine_kernel<D>), dim3((unsigned)rows), dim3(D), 0, stream, Opart, Lpart,
                       static_cast<uint16_t*>(p.o), p.lse, S);
  return hipGetLastError();
}

}  // namespace

size_t fwd_split_workspace_floats(int B, int H_q, int N_q, int d, int num_splits) {
  if (num_splits <= 1) return 0;
  return size_t(B) * H_q * N_q * num_splits * (size_t(d) + 1);
}

hipError_t launch_fwd_split_bf16(const FwdParams& p, int num_splits, float* workspace, hipStream_t stream) {
  if (p.d == 128)
    return p.causal ? launch<128, true>(p, num_splits, workspace, stream)
                    : launch<128, false>(p, num_splits, workspace, stream);
  return p.causal ? launch<64, true>(p, num_splits, workspace, stream)
                  : launch<64, false>(p, num_splits, workspace, stream);
}

}  // namespace fa

namespace fa {

hipError_t launch_fwd_split_fp8kv(const SplitFp8Params& p, int num_splits, float* workspace, hipStream_t stream) {
  if (p.d == 128)
    return p.causal ? launch_fp8kv<128, true>(p, num_splits, workspace, stream)
                    : launch_fp8kv<128, false>(p, num_splits, workspace, stream);
  return p.causal ? launch_fp8kv<64, true>(p, num_splits, workspace, stream)
                  : launch_fp8kv<64, false>(p, num_splits, workspace, stream);
}

}  // namespace fa

// ---- Statically reserved partials for the entry point that allocates
// nothing. In host code `scratch` names a host-side stand-in of the array,
// not its device address, so it is never handed to a kernel or a copy: the
// address each device holds it at is looked up once per device with
// hipGetSymbolAddress (with that device current) and cached.
namespace fa {
namespace {

static __device__ __align__(256) float scratch[FA_NOALLOC_SCRATCH_BYTES / sizeof(float)];

constexpr int kMaxDevices = 64;
std::atomic<float*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

}  // namespace

hipError_t split_scratch_pointer(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  float* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      void* addr = nullptr;
      e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
      if (e != hipSuccess || addr == nullptr) return e != hipSuccess ? e : hipErrorInvalidSymbol;
      p = static_cast<float*>(addr);
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace fa

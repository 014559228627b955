// Attention forward for float32 inputs (small problems and exact checks).
//
// The per-key streaming recurrence of "深度学习进阶（三十一）FlashAttention：IO 感知
// 的精确注意力" (rkmt.cn blog) §2.1, extended with the output accumulator of
// §2.2: for every key the running max m, the normalizer l and the output row
// are updated, with the previous terms rescaled by exp(m_prev - m_new). Key/value
// blocks are staged in LDS and shared by the 64 query rows of a workgroup; four
// lanes share one query row, each owning a quarter of the head dimension.
// Arithmetic is fp32 throughout with the accurate expf/logf.

#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kRows = 64;   // query rows per workgroup
constexpr int kKB = 64;     // keys per LDS block

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                      const float* __restrict__ V, float* __restrict__ O,
                                                      float* __restrict__ LSE, int H_q, int H_kv, int N_q,
                                                      int N_kv, int n_tiles, float scale) {
  constexpr int DP = D / 4;
  __shared__ float ks[kKB][D];
  __shared__ float vs[kKB][D];

  const int tid = threadIdx.x;
  const int r = tid >> 2;
  const int part = tid & 3;
  const int tile = blockIdx.x % n_tiles;
  const int h = (blockIdx.x / n_tiles) % H_q;
  const int b = blockIdx.x / n_tiles / H_q;
  const int G = H_q / H_kv;
  const int hk = h / G;
  const int qrow = tile * kRows + r;

  const size_t qbase = (size_t(b) * H_q + h) * size_t(N_q) * D;
  const size_t kvbase = (size_t(b) * H_kv + hk) * size_t(N_kv) * D;

  float qv[DP];
  {
    const float* qp = Q + qbase + size_t(min(qrow, N_q - 1)) * D + part * DP;
#pragma unroll
    for (int e = 0; e < DP; ++e) qv[e] = qp[e];
  }

  int kend = N_kv;
  if (CAUSAL) kend = min(N_kv, min(tile * kRows + kRows, N_q));  // keys <= last row of the tile

  float m = -INFINITY, l = 0.f;
  float o[DP];
#pragma unroll
  for (int e = 0; e < DP; ++e) o[e] = 0.f;

  for (int kb0 = 0; kb0 < kend; kb0 += kKB) {
    for (int idx = tid; idx < kKB * D; idx += 256) {
      const int kr = idx / D, kc = idx % D;
      const int key = min(kb0 + kr, N_kv - 1);
      ks[kr][kc] = K[kvbase + size_t(key) * D + kc];
      vs[kr][kc] = V[kvbase + size_t(key) * D + kc];
    }
    __syncthreads();
    const int nk = min(kKB, kend - kb0);
    for (int jj = 0; jj < nk; ++jj) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < DP; ++e) dot = fmaf(qv[e], ks[jj][part * DP + e], dot);
      dot += __shfl_xor(dot, 1);
      dot += __shfl_xor(dot, 2);
      const int key = kb0 + jj;
      if (!CAUSAL || key <= qrow) {
        const float s = dot * scale;
        const float m_new = fmaxf(m, s);
        const float a = expf(m - m_new);
        const float p = expf(s - m_new);
        l = l * a + p;
#pragma unroll
        for (int e = 0; e < DP; ++e) o[e] = fmaf(p, vs[jj][part * DP + e], o[e] * a);
        m = m_new;
      }
    }
    __syncthreads();
  }

  if (qrow < N_q) {
    const float inv = 1.0f / l;
    float* op = O + qbase + size_t(qrow) * D + part * DP;
#pragma unroll
    for (int e = 0; e < DP; ++e) op[e] = o[e] * inv;
    if (part == 0) LSE[(size_t(b) * H_q + h) * size_t(N_q) + qrow] = m + logf(l);
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdParams& p, hipStream_t stream) {
  const int n_tiles = (p.N_q + kRows - 1) / kRows;
  const unsigned grid = (unsigned)((long long)n_tiles * p.H_q * p.B);
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3(grid), dim3(256), 0, stream,
                     static_cast<const float*>(p.q), static_cast<const float*>(p.k),
                     static_cast<const float*>(p.v), static_cast<float*>(p.o), p.lse, p.H_q, p.H_kv,
                     p.N_q, p.N_kv, n_tiles, p.scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t stream) {
  if (p.d == 128) return p.causal ? launch<128, true>(p, stream) : launch<128, false>(p, stream);
  return p.causal ? launch<64, true>(p, stream) : launch<64, false>(p, stream);
}

}  // namespace fa

// Attention backward by recomputation on the vector ALUs (float32 inputs).
//
// "Flash-Attention" (Awesome System Papers Wiki), core-idea section: the
// backward pass does not keep the probability matrix; it rebuilds it from
// Q, K, V and the per-row statistics saved by the forward pass (here the
// logsumexp), trading extra arithmetic for memory and HBM traffic.
//
// With P_ij = exp(scale * q_i.k_j - lse_i) over the allowed keys:
//   D_i  = <dO_i, O_i>                       (delta kernel)
//   dq_i = scale * sum_j P_ij (<dO_i, v_j> - D_i) k_j          (dq kernel)
//   dv_j = sum_i P_ij dO_i,  dk_j = scale * sum_i P_ij (<dO_i, v_j> - D_i) q_i
//                                           (dk/dv kernel, over the G query
//                                            heads that share key head j)
// Each output element is produced by exactly one thread (no atomics), so
// results are deterministic. Four lanes share a row, a quarter of the head
// dimension each; dot products meet through two lane shuffles.

#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {
namespace {

__device__ __forceinline__ float to_f(float x) { return x; }

__device__ __forceinline__ float quad_sum(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  return x;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void delta_kernel(const T* __restrict__ O, const T* __restrict__ dO,
                                                    float* __restrict__ delta, long long rows) {
  constexpr int DP = D / 4;
  const long long row = (long long)blockIdx.x * 64 + (threadIdx.x >> 2);
  const int part = threadIdx.x & 3;
  const long long rc = row < rows ? row : rows - 1;
  float acc = 0.f;
  const T* op = O + rc * D + part * DP;
  const T* dp = dO + rc * D + part * DP;
#pragma unroll
  for (int e = 0; e < DP; ++e) acc = fmaf(to_f(op[e]), to_f(dp[e]), acc);
  acc = quad_sum(acc);
  if (row < rows && part == 0) delta[row] = acc;
}

constexpr int kQRows = 64;  // dq kernel: query rows per workgroup
constexpr int kKB = 64;     // dq kernel: keys per LDS block
constexpr int kKRows = 64;  // dk/dv kernel: keys per workgroup
constexpr int kQB = 32;     // dk/dv kernel: queries per LDS block

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256) void dq_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                 const T* __restrict__ V, const T* __restrict__ dO,
                                                 const float* __restrict__ LSE, const float* __restrict__ delta,
                                                 float* __restrict__ dQ, int H_q, int H_kv, int N_q, int N_kv,
                                                 int n_tiles, float scale) {
  constexpr int DP = D / 4;
  __shared__ float ks[kKB][D];
  __shared__ float vs[kKB][D];
  const int tid = threadIdx.x;
  const int r = tid >> 2;
  const int part = tid & 3;
  const int tile = blockIdx.x % n_tiles;
  const int h = (blockIdx.x / n_tiles) % H_q;
  const int b = blockIdx.x / n_tiles / H_q;
  const int hk = h / (H_q / H_kv);
  const int qrow = tile * kQRows + r;
  const int qr = min(qrow, N_q - 1);
  const size_t rowbase = (size_t(b) * H_q + h) * size_t(N_q);
  const size_t kvbase = (size_t(b) * H_kv + hk) * size_t(N_kv) * D;

  float qv[DP], gv[DP], acc[DP];
#pragma unroll
  for (int e = 0; e < DP; ++e) {
    qv[e] = to_f(Q[(rowbase + qr) * D + part * DP + e]);
    gv[e] = to_f(dO[(rowbase + qr) * D + part * DP + e]);
    acc[e] = 0.f;
  }
  const float lse = LSE[rowbase + qr];
  const float di = delta[rowbase + qr];

  int kend = N_kv;
  if (CAUSAL) kend = min(N_kv, min(tile * kQRows + kQRows, N_q));
  for (int kb0 = 0; kb0 < kend; kb0 += kKB) {
    for (int idx = tid; idx < kKB * D; idx += 256) {
      const int kr = idx / D, kc = idx % D;
      const int key = min(kb0 + kr, N_kv - 1);
      ks[kr][kc] = to_f(K[kvbase + size_t(key) * D + kc]);
      vs[kr][kc] = to_f(V[kvbase + size_t(key) * D + kc]);
    }
    __syncthreads();
    const int nk = min(kKB, kend - kb0);
    for (int jj = 0; jj < nk; ++jj) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < DP; ++e) {
        s = fmaf(qv[e], ks[jj][part * DP + e], s);
        dp = fmaf(gv[e], vs[jj][part * DP + e], dp);
      }
      s = quad_sum(s);
      dp = quad_sum(dp);
      if (!CAUSAL || kb0 + jj <= qrow) {
        const float p = expf(s * scale - lse);
        const float ds = p * (dp - di);
#pragma unroll
        for (int e = 0; e < DP; ++e) acc[e] = fmaf(ds, ks[jj][part * DP + e], acc[e]);
      }
    }
    __syncthreads();
  }
  if (qrow < N_q) {
#pragma unroll
    for (int e = 0; e < DP; ++e) dQ[(rowbase + qrow) * D + part * DP + e] = acc[e] * scale;
  }
}

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256) void dkdv_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                   const T* __restrict__ V, const T* __restrict__ dO,
                                                   const float* __restrict__ LSE, const float* __restrict__ delta,
                                                   float* __restrict__ dK, float* __restrict__ dV, int H_q,
                                                   int H_kv, int N_q, int N_kv, int n_tiles, float scale) {
  constexpr int DP = D / 4;
  __shared__ float qs[kQB][D];
  __shared__ float gs[kQB][D];
  __shared__ float ls[kQB];
  __shared__ float ds_[kQB];
  const int tid = threadIdx.x;
  const int r = tid >> 2;
  const int part = tid & 3;
  const int tile = blockIdx.x % n_tiles;
  const int hk = (blockIdx.x / n_tiles) % H_kv;
  const int b = blockIdx.x / n_tiles / H_kv;
  const int G = H_q / H_kv;
  const int key = tile * kKRows + r;
  const int kc = min(key, N_kv - 1);
  const size_t kvrow = (size_t(b) * H_kv + hk) * size_t(N_kv);

  float kv[DP], vv[DP], dk[DP], dv[DP];
#pragma unroll
  for (int e = 0; e < DP; ++e) {
    kv[e] = to_f(K[(kvrow + kc) * D + part * DP + e]);
    vv[e] = to_f(V[(kvrow + kc) * D + part * DP + e]);
    dk[e] = 0.f;
    dv[e] = 0.f;
  }
  // causal: queries before the tile's first key never attend it
  const int qstart = CAUSAL ? (tile * kKRows / kQB) * kQB : 0;
  for (int g = 0; g < G; ++g) {
    const int h = hk * G + g;
    const size_t rowbase = (size_t(b) * H_q + h) * size_t(N_q);
    for (int qb0 = qstart; qb0 < N_q; qb0 += kQB) {
      for (int idx = tid; idx < kQB * D; idx += 256) {
        const int qr = idx / D, qc = idx % D;
        const int qi = min(qb0 + qr, N_q - 1);
        qs[qr][qc] = to_f(Q[(rowbase + qi) * D + qc]);
        gs[qr][qc] = to_f(dO[(rowbase + qi) * D + qc]);
      }
      if (tid < kQB) {
        const int qi = min(qb0 + tid, N_q - 1);
        ls[tid] = LSE[rowbase + qi];
        ds_[tid] = delta[rowbase + qi];
      }
      __syncthreads();
      const int nq = min(kQB, N_q - qb0);
      for (int ii = 0; ii < nq; ++ii) {
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int e = 0; e < DP; ++e) {
          s = fmaf(qs[ii][part * DP + e], kv[e], s);
          dp = fmaf(gs[ii][part * DP + e], vv[e], dp);
        }
        s = quad_sum(s);
        dp = quad_sum(dp);
        if (!CAUSAL || key <= qb0 + ii) {
          const float p = expf(s * scale - ls[ii]);
          const float dsv = p * (dp - ds_[ii]);
#pragma unroll
          for (int e = 0; e < DP; ++e) {
            dv[e] = fmaf(p, gs[ii][part * DP + e], dv[e]);
            dk[e] = fmaf(dsv, qs[ii][part * DP + e], dk[e]);
          }
        }
      }
      __syncthreads();
    }
  }
  if (key < N_kv) {
#pragma unroll
    for (int e = 0; e < DP; ++e) {
      dK[(kvrow + key) * D + part * DP + e] = dk[e] * scale;
      dV[(kvrow + key) * D + part * DP + e] = dv[e];
    }
  }
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_all(const BwdParams& p, hipStream_t stream) {
  const long long rows = (long long)p.B * p.H_q * p.N_q;
  hipLaunchKernelGGL((delta_kernel<T, D>), dim3((unsigned)((rows + 63) / 64)), dim3(256), 0, stream,
                     static_cast<const T*>(p.o), static_cast<const T*>(p.dO), p.delta, rows);
  const int qt = (p.N_q + kQRows - 1) / kQRows;
  hipLaunchKernelGGL((dq_kernel<T, D, CAUSAL>), dim3((unsigned)((long long)qt * p.H_q * p.B)), dim3(256), 0,
                     stream, static_cast<const T*>(p.q), static_cast<const T*>(p.k),
                     static_cast<const T*>(p.v), static_cast<const T*>(p.dO), p.lse, p.delta, p.dq, p.H_q,
                     p.H_kv, p.N_q, p.N_kv, qt, p.scale);
  const int kt = (p.N_kv + kKRows - 1) / kKRows;
  hipLaunchKernelGGL((dkdv_kernel<T, D, CAUSAL>), dim3((unsigned)((long long)kt * p.H_kv * p.B)), dim3(256), 0,
                     stream, static_cast<const T*>(p.q), static_cast<const T*>(p.k),
                     static_cast<const T*>(p.v), static_cast<const T*>(p.dO), p.lse, p.delta, p.dk, p.dv,
                     p.H_q, p.H_kv, p.N_q, p.N_kv, kt, p.scale);
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch(const BwdParams& p, hipStream_t stream) {
  if (p.d == 128) return p.causal ? launch_all<T, 128, true>(p, stream) : launch_all<T, 128, false>(p, stream);
  return p.causal ? launch_all<T, 64, true>(p, stream) : launch_all<T, 64, false>(p, stream);
}

}  // namespace

hipError_t launch_bwd_f32(const BwdParams& p, hipStream_t stream) { return dispatch<float>(p, stream); }

}  // namespace fa

// On-GPU self-check of a forward result: for sampled query rows i,
//     e_i = | sum_j exp(scale * q_i . k_j - lse_i) - 1 |   over the allowed keys j.
// A correct logsumexp makes the probabilities of a row sum to one ("Flash-
// Attention" (Awesome System Papers Wiki), core-idea section: the saved
// per-row statistics are what the backward pass rebuilds the probabilities
// from, so a wrong statistic silently corrupts the gradients). The check
// recomputes the scores from q and k independently of the forward kernels:
// plain fp32 dot products on the vector ALU, one workgroup per (batch, query
// head, sampled row), keys strided over the threads, partial sums combined
// in a fixed order (deterministic). Cost: rows x N_kv x d multiply-adds per
// head, small next to the forward pass for a few rows.

#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kCheckThreads = 256;

__device__ __forceinline__ float load_elem(const void* p, size_t i, int dtype) {
  if (dtype == 1) return __uint_as_float(uint32_t(static_cast<const uint16_t*>(p)[i]) << 16);
  return static_cast<const float*>(p)[i];
}

template <int D>
__global__ __launch_bounds__(kCheckThreads) void check_kernel(const void* __restrict__ Q, const void* __restrict__ K,
                                                              const float* __restrict__ LSE,
                                                              const int* __restrict__ rows, int n_rows, int H_q,
                                                              int H_kv, int N_q, int N_kv, int causal, float scale,
                                                              int dtype, float* __restrict__ out) {
  __shared__ float qs[D];
  __shared__ float part[kCheckThreads];
  const int r = blockIdx.x % n_rows;
  const int bh = blockIdx.x / n_rows;  // b * H_q + h
  const int h = bh % H_q;
  const int b = bh / H_q;
  const int G = H_q / H_kv;
  const int hk = h / G;
  const int row = min(max(rows[r], 0), N_q - 1);
  const size_t qoff = (size_t(bh) * N_q + row) * D;
  for (int e = threadIdx.x; e < D; e += kCheckThreads) qs[e] = load_elem(Q, qoff + e, dtype);
  __syncthreads();
  const float lse = LSE[size_t(bh) * N_q + row];
  const int nk = causal ? min(row + 1, N_kv) : N_kv;
  const size_t kbase = (size_t(b) * H_kv + hk) * size_t(N_kv) * D;
  float acc = 0.f;
  for (int j = threadIdx.x; j < nk; j += kCheckThreads) {
    float s = 0.f;
#pragma unroll 8
    for (int e = 0; e < D; ++e) s = fmaf(qs[e], load_elem(K, kbase + size_t(j) * D + e, dtype), s);
    acc += __expf(scale * s - lse);
  }
  part[threadIdx.x] = acc;
  __syncthreads();
  for (unsigned w = kCheckThreads / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[size_t(bh) * n_rows + r] = fabsf(part[0] - 1.0f);
}

}  // namespace

hipError_t launch_check(const FwdParams& p, const int* rows, int n_rows, float* out, int dtype, hipStream_t stream) {
  const long long nwg = (long long)p.B * p.H_q * n_rows;
  if (p.d == 128)
    hipLaunchKernelGGL(check_kernel<128>, dim3((unsigned)nwg), dim3(kCheckThreads), 0, stream, p.q, p.k, p.lse, rows,
                       n_rows, p.H_q, p.H_kv, p.N_q, p.N_kv, p.causal, p.scale, dtype, out);
  else
    hipLaunchKernelGGL(check_kernel<64>, dim3((unsigned)nwg), dim3(kCheckThreads), 0, stream, p.q, p.k, p.lse, rows,
                       n_rows, p.H_q, p.H_kv, p.N_q, p.N_kv, p.causal, p.scale, dtype, out);
  return hipGetLastError();
}

}  // namespace fa

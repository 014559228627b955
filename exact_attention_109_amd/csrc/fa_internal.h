// Internal interface between the C-ABI front end (fa_api.cpp) and the kernel
// translation units. Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H_q, H_kv, N_q, N_kv, d;
  int causal;
  float scale;
};

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dO;
  float* dq;
  float* dk;
  float* dv;
  float* delta;  // workspace: D_i = <dO_i, o_i> then lse_i*log2(e), each [B][H_q][N_q] float32
  int B, H_q, H_kv, N_q, N_kv, d;
  int causal;
  float scale;
};

// Packed variable-length sequences: sequence b owns query rows
// cu_q[b] .. cu_q[b+1]-1 of the [H_q][total_q][d] tensors and key rows
// cu_k[b] .. cu_k[b+1]-1 of the [H_kv][total_k][d] ones (device int32 arrays).
struct VarlenParams {
  const int* cu_q;
  const int* cu_k;
  int total_q, total_k;
};

// Each launcher enqueues its kernels on `stream` and returns hipGetLastError().
// The front end has already validated every argument.
hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t stream);
// p.B = number of sequences, p.N_q = longest query sequence, p.N_kv unused
hipError_t launch_fwd_varlen_bf16(const FwdParams& p, const VarlenParams& vl, hipStream_t stream);
hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t stream);
hipError_t launch_bwd_f32(const BwdParams& p, hipStream_t stream);
// Zero-fill of n4 float4 elements at p (16-byte aligned).
hipError_t launch_zero_f32x4(float* p, size_t n4, hipStream_t stream);
// Self-check of a forward result on sampled rows (see fa_fwd_check).
hipError_t launch_check(const FwdParams& p, const int* rows, int n_rows, float* out, int dtype, hipStream_t stream);
// Split-KV forward (bf16, rows per key/value head <= 32); workspace holds
// fwd_split_workspace_floats(...) floats when num_splits > 1.
hipError_t launch_fwd_split_bf16(const FwdParams& p, int num_splits, float* workspace, hipStream_t stream);
size_t fwd_split_workspace_floats(int B, int H_q, int N_q, int d, int num_splits);
// Device address of the statically reserved split-KV partials array
// (FA_NOALLOC_SCRATCH_BYTES) on the current device, looked up once per device.
hipError_t split_scratch_pointer(float** out);

// FP8 forward: e4m3 codes with one float32 descale per 128-row block, all
// row-major; o is bf16, lse float32.
struct Fp8FwdParams {
  const void* q;
  const float* q_descale;
  const void* k;
  const float* k_descale;
  const void* v;
  const float* v_descale;
  void* o;
  float* lse;
  int B, H_q, H_kv, N_q, N_kv, d;
  int causal;
  float scale;
};
inline int fp8_v_pad(int n) { return (n + 127) / 128 * 128; }
// Split-KV forward with an FP8 key/value cache: q bf16 [B][H_q][N_q][d],
// k and v codes [B][H_kv][N_kv][d], descales [B][H_kv][ceil(N_kv/128)];
// o bf16, lse float32.
struct SplitFp8Params {
  const void* q;
  const void* k;
  const float* k_descale;
  const void* v;
  const float* v_descale;
  void* o;
  float* lse;
  int B, H_q, H_kv, N_q, N_kv, d;
  int causal;
  float scale;
};
hipError_t launch_fwd_split_fp8kv(const SplitFp8Params& p, int num_splits, float* workspace, hipStream_t stream);
hipError_t launch_fwd_fp8(const Fp8FwdParams& p, hipStream_t stream);
// Block quantizer: bf16 x [B][H][N][d] -> codes (row-major, or d-major with
// zero codes up to fp8_v_pad(N)) and descale [B][H][ceil(N/128)].
hipError_t launch_quantize_fp8(const void* x, void* codes, float* descale, int B, int H, int N, int d, int d_major,
                               hipStream_t stream);

}  // namespace fa

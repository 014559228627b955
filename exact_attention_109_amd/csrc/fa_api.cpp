// C-ABI front end of libfa.so: argument validation (pure C++, no HIP call),
// device check, kernel selection and launch. The operation and the argument
// conventions are documented in include/fa.h.

#include "fa.h"

#include <atomic>
#include <cmath>
#include <cstring>

#include "fa_internal.h"

#define FA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr int64_t kMaxSeq = int64_t(1) << 24;

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

Range range_of(const void* p, size_t bytes) {
  uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + bytes};
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elem_size(int dtype) { return dtype == FA_DTYPE_BF16 ? 2 : 4; }

// Shared shape checks. Returns FA_OK and sets *empty when there is nothing to do.
int check_shape(int B, int H_q, int H_kv, int N_q, int N_kv, int d, float scale, int dtype,
                bool* empty) {
  *empty = false;
  if (B < 0 || H_q < 0 || H_kv < 0 || N_q < 0 || N_kv < 0 || d < 0) return FA_ERR_INVALID_ARG;
  if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (B == 0 || H_q == 0 || N_q == 0) {
    *empty = true;
    return FA_OK;
  }
  if (H_kv == 0 || H_q % H_kv != 0) return FA_ERR_INVALID_ARG;
  if (N_kv == 0) return FA_ERR_INVALID_ARG;
  if (N_q > kMaxSeq || N_kv > kMaxSeq) return FA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return FA_ERR_INVALID_ARG;
  if (scale < 0.0f) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

// Device check: gfx950 only. Cached per device id (0 = unknown, 1 = ok, 2 = not ok).
std::atomic<int> g_device_ok[64];

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FA_ERR_HIP;
  if (dev < 0 || dev >= 64) return FA_ERR_UNSUPPORTED;
  int state = g_device_ok[dev].load(std::memory_order_relaxed);
  if (state == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FA_ERR_HIP;
    state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_device_ok[dev].store(state, std::memory_order_relaxed);
  }
  return state == 1 ? FA_OK : FA_ERR_UNSUPPORTED;
}

}  // namespace

FA_EXPORT const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK: success";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG: invalid pointer, size, scale or workspace argument";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: unsupported dtype, head dimension, scale sign or device";
    case FA_ERR_HIP: return "FA_ERR_HIP: the HIP runtime reported an error";
    default: return "unknown fa status code";
  }
}

FA_EXPORT int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int H_q, int H_kv, int N_q, int N_kv, int d,
                     int causal, float scale, int dtype, void* stream) {
  bool empty = false;
  int rc = check_shape(B, H_q, H_kv, N_q, N_kv, d, scale, dtype, &empty);
  if (rc != FA_OK || empty) return rc;

  const size_t es = elem_size(dtype);
  const size_t q_bytes = size_t(B) * H_q * N_q * d * es;
  const size_t kv_bytes = size_t(B) * H_kv * N_kv * d * es;
  const size_t lse_bytes = size_t(B) * H_q * N_q * sizeof(float);
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_INVALID_ARG;
  const Range in[3] = {range_of(q, q_bytes), range_of(k, kv_bytes), range_of(v, kv_bytes)};
  const Range out[2] = {range_of(o, q_bytes), range_of(lse, lse_bytes)};
  for (const Range& r : out)
    for (const Range& i : in)
      if (overlaps(r, i)) return FA_ERR_INVALID_ARG;
  if (overlaps(out[0], out[1])) return FA_ERR_INVALID_ARG;

  rc = check_device();
  if (rc != FA_OK) return rc;

  fa::FwdParams p{q, k, v, o, lse, B, H_q, H_kv, N_q, N_kv, d, causal ? 1 : 0, scale};
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t err = dtype == FA_DTYPE_BF16 ? fa::launch_fwd_bf16(p, s) : fa::launch_fwd_f32(p, s);
  return err == hipSuccess ? FA_OK : FA_ERR_HIP;
}

FA_EXPORT size_t fa_bwd_workspace_size(int B, int H_q, int N_q) {
  if (B <= 0 || H_q <= 0 || N_q <= 0) return 0;
  // two float32 values per query row: D_i = <dO_i, O_i> and lse_i * log2(e)
  size_t bytes = 2 * size_t(B) * H_q * N_q * sizeof(float);
  return (bytes + 255) & ~size_t(255);
}

FA_EXPORT int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* dO, float* dq, float* dk, float* dv,
                     void* workspace, size_t workspace_bytes,
                     int B, int H_q, int H_kv, int N_q, int N_kv, int d,
                     int causal, float scale, int dtype, void* stream) {
  bool empty = false;
  int rc = check_shape(B, H_q, H_kv, N_q, N_kv, d, scale, dtype, &empty);
  if (rc != FA_OK) return rc;
  if (empty) {
    // No query rows (H_q or N_q zero): no query attends any key, so dk and dv
    // are zero. They hold B*H_kv*N_kv*d elements, which may be non-zero.
    if (B == 0 || H_kv == 0 || N_kv == 0) return FA_OK;
    if (N_kv > kMaxSeq) return FA_ERR_INVALID_ARG;
    const size_t dkv_bytes = size_t(B) * H_kv * N_kv * d * sizeof(float);
    if (!dk || !dv || !aligned16(dk) || !aligned16(dv)) return FA_ERR_INVALID_ARG;
    if (overlaps(range_of(dk, dkv_bytes), range_of(dv, dkv_bytes))) return FA_ERR_INVALID_ARG;
    rc = check_device();
    if (rc != FA_OK) return rc;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t err = fa::launch_zero_f32x4(dk, dkv_bytes / 16, s);
    if (err == hipSuccess) err = fa::launch_zero_f32x4(dv, dkv_bytes / 16, s);
    return err == hipSuccess ? FA_OK : FA_ERR_HIP;
  }

  const size_t es = elem_size(dtype);
  const size_t q_bytes = size_t(B) * H_q * N_q * d * es;
  const size_t kv_bytes = size_t(B) * H_kv * N_kv * d * es;
  const size_t lse_bytes = size_t(B) * H_q * N_q * sizeof(float);
  const size_t dq_bytes = size_t(B) * H_q * N_q * d * sizeof(float);
  const size_t dkv_bytes = size_t(B) * H_kv * N_kv * d * sizeof(float);
  const size_t ws_need = fa_bwd_workspace_size(B, H_q, N_q);
  if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv || !workspace)
    return FA_ERR_INVALID_ARG;
  const void* ptrs[10] = {q, k, v, o, lse, dO, dq, dk, dv, workspace};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FA_ERR_INVALID_ARG;
  const Range in[6] = {range_of(q, q_bytes), range_of(k, kv_bytes), range_of(v, kv_bytes),
                       range_of(o, q_bytes), range_of(lse, lse_bytes), range_of(dO, q_bytes)};
  const Range out[4] = {range_of(dq, dq_bytes), range_of(dk, dkv_bytes), range_of(dv, dkv_bytes),
                        range_of(workspace, ws_need)};
  for (int a = 0; a < 4; ++a) {
    for (const Range& i : in)
      if (overlaps(out[a], i)) return FA_ERR_INVALID_ARG;
    for (int b = a + 1; b < 4; ++b)
      if (overlaps(out[a], out[b])) return FA_ERR_INVALID_ARG;
  }
  if (workspace_bytes < ws_need) return FA_ERR_INVALID_ARG;

  rc = check_device();
  if (rc != FA_OK) return rc;

  fa::BwdParams p{q, k, v, o, lse, dO, dq, dk, dv, static_cast<float*>(workspace),
                  B, H_q, H_kv, N_q, N_kv, d, causal ? 1 : 0, scale};
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t err = dtype == FA_DTYPE_BF16 ? fa::launch_bwd_bf16(p, s) : fa::launch_bwd_f32(p, s);
  return err == hipSuccess ? FA_OK : FA_ERR_HIP;
}

FA_EXPORT size_t fa_fwd_splitkv_workspace_size(int B, int H_q, int N_q, int d, int num_splits) {
  if (B <= 0 || H_q <= 0 || N_q <= 0 || d <= 0 || num_splits <= 1) return 0;
  const size_t bytes = fa::fwd_split_workspace_floats(B, H_q, N_q, d, num_splits) * sizeof(float);
  return (bytes + 255) & ~size_t(255);
}

namespace {

// Checks shared by fa_fwd_splitkv and fa_fwd_splitkv_noalloc, up to (not
// including) the workspace. Sets *empty when there is nothing to do.
int check_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H_q, int H_kv,
                  int N_q, int N_kv, int d, float scale, int dtype, int num_splits, bool* empty,
                  Range in[3], Range out[2]) {
  int rc = check_shape(B, H_q, H_kv, N_q, N_kv, d, scale, dtype, empty);
  if (rc != FA_OK || *empty) return rc;

  const size_t es = elem_size(dtype);
  const size_t q_bytes = size_t(B) * H_q * N_q * d * es;
  const size_t kv_bytes = size_t(B) * H_kv * N_kv * d * es;
  const size_t lse_bytes = size_t(B) * H_q * N_q * sizeof(float);
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_INVALID_ARG;
  in[0] = range_of(q, q_bytes);
  in[1] = range_of(k, kv_bytes);
  in[2] = range_of(v, kv_bytes);
  out[0] = range_of(o, q_bytes);
  out[1] = range_of(lse, lse_bytes);
  for (int r = 0; r < 2; ++r)
    for (int i = 0; i < 3; ++i)
      if (overlaps(out[r], in[i])) return FA_ERR_INVALID_ARG;
  if (overlaps(out[0], out[1])) return FA_ERR_INVALID_ARG;

  if (num_splits < 1 || num_splits > 256) return FA_ERR_INVALID_ARG;
  if (dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
  if ((H_q / H_kv) * N_q > 32) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

}  // namespace

FA_EXPORT int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                             int B, int H_q, int H_kv, int N_q, int N_kv, int d,
                             int causal, float scale, int dtype, int num_splits,
                             void* workspace, size_t workspace_bytes, void* stream) {
  bool empty = false;
  Range in[3], out[2];
  int rc = check_splitkv(q, k, v, o, lse, B, H_q, H_kv, N_q, N_kv, d, scale, dtype, num_splits, &empty, in, out);
  if (rc != FA_OK || empty) return rc;

  const size_t ws_need = fa_fwd_splitkv_workspace_size(B, H_q, N_q, d, num_splits);
  if (ws_need > 0) {
    if (!workspace || !aligned16(workspace) || workspace_bytes < ws_need) return FA_ERR_INVALID_ARG;
    const Range w = range_of(workspace, ws_need);
    for (const Range& i : in)
      if (overlaps(w, i)) return FA_ERR_INVALID_ARG;
    for (const Range& r : out)
      if (overlaps(w, r)) return FA_ERR_INVALID_ARG;
  }

  rc = check_device();
  if (rc != FA_OK) return rc;

  fa::FwdParams p{q, k, v, o, lse, B, H_q, H_kv, N_q, N_kv, d, causal ? 1 : 0, scale};
  hipError_t err = fa::launch_fwd_split_bf16(p, num_splits, static_cast<float*>(workspace),
                                             reinterpret_cast<hipStream_t>(stream));
  return err == hipSuccess ? FA_OK : FA_ERR_HIP;
}

FA_EXPORT int fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                     int B, int H_q, int H_kv, int N_q, int N_kv, int d,
                                     int causal, float scale, int dtype, int num_splits, void* stream) {
  bool empty = false;
  Range in[3], out[2];
  int rc = check_splitkv(q, k, v, o, lse, B, H_q, H_kv, N_q, N_kv, d, scale, dtype, num_splits, &empty, in, out);
  if (rc != FA_OK || empty) return rc;
  const size_t ws_need = fa_fwd_splitkv_workspace_size(B, H_q, N_q, d, num_splits);
  if (ws_need > FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_INVALID_ARG;

  rc = check_device();
  if (rc != FA_OK) return rc;
  float* ws = nullptr;
  if (ws_need > 0 && fa::split_scratch_pointer(&ws) != hipSuccess) return FA_ERR_HIP;

  fa::FwdParams p{q, k, v, o, lse, B, H_q, H_kv, N_q, N_kv, d, causal ? 1 : 0, scale};
  hipError_t err = fa::launch_fwd_split_bf16(p, num_splits, ws, reinterpret_cast<hipStream_t>(stream));
  return err == hipSuccess ? FA_OK : FA_ERR_HIP;
}

FA_EXPORT int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                            const int* cu_seqlens_q, const int* cu_seqlens_k, int num_seqs,
                            int total_q, int total_k, int max_seqlen_q,
                            int H_q, int H_kv, int d, int causal, float scale, int dtype, void* stream) {
  if (num_seqs < 0 || total_q < 0 || total_k < 0 || max_seqlen_q < 0 || H_q < 0 || H_kv < 0 || d < 0)
    return FA_ERR_INVALID_ARG;
  if (dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
  if (dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (num_seqs == 0 || H_q == 0 || total_q == 0 || max_seqlen_q == 0) return FA_OK;
  if (H_kv == 0 || H_q % H_kv != 0) return FA_ERR_INVALID_ARG;
  if (total_k == 0) return FA_ERR_INVALID_ARG;
  if (max_seqlen_q > kMaxSeq) return FA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return FA_ERR_INVALID_ARG;
  if (scale < 0.0f) return FA_ERR_UNSUPPORTED;

  const size_t q_bytes = size_t(H_q) * total_q * d * 2;
  const size_t kv_bytes = size_t(H_kv) * total_k * d * 2;
  const size_t lse_bytes = size_t(H_q) * total_q * sizeof(float);
  const size_t cu_bytes = (size_t(num_seqs) + 1) * sizeof(int);
  if (!q || !k || !v || !o || !lse || !cu_seqlens_q || !cu_seqlens_k) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(cu_seqlens_q) & 3u) || (reinterpret_cast<uintptr_t>(cu_seqlens_k) & 3u))
    return FA_ERR_INVALID_ARG;
  const Range in[5] = {range_of(q, q_bytes), range_of(k, kv_bytes), range_of(v, kv_bytes),
                       range_of(cu_seqlens_q, cu_bytes), range_of(cu_seqlens_k, cu_bytes)};
  const Range out[2] = {range_of(o, q_bytes), range_of(lse, lse_bytes)};
  for (const Range& r : out)
    for (const Range& i : in)
      if (overlaps(r, i)) return FA_ERR_INVALID_ARG;
  if (overlaps(out[0], out[1])) return FA_ERR_INVALID_ARG;

  int rc = check_device();
  if (rc != FA_OK) return rc;

  fa::FwdParams p{q, k, v, o, lse, num_seqs, H_q, H_kv, max_seqlen_q, 0, d, causal ? 1 : 0, scale};
  fa::VarlenParams vl{cu_seqlens_q, cu_seqlens_k, total_q, total_k};
  hipError_t err = fa::launch_fwd_varlen_bf16(p, vl, reinterpret_cast<hipStream_t>(stream));
  return err == hipSuccess ? FA_OK : FA_ERR_HIP;
}

FA_EXPORT int fa_fwd_check(const void* q, const void* k, const float* lse, const int* rows, int n_rows,
                           int B, int H_q, int H_kv, int N_q, int N_kv, int d, int causal, float scale, int dtype,
                           float* result, void* stream) {
  bool empty = false;
  int rc = check_shape(B, H_q, H_kv, N_q, N_kv, d, scale, dtype, &empty);
  if (rc != FA_OK || empty) return rc;
  if (n_rows < 0) return FA_ERR_INVALID_ARG;
  if (n_rows == 0) return FA_OK;

  const size_t es = elem_size(dtype);
  const size_t q_bytes = size_t(B) * H_q * N_q * d * es;
  const size_t kv_bytes = size_t(B) * H_kv * N_kv * d * es;
  const size_t lse_bytes = size_t(B) * H_q * N_q * sizeof(float);
  const size_t rows_bytes = size_t(n_rows) * sizeof(int);
  const size_t res_bytes = size_t(B) * H_q * n_rows * sizeof(float);
  if (!q || !k || !lse || !rows || !result) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(lse) || !aligned16(result)) return FA_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(rows) & 3u) return FA_ERR_INVALID_ARG;
  const Range in[4] = {range_of(q, q_bytes), range_of(k, kv_bytes), range_of(lse, lse_bytes),
                       range_of(rows, rows_bytes)};
  const Range out = range_of(result, res_bytes);
  for (const Range& i : in)
    if (overlaps(out, i)) return FA_ERR_INVALID_ARG;

  rc = check_device();
  if (rc != FA_OK) return rc;

  fa::FwdParams p{q, k, nullptr, nullptr, const_cast<float*>(lse), B, H_q, H_kv, N_q, N_kv, d, causal ? 1 : 0, scale};
  hipError_t err = fa::launch_check(p, rows, n_rows, result, dtype, reinterpret_cast<hipStream_t>(stream));
  return err == hipSuccess ? FA_OK : FA_ERR_HIP;
}

FA_EXPORT int fa_quantize_fp8(const void* x, void* codes, float* descale, int B, int H, int N, int d, int d_major,
                              int dtype, void* stream) {
  if (B < 0 || H < 0 || N < 0 || d < 0) return FA_ERR_INVALID_ARG;
  if (dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (B == 0 || H == 0 || N == 0) return FA_OK;
  if (N > kMaxSeq) return FA_ERR_INVALID_ARG;
  if (!x || !codes || !descale) return FA_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(descale)) return FA_ERR_INVALID_ARG;
  const size_t n_rows = d_major ? size_t(fa::fp8_v_pad(N)) : size_t(N);
  const size_t x_bytes = size_t(B) * H * N * d * 2;
  const size_t c_bytes = size_t(B) * H * n_rows * d;
  const size_t s_bytes = size_t(B) * H * ((N + 127) / 128) * sizeof(float);
  const Range rx = range_of(x, x_bytes), rc_ = range_of(codes, c_bytes), rs = range_of(descale, s_bytes);
  if (overlaps(rx, rc_) || overlaps(rx, rs) || overlaps(rc_, rs)) return FA_ERR_INVALID_ARG;

  int rc = check_device();
  if (rc != FA_OK) return rc;
  hipError_t err = fa::launch_quantize_fp8(x, codes, descale, B, H, N, d, d_major ? 1 : 0,
                                           reinterpret_cast<hipStream_t>(stream));
  return err == hipSuccess ? FA_OK : FA_ERR_HIP;
}

FA_EXPORT int fa_fwd_fp8(const void* q8, const float* q_descale, const void* k8, const float* k_descale,
                         const void* v8, const float* v_descale, void* o, float* lse,
                         int B, int H_q, int H_kv, int N_q, int N_kv, int d, int causal, float scale, void* stream) {
  bool empty = false;
  int rc = check_shape(B, H_q, H_kv, N_q, N_kv, d, scale, FA_DTYPE_BF16, &empty);
  if (rc != FA_OK || empty) return rc;

  const size_t q_bytes = size_t(B) * H_q * N_q * d;
  const size_t k_bytes = size_t(B) * H_kv * N_kv * d;
  const size_t v_bytes = k_bytes;
  const size_t qs_bytes = size_t(B) * H_q * ((N_q + 127) / 128) * sizeof(float);
  const size_t ks_bytes = size_t(B) * H_kv * ((N_kv + 127) / 128) * sizeof(float);
  const size_t o_bytes = size_t(B) * H_q * N_q * d * 2;
  const size_t lse_bytes = size_t(B) * H_q * N_q * sizeof(float);
  if (!q8 || !q_descale || !k8 || !k_descale || !v8 || !v_descale || !o || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned16(q8) || !aligned16(k8) || !aligned16(v8) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(q_descale) | reinterpret_cast<uintptr_t>(k_descale) |
       reinterpret_cast<uintptr_t>(v_descale)) & 3u)
    return FA_ERR_INVALID_ARG;
  const Range in[6] = {range_of(q8, q_bytes), range_of(k8, k_bytes), range_of(v8, v_bytes),
                       range_of(q_descale, qs_bytes), range_of(k_descale, ks_bytes), range_of(v_descale, ks_bytes)};
  const Range out[2] = {range_of(o, o_bytes), range_of(lse, lse_bytes)};
  for (const Range& r : out)
    for (const Range& i : in)
      if (overlaps(r, i)) return FA_ERR_INVALID_ARG;
  if (overlaps(out[0], out[1])) return FA_ERR_INVALID_ARG;

  rc = check_device();
  if (rc != FA_OK) return rc;

  fa::Fp8FwdParams p{q8, q_descale, k8, k_descale, v8, v_descale, o, lse,
                     B, H_q, H_kv, N_q, N_kv, d, causal ? 1 : 0, scale};
  hipError_t err = fa::launch_fwd_fp8(p, reinterpret_cast<hipStream_t>(stream));
  return err == hipSuccess ? FA_OK : FA_ERR_HIP;
}

FA_EXPORT int fa_fwd_splitkv_fp8(const void* q, const void* k8, const float* k_descale, const void* v8,
                                 const float* v_descale, void* o, float* lse, int B, int H_q, int H_kv, int N_q,
                                 int N_kv, int d, int causal, float scale, int num_splits, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  bool empty = false;
  int rc = check_shape(B, H_q, H_kv, N_q, N_kv, d, scale, FA_DTYPE_BF16, &empty);
  if (rc != FA_OK || empty) return rc;

  const size_t q_bytes = size_t(B) * H_q * N_q * d * 2;
  const size_t k_bytes = size_t(B) * H_kv * N_kv * d;
  const size_t v_bytes = k_bytes;
  const size_t s_bytes = size_t(B) * H_kv * ((N_kv + 127) / 128) * sizeof(float);
  const size_t lse_bytes = size_t(B) * H_q * N_q * sizeof(float);
  if (!q || !k8 || !k_descale || !v8 || !v_descale || !o || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k8) || !aligned16(v8) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(k_descale) | reinterpret_cast<uintptr_t>(v_descale)) & 3u)
    return FA_ERR_INVALID_ARG;
  const Range in[5] = {range_of(q, q_bytes), range_of(k8, k_bytes), range_of(v8, v_bytes),
                       range_of(k_descale, s_bytes), range_of(v_descale, s_bytes)};
  const Range out[2] = {range_of(o, q_bytes), range_of(lse, lse_bytes)};
  for (const Range& r : out)
    for (const Range& i : in)
      if (overlaps(r, i)) return FA_ERR_INVALID_ARG;
  if (overlaps(out[0], out[1])) return FA_ERR_INVALID_ARG;

  if (num_splits < 1 || num_splits > 256) return FA_ERR_INVALID_ARG;
  if ((H_q / H_kv) * N_q > 32) return FA_ERR_UNSUPPORTED;

  const size_t ws_need = fa_fwd_splitkv_workspace_size(B, H_q, N_q, d, num_splits);
  if (ws_need > 0) {
    if (!workspace || !aligned16(workspace) || workspace_bytes < ws_need) return FA_ERR_INVALID_ARG;
    const Range w = range_of(workspace, ws_need);
    for (const Range& i : in)
      if (overlaps(w, i)) return FA_ERR_INVALID_ARG;
    for (const Range& r : out)
      if (overlaps(w, r)) return FA_ERR_INVALID_ARG;
  }

  rc = check_device();
  if (rc != FA_OK) return rc;

  fa::SplitFp8Params p{q, k8, k_descale, v8, v_descale, o, lse, B, H_q, H_kv, N_q, N_kv, d, causal ? 1 : 0, scale};
  hipError_t err = fa::launch_fwd_split_fp8kv(p, num_splits, static_cast<float*>(workspace),
                                              reinterpret_cast<hipStream_t>(stream));
  return err == hipSuccess ? FA_OK : FA_ERR_HIP;
}

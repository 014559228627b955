/*
 * fa.h -- C ABI of the exact-attention library (libfa.so) for AMD MI355X (gfx950).
 *
 * The library computes exact scaled-dot-product attention
 *     O = softmax(scale * Q K^T) V
 * and its gradients, without ever writing the N_q x N_kv score or probability
 * matrix to device memory.
 *
 * Sources for the operation (the pages this library is built from):
 *   - "FlashAttention" (LLM Inference Handbook, Kernel Optimization), section
 *     on why attention is slow: the definition softmax(Q K^T / sqrt(d_k)) V;
 *     section on how FlashAttention works: tiles of Q, K, V are moved on chip,
 *     the work is fused into one kernel and the N x N matrix is never stored.
 *   - "深度学习进阶（三十一）FlashAttention：IO 感知的精确注意力" (rkmt.cn blog),
 *     §2.1 (safe and online softmax) and §2.2 (a Q block stays resident while
 *     every K/V block streams past it; each row keeps a running max, a
 *     normalizer and an output accumulator that are rescaled when the max grows).
 *   - "Flash-Attention" (Awesome System Papers Wiki), core-idea section: the
 *     backward pass recomputes the probabilities from Q, K, V and a few saved
 *     per-row statistics; design-space section: causal, non-causal and GQA.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers are DEVICE pointers on the calling thread's current HIP device.
 *    The caller owns every buffer; the library never allocates, frees or keeps
 *    a pointer after returning. Every pointer must be 16-byte aligned.
 *  - All tensors are contiguous row-major:
 *        q, o, dO, dq : [B][H_q][N_q][d]
 *        k, v, dk, dv : [B][H_kv][N_kv][d]
 *        lse          : [B][H_q][N_q]            (float32)
 *  - dtype: FA_DTYPE_F32 (float32) or FA_DTYPE_BF16 (bfloat16). It applies to
 *    q, k, v, o and dO. lse, dq, dk and dv are always float32.
 *  - GQA: H_q must be a multiple of H_kv; query head h reads key/value head
 *    h / (H_q / H_kv) (integer division: consecutive query heads share).
 *  - causal != 0: query row i may attend key j only when j <= i (aligned at the
 *    top-left corner for every N_q, N_kv). causal == 0: every key is allowed.
 *  - scale multiplies Q K^T; it must be finite and >= 0. The usual value is
 *    1/sqrt(d).
 *  - Supported head dimensions: d = 64 or d = 128. N_q, N_kv <= 2^24.
 *  - stream: a hipStream_t (NULL = the default stream). Calls are asynchronous
 *    with respect to the host; faults inside a kernel surface at the caller's
 *    next synchronization.
 *  - Argument checks happen before any HIP call, in this order: negative
 *    sizes; dtype; d; empty problem (B, H_q or N_q zero -> FA_OK, nothing
 *    launched; fa_bwd zero-fills dk and dv then, see there); H_kv; N_kv;
 *    sizes; scale; null and misaligned pointers;
 *    overlap of an output with an input or another output; workspace. Then
 *    the device is checked (gfx950) and the kernels are launched.
 *  - Results are deterministic: the same inputs give bitwise equal outputs.
 *  - No global mutable state besides a per-device cache of the device check;
 *    concurrent calls on different streams are safe.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
#define FA_OK 0              /* success (work enqueued on the stream) */
#define FA_ERR_INVALID_ARG 1 /* a pointer, size, scale or workspace argument is invalid */
#define FA_ERR_UNSUPPORTED 2 /* dtype, head dimension, negative scale or device not supported */
#define FA_ERR_HIP 3         /* the HIP runtime reported an error at launch */

/* Element types for q, k, v, o, dO. */
#define FA_DTYPE_F32 0
#define FA_DTYPE_BF16 1

/*
 * fa_fwd -- attention forward.
 *
 * For every batch b, query head h and query row i (h_kv = h / (H_q/H_kv)):
 *     s_ij      = scale * <q[b,h,i,:], k[b,h_kv,j,:]>      over the allowed keys j
 *     lse[b,h,i]= ln sum_j exp(s_ij)                         (natural log, float32)
 *     o[b,h,i,:]= sum_j exp(s_ij - lse[b,h,i]) * v[b,h_kv,j,:]
 * This is the attention definition of the Handbook page with the safe-softmax
 * of blog §2.1, evaluated by the blockwise update of blog §2.2.
 *
 * Inputs : q, k, v (dtype). Outputs: o (dtype; bf16 results are rounded to
 * nearest even) and lse (float32); every element of both is written.
 * Errors : see the conventions above. N_kv = 0 with a non-empty problem is
 * FA_ERR_INVALID_ARG (softmax over no keys is undefined).
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H_q, int H_kv, int N_q, int N_kv, int d,
           int causal, float scale, int dtype, void* stream);

/*
 * fa_bwd_workspace_size -- bytes of device workspace fa_bwd needs for a
 * problem with B batches, H_q query heads and N_q query rows (a multiple of
 * 256): two float32 values per query row. Its content on entry does not
 * matter and on return is unspecified.
 */
size_t fa_bwd_workspace_size(int B, int H_q, int N_q);

/*
 * fa_bwd -- attention backward by recomputation (Wiki core-idea section: the
 * probabilities are rebuilt from q, k, v and the saved lse instead of being
 * stored by the forward pass).
 *
 * Gradients of the scalar L = sum(dO * o), with P_ij = exp(s_ij - lse_i):
 *     dv_j = sum_i P_ij dO_i
 *     dS_ij= P_ij * (<dO_i, v_j> - D_i),   D_i = <dO_i, o_i>
 *     dq_i = scale * sum_j dS_ij k_j
 *     dk_j = scale * sum_i dS_ij q_i
 * where o and lse are the outputs of fa_fwd on the same q, k, v. For GQA the
 * dk and dv of a key/value head sum over its H_q/H_kv query heads.
 *
 * Inputs : q, k, v, o, dO (dtype), lse (float32).
 * Outputs: dq, dk, dv (float32), fully written; keys no query may attend get 0.
 * No query rows (H_q or N_q zero, with B, H_kv and N_kv non-zero): no key is
 * attended, so dk and dv are filled with zeros on the stream; only dk and dv
 * are checked (non-null, 16-byte aligned, not overlapping each other) and
 * written, and N_kv must be at most 2^24. B, H_kv or N_kv zero with no query
 * rows is a no-op.
 * workspace: device memory of at least fa_bwd_workspace_size(B, H_q, N_q)
 * bytes, 16-byte aligned, not overlapping any other argument.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dO, float* dq, float* dk, float* dv,
           void* workspace, size_t workspace_bytes,
           int B, int H_q, int H_kv, int N_q, int N_kv, int d,
           int causal, float scale, int dtype, void* stream);

/*
 * fa_fwd_splitkv_workspace_size -- bytes of device workspace fa_fwd_splitkv
 * needs: 0 for num_splits <= 1, else B*H_q*N_q*num_splits*(d+1) float32
 * values (a partial output row and a partial logsumexp per key range),
 * rounded up to a multiple of 256. Returns 0 for non-positive sizes.
 */
size_t fa_fwd_splitkv_workspace_size(int B, int H_q, int N_q, int d, int num_splits);

/*
 * fa_fwd_splitkv -- attention forward for few query rows against many keys
 * (decode-like shapes), with the keys of every (batch, key/value head) cut
 * into num_splits consecutive ranges processed in parallel and merged.
 *
 * Computes the same o and lse as fa_fwd (same arguments, conventions and
 * layouts). Method: "深度学习进阶（三十一）FlashAttention：IO 感知的精确注意力"
 * (rkmt.cn blog) §2.2 -- each key range yields an output normalised by its
 * own sum and a logsumexp; ranges are merged by rescaling each with the
 * exponential of its logsumexp minus the combined one (the same rule that
 * merges consecutive key blocks), in range order, so results are
 * deterministic. Key ranges hold ceil(N_kv/num_splits) keys rounded up to a
 * multiple of 32; ranges past the end (or past the last key any row may
 * attend, when causal) contribute nothing.
 *
 * Restrictions beyond fa_fwd: dtype must be FA_DTYPE_BF16 (else
 * FA_ERR_UNSUPPORTED); the rows of one key/value head, (H_q/H_kv)*N_q, must
 * be at most 32 (else FA_ERR_UNSUPPORTED; use fa_fwd); 1 <= num_splits <= 256
 * (else FA_ERR_INVALID_ARG). workspace: device memory of at least
 * fa_fwd_splitkv_workspace_size(B, H_q, N_q, d, num_splits) bytes, 16-byte
 * aligned, not overlapping any other argument (may be NULL when that size is
 * 0); its content on entry does not matter and on return is unspecified.
 * Argument checks happen in the order of fa_fwd, then num_splits, dtype and
 * the row count, then the workspace.
 */
int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H_q, int H_kv, int N_q, int N_kv, int d,
                   int causal, float scale, int dtype, int num_splits,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Size of the statically reserved device array fa_fwd_splitkv_noalloc uses
 * in place of a workspace (per device, held until the process ends). */
#define FA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/*
 * fa_fwd_splitkv_noalloc -- fa_fwd_splitkv without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * serving loops that must not call an allocator, harnesses that forbid it.
 *
 * Same arguments (minus workspace and workspace_bytes), checks, kernels and
 * results as fa_fwd_splitkv. The key-range partials live in a device array
 * of FA_NOALLOC_SCRATCH_BYTES that the library reserves statically on every
 * device it runs on (its address is looked up on the first call on a device)
 * and that stays reserved until the process ends. The call allocates and
 * frees nothing. Every (row, key range) partial is rewritten by each call, so
 * the array's content on entry does not matter.
 * Errors: as fa_fwd_splitkv, plus FA_ERR_INVALID_ARG (before any HIP call)
 * when fa_fwd_splitkv_workspace_size(B, H_q, N_q, d, num_splits) exceeds
 * FA_NOALLOC_SCRATCH_BYTES, and FA_ERR_HIP if the array's address cannot be
 * obtained. All calls on one device share the array: calls that may run at
 * the same time on one device (different streams, or different host threads
 * without ordering) race and give wrong results; order them on one stream.
 */
int fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H_q, int H_kv, int N_q, int N_kv, int d,
                           int causal, float scale, int dtype, int num_splits, void* stream);

/*
 * fa_fwd_varlen -- attention forward over a batch of sequences of different
 * lengths, packed without padding.
 *
 * Layouts (head-major, sequences packed along the row axis):
 *     q, o : [H_q][total_q][d]      k, v : [H_kv][total_k][d]
 *     lse  : [H_q][total_q]          (float32, natural log)
 * cu_seqlens_q, cu_seqlens_k: DEVICE int32 arrays of num_seqs + 1 prefix
 * offsets: sequence b owns query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1
 * and key rows cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1 (first entry 0,
 * non-decreasing, last entry total_q / total_k). max_seqlen_q must be at
 * least the longest query sequence (rows past it are not computed).
 * Within each sequence the operation is exactly that of fa_fwd (same scale,
 * causal rule counted from the sequence's first row and key, GQA mapping).
 * A sequence with no keys gets o = 0 and lse = -inf on its rows.
 * The offsets are read on the device and not validated on the host; offsets
 * outside [0, total] are clamped, so inconsistent ones give wrong rows but no
 * access outside the tensors.
 *
 * dtype must be FA_DTYPE_BF16 (else FA_ERR_UNSUPPORTED). Argument checks
 * before any HIP call: negative sizes (FA_ERR_INVALID_ARG); dtype and d;
 * empty problem (num_seqs, H_q, total_q or max_seqlen_q zero -> FA_OK);
 * H_kv; total_k = 0 (FA_ERR_INVALID_ARG); max_seqlen_q > 2^24; scale; null or
 * misaligned pointers (16 bytes; 4 for the offset arrays); an output
 * overlapping an input or the other output.
 */
int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                  const int* cu_seqlens_q, const int* cu_seqlens_k, int num_seqs,
                  int total_q, int total_k, int max_seqlen_q,
                  int H_q, int H_kv, int d, int causal, float scale, int dtype, void* stream);

/*
 * fa_fwd_check -- on-GPU self-check of a forward result. For each batch b,
 * query head h and each of the n_rows sampled query rows i = rows[r]
 * (DEVICE int32 array; values are clamped to [0, N_q-1]):
 *     result[b][h][r] = | sum_j exp(scale * <q[b,h,i,:], k[b,h_kv,j,:]> - lse[b,h,i]) - 1 |
 * over the keys row i may attend (float32, DEVICE array [B][H_q][n_rows]).
 * With the lse of fa_fwd the probabilities of every row sum to one, so each
 * value is near 0 (about the lse tolerance, 1e-3 for bf16); a corrupted
 * statistic shows up directly ("Flash-Attention" (Awesome System Papers Wiki),
 * core-idea section: the backward pass rebuilds the probabilities from these
 * statistics). The scores are recomputed with plain fp32 dot products,
 * independently of the forward kernels; deterministic.
 * q, k, lse: as for fa_fwd (dtype F32 or BF16). n_rows = 0 (or an empty
 * problem) is a no-op. Argument checks as fa_fwd, then n_rows < 0, null or
 * misaligned rows (4 bytes) / result (16 bytes), result overlapping an input.
 */
int fa_fwd_check(const void* q, const void* k, const float* lse, const int* rows, int n_rows,
                 int B, int H_q, int H_kv, int N_q, int N_kv, int d, int causal, float scale, int dtype,
                 float* result, void* stream);

/*
 * fa_quantize_fp8 -- block quantization of a bf16 tensor to OCP e4m3 codes.
 *
 * FP8 inputs are one of the low-precision paths of the FlashAttention line,
 * which must handle quantization scales and outliers ("Flash-Attention"
 * (Awesome System Papers Wiki), key-observation and design-space sections).
 * x: bf16 [B][H][N][d] (finite values). For every (b, h) and every block of
 * 128 consecutive rows (the last one may be shorter), in float32:
 *     amax = max |x| over the block, descale = amax / 448, inv = 448 / amax,
 *     code = e4m3(x * inv)       round to nearest even, saturated to +-448
 * (when inv is not finite, i.e. amax = 0 or below 448 / FLT_MAX, every code
 * of the block is 0). The value a code stands for is e4m3(code) * descale.
 * Outputs: descale float32 [B][H][ceil(N/128)]; codes uint8, either
 *   d_major == 0: [B][H][N][d]  (row-major: the layout fa_fwd_fp8 and
 *                 fa_fwd_splitkv_fp8 read for q, k and v)
 *   d_major != 0: [B][H][d][N_pad], N_pad = N rounded up to a multiple of 128,
 *                 codes past N are 0 (key index contiguous, for consumers that
 *                 want the transposed layout).
 * Deterministic and bit-exact (the float32 steps are correctly rounded).
 * d = 64 or 128, N <= 2^24; B, H or N = 0 is a no-op. Errors: negative
 * sizes, null or misaligned (16 bytes) pointers, outputs overlapping x or
 * each other -> FA_ERR_INVALID_ARG; other d or dtype != FA_DTYPE_BF16 ->
 * FA_ERR_UNSUPPORTED.
 */
int fa_quantize_fp8(const void* x, void* codes, float* descale, int B, int H, int N, int d, int d_major,
                    int dtype, void* stream);

/*
 * fa_fwd_fp8 -- attention forward on FP8 (e4m3) inputs with block scales.
 *
 * Computes O and LSE as fa_fwd does, for the dequantized inputs
 *     Q = e4m3(q8) * q_descale,  K = e4m3(k8) * k_descale,  V = e4m3(v8) * v_descale
 * (descale per 128-row block as written by fa_quantize_fp8), on the FP8
 * matrix instructions ("深度学习进阶（三十一）FlashAttention：IO 感知的精确注意力"
 * (rkmt.cn blog), version comparison table: FP8 is one of FlashAttention-3's
 * additions). The scores and the row sums are float32; the probabilities
 * are rounded to e4m3 (after multiplication by 8 * vd / vd_max of their V
 * block) for the P V product only, so one output element is within
 *     2^-4 * sum_j max(w_j, 2^-6 / (cv_j * L)) * |V_j|
 * of the exact value (w the exact probabilities, L = sum_j exp(s_j - max s),
 * cv_j = 8 * vd_j / vd_max), plus float32 and bf16 output rounding; the
 * LSE is as accurate as fa_fwd's in bf16.
 *   q8 [B][H_q][N_q][d], k8 and v8 [B][H_kv][N_kv][d]: row-major codes
 *       (fa_quantize_fp8 with d_major = 0);
 *   q_descale [B][H_q][ceil(N_q/128)], k_descale and v_descale
 *       [B][H_kv][ceil(N_kv/128)]: float32, finite and >= 0;
 *   o: bf16 [B][H_q][N_q][d]; lse: float32 [B][H_q][N_q] (natural log).
 * d = 64 or 128; causal, GQA, scale and the size limits as fa_fwd. Errors as
 * fa_fwd (dtype is implied); descale pointers must be 4-byte aligned.
 */
int fa_fwd_fp8(const void* q8, const float* q_descale, const void* k8, const float* k_descale,
               const void* v8, const float* v_descale, void* o, float* lse,
               int B, int H_q, int H_kv, int N_q, int N_kv, int d, int causal, float scale, void* stream);

/*
 * fa_fwd_splitkv_fp8 -- split-KV forward (as fa_fwd_splitkv) with the keys and
 * values in FP8: a bf16 query against an e4m3 key/value cache.
 *
 * Computes O and LSE for q (bf16 values) and the dequantized
 *     K = e4m3(k8) * k_descale,  V = e4m3(v8) * v_descale
 * (one scale per 128-key block, as fa_quantize_fp8 writes them). Decoding
 * reads every cached key once per new token, so the bytes per key decide its
 * speed; FP8 halves them (the split-KV idea of the FlashDecoding paragraph of
 * "深度学习进阶（三十一）FlashAttention：IO 感知的精确注意力" (rkmt.cn blog) §3,
 * with FP8 inputs, one of FlashAttention-3's additions in that blog's version
 * table). The codes are widened to bf16 exactly and the arithmetic is
 * fa_fwd_splitkv's, so the bf16 tolerances of fa_fwd apply against the
 * exact attention of q and the dequantized K, V.
 *   q, o: bf16 [B][H_q][N_q][d]; lse float32 [B][H_q][N_q];
 *   k8, v8: [B][H_kv][N_kv][d] codes, row-major like a bf16 cache (so that
 *       appending a token writes one row; fa_quantize_fp8 with d_major = 0);
 *   k_descale, v_descale: float32 [B][H_kv][ceil(N_kv/128)], finite, >= 0.
 * num_splits, workspace and the (H_q/H_kv)*N_q <= 32 limit as fa_fwd_splitkv
 * (fa_fwd_splitkv_workspace_size gives the workspace). Errors as
 * fa_fwd_splitkv; descale pointers must be 4-byte aligned.
 */
int fa_fwd_splitkv_fp8(const void* q, const void* k8, const float* k_descale, const void* v8,
                       const float* v_descale, void* o, float* lse, int B, int H_q, int H_kv, int N_q, int N_kv,
                       int d, int causal, float scale, int num_splits, void* workspace, size_t workspace_bytes,
                       void* stream);

/* fa_status_string -- a static, NUL-terminated description of a status code. */
const char* fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */

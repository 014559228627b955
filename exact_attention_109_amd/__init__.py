"""Exact attention on AMD MI355X (gfx950): Python binding of libfa.so.

The library's C ABI (include/fa.h) exports fa_fwd, fa_bwd,
fa_bwd_workspace_size, fa_fwd_splitkv, fa_fwd_splitkv_workspace_size,
fa_fwd_splitkv_noalloc, fa_fwd_varlen, fa_fwd_check, fa_quantize_fp8, fa_fwd_fp8, fa_fwd_splitkv_fp8 and fa_status_string. This module exposes the same names with the same
arguments (device pointers as integers, sizes, flags, a stream handle) plus
convenience wrappers over torch tensors:

    o, lse = fwd(q, k, v, causal=False, scale=None)
    o, lse = fwd_splitkv(q, k, v, num_splits, causal=False, scale=None)
    o, lse = fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, causal=False, scale=None)
    err = fwd_check(q, k, lse, rows, causal=False, scale=None)
    codes, descale = quantize_fp8(x, d_major=False)
    o, lse = fwd_fp8(q8, q_descale, k8, k_descale, v8, v_descale, causal=False, scale=None)
    o, lse = fwd_splitkv_fp8(q, k8, k_descale, v8, v_descale, num_splits, causal=False, scale=None)
    dq, dk, dv = bwd(q, k, v, o, lse, do, causal=False, scale=None)

The wrappers only marshal arguments: torch allocates device memory and
supplies the current stream; every step of the computation runs in the HIP
kernels of libfa.so. There is no fallback path: if the library is missing
or a call fails, an exception is raised.
"""

from __future__ import annotations

import ctypes
import math
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libfa.so")

FA_OK = 0
FA_ERR_INVALID_ARG = 1
FA_ERR_UNSUPPORTED = 2
FA_ERR_HIP = 3
FA_DTYPE_F32 = 0
FA_DTYPE_BF16 = 1
NOALLOC_SCRATCH_BYTES = 16 << 20   # FA_NOALLOC_SCRATCH_BYTES of include/fa.h

_lib = None


class FaError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {fa_status_string(status)} (status {status})")
        self.status = status


def library_path() -> str:
    """The library this process loads: libfa.so, or the build named by the
    FA_LIBRARY environment variable (the check builds of _build.py)."""
    return os.environ.get("FA_LIBRARY") or LIB_PATH


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load the library (once) and declare its entry points. Raises if it has
    not been built."""
    global _lib
    if _lib is not None:
        return _lib
    _lib = open_library(path or library_path())
    return _lib


def open_library(path: str) -> ctypes.CDLL:
    """A separate handle on a build of the library at `path`, with every entry
    point declared (for comparing builds; the module functions use
    load_library's)."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`"
                           " or `python exact_attention_109_amd/_build.py`")
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp]
    lib.fa_fwd.restype = i
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, i, f, i, vp]
    lib.fa_bwd.restype = i
    lib.fa_bwd_workspace_size.argtypes = [i, i, i]
    lib.fa_bwd_workspace_size.restype = sz
    lib.fa_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, i, vp, sz, vp]
    lib.fa_fwd_splitkv.restype = i
    lib.fa_fwd_splitkv_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, i, vp]
    lib.fa_fwd_splitkv_noalloc.restype = i
    lib.fa_fwd_splitkv_workspace_size.argtypes = [i, i, i, i, i]
    lib.fa_fwd_splitkv_workspace_size.restype = sz
    lib.fa_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, i, vp]
    lib.fa_fwd_varlen.restype = i
    lib.fa_fwd_check.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, i, vp, vp]
    lib.fa_fwd_check.restype = i
    lib.fa_quantize_fp8.argtypes = [vp, vp, vp, i, i, i, i, i, i, vp]
    lib.fa_quantize_fp8.restype = i
    lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp]
    lib.fa_fwd_fp8.restype = i
    lib.fa_fwd_splitkv_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp, sz, vp]
    lib.fa_fwd_splitkv_fp8.restype = i
    lib.fa_status_string.argtypes = [i]
    lib.fa_status_string.restype = ctypes.c_char_p
    return lib


# ---------------------------------------------------------------------------
# The C entry points, one to one
# ---------------------------------------------------------------------------

def fa_fwd(q, k, v, o, lse, B, H_q, H_kv, N_q, N_kv, d, causal, scale, dtype, stream) -> int:
    return load_library().fa_fwd(q, k, v, o, lse, B, H_q, H_kv, N_q, N_kv, d, int(causal), float(scale),
                                 dtype, stream)


def fa_bwd(q, k, v, o, lse, dO, dq, dk, dv, workspace, workspace_bytes, B, H_q, H_kv, N_q, N_kv, d,
           causal, scale, dtype, stream) -> int:
    return load_library().fa_bwd(q, k, v, o, lse, dO, dq, dk, dv, workspace, workspace_bytes, B, H_q, H_kv,
                                 N_q, N_kv, d, int(causal), float(scale), dtype, stream)


def fa_bwd_workspace_size(B, H_q, N_q) -> int:
    return load_library().fa_bwd_workspace_size(B, H_q, N_q)


def fa_fwd_splitkv(q, k, v, o, lse, B, H_q, H_kv, N_q, N_kv, d, causal, scale, dtype, num_splits, workspace,
                   workspace_bytes, stream) -> int:
    return load_library().fa_fwd_splitkv(q, k, v, o, lse, B, H_q, H_kv, N_q, N_kv, d, int(causal), float(scale),
                                         dtype, num_splits, workspace, workspace_bytes, stream)


def fa_fwd_splitkv_noalloc(q, k, v, o, lse, B, H_q, H_kv, N_q, N_kv, d, causal, scale, dtype, num_splits,
                           stream) -> int:
    return load_library().fa_fwd_splitkv_noalloc(q, k, v, o, lse, B, H_q, H_kv, N_q, N_kv, d, int(causal),
                                                 float(scale), dtype, num_splits, stream)


def fa_fwd_splitkv_workspace_size(B, H_q, N_q, d, num_splits) -> int:
    return load_library().fa_fwd_splitkv_workspace_size(B, H_q, N_q, d, num_splits)


def fa_fwd_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, num_seqs, total_q, total_k, max_seqlen_q, H_q,
                  H_kv, d, causal, scale, dtype, stream) -> int:
    return load_library().fa_fwd_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, num_seqs, total_q, total_k,
                                        max_seqlen_q, H_q, H_kv, d, int(causal), float(scale), dtype, stream)


def fa_fwd_check(q, k, lse, rows, n_rows, B, H_q, H_kv, N_q, N_kv, d, causal, scale, dtype, result, stream) -> int:
    return load_library().fa_fwd_check(q, k, lse, rows, n_rows, B, H_q, H_kv, N_q, N_kv, d, int(causal),
                                       float(scale), dtype, result, stream)


def fa_quantize_fp8(x, codes, descale, B, H, N, d, d_major, dtype, stream) -> int:
    return load_library().fa_quantize_fp8(x, codes, descale, B, H, N, d, int(d_major), dtype, stream)


def fa_fwd_fp8(q8, q_descale, k8, k_descale, v8, v_descale, o, lse, B, H_q, H_kv, N_q, N_kv, d, causal, scale,
               stream) -> int:
    return load_library().fa_fwd_fp8(q8, q_descale, k8, k_descale, v8, v_descale, o, lse, B, H_q, H_kv, N_q, N_kv,
                                     d, int(causal), float(scale), stream)


def fa_fwd_splitkv_fp8(q, k8, k_descale, v8, v_descale, o, lse, B, H_q, H_kv, N_q, N_kv, d, causal, scale,
                       num_splits, workspace, workspace_bytes, stream) -> int:
    return load_library().fa_fwd_splitkv_fp8(q, k8, k_descale, v8, v_descale, o, lse, B, H_q, H_kv, N_q, N_kv, d,
                                             int(causal), float(scale), num_splits, workspace, workspace_bytes,
                                             stream)


def fa_status_string(status: int) -> str:
    return load_library().fa_status_string(status).decode()


# ---------------------------------------------------------------------------
# torch tensor wrappers
# ---------------------------------------------------------------------------

def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return FA_DTYPE_BF16
    if t.dtype == torch.float32:
        return FA_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use torch.bfloat16 or torch.float32")


def _check(t, name, dtype=None, shape=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _stream_handle(t):
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def fwd(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None):
    """Attention forward on tensors q [B,H_q,N_q,d], k and v [B,H_kv,N_kv,d].

    Returns (o, lse): o like q, lse float32 [B,H_q,N_q] (natural log)."""
    import torch
    B, H_q, N_q, d = q.shape
    _, H_kv, N_kv, _ = k.shape
    _check(q, "q")
    _check(k, "k", q.dtype, (B, H_kv, N_kv, d))
    _check(v, "v", q.dtype, (B, H_kv, N_kv, d))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H_q, N_q), dtype=torch.float32, device=q.device)
    _check(out, "out", q.dtype, q.shape)
    _check(lse, "lse", torch.float32, (B, H_q, N_q))
    rc = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                B, H_q, H_kv, N_q, N_kv, d, causal, scale, _dtype_code(q), _stream_handle(q))
    if rc != FA_OK:
        raise FaError(rc, "fa_fwd")
    return out, lse


def default_num_splits(B: int, H_kv: int, N_kv: int, num_cus: int) -> int:
    """Key ranges per (batch, key/value head) for fwd_splitkv: enough
    workgroups for about two per compute unit, at least 4 tiles of 32 keys
    (one per wave) in each range, at most 256 ranges."""
    want = -(-2 * num_cus // max(1, B * H_kv))
    return int(max(1, min(want, 256, -(-N_kv // 128))))


def fwd_splitkv(q, k, v, num_splits: int | None = None, causal: bool = False, scale: float | None = None,
                out=None, lse=None, workspace=None):
    """Split-KV forward (bf16; (H_q/H_kv)*N_q <= 32): the same result as fwd,
    with the keys cut into num_splits ranges that run in parallel (default:
    default_num_splits for the current device)."""
    import torch
    B, H_q, N_q, d = q.shape
    _, H_kv, N_kv, _ = k.shape
    if num_splits is None:
        num_splits = default_num_splits(B, H_kv, N_kv, torch.cuda.get_device_properties(q.device).multi_processor_count)
    _check(q, "q")
    _check(k, "k", q.dtype, (B, H_kv, N_kv, d))
    _check(v, "v", q.dtype, (B, H_kv, N_kv, d))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H_q, N_q), dtype=torch.float32, device=q.device)
    _check(out, "out", q.dtype, q.shape)
    _check(lse, "lse", torch.float32, (B, H_q, N_q))
    ws_bytes = fa_fwd_splitkv_workspace_size(B, H_q, N_q, d, num_splits)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty((ws_bytes,), dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                        B, H_q, H_kv, N_q, N_kv, d, causal, scale, _dtype_code(q), num_splits, ws_ptr, ws_len,
                        _stream_handle(q))
    if rc != FA_OK:
        raise FaError(rc, "fa_fwd_splitkv")
    return out, lse


def fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, causal: bool = False,
               scale: float | None = None, out=None, lse=None):
    """Forward over packed sequences: q [H_q, total_q, d], k and v
    [H_kv, total_k, d] (bf16), cu_seqlens_* int32 GPU tensors of num_seqs + 1
    prefix offsets. Returns (o like q, lse float32 [H_q, total_q])."""
    import torch
    H_q, total_q, d = q.shape
    H_kv, total_k, _ = k.shape
    _check(q, "q")
    _check(k, "k", q.dtype, (H_kv, total_k, d))
    _check(v, "v", q.dtype, (H_kv, total_k, d))
    _check(cu_seqlens_q, "cu_seqlens_q", torch.int32)
    _check(cu_seqlens_k, "cu_seqlens_k", torch.int32, cu_seqlens_q.shape)
    num_seqs = cu_seqlens_q.numel() - 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((H_q, total_q), dtype=torch.float32, device=q.device)
    _check(out, "out", q.dtype, q.shape)
    _check(lse, "lse", torch.float32, (H_q, total_q))
    rc = fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                       cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), num_seqs, total_q, total_k, max_seqlen_q,
                       H_q, H_kv, d, causal, scale, _dtype_code(q), _stream_handle(q))
    if rc != FA_OK:
        raise FaError(rc, "fa_fwd_varlen")
    return out, lse


def fwd_check(q, k, lse, rows, causal: bool = False, scale: float | None = None):
    """Self-check of a forward result: |sum_j exp(scale q_i.k_j - lse_i) - 1|
    for the query rows `rows` (int32 GPU tensor) of every (batch, head).
    Returns a float32 tensor [B, H_q, len(rows)]."""
    import torch
    B, H_q, N_q, d = q.shape
    _, H_kv, N_kv, _ = k.shape
    _check(q, "q")
    _check(k, "k", q.dtype, (B, H_kv, N_kv, d))
    _check(lse, "lse", torch.float32, (B, H_q, N_q))
    _check(rows, "rows", torch.int32)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    result = torch.empty((B, H_q, rows.numel()), dtype=torch.float32, device=q.device)
    rc = fa_fwd_check(q.data_ptr(), k.data_ptr(), lse.data_ptr(), rows.data_ptr(), rows.numel(), B, H_q, H_kv,
                      N_q, N_kv, d, causal, scale, _dtype_code(q), result.data_ptr(), _stream_handle(q))
    if rc != FA_OK:
        raise FaError(rc, "fa_fwd_check")
    return result


def bwd(q, k, v, o, lse, do, causal: bool = False, scale: float | None = None, workspace=None):
    """Attention backward; o and lse from fwd on the same inputs.

    Returns (dq, dk, dv), all float32."""
    import torch
    B, H_q, N_q, d = q.shape
    _, H_kv, N_kv, _ = k.shape
    _check(q, "q")
    _check(k, "k", q.dtype, (B, H_kv, N_kv, d))
    _check(v, "v", q.dtype, (B, H_kv, N_kv, d))
    _check(o, "o", q.dtype, q.shape)
    _check(do, "do", q.dtype, q.shape)
    _check(lse, "lse", torch.float32, (B, H_q, N_q))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    dk = torch.empty(k.shape, dtype=torch.float32, device=q.device)
    dv = torch.empty(v.shape, dtype=torch.float32, device=q.device)
    ws_bytes = fa_bwd_workspace_size(B, H_q, N_q)
    if workspace is None:
        workspace = torch.empty((max(ws_bytes, 256),), dtype=torch.uint8, device=q.device)
    rc = fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(), workspace.numel(),
                B, H_q, H_kv, N_q, N_kv, d, causal, scale, _dtype_code(q), _stream_handle(q))
    if rc != FA_OK:
        raise FaError(rc, "fa_bwd")
    return dq, dk, dv


__all__ = ["fa_fwd", "fa_bwd", "fa_bwd_workspace_size", "fa_fwd_splitkv", "fa_fwd_splitkv_workspace_size",
           "fa_fwd_splitkv_noalloc", "NOALLOC_SCRATCH_BYTES",
           "fa_fwd_varlen", "fa_fwd_check", "fa_status_string", "fwd", "fwd_splitkv", "fwd_varlen", "fwd_check", "default_num_splits", "bwd", "load_library",
           "FaError", "FA_OK", "FA_ERR_INVALID_ARG", "FA_ERR_UNSUPPORTED", "FA_ERR_HIP", "FA_DTYPE_F32",
           "FA_DTYPE_BF16", "LIB_PATH", "library_path", "open_library"]


FP8_BLOCK = 128   # rows per descale block


def fp8_v_pad(n: int) -> int:
    """Row length of the quantizer's d-major layout: n rounded up to 128."""
    return (n + 127) // 128 * 128


def quantize_fp8(x, d_major: bool = False, codes=None, descale=None):
    """Block-quantize a bf16 tensor x [B, H, N, d] to e4m3 codes (uint8).

    Returns (codes, descale): codes [B, H, N, d] (the layout fwd_fp8 and
    fwd_splitkv_fp8 read), or [B, H, d, fp8_v_pad(N)] when d_major;
    descale float32 [B, H, ceil(N/128)]."""
    import torch
    _check(x, "x", torch.bfloat16)
    B, H, N, d = x.shape
    cshape = (B, H, d, fp8_v_pad(N)) if d_major else (B, H, N, d)
    if codes is None:
        codes = torch.empty(cshape, dtype=torch.uint8, device=x.device)
    if descale is None:
        descale = torch.empty((B, H, (N + FP8_BLOCK - 1) // FP8_BLOCK), dtype=torch.float32, device=x.device)
    _check(codes, "codes", torch.uint8, cshape)
    _check(descale, "descale", torch.float32, (B, H, (N + FP8_BLOCK - 1) // FP8_BLOCK))
    st = fa_quantize_fp8(x.data_ptr(), codes.data_ptr(), descale.data_ptr(), B, H, N, d, d_major,
                         FA_DTYPE_BF16, _stream_handle(x))
    if st != FA_OK:
        raise FaError(st, "fa_quantize_fp8")
    return codes, descale


def fwd_fp8(q8, q_descale, k8, k_descale, v8, v_descale, causal: bool = False, scale: float | None = None,
            out=None, lse=None):
    """Attention forward on FP8 codes: q8 [B,H_q,N_q,d], k8 and v8
    [B,H_kv,N_kv,d] (row-major), descales per 128-row block.
    Returns (o bf16 [B,H_q,N_q,d], lse float32 [B,H_q,N_q])."""
    import torch
    B, H_q, N_q, d = q8.shape
    _, H_kv, N_kv, _ = k8.shape
    _check(q8, "q8", torch.uint8)
    _check(k8, "k8", torch.uint8, (B, H_kv, N_kv, d))
    _check(v8, "v8", torch.uint8, (B, H_kv, N_kv, d))
    nbq = (N_q + FP8_BLOCK - 1) // FP8_BLOCK
    nbk = (N_kv + FP8_BLOCK - 1) // FP8_BLOCK
    _check(q_descale, "q_descale", torch.float32, (B, H_q, nbq))
    _check(k_descale, "k_descale", torch.float32, (B, H_kv, nbk))
    _check(v_descale, "v_descale", torch.float32, (B, H_kv, nbk))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H_q, N_q, d), dtype=torch.bfloat16, device=q8.device)
    if lse is None:
        lse = torch.empty((B, H_q, N_q), dtype=torch.float32, device=q8.device)
    _check(out, "out", torch.bfloat16, (B, H_q, N_q, d))
    _check(lse, "lse", torch.float32, (B, H_q, N_q))
    st = fa_fwd_fp8(q8.data_ptr(), q_descale.data_ptr(), k8.data_ptr(), k_descale.data_ptr(), v8.data_ptr(),
                    v_descale.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H_q, H_kv, N_q, N_kv, d, causal,
                    scale, _stream_handle(q8))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_fp8")
    return out, lse


def fwd_splitkv_fp8(q, k8, k_descale, v8, v_descale, num_splits: int | None = None, causal: bool = False,
                    scale: float | None = None, out=None, lse=None, workspace=None):
    """Split-KV forward of bf16 queries q [B,H_q,N_q,d] against an FP8 cache:
    k8 and v8 [B,H_kv,N_kv,d] (row-major codes), descales per 128-key block
    ((H_q/H_kv)*N_q <= 32)."""
    import torch
    _check(q, "q", torch.bfloat16)
    B, H_q, N_q, d = q.shape
    _, H_kv, N_kv, _ = k8.shape
    _check(k8, "k8", torch.uint8, (B, H_kv, N_kv, d))
    _check(v8, "v8", torch.uint8, (B, H_kv, N_kv, d))
    nbk = (N_kv + FP8_BLOCK - 1) // FP8_BLOCK
    _check(k_descale, "k_descale", torch.float32, (B, H_kv, nbk))
    _check(v_descale, "v_descale", torch.float32, (B, H_kv, nbk))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if num_splits is None:
        num_splits = default_num_splits(B, H_kv, N_kv, torch.cuda.get_device_properties(q.device).multi_processor_count)
    if out is None:
        out = torch.empty((B, H_q, N_q, d), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, H_q, N_q), dtype=torch.float32, device=q.device)
    _check(out, "out", torch.bfloat16, (B, H_q, N_q, d))
    _check(lse, "lse", torch.float32, (B, H_q, N_q))
    need = fa_fwd_splitkv_workspace_size(B, H_q, N_q, d, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty((need,), dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = fa_fwd_splitkv_fp8(q.data_ptr(), k8.data_ptr(), k_descale.data_ptr(), v8.data_ptr(), v_descale.data_ptr(),
                            out.data_ptr(), lse.data_ptr(), B, H_q, H_kv, N_q, N_kv, d, causal, scale, num_splits,
                            ws_ptr, ws_bytes, _stream_handle(q))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_splitkv_fp8")
    return out, lse

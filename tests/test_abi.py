"""The C ABI without a GPU: the library loads, exports every function that
include/fa.h declares, and rejects invalid arguments with the documented
status before making any HIP call."""

import ctypes
import os
import re
import subprocess

import pytest

from tests.gpu_util import ROOT, ensure_library
import exact_attention_109_amd as fa

HEADER = os.path.join(ROOT, "include", "fa.h")


@pytest.fixture(scope="module")
def lib():
    ensure_library()
    return fa.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    assert declared_functions() == ["fa_bwd", "fa_bwd_workspace_size", "fa_fwd", "fa_fwd_check", "fa_fwd_fp8",
                                    "fa_fwd_splitkv", "fa_fwd_splitkv_fp8", "fa_fwd_splitkv_noalloc",
                                    "fa_fwd_splitkv_workspace_size", "fa_fwd_varlen", "fa_quantize_fp8",
                                    "fa_status_string"]


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", fa.library_path()], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (fa_\w+)", out))
    assert set(declared_functions()) <= exported
    # nothing else with C linkage leaks out under the fa_ prefix
    assert exported == set(declared_functions())


def test_status_strings(lib):
    for code in (fa.FA_OK, fa.FA_ERR_INVALID_ARG, fa.FA_ERR_UNSUPPORTED, fa.FA_ERR_HIP):
        s = fa.fa_status_string(code)
        assert s.startswith("FA_")
    assert "unknown" in fa.fa_status_string(12345)


def test_workspace_size():
    assert fa.fa_bwd_workspace_size(2, 16, 4096) == 2 * 2 * 16 * 4096 * 4
    assert fa.fa_bwd_workspace_size(1, 1, 3) == 256
    assert fa.fa_bwd_workspace_size(0, 1, 3) == 0
    assert fa.fa_bwd_workspace_size(1, 1, 65) % 256 == 0


# Fake, never dereferenced "device" addresses: validation fails before any use.
A = 0x10000000
STEP = 0x01000000


def ptrs(n, base=A):
    return [base + i * STEP for i in range(n)]


def fwd_call(**kw):
    q, k, v, o, lse = ptrs(5)
    args = dict(q=q, k=k, v=v, o=o, lse=lse, B=1, H_q=2, H_kv=1, N_q=16, N_kv=16, d=64, causal=0,
                scale=0.125, dtype=fa.FA_DTYPE_BF16, stream=None)
    args.update(kw)
    return fa.fa_fwd(**args)


def bwd_call(**kw):
    q, k, v, o, lse, do, dq, dk, dv, ws = ptrs(10)
    args = dict(q=q, k=k, v=v, o=o, lse=lse, dO=do, dq=dq, dk=dk, dv=dv, workspace=ws, workspace_bytes=1 << 20,
                B=1, H_q=2, H_kv=1, N_q=16, N_kv=16, d=64, causal=0, scale=0.125, dtype=fa.FA_DTYPE_BF16,
                stream=None)
    args.update(kw)
    return fa.fa_bwd(**args)


INVALID = fa.FA_ERR_INVALID_ARG
UNSUP = fa.FA_ERR_UNSUPPORTED


@pytest.mark.parametrize("call", [fwd_call, bwd_call])
@pytest.mark.parametrize("kw,expect", [
    (dict(B=-1), INVALID),
    (dict(N_q=-3), INVALID),
    (dict(d=-64), INVALID),
    (dict(dtype=7), UNSUP),
    (dict(d=96), UNSUP),
    (dict(d=256), UNSUP),
    (dict(H_kv=3, H_q=4), INVALID),
    (dict(H_kv=0), INVALID),
    (dict(N_kv=0), INVALID),
    (dict(N_q=(1 << 24) + 1), INVALID),
    (dict(scale=float("nan")), INVALID),
    (dict(scale=float("inf")), INVALID),
    (dict(scale=-0.5), UNSUP),
    (dict(q=0), INVALID),
    (dict(k=0), INVALID),
    (dict(lse=0), INVALID),
    (dict(v=A + 8), INVALID),            # not 16-byte aligned
    (dict(lse=A + 4), INVALID),          # misaligned and overlapping
])
def test_invalid_arguments(call, kw, expect):
    assert call(**kw) == expect


def test_empty_problem_is_a_noop():
    # Nothing is launched (and no HIP call is made) when there are no rows.
    assert fwd_call(B=0) == fa.FA_OK
    assert fwd_call(N_q=0) == fa.FA_OK
    assert fwd_call(H_q=0, H_kv=0) == fa.FA_OK
    assert fwd_call(N_q=0, q=0, k=0, v=0, o=0, lse=0) == fa.FA_OK
    # bwd without query rows and without key rows: nothing to write
    assert bwd_call(N_q=0, N_kv=0) == fa.FA_OK
    assert bwd_call(B=0) == fa.FA_OK
    assert bwd_call(H_q=0, H_kv=0) == fa.FA_OK


def test_bwd_without_queries_checks_dk_dv():
    # No query rows but keys present: dk and dv must be zero-filled, so they
    # are validated (before any HIP call); the other pointers are not used.
    assert bwd_call(N_q=0, dk=0) == INVALID
    assert bwd_call(H_q=0, dv=0) == INVALID
    assert bwd_call(N_q=0, dv=A + 8) == INVALID                # misaligned
    dk = ptrs(1, A + 64 * STEP)[0]
    assert bwd_call(N_q=0, dk=dk, dv=dk + 1024) == INVALID     # dk and dv overlap
    assert bwd_call(N_q=0, N_kv=(1 << 24) + 1) == INVALID


def test_output_aliasing_an_input_is_rejected():
    q, k, v, o, lse = ptrs(5)
    assert fwd_call(o=q) == INVALID                 # o == q
    assert fwd_call(o=k + 256) == INVALID           # o starts inside k
    assert fwd_call(lse=v + 512) == INVALID         # lse inside v
    assert fwd_call(lse=o + 16) == INVALID          # two outputs overlapping
    # bwd: gradients and workspace may not overlap inputs or each other
    base = ptrs(10)
    assert bwd_call(dq=base[0]) == INVALID
    assert bwd_call(dk=base[6]) == INVALID
    assert bwd_call(workspace=base[8]) == INVALID
    assert bwd_call(dv=base[5] + 32) == INVALID


def test_workspace_too_small_is_rejected():
    assert bwd_call(workspace_bytes=0) == INVALID
    need = fa.fa_bwd_workspace_size(1, 2, 16)
    assert bwd_call(workspace_bytes=need - 1) == INVALID


# ---------------------------------------------------------------------------
# split-KV forward
# ---------------------------------------------------------------------------

def split_call(**kw):
    q, k, v, o, lse, ws = ptrs(6)
    args = dict(q=q, k=k, v=v, o=o, lse=lse, B=1, H_q=8, H_kv=2, N_q=1, N_kv=1000, d=128, causal=0,
                scale=0.088, dtype=fa.FA_DTYPE_BF16, num_splits=4, workspace=ws, workspace_bytes=1 << 20,
                stream=None)
    args.update(kw)
    return fa.fa_fwd_splitkv(**args)


def test_splitkv_workspace_size():
    # B*H_q*N_q*S*(d+1) floats, rounded up to 256 bytes; 0 without splitting
    assert fa.fa_fwd_splitkv_workspace_size(2, 32, 1, 128, 8) == 2 * 32 * 1 * 8 * 129 * 4
    assert fa.fa_fwd_splitkv_workspace_size(1, 1, 1, 64, 2) == 768
    assert fa.fa_fwd_splitkv_workspace_size(1, 4, 3, 64, 1) == 0
    assert fa.fa_fwd_splitkv_workspace_size(0, 4, 3, 64, 4) == 0
    assert fa.fa_fwd_splitkv_workspace_size(1, 1, 5, 128, 3) % 256 == 0


@pytest.mark.parametrize("kw,expect", [
    (dict(B=-1), INVALID),
    (dict(dtype=7), UNSUP),
    (dict(d=96), UNSUP),
    (dict(H_kv=3, H_q=8), INVALID),
    (dict(N_kv=0), INVALID),
    (dict(scale=float("nan")), INVALID),
    (dict(scale=-1.0), UNSUP),
    (dict(q=0), INVALID),
    (dict(o=A), INVALID),                       # o aliases q
    (dict(num_splits=0), INVALID),
    (dict(num_splits=257), INVALID),
    (dict(dtype=fa.FA_DTYPE_F32), UNSUP),       # bf16 only
    (dict(H_q=64, H_kv=1, N_q=1), UNSUP),       # 64 rows per key/value head
    (dict(H_q=8, H_kv=1, N_q=5), UNSUP),        # 40 rows
    (dict(workspace=0), INVALID),
    (dict(workspace=A + 8), INVALID),           # misaligned
    (dict(workspace_bytes=10), INVALID),
    (dict(workspace=A + 2 * STEP), INVALID),    # workspace aliases v
])
def test_splitkv_invalid_arguments(kw, expect):
    assert split_call(**kw) == expect


def test_splitkv_empty_and_unsplit_workspace():
    assert split_call(N_q=0) == fa.FA_OK
    assert split_call(B=0, workspace=0, workspace_bytes=0) == fa.FA_OK


# ---------------------------------------------------------------------------
# packed variable-length forward
# ---------------------------------------------------------------------------

def varlen_call(**kw):
    q, k, v, o, lse, cq, ck = ptrs(7)
    args = dict(q=q, k=k, v=v, o=o, lse=lse, cu_seqlens_q=cq, cu_seqlens_k=ck, num_seqs=3, total_q=100,
                total_k=120, max_seqlen_q=60, H_q=4, H_kv=2, d=128, causal=1, scale=0.088,
                dtype=fa.FA_DTYPE_BF16, stream=None)
    args.update(kw)
    return fa.fa_fwd_varlen(**args)


@pytest.mark.parametrize("kw,expect", [
    (dict(num_seqs=-1), INVALID),
    (dict(total_q=-5), INVALID),
    (dict(dtype=fa.FA_DTYPE_F32), UNSUP),
    (dict(dtype=9), UNSUP),
    (dict(d=32), UNSUP),
    (dict(H_kv=3), INVALID),
    (dict(total_k=0), INVALID),
    (dict(max_seqlen_q=(1 << 24) + 1), INVALID),
    (dict(scale=float("inf")), INVALID),
    (dict(scale=-2.0), UNSUP),
    (dict(cu_seqlens_q=0), INVALID),
    (dict(cu_seqlens_k=A + 6 * STEP + 2), INVALID),     # not 4-byte aligned
    (dict(o=A + 5 * STEP), INVALID),                    # o overlaps the query offsets
    (dict(lse=A + 2 * STEP + 64), INVALID),             # lse inside v
])
def test_varlen_invalid_arguments(kw, expect):
    assert varlen_call(**kw) == expect


def test_varlen_empty_is_a_noop():
    assert varlen_call(num_seqs=0) == fa.FA_OK
    assert varlen_call(total_q=0, q=0, o=0, lse=0) == fa.FA_OK
    assert varlen_call(max_seqlen_q=0) == fa.FA_OK


# ---------------------------------------------------------------------------
# self-check
# ---------------------------------------------------------------------------

def check_call(**kw):
    q, k, lse, rows, res = ptrs(5)
    args = dict(q=q, k=k, lse=lse, rows=rows, n_rows=4, B=1, H_q=2, H_kv=1, N_q=16, N_kv=16, d=64, causal=0,
                scale=0.125, dtype=fa.FA_DTYPE_BF16, result=res, stream=None)
    args.update(kw)
    return fa.fa_fwd_check(**args)


@pytest.mark.parametrize("kw,expect", [
    (dict(B=-1), INVALID),
    (dict(dtype=5), UNSUP),
    (dict(d=48), UNSUP),
    (dict(n_rows=-1), INVALID),
    (dict(rows=0), INVALID),
    (dict(rows=A + 3 * STEP + 2), INVALID),   # not 4-byte aligned
    (dict(result=A + 4 * STEP + 4), INVALID),  # not 16-byte aligned
    (dict(result=A + 8), INVALID),             # result inside q (and misaligned)
    (dict(result=A + STEP), INVALID),          # result == k
    (dict(scale=float("nan")), INVALID),
])
def test_check_invalid_arguments(kw, expect):
    assert check_call(**kw) == expect


def test_check_noop():
    assert check_call(n_rows=0) == fa.FA_OK
    assert check_call(N_q=0) == fa.FA_OK


# ---------------------------------------------------------------------------
# FP8: block quantizer and forward
# ---------------------------------------------------------------------------

def quant_call(**kw):
    x, c, sc = ptrs(3)
    args = dict(x=x, codes=c, descale=sc, B=2, H=4, N=300, d=128, d_major=0, dtype=fa.FA_DTYPE_BF16, stream=None)
    args.update(kw)
    return fa.fa_quantize_fp8(**args)


@pytest.mark.parametrize("kw,expect", [
    (dict(B=-1), INVALID),
    (dict(N=-3), INVALID),
    (dict(dtype=fa.FA_DTYPE_F32), UNSUP),
    (dict(d=96), UNSUP),
    (dict(N=(1 << 24) + 1), INVALID),
    (dict(x=0), INVALID),
    (dict(codes=A + STEP + 8), INVALID),        # misaligned
    (dict(codes=A + 64), INVALID),              # codes inside x
    (dict(descale=A + STEP + 1024), INVALID),   # descale inside the codes
])
def test_quantize_fp8_invalid_arguments(kw, expect):
    assert quant_call(**kw) == expect


def test_quantize_fp8_empty_is_a_noop():
    assert quant_call(N=0) == fa.FA_OK
    assert quant_call(B=0, x=0) == fa.FA_OK


def fp8_call(**kw):
    q, qs, k, ks, v, vs, o, lse = ptrs(8)
    args = dict(q8=q, q_descale=qs, k8=k, k_descale=ks, v8=v, v_descale=vs, o=o, lse=lse, B=1, H_q=8, H_kv=2,
                N_q=500, N_kv=700, d=128, causal=1, scale=0.088, stream=None)
    args.update(kw)
    return fa.fa_fwd_fp8(**args)


@pytest.mark.parametrize("kw,expect", [
    (dict(B=-1), INVALID),
    (dict(d=80), UNSUP),
    (dict(H_kv=3), INVALID),
    (dict(N_kv=0), INVALID),
    (dict(N_q=(1 << 24) + 1), INVALID),
    (dict(scale=float("nan")), INVALID),
    (dict(scale=-1.0), UNSUP),
    (dict(q8=0), INVALID),
    (dict(v_descale=0), INVALID),
    (dict(k_descale=A + 3 * STEP + 2), INVALID),   # not 4-byte aligned
    (dict(v8=A + 4 * STEP + 8), INVALID),          # not 16-byte aligned
    (dict(o=A + 2 * STEP + 256), INVALID),         # o inside k8
    (dict(lse=A + 6 * STEP + 512), INVALID),       # lse inside o
])
def test_fwd_fp8_invalid_arguments(kw, expect):
    assert fp8_call(**kw) == expect


def test_fwd_fp8_empty_is_a_noop():
    assert fp8_call(N_q=0) == fa.FA_OK
    assert fp8_call(B=0) == fa.FA_OK


def split8_call(**kw):
    q, k, ks, v, vs, o, lse, ws = ptrs(8)
    args = dict(q=q, k8=k, k_descale=ks, v8=v, v_descale=vs, o=o, lse=lse, B=2, H_q=8, H_kv=2, N_q=1, N_kv=5000,
                d=128, causal=0, scale=0.088, num_splits=4, workspace=ws, workspace_bytes=1 << 20, stream=None)
    args.update(kw)
    return fa.fa_fwd_splitkv_fp8(**args)


@pytest.mark.parametrize("kw,expect", [
    (dict(B=-1), INVALID),
    (dict(d=96), UNSUP),
    (dict(H_kv=3), INVALID),
    (dict(N_kv=0), INVALID),
    (dict(num_splits=0), INVALID),
    (dict(num_splits=257), INVALID),
    (dict(N_q=9), UNSUP),                          # 4 heads x 9 queries > 32 rows
    (dict(k8=0), INVALID),
    (dict(v_descale=A + 4 * STEP + 2), INVALID),   # not 4-byte aligned
    (dict(workspace=0), INVALID),
    (dict(workspace_bytes=16), INVALID),
    (dict(o=A + 3 * STEP + 64), INVALID),          # o inside v8
    (dict(scale=float("inf")), INVALID),
])
def test_splitkv_fp8_invalid_arguments(kw, expect):
    assert split8_call(**kw) == expect


def test_splitkv_fp8_empty_is_a_noop():
    assert split8_call(N_q=0) == fa.FA_OK
    assert split8_call(B=0) == fa.FA_OK


def noalloc_call(**kw):
    q, k, v, o, lse = ptrs(5)
    args = dict(q=q, k=k, v=v, o=o, lse=lse, B=2, H_q=8, H_kv=2, N_q=1, N_kv=4096, d=128, causal=0,
                scale=0.088, dtype=fa.FA_DTYPE_BF16, num_splits=8, stream=None)
    args.update(kw)
    return fa.fa_fwd_splitkv_noalloc(**args)


def test_splitkv_noalloc_checks():
    # the limit of the static partials array is enforced before any HIP call
    assert fa.NOALLOC_SCRATCH_BYTES == 16 << 20
    big = dict(B=64, H_q=32, H_kv=8, N_q=1, N_kv=4096, num_splits=256)
    assert fa.fa_fwd_splitkv_workspace_size(64, 32, 1, 128, 256) > fa.NOALLOC_SCRATCH_BYTES
    assert noalloc_call(**big) == INVALID
    # the checks shared with fa_fwd_splitkv
    assert noalloc_call(num_splits=0) == INVALID
    assert noalloc_call(num_splits=257) == INVALID
    assert noalloc_call(dtype=fa.FA_DTYPE_F32) == UNSUP
    assert noalloc_call(N_q=5, H_q=8, H_kv=1) == UNSUP          # 40 rows per key/value head
    assert noalloc_call(q=0) == INVALID
    assert noalloc_call(o=ptrs(1)[0]) == INVALID               # o aliases q
    assert noalloc_call(N_q=0) == fa.FA_OK                     # empty: nothing launched

"""Shared helpers for the GPU parity tests (imported by test modules only)."""

from __future__ import annotations

import math
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import exact_attention_109_amd as fa  # noqa: E402
from workloads import DTYPE_BF16, DTYPE_F32, Inputs, bf16_bits_to_f64  # noqa: E402

# Tolerances (max-abs against the fp64 oracle on the same rounded inputs).
TOL = {
    DTYPE_F32: {"o": 1e-5, "lse": 1e-5, "grad": 1e-5},
    DTYPE_BF16: {"o": 1e-2, "lse": 1e-3, "grad": 1e-2},
}


def ensure_library():
    if not os.path.exists(fa.LIB_PATH):
        from exact_attention_109_amd import _build
        _build.build()
    fa.load_library()


def to_f64(t) -> np.ndarray:
    """Copy a torch tensor (bf16 or fp32, any device) to a float64 numpy array."""
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f64(t.view(torch.int16).numpy().view(np.uint16))
    return t.double().numpy()


def upload(inp: Inputs, names=("q", "k", "v")):
    return [inp.torch(n, "cuda") for n in names]


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half a bf16 unit in the last place at |x| (0 for x == 0)."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, 2.0 ** (e - 8), 0.0)


def o_within(got, ref, dtype) -> bool:
    """Output check. fp32: max-abs <= 1e-5. bf16: per element
    |got - ref| <= 1e-2 + half a bf16 ulp of ref -- the output is stored in
    bf16, and rounding even the exact value to bf16 errs by up to half an ulp
    (0.0156 once |O| >= 4), so the 1e-2 budget applies to the computation on
    top of the output format's own rounding."""
    got = np.asarray(got)
    ref = np.asarray(ref)
    if dtype == DTYPE_F32:
        return max_abs(got, ref) <= TOL[DTYPE_F32]["o"]
    return bool(np.all(np.abs(got - ref) <= TOL[DTYPE_BF16]["o"] + bf16_half_ulp(ref)))


def sample_rows(n: int, rng: np.random.Generator, count: int = 96, tile: int = 128):
    rows = set(range(min(n, 16)))
    rows |= set(range(max(0, n - 16), n))
    for t in range(tile, n, tile * max(1, n // (tile * 8))):
        rows |= {t - 1, t, min(n - 1, t + 1)}
    rows |= set(rng.integers(0, n, size=count).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < n), dtype=np.int64)


def max_abs(a, b) -> float:
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.asarray(a).size else 0.0


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)

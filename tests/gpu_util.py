"""Shared helpers for the GPU parity tests (imported by test modules only)."""

from __future__ import annotations

import concurrent.futures as cf
import math
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import exact_attention_109_amd as fa  # noqa: E402
import oracle  # noqa: E402
from workloads import DTYPE_BF16, DTYPE_F32, Inputs, bf16_bits_to_f64  # noqa: E402

# Tolerances (max-abs against the fp64 oracle on the same rounded inputs).
TOL = {
    DTYPE_F32: {"o": 1e-5, "lse": 1e-5, "grad": 1e-5},
    DTYPE_BF16: {"o": 1e-2, "lse": 1e-3, "grad": 1e-2},
}


def ensure_library():
    if not os.path.exists(fa.library_path()):
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


def max_abs(a, b) -> float:
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.asarray(a).size else 0.0


def o_plain_ok(got, ref, dtype) -> bool:
    """The stated output bound: max-abs <= 1e-2 (bf16) or 1e-5 (fp32)."""
    return max_abs(got, ref) <= TOL[dtype]["o"]


def o_extreme_check(got, ref, q, k, v, causal, scale, G):
    """Output bound of the extreme-logit configuration (|s| in the hundreds,
    Q and K x 8), per element:
        |got - ref| <= half a bf16 ulp of ref + max(1e-2, 2^-8 sum_j w_j |v_j|)
    with w the exact probabilities of the row. The rows are nearly one-hot,
    so O is close to single value rows: it reaches |O| >= 4, where rounding
    even the exact value to bf16 errs by up to 2^-6 = 0.0156, and the bf16
    rounding of the probabilities before the P V product (relative error up
    to 2^-8 each) no longer averages out over many keys. The second term is
    formed only for the rows where 1e-2 + half an ulp is exceeded. Returns
    the number of elements past 1e-2 + half an ulp."""
    got = np.asarray(got)
    ref = np.asarray(ref)
    err = np.abs(got - ref)
    bad = np.argwhere(err > TOL[DTYPE_BF16]["o"] + bf16_half_ulp(ref))
    for (b, h, i) in sorted({(int(b), int(h), int(i)) for b, h, i, _ in bad}):
        w = oracle.head_probabilities(q[b, h], k[b, h // G], causal, scale, np.array([i]))[0]
        wv = w @ np.abs(v[b, h // G])
        bound = bf16_half_ulp(ref[b, h, i]) + np.maximum(TOL[DTYPE_BF16]["o"], 2.0 ** -8 * wv + 1e-5)
        assert np.all(err[b, h, i] <= bound), (b, h, i, float(np.max(err[b, h, i] - bound)))
    return len(bad)


def o_small_check(got, ref, dtype):
    """Output check of the tiny-shape grid. fp32: max-abs <= 1e-5. bf16:
    max-abs <= 1e-2 on every element whose exact value has |O| < 2. Rows of
    one to a few keys can hold |O| in [2, 4), where the output's own bf16
    rounding costs up to 2^-8 = 0.0078 and the bf16 probabilities of the P V
    product (unit roundoff 2^-8 each, not averaged out over so few keys) add
    to it; those elements are held to 1e-2 + half a bf16 ulp of the exact
    value. Returns the number of elements that needed that
    allowance (0 when the plain bound holds everywhere)."""
    got = np.asarray(got)
    ref = np.asarray(ref)
    if dtype == DTYPE_F32:
        assert max_abs(got, ref) <= TOL[DTYPE_F32]["o"]
        return 0
    err = np.abs(got - ref)
    plain = err <= TOL[DTYPE_BF16]["o"]
    big = np.abs(ref) >= 2.0
    assert np.all(plain | big), float(err[~big].max())
    assert np.all(err <= TOL[DTYPE_BF16]["o"] + bf16_half_ulp(ref)), float(err.max())
    return int(np.count_nonzero(~plain))


def sample_rows(n: int, rng: np.random.Generator, count: int = 96, tile: int = 128):
    rows = set(range(min(n, 16)))
    rows |= set(range(max(0, n - 16), n))
    for t in range(tile, n, tile * max(1, n // (tile * 8))):
        rows |= {t - 1, t, min(n - 1, t + 1)}
    rows |= set(rng.integers(0, n, size=count).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < n), dtype=np.int64)


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def host_workers() -> int:
    """Threads for running the oracle over independent heads: the host cores
    this process may use (at most 16)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def map_heads(fn, items):
    """Run fn over independent heads in a thread pool with the BLAS library
    held to one thread per call (numpy releases the GIL in its matrix
    products and element-wise kernels). Returns the results in order. This
    only distributes calls of the oracle; it changes none of its arithmetic."""
    items = list(items)
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=1)
    except ImportError:  # pragma: no cover - threadpoolctl is installed here
        limiter = None
    try:
        with cf.ThreadPoolExecutor(max_workers=host_workers()) as ex:
            return list(ex.map(fn, items))
    finally:
        if limiter is not None:
            limiter.restore_original_limits()


def oracle_forward_all(q, k, v, causal, scale, G):
    """The oracle's O and LSE for every (batch, head), heads run in parallel."""
    B, H_q = q.shape[0], q.shape[1]
    heads = [(b, h) for b in range(B) for h in range(H_q)]
    res = map_heads(lambda bh: oracle.head_forward(q[bh[0], bh[1]], k[bh[0], bh[1] // G], v[bh[0], bh[1] // G],
                                                   causal, scale), heads)
    O = np.empty(q.shape[:3] + (v.shape[3],), dtype=np.float64)
    L = np.empty(q.shape[:3], dtype=np.float64)
    for (b, h), (o, l) in zip(heads, res):
        O[b, h], L[b, h] = o, l
    return O, L

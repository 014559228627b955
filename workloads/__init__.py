"""Seeded synthetic inputs for the attention workloads.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark. It holds no attention arithmetic: it only draws i.i.d. Gaussian
tensors from a seed and, for the bf16 workloads, rounds them to bf16 bits so
that both sides of a comparison read exactly the same values.

Workload shapes follow the five attention configurations this library is
measured on (fp32 tiny check, bf16 MHA, long causal MHA, causal GQA at 16K
context with an extreme-logit variant, and the causal backward).

Layout everywhere is contiguous row-major ``[B, H, N, d]``; K and V use the
key/value head count.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

DTYPE_F32 = 0
DTYPE_BF16 = 1


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: int          # DTYPE_F32 or DTYPE_BF16
    B: int
    H_q: int
    H_kv: int
    N_q: int
    N_kv: int
    d: int
    causal: bool
    seed: int
    qk_multiplier: float = 1.0   # power of two; scales Q and K exactly
    with_grad: bool = False      # also draw dO

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def fwd_flop(self) -> float:
        """Metric FLOP count: 4*B*H_q*N_q*N_kv*d, halved when causal."""
        f = 4.0 * self.B * self.H_q * self.N_q * self.N_kv * self.d
        return f / 2.0 if self.causal else f

    @property
    def bwd_flop(self) -> float:
        """Backward FLOP convention: 2.5x the forward count."""
        return 2.5 * self.fwd_flop


WORKLOADS = {
    "c1": Workload("c1_fp32_tiny", DTYPE_F32, 1, 1, 1, 256, 256, 64, False, 1),
    "c2": Workload("c2_bf16_mha_n2048_d64", DTYPE_BF16, 4, 16, 16, 2048, 2048, 64, False, 2),
    "c3": Workload("c3_bf16_causal_mha_n8192_d128", DTYPE_BF16, 2, 32, 32, 8192, 8192, 128, True, 3),
    "c4": Workload("c4_bf16_causal_gqa_n16384_d128", DTYPE_BF16, 1, 32, 8, 16384, 16384, 128, True, 4),
    "c4x": Workload("c4x_bf16_causal_gqa_n16384_d128_qk_x8", DTYPE_BF16, 1, 32, 8, 16384, 16384, 128, True, 4,
                    qk_multiplier=8.0),
    "c5": Workload("c5_bf16_causal_bwd_n4096_d128", DTYPE_BF16, 2, 16, 16, 4096, 4096, 128, True, 5,
                   with_grad=True),
}


# Decode-like shapes for the split-KV forward: one new query row per
# sequence against a long key/value cache, GQA with 4 query heads per
# key/value head (not one of the five configurations above).
DECODE_WORKLOADS = {
    "d1": Workload("d1_bf16_decode_gqa_kv32768_d128", DTYPE_BF16, 8, 32, 8, 1, 32768, 128, False, 6),
}


# ---------------------------------------------------------------------------
# bf16 bit handling (exact; round-to-nearest-even)
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 with round-to-nearest-even.

    Returns the 16-bit patterns as uint16. NaN stays NaN (quiet)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    nan = np.isnan(x)
    if nan.any():
        rounded = np.where(nan, (u >> np.uint32(16)) | np.uint32(0x40), rounded)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(b).astype(np.float64)


# ---------------------------------------------------------------------------
# Generation
# ---------------------------------------------------------------------------

def _draw(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32)


def make_raw(B, H_q, H_kv, N_q, N_kv, d, seed, with_grad=False):
    """fp32 N(0,1) draws in the fixed order Q, K, V, (dO) from PCG64(seed)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _draw(rng, (B, H_q, N_q, d))
    k = _draw(rng, (B, H_kv, N_kv, d))
    v = _draw(rng, (B, H_kv, N_kv, d))
    do = _draw(rng, (B, H_q, N_q, d)) if with_grad else None
    return q, k, v, do


class Inputs:
    """One workload's inputs in host memory.

    For bf16 workloads ``bits`` holds the uint16 patterns and ``f64`` the
    exactly widened values; for fp32 both views come from the same float32
    arrays. ``names`` is ('q', 'k', 'v') or ('q', 'k', 'v', 'do')."""

    def __init__(self, dtype: int, arrays: dict):
        self.dtype = dtype
        self._arrays = arrays  # name -> float32 array (fp32) or uint16 bits (bf16)

    @property
    def names(self):
        return tuple(self._arrays)

    def raw(self, name: str) -> np.ndarray:
        return self._arrays[name]

    def f64(self, name: str) -> np.ndarray:
        a = self._arrays[name]
        if self.dtype == DTYPE_BF16:
            return bf16_bits_to_f64(a)
        return a.astype(np.float64)

    def torch(self, name: str, device="cpu"):
        import torch
        a = self._arrays[name]
        if self.dtype == DTYPE_BF16:
            t = torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16)
        else:
            t = torch.from_numpy(a.copy())
        return t.to(device)


def make_inputs_shape(dtype, B, H_q, H_kv, N_q, N_kv, d, seed, with_grad=False,
                      qk_multiplier=1.0) -> Inputs:
    q, k, v, do = make_raw(B, H_q, H_kv, N_q, N_kv, d, seed, with_grad)
    arrays = {"q": q, "k": k, "v": v}
    if do is not None:
        arrays["do"] = do
    if dtype == DTYPE_BF16:
        arrays = {n: f32_to_bf16_bits(a) for n, a in arrays.items()}
        if qk_multiplier != 1.0:
            # multiply by a power of two in the bf16 domain: exact
            for n in ("q", "k"):
                arrays[n] = f32_to_bf16_bits(bf16_bits_to_f32(arrays[n]) * np.float32(qk_multiplier))
    else:
        if qk_multiplier != 1.0:
            arrays["q"] = arrays["q"] * np.float32(qk_multiplier)
            arrays["k"] = arrays["k"] * np.float32(qk_multiplier)
    return Inputs(dtype, arrays)


def make_inputs(w: Workload) -> Inputs:
    return make_inputs_shape(w.dtype, w.B, w.H_q, w.H_kv, w.N_q, w.N_kv, w.d, w.seed,
                             with_grad=w.with_grad, qk_multiplier=w.qk_multiplier)


# ---------------------------------------------------------------------------
# Packed variable-length sequences
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class VarlenWorkload:
    """A batch of sequences of different lengths, packed head-major without
    padding: q [H_q, total_q, d], k and v [H_kv, total_k, d]. Query and key
    lengths are equal per sequence (self-attention), drawn uniformly from
    [min_len, max_len] by the seed."""
    name: str
    num_seqs: int
    min_len: int
    max_len: int
    H_q: int
    H_kv: int
    d: int
    causal: bool
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def lengths(self) -> np.ndarray:
        rng = np.random.Generator(np.random.PCG64(self.seed + 1000))
        return rng.integers(self.min_len, self.max_len + 1, size=self.num_seqs).astype(np.int64)

    def fwd_flop(self) -> float:
        """4*H_q*n^2*d per sequence of length n, halved when causal."""
        f = sum(4.0 * self.H_q * float(n) * float(n) * self.d for n in self.lengths())
        return f / 2.0 if self.causal else f


VARLEN_WORKLOADS = {
    "v1": VarlenWorkload("v1_bf16_causal_varlen_16seq_512to8192_d128", 16, 512, 8192, 32, 8, 128, True, 7),
}


def cu_seqlens(lengths) -> np.ndarray:
    """Prefix offsets [0, l0, l0+l1, ...] as int32."""
    out = np.zeros(len(lengths) + 1, dtype=np.int64)
    out[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return out.astype(np.int32)


def make_packed_inputs(dtype, H_q, H_kv, total_q, total_k, d, seed) -> Inputs:
    """q [H_q, total_q, d], k and v [H_kv, total_k, d]: i.i.d. N(0,1) drawn in
    that order from PCG64(seed), rounded to bf16 for DTYPE_BF16."""
    rng = np.random.Generator(np.random.PCG64(seed))
    arrays = {"q": _draw(rng, (H_q, total_q, d)), "k": _draw(rng, (H_kv, total_k, d)),
              "v": _draw(rng, (H_kv, total_k, d))}
    if dtype == DTYPE_BF16:
        arrays = {n: f32_to_bf16_bits(a) for n, a in arrays.items()}
    return Inputs(dtype, arrays)


# ---------------------------------------------------------------------------
# FP8 inputs: bf16 sources with a spread of magnitudes between row blocks
# ---------------------------------------------------------------------------

def block_spread_bits(bits: np.ndarray, seed: int, lo: int, hi: int, block: int = 128) -> np.ndarray:
    """Multiply every block of ``block`` rows (axis 2) of a bf16 tensor by its
    own power of two 2^k, k drawn uniformly from [lo, hi] by the seed (exact
    in bf16 while the values stay in range). Returns new bf16 bits."""
    B, H, N, d = bits.shape
    nb = (N + block - 1) // block
    k = np.random.Generator(np.random.PCG64(seed)).integers(lo, hi + 1, size=(B, H, nb))
    f = np.repeat(np.exp2(k).astype(np.float32), block, axis=2)[:, :, :N, None]
    return f32_to_bf16_bits(bf16_bits_to_f32(bits) * f)

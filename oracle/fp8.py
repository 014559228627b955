"""FP8 (e4m3) inputs for the attention forward: code format, block quantizer,
dequantization and the forward on dequantized inputs, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:
  * "Flash-Attention" (Awesome System Papers Wiki), 关键观察 (key
    observations) and 设计空间与取舍 (design space): FlashAttention-3 adds
    an FP8 path that is faster but has to deal with quantization and
    outliers, and a low-precision path must have its scales and error
    checked for the task at hand.
  * "深度学习进阶（三十一）FlashAttention：IO 感知的精确注意力" (rkmt.cn
    blog), the FA1/FA2/FA3 comparison table, and "FlashAttention" (LLM
    Inference Handbook), the version comparison table: FP8 support is one of
    FlashAttention-3's additions. The pages fix no format, scale granularity
    or rounding; the readings below are ours.

Readings (the pages are silent on all of them):
  * the 8-bit format is OCP e4m3 ("fn": sign, 4 exponent bits with bias 7,
    3 mantissa bits, no infinities, S.1111.111 is NaN, largest finite 448,
    subnormals k * 2^-9);
  * one scale per block of 128 consecutive rows of one (batch, head) for each
    of Q, K and V (the row block covers all d columns);
  * the block quantizer works in float32: amax = max |x| over the block,
    descale = amax / 448, inv = 448 / amax (both correctly rounded float32
    divisions), code = e4m3 round-to-nearest-even of the float32 product
    x * inv, saturated to +-448. When inv is not finite (amax = 0 or below
    448 / FLT_MAX) every code of the block is 0. Dequantized value =
    e4m3 value * descale;
  * the FP8 attention paths read Q, K and V row-major ([B][H][N][d], as the
    bf16 ones); a d-major copy ([B][H][d][N_pad], N_pad = N rounded up to
    128, zero codes in the padding) is an optional quantizer output;
  * the FP8 forward computes attention on the dequantized Q, K, V; its exact
    value is the float64 forward of those values (``fp8_attention_forward``).
"""

from __future__ import annotations

import numpy as np

from .attention import attention_forward

E4M3_MAX = 448.0
E4M3_BIAS = 7
QUANT_BLOCK = 128      # rows per scale block
V_PAD = 128            # key padding of the d-major V layout


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Value of each e4m3 code (uint8) as float64; NaN for S.1111.111."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = m * 2.0 ** (1 - E4M3_BIAS - 3)                 # e == 0: m * 2^-9
    nrm = (1.0 + m / 8.0) * np.exp2(e - E4M3_BIAS)
    val = np.where(e == 0, sub, nrm)
    val = np.where((e == 0xF) & (m == 0x7), np.nan, val)
    return sign * val


def _positive_table():
    """The 127 finite non-negative e4m3 values in increasing order and their codes."""
    codes = np.arange(0, 0x7F, dtype=np.uint8)          # 0x00 .. 0x7E
    return e4m3_decode(codes), codes


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even of each value to e4m3, saturated to +-448.

    The rounding quantum is 2^(e-3) for |y| in [2^e, 2^(e+1)), e >= -6,
    and 2^-9 below 2^-6 (subnormals); ties go to the even mantissa. The
    sign bit is kept for values that round to zero; NaN gives 0x7F."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    safe = np.where(np.isfinite(a) & (a > 0), a, 1.0)
    e = np.floor(np.log2(safe))
    # floor(log2) can be off by one next to a power of two; fix it exactly
    e = np.where(np.exp2(e) > safe, e - 1, e)
    e = np.where(np.exp2(e + 1) <= safe, e + 1, e)
    quantum = np.where(a < 2.0 ** -6, 2.0 ** -9, np.exp2(e - 3))
    r = np.round(a / quantum) * quantum                  # numpy rounds half to even
    r = np.minimum(r, E4M3_MAX)
    r = np.where(np.isnan(y), 0.0, r)                    # NaN is coded separately below
    vals, codes = _positive_table()
    idx = np.searchsorted(vals, r)                       # r is exactly one of vals
    idx = np.minimum(idx, vals.size - 1)
    assert np.all(vals[idx] == r), "rounded value is not an e4m3 value"
    mag = codes[idx]
    out = np.where(np.signbit(y), mag | 0x80, mag).astype(np.uint8)
    return np.where(np.isnan(y), np.uint8(0x7F), out).astype(np.uint8)


def quantize_blocks(x: np.ndarray, block: int = QUANT_BLOCK):
    """Block-quantize x [B, H, N, d] (float32 values) along N.

    Returns codes [B, H, N, d] (uint8) and descale [B, H, ceil(N/block)]
    (float32), following the float32 recipe in the module docstring."""
    x = np.asarray(x, dtype=np.float32)
    B, H, N, d = x.shape
    nb = (N + block - 1) // block
    codes = np.zeros((B, H, N, d), dtype=np.uint8)
    descale = np.zeros((B, H, nb), dtype=np.float32)
    f448 = np.float32(E4M3_MAX)
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        for b in range(B):
            for h in range(H):
                for i in range(nb):
                    blk = x[b, h, i * block:(i + 1) * block]
                    amax = np.float32(np.max(np.abs(blk))) if blk.size else np.float32(0)
                    descale[b, h, i] = np.float32(amax / f448)
                    inv = np.float32(f448 / amax)
                    if not np.isfinite(inv):
                        continue                          # codes stay 0
                    y = (blk * inv).astype(np.float32)    # float32 product, round to nearest
                    codes[b, h, i * block:(i + 1) * block] = e4m3_encode(y)
    return codes, descale


def to_d_major(codes: np.ndarray, pad: int = V_PAD) -> np.ndarray:
    """[B, H, N, d] codes -> [B, H, d, N_pad] with zero codes past N."""
    B, H, N, d = codes.shape
    n_pad = ((N + pad - 1) // pad) * pad
    out = np.zeros((B, H, d, n_pad), dtype=np.uint8)
    out[:, :, :, :N] = np.swapaxes(codes, 2, 3)
    return out


def dequantize(codes: np.ndarray, descale: np.ndarray, block: int = QUANT_BLOCK) -> np.ndarray:
    """codes [B, H, N, d] and descale [B, H, nb] -> float64 values."""
    B, H, N, d = codes.shape
    per_row = np.repeat(np.asarray(descale, dtype=np.float64), block, axis=2)[:, :, :N]
    return e4m3_decode(codes) * per_row[..., None]


def fp8_attention_forward(q8, q_descale, k8, k_descale, v8, v_descale, causal, scale, rows=None):
    """Exact attention (float64) on the dequantized row-major codes."""
    q = dequantize(q8, q_descale)
    k = dequantize(k8, k_descale)
    v = dequantize(v8, v_descale)
    return attention_forward(q, k, v, causal, scale, rows)

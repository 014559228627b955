"""CPU pins of the FP8 part of the oracle (oracle/fp8.py).

The e4m3 code table is pinned to the format's definition (OCP 8-bit float,
E4M3: bias 7, 3 mantissa bits, S.1111.111 is NaN, largest finite 448) and
to torch's float8_e4m3fn conversions (an independent library routine);
rounding is pinned by exhaustive midpoints; the block quantizer by closed
forms (the block's largest element maps to 448, power-of-two scaling,
independence of blocks, the rounding bound); the FP8 forward by inputs the
quantizer reproduces exactly, where it must equal the float64 forward.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from oracle import fp8 as of8

FINITE = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def test_decode_known_codes():
    cases = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x3F: 1.875,
             0x40: 2.0, 0x7E: 448.0, 0xC0: -2.0, 0xFE: -448.0, 0xB8: -1.0}
    for c, v in cases.items():
        assert of8.e4m3_decode(np.array([c], np.uint8))[0] == v, hex(c)
    assert np.isnan(of8.e4m3_decode(np.array([0x7F, 0xFF], np.uint8))).all()
    neg0 = of8.e4m3_decode(np.array([0x80], np.uint8))[0]
    assert neg0 == 0.0 and np.signbit(neg0)


def test_positive_table_is_increasing_and_complete():
    v = of8.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    assert v.size == 127 and np.all(np.diff(v) > 0) and v[-1] == 448.0
    # spacing: 2^-9 below 2^-6, then 2^(e-3) in [2^e, 2^(e+1))
    for a, b in zip(v[:-1], v[1:]):
        e = np.floor(np.log2(b)) if b > 0 else -9
        step = 2.0 ** -9 if a < 2.0 ** -6 else 2.0 ** (np.floor(np.log2(a)) - 3)
        assert b - a == step


def test_decode_matches_torch_float8():
    torch = pytest.importorskip("torch")
    t = torch.from_numpy(np.arange(256, dtype=np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = of8.e4m3_decode(np.arange(256, dtype=np.uint8))
    fin = np.isfinite(ours)
    assert np.array_equal(np.isnan(t), ~fin)
    assert np.array_equal(t[fin], ours[fin])


def test_encode_matches_torch_float8_in_range():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(200000) * 40, rng.uniform(-2.0 ** -5, 2.0 ** -5, 50000),
                        rng.standard_normal(20000) * 1e-3]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    t = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(of8.e4m3_encode(x), t)


def test_round_trip_every_finite_code():
    assert np.array_equal(of8.e4m3_encode(of8.e4m3_decode(FINITE)), FINITE)


def test_midpoints_round_to_even_and_neighbours_to_nearest():
    vals = of8.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    for c in range(0x7E):
        lo, hi = vals[c], vals[c + 1]
        mid = (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        assert of8.e4m3_encode(np.array([mid]))[0] == even
        assert of8.e4m3_encode(np.array([-mid]))[0] == even | 0x80
        eps = (hi - lo) * 1e-6
        assert of8.e4m3_encode(np.array([mid - eps]))[0] == c
        assert of8.e4m3_encode(np.array([mid + eps]))[0] == c + 1


def test_saturation_and_specials():
    enc = lambda *v: list(of8.e4m3_encode(np.array(v, dtype=np.float64)))
    assert enc(448.0, 463.9, 464.0, 1e9) == [0x7E] * 4
    assert enc(-448.0, -1e30) == [0xFE, 0xFE]
    assert enc(0.0, -0.0, 2.0 ** -10, -(2.0 ** -11)) == [0x00, 0x80, 0x00, 0x80]
    assert enc(3 * 2.0 ** -10) == [0x02]     # tie between 1 and 2 subnormal steps -> 2
    assert enc(float("nan")) == [0x7F]


# ---------------------------------------------------------------------------
# block quantizer
# ---------------------------------------------------------------------------

def _gauss(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


def test_block_max_maps_to_448_and_descale_is_amax_over_448():
    x = _gauss((1, 2, 300, 64), 1)
    codes, ds = of8.quantize_blocks(x)
    assert ds.shape == (1, 2, 3)
    for h in range(2):
        for i in range(3):
            blk = x[0, h, 128 * i:128 * (i + 1)]
            amax = np.float32(np.abs(blk).max())
            assert ds[0, h, i] == np.float32(amax / np.float32(448))
            at = np.unravel_index(np.argmax(np.abs(blk)), blk.shape)
            assert codes[0, h, 128 * i + at[0], at[1]] & 0x7F == 0x7E


def test_quantization_error_bound():
    x = _gauss((2, 1, 256, 128), 2, 3.0)
    x[0, 0, :128] *= 1e-3             # one block with much smaller values
    codes, ds = of8.quantize_blocks(x)
    deq = of8.dequantize(codes, ds)
    per_row = np.repeat(ds.astype(np.float64), 128, axis=2)[..., None]
    bound = (2.0 ** -4 * np.abs(x) + 2.0 ** -10 * per_row) * (1 + 1e-6) + 1e-6 * np.abs(x)
    assert np.all(np.abs(deq - x) <= bound)
    # and the rounding is to nearest: no code is off by a whole step
    assert np.mean(np.abs(deq - x) <= 0.5 * 2.0 ** -3 * np.abs(x) + 2.0 ** -10 * per_row) == 1.0


def test_power_of_two_scaling_commutes():
    x = _gauss((1, 1, 200, 64), 4)
    c1, d1 = of8.quantize_blocks(x)
    c2, d2 = of8.quantize_blocks(x * np.float32(2.0 ** 7))
    assert np.array_equal(c1, c2) and np.array_equal(d2, d1 * np.float32(2.0 ** 7))


def test_blocks_are_independent():
    x = _gauss((1, 1, 384, 64), 5)
    c1, d1 = of8.quantize_blocks(x)
    y = x.copy()
    y[0, 0, 128:256] *= 37.0          # only the middle block changes
    c2, d2 = of8.quantize_blocks(y)
    assert np.array_equal(c1[0, 0, :128], c2[0, 0, :128]) and np.array_equal(c1[0, 0, 256:], c2[0, 0, 256:])
    assert d1[0, 0, 0] == d2[0, 0, 0] and d1[0, 0, 2] == d2[0, 0, 2] and d1[0, 0, 1] != d2[0, 0, 1]


def test_zero_and_single_element_blocks():
    x = np.zeros((1, 1, 130, 64), np.float32)
    x[0, 0, 129, 5] = -3.0            # the second block holds one nonzero element
    codes, ds = of8.quantize_blocks(x)
    assert np.all(codes[0, 0, :128] == 0) and ds[0, 0, 0] == 0
    assert codes[0, 0, 129, 5] == 0xFE and ds[0, 0, 1] == np.float32(3.0) / np.float32(448)
    assert np.count_nonzero(codes) == 1


def test_d_major_layout():
    x = _gauss((2, 3, 200, 64), 6)
    codes, _ = of8.quantize_blocks(x)
    t = of8.to_d_major(codes)
    assert t.shape == (2, 3, 64, 256)
    assert np.array_equal(t[:, :, :, :200], np.swapaxes(codes, 2, 3)) and np.all(t[:, :, :, 200:] == 0)


# ---------------------------------------------------------------------------
# FP8 forward on exactly representable inputs
# ---------------------------------------------------------------------------

def _representable(shape, seed, block_exponents):
    """Values e4m3 * 2^k per 128-row block, each block holding +-448 * 2^k, so
    that quantization reproduces them exactly."""
    rng = np.random.default_rng(seed)
    codes = rng.choice(FINITE[(FINITE & 0x7F) < 0x7E], size=shape).astype(np.uint8)
    x = of8.e4m3_decode(codes)
    for i, k in enumerate(block_exponents):
        x[:, :, 128 * i:128 * (i + 1)] *= 2.0 ** k
        x[:, :, 128 * i, 0] = 448.0 * 2.0 ** k
    return x.astype(np.float32)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_forward_is_exact_attention_on_representable_inputs(causal):
    B, Hq, Hkv, nq, nkv, d = 1, 2, 1, 200, 300, 64
    q = _representable((B, Hq, nq, d), 7, [-9, -7])
    k = _representable((B, Hkv, nkv, d), 8, [-8, -10, -6])
    v = _representable((B, Hkv, nkv, d), 9, [-3, 2, -5])
    q8, qd = of8.quantize_blocks(q)
    k8, kd = of8.quantize_blocks(k)
    v8, vd = of8.quantize_blocks(v)
    assert np.array_equal(of8.dequantize(q8, qd), q.astype(np.float64))
    assert np.array_equal(of8.dequantize(v8, vd), v.astype(np.float64))
    O8, L8 = of8.fp8_attention_forward(q8, qd, k8, kd, v8, vd, causal, 0.125)
    O, L = oracle.attention_forward(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), causal,
                                    0.125)
    assert np.max(np.abs(O8 - O)) <= 1e-12 and np.max(np.abs(L8 - L)) <= 1e-12


def test_dequantize_uses_each_rows_block():
    codes = np.full((1, 1, 300, 64), 0x38, np.uint8)        # every code is 1.0
    ds = np.array([[[1.0, 2.0, 4.0]]], np.float32)
    deq = of8.dequantize(codes, ds)
    assert np.all(deq[0, 0, :128] == 1) and np.all(deq[0, 0, 128:256] == 2) and np.all(deq[0, 0, 256:] == 4)


# ---------------------------------------------------------------------------
# Planted mistakes in copies of the encoder must fail the checks above.
# ---------------------------------------------------------------------------

def _mutant_encode(kind):
    vals = of8.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))

    def enc(y):
        y = np.asarray(y, dtype=np.float64)
        a = np.abs(y)
        if kind == "half_away":          # ties away from zero instead of to even
            r = np.array([vals[np.argmin(np.abs(vals - t) - 1e-30 * vals)] for t in a])
            mids = [(lo + hi) / 2 for lo, hi in zip(vals[:-1], vals[1:])]
            r = np.array([vals[np.searchsorted(vals, t)] if t in mids else rr for t, rr in zip(a, r)])
        elif kind == "truncate":         # toward zero
            r = vals[np.clip(np.searchsorted(vals, a, side="right") - 1, 0, 126)]
        elif kind == "flush_subnormal":  # no subnormals
            r = vals[np.argmin(np.abs(vals[None, :] - a[:, None]), axis=1)]
            r = np.where(r < 2.0 ** -6, 0.0, r)
        idx = np.searchsorted(vals, np.minimum(r, 448.0))
        return np.where(np.signbit(y), idx | 0x80, idx).astype(np.uint8)
    return enc


def _encode_pins_pass(enc):
    torch = pytest.importorskip("torch")
    vals = of8.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    even = np.array([c if c % 2 == 0 else c + 1 for c in range(0x7E)], dtype=np.uint8)
    ok = np.array_equal(enc(mids), even)
    x = (np.random.default_rng(11).standard_normal(4000) * 0.05).astype(np.float32)
    ok &= np.array_equal(enc(x), torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy())
    return bool(ok)


def test_encoder_pins_accept_the_oracle():
    assert _encode_pins_pass(of8.e4m3_encode)


@pytest.mark.parametrize("kind", ["half_away", "truncate", "flush_subnormal"])
def test_encoder_pins_reject_planted_mistakes(kind):
    assert not _encode_pins_pass(_mutant_encode(kind))

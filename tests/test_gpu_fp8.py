"""GPU parity of the FP8 path: the block quantizer (bit-exact against the
oracle's float32 recipe) and the FP8 forward (against the float64 forward on
the dequantized inputs, within the bound of the probability rounding).

Inputs: seeded N(0,1) draws rounded to bf16, with per-128-row-block powers of
two so that the block scales differ; the forward's codes come from the
oracle's quantizer on the CPU, so no input of the oracle comes from the GPU.
"""

from __future__ import annotations

import numpy as np
import pytest

from oracle import attention as oatt
from oracle import fp8 as of8
from tests.gpu_util import bf16_half_ulp, default_scale, ensure_library, sample_rows, to_f64
from workloads import DTYPE_BF16, bf16_bits_to_f32, block_spread_bits, make_inputs_shape

pytestmark = pytest.mark.gpu

@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ensure_library()


def bits_to_torch(bits, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy()).view(torch.bfloat16).to(device)


def np_to_torch(a, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


# ---------------------------------------------------------------------------
# quantizer
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shape,d_major", [
    ((1, 1, 128, 64), False), ((2, 3, 300, 128), False), ((2, 3, 300, 128), True),
    ((1, 2, 1000, 64), True), ((1, 1, 5, 128), True), ((3, 2, 257, 64), False),
])
def test_quantizer_bit_exact(shape, d_major):
    import exact_attention_109_amd as fa
    B, H, N, d = shape
    bits = make_inputs_shape(DTYPE_BF16, B, H, H, N, N, d, seed=31).raw("q")
    bits = block_spread_bits(bits, 32, -20, 20)
    if N > 128:
        bits[0, 0, :128] = 0                       # an all-zero block
        bits[-1, -1, 128:256] = bits[-1, -1, 128:256] & np.uint16(0x807F) | np.uint16(0x0080)  # tiny values
    codes, ds = fa.quantize_fp8(bits_to_torch(bits), d_major=d_major)
    ref_codes, ref_ds = of8.quantize_blocks(bf16_bits_to_f32(bits))
    if d_major:
        ref_codes = of8.to_d_major(ref_codes)
    got_ds = ds.cpu().numpy()
    assert np.array_equal(got_ds.view(np.uint32), ref_ds.view(np.uint32))
    got = codes.cpu().numpy()
    mism = np.count_nonzero(got != ref_codes)
    assert mism == 0, f"{mism} codes differ"


def test_quantizer_two_calls_and_extremes():
    import exact_attention_109_amd as fa
    x = np.zeros((1, 1, 256, 128), np.float32)
    x[0, 0, 0, 0] = 3.0e38                          # near the largest bf16
    x[0, 0, 1, :] = np.linspace(-3e38, 3e38, 128)
    x[0, 0, 128:] = np.float32(1e-38)               # subnormal block: 448 / amax overflows
    from workloads import f32_to_bf16_bits
    bits = f32_to_bf16_bits(x)
    ref_codes, ref_ds = of8.quantize_blocks(bf16_bits_to_f32(bits))
    for d_major in (False, True):
        codes, ds = fa.quantize_fp8(bits_to_torch(bits), d_major=d_major)
        rc = of8.to_d_major(ref_codes) if d_major else ref_codes
        assert np.array_equal(codes.cpu().numpy(), rc)
        assert np.array_equal(ds.cpu().numpy().view(np.uint32), ref_ds.view(np.uint32))


# ---------------------------------------------------------------------------
# forward
# ---------------------------------------------------------------------------

def make_fp8_case(B, H_q, H_kv, N_q, N_kv, d, seed, spread=(-4, 4), zero_v_block=False, spread_v=None):
    """Seeded bf16 draws with each 128-row block of Q, K (spread) and V
    (spread_v, default the same) multiplied by 2^k, k uniform in the range,
    then quantized by the oracle's block quantizer."""
    inp = make_inputs_shape(DTYPE_BF16, B, H_q, H_kv, N_q, N_kv, d, seed)
    src = {}
    for i, n in enumerate(("q", "k", "v")):
        lo, hi = spread_v if (n == "v" and spread_v is not None) else spread
        bits = block_spread_bits(inp.raw(n), seed + 100 + i, lo, hi)
        src[n] = bf16_bits_to_f32(bits)
    if zero_v_block and N_kv > 128:
        src["v"][:, :, 128:256] = 0
    q8, qd = of8.quantize_blocks(src["q"])
    k8, kd = of8.quantize_blocks(src["k"])
    v8, vd = of8.quantize_blocks(src["v"])
    return dict(q8=q8, qd=qd, k8=k8, kd=kd, v8=v8, vd=vd)


def run_fp8(c, causal, scale):
    import exact_attention_109_amd as fa
    o, lse = fa.fwd_fp8(np_to_torch(c["q8"]), np_to_torch(c["qd"]), np_to_torch(c["k8"]), np_to_torch(c["kd"]),
                        np_to_torch(c["v8"]), np_to_torch(c["vd"]), causal=causal, scale=scale)
    return to_f64(o), lse.cpu().numpy().astype(np.float64)


# The FP8 matrix instruction does not sum its 64 products exactly: measured
# on gfx950 with random e4m3 operands, the error of one 32x32x64 step stays
# below 2^-11 of the largest |product| (2^-11.8 of the sum of |products|).
# The tests allow GAMMA = 2^-9 of the sum of |products| per score.
GAMMA = 2.0 ** -9


def _logsumexp_rows(a):
    m = np.max(a, axis=1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    return (m + np.log(np.sum(np.exp(a - m), axis=1, keepdims=True)))[:, 0]


def fp8_bound(c, b, h, G, causal, scale, rows):
    """Bounds for head (b, h), given rows: returns the oracle O and LSE, the
    per-element O bound and the per-row LSE bound.

    Scores: key j of row i is off by at most delta_ij = GAMMA * scale *
    sum_k |q_ik k_jk| (the FP8 instruction's summation) plus float32
    rounding. With w the exact probabilities, the LSE then moves by at most
    E_i = ln sum_j w_ij exp(delta_ij) (Jensen on both sides), and each
    probability by a factor within exp(+-(delta_ij + E_i)). Probability
    rounding (see fa_fwd_fp8): 2^-4 * sum_j max(w_j, 2^-6 wmax / cv_j) |v_j|.
    The PV sums: GAMMA of the same sum. Everything is formed in the log
    domain, so the bound is finite whenever the deltas are."""
    hk = h // G
    q = of8.dequantize(c["q8"][b:b + 1, h:h + 1], c["qd"][b:b + 1, h:h + 1])[0, 0]
    k = of8.dequantize(c["k8"][b:b + 1, hk:hk + 1], c["kd"][b:b + 1, hk:hk + 1])[0, 0]
    v = of8.dequantize(c["v8"][b:b + 1, hk:hk + 1], c["vd"][b:b + 1, hk:hk + 1])[0, 0]
    rows = np.asarray(rows)
    O, L = oatt.head_forward(q, k, v, causal, scale, rows)
    W = oatt.head_probabilities(q, k, causal, scale, rows)         # exact probabilities
    sig = scale * (np.abs(q[rows]) @ np.abs(k).T)
    allowed = np.ones_like(sig, dtype=bool)
    if causal:
        allowed = np.arange(k.shape[0])[None, :] <= rows[:, None]
    delta = np.where(allowed, GAMMA * sig + 1e-6 * (1.0 + np.abs(L)[:, None] + sig), 0.0)
    # a key whose exact probability underflows (w < e^-700) stays negligible
    # unless its score can move by hundreds
    assert float(delta.max()) < 30.0, float(delta.max())
    with np.errstate(divide="ignore"):
        logw = np.log(W)
    E = _logsumexp_rows(np.where(allowed, logw + delta, -np.inf))    # >= 0
    assert np.all(np.isfinite(E))
    r = np.expm1(delta + E[:, None])                                   # relative change of each w_ij
    vdb = np.repeat(c["vd"][b, hk].astype(np.float64), 128)[:k.shape[0]]
    cv = np.maximum(8.0 * vdb / max(float(c["vd"][b, hk].max()), 1e-38), 2.0 ** -20)
    wmax = W.max(axis=1, keepdims=True)                               # = 1 / L
    rmax = np.expm1(delta.max(axis=1, keepdims=True) + E[:, None])
    eff = np.maximum(W * (1.0 + r), 2.0 ** -6 * wmax * (1.0 + rmax) / cv[None, :])
    av = np.abs(v)
    wv = W @ av
    o_bound = ((W * r) @ av + 2.0 ** -4 * (eff @ av) + GAMMA * (eff @ av) * 1.07
               + 1e-5 * wv + 1e-6 * av.max())
    assert np.all(np.isfinite(o_bound))
    return O, L, o_bound, E + 1e-5


def check_case(c, B, H_q, H_kv, N_q, causal, scale, rows_per_head=None, seed=0):
    got_o, got_l = run_fp8(c, causal, scale)
    G = H_q // H_kv
    rng = np.random.default_rng(seed)
    worst = 0.0
    for b in range(B):
        for h in range(H_q):
            rows = np.arange(N_q) if rows_per_head is None else sample_rows(N_q, rng, rows_per_head)
            O, L, tol, ltol = fp8_bound(c, b, h, G, causal, scale, rows)
            err = np.abs(got_o[b, h, rows] - O)
            allowed = tol + bf16_half_ulp(O)
            assert np.all(err <= allowed), (b, h, float(np.max(err - allowed)))
            assert np.all(np.abs(got_l[b, h, rows] - L) <= ltol), (b, h)
            worst = max(worst, float(np.max(err / np.maximum(allowed, 1e-30))))
    return worst


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_fp8_small(d, causal):
    B, H_q, H_kv, N_q, N_kv = 2, 4, 2, 333, 333
    c = make_fp8_case(B, H_q, H_kv, N_q, N_kv, d, seed=41 + d + causal)
    check_case(c, B, H_q, H_kv, N_q, causal, default_scale(d))


@pytest.mark.parametrize("n_q,n_kv,causal", [(1, 77, False), (70, 1, False), (256, 1000, True),
                                             (1000, 256, True), (512, 700, False), (129, 129, True)])
def test_fwd_fp8_ragged_shapes(n_q, n_kv, causal):
    c = make_fp8_case(1, 2, 1, n_q, n_kv, 128, seed=50 + n_q + n_kv)
    check_case(c, 1, 2, 1, n_q, causal, default_scale(128))


def test_fwd_fp8_zero_v_block_and_wide_spread():
    """V blocks spread over 2^-12 .. 2^12 with one all-zero block (so the V
    scales of the P V product span 24 binades and one is 0), Q and K blocks
    over 2^-1 .. 2^1."""
    c = make_fp8_case(1, 2, 2, 400, 600, 128, seed=61, spread=(-1, 1), spread_v=(-12, 12), zero_v_block=True)
    assert float(c["vd"].max()) / float(c["vd"][c["vd"] > 0].min()) > 2.0 ** 12
    worst = check_case(c, 1, 2, 2, 400, True, default_scale(128))
    print(f"largest error as a fraction of its bound: {worst:.3f}")


def test_fwd_fp8_score_jumps_take_the_block_again():
    """K block scales that jump by 4x every three scale blocks (384 keys; no
    other spread): a jump lands on a key block whose predecessor left the
    running max alone, so the kernel takes its exponentials against the stale
    max, finds a lane sum above 2^8, forms the block max and takes the block
    again. Every element stays within its bound, causal and not."""
    c = make_fp8_case(1, 2, 2, 900, 900, 128, seed=81, spread=(0, 0))
    for i in range(c["kd"].shape[2]):
        c["kd"][:, :, i] = c["kd"][:, :, i] * np.float32(4.0 ** (i // 3))
    for causal in (False, True):
        worst = check_case(c, 1, 2, 2, 900, causal, default_scale(128))
        print(f"causal={causal}: largest error as a fraction of its bound: {worst:.3f}")


def test_fwd_fp8_uniform_attention_is_exact():
    """q = 0: every allowed key has weight 1/count; with power-of-two V block
    scale ratios every rounded probability is exact, so O is the mean of V up
    to float32 sums and the bf16 output rounding."""
    B, H, N, d = 1, 2, 700, 128
    c = make_fp8_case(B, H, H, N, N, d, seed=71, spread=(-3, 3))
    for i in range(c["vd"].shape[2]):               # block scales 2^k: exact ratios
        c["vd"][:, :, i] = np.float32(2.0 ** (-(i % 4)))
    c["q8"][:] = 0
    for causal in (False, True):
        got_o, got_l = run_fp8(c, causal, default_scale(d))
        deq = of8.dequantize(c["v8"], c["vd"])
        for h in range(H):
            cs = np.cumsum(deq[0, h], axis=0)
            ref = cs / np.arange(1, N + 1)[:, None] if causal else np.broadcast_to(cs[-1] / N, (N, d))
            lse_ref = np.log(np.arange(1, N + 1)) if causal else np.full(N, np.log(N))
            tol = bf16_half_ulp(ref) + 1e-5 * np.abs(deq[0, h]).max()
            assert np.all(np.abs(got_o[0, h] - ref) <= tol), h
            assert np.max(np.abs(got_l[0, h] - lse_ref)) <= 1e-5


def test_fwd_fp8_bench_shape_sampled():
    """The benchmark's FP8 configuration (B=2, H=32, N=8192, d=128, causal),
    sampled rows of a few heads against the oracle."""
    B, H, N, d = 2, 32, 8192, 128
    inp = make_inputs_shape(DTYPE_BF16, B, H, H, N, N, d, seed=3)
    src = {n: bf16_bits_to_f32(inp.raw(n)) for n in ("q", "k", "v")}
    c = {}
    for n, key in (("q", "q"), ("k", "k"), ("v", "v")):
        c[key + "8"], c[key + "d"] = of8.quantize_blocks(src[n])
    got_o, got_l = run_fp8(c, True, default_scale(d))
    rng = np.random.default_rng(5)
    for b, h in ((0, 0), (1, 31), (0, 17)):
        rows = sample_rows(N, rng, 48)
        O, L, tol, ltol = fp8_bound(c, b, h, 1, True, default_scale(d), rows)
        err = np.abs(got_o[b, h, rows] - O)
        assert np.all(err <= tol + bf16_half_ulp(O)), (b, h)
        assert np.all(np.abs(got_l[b, h, rows] - L) <= ltol), (b, h)


def test_fwd_fp8_zero_v_gives_zero_output():
    """V = 0 everywhere (every V scale 0): O is exactly 0 and the LSE is the
    oracle's (the scores do not depend on V)."""
    c = make_fp8_case(1, 2, 1, 200, 300, 128, seed=81)
    c["v8"][:] = 0
    c["vd"][:] = 0
    got_o, got_l = run_fp8(c, True, default_scale(128))
    assert np.all(got_o == 0)
    rows = np.arange(200)
    for h in range(2):
        _, L, _, ltol = fp8_bound(c, 0, h, 2, True, default_scale(128), rows)
        assert np.all(np.abs(got_l[0, h] - L) <= ltol), h

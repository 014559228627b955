"""Split-KV forward with an FP8 key/value cache (fa_fwd_splitkv_fp8) on the
GPU: bf16 queries against e4m3 K and V (row-major, as a cache) with 128-key
block scales, checked
against the fp64 oracle on q and the dequantized K, V, at the bf16
path's error bound scaled to the values (the codes are widened to bf16
exactly, so the arithmetic is the bf16 split-KV path's). The codes come from the oracle's quantizer on the
CPU (no oracle input comes from the GPU); the V scales of the blocks differ
by powers of two so that a wrong block scale shows."""

import numpy as np
import pytest

import oracle
from oracle import fp8 as of8
from tests.gpu_util import TOL, bf16_half_ulp, default_scale, ensure_library, max_abs, to_f64
from workloads import DTYPE_BF16, bf16_bits_to_f32, block_spread_bits, make_inputs_shape

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ensure_library()


def make_case(B, Hq, Hkv, nq, nkv, d, seed, spread=(-3, 3), k_spread=(-1, 1)):
    inp = make_inputs_shape(DTYPE_BF16, B, Hq, Hkv, nq, nkv, d, seed)
    k = bf16_bits_to_f32(block_spread_bits(inp.raw("k"), seed + 1, *k_spread))
    v = bf16_bits_to_f32(block_spread_bits(inp.raw("v"), seed + 2, *spread))
    k8, kd = of8.quantize_blocks(k)
    v8, vd = of8.quantize_blocks(v)
    return inp, k8, kd, v8, vd


def run(inp, k8, kd, v8, vd, causal, scale, S):
    import exact_attention_109_amd as fa
    import torch
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    q = inp.torch("q", "cuda")
    o, lse = fa.fwd_splitkv_fp8(q, dev(k8), dev(kd), dev(v8), dev(vd), S, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return to_f64(o), to_f64(lse)


def check_head(o, lse, q, k, v, causal, scale):
    """One head against the oracle. O: the bf16 path's bound, scaled to the
    values: P is rounded to bf16 (2^-8 relative per probability, allowed
    2^-7 here) before the PV product, and O itself is stored in bf16 (half
    an ulp). With the V blocks 2^-3 .. 2^3 apart, a fixed 1e-2 would not
    follow the magnitude of O. LSE: 1e-3 as for bf16."""
    O, L = oracle.head_forward(q, k, v, causal, scale)
    W = oracle.head_probabilities(q, k, causal, scale)
    tol = bf16_half_ulp(O) + 2.0 ** -7 * (W @ np.abs(v)) + 1e-5
    err = np.abs(o - O)
    assert np.all(err <= tol), float(np.max(err - tol))
    assert max_abs(lse, L) <= TOL[DTYPE_BF16]["lse"], max_abs(lse, L)


def check_all(o, lse, inp, k8, kd, v8, vd, causal, scale):
    B, Hq = o.shape[:2]
    Hkv = k8.shape[1]
    kk = of8.dequantize(k8, kd)
    vv = of8.dequantize(v8, vd)
    q = inp.f64("q")
    for b in range(B):
        for h in range(Hq):
            hk = h // (Hq // Hkv)
            check_head(o[b, h], lse[b, h], q[b, h], kk[b, hk], vv[b, hk], causal, scale)


# (B, H_q, H_kv, N_q, N_kv, d, causal, num_splits)
CASES = [
    (1, 1, 1, 1, 1, 128, False, 1),
    (1, 1, 1, 1, 1, 64, False, 4),
    (2, 8, 2, 1, 1000, 128, False, 4),
    (1, 32, 8, 1, 4097, 128, False, 16),
    (1, 8, 8, 1, 300, 64, False, 7),
    (2, 4, 4, 3, 517, 64, True, 3),
    (1, 8, 1, 4, 2048, 64, False, 8),
    (1, 4, 1, 2, 100, 128, True, 2),
    (1, 16, 2, 1, 33, 128, False, 256),
    (3, 6, 2, 5, 777, 128, False, 5),
    (1, 2, 1, 16, 64, 128, True, 1),
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}Hq{c[1]}Hkv{c[2]}Nq{c[3]}Nkv{c[4]}d{c[5]}{'c' if c[6] else 'n'}S{c[7]}" for c in CASES])
def test_against_oracle(case):
    B, Hq, Hkv, nq, nkv, d, causal, S = case
    print(f"case {case}", flush=True)
    inp, k8, kd, v8, vd = make_case(B, Hq, Hkv, nq, nkv, d, seed=900 + sum(case[:6]))
    scale = default_scale(d)
    o, lse = run(inp, k8, kd, v8, vd, causal, scale, S)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    check_all(o, lse, inp, k8, kd, v8, vd, causal, scale)


def test_zero_v_block_and_wide_spread():
    B, Hq, Hkv, nq, nkv, d = 1, 8, 2, 1, 1000, 128
    inp, k8, kd, v8, vd = make_case(B, Hq, Hkv, nq, nkv, d, seed=950, spread=(-12, 12), k_spread=(-3, 3))
    v8[:, :, 128:256] = 0
    vd[:, :, 1] = 0
    scale = default_scale(d)
    for S in (1, 3, 8):
        o, lse = run(inp, k8, kd, v8, vd, False, scale, S)
        check_all(o, lse, inp, k8, kd, v8, vd, False, scale)


def test_decode_workload_sampled():
    """The decode benchmark's per-workgroup configuration: its shape per
    (batch, key/value head) (H_q=32, H_kv=8, one query, 32768 keys, d=128)
    and its split count, on 2 of its 8 sequences (to keep the CPU side
    short), a few heads against the oracle."""
    import exact_attention_109_amd as fa
    import torch
    from workloads import DECODE_WORKLOADS
    w = DECODE_WORKLOADS["d1"]
    B = 2
    inp = make_inputs_shape(DTYPE_BF16, B, w.H_q, w.H_kv, w.N_q, w.N_kv, w.d, w.seed)
    k8, kd = of8.quantize_blocks(bf16_bits_to_f32(inp.raw("k")))
    v8, vd = of8.quantize_blocks(bf16_bits_to_f32(inp.raw("v")))
    S = fa.default_num_splits(w.B, w.H_kv, w.N_kv, torch.cuda.get_device_properties(0).multi_processor_count)
    o, lse = run(inp, k8, kd, v8, vd, w.causal, w.scale, S)
    G = w.H_q // w.H_kv
    for b, h in ((0, 0), (1, 17), (1, 31)):
        hk = h // G
        kk = of8.dequantize(k8[b:b + 1, hk:hk + 1], kd[b:b + 1, hk:hk + 1])[0, 0]
        vv = of8.dequantize(v8[b:b + 1, hk:hk + 1], vd[b:b + 1, hk:hk + 1])[0, 0]
        check_head(o[b, h], lse[b, h], inp.f64("q")[b, h], kk, vv, w.causal, w.scale)

"""Forward and backward parity on seeded random shapes: head counts, GQA
group sizes, sequence lengths from 1 to 1600 (so one to seven 256-row query
tiles, with the pairing of causal tiles r and n-1-r for odd and even tile
counts, ragged tails and N_q != N_kv), d = 64 or 128, causal or not. Every
element is compared with the fp64 oracle under the same bounds as the fixed
grids of test_gpu_fwd.py and test_gpu_bwd.py."""

import numpy as np
import pytest

import oracle
from tests.gpu_util import TOL, default_scale, ensure_library, map_heads, max_abs, o_small_check, to_f64, upload
from tests.test_gpu_bwd import grad_tol
from workloads import DTYPE_BF16, make_inputs_shape

pytestmark = pytest.mark.gpu

N_CASES = 24


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ensure_library()


def draw_cases():
    """The shapes, from a fixed generator (independent of the input seeds)."""
    rng = np.random.default_rng(20261203)
    cases = []
    for i in range(N_CASES):
        B = int(rng.integers(1, 3))
        H_kv = int(rng.integers(1, 4))
        G = int(rng.choice([1, 2, 4]))
        n_q = int(np.exp(rng.uniform(0.0, np.log(1600.0))))
        n_kv = n_q if rng.random() < 0.5 else int(np.exp(rng.uniform(0.0, np.log(1600.0))))
        d = int(rng.choice([64, 128]))
        causal = bool(rng.random() < 0.6)
        cases.append((i, B, G * H_kv, H_kv, max(1, n_q), max(1, n_kv), d, causal))
    return cases


def oracle_all(q, k, v, do, causal, scale, G, backward):
    B, H_q = q.shape[:2]
    heads = [(b, h) for b in range(B) for h in range(H_q)]
    fwd = map_heads(lambda bh: oracle.head_forward(q[bh[0], bh[1]], k[bh[0], bh[1] // G], v[bh[0], bh[1] // G],
                                                   causal, scale), heads)
    O = np.empty(q.shape[:3] + (v.shape[3],))
    L = np.empty(q.shape[:3])
    for (b, h), (o, l) in zip(heads, fwd):
        O[b, h], L[b, h] = o, l
    if not backward:
        return O, L, None
    bwd = map_heads(lambda bh: oracle.head_backward(q[bh[0], bh[1]], k[bh[0], bh[1] // G], v[bh[0], bh[1] // G],
                                                    do[bh[0], bh[1]], causal, scale), heads)
    gq = np.empty_like(q)
    gk = np.zeros_like(k)
    gv = np.zeros_like(v)
    for (b, h), (a, bk, bv) in zip(heads, bwd):
        gq[b, h] = a
        gk[b, h // G] += bk
        gv[b, h // G] += bv
    return O, L, (gq, gk, gv)


@pytest.mark.parametrize("case", draw_cases(), ids=lambda c: f"r{c[0]}")
def test_random_shape_against_oracle(case):
    import torch
    import exact_attention_109_amd as fa
    i, B, H_q, H_kv, n_q, n_kv, d, causal = case
    backward = i % 2 == 0
    print(f"case {i}: B={B} H_q={H_q} H_kv={H_kv} N_q={n_q} N_kv={n_kv} d={d} causal={causal} "
          f"backward={backward}", flush=True)
    inp = make_inputs_shape(DTYPE_BF16, B, H_q, H_kv, n_q, n_kv, d, 9000 + i, with_grad=backward)
    scale = default_scale(d)
    if backward:
        q, k, v, do = upload(inp, ("q", "k", "v", "do"))
    else:
        q, k, v = upload(inp)
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    grads = fa.bwd(q, k, v, o, lse, do, causal=causal, scale=scale) if backward else None
    torch.cuda.synchronize()
    O, L, G_ref = oracle_all(inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.f64("do") if backward else None,
                             causal, scale, H_q // H_kv, backward)
    o, lse = to_f64(o), to_f64(lse)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    n_allow = o_small_check(o, O, DTYPE_BF16)
    el = max_abs(lse, L)
    assert el <= TOL[DTYPE_BF16]["lse"], el
    msg = f"O {max_abs(o, O):.3e} ({n_allow} past the plain bound), LSE {el:.3e}"
    if backward:
        errs = []
        for got, ref in zip((to_f64(x) for x in grads), G_ref):
            assert np.all(np.isfinite(got))
            e = max_abs(got, ref)
            assert e <= grad_tol(ref, DTYPE_BF16), (e, float(np.abs(ref).max()))
            errs.append(e)
        msg += f", dQ/dK/dV {errs[0]:.3e} {errs[1]:.3e} {errs[2]:.3e}"
    print(msg, flush=True)

"""Parity on shapes chosen for the order in which causal tiles visit their
blocks (fp64 oracle, the bounds of the fixed grids).

Forward, d = 128, dense causal calls: a workgroup takes query tiles r and
n-1-r; the lighter tile r visits its diagonal key blocks first and then the
blocks below them from the diagonal down. The cases cover a lighter tile
with no diagonal block at all (N_kv below the tile's first row, so the
descent starts at the ragged last key block), a ragged key block among the
diagonal blocks, even and odd tile counts, and GQA with the pair ranks dealt
over the query heads of a key/value head.

Backward dK/dV, causal: a workgroup takes key tiles r and n-1-r; the lighter
one visits its query blocks from its diagonal up. The cases cover a lighter
key tile past every query (its dK and dV must be exact zeros) and ragged
query tails."""

import numpy as np
import pytest

from tests.gpu_util import TOL, default_scale, ensure_library, max_abs, o_small_check, to_f64, upload
from tests.test_gpu_bwd import grad_tol
from tests.test_gpu_random_shapes import oracle_all
from workloads import DTYPE_BF16, make_inputs_shape

pytestmark = pytest.mark.gpu

# (B, H_q, H_kv, N_q, N_kv, backward)
CASES = [
    (1, 2, 1, 1300, 200, True),    # lighter tiles 1, 2 have no diagonal block; 8-key tail
    (1, 2, 2, 1300, 700, True),    # tile 2's diagonal blocks end in the 60-key tail block
    (1, 4, 1, 200, 1300, True),    # key tiles 2..10 see no query: zero dK, dV
    (2, 2, 2, 1536, 1536, False),  # six tiles: pairs (0,5), (1,4), (2,3)
    (1, 32, 8, 600, 600, False),   # GQA 4:1, three tiles: pair (0,2) and tile 1 alone
]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ensure_library()


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}_Hq{c[1]}_Hkv{c[2]}_Nq{c[3]}_Nkv{c[4]}")
def test_causal_block_order(case):
    import torch
    import exact_attention_109_amd as fa
    B, H_q, H_kv, n_q, n_kv, backward = case
    d, causal = 128, True
    print(f"case B={B} H_q={H_q} H_kv={H_kv} N_q={n_q} N_kv={n_kv} d={d} causal backward={backward}", flush=True)
    inp = make_inputs_shape(DTYPE_BF16, B, H_q, H_kv, n_q, n_kv, d, 7100 + n_q + n_kv, with_grad=backward)
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
        if n_kv > n_q:
            # keys at or past N_q are attended by no query (causal, top-left)
            _, gk, gv = (to_f64(x) for x in grads)
            assert np.all(gk[:, :, n_q:] == 0.0) and np.all(gv[:, :, n_q:] == 0.0)
        msg += f", dQ/dK/dV {errs[0]:.3e} {errs[1]:.3e} {errs[2]:.3e}"
    print(msg, flush=True)

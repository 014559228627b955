"""Backward parity on the GPU: fa_bwd (fed by fa_fwd's O and LSE) against
the fp64 oracle's textbook gradients on the same rounded inputs."""

import numpy as np
import pytest

import oracle
from tests.gpu_util import TOL, default_scale, ensure_library, map_heads, max_abs, to_f64, upload
from workloads import DTYPE_BF16, DTYPE_F32, WORKLOADS, make_inputs, make_inputs_shape

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ensure_library()


def run_fwd_bwd(inp, causal, scale):
    import torch
    import exact_attention_109_amd as fa
    q, k, v, do = upload(inp, ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return to_f64(dq), to_f64(dk), to_f64(dv)


def grad_tol(ref, dtype):
    """Gradient tolerance of the tiny-shape grid: TOL['grad'] for gradients of
    magnitude <= 1, the same fraction of max|ref| beyond. In bf16 the
    probabilities and dS are rounded to bf16 before each contraction and D_i
    comes from the bf16 forward output, each a relative error of up to 2^-8
    (the bf16 unit roundoff) per term, so the absolute error of a gradient
    grows with its magnitude; with few keys per row (tiny N_kv) these errors
    do not average out. In
    fp32 the grid reaches |dV| = 80 (300 queries on one key, two query heads
    summed), where one fp32 ulp is 7.6e-6 and a 600-term fp32 sum errs by
    far more than 1e-5 absolute."""
    return TOL[dtype]["grad"] * max(1.0, float(np.abs(ref).max()))


PAIRS = [(1, 1), (3, 17), (17, 3), (64, 64), (65, 65), (127, 129), (128, 128), (129, 255), (300, 255),
         (1, 300), (300, 1), (513, 511)]
HEADS = [(1, 1, 1), (2, 2, 1), (1, 4, 2), (1, 4, 1)]


@pytest.mark.parametrize("dtype", [DTYPE_BF16, DTYPE_F32])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_small_shapes_against_oracle(dtype, d, causal):
    tol = TOL[dtype]["grad"]
    seed = 500
    worst = 0.0
    for (nq, nkv) in PAIRS:
        for (B, Hq, Hkv) in HEADS:
            seed += 1
            print(f"case dtype={dtype} d={d} causal={causal} B={B} Hq={Hq} Hkv={Hkv} nq={nq} nkv={nkv}", flush=True)
            inp = make_inputs_shape(dtype, B, Hq, Hkv, nq, nkv, d, seed, with_grad=True)
            scale = default_scale(d)
            dq, dk, dv = run_fwd_bwd(inp, causal, scale)
            gq, gk, gv = oracle.attention_backward(inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.f64("do"),
                                                   causal, scale)
            errs = (max_abs(dq, gq), max_abs(dk, gk), max_abs(dv, gv))
            assert all(np.all(np.isfinite(x)) for x in (dq, dk, dv))
            for got, ref, e in zip((dq, dk, dv), (gq, gk, gv), errs):
                assert e <= grad_tol(ref, dtype), (nq, nkv, B, Hq, Hkv, errs)
            worst = max(worst, max(errs))
    print(f"worst gradient max-abs {worst:.3e}")


def test_config_c5():
    """Every element of dQ, dK, dV of the backward configuration against the
    oracle, and a second backward launch on the same device inputs bitwise
    equal to the first. Bound: grad_tol (1e-2 of max(1, max|ref|)). The few
    elements past a plain 1e-2 sit on the first causal rows, where a row has
    one or two keys, gradients reach |4.5|, D_i comes from the bf16 forward
    output (up to 0.05 from its exact value there) and the bf16 P and dS are
    not averaged over many keys."""
    import torch
    import exact_attention_109_amd as fa
    w = WORKLOADS["c5"]
    print(f"config c5: {w}", flush=True)
    inp = make_inputs(w)
    q, k, v, do = upload(inp, ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, causal=w.causal, scale=w.scale)
    g1 = fa.bwd(q, k, v, o, lse, do, causal=w.causal, scale=w.scale)
    g2 = fa.bwd(q, k, v, o, lse, do, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(g1, g2)), "two backward launches differ"
    dq, dk, dv = (to_f64(x) for x in g1)
    del g1, g2, q, k, v, do, o, lse
    assert all(np.all(np.isfinite(x)) for x in (dq, dk, dv))
    Q, K, V, dO = inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.f64("do")
    G = w.H_q // w.H_kv
    heads = [(b, h) for b in range(w.B) for h in range(w.H_q)]
    refs = map_heads(lambda bh: oracle.head_backward(Q[bh[0], bh[1]], K[bh[0], bh[1] // G], V[bh[0], bh[1] // G],
                                                     dO[bh[0], bh[1]], w.causal, w.scale), heads)
    gq = np.empty_like(dq)
    gk = np.zeros_like(dk)
    gv = np.zeros_like(dv)
    for (b, h), (a, bk, bv) in zip(heads, refs):
        gq[b, h] = a
        gk[b, h // G] += bk
        gv[b, h // G] += bv
    errs = (max_abs(dq, gq), max_abs(dk, gk), max_abs(dv, gv))
    rel = tuple(e / np.abs(r).max() for e, r in zip(errs, (gq, gk, gv)))
    heads_over = sorted({(b, h) for (b, h) in heads
                         if max(max_abs(dq[b, h], gq[b, h]), max_abs(dk[b, h // G], gk[b, h // G]),
                                max_abs(dv[b, h // G], gv[b, h // G])) > TOL[DTYPE_BF16]["grad"]})
    print(f"c5 max-abs (dq, dk, dv) {errs}, relative to max|ref| {rel}; heads past a plain 1e-2: {heads_over}")
    for got, ref, e in zip((dq, dk, dv), (gq, gk, gv), errs):
        assert e <= grad_tol(ref, DTYPE_BF16), errs


def test_gqa_config_c4_shape_reduced():
    """GQA backward at c4's head layout (32 query heads on 8 KV heads) with a
    shorter sequence so the oracle stays fast."""
    inp = make_inputs_shape(DTYPE_BF16, 1, 32, 8, 1024, 1024, 128, seed=44, with_grad=True)
    dq, dk, dv = run_fwd_bwd(inp, True, default_scale(128))
    q, k, v, do = inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.f64("do")
    gq, gk, gv = oracle.attention_backward(q[:, :8], k[:, :2], v[:, :2], do[:, :8], True, default_scale(128))
    errs = (max_abs(dq[:, :8], gq), max_abs(dk[:, :2], gk), max_abs(dv[:, :2], gv))
    print("GQA max-abs (dq, dk, dv):", errs, "max|ref|:", (np.abs(gq).max(), np.abs(gk).max(), np.abs(gv).max()))
    for e, ref in zip(errs, (gq, gk, gv)):
        assert e <= grad_tol(ref, DTYPE_BF16)


@pytest.mark.parametrize("dtype", [DTYPE_BF16, DTYPE_F32])
@pytest.mark.parametrize("Hq,Hkv,nq", [(2, 1, 0), (0, 3, 5)])
def test_no_query_rows_zero_dk_dv(dtype, Hq, Hkv, nq):
    """No query rows (N_q = 0, or H_q = 0) while keys exist: no key is
    attended, so dk and dv come back as exact zeros (buffers pre-filled with
    NaN, through the C entry point)."""
    import torch
    import exact_attention_109_amd as fa
    tdt = torch.bfloat16 if dtype == DTYPE_BF16 else torch.float32
    B, nkv, d = 2, 300, 128
    dev = "cuda"
    q = torch.zeros((B, Hq, nq, d), dtype=tdt, device=dev)
    k = torch.randn((B, Hkv, nkv, d), device=dev).to(tdt)
    v = torch.randn((B, Hkv, nkv, d), device=dev).to(tdt)
    lse = torch.zeros((B, Hq, nq), dtype=torch.float32, device=dev)
    dq = torch.zeros((B, Hq, nq, d), dtype=torch.float32, device=dev)
    dk = torch.full((B, Hkv, nkv, d), float("nan"), device=dev)
    dv = torch.full((B, Hkv, nkv, d), float("nan"), device=dev)
    ws = torch.empty((256,), dtype=torch.uint8, device=dev)
    rc = fa.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), q.data_ptr(), lse.data_ptr(), q.data_ptr(),
                   dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), 256, B, Hq, Hkv, nq, nkv, d,
                   1, default_scale(d), dtype, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == fa.FA_OK
    assert torch.count_nonzero(dk).item() == 0 and torch.count_nonzero(dv).item() == 0
    assert not torch.isnan(dk).any().item() and not torch.isnan(dv).any().item()


def test_determinism():
    import torch
    import exact_attention_109_amd as fa
    inp = make_inputs_shape(DTYPE_BF16, 1, 4, 2, 700, 700, 128, seed=34, with_grad=True)
    q, k, v, do = upload(inp, ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, causal=True)
    a = fa.bwd(q, k, v, o, lse, do, causal=True)
    b = fa.bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,Hq,Hkv,N", [(1, 2, 2, 2112), (1, 4, 2, 2048)])
def test_noncausal_long_sequences(d, B, Hq, Hkv, N):
    """Non-causal backward over many streamed query blocks: 33 blocks of 64
    queries per head (an odd count, which takes the pipeline's tail path) and
    a GQA case whose dK/dV sum over two query heads of 32 blocks each."""
    print(f"case d={d} B={B} Hq={Hq} Hkv={Hkv} N={N}", flush=True)
    inp = make_inputs_shape(DTYPE_BF16, B, Hq, Hkv, N, N, d, seed=700 + d + N, with_grad=True)
    scale = default_scale(d)
    dq, dk, dv = run_fwd_bwd(inp, False, scale)
    gq, gk, gv = oracle.attention_backward(inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.f64("do"), False, scale)
    errs = (max_abs(dq, gq), max_abs(dk, gk), max_abs(dv, gv))
    print("max-abs (dq, dk, dv):", errs, flush=True)
    for got, ref, e in zip((dq, dk, dv), (gq, gk, gv), errs):
        assert np.all(np.isfinite(got))
        assert e <= grad_tol(ref, DTYPE_BF16), errs


@pytest.mark.parametrize("causal", [False, True])
def test_extreme_logits(causal):
    """Q and K scaled by 8 (exact in bf16) so that scaled scores reach a few
    hundred and each probability row is nearly one-hot: the gradients stay
    finite and match the oracle's."""
    inp = make_inputs_shape(DTYPE_BF16, 1, 4, 2, 640, 640, 128, seed=911 + int(causal), with_grad=True,
                            qk_multiplier=8.0)
    scale = default_scale(128)
    dq, dk, dv = run_fwd_bwd(inp, causal, scale)
    q, k, v, do = inp.f64("q"), inp.f64("k"), inp.f64("v"), inp.f64("do")
    print("max |scaled score| of head 0:", float(np.abs(q[0, 0] @ k[0, 0].T).max() * scale), flush=True)
    gq, gk, gv = oracle.attention_backward(q, k, v, do, causal, scale)
    errs = (max_abs(dq, gq), max_abs(dk, gk), max_abs(dv, gv))
    print("max-abs (dq, dk, dv):", errs, "max|ref|:", (np.abs(gq).max(), np.abs(gk).max(), np.abs(gv).max()))
    for got, ref, e in zip((dq, dk, dv), (gq, gk, gv), errs):
        assert np.all(np.isfinite(got))
        assert e <= grad_tol(ref, DTYPE_BF16), errs


@pytest.mark.parametrize("causal", [False, True])
def test_zero_scale_closed_form(causal):
    """scale = 0: every allowed key has the same probability, so dQ and dK
    are exactly zero (both carry the factor scale) and dV_j is the sum of
    dO_i / (number of keys row i sees) over the rows i that see key j."""
    B, Hq, Hkv, N, d = 1, 2, 1, 300, 64
    inp = make_inputs_shape(DTYPE_BF16, B, Hq, Hkv, N, N, d, seed=77 + int(causal), with_grad=True)
    dq, dk, dv = run_fwd_bwd(inp, causal, 0.0)
    assert np.all(dq == 0.0) and np.all(dk == 0.0)
    do = inp.f64("do")
    ref = np.zeros((B, Hkv, N, d))
    bound = np.zeros((B, Hkv, N, d))
    for h in range(Hq):
        for i in range(N):
            cnt = i + 1 if causal else N
            ref[0, h // (Hq // Hkv), :cnt] += do[0, h, i] / cnt
            bound[0, h // (Hq // Hkv), :cnt] += np.abs(do[0, h, i]) / cnt
    err = np.abs(dv - ref)
    print("dV max-abs against the closed form:", float(err.max()), flush=True)
    # each P = 1/count is rounded to bf16 (relative error <= 2^-8) before
    # P^T dO; 1/count itself comes from exp2 in fp32 (a few ulp); the sum of
    # Hq * N products is accumulated in fp32 ((n - 1) * 2^-24 of sum |terms|)
    n_terms = Hq * N
    rel = 2.0 ** -8 + 2.0 ** -20 + n_terms * 2.0 ** -24
    assert np.all(err <= rel * bound + 1e-6), float((err - rel * bound).max())

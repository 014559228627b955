"""Pins for the CPU oracle (no GPU).

Each test ties the oracle to something other than itself: the values the
blog page prints for its online-softmax example, closed forms, invariants,
an independent brute-force route, and finite differences. The mutation tests
at the end plant plausible mistakes in copies of the oracle and check that
the pins catch them.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import attention as oatt
from workloads import (DTYPE_BF16, make_inputs_shape, f32_to_bf16_bits, bf16_bits_to_f32)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "online_softmax_worked_example.json")


def rand_qkv(rng, B, H_q, H_kv, N_q, N_kv, d, scale_qk=1.0):
    q = rng.standard_normal((B, H_q, N_q, d)) * scale_qk
    k = rng.standard_normal((B, H_kv, N_kv, d)) * scale_qk
    v = rng.standard_normal((B, H_kv, N_kv, d))
    return q, k, v


# ---------------------------------------------------------------------------
# C-4 #1: the worked example printed on the blog page (§2.1)
# ---------------------------------------------------------------------------

def test_worked_example_printed_values():
    g = json.load(open(GOLDEN))
    m, d, y, steps = oracle.online_normalizer(g["x"], trace=True)
    tol = g["printed_tolerance"]
    assert len(steps) == len(g["steps"])
    for (mi, di), ref in zip(steps, g["steps"]):
        assert abs(mi - ref["m"]) <= tol
        assert abs(di - ref["d"]) <= tol
    assert np.max(np.abs(y - np.array(g["softmax"]))) <= tol


def test_worked_example_closed_form():
    m, d, y, steps = oracle.online_normalizer([2.0, 1.0, 3.0], trace=True)
    e = math.e
    assert steps[0] == (2.0, 1.0)
    assert abs(steps[1][1] - (1 + 1 / e)) <= 1e-12
    assert abs(steps[2][1] - (1 + 1 / e + 1 / e ** 2)) <= 1e-12
    ref = np.array([1 / e, 1 / e ** 2, 1.0]) / (1 + 1 / e + 1 / e ** 2)
    assert np.max(np.abs(y - ref)) <= 1e-12
    assert abs(ref[0] - 0.2447284711) < 1e-10 and abs(ref[2] - 0.6652409558) < 1e-10
    lse = oracle.logsumexp_from_state(m, d)
    assert abs(lse - math.log(math.exp(2) + math.exp(1) + math.exp(3))) <= 1e-12
    assert abs(lse - 3.4076059644) <= 1e-9


# ---------------------------------------------------------------------------
# C-4 #2: online recurrence == safe softmax (blog §2.1 says they coincide)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 2, 3, 17, 128, 1000, 4096])
@pytest.mark.parametrize("mult", [1.0, 8.0, 100.0])
def test_online_equals_safe(n, mult):
    rng = np.random.default_rng(n * 7 + int(mult))
    x = rng.standard_normal(n) * mult
    if n > 4:
        x[rng.integers(0, n, size=n // 5)] = -np.inf   # masked entries
        x[0] = x[1]                                       # ties
        x[rng.integers(0, n)] = np.max(x[np.isfinite(x)])  # tie at the max
    m, d, y = oracle.online_normalizer(x)
    ref = oracle.safe_softmax(x)
    assert m == np.max(x)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=0)
    assert abs(np.sum(y) - 1.0) <= 1e-12
    # d_n equals the safe-softmax denominator sum exp(x - max)
    assert abs(d - np.sum(np.exp(x - np.max(x)))) <= 1e-12 * d


def test_online_matches_textbook_softmax_moderate_range():
    # Without overflow the plain softmax e^x / sum e^x is the textbook routine.
    x = np.linspace(-5, 5, 31)
    _, _, y = oracle.online_normalizer(x)
    ref = np.exp(x) / np.sum(np.exp(x))
    np.testing.assert_allclose(y, ref, rtol=1e-13)


def test_safe_softmax_survives_overflowing_exponents():
    # e^1000 overflows; the max-subtracted form does not.
    x = np.array([1000.0, 999.0, 998.0])
    y = oracle.safe_softmax(x)
    assert np.all(np.isfinite(y))
    np.testing.assert_allclose(y, oracle.safe_softmax(x - 1000.0), rtol=1e-15)


# ---------------------------------------------------------------------------
# C-4 #3: blockwise (m, d, O) update == materialized softmax * V (blog §2.2)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("block", [1, 7, 64, "all", "random"])
def test_blockwise_equals_materialized(causal, block):
    rng = np.random.default_rng(11)
    n, d = 150, 16
    q = rng.standard_normal((n, d))
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    scale = 1 / math.sqrt(d)
    if block == "all":
        blocks = [(0, n)]
    elif block == "random":
        blocks = oracle.random_blocks(n, rng, 40)
    else:
        blocks = oracle.even_blocks(n, block)
    O_ref, L_ref = oracle.head_forward(q, k, v, causal, scale)
    O_blk, L_blk = oracle.blockwise_head_forward(q, k, v, causal, scale, blocks, q_block=37)
    assert np.max(np.abs(O_blk - O_ref)) <= 1e-12
    assert np.max(np.abs(L_blk - L_ref)) <= 1e-12


def test_blockwise_extreme_logits():
    rng = np.random.default_rng(3)
    n, d = 200, 32
    q = rng.standard_normal((n, d)) * 8
    k = rng.standard_normal((n, d)) * 8
    v = rng.standard_normal((n, d))
    O_ref, L_ref = oracle.head_forward(q, k, v, True, 1 / math.sqrt(d))
    O_blk, L_blk = oracle.blockwise_head_forward(q, k, v, True, 1 / math.sqrt(d), oracle.even_blocks(n, 13))
    assert np.max(np.abs(O_blk - O_ref)) <= 1e-11
    assert np.max(np.abs(L_blk - L_ref)) <= 1e-12 * np.max(np.abs(L_ref))


# ---------------------------------------------------------------------------
# C-4 #4: probability rows sum to 1
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_rows_sum_to_one(causal):
    rng = np.random.default_rng(5)
    q, k, v = rand_qkv(rng, 1, 1, 1, 300, 280, 64)
    P = oracle.head_probabilities(q[0, 0], k[0, 0], causal, 0.125)
    assert np.max(np.abs(P.sum(axis=1) - 1.0)) <= 1e-12
    assert np.all(P >= 0)
    if causal:
        assert np.all(P[np.triu_indices(P.shape[0], 1, P.shape[1])] == 0)


# ---------------------------------------------------------------------------
# C-4 #5: brute force on tiny shapes (independent scalar loops)
# ---------------------------------------------------------------------------

TINY = [(B, Hq, Hkv, nq, nkv, d)
        for (B, Hq, Hkv) in [(1, 1, 1), (2, 2, 1), (1, 4, 2), (1, 4, 1)]
        for (nq, nkv) in [(1, 1), (2, 3), (5, 5), (17, 5), (3, 17)]
        for d in [1, 4, 8]]


def _f32_via_struct(x: float) -> float:
    """float32 rounding through the C library's double -> float conversion
    (round to nearest even), independent of numpy."""
    import struct
    return struct.unpack("<f", struct.pack("<f", x))[0]


def test_fp32_scale_is_the_float32_value():
    """The library takes the scale as a C float; the oracle must use exactly
    that value, not the float64 one (the default 1/sqrt(d) is not a float32
    number for d = 128)."""
    x = 1.0 / math.sqrt(128.0)
    got = oracle.fp32_scale(x)
    assert got != x                                         # the float64 value is not kept
    assert got == _f32_via_struct(x)
    import struct
    assert struct.pack("<f", got) == bytes.fromhex("f304b53d")  # 0x3DB504F3
    assert abs(got - x) <= 2.0 ** -28                       # half a float32 ulp in [2^-4, 2^-3)
    for exact in (0.125, 0.5, 1.0, 0.0, 3.0):               # float32 numbers pass unchanged
        assert oracle.fp32_scale(exact) == exact
    # ties round to even: 1 + 2^-24 lies halfway between 1 and 1 + 2^-23
    assert oracle.fp32_scale(1.0 + 2.0 ** -24) == 1.0
    assert oracle.fp32_scale(1.0 + 3 * 2.0 ** -24) == 1.0 + 2.0 ** -22


@pytest.mark.parametrize("shape", TINY[::3] + TINY[1::7])
@pytest.mark.parametrize("causal", [False, True])
def test_bruteforce_matches(shape, causal):
    B, Hq, Hkv, nq, nkv, d = shape
    rng = np.random.default_rng(hash(shape) % 2**32)
    q, k, v = rand_qkv(rng, B, Hq, Hkv, nq, nkv, d)
    scale = 1 / math.sqrt(d)
    O, L = oracle.attention_forward(q, k, v, causal, scale)
    Ob, Lb = oracle.bruteforce_attention(q.tolist(), k.tolist(), v.tolist(), causal, _f32_via_struct(scale))
    assert np.max(np.abs(O - np.array(Ob))) <= 1e-12
    assert np.max(np.abs(L - np.array(Lb))) <= 1e-12


# ---------------------------------------------------------------------------
# C-4 #6: closed forms
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_gives_uniform_average(causal):
    rng = np.random.default_rng(8)
    n_q, n_kv, d = 40, 40, 8
    q = np.zeros((1, 1, n_q, d))
    k = rng.standard_normal((1, 1, n_kv, d))
    v = rng.standard_normal((1, 1, n_kv, d))
    O, L = oracle.attention_forward(q, k, v, causal, 0.3)
    for i in range(n_q):
        allowed = (i + 1) if causal else n_kv
        assert np.max(np.abs(O[0, 0, i] - v[0, 0, :allowed].mean(axis=0))) <= 1e-13
        assert abs(L[0, 0, i] - math.log(allowed)) <= 1e-13


def test_single_key_returns_its_value():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((1, 2, 7, 8))
    k = rng.standard_normal((1, 2, 1, 8))
    v = rng.standard_normal((1, 2, 1, 8))
    O, L = oracle.attention_forward(q, k, v, False, 0.5)
    for h in range(2):
        assert np.max(np.abs(O[0, h] - v[0, h, 0][None, :])) <= 1e-14
        s = oracle.fp32_scale(0.5)
        np.testing.assert_allclose(L[0, h], s * (q[0, h] @ k[0, h, 0]), rtol=1e-14, atol=1e-14)


def test_causal_row_zero():
    rng = np.random.default_rng(10)
    q, k, v = rand_qkv(rng, 1, 1, 1, 9, 9, 8)
    O, L = oracle.attention_forward(q, k, v, True, 0.25)
    assert np.max(np.abs(O[0, 0, 0] - v[0, 0, 0])) == 0.0
    assert abs(L[0, 0, 0] - 0.25 * float(q[0, 0, 0] @ k[0, 0, 0])) <= 1e-14


def x213_as_attention(d=64):
    """The blog's x=[2,1,3] example as an attention call: one query e_0,
    keys x_j * e_0, values e_j, scale 1."""
    q = np.zeros((1, 1, 1, d))
    q[0, 0, 0, 0] = 1.0
    k = np.zeros((1, 1, 3, d))
    k[0, 0, :, 0] = [2.0, 1.0, 3.0]
    v = np.zeros((1, 1, 3, d))
    for j in range(3):
        v[0, 0, j, j] = 1.0
    return q, k, v


def test_x213_through_attention():
    g = json.load(open(GOLDEN))
    q, k, v = x213_as_attention()
    O, L = oracle.attention_forward(q, k, v, False, 1.0)
    assert np.max(np.abs(O[0, 0, 0, :3] - np.array(g["softmax"]))) <= g["printed_tolerance"]
    _, _, y = oracle.online_normalizer(g["x"])
    assert np.max(np.abs(O[0, 0, 0, :3] - y)) <= 1e-15
    assert np.all(O[0, 0, 0, 3:] == 0)
    assert abs(L[0, 0, 0] - 3.4076059644) <= 1e-9


# ---------------------------------------------------------------------------
# C-4 #7: GQA == MHA with K/V repeated
# ---------------------------------------------------------------------------

def test_gqa_equals_repeated_mha():
    rng = np.random.default_rng(12)
    B, Hq, Hkv, n, d = 2, 8, 2, 33, 8
    q, k, v = rand_qkv(rng, B, Hq, Hkv, n, n, d)
    do = rng.standard_normal(q.shape)
    G = Hq // Hkv
    kr = np.repeat(k, G, axis=1)
    vr = np.repeat(v, G, axis=1)
    for causal in (False, True):
        O1, L1 = oracle.attention_forward(q, k, v, causal, 0.3)
        O2, L2 = oracle.attention_forward(q, kr, vr, causal, 0.3)
        assert np.array_equal(O1, O2) and np.array_equal(L1, L2)
        dq1, dk1, dv1 = oracle.attention_backward(q, k, v, do, causal, 0.3)
        dq2, dk2, dv2 = oracle.attention_backward(q, kr, vr, do, causal, 0.3)
        assert np.max(np.abs(dq1 - dq2)) <= 1e-13
        assert np.max(np.abs(dk1 - dk2.reshape(B, Hkv, G, n, d).sum(axis=2))) <= 1e-12
        assert np.max(np.abs(dv1 - dv2.reshape(B, Hkv, G, n, d).sum(axis=2))) <= 1e-12


# ---------------------------------------------------------------------------
# C-4 #8: extreme logits (Q and K scaled by 8, |s| in the hundreds)
# ---------------------------------------------------------------------------

def test_extreme_logits_bounds():
    inp = make_inputs_shape(DTYPE_BF16, 1, 2, 1, 512, 512, 128, seed=4, qk_multiplier=8.0)
    q, k, v = inp.f64("q"), inp.f64("k"), inp.f64("v")
    scale = 1 / math.sqrt(128)
    O, L = oracle.attention_forward(q, k, v, True, scale)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))
    s = oracle.fp32_scale(scale)
    for h in range(2):
        S = s * (q[0, h] @ k[0, 0].T)
        S = np.where(np.tril(np.ones_like(S, dtype=bool)), S, -np.inf)
        mx = S.max(axis=1)
        assert np.max(np.abs(mx)) > 200          # the recipe does reach extreme logits
        assert np.all(mx <= L[0, h] + 1e-12)
        assert np.all(L[0, h] <= mx + np.log(np.arange(1, 513)) + 1e-12)


def test_bf16_rounding_helper():
    # RNE ties and exactness of the power-of-two multiply used by the recipe.
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -2.5, 3.14159], dtype=np.float32)
    b = f32_to_bf16_bits(x)
    back = bf16_bits_to_f32(b)
    assert back[0] == 1.0 and back[1] == 1.0          # tie to even (down)
    assert back[2] == 1.0 + 4 * 2**-8                 # tie to even (up)
    assert back[3] == -2.5
    assert abs(back[4] - 3.14159) <= 2**-7 * 4


# ---------------------------------------------------------------------------
# C-4 #9: backward vs finite differences, and identities
# ---------------------------------------------------------------------------

def _loss(q, k, v, do, causal, scale):
    O, _ = oracle.attention_forward(q, k, v, causal, scale)
    return float(np.sum(O * do))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 2, 1, 5, 5, 4), (1, 1, 1, 3, 5, 4), (2, 2, 2, 4, 3, 2)])
def test_backward_finite_differences(causal, shape):
    B, Hq, Hkv, nq, nkv, d = shape
    rng = np.random.default_rng(21)
    q, k, v = rand_qkv(rng, B, Hq, Hkv, nq, nkv, d)
    do = rng.standard_normal(q.shape)
    scale = 0.7
    dq, dk, dv = oracle.attention_backward(q, k, v, do, causal, scale)
    h = 1e-6
    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = arr[idx]
            arr[idx] = old + h
            lp = _loss(q, k, v, do, causal, scale)
            arr[idx] = old - h
            lm = _loss(q, k, v, do, causal, scale)
            arr[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        err = np.max(np.abs(num - grad)) / max(1.0, np.max(np.abs(grad)))
        assert err <= 1e-6, (name, err)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_identities(causal):
    rng = np.random.default_rng(22)
    B, Hq, Hkv, nq, nkv, d = 1, 4, 2, 40, 56, 8
    q, k, v = rand_qkv(rng, B, Hq, Hkv, nq, nkv, d)
    do = rng.standard_normal(q.shape)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, causal, 0.4)
    G = Hq // Hkv
    for hk in range(Hkv):
        # probabilities of each row sum to 1 -> sum_j dV_j = sum_i dO_i over the group
        grp = do[0, hk * G:(hk + 1) * G].sum(axis=(0, 1))
        assert np.max(np.abs(dv[0, hk].sum(axis=0) - grp)) <= 1e-12
        # shifting every key by one vector leaves each row's softmax unchanged
        assert np.max(np.abs(dk[0, hk].sum(axis=0))) <= 1e-12
    if causal:
        # keys no query may attend (j >= N_q) get zero gradient
        assert np.all(dk[0, :, nq:] == 0) and np.all(dv[0, :, nq:] == 0)
    # dQ of a row subset equals the full dQ rows
    rows = np.array([0, 5, 39])
    sub = oracle.head_dq_rows(q[0, 1], k[0, 0], v[0, 0], do[0, 1], causal, 0.4, rows)
    assert np.max(np.abs(sub - dq[0, 1, rows])) <= 1e-13


# ---------------------------------------------------------------------------
# Planted mistakes: copies of the oracle with one plausible bug each must
# fail at least one of the independent checks above.
# ---------------------------------------------------------------------------

def _mutant_forward(kind):
    def head_forward(q, k, v, causal, scale, rows=None, row_block=1024):
        s = oracle.fp32_scale(scale)
        n_q, n_kv = q.shape[0], k.shape[0]
        rows = np.arange(n_q) if rows is None else np.asarray(rows)
        S = s * (q[rows] @ k.T)
        if kind == "no_scale":
            S = q[rows] @ k.T
        if causal:
            keys = np.arange(n_kv)[None, :]
            allowed = keys < rows[:, None] if kind == "strict_causal" else keys <= rows[:, None]
            if kind == "causal_transposed":
                allowed = keys >= rows[:, None]
            S = np.where(allowed, S, -np.inf)
        m = S.max(axis=1, keepdims=True)
        with np.errstate(invalid="ignore", divide="ignore"):  # a strict mask leaves row 0 without keys
            P = np.exp(S - m)
            l = P.sum(axis=1, keepdims=True)
            if kind != "no_normalize":
                P = P / l
        out = P @ v
        if kind == "lse_log2":
            lse = (m + np.log2(l))[:, 0]
        elif kind == "lse_no_max":
            lse = np.log(l)[:, 0]
        else:
            lse = (m + np.log(l))[:, 0]
        return out, lse
    return head_forward


def _pins_pass(head_forward, gqa_kind=None):
    """Run a compact version of the independent checks against a forward."""
    rng = np.random.default_rng(99)
    ok = True
    # brute force on a tiny GQA shape, both masks
    B, Hq, Hkv, nq, nkv, d = 1, 4, 2, 5, 7, 4
    q, k, v = rand_qkv(rng, B, Hq, Hkv, nq, nkv, d)
    for causal in (False, True):
        Ob, Lb = oracle.bruteforce_attention(q.tolist(), k.tolist(), v.tolist(), causal, oracle.fp32_scale(0.5))
        G = Hq // Hkv
        for h in range(Hq):
            hk = h // G if gqa_kind is None else h % Hkv
            O, L = head_forward(q[0, h], k[0, hk], v[0, hk], causal, 0.5)
            ok &= np.max(np.abs(O - np.array(Ob[0][h]))) <= 1e-12
            ok &= np.max(np.abs(L - np.array(Lb[0][h]))) <= 1e-12
    # the worked example through attention
    q, k, v = x213_as_attention(8)
    O, L = head_forward(q[0, 0], k[0, 0], v[0, 0], False, 1.0)
    ok &= abs(L[0] - 3.4076059644) <= 1e-9
    ok &= np.max(np.abs(O[0, :3] - np.array([0.2447284711, 0.0900305732, 0.6652409558]))) <= 1e-9
    return bool(ok)


def test_pins_accept_the_oracle():
    assert _pins_pass(oatt.head_forward)


@pytest.mark.parametrize("kind", ["no_scale", "strict_causal", "causal_transposed", "no_normalize",
                                  "lse_log2", "lse_no_max"])
def test_pins_reject_planted_mistakes(kind):
    assert not _pins_pass(_mutant_forward(kind))


def test_pins_reject_wrong_gqa_mapping():
    assert not _pins_pass(oatt.head_forward, gqa_kind="modulo")


# ---------------------------------------------------------------------------
# Planted mistakes in the backward: copies of the textbook gradients with one
# plausible bug each must fail the finite-difference pin or the identities.
# ---------------------------------------------------------------------------

def _mutant_backward(kind):
    def backward(q, k, v, do, causal, scale):
        B, H_q, N_q, d = q.shape
        H_kv = k.shape[1]
        G = H_q // H_kv
        s = oracle.fp32_scale(scale)
        dq = np.zeros(q.shape)
        dk = np.zeros(k.shape)
        dv = np.zeros(v.shape)
        for b in range(B):
            for h in range(H_q):
                hk = h // G
                qh, kh, vh, doh = q[b, h], k[b, hk], v[b, hk], do[b, h]
                P = oracle.head_probabilities(qh, kh, causal, scale)
                dP = doh @ vh.T
                D = np.sum(P * dP, axis=1, keepdims=True)
                if kind == "d_from_do_only":
                    D = np.sum(doh, axis=1, keepdims=True)
                dS = P * (dP - D)
                if kind == "no_minus_d":
                    dS = P * dP
                gq = s * (dS @ kh)
                gk = s * (dS.T @ qh)
                gv = P.T @ doh
                if kind == "dq_no_scale":
                    gq = dS @ kh
                if kind == "dk_uses_do":
                    gk = s * (dS.T @ doh)
                if kind == "dv_uses_dp":
                    gv = dS.T @ doh
                dq[b, h] = gq
                if kind == "gqa_overwrite":
                    dk[b, hk] = gk
                    dv[b, hk] = gv
                else:
                    dk[b, hk] += gk
                    dv[b, hk] += gv
        return dq, dk, dv
    return backward


def _backward_pins_pass(backward):
    """Central differences on a tiny GQA shape (both masks) and the
    sum identities of dV and dK."""
    rng = np.random.default_rng(31)
    B, Hq, Hkv, nq, nkv, d = 1, 2, 1, 4, 5, 3
    q, k, v = rand_qkv(rng, B, Hq, Hkv, nq, nkv, d)
    do = rng.standard_normal(q.shape)
    scale = 0.7
    ok = True
    for causal in (False, True):
        dq, dk, dv = backward(q, k, v, do, causal, scale)
        for arr, grad in ((q, dq), (k, dk), (v, dv)):
            num = np.zeros_like(arr)
            it = np.nditer(arr, flags=["multi_index"])
            for _ in it:
                idx = it.multi_index
                old = arr[idx]
                arr[idx] = old + 1e-6
                lp = _loss(q, k, v, do, causal, scale)
                arr[idx] = old - 1e-6
                lm = _loss(q, k, v, do, causal, scale)
                arr[idx] = old
                num[idx] = (lp - lm) / 2e-6
            ok &= np.max(np.abs(num - grad)) / max(1.0, np.max(np.abs(grad))) <= 1e-6
        ok &= np.max(np.abs(dv[0, 0].sum(axis=0) - do[0].sum(axis=(0, 1)))) <= 1e-12
        ok &= np.max(np.abs(dk[0, 0].sum(axis=0))) <= 1e-12
    return bool(ok)


def test_backward_pins_accept_the_oracle():
    assert _backward_pins_pass(oracle.attention_backward)


@pytest.mark.parametrize("kind", ["no_minus_d", "d_from_do_only", "dq_no_scale", "dk_uses_do", "dv_uses_dp",
                                  "gqa_overwrite"])
def test_backward_pins_reject_planted_mistakes(kind):
    assert not _backward_pins_pass(_mutant_backward(kind))

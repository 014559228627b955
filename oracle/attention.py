"""Exact scaled-dot-product attention in float64, materialized.

Sources:
  * "FlashAttention" (LLM Inference Handbook, Kernel Optimization), section
    "attention 为什么一开始就很慢": the definition softmax(QK^T / sqrt(d_k)) V
    and the three naive steps (scores, softmax, weighted sum of V).
  * "深度学习进阶（三十一）FlashAttention：IO 感知的精确注意力" (rkmt.cn blog),
    §2.1: softmax is evaluated in the safe, max-subtracted form.
  * "Flash-Attention" (Awesome System Papers Wiki), 核心思想 (core idea): the
    backward pass rebuilds the probabilities from Q, K, V and a few per-row
    statistics; 设计空间与取舍 (design space): causal, non-causal and GQA
    (query heads sharing a K/V head) are the mask and head-sharing variants.

The pages give no backward formulas; the ones here are the textbook
derivatives of the forward definition (checked against finite differences).

Readings taken where the pages are silent:
  * the score scale is passed in (default 1/sqrt(d)); the oracle uses the
    float32 value of it exactly, as the library does;
  * causal means query i may attend keys j <= i (top-left aligned);
  * GQA maps query head h to key/value head floor(h / G), G = H_q / H_kv;
  * the saved statistic is LSE_i = ln sum_{allowed j} exp(s_ij), natural log;
  * gradients are those of the scalar L = sum(dO * O).

Test infrastructure only: nothing in the library's product path imports this.
"""

from __future__ import annotations

import numpy as np


def fp32_scale(scale: float) -> float:
    """The scale as the library sees it: rounded to float32, then widened."""
    return float(np.float32(scale))


def _allowed_mask(rows: np.ndarray, n_kv: int, causal: bool) -> np.ndarray | None:
    if not causal:
        return None
    return np.arange(n_kv)[None, :] <= rows[:, None]


def head_forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool, scale: float,
                 rows: np.ndarray | None = None, row_block: int = 1024):
    """One head: q [N_q, d], k and v [N_kv, d] (float64).

    Returns O [R, d] and LSE [R] for the query rows ``rows`` (all rows when
    None). Each row's full probability vector over all N_kv keys is formed
    explicitly, which is the point of this reference."""
    n_q, d = q.shape
    n_kv = k.shape[0]
    s = fp32_scale(scale)
    if rows is None:
        rows = np.arange(n_q)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.size, v.shape[1]), dtype=np.float64)
    lse = np.empty((rows.size,), dtype=np.float64)
    for r0 in range(0, rows.size, row_block):
        idx = rows[r0:r0 + row_block]
        S = s * (q[idx] @ k.T)                       # scores
        allowed = _allowed_mask(idx, n_kv, causal)
        if allowed is not None:
            S = np.where(allowed, S, -np.inf)
        m = S.max(axis=1, keepdims=True)              # safe-softmax shift
        P = np.exp(S - m)
        l = P.sum(axis=1, keepdims=True)
        P /= l                                        # probabilities
        out[r0:r0 + idx.size] = P @ v                 # weighted sum of V
        lse[r0:r0 + idx.size] = (m + np.log(l))[:, 0]
    return out, lse


def head_probabilities(q, k, causal, scale, rows=None):
    """The full probability matrix P [R, N_kv] of one head (for checks)."""
    n_q = q.shape[0]
    n_kv = k.shape[0]
    s = fp32_scale(scale)
    if rows is None:
        rows = np.arange(n_q)
    rows = np.asarray(rows, dtype=np.int64)
    S = s * (q[rows] @ k.T)
    allowed = _allowed_mask(rows, n_kv, causal)
    if allowed is not None:
        S = np.where(allowed, S, -np.inf)
    m = S.max(axis=1, keepdims=True)
    P = np.exp(S - m)
    return P / P.sum(axis=1, keepdims=True)


def attention_forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool, scale: float,
                      rows: np.ndarray | None = None):
    """q [B, H_q, N_q, d], k and v [B, H_kv, N_kv, d] -> O [B, H_q, R, d], LSE [B, H_q, R].

    ``rows`` optionally restricts the output to a subset of query rows (the
    same subset for every head); each output row depends only on its own
    query and on all keys, so a subset is computed exactly as in the full
    result."""
    B, H_q, N_q, d = q.shape
    H_kv = k.shape[1]
    assert H_q % H_kv == 0
    G = H_q // H_kv
    R = N_q if rows is None else len(rows)
    O = np.empty((B, H_q, R, v.shape[3]), dtype=np.float64)
    L = np.empty((B, H_q, R), dtype=np.float64)
    for b in range(B):
        for h in range(H_q):
            hk = h // G
            O[b, h], L[b, h] = head_forward(q[b, h], k[b, hk], v[b, hk], causal, scale, rows)
    return O, L


def head_backward(q, k, v, do, causal, scale):
    """Gradients of L = sum(dO * O) for one head (float64).

    With P the probabilities of the forward definition:
        dV = P^T dO
        dP = dO V^T
        D_i = sum_j P_ij dP_ij
        dS = P * (dP - D)             (zero where P is masked)
        dQ = scale * dS K
        dK = scale * dS^T Q
    Returns dq [N_q, d], dk [N_kv, d], dv [N_kv, d]."""
    s = fp32_scale(scale)
    P = head_probabilities(q, k, causal, scale)
    dv = P.T @ do
    dP = do @ v.T
    D = np.sum(P * dP, axis=1, keepdims=True)
    dS = P * (dP - D)
    dq = s * (dS @ k)
    dk = s * (dS.T @ q)
    return dq, dk, dv


def attention_backward(q, k, v, do, causal, scale):
    """Full-batch gradients. dK and dV of a key/value head sum the
    contributions of its G query heads."""
    B, H_q, N_q, d = q.shape
    H_kv = k.shape[1]
    G = H_q // H_kv
    dq = np.zeros(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    for b in range(B):
        for h in range(H_q):
            hk = h // G
            gq, gk, gv = head_backward(q[b, h], k[b, hk], v[b, hk], do[b, h], causal, scale)
            dq[b, h] = gq
            dk[b, hk] += gk
            dv[b, hk] += gv
    return dq, dk, dv


def head_dq_rows(q, k, v, do, causal, scale, rows):
    """dQ for a subset of query rows of one head (each row is independent)."""
    s = fp32_scale(scale)
    rows = np.asarray(rows, dtype=np.int64)
    P = head_probabilities(q, k, causal, scale, rows)
    dP = do[rows] @ v.T
    D = np.sum(P * dP, axis=1, keepdims=True)
    return s * ((P * (dP - D)) @ k)

"""The blockwise online-softmax update of attention, in float64.

Source: "深度学习进阶（三十一）FlashAttention：IO 感知的精确注意力" (rkmt.cn
blog), §2.2 "把 Online Softmax 嵌入注意力": one block of queries stays fixed
while the key/value blocks stream past it; every query row carries a running
maximum m, a normalizer d and an output O; for block j the steps are the
block scores S_j, their row maximum m_j, the new maximum m_new, the updated
normalizer d_new and the updated output O_new.

Reading taken where the page is ambiguous: in the O update the factor written
"softmax_j(S_j)" is the unnormalized exp(S_j - m_j) (the sum of the same
terms already sits in d_new, and with this reading the update is exact).
The blog's S_j carries no scale; the scale of the attention definition is
applied to the scores here.

This is the oracle's second route to the attention output, used only to
cross-check the materialized definition. Test infrastructure only.
"""

from __future__ import annotations

import numpy as np

from .attention import fp32_scale


def blockwise_head_forward(q, k, v, causal, scale, kv_blocks, q_block=None):
    """One head, Q-stationary: for each query block, stream the key/value
    blocks given by ``kv_blocks`` (a list of (start, stop) covering
    [0, N_kv) in order) and apply the update of blog §2.2.

    Returns O [N_q, d_v] and LSE [N_q] (LSE = m + ln d)."""
    n_q = q.shape[0]
    n_kv = k.shape[0]
    s = fp32_scale(scale)
    if q_block is None:
        q_block = n_q
    O_all = np.empty((n_q, v.shape[1]))
    L_all = np.empty((n_q,))
    for q0 in range(0, n_q, q_block):
        rows = np.arange(q0, min(n_q, q0 + q_block))
        m = np.full((rows.size, 1), -np.inf)
        d = np.zeros((rows.size, 1))
        O = np.zeros((rows.size, v.shape[1]))
        for (k0, k1) in kv_blocks:
            S = s * (q[rows] @ k[k0:k1].T)                      # step 1: block scores
            if causal:
                keys = np.arange(k0, k1)
                S = np.where(keys[None, :] <= rows[:, None], S, -np.inf)
            m_j = S.max(axis=1, keepdims=True)                  # step 2: block max
            m_new = np.maximum(m, m_j)                          # step 3: running max
            # Every row may attend key 0, which sits in the first block, so the
            # running max is finite from the first block on.
            assert np.all(np.isfinite(m_new))
            # A row whose keys in this block are all masked has m_j = -inf and
            # contributes nothing; any finite shift keeps its terms at exactly 0.
            m_j = np.where(np.isfinite(m_j), m_j, m_new)
            E = np.exp(S - m_j)                                 # exp(S_j - m_j), unnormalized
            a_prev = np.exp(m - m_new)                          # 0 on the first block
            a_blk = np.exp(m_j - m_new)
            d_new = a_prev * d + a_blk * E.sum(axis=1, keepdims=True)          # step 4
            O_new = (d / d_new) * a_prev * O + (a_blk / d_new) * (E @ v[k0:k1])  # step 5
            m, d, O = m_new, d_new, O_new
        O_all[rows] = O
        L_all[rows] = (m + np.log(d))[:, 0]
    return O_all, L_all


def even_blocks(n: int, size: int):
    """[(0, size), (size, 2*size), ...] covering [0, n)."""
    return [(i, min(n, i + size)) for i in range(0, n, size)]


def random_blocks(n: int, rng: np.random.Generator, max_size: int):
    """A random partition of [0, n) into consecutive blocks of 1..max_size."""
    out = []
    i = 0
    while i < n:
        size = int(rng.integers(1, max_size + 1))
        out.append((i, min(n, i + size)))
        i += size
    return out

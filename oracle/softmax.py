"""Softmax references in float64: the safe softmax and the streaming
(online) normalizer recurrence.

Sources (the pages this library is built from):
  * "深度学习进阶（三十一）FlashAttention：IO 感知的精确注意力" (rkmt.cn blog),
    §2.1 "Online Softmax": the plain softmax, the safe softmax that subtracts
    the vector maximum, the per-element recurrence for the running maximum
    m_i and normalizer d_i, and the worked example on x = [2, 1, 3].

Test infrastructure only: nothing in the library's product path imports this.
"""

from __future__ import annotations

import math

import numpy as np


def safe_softmax(x) -> np.ndarray:
    """Safe softmax of a 1-D vector (blog §2.1, the max-subtracted form).

    Subtracting m = max(x) leaves the ratio e^{x_i}/sum_j e^{x_j} unchanged and
    keeps every exponent <= 0. Entries equal to -inf get probability 0. At least
    one entry must be finite."""
    x = np.asarray(x, dtype=np.float64)
    m = np.max(x)
    e = np.exp(x - m)
    return e / np.sum(e)


def online_normalizer(x, trace: bool = False):
    """The streaming recurrence of blog §2.1, one element at a time.

    Starting from m_0 = -inf and d_0 = 0, element x_i updates
        m_i = max(m_{i-1}, x_i)
        d_i = d_{i-1} * e^{m_{i-1} - m_i} + e^{x_i - m_i}
    and the probabilities are y_i = e^{x_i - m_n} / d_n once the stream ends.

    e^{-inf} is read as 0 (the first step multiplies d_0 = 0 by it). A
    rescale factor e^{m_{i-1} - m_i} with both maxima -inf (a stream that has
    seen only -inf so far) is taken as 1 so that d stays 0.

    Returns (m_n, d_n, y) and, with trace=True, also the list of (m_i, d_i)."""
    m = -math.inf
    d = 0.0
    steps = []
    for xi in np.asarray(x, dtype=np.float64).tolist():
        m_new = max(m, xi)
        if m_new == -math.inf:
            alpha = 1.0
            term = 0.0
        else:
            alpha = math.exp(m - m_new)  # exp(-inf) == 0.0
            term = math.exp(xi - m_new)
        d = d * alpha + term
        m = m_new
        steps.append((m, d))
    xs = np.asarray(x, dtype=np.float64)
    y = np.exp(xs - m) / d
    if trace:
        return m, d, y, steps
    return m, d, y


def logsumexp_from_state(m: float, d: float) -> float:
    """ln(sum_i e^{x_i}) from the recurrence's final state: m + ln d."""
    return m + math.log(d)

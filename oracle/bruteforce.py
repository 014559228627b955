"""Attention by scalar loops in plain Python, for tiny shapes only.

Source: the definition softmax(QK^T / sqrt(d_k)) V in "FlashAttention" (LLM
Inference Handbook, Kernel Optimization), section "attention 为什么一开始就很慢",
with softmax in the max-subtracted form of "深度学习进阶（三十一）FlashAttention：
IO 感知的精确注意力" (rkmt.cn blog) §2.1. Every dot product and sum is an explicit
loop (math.fsum for sums), with no numpy linear algebra, so it is an
independent route to the same numbers as the materialized oracle.

Test infrastructure only.
"""

from __future__ import annotations

import math


def bruteforce_attention(q, k, v, causal, scale):
    """q: nested lists [B][H_q][N_q][d]; k, v: [B][H_kv][N_kv][d].

    Returns (O, LSE) as nested lists. scale is used as given (pass the
    float32-rounded value to match the library)."""
    B = len(q)
    H_q = len(q[0])
    H_kv = len(k[0])
    G = H_q // H_kv
    O = []
    LSE = []
    for b in range(B):
        Ob, Lb = [], []
        for h in range(H_q):
            hk = h // G
            Oh, Lh = [], []
            n_q = len(q[b][h])
            n_kv = len(k[b][hk])
            for i in range(n_q):
                scores = []
                for j in range(n_kv):
                    if causal and j > i:
                        continue
                    dot = math.fsum(q[b][h][i][t] * k[b][hk][j][t] for t in range(len(q[b][h][i])))
                    scores.append((j, scale * dot))
                mx = max(sc for _, sc in scores)
                weights = [(j, math.exp(sc - mx)) for j, sc in scores]
                total = math.fsum(w for _, w in weights)
                dv = len(v[b][hk][0])
                row = [math.fsum(w * v[b][hk][j][t] for j, w in weights) / total for t in range(dv)]
                Oh.append(row)
                Lh.append(mx + math.log(total))
            Ob.append(Oh)
            Lb.append(Lh)
        O.append(Ob)
        LSE.append(Lb)
    return O, LSE

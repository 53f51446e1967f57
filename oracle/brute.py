"""Pure-Python brute-force attention for tiny shapes (test infrastructure only).

Independent of ``oracle.c``: it builds the whole masked score matrix, then
applies the textbook softmax exp(s_ij) / sum_k exp(s_ik) with no max shift
(safe only for the small scores of tiny test shapes), sums with math.fsum,
and returns LSE_i = log(sum_j exp(s_ij)).  Definition as on the
Kernel-Inference-Engine page (softmax(QK^T / sqrt(d)) V, attention-block
chart) with the causal and padding masks of the gpu-inference page
(section 02) and the bottom-right causal alignment j <= i + Nk - Nq.
"""
from __future__ import annotations

import math


def attention(q, k, v, scale, causal=False, kv_len=None):
    """q: Nq x d, k/v: Nk x d nested lists of floats.  Returns (O, LSE) lists."""
    Nq, Nk = len(q), len(k)
    n = Nk if kv_len is None else max(0, min(kv_len, Nk))
    mask = [[(j < n) and (not causal or j <= i + Nk - Nq) for j in range(Nk)]
            for i in range(Nq)]
    S = [[scale * math.fsum(a * b for a, b in zip(q[i], k[j])) for j in range(Nk)]
         for i in range(Nq)]
    O, LSE = [], []
    for i in range(Nq):
        ex = [math.exp(S[i][j]) if mask[i][j] else 0.0 for j in range(Nk)]
        z = math.fsum(ex)
        if z == 0.0:
            O.append([0.0] * len(v[0]) if v else [])
            LSE.append(-math.inf)
            continue
        O.append([math.fsum(ex[j] * v[j][t] for j in range(Nk)) / z
                  for t in range(len(v[0]))])
        LSE.append(math.log(z))
    return O, LSE

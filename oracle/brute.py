"""Pure-Python brute force for tiny inputs (test infrastructure only).

Independent of numpy's BLAS: scalar loops, ``math.exp`` and correctly rounded
``math.fsum``. Attention is written as ordinary multi-head attention where every
head has its own K and V arrays; the caller passes copies of the one shared
K/V head for each of the H heads, which is what sharing a single K and V head
means (Step-3 paper summary, "Key claims": 64 query heads sharing one K and one
V head).
"""

from __future__ import annotations

import math


def matvec_t(x, w):
    """y[n] = sum_k x[k] * w[n][k] for a row vector x and [out, in] matrix w."""
    return [math.fsum(xk * wk for xk, wk in zip(x, row)) for row in w]


def rms_norm(c, eps):
    ms = math.fsum(v * v for v in c) / len(c)
    r = 1.0 / math.sqrt(ms + eps)
    return [v * r for v in c]


def mha(q_heads, k_heads, v_heads, scale):
    """Per head h: softmax(q_h . k_{h,j} * scale)_j weighted sum of v_{h,j}.

    q_heads[h] is a list of D floats; k_heads[h], v_heads[h] are lists of L rows.
    Returns (out[h][d], lse[h]).
    """
    outs, lses = [], []
    for qh, kh, vh in zip(q_heads, k_heads, v_heads):
        if not kh:
            outs.append([0.0] * len(vh[0]) if vh else [])
            lses.append(-math.inf)
            continue
        s = [math.fsum(a * b for a, b in zip(qh, kr)) * scale for kr in kh]
        m = max(s)
        e = [math.exp(v - m) for v in s]
        l = math.fsum(e)
        d = len(vh[0])
        outs.append([math.fsum(e[j] * vh[j][i] for j in range(len(e))) / l for i in range(d)])
        lses.append(m + math.log(l))
    return outs, lses

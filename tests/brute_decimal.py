"""Attention evaluated in 40-digit decimal arithmetic straight from its
definition: s_ij = scale * q_i . k_j, O_i = sum_j e^{s_ij} v_j / sum_j e^{s_ij},
LSE_i = ln sum_j e^{s_ij}, over the allowed keys j <= i + Nk - Nq when causal.
No maximum is subtracted (exact arithmetic does not need it), which makes this
a different computation from the oracle's.  Tiny inputs only."""
from decimal import Decimal, localcontext

import numpy as np


def attention_decimal(q, k, v, causal, scale, digits=40):
    Nq, d = q.shape
    Nk = k.shape[0]
    o = np.zeros((Nq, v.shape[1]))
    lse = np.zeros(Nq)
    with localcontext() as ctx:
        ctx.prec = digits
        sc = Decimal(float(scale))
        for i in range(Nq):
            keys = [j for j in range(Nk) if not causal or j <= i + Nk - Nq]
            if not keys:
                lse[i] = -np.inf
                continue
            w = []
            for j in keys:
                dot = sum(Decimal(float(q[i, c])) * Decimal(float(k[j, c])) for c in range(d))
                w.append((sc * dot).exp())
            z = sum(w)
            for c in range(v.shape[1]):
                o[i, c] = float(sum(wj * Decimal(float(v[j, c])) for wj, j in zip(w, keys)) / z)
            lse[i] = float(z.ln())
    return o, lse

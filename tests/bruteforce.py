"""40-digit decimal brute force of softmax attention, for tiny inputs only.

Written independently of ``oracle/``: every score, exponential, sum and
logarithm is evaluated in ``decimal`` arithmetic at 40 significant digits
from the exact binary values of the inputs, looping over every index.
"""

from __future__ import annotations

from decimal import Decimal, localcontext

import numpy as np


def attention_decimal(q, k, v, scale, causal, window=(-1, -1)):
    """q [B,Lq,Hq,D], k/v [B,Lk,Hkv,D] float arrays -> (O, lse) as float64.

    ``window`` = (left, right): row i sees keys from i + Lk - Lq - left to
    i + Lk - Lq + right (a negative value leaves that side open)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Lq, Hq, D = q.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    grp = Hq // Hkv
    O = np.zeros((B, Lq, Hq, v.shape[3]))
    lse = np.zeros((B, Hq, Lq))
    with localcontext() as ctx:
        ctx.prec = 40
        sc = Decimal(float(scale))
        for b in range(B):
            for h in range(Hq):
                kv = h // grp
                for i in range(Lq):
                    diag = i + Lk - Lq  # the key on this row's diagonal
                    keys = [j for j in range(Lk)
                            if ((not causal) or j <= diag)
                            and (window[0] < 0 or j >= diag - window[0])
                            and (window[1] < 0 or j <= diag + window[1])]
                    if not keys:
                        O[b, i, h, :] = 0.0
                        lse[b, h, i] = -np.inf
                        continue
                    s = {}
                    for j in keys:
                        acc = Decimal(0)
                        for d in range(D):
                            acc += Decimal(float(q[b, i, h, d])) * Decimal(float(k[b, j, kv, d]))
                        s[j] = sc * acc
                    m = max(s.values())
                    e = {j: (s[j] - m).exp() for j in keys}
                    tot = sum(e.values())
                    for d in range(v.shape[3]):
                        num = sum(e[j] * Decimal(float(v[b, j, kv, d])) for j in keys)
                        O[b, i, h, d] = float(num / tot)
                    lse[b, h, i] = float(m + tot.ln())
    return O, lse

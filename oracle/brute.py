"""Scalar pure-Python attention for tiny inputs.

TEST INFRASTRUCTURE ONLY (see the package docstring). A second, loop-only
statement of the same definition as ``paged_attention.attend`` [P1 §04 six
steps], used to cross-check the vectorised oracle on small shapes. It works
on nested Python lists of floats, uses ``math.exp``/``math.log`` and no numpy.
"""

import math


def attend_loops(q, k, v, scale, causal=True):
    """``q[n][Hq][D]``, ``k``/``v[L][Hkv][D]`` -> (out[n][Hq][D], lse[n][Hq])."""
    n = len(q)
    length = len(k)
    hq = len(q[0]) if n else 0
    hkv = len(k[0]) if length else 1
    d = len(q[0][0]) if n else 0
    group = hq // hkv if hkv else 1
    out = [[[0.0] * d for _ in range(hq)] for _ in range(n)]
    lse = [[-math.inf] * hq for _ in range(n)]
    for i in range(n):
        last = (length - n + i) if causal else (length - 1)
        for h in range(hq):
            kvh = h // group
            scores = []
            for t in range(0, last + 1):
                acc = 0.0
                for e in range(d):
                    acc += q[i][h][e] * k[t][kvh][e]
                scores.append(scale * acc)
            if not scores:
                continue
            top = max(scores)
            weights = [math.exp(s - top) for s in scores]
            denom = sum(weights)
            for e in range(d):
                acc = 0.0
                for t, w in enumerate(weights):
                    acc += w * v[t][kvh][e]
                out[i][h][e] = acc / denom
            lse[i][h] = top + math.log(denom)
    return out, lse

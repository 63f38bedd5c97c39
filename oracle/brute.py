"""Scalar pure-Python brute force of RoPE attention -- TEST INFRASTRUCTURE ONLY.

An independent second implementation for tiny inputs: explicit loops over
keys, dimensions and heads with math.cos/math.sin/math.exp, no NumPy.  It
pins oracle.lazy_oracle on small cases (the definitions are those of
"LazyAttention", §3.1 Eq. 4 with RoPE applied to q and k, §3.2 rotation
formula over half-dimensions).
"""
from __future__ import annotations

import math

__all__ = ["brute_attention", "brute_rotate"]


def brute_rotate(vec, pos, base):
    """Rotate one vector (list) to position pos: pair (i, i + D/2) by pos * base^(-2i/D)."""
    D = len(vec)
    h = D // 2
    out = [0.0] * D
    for i in range(h):
        ang = pos * (base ** (-2.0 * i / D))
        c, s = math.cos(ang), math.sin(ang)
        out[i] = vec[i] * c - vec[i + h] * s
        out[i + h] = vec[i] * s + vec[i + h] * c
    return out


def brute_attention(queries, keys, scale, base):
    """queries: list of (qvec, qpos); keys: list of (kvec, vvec, kpos, causal).

    A key marked causal is visible to a query only when kpos <= qpos.
    Returns list of (out vector, lse) per query.
    """
    res = []
    for qv, qp in queries:
        qr = brute_rotate(qv, qp, base)
        scores, vals = [], []
        for kv, vv, kp, causal in keys:
            if causal and kp > qp:
                continue
            kr = brute_rotate(kv, kp, base)
            dot = 0.0
            for a, b in zip(qr, kr):
                dot += a * b
            scores.append(scale * dot)
            vals.append(vv)
        mx = max(scores)
        ws = [math.exp(s - mx) for s in scores]
        z = sum(ws)
        D = len(vals[0])
        out = [0.0] * D
        for w, vv in zip(ws, vals):
            for d in range(D):
                out[d] += w * vv[d]
        res.append(([o / z for o in out], mx + math.log(z)))
    return res

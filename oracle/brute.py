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


def brute_rotate(vec, pos, base, interleaved=False):
    """Rotate one vector (list) to position pos.

    Pair i -- (i, i + D/2), or (2i, 2i + 1) when interleaved -- turns by
    pos * base^(-2i/D).
    """
    D = len(vec)
    h = D // 2
    out = [0.0] * D
    for i in range(h):
        ang = pos * (base ** (-2.0 * i / D))
        c, s = math.cos(ang), math.sin(ang)
        a, b = (2 * i, 2 * i + 1) if interleaved else (i, i + h)
        out[a] = vec[a] * c - vec[b] * s
        out[b] = vec[a] * s + vec[b] * c
    return out


def brute_attention(queries, keys, scale, base, interleaved=False, alibi_slope=None):
    """queries: list of (qvec, qpos); keys: list of (kvec, vvec, kpos, causal).

    A key marked causal is visible to a query only when kpos <= qpos.  With
    alibi_slope set, no rotation is applied and slope * (kpos - qpos) is added
    to each score.  Returns list of (out vector, lse) per query.
    """
    res = []
    for qv, qp in queries:
        qr = qv if alibi_slope is not None else brute_rotate(qv, qp, base, interleaved)
        scores, vals = [], []
        for kv, vv, kp, causal in keys:
            if causal and kp > qp:
                continue
            kr = kv if alibi_slope is not None else brute_rotate(kv, kp, base, interleaved)
            dot = 0.0
            for a, b in zip(qr, kr):
                dot += a * b
            sc = scale * dot
            if alibi_slope is not None:
                sc += alibi_slope * (kp - qp)
            scores.append(sc)
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

"""Plain float64 oracle of attention over a position-free paged KV pool.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and
bench.py's cpu_baseline leg, never by the product path.

What it computes.  LazyAttention (§1, §3.1 "Deferred encoding") stores keys
and values without positions and claims results identical to eagerly
re-encoding the cache at each request's positions.  The oracle therefore
computes the plain definition: it *materialises* the re-encoded keys
R_p k for every key at its logical position p, rotates the query to its own
position, and runs textbook softmax attention (§3.1 Eq. 4 with RoPE applied to
Q and K).  Nothing is tiled, fused or reordered.

Readings of the pages (listed with reasons in the design notes):
  * RoPE pairs dimension i with i + D/2 (the "half-dimension" K1/K2 split of
    §3.2 "Prefilling" and the Fig. 3 caption), rotating by +p*theta_i as in
    the §3.2 rotation formula k1' = k1 cos - k2 sin, k2' = k1 sin + k2 cos;
  * theta_i = base^(-2i/D), i < D/2 (the frequencies are never printed; the
    pages write the angle as m*theta_i in App. C.4);
  * scale 1/sqrt(D) multiplies the rotated q.k (Eq. 4);
  * GQA: query head h reads kv head floor(h / G) (§3.5 "GQA/MQA");
  * decode attends exactly the listed segments; prefill sees every cached
    key and, among the new tokens, keys at positions <= the query's;
  * a document-local pool (§3.2 "Prefilling": each document's cache indexed
    from position 0; Example 3.1) holds R_t k for token t of a segment, so
    its encoding at logical position s + t is R_s applied to what is stored
    (R_s R_t = R_{s+t}); the oracle re-encodes stored keys that way.

Inputs are the exact values handed to the GPU: bf16 pools/queries arrive as
uint16 bit patterns and are widened exactly to float64 here.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "rope_theta",
    "rope_rotate",
    "alibi_slopes",
    "rope_theta_scaled",
    "gather_request",
    "attention_decode",
    "attention_prefill",
    "attention_decode_relative",
    "store_kv",
    "run_decode",
    "run_prefill",
]


def _as_f64(a) -> np.ndarray:
    """Widen float or bf16-bit (uint16) arrays to float64 exactly."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def rope_theta(head_dim: int, base: float) -> np.ndarray:
    """RoPE frequencies theta_i = base^(-2i/D), i = 0 .. D/2-1, in float64.

    Pin: the identity table (theta = 0) special case and the textbook causal
    RoPE attention special case in tests/test_oracle.py.
    """
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / float(head_dim))


def rope_rotate(x, pos, theta, pairing: str = "half", amp: float = 1.0) -> np.ndarray:
    """Rotate x[..., D] to position(s) pos (broadcast over leading axes).

    pairing="half": pair (i, i+D/2) is rotated by angle pos*theta_i:
      y_i = x_i cos - x_{i+D/2} sin,   y_{i+D/2} = x_i sin + x_{i+D/2} cos
    (§3.2 "Prefilling", the relative-rotation formula with the offset taken
    as the absolute position).  pairing="interleaved": the same rotation on
    the adjacent pair (2i, 2i+1), the interleaved RoPE of §3.5.

    Pins: equals multiplication of x_i + j x_{i+D/2} (interleaved:
    x_{2i} + j x_{2i+1}) by exp(j pos theta_i) (RoPE's complex form, computed
    with numpy complex arithmetic); Fact 3.2 (R_m q).(R_n k) = q.R_{n-m} k;
    norm preservation; rot(x, 0) = x.  amp scales cos and sin alike (the
    attention factor of YaRN tables).
    """
    x = np.asarray(x, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.float64)
    ang = pos[..., None] * np.asarray(theta, dtype=np.float64)
    c, s = amp * np.cos(ang), amp * np.sin(ang)
    if pairing == "interleaved":
        x1, x2 = x[..., 0::2], x[..., 1::2]
        y = np.empty(np.broadcast_shapes(x.shape, ang.shape[:-1] + (x.shape[-1],)))
        y[..., 0::2] = x1 * c - x2 * s
        y[..., 1::2] = x1 * s + x2 * c
        return y
    if pairing != "half":
        raise ValueError(f"unknown pairing {pairing!r}")
    half = x.shape[-1] // 2
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def rope_theta_scaled(head_dim: int, base: float, scaling=None):
    """Frequencies and amplitude of the scaled RoPE variants of §3.5.

    The paper only says that scaled / NTK / YaRN variants keep the score
    q^T R_{n-m} k with variant-specific metadata; the variants themselves are
    the published ones, restated here (float64):
      linear  (position interpolation): theta_i / s;
      ntk     (NTK-aware): base' = base * s^(D / (D - 2));
      yarn:   per pair, wavelength-dependent blend of theta_i (fast pairs) and
              theta_i / s (slow pairs) over a linear ramp between the pair
              indices where the rotation count over the original context is
              beta_fast (rounded down) and beta_slow (rounded up, clamped to
              D - 1 as in the published correction range); cos and sin scaled
              by the attention factor (default 0.1 ln s + 1);
      llama3: wavelength 2 pi / theta_i below L/high_freq_factor kept, above
              L/low_freq_factor divided by s, smooth blend in between.
    scaling: None or a dict with "type" and the parameters above
    (factor, original_max_pos, beta_fast, beta_slow, attn_factor,
    low_freq_factor, high_freq_factor).  Returns (theta [D/2], amplitude).

    Pins (tests/test_oracle.py): factor 1 is the plain table for every type;
    linear scaling maps positions (s m, s n) to the plain scores at (m, n);
    NTK keeps the fastest pair and divides the slowest by s; YaRN and llama3
    keep fast pairs, divide slow pairs by s and are monotone between; YaRN's
    amplitude at s = e is 1.1; the exact ramp ends lo = 40, hi = 65 and the
    resulting frequencies at D = 128, base 1e4, original context 65536, where
    the D - 1 clamp matters (hi > D/2 - 1).
    """
    theta = rope_theta(head_dim, base)
    if scaling is None or scaling.get("type", "none") == "none":
        return theta, 1.0
    kind = scaling["type"]
    f = float(scaling["factor"])
    D = head_dim
    if kind == "linear":
        return theta / f, 1.0
    if kind == "ntk":
        return rope_theta(D, base * f ** (D / (D - 2.0))), 1.0
    if kind == "yarn":
        L = float(scaling["original_max_pos"])
        bf, bs = float(scaling.get("beta_fast", 32.0)), float(scaling.get("beta_slow", 1.0))

        def pair_index(rotations):  # pair whose rotations over L equal `rotations`
            return D * np.log(L / (rotations * 2.0 * np.pi)) / (2.0 * np.log(base))

        # The published correction range: floor / ceil of the two fractional
        # pair indices, clamped to [0, D - 1] (an upper bound above the last
        # pair index D/2 - 1: when it binds, the ramp over the D/2 pairs stops
        # short of 1 and the slowest pairs are only partly interpolated).
        lo = max(np.floor(pair_index(bf)), 0.0)
        hi = min(np.ceil(pair_index(bs)), D - 1.0)
        if lo == hi:
            hi += 0.001
        ramp = np.clip((np.arange(D // 2) - lo) / (hi - lo), 0.0, 1.0)
        th = theta / f * ramp + theta * (1.0 - ramp)
        af = float(scaling.get("attn_factor", 0.0)) or (0.1 * np.log(f) + 1.0 if f > 1 else 1.0)
        return th, af
    if kind == "llama3":
        L = float(scaling["original_max_pos"])
        lo_f, hi_f = float(scaling["low_freq_factor"]), float(scaling["high_freq_factor"])
        wl = 2.0 * np.pi / theta
        smooth = np.clip((L / wl - lo_f) / (hi_f - lo_f), 0.0, 1.0)
        th = np.where(wl < L / hi_f, theta,
                      np.where(wl > L / lo_f, theta / f, (1 - smooth) * theta / f + smooth * theta))
        return th, 1.0
    raise ValueError(f"unknown RoPE scaling {kind!r}")


def alibi_slopes(num_heads: int) -> np.ndarray:
    """ALiBi head slopes (the score-space method of §3.5, published rule).

    For n a power of two the slopes are the geometric sequence
    2^(-8/n), 2^(-16/n), ..., 2^(-8); otherwise the n' = 2^floor(log2 n)
    sequence is followed by every other slope of the 2n' sequence.
    Pins: n = 8 gives 1/2, 1/4, ..., 1/256; the first values for n = 12.
    """
    def pow2(n):
        start = 2.0 ** (-8.0 / n)
        return [start ** (i + 1) for i in range(n)]
    n = int(num_heads)
    p = 1 << (n.bit_length() - 1)
    if p == n:
        return np.array(pow2(n))
    return np.array(pow2(p) + pow2(2 * p)[0::2][: n - p])


def gather_request(k_pool, v_pool, segments, block_size: int, kv_head: int):
    """Collect one request's keys/values for one kv head, in table order.

    Token t of a segment starting at s lives in block blocks[t // BS], slot
    t % BS, at logical position s + t.  Returns (K [n, D], V [n, D] float64,
    positions [n] int64, is_new [n] bool).
    """
    ks, vs, ps, ns = [], [], [], []
    for seg in segments:
        n = int(seg.n_tokens)
        if n == 0:
            continue
        t = np.arange(n)
        blk = np.asarray(seg.blocks, dtype=np.int64)[t // block_size]
        slot = t % block_size
        ks.append(_as_f64(k_pool[blk, kv_head, slot, :]))
        vs.append(_as_f64(v_pool[blk, kv_head, slot, :]))
        ps.append(int(seg.start) + t)
        ns.append(np.full(n, bool(seg.is_new)))
    if not ks:
        D = k_pool.shape[-1]
        return (np.zeros((0, D)), np.zeros((0, D)), np.zeros(0, np.int64), np.zeros(0, bool))
    return np.concatenate(ks), np.concatenate(vs), np.concatenate(ps), np.concatenate(ns)


def _segment_starts(segments) -> np.ndarray:
    """Logical start s of the segment of every gathered key, in gather order."""
    parts = [np.full(int(seg.n_tokens), int(seg.start), np.int64) for seg in segments
             if int(seg.n_tokens) > 0]
    return np.concatenate(parts) if parts else np.zeros(0, np.int64)


def _encode_keys(K, pos, segments, theta, doc_local, pairing="half", amp=1.0):
    """Keys encoded at their logical positions.

    Position-free pool: R_p k (with the table's amplitude amp).
    Document-local pool (stored amp R_t k, written with the same table): the
    pure rotation by s = the segment's start of the stored key, which is
    amp R_{s+t} k -- the amplitude is already in the stored key, so a scaled
    table's attention factor is applied once per key either way.
    """
    if doc_local:
        return rope_rotate(K, _segment_starts(segments), theta, pairing)
    return rope_rotate(K, pos, theta, pairing, amp)


def store_kv(k, v, slots, rope_pos, k_pool, v_pool, *, block_size, theta, pairing="half",
             amp=1.0):
    """The cache write: new tokens' keys and values into pool slots.

    Token n goes to block slots[n] // BS, slot slots[n] % BS; its key is
    stored as given (rope_pos None: the position-free pool of §3.1 "Deferred
    encoding") or rotated to rope_pos[n] (R_p k; p = the index inside its
    document for a document-local pool, §3.2 "Prefilling"), its value as
    given.  Returns float64 copies of the logical [nb, Hkv, BS, D] pools;
    slots not listed keep their old contents.  With interleaved pairing the
    key is rotated on pairs (2i, 2i+1) and then stored with its dimensions in
    the order (even dims, odd dims) -- the storage order of such pools, which
    turns each pair back into (i, i + D/2).  amp is the amplitude of a scaled
    table's rows (its cos and sin both carry it), applied with the rotation.

    Pins: rope_pos None is an exact copy; a rotated key equals the complex
    product x * exp(j p theta) and keeps its norm; Example 3.1 through
    attention (tests/test_oracle.py).
    """
    kp = _as_f64(k_pool).copy()
    vp = _as_f64(v_pool).copy()
    kf, vf = _as_f64(k), _as_f64(v)
    slots = np.asarray(slots, np.int64)
    blk, sl = slots // block_size, slots % block_size
    if rope_pos is not None:
        kf = rope_rotate(kf, np.asarray(rope_pos, np.int64)[:, None], theta, pairing, amp)
    if pairing == "interleaved":
        kf = np.concatenate([kf[..., 0::2], kf[..., 1::2]], axis=-1)
    kp[blk, :, sl, :] = kf
    vp[blk, :, sl, :] = vf
    return kp, vp


def _softmax_attend(scores: np.ndarray, V: np.ndarray):
    """Textbook softmax over the last axis (Eq. 4), returning (out, lse)."""
    if scores.shape[-1] == 0:
        raise ValueError("attention over zero keys is undefined")
    mx = np.max(scores, axis=-1, keepdims=True)
    if not np.all(np.isfinite(mx)):
        raise ValueError("a query row sees no key (fully masked)")
    e = np.exp(scores - mx)
    z = np.sum(e, axis=-1, keepdims=True)
    out = (e @ V) / z
    lse = (mx + np.log(z))[..., 0]
    return out, lse


def attention_decode(q, q_pos, segments, k_pool, v_pool, *, block_size, num_kv_heads,
                     theta, scale, rotate=True, doc_local=False, pairing="half",
                     alibi=None, amp=1.0):
    """One decode query (all heads) of one request, eager RoPE.

    q: [Hq, D]; q_pos: the query's logical position m.  Keys are gathered,
    re-encoded at their positions (the materialised cache the method avoids)
    and attended with textbook softmax.  Returns out [Hq, D], lse [Hq].
    rotate=False drops RoPE entirely (used by the identity-table pin);
    doc_local=True reads a document-local pool (stored keys R_t k);
    pairing selects the RoPE pairs (see rope_rotate).  alibi, an array of Hq
    slopes, replaces RoPE by the ALiBi score bias slope_h * (p - m) (§3.5
    "Score-space positional methods"; -slope times the distance for keys at
    or before the query).  amp is the cos/sin amplitude of a scaled table.
    """
    qf = _as_f64(q)
    Hq, D = qf.shape
    G = Hq // num_kv_heads
    out = np.empty((Hq, D))
    lse = np.empty(Hq)
    for g in range(num_kv_heads):
        K, V, pos, _ = gather_request(k_pool, v_pool, segments, block_size, g)
        qs = qf[g * G:(g + 1) * G]
        if rotate and alibi is None:
            Kt = _encode_keys(K, pos, segments, theta, doc_local, pairing, amp)
            qt = rope_rotate(qs, np.full(G, q_pos), theta, pairing, amp)
        else:
            Kt, qt = K, qs
        s = scale * (qt @ Kt.T)
        if alibi is not None:
            sl = np.asarray(alibi, np.float64)[g * G:(g + 1) * G]
            s = s + sl[:, None] * (pos[None, :] - float(q_pos))
        o, l = _softmax_attend(s, V)
        out[g * G:(g + 1) * G] = o
        lse[g * G:(g + 1) * G] = l
    return out, lse


def attention_decode_relative(q, q_pos, segments, k_pool, v_pool, *, block_size, num_kv_heads,
                              theta, scale):
    """Same decode query, computed the lazy way on the un-rotated pool.

    Each score is scale * q^T R_{p-m} k (Fact 3.2, §3.2): only the relative
    offset p - m is applied, to the stored key; the query stays un-rotated.
    Pin: must equal attention_decode (eager) to 1e-12.
    """
    qf = _as_f64(q)
    Hq, D = qf.shape
    G = Hq // num_kv_heads
    out = np.empty((Hq, D))
    lse = np.empty(Hq)
    for g in range(num_kv_heads):
        K, V, pos, _ = gather_request(k_pool, v_pool, segments, block_size, g)
        Kr = rope_rotate(K, pos - int(q_pos), theta)
        s = scale * (qf[g * G:(g + 1) * G] @ Kr.T)
        o, l = _softmax_attend(s, V)
        out[g * G:(g + 1) * G] = o
        lse[g * G:(g + 1) * G] = l
    return out, lse


def attention_prefill(q, q_pos0, segments, k_pool, v_pool, *, block_size, num_kv_heads,
                      theta, scale, rotate=True, rows=None, doc_local=False, pairing="half",
                      alibi=None, amp=1.0):
    """New-token attention of one request, eager RoPE.

    q: [T, Hq, D]; new token j sits at position q_pos0 + j.  Keys of cached
    segments are all visible; keys of the new-token segment are visible iff
    their position is <= the query's.  rows optionally restricts the query
    rows computed (sampled parity).  Returns out [T', Hq, D], lse [T', Hq].
    doc_local=True reads a document-local pool (stored keys R_t k);
    pairing, alibi and amp as for attention_decode.
    """
    qf = _as_f64(q)
    T, Hq, D = qf.shape
    G = Hq // num_kv_heads
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    qpos = int(q_pos0) + rows
    out = np.empty((len(rows), Hq, D))
    lse = np.empty((len(rows), Hq))
    for g in range(num_kv_heads):
        K, V, pos, new = gather_request(k_pool, v_pool, segments, block_size, g)
        use_rope = rotate and alibi is None
        Kt = _encode_keys(K, pos, segments, theta, doc_local, pairing, amp) if use_rope else K
        visible = (~new)[None, :] | (pos[None, :] <= qpos[:, None])  # [T', n]
        for hh in range(G):
            h = g * G + hh
            qs = qf[rows, h, :]
            qt = rope_rotate(qs, qpos, theta, pairing, amp) if use_rope else qs
            s = scale * (qt @ Kt.T)
            if alibi is not None:
                s = s + float(alibi[h]) * (pos[None, :] - qpos[:, None])
            s = np.where(visible, s, -np.inf)
            o, l = _softmax_attend(s, V)
            out[:, h, :] = o
            lse[:, h] = l
    return out, lse


def run_decode(w, requests=None, rotate=True, pools=None, doc_local=False, pairing="half",
               alibi=None, scaling=None):
    """Oracle outputs for decode workload w: {r: (out [Hq, D], lse [Hq])}.

    pools, if given, replaces (w.k_pool, w.v_pool), e.g. by a document-local
    pool written with store_kv (then doc_local=True).  pairing / alibi select
    the positional encoding (see attention_decode); scaling a scaled RoPE
    table (see rope_theta_scaled).
    """
    th, amp = rope_theta_scaled(w.head_dim, w.rope_base, scaling)
    kp, vp = (w.k_pool, w.v_pool) if pools is None else pools
    reqs = range(w.batch) if requests is None else requests
    res = {}
    for r in reqs:
        res[r] = attention_decode(w.q[r], int(w.q_pos[r]), w.requests[r], kp, vp,
                                  block_size=w.block_size, num_kv_heads=w.num_kv_heads,
                                  theta=th, scale=w.scale, rotate=rotate, doc_local=doc_local,
                                  pairing=pairing, alibi=alibi, amp=amp)
    return res


def run_prefill(w, requests=None, rows=None, rotate=True, pools=None, doc_local=False,
                pairing="half", alibi=None, scaling=None):
    """Oracle outputs for prefill workload w: {r: (out [T', Hq, D], lse [T', Hq])}.

    rows, if given, maps request -> array of new-token indices to compute;
    pools / doc_local / pairing / alibi / scaling as for run_decode.
    """
    th, amp = rope_theta_scaled(w.head_dim, w.rope_base, scaling)
    kp, vp = (w.k_pool, w.v_pool) if pools is None else pools
    reqs = range(w.batch) if requests is None else requests
    res = {}
    for r in reqs:
        a, b = int(w.cu_q[r]), int(w.cu_q[r + 1])
        rr = None if rows is None else rows.get(r)
        res[r] = attention_prefill(w.q[a:b], int(w.q_pos[r]), w.requests[r], kp, vp,
                                   block_size=w.block_size, num_kv_heads=w.num_kv_heads,
                                   theta=th, scale=w.scale, rotate=rotate, rows=rr,
                                   doc_local=doc_local, pairing=pairing, alibi=alibi,
                                   amp=amp)
    return res

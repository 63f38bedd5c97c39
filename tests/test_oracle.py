"""Pins of the CPU oracle against what the LazyAttention paper and mathematics fix.

Every check here is independent of the oracle's own formulas: RoPE's complex
form, torch's scaled_dot_product_attention (float64, CPU), scipy's Hurwitz
zeta, closed forms of softmax, a pure-Python brute force, invariances the
paper states (Fact 3.2 and the shift invariance it implies, zero-copy reuse),
and the numbers the paper prints.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import (
    attention_decode,
    attention_decode_relative,
    attention_prefill,
    decode_trigger_overhead,
    hit_ratio_gap,
    naive_flops_overhead,
    naive_io_overhead,
    prefill_flops_overhead,
    prefill_table_bandwidth,
    rope_rotate,
    rope_theta,
    run_decode,
    run_prefill,
)
from oracle.analysis import zipf_partial_sum
from oracle.brute import brute_attention
from workloads import Segment, bf16_bits_to_f32, build_workload, make_config

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "paper_figures.json")
RNG = np.random.default_rng(7)


def _tiny(kind="decode", dtype="bf16", Hq=4, Hkv=2, D=16, BS=4, base=1e4, requests=None,
          doc_lens=(7, 9, 4, 12), seed=3, poison=False):
    if requests is None:
        if kind == "decode":
            requests = [[("doc", 0), ("doc", 1), ("priv", 3)],
                        [("doc", 1), ("doc", 2), ("doc", 0, 40)],
                        [("doc", 3), ("doc", 1), ("doc", 3, 100)]]
        else:
            requests = [[("doc", 0), ("doc", 2), ("new", 6)],
                        [("doc", 3), ("doc", 0), ("new", 9)]]
    return build_workload(name="tiny", kind=kind, dtype=dtype, num_q_heads=Hq, num_kv_heads=Hkv,
                          head_dim=D, block_size=BS, rope_base=base, doc_lens=list(doc_lens),
                          requests=requests, seed=seed, poison_tail=poison)


# ---------------------------------------------------------------- rotation
def test_rotation_is_complex_multiplication():
    """rot(x, p) pairs (i, i+D/2) like x_i + j x_{i+D/2} multiplied by e^{j p theta_i}."""
    D = 64
    th = rope_theta(D, 1e4)
    # Textbook RoPE frequencies, written independently: base^(-(0,2,4,..)/D).
    th_ref = 1.0 / (1e4 ** (np.arange(0, D, 2, dtype=np.float64) / D))
    np.testing.assert_allclose(th, th_ref, rtol=1e-15)
    x = RNG.standard_normal((5, D))
    pos = np.array([0, 1, 17, 4096, 131071])
    z = (x[:, : D // 2] + 1j * x[:, D // 2:]) * np.exp(1j * pos[:, None] * th_ref[None, :])
    ref = np.concatenate([z.real, z.imag], axis=1)
    # complex exp and cos/sin round large angles (~1.3e5 rad) differently: ~1e-11
    np.testing.assert_allclose(rope_rotate(x, pos, th), ref, rtol=0, atol=1e-10)
    np.testing.assert_allclose(rope_rotate(x[:3], pos[:3], th), ref[:3], rtol=0, atol=1e-13)


def test_rotation_group_properties():
    D = 128
    th = rope_theta(D, 5e5)
    x = RNG.standard_normal((3, D))
    np.testing.assert_array_equal(rope_rotate(x, np.zeros(3), th), x)
    for p in (1, 333, 65536):
        y = rope_rotate(x, np.full(3, p), th)
        np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    a, b = 1234, 4321
    np.testing.assert_allclose(rope_rotate(rope_rotate(x, np.full(3, a), th), np.full(3, b), th),
                               rope_rotate(x, np.full(3, a + b), th), atol=1e-10)


@pytest.mark.parametrize("m,n", [(0, 5), (160, 3), (5184, 17), (131071, 65536), (7, 130000)])
def test_fact_3_2_relative_rotation(m, n):
    """(R_m q)^T (R_n k) = q^T R_{n-m} k  (LazyAttention §3.2, Fact 3.2)."""
    D = 128
    th = rope_theta(D, 5e5)
    q = RNG.standard_normal(D)
    k = RNG.standard_normal(D)
    lhs = rope_rotate(q, m, th) @ rope_rotate(k, n, th)
    rhs = q @ rope_rotate(k, n - m, th)
    # angles reach ~1.3e5 rad; fp64 rounding of p*theta bounds the agreement
    tol = 1e-12 if max(m, n) < 1000 else 1e-8
    assert abs(lhs - rhs) <= tol * (1 + abs(lhs))


# ------------------------------------------------------- lazy equals eager
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_lazy_equals_eager(dtype):
    """The un-rotated pool + relative rotation equals the re-encoded cache (§1, §3.1)."""
    w = _tiny(dtype=dtype)
    th = rope_theta(w.head_dim, w.rope_base)
    for r in range(w.batch):
        kw = dict(block_size=w.block_size, num_kv_heads=w.num_kv_heads, theta=th, scale=w.scale)
        o1, l1 = attention_decode(w.q[r], int(w.q_pos[r]), w.requests[r], w.k_pool, w.v_pool, **kw)
        o2, l2 = attention_decode_relative(w.q[r], int(w.q_pos[r]), w.requests[r], w.k_pool,
                                           w.v_pool, **kw)
        np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)


def _shifted(segs, c):
    return [Segment(s.start + c, s.n_tokens, s.blocks, s.is_new) for s in segs]


@pytest.mark.parametrize("c", [1, 777, 60000])
def test_shift_invariance(c):
    """Moving every position by a constant leaves all scores unchanged (Fact 3.2)."""
    w = _tiny()
    th = rope_theta(w.head_dim, w.rope_base)
    kw = dict(block_size=w.block_size, num_kv_heads=w.num_kv_heads, theta=th, scale=w.scale)
    for r in range(w.batch):
        o1, l1 = attention_decode(w.q[r], int(w.q_pos[r]), w.requests[r], w.k_pool, w.v_pool, **kw)
        o2, l2 = attention_decode(w.q[r], int(w.q_pos[r]) + c, _shifted(w.requests[r], c),
                                  w.k_pool, w.v_pool, **kw)
        np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-10)
    wp = _tiny(kind="prefill")
    for r in range(wp.batch):
        a, b = wp.cu_q[r], wp.cu_q[r + 1]
        kw2 = dict(block_size=wp.block_size, num_kv_heads=wp.num_kv_heads, theta=th, scale=wp.scale)
        o1, _ = attention_prefill(wp.q[a:b], int(wp.q_pos[r]), wp.requests[r], wp.k_pool, wp.v_pool, **kw2)
        o2, _ = attention_prefill(wp.q[a:b], int(wp.q_pos[r]) + c, _shifted(wp.requests[r], c),
                                  wp.k_pool, wp.v_pool, **kw2)
        np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-10)


# ------------------------------------------- special cases = library routine
def _sdpa(q, k, v, causal=False, mask=None):
    """torch SDPA in float64 on CPU; q [Hq, T, D], k/v [Hkv, n, D]; GQA by torch."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))[None]
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=m,
                                                         is_causal=causal, enable_gqa=True)
    return o[0].numpy()


def _gathered_by_test(w, r, g):
    """Independent gather for the test: walk the request token by token."""
    ks, vs = [], []
    for s in w.requests[r]:
        for t in range(s.n_tokens):
            b = int(s.blocks[t // w.block_size])
            ks.append(w.values_f32(w.k_pool[b, g, t % w.block_size]))
            vs.append(w.values_f32(w.v_pool[b, g, t % w.block_size]))
    return np.array(ks, np.float64), np.array(vs, np.float64)


def test_identity_table_is_textbook_attention():
    """With no rotation (theta = 0) the result is softmax(q K^T / sqrt(D)) V with GQA."""
    w = _tiny(Hq=6, Hkv=2)
    zero = np.zeros(w.head_dim // 2)
    for r in range(w.batch):
        o, _ = attention_decode(w.q[r], int(w.q_pos[r]), w.requests[r], w.k_pool, w.v_pool,
                                block_size=w.block_size, num_kv_heads=w.num_kv_heads,
                                theta=zero, scale=w.scale)
        K = np.stack([_gathered_by_test(w, r, g)[0] for g in range(w.num_kv_heads)])
        V = np.stack([_gathered_by_test(w, r, g)[1] for g in range(w.num_kv_heads)])
        q = w.values_f32(w.q[r]).astype(np.float64)[:, None, :]
        ref = _sdpa(q, K, V)[:, 0, :]
        np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def _rope_complex(x, pos, base):
    D = x.shape[-1]
    inv = 1.0 / (base ** (np.arange(0, D, 2, dtype=np.float64) / D))
    z = (x[..., : D // 2] + 1j * x[..., D // 2:]) * np.exp(1j * pos[:, None] * inv[None, :])
    return np.concatenate([z.real, z.imag], axis=-1)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_contiguous_placement_is_causal_rope_attention(dtype):
    """One request tiling [0, L) is standard causal RoPE attention over the sequence.

    The test writes a contiguous key/value sequence into randomly permuted pool
    blocks itself, so a wrong block/slot mapping in the oracle fails here.
    """
    Hq, Hkv, D, BS, base = 4, 2, 32, 4, 1e4
    doc_lens, new = [10, 8, 5], 7
    L = sum(doc_lens) + new
    rng = np.random.default_rng(11)
    Kseq = rng.standard_normal((Hkv, L, D)).astype(np.float32)
    Vseq = rng.standard_normal((Hkv, L, D)).astype(np.float32)
    Qseq = rng.standard_normal((Hq, L, D)).astype(np.float32)
    # scatter into permuted blocks
    seg_lens = doc_lens + [new]
    nblk = sum((n + BS - 1) // BS for n in seg_lens)
    perm = rng.permutation(nblk + 3)[:nblk]
    kpool = np.zeros((nblk + 3, Hkv, BS, D), np.float32)
    vpool = np.zeros_like(kpool)
    segs, cur, bi = [], 0, 0
    for i, n in enumerate(seg_lens):
        nb = (n + BS - 1) // BS
        blocks = perm[bi:bi + nb]
        for t in range(n):
            kpool[blocks[t // BS], :, t % BS] = Kseq[:, cur + t]
            vpool[blocks[t // BS], :, t % BS] = Vseq[:, cur + t]
        segs.append(Segment(cur, n, blocks, i == len(seg_lens) - 1))
        cur += n
        bi += nb
    pos = np.arange(L, dtype=np.float64)
    Qr = _rope_complex(Qseq.astype(np.float64), pos, base)
    Kr = _rope_complex(Kseq.astype(np.float64), pos, base)
    full = _sdpa(Qr, Kr, Vseq, causal=True)  # [Hq, L, D]
    th = rope_theta(D, base)
    q_new = np.transpose(Qseq[:, L - new:, :], (1, 0, 2))  # [T, Hq, D]
    o, _ = attention_prefill(q_new, L - new, segs, kpool, vpool, block_size=BS,
                             num_kv_heads=Hkv, theta=th, scale=1 / math.sqrt(D))
    np.testing.assert_allclose(o, np.transpose(full[:, L - new:, :], (1, 0, 2)), rtol=0, atol=1e-12)
    # decode: one more query at position L attends exactly the L listed keys
    qd = rng.standard_normal((Hq, D)).astype(np.float32)
    qdr = _rope_complex(qd.astype(np.float64)[:, None, :], np.array([float(L)]), base)
    ref = _sdpa(qdr, Kr, Vseq)[:, 0, :]
    od, _ = attention_decode(qd, L, [Segment(s.start, s.n_tokens, s.blocks, False) for s in segs],
                             kpool, vpool, block_size=BS, num_kv_heads=Hkv, theta=th,
                             scale=1 / math.sqrt(D))
    np.testing.assert_allclose(od, ref, rtol=0, atol=1e-12)


# ------------------------------------------------------ softmax closed forms
def test_single_key_returns_its_value():
    D, BS = 8, 4
    kp = RNG.standard_normal((1, 1, BS, D)).astype(np.float32)
    vp = RNG.standard_normal((1, 1, BS, D)).astype(np.float32)
    q = RNG.standard_normal((1, D)).astype(np.float32)
    th = rope_theta(D, 1e4)
    o, l = attention_decode(q, 9, [Segment(5, 1, np.array([0]), False)], kp, vp, block_size=BS,
                            num_kv_heads=1, theta=th, scale=0.5)
    np.testing.assert_allclose(o[0], vp[0, 0, 0], atol=1e-15)
    # lse of one key is its score: 0.5 * q^T R_{5-9} k (complex-form rotation, relative)
    qk = _rope_complex(q.astype(np.float64), np.array([9.0]), 1e4) @ \
        _rope_complex(kp[0, 0, :1].astype(np.float64), np.array([5.0]), 1e4).T
    assert abs(l[0] - 0.5 * qk[0, 0]) < 1e-12


def test_zero_keys_average_values():
    D, BS, n = 8, 4, 11
    kp = np.zeros((3, 1, BS, D), np.float32)
    vp = RNG.standard_normal((3, 1, BS, D)).astype(np.float32)
    q = RNG.standard_normal((1, D)).astype(np.float32)
    th = rope_theta(D, 1e4)
    o, l = attention_decode(q, 40, [Segment(0, n, np.array([2, 0, 1]), False)], kp, vp,
                            block_size=BS, num_kv_heads=1, theta=th, scale=1.0)
    vals = np.concatenate([vp[2, 0], vp[0, 0], vp[1, 0]])[:n].astype(np.float64)
    np.testing.assert_allclose(o[0], vals.mean(axis=0), atol=1e-14)
    assert abs(l[0] - math.log(n)) < 1e-14


def test_dominant_score_selects_value():
    D, BS = 8, 4
    kp = np.zeros((2, 1, BS, D), np.float32)
    vp = RNG.standard_normal((2, 1, BS, D)).astype(np.float32)
    kp[1, 0, 2, 0] = 1.0
    q = np.zeros((1, D), np.float32)
    q[0, 0] = 1.0
    th = np.zeros(D // 2)  # identity rotation: the score of key (1,2) is 1e4 * 1
    o, _ = attention_decode(q, 8, [Segment(0, 8, np.array([0, 1]), False)], kp, vp,
                            block_size=BS, num_kv_heads=1, theta=th, scale=1e4)
    np.testing.assert_allclose(o[0], vp[1, 0, 2], atol=1e-12)


# ------------------------------------------------------------ brute force
def _brute_case(w, r, qrows=None):
    out = []
    for h in range(w.num_q_heads):
        g = h // w.group
        keys = []
        for s in w.requests[r]:
            for t in range(s.n_tokens):
                b = int(s.blocks[t // w.block_size])
                keys.append((w.values_f32(w.k_pool[b, g, t % w.block_size]).tolist(),
                             w.values_f32(w.v_pool[b, g, t % w.block_size]).tolist(),
                             s.start + t, s.is_new))
        if w.kind == "decode":
            qs = [(w.values_f32(w.q[r, h]).tolist(), int(w.q_pos[r]))]
        else:
            a = int(w.cu_q[r])
            qs = [(w.values_f32(w.q[a + j, h]).tolist(), int(w.q_pos[r]) + j)
                  for j in range(w.q_len(r))]
        out.append(brute_attention(qs, keys, w.scale, w.rope_base))
    return out


def test_brute_force_config1():
    w = make_config(1)
    ref = _brute_case(w, 0)
    o, l = run_decode(w)[0]
    np.testing.assert_allclose(o[0], ref[0][0][0], atol=1e-12)
    assert abs(l[0] - ref[0][0][1]) < 1e-12
    assert int(w.q_pos[0]) == 160 and w.keys_per_request()[0] == 160


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_brute_force_tiny_decode(dtype):
    """Partial blocks, GQA 2, a document repeated at two offsets in one request."""
    w = _tiny(dtype=dtype)
    res = run_decode(w)
    for r in range(w.batch):
        ref = _brute_case(w, r)
        for h in range(w.num_q_heads):
            np.testing.assert_allclose(res[r][0][h], ref[h][0][0], atol=1e-12)
            assert abs(res[r][1][h] - ref[h][0][1]) < 1e-12


def test_brute_force_tiny_prefill():
    w = _tiny(kind="prefill")
    res = run_prefill(w)
    for r in range(w.batch):
        ref = _brute_case(w, r)
        for h in range(w.num_q_heads):
            for j in range(w.q_len(r)):
                np.testing.assert_allclose(res[r][0][j, h], ref[h][j][0], atol=1e-12)
                assert abs(res[r][1][j, h] - ref[h][j][1]) < 1e-12


# --------------------------------------------------- zero-copy invariances
def test_segment_order_and_block_relocation():
    w = _tiny()
    th = rope_theta(w.head_dim, w.rope_base)
    kw = dict(block_size=w.block_size, num_kv_heads=w.num_kv_heads, theta=th, scale=w.scale)
    r = 1
    o1, _ = attention_decode(w.q[r], int(w.q_pos[r]), w.requests[r], w.k_pool, w.v_pool, **kw)
    rev = list(reversed(w.requests[r]))
    o2, _ = attention_decode(w.q[r], int(w.q_pos[r]), rev, w.k_pool, w.v_pool, **kw)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    # relocate every block of the request to fresh ids at the end of the pool
    kp = np.concatenate([w.k_pool, w.k_pool])
    vp = np.concatenate([w.v_pool, w.v_pool])
    nb = w.num_blocks
    moved = [Segment(s.start, s.n_tokens, s.blocks + nb, s.is_new) for s in w.requests[r]]
    o3, _ = attention_decode(w.q[r], int(w.q_pos[r]), moved, kp, vp, **kw)
    np.testing.assert_array_equal(o1, o3)


def test_poisoned_tail_slots_are_never_read():
    w = _tiny(poison=True)
    for r, (o, l) in run_decode(w).items():
        assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))


# -------------------------------------------------------- closed forms, Eq. 3
def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_eq3_hit_ratio_gap_printed_value():
    """2.86x at D=20, C=100 (§1, §2 Eq. 3); the printed alpha-free value needs alpha ~ 0.853."""
    g = _golden()["eq3_hit_ratio_gap"]
    gap = hit_ratio_gap(g["C"], g["D"], 0.853)
    assert round(gap, 2) == g["printed_gap"]
    # none of the skews printed elsewhere in the paper reproduces it
    for a in (1.1, 1.5, 2.1):
        assert round(hit_ratio_gap(g["C"], g["D"], a), 2) != g["printed_gap"]
    # uniform popularity: the ratio of counts C / floor(C/D)
    assert hit_ratio_gap(100, 20, 0.0) == pytest.approx(20.0, abs=1e-12)
    gaps = [hit_ratio_gap(100, 20, a) for a in np.linspace(0, 3, 31)]
    assert all(x > y for x, y in zip(gaps, gaps[1:]))


@pytest.mark.parametrize("alpha", [1.1, 1.5, 2.1])
def test_zipf_sums_match_hurwitz_zeta(alpha):
    from scipy.special import zeta
    for n in (1, 5, 100, 100000):
        ref = zeta(alpha, 1) - zeta(alpha, n + 1)
        assert zipf_partial_sum(n, alpha) == pytest.approx(ref, rel=1e-10)


def test_cost_model_printed_percentages():
    g = _golden()
    for c in g["naive_flops_overhead"]["cases"]:
        assert round(100 * naive_flops_overhead(c["M"]), 2) == c["printed_percent"]
    (c,) = g["naive_io_overhead"]["cases"]
    v = naive_io_overhead(c["M"], c["N"])
    assert 0.95 < v < 1.0  # "approaching 100%"
    (c,) = g["prefill_flops_overhead"]["cases"]
    assert round(100 * prefill_flops_overhead(c["M"]), 2) == c["printed_percent"]
    (c,) = g["prefill_table_bandwidth"]["cases"]
    assert round(100 * prefill_table_bandwidth(c["N"]), 1) == c["printed_percent"]
    (c,) = g["decode_trigger_overhead"]["cases"]
    assert round(100 * decode_trigger_overhead(c["N"]), 2) == c["printed_percent"]


# ------------------------------------------------ document-local pools
def _doc_local_pools(w):
    """Write w's segments into a fresh pool pair the document-local way."""
    from oracle import store_kv
    from workloads import segment_writes
    k, v, slots, idx = segment_writes(w, "index")
    zeros = np.zeros(w.k_pool.shape)
    return store_kv(k, v, slots, idx, zeros, zeros, block_size=w.block_size,
                    theta=rope_theta(w.head_dim, w.rope_base))


def test_store_kv_copy_rotation_and_untouched_slots():
    from oracle import store_kv
    nb, Hkv, BS, D, base = 5, 2, 4, 16, 1e4
    old_k = RNG.standard_normal((nb, Hkv, BS, D))
    old_v = RNG.standard_normal((nb, Hkv, BS, D))
    slots = np.array([3, 17, 8, 9, 0])
    k = RNG.standard_normal((5, Hkv, D))
    v = RNG.standard_normal((5, Hkv, D))
    th = rope_theta(D, base)
    kp, vp = store_kv(k, v, slots, None, old_k, old_v, block_size=BS, theta=th)
    pos = np.array([0, 5, 130000, 7, 31])
    kr, vr = store_kv(k, v, slots, pos, old_k, old_v, block_size=BS, theta=th)
    touched = np.zeros((nb, BS), bool)
    for n, s in enumerate(slots):
        b, t = divmod(int(s), BS)
        touched[b, t] = True
        np.testing.assert_array_equal(kp[b, :, t], k[n])
        np.testing.assert_array_equal(vp[b, :, t], v[n])
        np.testing.assert_array_equal(vr[b, :, t], v[n])
        want = _rope_complex(k[n], np.full(Hkv, pos[n], np.float64), base)
        np.testing.assert_allclose(kr[b, :, t], want, rtol=0, atol=1e-10)
        np.testing.assert_allclose(np.linalg.norm(kr[b, :, t], axis=-1),
                                   np.linalg.norm(k[n], axis=-1), rtol=1e-13)
    keep = ~touched[:, None, :].repeat(Hkv, axis=1)  # [nb, Hkv, BS]
    np.testing.assert_array_equal(kp[keep], old_k[keep])
    np.testing.assert_array_equal(vr[keep], old_v[keep])


def test_example_3_1_rotate_query_back_by_first_document():
    """Example 3.1: caches C1, C2 of two documents, both indexed from position 0.

    Reusing C2 right after d1 means rotating the query back by |d1| before it
    meets C2's keys (C1's keys need no shift).  The brute force below does
    exactly that with scalar loops; the oracle must agree both on the
    document-local pool and, through the position-free pool, with keys
    encoded at their logical positions.
    """
    from oracle.brute import brute_rotate
    D, BS, base, scale = 8, 4, 1e4, 0.3
    n1, n2 = 5, 7
    m = n1 + n2 + 2  # the query after both documents
    raw_k = RNG.standard_normal((n1 + n2, D))
    raw_v = RNG.standard_normal((n1 + n2, D))
    q = RNG.standard_normal(D)
    c1 = [brute_rotate(raw_k[t].tolist(), t, base) for t in range(n1)]       # C1: from 0
    c2 = [brute_rotate(raw_k[n1 + t].tolist(), t, base) for t in range(n2)]  # C2: from 0
    scores, vals = [], []
    q_for_c1 = brute_rotate(q.tolist(), m, base)
    q_for_c2 = brute_rotate(q.tolist(), m - n1, base)  # rotated back by |d1|
    for t in range(n1):
        scores.append(scale * sum(a * b for a, b in zip(q_for_c1, c1[t])))
        vals.append(raw_v[t])
    for t in range(n2):
        scores.append(scale * sum(a * b for a, b in zip(q_for_c2, c2[t])))
        vals.append(raw_v[n1 + t])
    mx = max(scores)
    wts = [math.exp(s - mx) for s in scores]
    z = sum(wts)
    want = sum(wt * vv for wt, vv in zip(wts, vals)) / z
    want_lse = mx + math.log(z)

    # pools: d1 in blocks 0,1; d2 in blocks 2,3 (partial last blocks)
    nb = 4
    kp = np.zeros((nb, 1, BS, D))
    vp = np.zeros((nb, 1, BS, D))
    for t in range(n1):
        kp[t // BS, 0, t % BS], vp[t // BS, 0, t % BS] = raw_k[t], raw_v[t]
    for t in range(n2):
        kp[2 + t // BS, 0, t % BS], vp[2 + t // BS, 0, t % BS] = raw_k[n1 + t], raw_v[n1 + t]
    segs = [Segment(0, n1, np.array([0, 1]), False), Segment(n1, n2, np.array([2, 3]), False)]
    th = rope_theta(D, base)
    from oracle import store_kv
    slots = np.array([t for t in range(n1)] + [2 * BS + t for t in range(n2)])
    idx = np.array(list(range(n1)) + list(range(n2)))
    kd, vd = store_kv(raw_k[:, None, :], raw_v[:, None, :], slots, idx, np.zeros_like(kp),
                      np.zeros_like(vp), block_size=BS, theta=th)
    kw = dict(block_size=BS, num_kv_heads=1, theta=th, scale=scale)
    o, l = attention_decode(q[None, :], m, segs, kd, vd, doc_local=True, **kw)
    np.testing.assert_allclose(o[0], want, rtol=0, atol=1e-12)
    assert abs(l[0] - want_lse) < 1e-12
    o2, l2 = attention_decode(q[None, :], m, segs, kp, vp, **kw)
    np.testing.assert_allclose(o2[0], want, rtol=0, atol=1e-12)
    assert abs(l2[0] - want_lse) < 1e-12


@pytest.mark.parametrize("kind", ["decode", "prefill"])
def test_doc_local_pool_equals_position_free(kind):
    """Same documents at several offsets (one repeated in a request), GQA 2, partial blocks."""
    w = _tiny(kind, dtype="f32")
    pools = _doc_local_pools(w)
    if kind == "decode":
        a, b = run_decode(w), run_decode(w, pools=pools, doc_local=True)
    else:
        a, b = run_prefill(w), run_prefill(w, pools=pools, doc_local=True)
    for r in a:
        np.testing.assert_allclose(b[r][0], a[r][0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(b[r][1], a[r][1], rtol=0, atol=1e-12)


def test_doc_local_reading_is_not_position_free_reading():
    """The two pool readings differ on the same bytes (so the flag matters)."""
    w = _tiny("decode", dtype="f32")
    pools = _doc_local_pools(w)
    a = run_decode(w, pools=pools, doc_local=True)
    b = run_decode(w, pools=pools, doc_local=False)
    assert max(np.max(np.abs(a[r][0] - b[r][0])) for r in a) > 1e-3


def test_absolute_prerotated_pool_is_doc_local_with_zero_starts():
    """Keys pre-rotated at absolute positions = doc-local pool with every start 0."""
    from oracle import store_kv
    from workloads import segment_writes
    w = _tiny("decode", dtype="f32", requests=[[("doc", 0), ("doc", 2), ("priv", 3)],
                                               [("doc", 1, 30), ("doc", 3, 50)]])
    k, v, slots, pos = segment_writes(w, "absolute")
    zeros = np.zeros(w.k_pool.shape)
    pools = store_kv(k, v, slots, pos, zeros, zeros, block_size=w.block_size,
                     theta=rope_theta(w.head_dim, w.rope_base))
    import copy
    w0 = copy.copy(w)
    w0.requests = [[Segment(0, s.n_tokens, s.blocks, s.is_new) for s in segs]
                   for segs in w.requests]
    a, b = run_decode(w), run_decode(w0, pools=pools, doc_local=True)
    for r in a:
        np.testing.assert_allclose(b[r][0], a[r][0], rtol=0, atol=1e-12)
    with pytest.raises(ValueError, match="no single absolute"):
        segment_writes(_tiny("decode", dtype="f32"), "absolute")


# ------------------------------------------------ interleaved RoPE pairing
def test_interleaved_rotation_is_complex_multiplication():
    D, base = 32, 1e4
    th = rope_theta(D, base)
    x = RNG.standard_normal((5, D))
    pos = np.array([0, 1, 17, 4096, 131071])
    inv = 1.0 / (base ** (np.arange(0, D, 2, dtype=np.float64) / D))
    z = (x[:, 0::2] + 1j * x[:, 1::2]) * np.exp(1j * pos[:, None] * inv[None, :])
    want = np.empty_like(x)
    want[:, 0::2], want[:, 1::2] = z.real, z.imag
    np.testing.assert_allclose(rope_rotate(x, pos, th, "interleaved"), want, rtol=0, atol=1e-10)


def test_interleaved_fact_3_2():
    D = 64
    th = rope_theta(D, 5e5)
    q, k = RNG.standard_normal(D), RNG.standard_normal(D)
    for m, n in [(0, 5), (700, 3), (65536, 131071)]:
        lhs = rope_rotate(q, m, th, "interleaved") @ rope_rotate(k, n, th, "interleaved")
        rhs = q @ rope_rotate(k, n - m, th, "interleaved")
        assert abs(lhs - rhs) < 1e-10


def _deinterleaved(w):
    """Copy of w with q and K stored in (even dims, odd dims) order."""
    import copy
    w2 = copy.copy(w)
    perm = np.concatenate([np.arange(0, w.head_dim, 2), np.arange(1, w.head_dim, 2)])
    w2.q = w.q[..., perm]
    w2.k_pool = w.k_pool[..., perm]
    return w2


@pytest.mark.parametrize("kind", ["decode", "prefill"])
def test_interleaved_equals_half_split_on_permuted_dims(kind):
    """Interleaved pairs of (q, k) are the half-split pairs of the permuted vectors."""
    w = _tiny(kind, dtype="f32")
    run = run_decode if kind == "decode" else run_prefill
    a = run(w, pairing="interleaved")
    b = run(_deinterleaved(w))
    for r in a:
        np.testing.assert_allclose(a[r][0], b[r][0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(a[r][1], b[r][1], rtol=0, atol=1e-12)


@pytest.mark.parametrize("kind", ["decode", "prefill"])
def test_brute_force_interleaved_and_alibi(kind):
    from oracle import alibi_slopes
    w = _tiny(kind, dtype="f32")
    sl = alibi_slopes(w.num_q_heads)
    run = run_decode if kind == "decode" else run_prefill
    inter = run(w, pairing="interleaved")
    ali = run(w, alibi=sl)
    for r in range(w.batch):
        for h in range(w.num_q_heads):
            g = h // w.group
            keys = []
            for s in w.requests[r]:
                for t in range(s.n_tokens):
                    b = int(s.blocks[t // w.block_size])
                    keys.append((w.values_f32(w.k_pool[b, g, t % w.block_size]).tolist(),
                                 w.values_f32(w.v_pool[b, g, t % w.block_size]).tolist(),
                                 s.start + t, s.is_new))
            if kind == "decode":
                qs = [(w.values_f32(w.q[r, h]).tolist(), int(w.q_pos[r]))]
            else:
                a0 = int(w.cu_q[r])
                qs = [(w.values_f32(w.q[a0 + j, h]).tolist(), int(w.q_pos[r]) + j)
                      for j in range(w.q_len(r))]
            bi = brute_attention(qs, keys, w.scale, w.rope_base, interleaved=True)
            ba = brute_attention(qs, keys, w.scale, w.rope_base, alibi_slope=float(sl[h]))
            for j, (o, l) in enumerate(bi):
                oi = inter[r][0][h] if kind == "decode" else inter[r][0][j, h]
                np.testing.assert_allclose(oi, o, rtol=0, atol=1e-12)
            for j, (o, l) in enumerate(ba):
                oa = ali[r][0][h] if kind == "decode" else ali[r][0][j, h]
                la = ali[r][1][h] if kind == "decode" else ali[r][1][j, h]
                np.testing.assert_allclose(oa, o, rtol=0, atol=1e-12)
                assert abs(la - l) < 1e-12


# ------------------------------------------------------------------ ALiBi
def test_alibi_slopes_published_values():
    from oracle import alibi_slopes
    np.testing.assert_allclose(alibi_slopes(8), [2.0 ** -k for k in range(1, 9)], rtol=1e-15)
    want12 = [2.0 ** -k for k in range(1, 9)] + [2.0 ** -0.5, 2.0 ** -1.5, 2.0 ** -2.5,
                                                  2.0 ** -3.5]
    np.testing.assert_allclose(alibi_slopes(12), want12, rtol=1e-15)
    np.testing.assert_allclose(alibi_slopes(1), [2.0 ** -8], rtol=1e-15)


def test_alibi_closed_form_two_equal_keys():
    """Equal q.k: weights follow exp(slope * (p - m)) alone."""
    D, s_, m = 8, 0.25, 40
    k = RNG.standard_normal(D)
    v = RNG.standard_normal((2, D))
    kp = np.zeros((2, 1, 4, D))
    vp = np.zeros((2, 1, 4, D))
    kp[0, 0, 0], kp[1, 0, 0] = k, k
    vp[0, 0, 0], vp[1, 0, 0] = v[0], v[1]
    segs = [Segment(30, 1, np.array([0]), False), Segment(37, 1, np.array([1]), False)]
    q = RNG.standard_normal((1, D))
    o, _ = attention_decode(q, m, segs, kp, vp, block_size=4, num_kv_heads=1,
                            theta=rope_theta(D, 1e4), scale=0.5, alibi=np.array([s_]))
    w1, w2 = math.exp(s_ * (30 - m)), math.exp(s_ * (37 - m))
    np.testing.assert_allclose(o[0], (w1 * v[0] + w2 * v[1]) / (w1 + w2), rtol=0, atol=1e-13)


def test_alibi_zero_slopes_is_unrotated_attention_and_shift_invariant():
    w = _tiny("decode", dtype="f32")
    a = run_decode(w, alibi=np.zeros(w.num_q_heads))
    b = run_decode(w, rotate=False)
    for r in a:
        np.testing.assert_allclose(a[r][0], b[r][0], rtol=0, atol=1e-13)
    from oracle import alibi_slopes
    sl = alibi_slopes(w.num_q_heads)
    c = run_decode(w, alibi=sl)
    import copy
    w2 = copy.copy(w)
    w2.requests = [_shifted(segs, 1000) for segs in w.requests]
    w2.q_pos = w.q_pos + 1000
    d = run_decode(w2, alibi=sl)
    for r in c:
        np.testing.assert_allclose(c[r][0], d[r][0], rtol=0, atol=1e-11)


# ------------------------------------------------------ scaled RoPE tables
_SCALINGS = [
    {"type": "linear", "factor": 4.0},
    {"type": "ntk", "factor": 4.0},
    {"type": "yarn", "factor": 16.0, "original_max_pos": 4096, "beta_fast": 32.0,
     "beta_slow": 1.0},
    {"type": "llama3", "factor": 8.0, "original_max_pos": 8192, "low_freq_factor": 1.0,
     "high_freq_factor": 4.0},
]


@pytest.mark.parametrize("sc", _SCALINGS, ids=lambda d: d["type"])
def test_scaled_factor_one_is_plain(sc):
    from oracle import rope_theta_scaled
    th, amp = rope_theta_scaled(128, 5e5, dict(sc, factor=1.0))
    np.testing.assert_allclose(th, rope_theta(128, 5e5), rtol=1e-14)
    assert amp == 1.0


@pytest.mark.parametrize("sc", _SCALINGS, ids=lambda d: d["type"])
def test_scaled_tables_keep_fact_3_2(sc):
    """Every variant is still a rotation: scores depend on n - m only (times amp^2)."""
    from oracle import rope_theta_scaled
    th, amp = rope_theta_scaled(64, 1e4, sc)
    q, k = RNG.standard_normal(64), RNG.standard_normal(64)
    for m, n in [(3, 9), (5000, 70000)]:
        lhs = rope_rotate(q, m, th, amp=amp) @ rope_rotate(k, n, th, amp=amp)
        rhs = amp * amp * (q @ rope_rotate(k, n - m, th))
        assert abs(lhs - rhs) < 1e-9 * max(1.0, abs(rhs))


def test_linear_scaling_is_position_interpolation():
    """Positions s*p under linear scaling see the plain rotation at p."""
    from oracle import rope_theta_scaled
    th4, _ = rope_theta_scaled(64, 1e4, {"type": "linear", "factor": 4.0})
    x = RNG.standard_normal((6, 64))
    p = np.array([0, 1, 7, 100, 2048, 30000])
    np.testing.assert_allclose(rope_rotate(x, 4 * p, th4), rope_rotate(x, p, rope_theta(64, 1e4)),
                               rtol=0, atol=1e-9)


def test_ntk_keeps_fastest_and_interpolates_slowest_pair():
    from oracle import rope_theta_scaled
    D, f = 128, 8.0
    th, _ = rope_theta_scaled(D, 1e4, {"type": "ntk", "factor": f})
    th0 = rope_theta(D, 1e4)
    assert th[0] == th0[0] == 1.0
    assert abs(th[-1] - th0[-1] / f) < 1e-15 * th0[-1] * 10
    assert np.all(np.diff(th / th0) < 0)  # more interpolation the slower the pair


def _rotations_over(L, th):
    return L * th / (2 * np.pi)


def test_yarn_ramp_follows_rotation_counts_and_attention_factor():
    from oracle import rope_theta_scaled
    D, base, L, s_ = 128, 1e4, 4096, 16.0
    th0 = rope_theta(D, base)
    th, amp = rope_theta_scaled(D, base, {"type": "yarn", "factor": s_, "original_max_pos": L,
                                          "beta_fast": 32.0, "beta_slow": 1.0})
    r = _rotations_over(L, th0)
    step = base ** (2.0 / D)  # one pair index = this ratio in rotation count
    fast = r > 32.0 * step
    slow = r < 1.0 / step
    assert fast.any() and slow.any()
    np.testing.assert_allclose(th[fast], th0[fast], rtol=1e-15)
    np.testing.assert_allclose(th[slow], th0[slow] / s_, rtol=1e-15)
    ratio = th / th0
    assert np.all(np.diff(ratio) <= 1e-15)  # monotone blend from 1 down to 1/s
    assert abs(amp - (0.1 * math.log(s_) + 1.0)) < 1e-15
    _, amp_e = rope_theta_scaled(D, base, {"type": "yarn", "factor": math.e,
                                           "original_max_pos": L})
    assert abs(amp_e - 1.1) < 1e-15


def test_yarn_ramp_ends_where_the_upper_clamp_binds():
    """YaRN's correction range, hand-computed for D = 128, base 1e4, original
    context L = 65536, beta_fast 32, beta_slow 1 (the published definition the
    table restates; LazyAttention §3.5 only says scaled variants change the
    table).  The pair index turning b times over L is
    D ln(L / (2 pi b)) / (2 ln base): 40.21 for b = 32 and 64.29 for b = 1, so
    the ramp runs from lo = floor(40.21) = 40 to hi = ceil(64.29) = 65.  hi lies
    past the last pair (63): the published range clamps it to D - 1 = 127,
    not to 63, so pair 63 is only 23/25 interpolated.  A floor/ceil swap at
    either end, or a D/2 - 1 clamp, changes pair 41 or pair 63 below.
    """
    from oracle import rope_theta_scaled
    D, base, L, f = 128, 1e4, 65536, 16.0
    th, amp = rope_theta_scaled(D, base, {"type": "yarn", "factor": f, "original_max_pos": L,
                                          "beta_fast": 32.0, "beta_slow": 1.0})
    th0 = 1.0 / (1e4 ** (np.arange(0, D, 2, dtype=np.float64) / D))  # textbook frequencies
    lo, hi = 40, 65  # literal, from the arithmetic in the docstring
    for i, ramp in [(0, 0.0), (39, 0.0), (40, 0.0), (41, 1 / 25), (52, 12 / 25), (63, 23 / 25)]:
        want = th0[i] * (1.0 - ramp) + th0[i] / f * ramp
        assert abs(th[i] - want) <= 1e-15 * th0[i], (i, th[i], want)
        assert ramp == max(0.0, min(1.0, (i - lo) / (hi - lo)))
    assert abs(amp - (0.1 * math.log(16.0) + 1.0)) < 1e-15


def test_scaled_amplitude_enters_every_score_squared_in_both_pool_readings():
    """A table whose rows carry an amplitude a (cos and sin both times a) scales
    every score by a^2 -- once through the query, once through the key -- in the
    position-free reading and in the document-local one, where the stored key
    (written with the table) already carries a and the relative rotation by the
    segment start is a pure rotation.  Pinned to the scalar brute force with
    scale * a^2 (LazyAttention §3.5: a scaled variant keeps q^T R_{n-m} k)."""
    from oracle import store_kv
    from oracle.brute import brute_attention
    a = 1.37
    for kind in ("decode", "prefill"):
        w = _tiny(kind, dtype="f32")
        th = rope_theta(w.head_dim, w.rope_base)
        slots, idx, ks, vs = [], [], [], []
        seen = set()
        for segs in w.requests:
            for seg in segs:
                key = tuple(int(b) for b in seg.blocks)
                if key in seen:
                    continue
                seen.add(key)
                t = np.arange(seg.n_tokens)
                blk = np.asarray(seg.blocks)[t // w.block_size]
                slots.append(blk * w.block_size + t % w.block_size)
                idx.append(t)
                ks.append(w.k_pool[blk, :, t % w.block_size, :])
                vs.append(w.v_pool[blk, :, t % w.block_size, :])
        slots, idx = np.concatenate(slots), np.concatenate(idx)
        base_pool = np.zeros(w.k_pool.shape)
        pools = store_kv(np.concatenate(ks), np.concatenate(vs), slots, idx, base_pool, base_pool,
                         block_size=w.block_size, theta=th, amp=a)
        kw = dict(block_size=w.block_size, num_kv_heads=w.num_kv_heads, theta=th, scale=w.scale,
                  amp=a)
        G = w.num_q_heads // w.num_kv_heads
        for r, segs in enumerate(w.requests):
            if kind == "decode":
                o_pf, _ = attention_decode(w.q[r], int(w.q_pos[r]), segs, w.k_pool, w.v_pool, **kw)
                o_dl, _ = attention_decode(w.q[r], int(w.q_pos[r]), segs, *pools, doc_local=True,
                                           **kw)
                qrows = [(w.q[r][h], int(w.q_pos[r]), h) for h in range(w.num_q_heads)]
            else:
                qa, qb = int(w.cu_q[r]), int(w.cu_q[r + 1])
                o_pf, _ = attention_prefill(w.q[qa:qb], int(w.q_pos[r]), segs, w.k_pool, w.v_pool,
                                            **kw)
                o_dl, _ = attention_prefill(w.q[qa:qb], int(w.q_pos[r]), segs, *pools,
                                            doc_local=True, **kw)
                qrows = [(w.q[qa + j][h], int(w.q_pos[r]) + j, (j, h))
                         for j in range(qb - qa) for h in range(w.num_q_heads)]
            for qv, qp, at in qrows:
                h = at if kind == "decode" else at[1]
                g = h // G
                keys = []
                for seg in segs:
                    for t in range(seg.n_tokens):
                        b, sl = int(seg.blocks[t // w.block_size]), t % w.block_size
                        keys.append((w.k_pool[b, g, sl].tolist(), w.v_pool[b, g, sl].tolist(),
                                     int(seg.start) + t, bool(seg.is_new)))
                (want, _), = brute_attention([(qv.tolist(), qp)], keys, w.scale * a * a,
                                             w.rope_base)
                got_pf = o_pf[h] if kind == "decode" else o_pf[at]
                got_dl = o_dl[h] if kind == "decode" else o_dl[at]
                np.testing.assert_allclose(got_pf, want, rtol=0, atol=1e-12)
                np.testing.assert_allclose(got_dl, want, rtol=0, atol=1e-12)


def test_llama3_scaling_wavelength_classes():
    from oracle import rope_theta_scaled
    D, base, L = 128, 5e5, 8192
    th0 = rope_theta(D, base)
    th, amp = rope_theta_scaled(D, base, {"type": "llama3", "factor": 8.0, "original_max_pos": L,
                                          "low_freq_factor": 1.0, "high_freq_factor": 4.0})
    wl = 2 * np.pi / th0
    keep, scaled = wl < L / 4.0, wl > L / 1.0
    assert keep.any() and scaled.any() and (~keep & ~scaled).any()
    np.testing.assert_allclose(th[keep], th0[keep], rtol=1e-15)
    np.testing.assert_allclose(th[scaled], th0[scaled] / 8.0, rtol=1e-15)
    mid = ~keep & ~scaled
    assert np.all((th[mid] < th0[mid]) & (th[mid] > th0[mid] / 8.0))
    assert amp == 1.0


def test_llama3_blend_is_continuous_at_band_edges():
    """Inside the smooth band the ratio theta'/theta runs from 1 (fast edge) to 1/s (slow edge)."""
    from oracle import rope_theta_scaled
    D, base, L, s_ = 4096, 5e5, 8192, 8.0
    th0 = rope_theta(D, base)
    th, _ = rope_theta_scaled(D, base, {"type": "llama3", "factor": s_, "original_max_pos": L,
                                        "low_freq_factor": 1.0, "high_freq_factor": 4.0})
    wl = 2 * np.pi / th0
    ratio = th / th0
    fast_edge = (wl > L / 4.0) & (wl < L / 4.0 * 1.02)
    slow_edge = (wl < L / 1.0) & (wl > L / 1.0 * 0.98)
    assert fast_edge.any() and slow_edge.any()
    assert np.all(np.abs(ratio[fast_edge] - 1.0) < 0.05)
    assert np.all(np.abs(ratio[slow_edge] * s_ - 1.0) < 0.05)


def test_interleaved_storage_order_through_attention():
    """Keys written with interleaved pairing, read as half-split pairs with q split the same way,
    give the interleaved RoPE attention of the raw keys (document-local and position-free)."""
    from oracle import store_kv
    from workloads import segment_writes
    w = _tiny("decode", dtype="f32")
    th = rope_theta(w.head_dim, w.rope_base)
    k, v, slots, idx = segment_writes(w, "index")
    zeros = np.zeros(w.k_pool.shape)
    perm = np.concatenate([np.arange(0, w.head_dim, 2), np.arange(1, w.head_dim, 2)])
    import copy
    wq = copy.copy(w)
    wq.q = w.q[..., perm]  # q read the way the kernels read it
    want = run_decode(w, pairing="interleaved")
    for rope_pos, doc_local in ((None, False), (idx, True)):
        pools = store_kv(k, v, slots, rope_pos, zeros, zeros, block_size=w.block_size, theta=th,
                         pairing="interleaved")
        got = run_decode(wq, pools=pools, doc_local=doc_local)
        for r in want:
            np.testing.assert_allclose(got[r][0], want[r][0], rtol=0, atol=1e-12)

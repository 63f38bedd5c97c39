"""Seeded random sweep of small cases across every kernel variant, against the oracle.

Each small case draws its own document lengths (1..100 tokens, so ragged tails and
one-token blocks occur), request mixes (documents shared between and within
requests, explicit offsets leaving gaps, keys after the decode query),
GQA group, dtype, pool mode (position-free or document-local), positional
encoding (half-split RoPE, interleaved RoPE, ALiBi) and decode split size.
The combinations are fixed by the seed, so a failure names a reproducible case.
"""
import numpy as np
import pytest
import torch

from oracle import alibi_slopes, run_decode, run_prefill
from position_agnostic_kv_lazy_amd.prepare import store_pool
from workloads import build_workload, segment_writes

from gpu_util import Device, assert_lse, assert_parity, log

pytestmark = pytest.mark.gpu

N_CASES = 40
GROUPS = [(2, 2), (4, 2), (8, 2), (16, 2), (32, 2)]  # G = 1, 2, 4, 8, 16


def _case(i):
    rng = np.random.default_rng([7100, i])
    kind = "decode" if i % 2 == 0 else "prefill"
    dtype = "bf16" if (i // 2) % 2 == 0 else "f32"
    Hq, Hkv = GROUPS[int(rng.integers(len(GROUPS)))]
    enc = ["rope_half", "rope_interleaved", "alibi"][int(rng.integers(3))]
    pool = "position_free" if enc == "alibi" else ["position_free", "doc_local"][int(rng.integers(2))]
    n_docs = int(rng.integers(3, 8))
    doc_lens = [int(x) for x in rng.integers(1, 101, size=n_docs)]
    batch = int(rng.integers(1, 5))
    requests = []
    for _ in range(batch):
        items = []
        for _ in range(int(rng.integers(1, 6))):
            d = int(rng.integers(n_docs))
            if kind == "decode" and rng.random() < 0.3:
                items.append(("doc", d, int(rng.integers(0, 400))))  # explicit offset
            else:
                items.append(("doc", d))
        if kind == "decode":
            if rng.random() < 0.5:
                items.append(("priv", int(rng.integers(1, 40))))
        else:
            items.append(("new", int(rng.integers(1, 150))))
        requests.append(items)
    split = int(rng.integers(0, 4)) if kind == "decode" else 0
    w = build_workload(name=f"rand{i}", kind=kind, dtype=dtype, num_q_heads=Hq,
                       num_kv_heads=Hkv, head_dim=128, block_size=16, rope_base=5e5,
                       doc_lens=doc_lens, requests=requests, seed=7200 + i)
    return w, enc, pool, split


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(i):
    w, enc, pool, split = _case(i)
    log(f"random case {i}: {w.kind} {w.dtype} Hq={w.num_q_heads} Hkv={w.num_kv_heads} "
        f"{enc} {pool} split={split} batch={w.batch}")
    if enc == "rope_interleaved" or pool == "doc_local":
        # keys go through the cache write: permuted to (even, odd) storage for
        # interleaved pairs, rotated by their index in the segment for doc-local
        k, v, slots, idx = segment_writes(w, "index")
        kd, vd = store_pool(w, k, v, slots, idx if pool == "doc_local" else None,
                            pos_encoding=enc)
        torch.cuda.synchronize()
        dev = Device.from_device_pools(kd, vd)
    else:
        dev = Device(w)
    out, lse, _ = dev.run(w, split_blocks=split, pool_mode=pool, pos_encoding=enc)
    # Every variant must give RoPE (or ALiBi) attention at the logical
    # positions over the raw keys: the oracle's position-free definition.
    kw = dict(pairing="interleaved" if enc == "rope_interleaved" else "half",
              alibi=alibi_slopes(w.num_q_heads) if enc == "alibi" else None)
    if w.kind == "decode":
        ref = run_decode(w, **kw)
        for r in range(w.batch):
            assert_parity(out[r], ref[r][0], w.dtype, f"case {i} req {r}")
            assert_lse(lse[r], ref[r][1], w.dtype, f"case {i} req {r}")
        if w.dtype == "bf16" and enc != "alibi":  # the shared-segment decode too
            mib = [0, 1, 3][i % 3]
            out, lse, _ = dev.run(w, pool_mode=pool, pos_encoding=enc, shared=True,
                                  max_item_blocks=mib, check_tables=True)
            for r in range(w.batch):
                assert_parity(out[r], ref[r][0], w.dtype, f"case {i} shared req {r}")
                assert_lse(lse[r], ref[r][1], w.dtype, f"case {i} shared req {r}")
    else:
        ref = run_prefill(w, **kw)
        for r in range(w.batch):
            a, b = int(w.cu_q[r]), int(w.cu_q[r + 1])
            assert_parity(out[a:b], ref[r][0], w.dtype, f"case {i} req {r}")
            assert_lse(lse[a:b], ref[r][1], w.dtype, f"case {i} req {r}")


N_SHARED = 48


def _shared_case(i):
    """A decode batch with heavy sharing: up to 12 requests drawing from a few
    documents (Zipf-like), repeats within a request, explicit offsets, private
    segments; every group size and both pool modes; chunk lengths forced down
    to one block."""
    rng = np.random.default_rng([7300, i])
    Hq, Hkv = GROUPS[i % len(GROUPS)]
    enc = ["rope_half", "rope_interleaved"][int(rng.integers(2))]
    pool = ["position_free", "doc_local"][int(rng.integers(2))]
    n_docs = int(rng.integers(2, 6))
    doc_lens = [int(x) for x in rng.integers(1, 101, size=n_docs)]
    pop = 1.0 / np.arange(1, n_docs + 1)
    pop /= pop.sum()
    requests = []
    for _ in range(int(rng.integers(1, 13))):
        items = []
        for _ in range(int(rng.integers(1, 6))):
            d = int(rng.choice(n_docs, p=pop))
            if rng.random() < 0.4:
                items.append(("doc", d, int(rng.integers(0, 600))))
            else:
                items.append(("doc", d))
        if rng.random() < 0.6:
            items.append(("priv", int(rng.integers(1, 40))))
        requests.append(items)
    mib = [0, 1, 2, 5, 16][int(rng.integers(5))]
    w = build_workload(name=f"shared{i}", kind="decode", dtype="bf16", num_q_heads=Hq,
                       num_kv_heads=Hkv, head_dim=128, block_size=16, rope_base=5e5,
                       doc_lens=doc_lens, requests=requests, seed=7400 + i)
    return w, enc, pool, mib


@pytest.mark.parametrize("i", range(N_SHARED))
def test_random_shared_case(i):
    w, enc, pool, mib = _shared_case(i)
    log(f"random shared case {i}: Hq={w.num_q_heads} Hkv={w.num_kv_heads} {enc} {pool} "
        f"chunk={mib} batch={w.batch}")
    if enc == "rope_interleaved" or pool == "doc_local":
        k, v, slots, idx = segment_writes(w, "index")
        kd, vd = store_pool(w, k, v, slots, idx if pool == "doc_local" else None,
                            pos_encoding=enc)
        torch.cuda.synchronize()
        dev = Device.from_device_pools(kd, vd)
    else:
        dev = Device(w)
    out, lse, _ = dev.run(w, pool_mode=pool, pos_encoding=enc, shared=True, max_item_blocks=mib,
                          check_tables=True)
    ref = run_decode(w, pairing="interleaved" if enc == "rope_interleaved" else "half")
    for r in range(w.batch):
        assert_parity(out[r], ref[r][0], "bf16", f"shared case {i} req {r}")
        assert_lse(lse[r], ref[r][1], "bf16", f"shared case {i} req {r}")


N_MEDIUM = 16
MEDIUM_GROUPS = GROUPS + [(32, 8)]


def _medium_case(i):
    """Longer documents (100..2000 tokens): several split groups and chunks per
    request in decode (both kernels), multi-tile causal prefill (up to 600 new
    tokens, many q tiles), every encoding and both pool modes."""
    rng = np.random.default_rng([7500, i])
    kind = "decode" if i % 2 == 0 else "prefill"
    dtype = "f32" if i % 4 == 3 else "bf16"
    Hq, Hkv = MEDIUM_GROUPS[int(rng.integers(len(MEDIUM_GROUPS)))]
    enc = ["rope_half", "rope_interleaved", "alibi"][int(rng.integers(3))]
    pool = "position_free" if enc == "alibi" else ["position_free", "doc_local"][int(rng.integers(2))]
    n_docs = int(rng.integers(3, 7))
    doc_lens = [int(x) for x in rng.integers(100, 2001, size=n_docs)]
    requests = []
    for _ in range(int(rng.integers(1, 6))):
        items = []
        for _ in range(int(rng.integers(2, 6))):
            d = int(rng.integers(n_docs))
            if kind == "decode" and rng.random() < 0.3:
                items.append(("doc", d, int(rng.integers(0, 20000))))
            else:
                items.append(("doc", d))
        if kind == "decode":
            if rng.random() < 0.5:
                items.append(("priv", int(rng.integers(1, 300))))
        else:
            items.append(("new", int(rng.integers(64, 601))))
        requests.append(items)
    w = build_workload(name=f"medium{i}", kind=kind, dtype=dtype, num_q_heads=Hq,
                       num_kv_heads=Hkv, head_dim=128, block_size=16, rope_base=5e5,
                       doc_lens=doc_lens, requests=requests, seed=7600 + i)
    return w, enc, pool, rng


@pytest.mark.parametrize("i", range(N_MEDIUM))
def test_random_medium_case(i):
    w, enc, pool, rng = _medium_case(i)
    log(f"random medium case {i}: {w.kind} {w.dtype} Hq={w.num_q_heads} Hkv={w.num_kv_heads} "
        f"{enc} {pool} batch={w.batch} keys={[sum(s.n_tokens for s in r) for r in w.requests]}")
    if enc == "rope_interleaved" or pool == "doc_local":
        k, v, slots, idx = segment_writes(w, "index")
        kd, vd = store_pool(w, k, v, slots, idx if pool == "doc_local" else None,
                            pos_encoding=enc)
        torch.cuda.synchronize()
        dev = Device.from_device_pools(kd, vd)
    else:
        dev = Device(w)
    out, lse, _ = dev.run(w, pool_mode=pool, pos_encoding=enc)
    kw = dict(pairing="interleaved" if enc == "rope_interleaved" else "half",
              alibi=alibi_slopes(w.num_q_heads) if enc == "alibi" else None)
    if w.kind == "decode":
        ref = run_decode(w, **kw)
        for r in range(w.batch):
            assert_parity(out[r], ref[r][0], w.dtype, f"medium {i} req {r}")
            assert_lse(lse[r], ref[r][1], w.dtype, f"medium {i} req {r}")
        if w.dtype == "bf16" and enc != "alibi":
            out, lse, _ = dev.run(w, pool_mode=pool, pos_encoding=enc, shared=True,
                                  check_tables=True)
            for r in range(w.batch):
                assert_parity(out[r], ref[r][0], w.dtype, f"medium {i} shared req {r}")
                assert_lse(lse[r], ref[r][1], w.dtype, f"medium {i} shared req {r}")
    else:
        # rows sampled per request (the first and last included): the oracle
        # computes each sampled row over the request's whole key list
        rows = {}
        for r in range(w.batch):
            nq = w.q_len(r)
            pick = rng.choice(nq, size=min(nq, 24), replace=False)
            rows[r] = np.unique(np.concatenate([pick, [0, nq - 1]]))
        ref = run_prefill(w, rows=rows, **kw)
        for r, rr in rows.items():
            a = int(w.cu_q[r])
            assert_parity(out[a + rr], ref[r][0], w.dtype, f"medium {i} req {r}")
            assert_lse(lse[a + rr], ref[r][1], w.dtype, f"medium {i} req {r}")

"""Document-cache simulator (host C++, lazy_attn_cache_simulate) against the oracle.

The hit-ratio model of "LazyAttention" §2: Eq. 1 (position-agnostic cache of C
documents), Eq. 2 (position-aware cache: C entries cover about C / D documents)
and their ratio, Eq. 3.  Table 1's cells depend on a document size and an
eviction policy the paper does not state, so they are not pinned; the static
top-C cache is pinned to Eqs. 1-2 and LRU to hand-worked traces and to the
plain-Python reference replay.
"""
import numpy as np
import pytest

import position_agnostic_kv_lazy_amd as la
from oracle import hit_ratio_agnostic, hit_ratio_aware, simulate_cache
from workloads import doc_trace, zipf_probs


def test_lru_hand_worked():
    docs = [0, 1, 0, 2, 1, 0]
    # capacity 2: miss, miss, hit, miss (evicts 1), miss (evicts 0), miss
    assert la.lazy_attn_cache_simulate(docs, None, 1, 2) == 1
    assert simulate_cache(docs, None, 1, 2) == 1
    # capacity 3 holds everything: only first touches miss
    assert la.lazy_attn_cache_simulate(docs, None, 1, 3) == 3
    # position-aware keys: (0, 0), (0, 1), (0, 0)
    d, p = [0, 0, 0], [0, 1, 0]
    assert la.lazy_attn_cache_simulate(d, p, 2, 2, "aware") == 1
    assert la.lazy_attn_cache_simulate(d, p, 2, 1, "aware") == 0
    assert la.lazy_attn_cache_simulate(d, p, 2, 1, "agnostic") == 2
    assert la.lazy_attn_cache_simulate(d, p, 2, 0, "agnostic") == 0


@pytest.mark.parametrize("alpha", [0.8, 1.1, 2.1])
@pytest.mark.parametrize("policy", ["agnostic", "aware"])
@pytest.mark.parametrize("eviction", ["lru", "static_top"])
def test_matches_reference_replay(alpha, policy, eviction):
    docs, pos = doc_trace(400, 500, alpha, 10, seed=int(alpha * 10))
    for cap in (0, 1, 7, 40, 333, 5000):
        got = la.lazy_attn_cache_simulate(docs, pos, 10, cap, policy, eviction)
        want = simulate_cache(docs, pos, 10, cap, policy, eviction)
        assert got == want, (cap, got, want)


@pytest.mark.parametrize("alpha", [0.853, 1.1, 1.5])
def test_static_cache_reaches_eqs_1_and_2(alpha):
    """iid Zipf accesses at uniform positions: the static hit ratios are Eq. 1 / Eq. 2."""
    N, D, C, n = 2000, 20, 100, 400_000
    rng = np.random.default_rng(11)
    docs = rng.choice(N, size=n, p=zipf_probs(N, alpha))
    pos = rng.integers(0, D, size=n).astype(np.int32)
    h1 = la.lazy_attn_cache_simulate(docs, pos, D, C, "agnostic", "static_top") / n
    h2 = la.lazy_attn_cache_simulate(docs, pos, D, C, "aware", "static_top") / n
    e1, e2 = hit_ratio_agnostic(C, N, alpha), hit_ratio_aware(C, D, N, alpha)
    for got, want in ((h1, e1), (h2, e2)):
        sigma = np.sqrt(want * (1 - want) / n)
        assert abs(got - want) < 5 * sigma, (got, want, sigma)


def test_agnostic_beats_aware_under_lru():
    docs, pos = doc_trace(3000, 20000, 1.1, 10, seed=4)
    for cap in (50, 200, 1000):
        a = la.lazy_attn_cache_simulate(docs, pos, 10, cap, "agnostic")
        b = la.lazy_attn_cache_simulate(docs, pos, 10, cap, "aware")
        assert a > b
    hits = [la.lazy_attn_cache_simulate(docs, pos, 10, c, "agnostic") for c in (10, 100, 1000)]
    assert hits == sorted(hits)


def test_argument_checks():
    with pytest.raises(la.LazyAttnError, match="position"):
        la.lazy_attn_cache_simulate([0, 1], [0, 5], 2, 4, "aware")
    with pytest.raises(la.LazyAttnError, match="document id"):
        la.lazy_attn_cache_simulate([-1], None, 1, 4)
    with pytest.raises(la.LazyAttnError, match="pos is NULL"):
        la.lazy_attn_cache_simulate([0], None, 2, 4, "aware")


def test_table_1_shaped_report():
    from position_agnostic_kv_lazy_amd.cache_sim import BUDGETS_GB, SKEWS, table
    t = table(queries=500, docs=5000, docs_per_query=10)
    assert len(t["rows"]) == len(BUDGETS_GB) * len(SKEWS)
    for name in SKEWS:
        ag = [t["rows"][f"{gb}GB/{name}"]["agnostic"] for gb in BUDGETS_GB]
        aw = [t["rows"][f"{gb}GB/{name}"]["aware"] for gb in BUDGETS_GB]
        assert ag == sorted(ag) and aw == sorted(aw)  # more budget, more hits
        assert all(a >= b for a, b in zip(ag, aw))

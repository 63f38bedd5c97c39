"""Table-1-shaped hit ratios from the document-cache simulator.

    python -m position_agnostic_kv_lazy_amd.cache_sim [--queries Q] [--docs N]
        [--docs-per-query K] [--doc-tokens T] [--bytes-per-token B]

Replays a synthetic RAG query stream (Zipf document popularity at the paper's
Low / Mid / High skews 1.1 / 1.5 / 2.1, K documents per query in random order,
a document's prompt position = its slot) against KV budgets of 1, 5, 10, 50 GB
and the ~66 GB left on a 96 GB GPU ("LazyAttention" §2 Table 1 and its
footnote), for a position-agnostic cache (one copy per document: this
library's pool) and a position-aware one (one copy per (document, position)),
both with LRU eviction, through lazy_attn_cache_simulate.  A budget holds
budget / (T x B) entries; the paper states neither T nor its eviction policy,
so the cells are an illustration of the model, not a reproduction of Table 1.
Prints one JSON object.
"""
from __future__ import annotations

import argparse
import json
import os
import sys

BUDGETS_GB = (1, 5, 10, 50, 66)
SKEWS = {"low": 1.1, "mid": 1.5, "high": 2.1}


def table(queries=20000, docs=100_000, docs_per_query=10, doc_tokens=512,
          bytes_per_token=131072, seed=0):
    from workloads import doc_trace

    from .binding import lazy_attn_cache_simulate
    per_entry = doc_tokens * bytes_per_token
    out = {"entry_bytes": per_entry, "queries": queries, "docs": docs,
           "docs_per_query": docs_per_query, "rows": {}}
    for name, alpha in SKEWS.items():
        d, p = doc_trace(queries, docs, alpha, docs_per_query, seed)
        for gb in BUDGETS_GB:
            cap = int(gb * 1e9 // per_entry)
            row = {}
            for policy in ("agnostic", "aware"):
                h = lazy_attn_cache_simulate(d, p, docs_per_query, cap, policy, "lru")
                row[policy] = round(100.0 * h / len(d), 2)
            out["rows"][f"{gb}GB/{name}"] = dict(row, entries=cap)
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--queries", type=int, default=20000)
    ap.add_argument("--docs", type=int, default=100_000)
    ap.add_argument("--docs-per-query", type=int, default=10)
    ap.add_argument("--doc-tokens", type=int, default=512)
    ap.add_argument("--bytes-per-token", type=int, default=131072,
                    help="K+V bytes per token over all layers (Llama-3-8B bf16: 131072)")
    a = ap.parse_args(argv)
    print(json.dumps(table(a.queries, a.docs, a.docs_per_query, a.doc_tokens,
                           a.bytes_per_token)))


if __name__ == "__main__":
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    if root not in sys.path:
        sys.path.insert(0, root)
    main()

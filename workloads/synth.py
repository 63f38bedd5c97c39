"""Seeded synthetic workloads for lazy-RoPE paged attention.

A *document* is a run of tokens whose key/value vectors live once in a shared
block pool; a *request* lists segments (documents, private question blocks or
new prompt tokens), each with the logical position of its first token.  The
same physical document may be placed at different logical offsets by
different requests, which is the reuse pattern the LazyAttention paper
("LazyAttention: Efficient Retrieval-Augmented Generation with Deferred
Positional Encoding", §1 problem statement and §2 Zipf model) is about.

Value recipe (all seeded, reproducible):
  * key/value/query entries are N(0, 1) float32 draws; in bf16 workloads they
    are rounded to bf16 with round-to-nearest-even and stored as raw uint16
    bits, so the GPU and the oracle see the identical numbers;
  * every document draws from its own generator, seeded by
    (value seed, tag, document id), so any subset of the pool can be
    regenerated independently;
  * document mixes: popularity of document d is proportional to (d+1)^-alpha;
    a request draws its documents without replacement, shuffles them and
    places them back to back from position 0, followed by an optional private
    question segment (decode) or the new prompt tokens (prefill).

Pool layout in this module is the *logical* one, [block, kv_head, slot, dim],
for both K and V; the device layout of V is produced at upload time.
"""
from __future__ import annotations

import concurrent.futures as _cf
import math
import os
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

__all__ = [
    "Segment",
    "Workload",
    "MixedWorkload",
    "CONFIGS",
    "segment_writes",
    "doc_trace",
    "segment_slots",
    "private_copies",
    "make_config",
    "make_no_sharing_decode",
    "build_workload",
    "zipf_probs",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
]


# --------------------------------------------------------------------------
# bf16 storage helpers (value encoding only)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round-to-nearest-even), returning uint16 bits.

    Inputs here are finite N(0,1) draws, so NaN/Inf handling is not needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


BF16_QNAN = np.uint16(0x7FC0)


# --------------------------------------------------------------------------
# Data model
# --------------------------------------------------------------------------
@dataclass
class Segment:
    """A contiguous run of tokens at logical positions start .. start+n_tokens-1.

    Token t of the segment sits in physical block blocks[t // block_size],
    slot t % block_size.  is_new marks the new prompt tokens of a prefill
    request (causally masked among themselves).
    """

    start: int
    n_tokens: int
    blocks: np.ndarray
    is_new: bool = False


@dataclass
class Workload:
    name: str
    kind: str  # "decode" or "prefill"
    dtype: str  # "bf16" or "f32"
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    rope_base: float
    scale: float
    k_pool: np.ndarray  # [nb, Hkv, BS, D]; uint16 bf16 bits or float32
    v_pool: np.ndarray  # [nb, Hkv, BS, D]; same encoding as k_pool
    requests: List[List[Segment]]
    q: np.ndarray  # decode [B, Hq, D]; prefill [T, Hq, D]
    q_pos: np.ndarray  # decode: query position per request; prefill: first new-token position
    cu_q: Optional[np.ndarray] = None  # prefill: [B+1] row offsets into q
    meta: dict = field(default_factory=dict)

    # ---- derived sizes -------------------------------------------------
    @property
    def batch(self) -> int:
        return len(self.requests)

    @property
    def num_blocks(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def blocks_per_request(self) -> np.ndarray:
        return np.array([sum(len(s.blocks) for s in r) for r in self.requests], dtype=np.int64)

    def keys_per_request(self) -> np.ndarray:
        return np.array([sum(s.n_tokens for s in r) for r in self.requests], dtype=np.int64)

    def q_len(self, r: int) -> int:
        if self.kind == "decode":
            return 1
        return int(self.cu_q[r + 1] - self.cu_q[r])

    def max_position(self) -> int:
        """Largest logical position used by any key or query."""
        mx = 0
        for r, segs in enumerate(self.requests):
            for s in segs:
                if s.n_tokens:
                    mx = max(mx, s.start + s.n_tokens - 1)
            if self.kind == "decode":
                mx = max(mx, int(self.q_pos[r]))
            else:
                mx = max(mx, int(self.q_pos[r]) + self.q_len(r) - 1)
        return mx

    def table_rows(self) -> int:
        """Rows of cos/sin table that cover every position (at least one block)."""
        return max(self.max_position() + 1, self.block_size)

    def is_bf16(self) -> bool:
        return self.dtype == "bf16"

    def values_f32(self, arr: np.ndarray) -> np.ndarray:
        return bf16_bits_to_f32(arr) if self.is_bf16() else np.asarray(arr, dtype=np.float32)

    def logical_kv_bytes(self) -> int:
        """K+V bytes a decode step must read: keys x kv_heads x D x 2 (K,V) x elem size."""
        elem = 2 if self.is_bf16() else 4
        return int(self.keys_per_request().sum()) * self.num_kv_heads * self.head_dim * 2 * elem

    def unique_kv_bytes(self) -> int:
        """K+V bytes of the distinct pool blocks the tables touch, each counted once
        with its valid slots: what HBM must deliver at least when every shared
        block is read once per launch."""
        elem = 2 if self.is_bf16() else 4
        tokens = {}
        for segs in self.requests:
            for s in segs:
                for k, b in enumerate(np.asarray(s.blocks).ravel()):
                    nv = min(self.block_size, int(s.n_tokens) - k * self.block_size)
                    tokens[int(b)] = max(tokens.get(int(b), 0), nv)
        return int(sum(tokens.values())) * self.num_kv_heads * self.head_dim * 2 * elem

    def prefill_flops(self) -> int:
        """4*D*Hq per unmasked (query, key) pair, summed over all new tokens."""
        assert self.kind == "prefill"
        total = 0
        for r, segs in enumerate(self.requests):
            T = self.q_len(r)
            p0 = int(self.q_pos[r])
            for s in segs:
                if not s.is_new:
                    total += T * s.n_tokens
                else:
                    # key at position s.start+t visible to query at p0+j iff s.start+t <= p0+j
                    for j in range(T):
                        total += max(0, min(s.n_tokens, p0 + j - s.start + 1))
        return 4 * self.head_dim * self.num_q_heads * total


@dataclass
class MixedWorkload:
    """One decode batch and one prefill batch over one shared pool."""

    name: str
    decode: Workload
    prefill: Workload


# --------------------------------------------------------------------------
# Generators
# --------------------------------------------------------------------------
def zipf_probs(n: int, alpha: float) -> np.ndarray:
    w = np.arange(1, n + 1, dtype=np.float64) ** (-float(alpha))
    return w / w.sum()


def _normal_block(seed_words: Sequence[int], shape, encode_bf16: bool) -> np.ndarray:
    rng = np.random.default_rng(list(seed_words))
    x = rng.standard_normal(shape, dtype=np.float32)
    return f32_to_bf16_bits(x) if encode_bf16 else x


_TAG_K, _TAG_V, _TAG_Q, _TAG_PK, _TAG_PV = 1, 2, 3, 4, 5


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def build_workload(
    *,
    name: str,
    kind: str,
    dtype: str,
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    block_size: int,
    rope_base: float,
    doc_lens: Sequence[int],
    requests: Sequence[Sequence[tuple]],
    seed: int,
    scale: Optional[float] = None,
    q_pos_override: Optional[Sequence[int]] = None,
    poison_tail: bool = False,
    shared_pool: Optional[tuple] = None,
    extra_blocks: int = 0,
) -> Workload:
    """Materialise a workload from explicit request specs.

    Each request is a sequence of items:
      ("doc", d)            document d at the running cursor
      ("doc", d, start)     document d at an explicit start position
      ("priv", n)           n private (unshared) tokens at the cursor
      ("priv", n, start)    ... at an explicit start position
      ("new", n)            n new prompt tokens (prefill; must be last)
    The cursor advances past every item.  For decode the query position is
    the final cursor unless q_pos_override gives it.

    Documents occupy consecutive pool blocks in id order; private and new
    segments get fresh blocks appended after the documents.  poison_tail fills
    the unused slots of partial blocks with NaN so tests can prove they are
    never read into the result.
    """
    assert kind in ("decode", "prefill") and dtype in ("bf16", "f32")
    BS, Hkv, D = block_size, num_kv_heads, head_dim
    bf = dtype == "bf16"
    doc_lens = [int(x) for x in doc_lens]
    doc_blocks = [(n + BS - 1) // BS for n in doc_lens]
    doc_first = np.concatenate([[0], np.cumsum(doc_blocks)]).astype(np.int64)
    n_doc_blocks = int(doc_first[-1])

    # ---- lay out segments and count private blocks -------------------
    plan = []  # per request: list of (kind, start, n_tokens, payload)
    n_priv_blocks = 0
    for items in requests:
        cursor = 0
        segs = []
        for it in items:
            tag = it[0]
            if tag == "doc":
                d = int(it[1])
                start = int(it[2]) if len(it) > 2 else cursor
                segs.append(("doc", start, doc_lens[d], d))
                cursor = start + doc_lens[d]
            elif tag in ("priv", "new"):
                n = int(it[1])
                start = int(it[2]) if len(it) > 2 else cursor
                nb = (n + BS - 1) // BS
                segs.append((tag, start, n, (n_priv_blocks, nb)))
                n_priv_blocks += nb
                cursor = start + n
            else:
                raise ValueError(f"unknown request item {it!r}")
        plan.append((segs, cursor))

    priv_base = n_doc_blocks + int(extra_blocks)
    nb_total = priv_base + n_priv_blocks

    # ---- pool values ---------------------------------------------------
    if shared_pool is not None:
        k_pool, v_pool, shared_priv_base = shared_pool
        priv_base = shared_priv_base
        assert k_pool.shape[0] >= priv_base + n_priv_blocks
    else:
        store = np.uint16 if bf else np.float32
        k_pool = np.empty((nb_total, Hkv, BS, D), dtype=store)
        v_pool = np.empty((nb_total, Hkv, BS, D), dtype=store)

        def fill_doc(d):
            a, nb = int(doc_first[d]), doc_blocks[d]
            shp = (nb, Hkv, BS, D)
            k_pool[a:a + nb] = _normal_block((seed, _TAG_K, d), shp, bf)
            v_pool[a:a + nb] = _normal_block((seed, _TAG_V, d), shp, bf)

        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill_doc, range(len(doc_lens))))
        if extra_blocks:
            shp = (int(extra_blocks), Hkv, BS, D)
            k_pool[n_doc_blocks:priv_base] = _normal_block((seed, _TAG_PK, 1 << 30), shp, bf)
            v_pool[n_doc_blocks:priv_base] = _normal_block((seed, _TAG_PV, 1 << 30), shp, bf)
        if n_priv_blocks:
            shp = (n_priv_blocks, Hkv, BS, D)
            k_pool[priv_base:] = _normal_block((seed, _TAG_PK, 0), shp, bf)
            v_pool[priv_base:] = _normal_block((seed, _TAG_PV, 0), shp, bf)

    # ---- segments ------------------------------------------------------
    reqs: List[List[Segment]] = []
    q_pos = []
    q_rows = []
    for r, (segs, cursor) in enumerate(plan):
        out = []
        newcount = 0
        newstart = None
        for tag, start, n, payload in segs:
            if tag == "doc":
                a = int(doc_first[payload])
                blocks = np.arange(a, a + (n + BS - 1) // BS, dtype=np.int64)
                out.append(Segment(start, n, blocks, False))
            else:
                off, nb = payload
                blocks = np.arange(priv_base + off, priv_base + off + nb, dtype=np.int64)
                out.append(Segment(start, n, blocks, tag == "new"))
                if tag == "new":
                    newcount, newstart = n, start
        reqs.append(out)
        if kind == "decode":
            q_pos.append(int(q_pos_override[r]) if q_pos_override is not None else cursor)
            q_rows.append(1)
        else:
            if newstart is None:
                raise ValueError("prefill request needs a ('new', n) item")
            q_pos.append(newstart)
            q_rows.append(newcount)

    if poison_tail:
        nan = BF16_QNAN if bf else np.float32(np.nan)
        for segs in reqs:
            for s in segs:
                tail = s.n_tokens % BS
                if tail:
                    b = int(s.blocks[-1])
                    k_pool[b, :, tail:, :] = nan
                    v_pool[b, :, tail:, :] = nan

    T = int(sum(q_rows))
    q = _normal_block((seed, _TAG_Q, 0), (T, num_q_heads, D), bf)
    cu_q = None
    if kind == "prefill":
        cu_q = np.concatenate([[0], np.cumsum(q_rows)]).astype(np.int64)

    return Workload(
        name=name,
        kind=kind,
        dtype=dtype,
        num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads,
        head_dim=D,
        block_size=BS,
        rope_base=float(rope_base),
        scale=float(scale) if scale is not None else 1.0 / math.sqrt(D),
        k_pool=k_pool,
        v_pool=v_pool,
        requests=reqs,
        q=q,
        q_pos=np.asarray(q_pos, dtype=np.int64),
        cu_q=cu_q,
        meta={"priv_base": priv_base, "n_doc_blocks": n_doc_blocks, "seed": seed},
    )


def zipf_requests(n_req, n_pool_docs, docs_per_req, alpha, seed, tail_item=None):
    """Request specs: docs drawn Zipf(alpha) without replacement, shuffled."""
    rng = np.random.default_rng(seed)
    p = zipf_probs(n_pool_docs, alpha)
    specs = []
    for _ in range(n_req):
        docs = rng.choice(n_pool_docs, size=docs_per_req, replace=False, p=p)
        docs = rng.permutation(docs)
        items = [("doc", int(d)) for d in docs]
        if tail_item is not None:
            items.append(tail_item)
        specs.append(items)
    return specs


# --------------------------------------------------------------------------
# The five benchmark configurations
# --------------------------------------------------------------------------
CONFIGS = {
    1: "tiny_decode_f32: 1 request, Hq=Hkv=1, D=64, fp32, 4 docs x 32 tokens at 0/32/64/96, "
    "32-token question at 128..159, query at 160, theta 1e4",
    2: "llama3_8b_decode: B=64, Hq=32/Hkv=8, D=128, bf16, BS=16, 200-doc pool x 512 tokens, "
    "10 docs per request Zipf(1.0) + 64-token question, theta 5e5",
    3: "llama3_8b_prefill: B=8, 20 docs x 512 per request Zipf(1.0) over 500 docs, 512 new tokens",
    4: "long_decode: B=16, 64 docs x 1024 per request Zipf(1.2) over 2000 docs (64K context)",
    5: "mixed: 1000-doc pool x 512; 128 decode requests x 20 docs Zipf(0.8) + "
    "4 prefill requests x 20 docs + 1024 new tokens",
}


def make_config(cfg: int, *, dtype: Optional[str] = None, scale_down: int = 1):
    """Build benchmark configuration cfg (1..5).

    dtype overrides the element type (e.g. "f32" for the fp32 test mode).
    scale_down > 1 shrinks batch and document counts for quick tests while
    keeping head shapes, block size and the Zipf structure.
    """
    vs, zs = 1000 + cfg, 2000 + cfg
    sd = max(1, int(scale_down))
    if cfg == 1:
        return build_workload(
            name="tiny_decode_f32", kind="decode", dtype=dtype or "f32",
            num_q_heads=1, num_kv_heads=1, head_dim=64, block_size=16, rope_base=1e4,
            doc_lens=[32, 32, 32, 32],
            requests=[[("doc", 0), ("doc", 1), ("doc", 2), ("doc", 3), ("priv", 32)]],
            seed=vs,
        )
    common = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16)
    if cfg == 2:
        n_docs, B = 200, max(1, 64 // sd)
        specs = zipf_requests(B, n_docs, 10, 1.0, zs, tail_item=("priv", 64))
        return build_workload(name="llama3_8b_decode", kind="decode", dtype=dtype or "bf16",
                              rope_base=5e5, doc_lens=[512] * n_docs, requests=specs, seed=vs, **common)
    if cfg == 3:
        n_docs, B = 500, max(1, 8 // sd)
        new = 512 // sd
        specs = zipf_requests(B, n_docs, 20, 1.0, zs, tail_item=("new", new))
        return build_workload(name="llama3_8b_prefill", kind="prefill", dtype=dtype or "bf16",
                              rope_base=5e5, doc_lens=[512] * n_docs, requests=specs, seed=vs, **common)
    if cfg == 4:
        n_docs, B, per = 2000 // sd, max(1, 16 // sd), 64 // sd
        specs = zipf_requests(B, n_docs, per, 1.2, zs)
        return build_workload(name="long_decode", kind="decode", dtype=dtype or "bf16",
                              rope_base=5e5, doc_lens=[1024] * n_docs, requests=specs, seed=vs, **common)
    if cfg == 5:
        n_docs = 1000 // sd
        Bd, Bp, new = max(1, 128 // sd), max(1, 4 // sd), 1024 // sd
        dspecs = zipf_requests(Bd, n_docs, 20, 0.8, zs)
        pspecs = zipf_requests(Bp, n_docs, 20, 0.8, zs + 100, tail_item=("new", new))
        pre = build_workload(name="mixed_prefill", kind="prefill", dtype=dtype or "bf16",
                             rope_base=5e5, doc_lens=[512] * n_docs, requests=pspecs, seed=vs, **common)
        dec = build_workload(name="mixed_decode", kind="decode", dtype=dtype or "bf16",
                             rope_base=5e5, doc_lens=[512] * n_docs, requests=dspecs, seed=vs,
                             shared_pool=(pre.k_pool, pre.v_pool, pre.meta["priv_base"]), **common)
        return MixedWorkload(name="mixed_step", decode=dec, prefill=pre)
    raise ValueError(f"unknown config {cfg}")


def make_no_sharing_decode(*, dtype: Optional[str] = None, scale_down: int = 1):
    """Configuration 2's shapes with no document shared between requests.

    64 requests x 10 documents of 512 tokens + a 64-token question, as in
    configuration 2, but request r reads its own documents 10r .. 10r+9 (in a
    seeded random order), so no block is read twice in a launch and the
    logical K+V bytes equal the unique bytes: a control for the cache-assisted
    rate of the shared-document mix.
    """
    sd = max(1, int(scale_down))
    B, per = max(1, 64 // sd), 10
    rng = np.random.default_rng(2012)
    specs = []
    for r in range(B):
        docs = rng.permutation(np.arange(per * r, per * (r + 1)))
        specs.append([("doc", int(d)) for d in docs] + [("priv", 64)])
    return build_workload(name="llama3_8b_decode_no_sharing", kind="decode",
                          dtype=dtype or "bf16", num_q_heads=32, num_kv_heads=8, head_dim=128,
                          block_size=16, rope_base=5e5, doc_lens=[512] * (per * B),
                          requests=specs, seed=1012)


def segment_slots(w, positions: str = "index"):
    """Flat slot ids and position indices of every distinct segment (see segment_writes)."""
    BS = w.block_size
    seen = {}
    sl, ps = [], []
    for segs in w.requests:
        for seg in segs:
            key = tuple(int(b) for b in np.asarray(seg.blocks).ravel())
            if key in seen:
                if positions == "absolute" and seen[key] != int(seg.start):
                    raise ValueError(f"blocks {key[:3]}... placed at starts {seen[key]} and "
                                     f"{int(seg.start)}: no single absolute position")
                continue
            seen[key] = int(seg.start)
            t = np.arange(int(seg.n_tokens))
            blk = np.asarray(key, np.int64)[t // BS]
            sl.append(blk * BS + t % BS)
            ps.append(t if positions == "index" else int(seg.start) + t)
    return np.concatenate(sl).astype(np.int64), np.concatenate(ps).astype(np.int32)


def private_copies(w):
    """Per-request private copies of every segment, as a materialising cache would hold them.

    Request r's segments are laid out in fresh blocks of a new pool (numbered
    from 0), each at its own logical positions.  Returns (requests, src_slots,
    dst_slots, positions): the new segment lists (with start 0, for a pool
    whose keys are pre-rotated at absolute positions), and per token the
    source slot in w's pool, the destination slot and the logical position.
    Pure bookkeeping.
    """
    BS = w.block_size
    nxt = 0
    reqs, src, dst, pos = [], [], [], []
    for segs in w.requests:
        out = []
        for seg in segs:
            n = int(seg.n_tokens)
            nb = (n + BS - 1) // BS
            blocks = np.arange(nxt, nxt + nb, dtype=np.int64)
            nxt += nb
            t = np.arange(n)
            src.append(np.asarray(seg.blocks, np.int64)[t // BS] * BS + t % BS)
            dst.append(blocks[t // BS] * BS + t % BS)
            pos.append(int(seg.start) + t)
            out.append(Segment(0, n, blocks, seg.is_new))
        reqs.append(out)
    return (reqs, np.concatenate(src).astype(np.int64), np.concatenate(dst).astype(np.int64),
            np.concatenate(pos).astype(np.int32))


def segment_writes(w, positions: str = "index"):
    """Token-level cache-write inputs for the physical segments of w's tables.

    Every distinct block list in w.requests is listed once; its token t (at
    block blocks[t // BS], slot t % BS) contributes the raw key and value from
    w's pools, the flat slot id blocks[t // BS] * BS + t % BS and a position
    index: t itself (positions="index", the in-document index) or the logical
    position start + t (positions="absolute"; a block list placed at two
    different starts then has no single absolute position and is rejected).
    Pure bookkeeping -- no rotation happens here.

    Returns (k [n, Hkv, D], v [n, Hkv, D], slots int64 [n], pos int32 [n]).
    """
    BS = w.block_size
    seen = {}
    ks, vs, sl, ps = [], [], [], []
    for segs in w.requests:
        for seg in segs:
            key = tuple(int(b) for b in np.asarray(seg.blocks).ravel())
            if key in seen:
                if positions == "absolute" and seen[key] != int(seg.start):
                    raise ValueError(f"blocks {key[:3]}... placed at starts {seen[key]} and "
                                     f"{int(seg.start)}: no single absolute position")
                continue
            seen[key] = int(seg.start)
            t = np.arange(int(seg.n_tokens))
            blk = np.asarray(key, np.int64)[t // BS]
            slot = t % BS
            ks.append(w.k_pool[blk, :, slot, :])
            vs.append(w.v_pool[blk, :, slot, :])
            sl.append(blk * BS + slot)
            ps.append(t if positions == "index" else int(seg.start) + t)
    return (np.ascontiguousarray(np.concatenate(ks)), np.ascontiguousarray(np.concatenate(vs)),
            np.concatenate(sl).astype(np.int64), np.concatenate(ps).astype(np.int32))


def doc_trace(n_queries: int, num_docs: int, alpha: float, docs_per_query: int, seed: int):
    """Document accesses of a RAG query stream (the §2 / Table 1 workload shape).

    Each query retrieves docs_per_query distinct documents drawn with Zipf
    popularity p(d) ~ (d+1)^-alpha (d = popularity rank), in random order; a
    document's prompt position is its slot in the query (0 .. K-1), so it may
    appear at D = docs_per_query positions.  Returns (docs int64, pos int32),
    one entry per access, query after query.  Pure sampling.
    """
    rng = np.random.default_rng([3000, seed])
    cdf = np.cumsum(zipf_probs(num_docs, alpha))
    K = docs_per_query
    if K > num_docs:
        raise ValueError("more documents per query than documents")

    def draws(n):  # inverse-CDF Zipf samples
        return np.minimum(np.searchsorted(cdf, rng.random(n), side="right"), num_docs - 1)

    docs = np.empty((n_queries, K), np.int64)
    stream = draws(4 * K * n_queries + 64).tolist()
    at = 0
    for qi in range(n_queries):
        row, seen = [], set()
        while len(row) < K:  # distinct documents per query
            if at == len(stream):
                stream, at = draws(4 * K + 64).tolist(), 0
            d = stream[at]
            at += 1
            if d not in seen:
                seen.add(d)
                row.append(d)
        docs[qi] = row
    docs = rng.permuted(docs, axis=1)
    pos = np.broadcast_to(np.arange(K, dtype=np.int32), (n_queries, K))
    return docs.ravel(), np.ascontiguousarray(pos).ravel()

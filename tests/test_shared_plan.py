"""The shared-segment decode plan (host only): structure and coverage.

The plan must hand every (request, key) of the segment lists to exactly one
(work item, member) with the right logical position, group identical
segments of different requests into shared items, give each request a
contiguous range of partial slots, and respect the per-item member limit
32 / G.  Everything here is host code; no kernel runs.
"""
import numpy as np
import pytest

import position_agnostic_kv_lazy_amd as la
from workloads import Segment, make_config


def _params(**kw):
    d = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, num_blocks=100000,
             dtype="bf16", scale=0.088, max_pos=200000)
    d.update(kw)
    return la.make_params(**d)


def decode_plan(info, blob):
    """Split the blob into its sections (layout of lazy_attn.h)."""
    n_items, n_mem, batch, n_words = info.n_items, info.n_members, info.batch, info.n_words
    b = blob.view(np.uint8)
    items = b[:16 * n_items].view(np.int32).reshape(n_items, 4)
    o = 16 * n_items
    mem = b[o:o + 16 * n_mem].view(np.int32).reshape(n_mem, 4)
    o += 16 * n_mem
    rps = b[o:o + 4 * (batch + 1)].view(np.int32)
    o += (4 * (batch + 1) + 15) // 16 * 16
    words = b[o:o + 8 * n_words].view(np.uint64)
    assert o + 8 * n_words == info.plan_bytes == len(blob)
    return items, mem, rps, words


def covered(info, blob, BS=16):
    """{(request, position): (block, slot)} and the slots of each member, from the plan."""
    items, mem, rps, words = decode_plan(info, blob)
    seen = {}
    slot_owner = {}
    for w0, nb, m0, nm in items:
        ws = words[w0:w0 + nb]
        ids = (ws & np.uint64(0xFFFFFFFF)).astype(np.int64)
        t0 = ((ws >> np.uint64(32)) & np.uint64(0xFFFFFF)).astype(np.int64)
        nv = ((ws >> np.uint64(56)) & np.uint64(0x7F)).astype(np.int64) + 1
        for r, s, slot, pad in mem[m0:m0 + nm]:
            assert pad == 0
            assert rps[r] <= slot < rps[r + 1], "partial slot outside its request's range"
            slot_owner.setdefault(int(slot), set()).add((int(r), int(s), int(w0)))
            for b, t, n in zip(ids, t0, nv):
                for i in range(n):
                    key = (int(r), int(s) + int(t) + i)
                    assert key not in seen, f"key {key} covered twice"
                    seen[key] = (int(b), i)
    return seen, slot_owner, items, mem, rps


def expected(requests, BS=16):
    out = {}
    for r, segs in enumerate(requests):
        for sg in segs:
            for t in range(sg.n_tokens):
                out[(r, sg.start + t)] = (int(sg.blocks[t // BS]), t % BS)
    return out


def _reqs(w):
    return [[Segment(int(s.start), int(s.n_tokens), np.asarray(s.blocks), bool(s.is_new))
             for s in segs] for segs in w.requests]


@pytest.mark.parametrize("mib", [0, 1, 3, 7])
def test_plan_covers_every_key_once_config2(mib):
    w = make_config(2, scale_down=4)
    p = _params(num_blocks=w.num_blocks, max_pos=w.table_rows())
    info, blob = la.lazy_attn_plan_shared_decode(p, w.requests, mib)
    seen, slots, items, mem, rps = covered(info, blob)
    assert seen == expected(_reqs(w))
    # one member per partial slot, and every slot of every request used
    assert sorted(slots) == list(range(info.n_members))
    assert all(len(v) == 1 for v in slots.values())
    assert rps[0] == 0 and rps[-1] == info.n_members and np.all(np.diff(rps) > 0)
    assert info.members_per_item == 32 // 4
    assert np.all(items[:, 3] <= 8) and np.all(items[:, 3] >= 1)
    assert np.all(np.diff(items[:, 1]) <= 0)  # longest chunks first
    if mib:
        assert info.max_item_blocks == mib
    else:
        assert 16 <= info.max_item_blocks <= 96
    assert np.all(items[:, 1] <= info.max_item_blocks)
    assert info.workspace_bytes == info.n_members * 32 * 130 * 4


def test_automatic_chunk_length():
    """The automatic length comes from the launch-time model over 16..96 blocks,
    and every unit is cut into chunks of nearly equal length (no short tail)."""
    from workloads import make_no_sharing_decode
    w = make_no_sharing_decode()  # 64 requests, each one private run of 324 blocks
    p = _params(num_blocks=w.num_blocks, max_pos=w.table_rows())
    info, blob = la.lazy_attn_plan_shared_decode(p, w.requests)
    assert info.max_item_blocks == 96
    items = decode_plan(info, blob)[0]
    # 4 chunks of 81 per request: 256 items x 8 kv heads fill the 2048 wave slots once
    assert info.n_items == 256 and set(items[:, 1].tolist()) == {81}
    w = make_config(2)
    p = _params(num_blocks=w.num_blocks, max_pos=w.table_rows())
    info, blob = la.lazy_attn_plan_shared_decode(p, w.requests)
    assert info.max_item_blocks == 32
    seen, slots, items, mem, rps = covered(info, blob)
    assert seen == expected(_reqs(w))
    for L in (0, 24, 40):
        info, blob = la.lazy_attn_plan_shared_decode(p, w.requests, L)
        assert 16 <= info.max_item_blocks <= 96
        items = decode_plan(info, blob)[0]
        assert items[:, 1].max() <= info.max_item_blocks


def test_passing_the_chosen_length_back_gives_the_same_plan():
    import ctypes
    from position_agnostic_kv_lazy_amd import binding as B
    w = make_config(2, scale_down=2)
    p = _params(num_blocks=w.num_blocks, max_pos=w.table_rows())
    a = B._segment_arrays(w.requests)
    ptrs = (a[0].ctypes.data_as(B._i64p), a[1].ctypes.data_as(B._i64p),
            a[2].ctypes.data_as(B._i64p), a[3].ctypes.data_as(B._u8p),
            a[4].ctypes.data_as(B._i64p), a[5].ctypes.data_as(B._i64p))
    info = B.la_shared_plan_info()
    assert B._lib.lazy_attn_plan_shared_decode(ctypes.byref(p), len(w.requests), *ptrs, 0,
                                               ctypes.byref(info), None, 0) == 0
    auto = np.zeros(int(info.plan_bytes), np.uint8)
    assert B._lib.lazy_attn_plan_shared_decode(ctypes.byref(p), len(w.requests), *ptrs, 0,
                                               ctypes.byref(info), auto.ctypes.data,
                                               auto.nbytes) == 0
    info2, fixed = la.lazy_attn_plan_shared_decode(p, w.requests, int(info.max_item_blocks))
    assert info2.max_item_blocks == info.max_item_blocks
    assert np.array_equal(auto, fixed)


def test_chunks_of_a_unit_differ_by_at_most_one_block():
    doc = np.arange(10)  # 10 blocks, shared by two requests
    reqs = [[Segment(0, 160, doc, False)], [Segment(500, 160, doc, False)]]
    p = _params(num_blocks=20, max_pos=2000)
    for L, want in ((4, [3, 3, 4]), (3, [2, 2, 3, 3]), (10, [10]), (9, [5, 5])):
        info, blob = la.lazy_attn_plan_shared_decode(p, reqs, L)
        seen, _, items, _, rps = covered(info, blob)
        assert seen == expected(reqs)
        assert sorted(items[:, 1].tolist()) == want, L
        assert list(np.diff(rps)) == [len(want)] * 2


def test_identical_segments_share_items():
    """A document listed by several requests at different offsets is one item
    (up to 32 / G members); different documents are not merged."""
    A, B = np.array([3, 4]), np.array([7, 8])
    reqs = [[Segment(0, 20, A, False), Segment(20, 32, B, False)],
            [Segment(0, 32, B, False), Segment(32, 20, A, False)],
            [Segment(100, 20, A, False)],
            [Segment(5, 20, np.array([3, 9]), False)]]  # same first block, other list
    p = _params(num_blocks=20, max_pos=300)
    info, blob = la.lazy_attn_plan_shared_decode(p, reqs)
    seen, slots, items, mem, rps = covered(info, blob)
    assert seen == expected(reqs)
    assert info.n_items == 3 and info.n_words == 6
    nmem = sorted(int(x) for x in items[:, 3])
    assert nmem == [1, 2, 3]  # A: 3 requests, B: 2, the other list: 1


@pytest.mark.parametrize("Hq,Hkv,C", [(16, 16, 32), (16, 8, 16), (32, 8, 8), (32, 4, 4),
                                      (32, 2, 2)])
def test_members_per_item_follow_the_group_size(Hq, Hkv, C):
    doc = np.arange(4)
    reqs = [[Segment(17 * r, 64, doc, False)] for r in range(70)]
    p = _params(num_q_heads=Hq, num_kv_heads=Hkv, num_blocks=10, max_pos=2000)
    info, blob = la.lazy_attn_plan_shared_decode(p, reqs)
    seen, slots, items, mem, rps = covered(info, blob)
    assert seen == expected(reqs)
    assert info.members_per_item == C
    assert info.n_items == -(-70 // C) and int(items[:, 3].max()) == C


def test_same_document_twice_in_one_request_and_partial_blocks():
    doc = np.array([5, 6, 2])  # 40 tokens: the last block holds 8
    reqs = [[Segment(0, 40, doc, False), Segment(300, 40, doc, False), Segment(40, 3, np.array([9]), True)],
            [Segment(1000, 40, doc, False)]]
    p = _params(num_blocks=10, max_pos=2000)
    info, blob = la.lazy_attn_plan_shared_decode(p, reqs, 2)
    seen, slots, items, mem, rps = covered(info, blob)
    assert seen == expected(reqs)
    # request 0: two chunks per copy of the document + the new-token segment
    assert list(np.diff(rps)) == [5, 2]


def test_plan_rejects_what_the_kernel_cannot_run():
    seg = [[Segment(0, 16, np.array([1]), False)]]
    with pytest.raises(la.LazyAttnError, match="UNSUPPORTED"):
        la.lazy_attn_plan_shared_decode(_params(dtype="f32"), seg)
    with pytest.raises(la.LazyAttnError, match="UNSUPPORTED"):
        la.lazy_attn_plan_shared_decode(_params(pos_encoding="alibi"), seg)
    with pytest.raises(la.LazyAttnError, match="block id"):
        la.lazy_attn_plan_shared_decode(_params(num_blocks=1), seg)
    with pytest.raises(la.LazyAttnError, match="max_pos"):
        la.lazy_attn_plan_shared_decode(_params(max_pos=10), seg)
    with pytest.raises(la.LazyAttnError, match="max_item_blocks"):
        la.lazy_attn_plan_shared_decode(_params(), seg, -1)


def test_decode_shared_checks_arguments_before_launch():
    seg = [[Segment(0, 16, np.array([1]), False)], [Segment(0, 16, np.array([1]), False)]]
    p = _params()
    info, blob = la.lazy_attn_plan_shared_decode(p, seg)
    fake = 1 << 40  # never dereferenced: the checks fail first
    with pytest.raises(la.LazyAttnError, match="batch 3 does not match"):
        la.lazy_attn_decode_shared(p, info, fake, fake, fake, fake, fake, fake, 3, fake)
    with pytest.raises(la.LazyAttnError, match="WORKSPACE_TOO_SMALL"):
        la.lazy_attn_decode_shared(p, info, fake, fake, fake, fake, fake, fake, 2, fake)
    p16 = _params(num_q_heads=32, num_kv_heads=2)  # a plan built for another group size
    with pytest.raises(la.LazyAttnError, match="do not fit"):
        la.lazy_attn_decode_shared(p16, info, fake, fake, fake, fake, fake, fake, 2, fake)
    with pytest.raises(la.LazyAttnError, match="aligned"):
        la.lazy_attn_decode_shared(p, info, fake + 4, fake, fake, fake, fake, fake, 2, fake)


def test_unshared_segments_form_one_private_run():
    """In a position-free pool a request's segments that no other request lists
    become one unit: absolute block positions, member start 0.  A document-local
    pool indexes keys inside their segment, so each segment stays its own unit."""
    D = np.array([1, 2])
    reqs = [[Segment(0, 32, D, False), Segment(32, 20, np.array([3, 4]), False),
             Segment(52, 16, np.array([5]), False), Segment(68, 2, np.array([6]), True)],
            [Segment(7, 32, D, False), Segment(39, 5, np.array([8]), True)]]
    p = _params(num_blocks=20, max_pos=300)
    info, blob = la.lazy_attn_plan_shared_decode(p, reqs)
    seen, slots, items, mem, rps = covered(info, blob)
    assert seen == expected(reqs)
    # D (2 members), request 0's run (4 blocks), request 1's run (1 block)
    assert info.n_items == 3 and info.n_words == 2 + 4 + 1
    assert list(np.diff(rps)) == [2, 2]
    _, _, _, words = decode_plan(info, blob)
    runs = [it for it in items if it[3] == 1]
    for w0, nb, m0, nm in runs:
        assert mem[m0][1] == 0  # the member starts at 0: positions are absolute
    t0 = ((words >> np.uint64(32)) & np.uint64(0xFFFFFF)).astype(np.int64)
    run0 = next(it for it in runs if mem[it[2]][0] == 0)
    assert list(t0[run0[0]:run0[0] + run0[1]]) == [32, 48, 52, 68]
    pl = _params(num_blocks=20, max_pos=300, pool_mode="doc_local")
    info_l, blob_l = la.lazy_attn_plan_shared_decode(pl, reqs)
    seen_l, _, items_l, mem_l, _ = covered(info_l, blob_l)
    assert seen_l == expected(reqs)
    assert info_l.n_items == 1 + 3 + 1  # every segment its own unit

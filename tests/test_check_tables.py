"""la_params.check_tables: the GPU entry points check their tables on the
host before anything is enqueued (host only here; every case below fails its
check, so no launch is attempted and no pointer is dereferenced on a device).
"""
import numpy as np
import pytest
import torch

import position_agnostic_kv_lazy_amd as la
from workloads import Segment

FAKE = 1 << 40  # stands for device buffers the checks never reach


def _params(**kw):
    d = dict(num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16, num_blocks=10,
             dtype="bf16", scale=0.088, max_pos=1024, check_tables=True)
    d.update(kw)
    return la.make_params(**d)


def _table(p, segs):
    words, rbs, maxb = la.lazy_attn_pack_segments(p, segs)
    return np.ascontiguousarray(words), np.ascontiguousarray(rbs), maxb


def _decode(p, words, rbs, qpos, maxb, noalloc=False):
    args = (p, FAKE, FAKE, FAKE, words.ctypes.data, rbs.ctypes.data, qpos.ctypes.data, FAKE,
            len(qpos), maxb, FAKE)
    if noalloc:
        la.lazy_attn_decode_noalloc(*args)
    else:
        la.lazy_attn_decode(*args)


SEGS = [[Segment(0, 40, np.array([1, 2, 3]), False)], [Segment(5, 16, np.array([4]), False)]]


@pytest.mark.parametrize("noalloc", [False, True])
def test_decode_rejects_a_bad_block_id(noalloc):
    p = _params()
    words, rbs, maxb = _table(p, SEGS)
    qpos = np.array([40, 21], np.int32)
    words[1] = (words[1] & ~np.uint64(0xFFFFFFFF)) | np.uint64(10)  # id = num_blocks
    with pytest.raises(la.LazyAttnError, match="INVALID_ARG.*block id 10"):
        _decode(p, words, rbs, qpos, maxb, noalloc)


def test_decode_rejects_a_query_past_the_table_and_a_short_block_bound():
    p = _params()
    words, rbs, maxb = _table(p, SEGS)
    with pytest.raises(la.LazyAttnError, match="INVALID_ARG.*query positions"):
        _decode(p, words, rbs, np.array([40, 1024], np.int32), maxb)
    with pytest.raises(la.LazyAttnError, match="INVALID_ARG.*max_blocks_per_req"):
        _decode(p, words, rbs, np.array([40, 21], np.int32), maxb - 1)


def test_prefill_rejects_a_row_that_sees_no_key():
    p = _params()
    segs = [[Segment(100, 20, np.array([5, 6]), True)]]  # new tokens only, causal
    words, rbs, _ = _table(p, segs)
    cu = np.array([0, 20], np.int32)
    q0 = np.array([99], np.int32)  # the first row at 99 sees no key (keys start at 100)
    with pytest.raises(la.LazyAttnError, match="INVALID_ARG.*sees no key"):
        la.lazy_attn_prefill(p, FAKE, FAKE, FAKE, words.ctypes.data, rbs.ctypes.data,
                             cu.ctypes.data, q0.ctypes.data, FAKE, 1, 20, FAKE)


def _shared(p, blob, info, qpos):
    ws = torch.empty(int(info.workspace_bytes), dtype=torch.uint8)  # host: only its size is read
    plan = np.empty(len(blob) + 16, np.uint8)  # 16-byte aligned copy of the blob
    off = (-plan.ctypes.data) % 16
    plan[off:off + len(blob)] = blob
    la.lazy_attn_decode_shared(p, info, plan.ctypes.data + off, FAKE, FAKE, FAKE,
                               qpos.ctypes.data, FAKE, len(qpos), FAKE, None, ws)


def _plan(p, reqs):
    info, blob = la.lazy_attn_plan_shared_decode(p, reqs)
    return info, blob.copy(), 16 * info.n_items  # members start after the items


def test_shared_decode_rejects_a_corrupted_plan():
    p = _params()
    reqs = [[Segment(0, 40, np.array([1, 2, 3]), False)], [Segment(60, 40, np.array([1, 2, 3]), False)]]
    qpos = np.array([40, 100], np.int32)
    info, blob, mem0 = _plan(p, reqs)
    # a partial slot written twice (and another never)
    bad = blob.copy()
    bm = bad[mem0:mem0 + 16 * info.n_members].view(np.int32).reshape(-1, 4)
    assert info.n_members == 2
    bm[1, 2] = bm[0, 2]
    with pytest.raises(la.LazyAttnError, match="INVALID_ARG.*(outside request|twice)"):
        _shared(p, bad, info, qpos)
    # a member of a request that does not exist
    bad = blob.copy()
    bm = bad[mem0:mem0 + 16 * info.n_members].view(np.int32).reshape(-1, 4)
    bm[0, 0] = 7
    with pytest.raises(la.LazyAttnError, match="INVALID_ARG.*member 0 is malformed"):
        _shared(p, bad, info, qpos)
    # a block id outside the pool
    bad = blob.copy()
    wo = len(bad) - 8 * info.n_words
    w = bad[wo:].view(np.uint64)
    w[0] = (w[0] & ~np.uint64(0xFFFFFFFF)) | np.uint64(99)
    with pytest.raises(la.LazyAttnError, match="INVALID_ARG.*block id 99"):
        _shared(p, bad, info, qpos)
    # a query whose rotation row |m - s| is past the table
    with pytest.raises(la.LazyAttnError, match="INVALID_ARG.*rotation row"):
        _shared(p, blob, info, np.array([40, 1100], np.int32))


def test_store_kv_rejects_duplicate_slots_and_positions_past_the_table():
    p = _params()
    slots = np.array([3, 17, 3], np.int64)
    with pytest.raises(la.LazyAttnError, match="INVALID_ARG.*slot 3 is written twice"):
        la.lazy_attn_store_kv(p, FAKE, FAKE, 3, slots.ctypes.data, None, None, FAKE, FAKE)
    slots = np.array([3, 17, 160], np.int64)  # 10 blocks x 16 slots
    with pytest.raises(la.LazyAttnError, match="INVALID_ARG.*outside the pool"):
        la.lazy_attn_store_kv(p, FAKE, FAKE, 3, slots.ctypes.data, None, None, FAKE, FAKE)
    slots = np.array([3, 17, 18], np.int64)
    pos = np.array([0, 5, 1024], np.int32)
    with pytest.raises(la.LazyAttnError, match="INVALID_ARG.*rotation position 1024"):
        la.lazy_attn_store_kv(p, FAKE, FAKE, 3, slots.ctypes.data, pos.ctypes.data, FAKE, FAKE,
                              FAKE)

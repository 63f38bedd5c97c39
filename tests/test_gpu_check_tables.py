"""la_params.check_tables on the GPU: with valid tables every launch gives
the same bits as without the check; a corrupted device table is refused
before anything is enqueued (so no kernel ever reads it)."""
import numpy as np
import pytest

from workloads import build_workload

from gpu_util import log

pytestmark = pytest.mark.gpu

COMMON = dict(num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16, rope_base=5e5,
              doc_lens=[40, 33, 64], seed=21)


def _dec():
    return build_workload(name="ct_decode", kind="decode", dtype="bf16",
                          requests=[[("doc", 0), ("doc", 1), ("doc", 2)],
                                    [("doc", 2), ("doc", 0, 500), ("priv", 5)]], **COMMON)


def _outs(db):
    import torch
    db.run()
    torch.cuda.synchronize()
    return db.out.cpu().numpy().copy(), db.lse.cpu().numpy().copy()


@pytest.mark.parametrize("shared", [False, True])
def test_decode_same_bits_with_the_check(shared):
    from position_agnostic_kv_lazy_amd.prepare import prepare, upload_pool
    w = _dec()
    k, v = upload_pool(w.k_pool, w.v_pool)
    log(f"check_tables decode shared={shared}")
    a = _outs(prepare(w, k, v, shared=shared))
    b = _outs(prepare(w, k, v, shared=shared, check_tables=True))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_prefill_same_bits_with_the_check():
    from position_agnostic_kv_lazy_amd.prepare import prepare, upload_pool
    w = build_workload(name="ct_prefill", kind="prefill", dtype="bf16",
                       requests=[[("doc", 1), ("doc", 0), ("new", 37)]], **COMMON)
    k, v = upload_pool(w.k_pool, w.v_pool)
    log("check_tables prefill")
    a = _outs(prepare(w, k, v))
    b = _outs(prepare(w, k, v, check_tables=True))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_corrupted_device_tables_are_refused():
    import torch

    import position_agnostic_kv_lazy_amd as la
    from position_agnostic_kv_lazy_amd.prepare import prepare, upload_pool
    w = _dec()
    k, v = upload_pool(w.k_pool, w.v_pool)
    db = prepare(w, k, v, check_tables=True)
    bad = db.host_words.copy()
    bad[2] = (bad[2] & ~np.uint64(0xFFFFFFFF)) | np.uint64(db.params.num_blocks)
    words = torch.from_numpy(bad.view(np.int64)).cuda()
    log("check_tables: corrupted block word on the device")
    with pytest.raises(la.LazyAttnError, match="INVALID_ARG.*block id"):
        la.lazy_attn_decode(db.params, db.q, db.k_pool, db.v_pool, words, db.req_blk_start,
                            db.q_pos, db.cos_sin, db.batch, db.max_blocks, db.out, db.lse,
                            db.workspace)
    ds = prepare(w, k, v, shared=True, check_tables=True)
    plan = ds.host_plan.copy()
    info = ds.plan_info
    wo = len(plan) - 8 * info.n_words
    pw = plan[wo:].view(np.uint64)
    pw[0] = (pw[0] & ~np.uint64(0xFFFFFFFF)) | np.uint64(ds.params.num_blocks)
    dplan = torch.from_numpy(plan).cuda()
    log("check_tables: corrupted shared-decode plan on the device")
    with pytest.raises(la.LazyAttnError, match="INVALID_ARG.*block id"):
        la.lazy_attn_decode_shared(ds.params, info, dplan, ds.q, ds.k_pool, ds.v_pool, ds.q_pos,
                                   ds.cos_sin, ds.batch, ds.out, ds.lse, ds.workspace)
    # the valid tables still run afterwards
    _outs(db)
    _outs(ds)

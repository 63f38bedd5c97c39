"""Streams, threads and HIP graphs: the library keeps no state between calls.

* Decode and prefill captured into one HIP graph (torch.cuda.CUDAGraph on a
  side stream) replay to the eager result, replay after replay, with eager
  work and synchronisations between replays; the shared-segment decode too.
* Calls from two host threads on two streams, interleaved, give the results
  of the same calls made alone.
"""
import threading

import numpy as np
import pytest
import torch

from position_agnostic_kv_lazy_amd.prepare import prepare, upload_pool
from workloads import build_workload

from gpu_util import assert_parity, log

pytestmark = pytest.mark.gpu


def _pair():
    dec = build_workload(name="g", kind="decode", dtype="bf16", num_q_heads=8, num_kv_heads=2,
                         head_dim=128, block_size=16, rope_base=5e5, doc_lens=[48, 37, 64, 20],
                         requests=[[("doc", 0), ("doc", 1), ("priv", 5)],
                                   [("doc", 2), ("doc", 0, 200), ("doc", 3)]], seed=71)
    pre = build_workload(name="g", kind="prefill", dtype="bf16", num_q_heads=8, num_kv_heads=2,
                         head_dim=128, block_size=16, rope_base=5e5, doc_lens=[48, 37, 64, 20],
                         requests=[[("doc", 0), ("doc", 2), ("new", 70)],
                                   [("doc", 1), ("new", 33)]], seed=72)
    return dec, pre


def test_graph_replays_match_eager():
    dec, pre = _pair()
    kd, vd = upload_pool(dec.k_pool, dec.v_pool)
    kp, vp = upload_pool(pre.k_pool, pre.v_pool)
    dd, dp = prepare(dec, kd, vd, split_blocks=2), prepare(pre, kp, vp)
    dd.run(); dp.run()
    torch.cuda.synchronize()
    eager_d, eager_p = dd.out_f32().copy(), dp.out_f32().copy()

    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        dd.run(side)
        dp.run(side)
    for rep in range(4):
        dd.out.zero_()
        dp.out.zero_()
        scratch = torch.randn(1 << 20, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log(f"graph replay {rep}")
        np.testing.assert_array_equal(dd.out_f32(), eager_d)
        np.testing.assert_array_equal(dp.out_f32(), eager_p)
        del scratch


def test_shared_decode_graph_replays_match_eager():
    """The shared-segment decode (decode + merge kernels) captured alone."""
    dec, _ = _pair()
    kd, vd = upload_pool(dec.k_pool, dec.v_pool)
    ds = prepare(dec, kd, vd, shared=True)
    ds.run()
    torch.cuda.synchronize()
    eager = ds.out_f32().copy()
    eager_lse = ds.lse.cpu().numpy().copy()
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        ds.run(side)
    for rep in range(4):
        ds.out.zero_()
        ds.lse.zero_()
        ds.workspace.zero_()  # partials are rewritten by every replay
        scratch = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log(f"shared graph replay {rep}")
        np.testing.assert_array_equal(ds.out_f32(), eager)
        np.testing.assert_array_equal(ds.lse.cpu().numpy(), eager_lse)
        del scratch


def test_two_threads_two_streams():
    dec, pre = _pair()
    kd, vd = upload_pool(dec.k_pool, dec.v_pool)
    kp, vp = upload_pool(pre.k_pool, pre.v_pool)
    dd, dp = prepare(dec, kd, vd), prepare(pre, kp, vp)
    dd.run(); dp.run()
    torch.cuda.synchronize()
    ref_d, ref_p = dd.out_f32().copy(), dp.out_f32().copy()
    dd.out.zero_(); dp.out.zero_()
    torch.cuda.synchronize()
    errors = []

    def work(db, n):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(n):
                    db.run(s)
            s.synchronize()
        except Exception as e:  # reported below
            errors.append(e)

    ts = [threading.Thread(target=work, args=(dd, 20)), threading.Thread(target=work, args=(dp, 20))]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    np.testing.assert_array_equal(dd.out_f32(), ref_d)
    np.testing.assert_array_equal(dp.out_f32(), ref_p)
    assert_parity(dd.out_f32(), ref_d, "bf16", "threaded decode")

"""Pools past 4 GiB: every kernel addresses blocks with 64-bit offsets.

A small batch is run twice on the same blocks: once in a compact pool, once
relocated to the top of a pool whose K and V tensors each span more than
2^32 bytes (element offsets past 2^31), with the low blocks left
uninitialised and never listed.  Identical inputs on an identical schedule
give identical bits, so any truncated offset shows as a mismatch (or reads
garbage).  The compact run is itself checked against the oracle.  The
physical placement of a document's blocks is free in the method (the same
document at different offsets and places, "LazyAttention" §1 and §3 problem
statement); this covers the largest placements a pool of this size allows.
"""
import numpy as np
import pytest
import torch

from oracle import run_decode, run_prefill
from position_agnostic_kv_lazy_amd.prepare import store_pool, upload_pool
from workloads import Segment, build_workload

from gpu_util import Device, assert_lse, assert_parity, log

pytestmark = pytest.mark.gpu

FOUR_GIB = 1 << 32


def _tiny(kind, dtype="bf16"):
    requests = ([[("doc", 0), ("doc", 1), ("doc", 2), ("priv", 5)],
                 [("doc", 3), ("doc", 0), ("doc", 1)],
                 [("doc", 1), ("doc", 2)]] if kind == "decode" else
                [[("doc", 0), ("doc", 1), ("new", 40)], [("doc", 3), ("doc", 2), ("new", 70)]])
    return build_workload(name="big", kind=kind, dtype=dtype, num_q_heads=8, num_kv_heads=2,
                          head_dim=128, block_size=16, rope_base=5e5, doc_lens=[48, 37, 64, 20],
                          requests=requests, seed=33)


def _check_oracle(w, out, lse):
    if w.kind == "decode":
        res = run_decode(w)
        for r in range(w.batch):
            assert_parity(out[r], res[r][0], w.dtype, f"compact pool req {r}")
            assert_lse(lse[r], res[r][1], w.dtype, f"compact pool req {r}")
    else:
        res = run_prefill(w)
        for r in range(w.batch):
            a, b = int(w.cu_q[r]), int(w.cu_q[r + 1])
            assert_parity(out[a:b], res[r][0], w.dtype, f"compact pool req {r}")
            assert_lse(lse[a:b], res[r][1], w.dtype, f"compact pool req {r}")


def _relocated(w, offset):
    import copy
    w2 = copy.copy(w)
    w2.requests = [[Segment(s.start, s.n_tokens, s.blocks + offset, s.is_new) for s in segs]
                   for segs in w.requests]
    return w2


def _big_pools(k_small, v_small, offset):
    """Device pools of offset + nb blocks, the small pool copied to the top."""
    nb = k_small.shape[0]
    k = torch.empty((offset + nb,) + tuple(k_small.shape[1:]), dtype=k_small.dtype, device="cuda")
    v = torch.empty((offset + nb,) + tuple(v_small.shape[1:]), dtype=v_small.dtype, device="cuda")
    k[offset:] = k_small
    v[offset:] = v_small
    torch.cuda.synchronize()
    assert k[offset:].numel() and k.numel() * k.element_size() > FOUR_GIB
    assert v.numel() * v.element_size() > FOUR_GIB
    return k, v


def _offset_for(k_small):
    """First block id whose byte offset (K and V alike) lies past 4 GiB."""
    block_bytes = k_small[0].numel() * k_small.element_size()
    return FOUR_GIB // block_bytes + 17


@pytest.mark.parametrize("kind,dtype,shared", [("decode", "bf16", False),
                                               ("decode", "bf16", True),
                                               ("prefill", "bf16", False),
                                               ("decode", "f32", False),
                                               ("prefill", "f32", False)])
def test_blocks_past_4gib(kind, dtype, shared):
    w = _tiny(kind, dtype)
    k_small, v_small = upload_pool(w.k_pool, w.v_pool, "cuda")
    offset = _offset_for(k_small)
    log(f"case {kind} {dtype} shared={shared}: block ids from {offset}, "
        f"{(offset + w.num_blocks) * k_small[0].numel() * k_small.element_size() / 2**30:.2f} GiB per pool")
    o1, l1, _ = Device.from_device_pools(k_small, v_small).run(w, shared=shared)
    _check_oracle(w, o1, l1)
    k, v = _big_pools(k_small, v_small, offset)
    o2, l2, _ = Device.from_device_pools(k, v).run(_relocated(w, offset), shared=shared,
                                                  check_tables=True)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    del k, v
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_store_kv_past_4gib(dtype):
    """The cache write lands in the same bytes at the top of a > 4 GiB pool."""
    w = _tiny("decode", dtype)
    rng = np.random.default_rng(5)
    n = 40  # two whole blocks (the block-tile path) and a partial one (per element)
    k_tok = rng.standard_normal((n, w.num_kv_heads, w.head_dim)).astype(np.float32)
    v_tok = rng.standard_normal((n, w.num_kv_heads, w.head_dim)).astype(np.float32)
    if dtype == "bf16":
        k_tok = (k_tok.view(np.uint32) >> 16).astype(np.uint16)
        v_tok = (v_tok.view(np.uint32) >> 16).astype(np.uint16)
    slots_small = np.arange(n, dtype=np.int64) + 16  # blocks 1, 2 and part of 3
    pos = (np.arange(n) + 1000).astype(np.int32)
    ks, vs = store_pool(w, k_tok, v_tok, slots_small, pos, num_blocks=4, max_pos=2048)
    offset = _offset_for(ks)
    log(f"store_kv {dtype}: slots from block {offset + 1}")
    kb, vb = store_pool(w, k_tok, v_tok, slots_small + offset * w.block_size, pos,
                        num_blocks=offset + 4, max_pos=2048)
    assert kb.numel() * kb.element_size() > FOUR_GIB
    torch.cuda.synchronize()
    assert torch.equal(ks, kb[offset:])
    assert torch.equal(vs, vb[offset:])
    del kb, vb
    torch.cuda.empty_cache()

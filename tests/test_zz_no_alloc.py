"""The allocation-free decode entry point (lazy_attn_decode_noalloc) on the GPU.

It must return exactly what lazy_attn_decode returns with a caller-provided
workspace (same kernels; only where the split-group partials live differs),
on two calls in a row on one device -- the second with a smaller input, so
it runs over the scratch contents the first call left -- and both must meet
the oracle's bf16 bar on sampled requests.
"""
import numpy as np
import pytest
import torch

from oracle import run_decode
from position_agnostic_kv_lazy_amd import binding as B
from position_agnostic_kv_lazy_amd.prepare import prepare, upload_pool

from gpu_util import assert_lse, assert_parity, config, log

pytestmark = pytest.mark.gpu


def _widen(t):
    return (t.cpu().numpy().view(np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _check(w, target_workgroups, sample):
    k, v = upload_pool(w.k_pool, w.v_pool, "cuda")
    db = prepare(w, k, v, target_workgroups=target_workgroups)
    need = B.lazy_attn_decode_workspace_size(db.params, db.batch, db.max_blocks)
    log(f"noalloc decode {w.name}: batch {w.batch}, {need} scratch bytes")
    assert 0 < need <= B.LA_DECODE_NOALLOC_SCRATCH_BYTES  # the shape uses split partials
    db.run()
    torch.cuda.synchronize()
    ref_out, ref_lse = db.out.clone(), db.lse.clone()
    for rep in range(2):
        out = torch.full_like(db.out, 0x7FC0)  # bf16 NaN bits: every element must be written
        lse = torch.full_like(db.lse, float("nan"))
        B.lazy_attn_decode_noalloc(db.params, db.q, db.k_pool, db.v_pool, db.words,
                                   db.req_blk_start, db.q_pos, db.cos_sin, db.batch,
                                   db.max_blocks, out, lse)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"rep {rep}: output differs from lazy_attn_decode"
        assert torch.equal(lse, ref_lse), f"rep {rep}: lse differs from lazy_attn_decode"
    got, got_lse = _widen(out), lse.cpu().numpy()
    ref = run_decode(w, requests=sample)
    for r in sample:
        assert_parity(got[r], ref[r][0], "bf16", f"noalloc {w.name} req {r}")
        assert_lse(got_lse[r], ref[r][1], "bf16", f"noalloc {w.name} req {r}")
    del k, v, db
    torch.cuda.empty_cache()


def test_noalloc_decode_matches_workspace_decode_twice():
    # first: 32 requests x 5,184 keys, 2 split groups per (request, kv head)
    w1 = config(2, scale_down=2)
    _check(w1, 0, [0, 17, w1.batch - 1])
    # then a smaller batch over the same scratch: 8 requests, fewer partials
    w2 = config(2, scale_down=8)
    _check(w2, 128, [0, 3, w2.batch - 1])

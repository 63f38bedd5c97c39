"""Shared helpers of the GPU parity tests: run the HIP path, compare to the oracle."""
from __future__ import annotations

import functools
import sys

import numpy as np

from workloads import make_config

BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 5e-3
F32_MAX_ABS = 1e-5


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def errors(gpu: np.ndarray, ref: np.ndarray):
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    max_abs = float(np.max(np.abs(g - r))) if g.size else 0.0
    rel = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300))
    return max_abs, rel


def assert_parity(gpu, ref, dtype, what=""):
    max_abs, rel = errors(gpu, ref)
    log(f"  parity {what}: max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU output"
    if dtype == "bf16":
        assert max_abs <= BF16_MAX_ABS, f"{what}: max_abs {max_abs:.3e} > {BF16_MAX_ABS}"
        assert rel <= BF16_REL_L2, f"{what}: rel_l2 {rel:.3e} > {BF16_REL_L2}"
    else:
        assert max_abs <= F32_MAX_ABS, f"{what}: max_abs {max_abs:.3e} > {F32_MAX_ABS}"


def assert_lse(gpu, ref, dtype, what=""):
    tol = 2e-2 if dtype == "bf16" else 1e-5
    d = float(np.max(np.abs(np.asarray(gpu, np.float64) - ref)))
    log(f"  lse {what}: max_abs={d:.3e}")
    assert d <= tol, f"{what}: lse max_abs {d:.3e} > {tol}"


@functools.lru_cache(maxsize=4)
def config(cfg: int, dtype=None, scale_down=1):
    return make_config(cfg, dtype=dtype, scale_down=scale_down)


class Device:
    """One uploaded pool plus prepared batches, run through the C ABI."""

    def __init__(self, w, pool_of=None):
        import torch
        from position_agnostic_kv_lazy_amd.prepare import upload_pool
        src = pool_of if pool_of is not None else w
        self.k, self.v = upload_pool(src.k_pool, src.v_pool, "cuda")
        torch.cuda.synchronize()

    @classmethod
    def from_device_pools(cls, k, v):
        self = cls.__new__(cls)
        self.k, self.v = k, v
        return self

    def run(self, w, split_blocks=0, target_workgroups=0, validate=True, max_pos=None,
            pool_mode="position_free", pos_encoding="rope_half", table=None, shared=False,
            max_item_blocks=0, check_tables=False):
        import torch
        from position_agnostic_kv_lazy_amd import lazy_attn_validate_table
        from position_agnostic_kv_lazy_amd.prepare import prepare
        db = prepare(w, self.k, self.v, split_blocks=split_blocks,
                     target_workgroups=target_workgroups, max_pos=max_pos, pool_mode=pool_mode,
                     pos_encoding=pos_encoding, table=table, shared=shared,
                     max_item_blocks=max_item_blocks, check_tables=check_tables)
        if validate:
            cu = None if w.kind == "decode" else np.asarray(w.cu_q, np.int32)
            lazy_attn_validate_table(db.params, db.batch, db.host_words, db.host_rbs,
                                     np.asarray(w.q_pos, np.int32), cu, db.max_blocks,
                                     db.max_q if cu is not None else 0)
        db.run()
        torch.cuda.synchronize()
        return db.out_f32(), db.lse.cpu().numpy(), db

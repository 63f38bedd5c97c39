"""Stage host-side inputs in device memory in the layouts the C ABI expects.

Input preparation only (outside any timed region): it converts a host pool to
the device layout (V tiles dim-major), builds the cos/sin table and the packed
block table through the library's own host entry points, and allocates
outputs and the decode workspace.  All attention arithmetic happens in the
HIP kernels behind lazy_attn_decode / lazy_attn_prefill.

A "batch description" is any object with the attributes used below
(kind, dtype, num_q_heads, num_kv_heads, head_dim, block_size, rope_base,
scale, requests, q, q_pos, cu_q, table_rows(), batch); the pools are passed
separately so several batches can share one device pool.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import binding as B


def _to_device_bits(a: np.ndarray, device) -> torch.Tensor:
    """uint16 (bf16 bits) -> int16 tensor with the same bits; float32 as is."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def upload_pool(k_pool: np.ndarray, v_pool: np.ndarray, device="cuda", chunk_blocks=8192):
    """Copy a logical [nb, Hkv, BS, D] pool pair to the device layouts.

    K keeps [nb, Hkv, BS, D]; V becomes [nb, Hkv, D, BS] (dim-major tiles).
    Large pools are streamed in chunks to bound host and device staging.
    """
    nb = k_pool.shape[0]
    k_dev = _to_device_bits(k_pool, device)
    shape_t = (nb, v_pool.shape[1], v_pool.shape[3], v_pool.shape[2])
    dt = torch.int16 if v_pool.dtype == np.uint16 else torch.float32
    v_dev = torch.empty(shape_t, dtype=dt, device=device)
    for a in range(0, nb, chunk_blocks):
        b = min(nb, a + chunk_blocks)
        v_dev[a:b] = _to_device_bits(v_pool[a:b], device).transpose(-1, -2)
    return k_dev, v_dev


@dataclass
class DeviceBatch:
    kind: str
    params: B.la_params
    q: torch.Tensor
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    words: torch.Tensor
    req_blk_start: torch.Tensor
    q_pos: torch.Tensor
    cu_q: Optional[torch.Tensor]
    cos_sin: torch.Tensor
    out: torch.Tensor
    lse: torch.Tensor
    workspace: Optional[torch.Tensor]
    batch: int
    max_blocks: int
    max_q: int
    host_words: np.ndarray
    host_rbs: np.ndarray
    plan: Optional[torch.Tensor] = None       # shared-segment decode plan (device)
    plan_info: Optional[B.la_shared_plan_info] = None
    host_plan: Optional[np.ndarray] = None    # the same plan blob on the host

    def run(self, stream=None):
        if self.kind == "decode" and self.plan is not None:
            B.lazy_attn_decode_shared(self.params, self.plan_info, self.plan, self.q, self.k_pool,
                                      self.v_pool, self.q_pos, self.cos_sin, self.batch, self.out,
                                      self.lse, self.workspace, stream)
        elif self.kind == "decode":
            B.lazy_attn_decode(self.params, self.q, self.k_pool, self.v_pool, self.words,
                               self.req_blk_start, self.q_pos, self.cos_sin, self.batch,
                               self.max_blocks, self.out, self.lse, self.workspace, stream)
        else:
            B.lazy_attn_prefill(self.params, self.q, self.k_pool, self.v_pool, self.words,
                                self.req_blk_start, self.cu_q, self.q_pos, self.cos_sin,
                                self.batch, self.max_q, self.out, self.lse, stream)

    def out_f32(self) -> np.ndarray:
        """Output as float32 numpy (bf16 bits widened exactly)."""
        o = self.out.cpu().numpy()
        if o.dtype == np.int16:
            return (o.view(np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
        return o


def params_for(w, num_blocks: int, max_pos: Optional[int] = None, split_blocks: int = 0,
               target_workgroups: int = 0, pool_mode="position_free",
               pos_encoding="rope_half", check_tables: bool = False) -> B.la_params:
    """la_params describing batch w over a pool of num_blocks blocks."""
    rows = int(max_pos) if max_pos is not None else int(w.table_rows())
    return B.make_params(num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
                         head_dim=w.head_dim, block_size=w.block_size, num_blocks=int(num_blocks),
                         dtype=w.dtype, scale=w.scale, max_pos=rows, split_blocks=split_blocks,
                         target_workgroups=target_workgroups, pool_mode=pool_mode,
                         pos_encoding=pos_encoding, check_tables=check_tables)


def store_pool(w, k_tok: np.ndarray, v_tok: np.ndarray, slots: np.ndarray,
               rope_pos: Optional[np.ndarray], device="cuda", num_blocks: Optional[int] = None,
               max_pos: Optional[int] = None, fill: float = 0.0, stream=None,
               pos_encoding="rope_half", table: Optional[np.ndarray] = None):
    """Build a device pool pair by writing tokens with lazy_attn_store_kv.

    k_tok / v_tok: host [n, Hkv, D] in the pool encoding; slots: flat slot ids;
    rope_pos: per-token rotation position or None (keys stored as given).
    pos_encoding="rope_interleaved" rotates pairs (2i, 2i+1) and stores keys in
    (even dims, odd dims) order.  table overrides the cos/sin rows used for
    the rotation (e.g. a scaled RoPE table).  Unlisted slots hold `fill`.
    Returns (k_dev, v_dev) in the device layouts.
    """
    nb = int(num_blocks) if num_blocks is not None else int(w.num_blocks)
    rows = int(max_pos) if max_pos is not None else int(w.table_rows())
    slots = np.asarray(slots, np.int64)
    # the kernel trusts slots and positions: check them here, before the launch
    if slots.size and (slots.min() < 0 or slots.max() >= nb * w.block_size):
        raise ValueError("slot id outside the pool")
    if len(np.unique(slots)) != len(slots):
        raise ValueError("slot ids must be distinct")
    if rope_pos is not None and len(rope_pos) and (np.min(rope_pos) < 0 or np.max(rope_pos) >= rows):
        raise ValueError("rope position outside the cos/sin table")
    if k_tok.shape != (len(slots), w.num_kv_heads, w.head_dim) or v_tok.shape != k_tok.shape:
        raise ValueError("k/v token arrays must be [n, Hkv, D]")
    params = params_for(w, nb, rows, pos_encoding=pos_encoding)
    bf16 = k_tok.dtype == np.uint16
    dt = torch.int16 if bf16 else torch.float32
    Hkv, BS, D = w.num_kv_heads, w.block_size, w.head_dim
    if bf16:
        fb = int(np.float32(fill).view(np.uint32) >> np.uint32(16))
        fb = fb - 65536 if fb >= 32768 else fb
        k_dev = torch.full((nb, Hkv, BS, D), fb, dtype=dt, device=device)
        v_dev = torch.full((nb, Hkv, D, BS), fb, dtype=dt, device=device)
    else:
        k_dev = torch.full((nb, Hkv, BS, D), fill, dtype=dt, device=device)
        v_dev = torch.full((nb, Hkv, D, BS), fill, dtype=dt, device=device)
    k = _to_device_bits(k_tok, device)
    v = _to_device_bits(v_tok, device)
    sl = torch.from_numpy(np.asarray(slots, np.int64)).to(device)
    rp = None if rope_pos is None else torch.from_numpy(np.asarray(rope_pos, np.int32)).to(device)
    cs = None
    if rope_pos is not None:
        if table is None:
            table = B.lazy_attn_rope_table(w.rope_base, D, rows)
        cs = torch.from_numpy(np.ascontiguousarray(table, np.float32)).to(device)
    B.lazy_attn_store_kv(params, k, v, len(slots), sl, rp, cs, k_dev, v_dev, stream)
    return k_dev, v_dev


def prepare(w, k_dev: torch.Tensor, v_dev: torch.Tensor, device="cuda", split_blocks: int = 0,
            target_workgroups: int = 0, max_pos: Optional[int] = None,
            pool_mode="position_free", pos_encoding="rope_half",
            table: Optional[np.ndarray] = None, shared: bool = False,
            max_item_blocks: int = 0, check_tables: bool = False) -> DeviceBatch:
    """Pack and upload everything lazy_attn_decode/prefill need for batch w.

    table overrides the position table handed to the kernels: by default the
    RoPE cos/sin rows (lazy_attn_rope_table) or, for ALiBi, the standard
    slopes (lazy_attn_alibi_slopes).  shared=True (decode) builds a
    shared-segment plan (lazy_attn_plan_shared_decode) and runs
    lazy_attn_decode_shared instead of lazy_attn_decode.  check_tables sets
    la_params.check_tables (every launch checks its tables first).
    """
    rows = int(max_pos) if max_pos is not None else int(w.table_rows())
    params = params_for(w, int(k_dev.shape[0]), rows, split_blocks, target_workgroups, pool_mode,
                        pos_encoding, check_tables)
    words, rbs, maxb = B.lazy_attn_pack_segments(params, w.requests)
    if table is None:
        table = (B.lazy_attn_alibi_slopes(w.num_q_heads) if pos_encoding == "alibi"
                 else B.lazy_attn_rope_table(w.rope_base, w.head_dim, rows))
    q = _to_device_bits(w.q, device)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=device)
    q_pos = torch.from_numpy(np.asarray(w.q_pos, dtype=np.int32)).to(device)
    cu_q = None
    max_q = 1
    if w.kind == "prefill":
        cu = np.asarray(w.cu_q, dtype=np.int32)
        cu_q = torch.from_numpy(cu).to(device)
        max_q = int(np.max(np.diff(cu)))
    ws = None
    plan = info = blob = None
    if w.kind == "decode" and shared:
        info, blob = B.lazy_attn_plan_shared_decode(params, w.requests, max_item_blocks)
        plan = torch.from_numpy(blob).to(device)
        ws = torch.empty(int(info.workspace_bytes), dtype=torch.uint8, device=device)
    elif w.kind == "decode":
        nbytes = B.lazy_attn_decode_workspace_size(params, w.batch, maxb)
        if nbytes:
            ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return DeviceBatch(
        kind=w.kind, params=params, q=q, k_pool=k_dev, v_pool=v_dev,
        words=torch.from_numpy(words.view(np.int64)).to(device),
        req_blk_start=torch.from_numpy(rbs).to(device), q_pos=q_pos, cu_q=cu_q,
        cos_sin=torch.from_numpy(np.ascontiguousarray(table, np.float32)).to(device), out=out,
        lse=lse, workspace=ws,
        batch=w.batch, max_blocks=maxb, max_q=max_q, host_words=words, host_rbs=rbs,
        plan=plan, plan_info=info, host_plan=blob)

"""ctypes binding of liblazyattn.so (the C ABI in include/lazy_attn.h).

Argument marshalling only: every function forwards to the C entry point of
the same name.  Device arguments are torch tensors (their data_ptr() is
passed) and the stream is a torch.cuda.Stream or a raw hipStream_t integer.
There is no fallback: if the library is missing, importing this module
raises, and every non-OK status raises LazyAttnError.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("LAZYATTN_LIB", os.path.join(_PKG, "liblazyattn.so"))

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} not found: build it with `python position_agnostic_kv_lazy_amd/build.py` "
        "(or __graft_entry__.build())")

# PyTorch ships its own libamdhip64 under the same soname as ROCm's.  Loading
# torch first makes the loader bind this library's libamdhip64.so.7 to that
# copy, so both share one HIP runtime (one device context, one set of streams
# and allocations).  Loaded the other way round, the process would hold two
# independent HIP runtimes and this library could not see torch's device.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

LA_OK, LA_ERR_INVALID_ARG, LA_ERR_UNSUPPORTED, LA_ERR_WORKSPACE_TOO_SMALL, LA_ERR_HIP = range(5)
LA_DECODE_NOALLOC_SCRATCH_BYTES = 8 << 20  # the header's fixed decode scratch per GPU
LA_BF16, LA_FP32 = 0, 1
LA_POOL_POSITION_FREE, LA_POOL_DOC_LOCAL = 0, 1
LA_ROPE_HALF, LA_ROPE_INTERLEAVED, LA_ALIBI = 0, 1, 2
LA_CACHE_POSITION_AGNOSTIC, LA_CACHE_POSITION_AWARE = 0, 1
LA_EVICT_LRU, LA_EVICT_STATIC_TOP = 0, 1

EXPORTED = (
    "lazy_attn_status_string",
    "lazy_attn_last_error",
    "lazy_attn_rope_table",
    "lazy_attn_rope_table_scaled",
    "lazy_attn_alibi_slopes",
    "lazy_attn_pack_segments",
    "lazy_attn_validate_table",
    "lazy_attn_decode_workspace_size",
    "lazy_attn_store_kv",
    "lazy_attn_decode",
    "lazy_attn_decode_noalloc",
    "lazy_attn_plan_shared_decode",
    "lazy_attn_decode_shared",
    "lazy_attn_prefill",
    "lazy_attn_cache_simulate",
)


class la_params(ctypes.Structure):
    _fields_ = [
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int64),
        ("dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("max_pos", ctypes.c_int32),
        ("split_blocks", ctypes.c_int32),
        ("target_workgroups", ctypes.c_int32),
        ("pool_mode", ctypes.c_int32),
        ("pos_encoding", ctypes.c_int32),
        ("check_tables", ctypes.c_int32),
        ("reserved", ctypes.c_int32 * 2),
    ]


class la_rope_scaling(ctypes.Structure):
    _fields_ = [
        ("type", ctypes.c_int32),
        ("original_max_pos", ctypes.c_int32),
        ("factor", ctypes.c_double),
        ("low_freq_factor", ctypes.c_double),
        ("high_freq_factor", ctypes.c_double),
        ("beta_fast", ctypes.c_double),
        ("beta_slow", ctypes.c_double),
        ("attn_factor", ctypes.c_double),
    ]


class la_shared_plan_info(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("n_items", ctypes.c_int32),
        ("n_members", ctypes.c_int32),
        ("n_words", ctypes.c_int32),
        ("members_per_item", ctypes.c_int32),
        ("max_item_blocks", ctypes.c_int32),
        ("plan_bytes", ctypes.c_int64),
        ("workspace_bytes", ctypes.c_int64),
    ]


SCALING_TYPES = {"none": 0, "linear": 1, "ntk": 2, "yarn": 3, "llama3": 4}


def make_scaling(type="none", factor=1.0, original_max_pos=0, low_freq_factor=0.0,
                 high_freq_factor=0.0, beta_fast=0.0, beta_slow=0.0,
                 attn_factor=0.0) -> la_rope_scaling:
    s = la_rope_scaling()
    s.type = SCALING_TYPES.get(type, type)
    s.original_max_pos = int(original_max_pos)
    s.factor = float(factor)
    s.low_freq_factor = float(low_freq_factor)
    s.high_freq_factor = float(high_freq_factor)
    s.beta_fast = float(beta_fast)
    s.beta_slow = float(beta_slow)
    s.attn_factor = float(attn_factor)
    return s


class LazyAttnError(RuntimeError):
    def __init__(self, status: int, func: str):
        self.status = status
        msg = _lib.lazy_attn_last_error().decode()
        name = _lib.lazy_attn_status_string(status).decode()
        super().__init__(f"{func}: {name}: {msg}")


_P = ctypes.c_void_p
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_u64p = ctypes.POINTER(ctypes.c_uint64)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_f32p = ctypes.POINTER(ctypes.c_float)
_prm = ctypes.POINTER(la_params)

_lib.lazy_attn_status_string.restype = ctypes.c_char_p
_lib.lazy_attn_status_string.argtypes = [ctypes.c_int]
_lib.lazy_attn_last_error.restype = ctypes.c_char_p
_lib.lazy_attn_last_error.argtypes = []
_lib.lazy_attn_rope_table.restype = ctypes.c_int
_lib.lazy_attn_rope_table.argtypes = [ctypes.c_double, ctypes.c_int32, ctypes.c_int32, _f32p]
_lib.lazy_attn_rope_table_scaled.restype = ctypes.c_int
_lib.lazy_attn_rope_table_scaled.argtypes = [ctypes.c_double, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.POINTER(la_rope_scaling), _f32p]
_lib.lazy_attn_alibi_slopes.restype = ctypes.c_int
_lib.lazy_attn_alibi_slopes.argtypes = [ctypes.c_int32, _f32p]
_lib.lazy_attn_pack_segments.restype = ctypes.c_int
_lib.lazy_attn_pack_segments.argtypes = [_prm, ctypes.c_int32, _i64p, _i64p, _i64p, _u8p, _i64p,
                                         _i64p, _u64p, ctypes.c_int64, _i32p, _i32p]
_lib.lazy_attn_validate_table.restype = ctypes.c_int
_lib.lazy_attn_validate_table.argtypes = [_prm, ctypes.c_int32, _P, _P, _P, _P, ctypes.c_int32,
                                          ctypes.c_int32]
_lib.lazy_attn_decode_workspace_size.restype = ctypes.c_int
_lib.lazy_attn_decode_workspace_size.argtypes = [_prm, ctypes.c_int32, ctypes.c_int32,
                                                 ctypes.POINTER(ctypes.c_size_t)]
_lib.lazy_attn_store_kv.restype = ctypes.c_int
_lib.lazy_attn_store_kv.argtypes = [_prm, _P, _P, ctypes.c_int64, _P, _P, _P, _P, _P, _P]
_lib.lazy_attn_decode.restype = ctypes.c_int
_lib.lazy_attn_decode.argtypes = [_prm, _P, _P, _P, _P, _P, _P, _P, ctypes.c_int32, ctypes.c_int32,
                                  _P, _P, _P, ctypes.c_size_t, _P]
_lib.lazy_attn_decode_noalloc.restype = ctypes.c_int
_lib.lazy_attn_decode_noalloc.argtypes = [_prm, _P, _P, _P, _P, _P, _P, _P, ctypes.c_int32,
                                          ctypes.c_int32, _P, _P, _P]
_lib.lazy_attn_plan_shared_decode.restype = ctypes.c_int
_lib.lazy_attn_plan_shared_decode.argtypes = [_prm, ctypes.c_int32, _i64p, _i64p, _i64p, _u8p,
                                              _i64p, _i64p, ctypes.c_int32,
                                              ctypes.POINTER(la_shared_plan_info), _P,
                                              ctypes.c_int64]
_lib.lazy_attn_decode_shared.restype = ctypes.c_int
_lib.lazy_attn_decode_shared.argtypes = [_prm, ctypes.POINTER(la_shared_plan_info), _P, _P, _P,
                                         _P, _P, _P, ctypes.c_int32, _P, _P, _P, ctypes.c_size_t,
                                         _P]
_lib.lazy_attn_cache_simulate.restype = ctypes.c_int
_lib.lazy_attn_cache_simulate.argtypes = [ctypes.c_int64, _i64p, _i32p, ctypes.c_int32,
                                          ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _i64p]
_lib.lazy_attn_prefill.restype = ctypes.c_int
_lib.lazy_attn_prefill.argtypes = [_prm, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_int32,
                                   ctypes.c_int32, _P, _P, _P]


def _check(status: int, func: str):
    if status != LA_OK:
        raise LazyAttnError(status, func)


def make_params(*, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, dtype, scale,
                max_pos, split_blocks=0, target_workgroups=0, pool_mode=0,
                pos_encoding=0, check_tables=False) -> la_params:
    p = la_params()
    p.num_q_heads = num_q_heads
    p.num_kv_heads = num_kv_heads
    p.head_dim = head_dim
    p.block_size = block_size
    p.num_blocks = num_blocks
    p.dtype = {"bf16": LA_BF16, "f32": LA_FP32}.get(dtype, dtype)
    p.scale = scale
    p.max_pos = max_pos
    p.split_blocks = split_blocks
    p.target_workgroups = target_workgroups
    p.pool_mode = {"position_free": LA_POOL_POSITION_FREE,
                   "doc_local": LA_POOL_DOC_LOCAL}.get(pool_mode, pool_mode)
    p.pos_encoding = {"rope_half": LA_ROPE_HALF, "rope_interleaved": LA_ROPE_INTERLEAVED,
                      "alibi": LA_ALIBI}.get(pos_encoding, pos_encoding)
    p.check_tables = 1 if check_tables else 0
    return p


def _ptr(t) -> Optional[int]:
    """Device pointer of a tensor (None passes NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def lazy_attn_status_string(status: int) -> str:
    return _lib.lazy_attn_status_string(status).decode()


def lazy_attn_last_error() -> str:
    return _lib.lazy_attn_last_error().decode()


def lazy_attn_rope_table(base: float, head_dim: int, rows: int) -> np.ndarray:
    """Host float32 table [rows, head_dim] (cos half, then sin half)."""
    out = np.empty((rows, head_dim), dtype=np.float32)
    _check(_lib.lazy_attn_rope_table(float(base), head_dim, rows,
                                     out.ctypes.data_as(_f32p)), "lazy_attn_rope_table")
    return out


def lazy_attn_rope_table_scaled(base: float, head_dim: int, rows: int, scaling=None) -> np.ndarray:
    """Host float32 table [rows, head_dim] of a scaled RoPE variant.

    scaling: None, a la_rope_scaling, or a dict of make_scaling arguments.
    """
    if isinstance(scaling, dict):
        scaling = make_scaling(**scaling)
    out = np.empty((rows, head_dim), dtype=np.float32)
    ptr = None if scaling is None else ctypes.byref(scaling)
    _check(_lib.lazy_attn_rope_table_scaled(float(base), head_dim, rows, ptr,
                                            out.ctypes.data_as(_f32p)),
           "lazy_attn_rope_table_scaled")
    return out


def lazy_attn_alibi_slopes(num_heads: int) -> np.ndarray:
    """Host float32 [num_heads] standard ALiBi slopes."""
    out = np.empty(num_heads, dtype=np.float32)
    _check(_lib.lazy_attn_alibi_slopes(num_heads, out.ctypes.data_as(_f32p)),
           "lazy_attn_alibi_slopes")
    return out


def _segment_arrays(requests):
    """CSR arrays of segment lists (the layout lazy_attn_pack_segments takes)."""
    req_seg, starts, lens, news, blk_start, blocks = [0], [], [], [], [0], []
    for segs in requests:
        for s in segs:
            st, n, bl, nw = (s.start, s.n_tokens, s.blocks, s.is_new) if hasattr(s, "start") else s
            starts.append(int(st))
            lens.append(int(n))
            news.append(1 if nw else 0)
            bl = np.asarray(bl, dtype=np.int64).ravel()
            blocks.append(bl)
            blk_start.append(blk_start[-1] + len(bl))
        req_seg.append(len(starts))
    return (np.asarray(req_seg, np.int64), np.asarray(starts, np.int64),
            np.asarray(lens, np.int64), np.asarray(news, np.uint8),
            np.asarray(blk_start, np.int64),
            np.concatenate(blocks).astype(np.int64) if blocks else np.zeros(0, np.int64))


def lazy_attn_plan_shared_decode(params: la_params, requests: Sequence[Sequence],
                                 max_item_blocks: int = 0):
    """Shared-segment decode plan: (la_shared_plan_info, plan blob as uint8 numpy).

    The first call returns the sizes and the chunk length it chose; the
    second passes that length back, which gives the same plan without
    searching again."""
    a_req, a_st, a_len, a_new, a_bs, a_bl = _segment_arrays(requests)
    info = la_shared_plan_info()
    args = (ctypes.byref(params), len(requests), a_req.ctypes.data_as(_i64p),
            a_st.ctypes.data_as(_i64p), a_len.ctypes.data_as(_i64p), a_new.ctypes.data_as(_u8p),
            a_bs.ctypes.data_as(_i64p), a_bl.ctypes.data_as(_i64p))
    _check(_lib.lazy_attn_plan_shared_decode(*args, int(max_item_blocks), ctypes.byref(info),
                                             None, 0), "lazy_attn_plan_shared_decode")
    blob = np.zeros(int(info.plan_bytes), np.uint8)
    _check(_lib.lazy_attn_plan_shared_decode(*args, int(info.max_item_blocks), ctypes.byref(info),
                                             blob.ctypes.data, blob.nbytes),
           "lazy_attn_plan_shared_decode")
    return info, blob


def lazy_attn_decode_shared(params: la_params, info: la_shared_plan_info, plan, q, k_pool,
                            v_pool, q_pos, cos_sin, batch: int, out, lse=None, workspace=None,
                            stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.lazy_attn_decode_shared(ctypes.byref(params), ctypes.byref(info), _ptr(plan),
                                        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(q_pos),
                                        _ptr(cos_sin), batch, _ptr(out), _ptr(lse),
                                        _ptr(workspace), ws_bytes, _stream(stream)),
           "lazy_attn_decode_shared")


def lazy_attn_pack_segments(params: la_params, requests: Sequence[Sequence]):
    """Pack segment lists into (blk_words uint64, req_blk_start int32, max_blocks).

    requests[r] is a sequence of segments with attributes start, n_tokens,
    blocks and is_new (or tuples in that order).
    """
    req_seg, starts, lens, news, blk_start, blocks = [0], [], [], [], [0], []
    for segs in requests:
        for s in segs:
            st, n, bl, nw = (s.start, s.n_tokens, s.blocks, s.is_new) if hasattr(s, "start") else s
            starts.append(int(st))
            lens.append(int(n))
            news.append(1 if nw else 0)
            bl = np.asarray(bl, dtype=np.int64).ravel()
            blocks.append(bl)
            blk_start.append(blk_start[-1] + len(bl))
        req_seg.append(len(starts))
    a_req = np.asarray(req_seg, np.int64)
    a_st = np.asarray(starts, np.int64)
    a_len = np.asarray(lens, np.int64)
    a_new = np.asarray(news, np.uint8)
    a_bs = np.asarray(blk_start, np.int64)
    a_bl = np.concatenate(blocks).astype(np.int64) if blocks else np.zeros(0, np.int64)
    cap = max(1, int(a_bs[-1]))
    words = np.zeros(cap, np.uint64)
    rbs = np.zeros(len(requests) + 1, np.int32)
    maxb = ctypes.c_int32(0)
    _check(_lib.lazy_attn_pack_segments(
        ctypes.byref(params), len(requests), a_req.ctypes.data_as(_i64p),
        a_st.ctypes.data_as(_i64p), a_len.ctypes.data_as(_i64p), a_new.ctypes.data_as(_u8p),
        a_bs.ctypes.data_as(_i64p), a_bl.ctypes.data_as(_i64p), words.ctypes.data_as(_u64p), cap,
        rbs.ctypes.data_as(_i32p), ctypes.byref(maxb)), "lazy_attn_pack_segments")
    return words[: int(rbs[-1])], rbs, int(maxb.value)


def _hptr(x):
    """Pointer for host numpy arrays or device tensors."""
    if x is None:
        return None
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    return _ptr(x)


def lazy_attn_validate_table(params: la_params, batch: int, blk_words, req_blk_start, q_pos,
                             cu_q=None, max_blocks_per_req: int = 0, max_q_per_req: int = 0):
    _check(_lib.lazy_attn_validate_table(ctypes.byref(params), batch, _hptr(blk_words),
                                         _hptr(req_blk_start), _hptr(q_pos), _hptr(cu_q),
                                         int(max_blocks_per_req), int(max_q_per_req)),
           "lazy_attn_validate_table")


def lazy_attn_decode_workspace_size(params: la_params, batch: int, max_blocks_per_req: int) -> int:
    n = ctypes.c_size_t(0)
    _check(_lib.lazy_attn_decode_workspace_size(ctypes.byref(params), batch, max_blocks_per_req,
                                                ctypes.byref(n)), "lazy_attn_decode_workspace_size")
    return int(n.value)


def lazy_attn_store_kv(params: la_params, k, v, n_tokens: int, slots, rope_pos, cos_sin, k_pool,
                       v_pool, stream=None):
    _check(_lib.lazy_attn_store_kv(ctypes.byref(params), _ptr(k), _ptr(v), int(n_tokens),
                                   _ptr(slots), _ptr(rope_pos), _ptr(cos_sin), _ptr(k_pool),
                                   _ptr(v_pool), _stream(stream)), "lazy_attn_store_kv")


def lazy_attn_decode(params: la_params, q, k_pool, v_pool, blk_words, req_blk_start, q_pos,
                     cos_sin, batch: int, max_blocks_per_req: int, out, lse=None, workspace=None,
                     stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.lazy_attn_decode(ctypes.byref(params), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                 _ptr(blk_words), _ptr(req_blk_start), _ptr(q_pos), _ptr(cos_sin),
                                 batch, max_blocks_per_req, _ptr(out), _ptr(lse), _ptr(workspace),
                                 ws_bytes, _stream(stream)), "lazy_attn_decode")


def lazy_attn_decode_noalloc(params: la_params, q, k_pool, v_pool, blk_words, req_blk_start,
                             q_pos, cos_sin, batch: int, max_blocks_per_req: int, out, lse=None,
                             stream=None):
    _check(_lib.lazy_attn_decode_noalloc(ctypes.byref(params), _ptr(q), _ptr(k_pool),
                                         _ptr(v_pool), _ptr(blk_words), _ptr(req_blk_start),
                                         _ptr(q_pos), _ptr(cos_sin), batch, max_blocks_per_req,
                                         _ptr(out), _ptr(lse), _stream(stream)),
           "lazy_attn_decode_noalloc")


def lazy_attn_prefill(params: la_params, q, k_pool, v_pool, blk_words, req_blk_start, cu_q,
                      q_pos0, cos_sin, batch: int, max_q_per_req: int, out, lse=None,
                      stream=None):
    _check(_lib.lazy_attn_prefill(ctypes.byref(params), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                  _ptr(blk_words), _ptr(req_blk_start), _ptr(cu_q), _ptr(q_pos0),
                                  _ptr(cos_sin), batch, max_q_per_req, _ptr(out), _ptr(lse),
                                  _stream(stream)), "lazy_attn_prefill")


def lazy_attn_cache_simulate(docs, pos, num_positions: int, capacity: int, policy="agnostic",
                             eviction="lru") -> int:
    """Hits of a document-cache access trace (host arrays); see the C header."""
    d = np.ascontiguousarray(docs, dtype=np.int64)
    p = None if pos is None else np.ascontiguousarray(pos, dtype=np.int32)
    pol = {"agnostic": LA_CACHE_POSITION_AGNOSTIC, "aware": LA_CACHE_POSITION_AWARE}.get(policy,
                                                                                         policy)
    ev = {"lru": LA_EVICT_LRU, "static_top": LA_EVICT_STATIC_TOP}.get(eviction, eviction)
    hits = ctypes.c_int64(0)
    _check(_lib.lazy_attn_cache_simulate(len(d), d.ctypes.data_as(_i64p),
                                         None if p is None else p.ctypes.data_as(_i32p),
                                         int(num_positions), int(capacity), pol, ev,
                                         ctypes.byref(hits)), "lazy_attn_cache_simulate")
    return int(hits.value)

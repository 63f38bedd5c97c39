"""Lazy-RoPE paged attention on MI355X (gfx950).

liblazyattn.so (HIP kernels + C ABI, include/lazy_attn.h) computes attention
over a key/value block pool stored without positional encoding, applying RoPE
inside the kernels at each request's logical positions.  This package holds
the HIP sources (csrc/), the build script and a thin ctypes binding whose
functions carry the C names.
"""
from .binding import (  # noqa: F401
    LA_BF16,
    LA_FP32,
    LA_POOL_POSITION_FREE,
    LA_POOL_DOC_LOCAL,
    LA_ROPE_HALF,
    LA_ROPE_INTERLEAVED,
    LA_ALIBI,
    LazyAttnError,
    la_params,
    make_params,
    lazy_attn_status_string,
    lazy_attn_last_error,
    lazy_attn_rope_table,
    lazy_attn_rope_table_scaled,
    la_rope_scaling,
    make_scaling,
    lazy_attn_alibi_slopes,
    lazy_attn_pack_segments,
    lazy_attn_validate_table,
    lazy_attn_decode_workspace_size,
    lazy_attn_store_kv,
    lazy_attn_decode,
    lazy_attn_decode_noalloc,
    lazy_attn_plan_shared_decode,
    lazy_attn_decode_shared,
    la_shared_plan_info,
    lazy_attn_prefill,
    lazy_attn_cache_simulate,
)

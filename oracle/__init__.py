"""CPU oracle for lazy-RoPE paged attention -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import anything from this package.  The product path (the HIP library and its
Python binding) never imports, links or executes it, and shares no code with
it: the oracle recomputes RoPE frequencies, rotations and softmax attention
itself, in float64, from the definitions in "LazyAttention: Efficient
Retrieval-Augmented Generation with Deferred Positional Encoding" (§3.1
Eq. 4 and the RoPE form of attention, §3.2 Fact 3.2 and the rotation
formula, §2 Eqs. 1-3, §3.1-§3.2 cost model).

Every function is pinned by tests/test_oracle.py or tests/test_cache_sim.py
to something other than itself (each docstring names its pin): closed forms
(Eq. 3's 2.86x, Eqs. 1-2, the cost-model percentages), identities (Fact 3.2,
lazy = eager, shift invariance), special cases that reduce to a library or
textbook routine (identity table -> scaled dot-product attention, contiguous
placement -> causal RoPE attention, published NTK/YaRN/Llama-3.1 and ALiBi
formulas), and brute force in scalar Python on tiny inputs.  The pages print
no attention outputs, so no pin is a worked example of the attention itself.
The only result left unpinned is a reproduction of Table 1's cells: the pages
state neither the document size nor the eviction policy behind them.
"""
from .lazy_oracle import (  # noqa: F401
    rope_theta,
    rope_rotate,
    alibi_slopes,
    rope_theta_scaled,
    gather_request,
    attention_decode,
    attention_prefill,
    attention_decode_relative,
    store_kv,
    run_decode,
    run_prefill,
)
from .analysis import (  # noqa: F401
    hit_ratio_agnostic,
    hit_ratio_aware,
    hit_ratio_gap,
    naive_flops_overhead,
    naive_io_overhead,
    prefill_flops_overhead,
    prefill_table_bandwidth,
    decode_trigger_overhead,
    decode_overhead,
)
from .cache_oracle import simulate_cache  # noqa: F401,E402

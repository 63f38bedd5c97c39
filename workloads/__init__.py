"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This package generates data only: document pools of bf16/fp32 key and value
vectors, Zipf-skewed document mixes and segment lists.  It performs none of
the attention arithmetic (no rotation, no scores, no softmax), so both the
GPU path and the oracle can consume its output without sharing any method
code.
"""
from .synth import (  # noqa: F401
    Segment,
    Workload,
    MixedWorkload,
    CONFIGS,
    make_config,
    make_no_sharing_decode,
    build_workload,
    segment_writes,
    doc_trace,
    segment_slots,
    private_copies,
    zipf_probs,
    f32_to_bf16_bits,
    bf16_bits_to_f32,
)

"""Seeded synthetic workloads for the DSA-indexer Top-K path.

This package only draws random inputs and stores them in the storage formats
the library accepts (fp32, bf16 bits, OCP fp8 E4M3FN bits plus a per-token
fp32 scale).  It holds none of the indexer's arithmetic: no scores, no bounds,
no selection.  Both the CPU oracle and the GPU path take their inputs from it.
"""
from .workloads import (  # noqa: F401
    Workload,
    WORKLOADS,
    make_workload,
    tiny_prefill,
    dsa_prefill_32k,
    long_prefill_128k,
    decode_mtp,
    million_chunk,
    correlated_heads,
    correlated_decode,
    split_decode_steps,
    custom,
    quantize_fp8_per_token,
    to_bf16_bits,
)

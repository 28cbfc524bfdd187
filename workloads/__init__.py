"""Seeded synthetic inputs for paged KV-cache attention.

This package draws random numbers and lays them out in the paged-pool format;
it computes no attention.  It is the only code shared between the fp64 oracle
(``oracle/``) and the GPU path (``paged_kv_cache_attn_amd``): both read the
same host arrays, bit for bit.
"""

from .synth import (  # noqa: F401
    BF16_NAN_BITS,
    F32_NAN_BITS,
    Workload,
    bf16_round_bits,
    build_workload,
    WORKLOADS,
    named_workload,
)

"""fp64 CPU oracle for paged KV-cache attention.

TEST INFRASTRUCTURE ONLY.  This package states, slowly and in double
precision, what the GPU path must compute.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it; the product path (``paged_kv_cache_attn_amd``) never does, and the
two share no code.  See ``oracle/paged.py`` for the definitions and
the passages of the source pages each one follows.
"""

from .paged import (  # noqa: F401
    BlockMask,
    ScoreMods,
    attention_dense,
    bits_to_f64,
    gather_sequence,
    kv_append,
    paged_attention,
    v_group,
)

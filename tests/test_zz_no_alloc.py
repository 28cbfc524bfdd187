"""paged_attn_decode_noalloc: the decode on the library's own per-device
scratch (no workspace argument, no allocation) gives the bits of
paged_attn_decode with a caller workspace, call after call, and matches the
fp64 oracle."""

import numpy as np
import pytest
import torch

import oracle
from oracle.paged import bits_to_f64
from workloads import build_workload, named_workload
from workloads.device import to_numpy_bits, upload

pytestmark = pytest.mark.gpu


def _both(lib, w, split):
    """(noalloc output bits, caller-workspace output bits) after the append."""
    t = upload(w)
    lib.kv_append(t["k_new"], t["v_new"], t["k_cache"], t["v_cache"], t["slot_mapping"])
    out_a = torch.full_like(t["q"], float("nan"))
    out_b = torch.full_like(t["q"], float("nan"))
    lib.paged_attn_decode_noalloc(out_a, t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                                  w.scale, w.max_context_len, split)
    torch.cuda.synchronize()
    lib.paged_attn_decode(out_b, t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                          w.scale, w.max_context_len, split)
    torch.cuda.synchronize()
    return to_numpy_bits(out_a), to_numpy_bits(out_b)


def _oracle(w):
    kp, vp = oracle.kv_append(w.k_pool, w.v_pool, w.k_new, w.v_new, w.slot_mapping, w.bs)
    return oracle.paged_attention(w.q, kp, vp, w.block_table, w.context_lens, w.cu_q_lens, w.scale, w.bs, w.dtype)


@pytest.mark.parametrize("split", [0, -2, 512])
def test_noalloc_decode_matches_workspace_decode_twice(gpu_lib, split):
    """Two calls in a row on one device, the second on a smaller batch: the
    scratch keeps the first call's contents, which must not leak into the
    second."""
    w1 = named_workload("gqa_decode_bf16")
    w2 = build_workload(name="small", seed=77, kind="decode", dtype="bf16", Hq=32, Hkv=8, D=128, bs=16,
                        context_lens=[700, 1300], append_lens=[1, 1])
    assert gpu_lib.decode_workspace_size(w1.B, w1.Hq, w1.Hkv, w1.D, w1.max_context_len, split) > \
        gpu_lib.decode_workspace_size(w2.B, w2.Hq, w2.Hkv, w2.D, w2.max_context_len, split) > 0
    for w in (w1, w2):
        a, b = _both(gpu_lib, w, split)
        assert np.array_equal(a, b)
        got = bits_to_f64(a, "bf16")
        assert np.all(np.isfinite(got))
        assert np.max(np.abs(got - _oracle(w))) <= 2e-2


def test_noalloc_decode_long_batch_fits(gpu_lib):
    """The long-context batch (64 sequences, up to 32,768 keys) runs within
    the scratch; five sequences are checked against the oracle, all bits
    against the workspace decode."""
    w = named_workload("long_decode_bf16")
    assert gpu_lib.decode_workspace_size(w.B, w.Hq, w.Hkv, w.D, w.max_context_len, 0) <= gpu_lib.DECODE_SCRATCH_BYTES
    a, b = _both(gpu_lib, w, 0)
    assert np.array_equal(a, b)
    seqs = [0, 1, int(np.argmax(w.context_lens)), int(np.argmin(w.context_lens)), 63]
    kp, vp = oracle.kv_append(w.k_pool, w.v_pool, w.k_new, w.v_new, w.slot_mapping, w.bs)
    ref = oracle.paged_attention(w.q, kp, vp, w.block_table, w.context_lens, w.cu_q_lens, w.scale, w.bs, w.dtype,
                                 seqs=seqs)
    assert np.max(np.abs(bits_to_f64(a, "bf16")[seqs] - ref[seqs])) <= 2e-2


def test_noalloc_decode_refuses_oversized_batches(gpu_lib):
    w = build_workload(name="tiny", seed=5, kind="decode", dtype="bf16", Hq=64, Hkv=8, D=128, bs=16,
                       context_lens=[40, 50], append_lens=[1, 1])
    t = upload(w)
    out = torch.empty_like(t["q"])
    # a host bound on the context length this large needs more than 16 MiB of partials
    with pytest.raises(ValueError, match="scratch"):
        gpu_lib.paged_attn_decode_noalloc(out, t["q"], t["k_cache"], t["v_cache"], t["block_tables"],
                                          t["context_lens"], w.scale, 1 << 24, 16)


@pytest.mark.parametrize("split", [0, -2])
def test_noalloc_decode_inside_graph_replays(gpu_lib, split):
    """The callers this entry point is for capture it in HIP graphs: an
    append + decode + prefill step with the allocation-free decode, captured
    once and replayed after eager work that changes the inputs, gives the
    eager calls' bits on every replay."""
    from test_gpu_graphs import test_graph_replays_match_eager_calls
    test_graph_replays_match_eager_calls(gpu_lib, split, entry="noalloc")

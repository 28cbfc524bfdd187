"""The C-ABI calls on other streams and inside captured HIP graphs.

No call allocates or clears memory, so an append + decode + prefill step can
be captured once and replayed.  Each replay runs after eager work that
changes the inputs, and must give exactly the eager calls' result on the same
inputs.  The calls also take a non-default stream (default priority) and give
bit-identical results there.
"""

import numpy as np
import pytest
import torch

from workloads import build_workload
from workloads.device import to_numpy_bits, upload

pytestmark = pytest.mark.gpu


def _decode_batch():
    return build_workload(name="graph_decode", seed=901, kind="decode", dtype="bf16", Hq=32, Hkv=8, D=128, bs=16,
                          context_lens=[40, 700, 1500, 3000], append_lens=[1, 1, 1, 1])


def _prefill_batch():
    return build_workload(name="graph_prefill", seed=902, kind="prefill", dtype="bf16", Hq=32, Hkv=8, D=128, bs=16,
                          context_lens=[300, 520], q_lens=[100, 200], append_lens=[100, 200], causal=True)


@pytest.mark.parametrize("split", [0, -2, 64])
def test_graph_replays_match_eager_calls(gpu_lib, split, entry="workspace"):
    """The decode's split: the library's choice (512-key pieces as
    work-groups here), the balanced split, 64-key pieces.  `entry` =
    "noalloc" runs the allocation-free decode instead (tests/test_zz_no_alloc.py)."""
    wd, wp = _decode_batch(), _prefill_batch()
    td, tp = upload(wd), upload(wp)
    k0, v0 = td["k_cache"].clone(), td["v_cache"].clone()
    kp0, vp0 = tp["k_cache"].clone(), tp["v_cache"].clone()
    out_d = torch.empty_like(td["q"])
    out_p = torch.empty_like(tp["q"])
    ws = gpu_lib.decode_workspace(td["q"], wd.Hkv, wd.max_context_len, split)

    def step():
        gpu_lib.kv_append(td["k_new"], td["v_new"], td["k_cache"], td["v_cache"], td["slot_mapping"])
        if entry == "noalloc":
            gpu_lib.paged_attn_decode_noalloc(out_d, td["q"], td["k_cache"], td["v_cache"], td["block_tables"],
                                              td["context_lens"], wd.scale, wd.max_context_len, split)
        else:
            gpu_lib.paged_attn_decode(out_d, td["q"], td["k_cache"], td["v_cache"], td["block_tables"],
                                      td["context_lens"], wd.scale, wd.max_context_len, split, workspace=ws)
        gpu_lib.kv_append(tp["k_new"], tp["v_new"], tp["k_cache"], tp["v_cache"], tp["slot_mapping"])
        gpu_lib.paged_attn_prefill(out_p, tp["q"], tp["cu_q_lens"], tp["k_cache"], tp["v_cache"],
                                   tp["block_tables"], tp["context_lens"], wp.scale, wp.max_q_len, True)

    def reset(seed):
        # eager work between replays: fresh pools and new queries
        td["k_cache"].copy_(k0)
        td["v_cache"].copy_(v0)
        tp["k_cache"].copy_(kp0)
        tp["v_cache"].copy_(vp0)
        g = torch.Generator(device="cuda").manual_seed(seed)
        td["q"].copy_(torch.randn(td["q"].shape, generator=g, device="cuda").to(td["q"].dtype))
        tp["q"].copy_(torch.randn(tp["q"].shape, generator=g, device="cuda").to(tp["q"].dtype))
        torch.cuda.synchronize()

    step()  # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    reset(0)
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for seed in (1, 2, 3):
        reset(seed)
        step()
        torch.cuda.synchronize()
        want_d, want_p = to_numpy_bits(out_d).copy(), to_numpy_bits(out_p).copy()
        reset(seed)
        out_d.zero_()
        out_p.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_numpy_bits(out_d), want_d), f"decode replay {seed}"
        assert np.array_equal(to_numpy_bits(out_p), want_p), f"prefill replay {seed}"


def test_calls_on_a_side_stream(gpu_lib):
    w = _decode_batch()
    t = upload(w)
    gpu_lib.kv_append(t["k_new"], t["v_new"], t["k_cache"], t["v_cache"], t["slot_mapping"])
    ref = torch.empty_like(t["q"])
    gpu_lib.paged_attn_decode(ref, t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                              w.scale, w.max_context_len, 0)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()  # default priority
    out = torch.empty_like(t["q"])
    ws = gpu_lib.decode_workspace(t["q"], w.Hkv, w.max_context_len, 0)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gpu_lib.paged_attn_decode(out, t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                                  w.scale, w.max_context_len, 0, workspace=ws)
    side.synchronize()
    assert np.array_equal(to_numpy_bits(out), to_numpy_bits(ref))


def test_two_phase_decode_replays_in_a_graph(gpu_lib):
    """The two-phase decode (shared parts on the matrix cores, own keys by the
    decode, then the merge: four launches) captured in a graph: every replay,
    after eager calls on new queries, gives the eager call's bits; the eager
    result matches the oracle."""
    from tests.test_gpu_cascade import device_level, grouped
    from tests.test_gpu_parity import assert_close, oracle_out
    w, starts, prefix = grouped(912, [(5, 12), (3, 4)], [40, 1, 300, 17, 9, 200, 64, 1])
    t = upload(w)
    gpu_lib.kv_append(t["k_new"], t["v_new"], t["k_cache"], t["v_cache"], t["slot_mapping"])
    levels = [device_level(gpu_lib, starts, prefix)]
    out = torch.empty_like(t["q"])
    ws = gpu_lib.decode_cascade_workspace(t["q"], w.Hkv, levels, w.max_context_len)

    def call():
        gpu_lib.paged_attn_decode_cascade(out, t["q"], t["k_cache"], t["v_cache"], t["block_tables"],
                                          t["context_lens"], levels, w.scale, w.max_context_len, workspace=ws,
                                          mode="two_phase")

    call()
    torch.cuda.synchronize()
    assert_close(to_numpy_bits(out), oracle_out(w), "bf16")
    q0 = t["q"].clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for seed in (1, 2, 3):
        g = torch.Generator(device="cuda").manual_seed(seed)
        t["q"].copy_((q0.float() + 0.25 * torch.randn(q0.shape, generator=g, device="cuda")).to(q0.dtype))
        call()
        torch.cuda.synchronize()
        want = to_numpy_bits(out).copy()
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_numpy_bits(out), want), f"two-phase replay {seed}"


def test_split_prefill_replays_in_a_graph(gpu_lib):
    """The key-split prefill (ranges on the matrix cores, then the merge of
    their fp32 states through the caller's workspace) captured in a graph:
    every replay, after eager calls on new queries, gives the eager call's
    bits; the eager result matches the oracle."""
    from workloads import named_workload
    from tests.test_gpu_parity import assert_close, oracle_out
    w = named_workload("chunked_prefill_bf16", tp=8, batch=2)
    t = upload(w)
    gpu_lib.kv_append(t["k_new"], t["v_new"], t["k_cache"], t["v_cache"], t["slot_mapping"])
    out = torch.empty_like(t["q"])
    max_ctx = int(w.context_lens.max())
    ws = gpu_lib.prefill_workspace(t["q"], w.B, w.Hkv, w.max_q_len, max_ctx)
    assert ws is not None  # 32 work-groups: the library splits the keys

    def call():
        gpu_lib.paged_attn_prefill(out, t["q"], t["cu_q_lens"], t["k_cache"], t["v_cache"], t["block_tables"],
                                   t["context_lens"], w.scale, w.max_q_len, True, max_context_len=max_ctx,
                                   workspace=ws)

    call()
    torch.cuda.synchronize()
    assert_close(to_numpy_bits(out), oracle_out(w, causal=True), "bf16")
    q0 = t["q"].clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for seed in (1, 2, 3):
        g = torch.Generator(device="cuda").manual_seed(seed)
        t["q"].copy_((q0.float() + 0.25 * torch.randn(q0.shape, generator=g, device="cuda")).to(q0.dtype))
        call()
        torch.cuda.synchronize()
        want = to_numpy_bits(out).copy()
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_numpy_bits(out), want), f"split prefill replay {seed}"

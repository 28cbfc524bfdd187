"""GPU parity of the two-phase (shared-prefix) decode against the fp64 oracle.

Groups of consecutive sequences share their first blocks; the call computes
the shared prefix once per group and each sequence's own keys separately, and
must give the same attention as the plain definition over each sequence's
whole context (the oracle reads every sequence through its own table).
Tolerance: max-abs 2e-2 (bf16 inputs, fp32 accumulation), as for decode.
"""

import numpy as np
import pytest
import torch

from workloads import build_workload
from workloads.device import to_numpy_bits, upload

from tests.test_gpu_parity import TOL, assert_close, oracle_out
import oracle

pytestmark = pytest.mark.gpu


def grouped(seed, groups, private, cuts=None, Hq=32, Hkv=8, D=128, bs=16):
    """Decode batch whose groups (members, shared blocks) share their first
    blocks; sequence b has ``private[b]`` further tokens (the last one appended
    this step).  The group's prefix length is its shared blocks' tokens minus
    ``cuts[g]`` (a prefix may end inside a block)."""
    S_b = np.repeat([s for _, s in groups], [m for m, _ in groups]).astype(np.int64)
    private = np.asarray(private, np.int64)
    ctx = S_b * bs + private
    w = build_workload(name="cascade", seed=seed, kind="decode", dtype="bf16", Hq=Hq, Hkv=Hkv, D=D, bs=bs,
                       context_lens=ctx, append_lens=(private > 0).astype(np.int64), prefix_groups=groups)
    starts = np.concatenate([[0], np.cumsum([m for m, _ in groups])]).astype(np.int32)
    cuts = np.zeros(len(groups), np.int64) if cuts is None else np.asarray(cuts, np.int64)
    prefix = np.array([max(0, s * bs - c) for (_, s), c in zip(groups, cuts)], np.int32)
    return w, starts, prefix


def gpu_cascade(lib, w, starts, prefix, t=None, workspace=None, **mods):
    t = t or upload(w)
    if len(w.slot_mapping):
        lib.kv_append(t["k_new"], t["v_new"], t["k_cache"], t["v_cache"], t["slot_mapping"])
    out = torch.empty_like(t["q"])
    gs = torch.from_numpy(starts).cuda()
    pl = torch.from_numpy(prefix).cuda()
    max_group = int(np.max(np.diff(starts))) if len(starts) > 1 else 1
    lib.paged_attn_decode_cascade(out, t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                                  gs, pl, w.scale, w.max_context_len, max(1, max_group),
                                  int(prefix.max(initial=0)), workspace=workspace, **mods)
    torch.cuda.synchronize()
    return to_numpy_bits(out)


CASES = {
    # groups (members, shared blocks), private tokens per sequence, cuts per group
    "mixed": dict(groups=[(5, 8), (1, 3), (4, 0), (2, 20), (1, 0)],
                  private=[40, 0, 300, 17, 1, 5, 260, 0, 33, 64, 9, 128, 0], cuts=[3, 0, 0, 15, 0]),
    "d64_g4_bs64": dict(groups=[(3, 4), (6, 2)], private=[1, 100, 64, 0, 7, 300, 65, 2, 190], cuts=[10, 63],
                        Hq=16, Hkv=4, D=64, bs=64),
    "mha_bs256": dict(groups=[(4, 2), (2, 1)], private=[1, 500, 3, 256, 0, 77], cuts=[100, 0], Hq=8, Hkv=8,
                      bs=256),
    "g16_two_query_tiles": dict(groups=[(9, 5), (3, 1)], private=[1, 2, 3, 40, 50, 60, 70, 80, 90, 0, 16, 17],
                                cuts=[7, 1], Hq=32, Hkv=2),
    "empty_suffixes": dict(groups=[(6, 4)], private=[0] * 6, cuts=[0]),
    "empty_prefixes": dict(groups=[(3, 0), (2, 0)], private=[30, 1, 0, 500, 16], cuts=[0, 0]),
    # two key ranges of 320 keys; the second group's prefix leaves its second range empty
    "two_key_ranges": dict(groups=[(3, 40), (2, 3), (4, 20)], private=[1, 9, 77, 0, 5, 1, 2, 3, 300],
                           cuts=[5, 0, 17]),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_cascade_matches_oracle(gpu_lib, case):
    c = dict(CASES[case])
    groups, private, cuts = c.pop("groups"), c.pop("private"), c.pop("cuts")
    w, starts, prefix = grouped(700 + len(case), groups, private, cuts, **c)
    got = gpu_cascade(gpu_lib, w, starts, prefix)
    zero_rows = np.nonzero(w.context_lens == 0)[0]
    if len(zero_rows):
        assert np.all(got[zero_rows] == 0)
    assert_close(got, oracle_out(w), "bf16")


def test_cascade_softcap(gpu_lib):
    w, starts, prefix = grouped(711, [(4, 6), (3, 2)], [5, 1, 90, 0, 12, 300, 1], [5, 0])
    got = gpu_cascade(gpu_lib, w, starts, prefix, softcap=2.0)
    assert_close(got, oracle_out(w, oracle.ScoreMods(softcap=2.0)), "bf16")


def test_cascade_long_shared_prefix_sampled(gpu_lib):
    """64 sequences behind one 4059-token prefix (16 key ranges, the last
    one partial; four query tiles per kv-head); oracle on a sample of
    sequences."""
    rng = np.random.default_rng(712)
    private = rng.integers(0, 513, size=64)
    private[0] = 0
    w, starts, prefix = grouped(712, [(64, 256)], private, [37], Hq=64, Hkv=8)
    got = gpu_cascade(gpu_lib, w, starts, prefix)
    seqs = [0, 1, 17, 40, 63]
    assert_close(got, oracle_out(w, seqs=seqs), "bf16", rows=seqs)  # decode: row b is sequence b


def test_cascade_agrees_with_plain_decode(gpu_lib):
    """Same batch through paged_attn_decode: both are the same attention."""
    w, starts, prefix = grouped(713, [(8, 16), (8, 3)], list(range(1, 17)) * 1, [0, 9])
    t = upload(w)
    got = gpu_cascade(gpu_lib, w, starts, prefix, t=t)
    out = torch.empty_like(t["q"])  # the appended tokens are in the cache already
    gpu_lib.paged_attn_decode(out, t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                              w.scale, w.max_context_len, 0)
    torch.cuda.synchronize()
    from oracle.paged import bits_to_f64
    a, b = bits_to_f64(got, "bf16"), bits_to_f64(to_numpy_bits(out), "bf16")
    assert np.max(np.abs(a - b)) <= TOL["bf16"]


def test_cascade_workspace_reuse(gpu_lib):
    """One workspace, two calls in a row: the second (fewer groups, shorter
    prefixes) must not see the first call's states."""
    w1, s1, p1 = grouped(714, [(6, 12), (2, 5)], [3, 0, 50, 1, 7, 200, 9, 1], [0, 4])
    w2, s2, p2 = grouped(715, [(3, 2)], [1, 2, 3], [5])
    t1 = upload(w1)
    ws = gpu_lib.decode_cascade_workspace(t1["q"], w1.Hkv, len(p1), 6, w1.max_context_len, int(p1.max()))
    assert_close(gpu_cascade(gpu_lib, w1, s1, p1, t=t1, workspace=ws), oracle_out(w1), "bf16")
    assert_close(gpu_cascade(gpu_lib, w2, s2, p2, workspace=ws), oracle_out(w2), "bf16")

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


def device_level(lib, starts, ends, prefix_starts=None):
    """One prefix level from host arrays (group starts, range ends, range starts)."""
    starts = np.asarray(starts, np.int32)
    ends = np.asarray(ends, np.int32)
    lo = np.zeros_like(ends) if prefix_starts is None else np.asarray(prefix_starts, np.int32)
    return lib.prefix_level(torch.from_numpy(starts).cuda(), torch.from_numpy(ends).cuda(),
                            max(1, int(np.max(np.diff(starts), initial=1))), int(np.max(ends - lo, initial=0)),
                            None if prefix_starts is None else torch.from_numpy(lo).cuda())


def gpu_cascade_levels(lib, w, levels, t=None, workspace=None, **mods):
    t = t or upload(w)
    if len(w.slot_mapping):
        lib.kv_append(t["k_new"], t["v_new"], t["k_cache"], t["v_cache"], t["slot_mapping"])
    out = torch.empty_like(t["q"])
    lib.paged_attn_decode_cascade(out, t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                                  levels, w.scale, w.max_context_len, workspace=workspace, mode="two_phase", **mods)
    torch.cuda.synchronize()
    return to_numpy_bits(out)


def gpu_cascade(lib, w, starts, prefix, t=None, workspace=None, **mods):
    return gpu_cascade_levels(lib, w, [device_level(lib, starts, prefix)], t=t, workspace=workspace, **mods)


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
    ws = gpu_lib.decode_cascade_workspace(t1["q"], w1.Hkv, [device_level(gpu_lib, s1, p1)], w1.max_context_len)
    assert_close(gpu_cascade(gpu_lib, w1, s1, p1, t=t1, workspace=ws), oracle_out(w1), "bf16")
    assert_close(gpu_cascade(gpu_lib, w2, s2, p2, workspace=ws), oracle_out(w2), "bf16")


# ------------------------------------------------------------------------------------------
# nested prefixes (several levels)
# ------------------------------------------------------------------------------------------

def nested(seed, specs, private, cuts, Hq=32, Hkv=8, D=128, bs=16):
    """Decode batch with nested shared prefixes.  ``specs[l]`` lists level l's
    groups as (members, blocks): the members share ``blocks`` more blocks
    after the previous levels' (groups nest: each level refines the one
    before).  The tables of the members are pointed at the group leader's
    blocks; the prefix ranges end ``cuts[l][g]`` keys before the shared
    blocks do (a range may end inside a block)."""
    B = len(private)
    cum = np.zeros(B, np.int64)
    for spec in specs:
        assert sum(m for m, _ in spec) == B
        cum += np.repeat([nb for _, nb in spec], [m for m, _ in spec])
    private = np.asarray(private, np.int64)
    ctx = cum * bs + private
    w = build_workload(name="nested", seed=seed, kind="decode", dtype="bf16", Hq=Hq, Hkv=Hkv, D=D, bs=bs,
                       context_lens=ctx, append_lens=(private > 0).astype(np.int64))
    table = w.block_table
    levels = []
    off_blocks = np.zeros(B, np.int64)
    prev_end = np.zeros(B, np.int64)
    for spec, cut in zip(specs, cuts):
        starts = np.concatenate([[0], np.cumsum([m for m, _ in spec])]).astype(np.int32)
        lo, hi = [], []
        for g, (m, nb) in enumerate(spec):
            mem = range(starts[g], starts[g + 1])
            if m == 0:
                lo.append(0)
                hi.append(0)
                continue
            lead = starts[g]
            b0 = int(off_blocks[lead])
            assert all(off_blocks[b] == b0 and prev_end[b] == prev_end[lead] for b in mem)
            for b in mem:
                table[b, b0:b0 + nb] = table[lead, b0:b0 + nb]
            start = int(prev_end[lead])
            end = max(start, (b0 + nb) * bs - int(cut[g]))
            lo.append(start)
            hi.append(end)
            for b in mem:
                off_blocks[b] = b0 + nb
                prev_end[b] = end
        levels.append((starts, np.array(hi, np.int32), np.array(lo, np.int32)))
    return w, levels


NESTED = {
    "two_levels": dict(specs=[[(12, 16)], [(4, 8), (4, 0), (3, 20), (1, 2)]],
                       private=[1, 40, 0, 7, 300, 1, 2, 3, 64, 0, 90, 5], cuts=[[5], [3, 0, 15, 0]]),
    "three_levels_g8": dict(specs=[[(9, 4)], [(5, 2), (4, 3)], [(2, 1), (3, 0), (4, 5)]],
                            private=[1, 2, 30, 0, 17, 200, 1, 5, 64], cuts=[[0], [7, 0], [1, 0, 9]],
                            Hq=64, Hkv=8),
    "two_groups_per_level_d64": dict(specs=[[(3, 6), (3, 2)], [(1, 1), (2, 4), (3, 0)]],
                                     private=[5, 1, 300, 0, 33, 2], cuts=[[0, 9], [2, 0, 0]], Hq=16, Hkv=4,
                                     D=64),
}


@pytest.mark.parametrize("case", sorted(NESTED))
def test_nested_prefixes_match_oracle(gpu_lib, case):
    c = dict(NESTED[case])
    specs, private, cuts = c.pop("specs"), c.pop("private"), c.pop("cuts")
    w, lv = nested(800 + len(case), specs, private, cuts, **c)
    levels = [device_level(gpu_lib, st, hi, lo) for st, hi, lo in lv]
    assert_close(gpu_cascade_levels(gpu_lib, w, levels), oracle_out(w), "bf16")


def test_nested_long_prefixes_sampled(gpu_lib):
    """64 sequences: a 2048-token prompt for all, then 8 conversations of 8
    sharing 1021 more tokens, then up to 256 own tokens; several key ranges
    at both levels.  Oracle on a sample of sequences."""
    rng = np.random.default_rng(830)
    private = rng.integers(0, 257, size=64)
    private[5] = 0
    w, lv = nested(830, [[(64, 128)], [(8, 64)] * 8], private, [[0], [3] * 8], Hq=64, Hkv=8)
    levels = [device_level(gpu_lib, st, hi, lo) for st, hi, lo in lv]
    got = gpu_cascade_levels(gpu_lib, w, levels)
    seqs = [0, 5, 9, 31, 63]
    assert_close(got, oracle_out(w, seqs=seqs), "bf16", rows=seqs)


# ------------------------------------------------------------------------------------------
# score mods through the two-phase decode
# ------------------------------------------------------------------------------------------

def _mods_for(w, seed, window=0, softcap=0.0, alibi=False, docs=False):
    """Device mods and the oracle's ScoreMods for a decode batch."""
    rng = np.random.default_rng(seed)
    kw, om = {}, dict(window=window, softcap=softcap)
    if window:
        kw["window"] = window
    if softcap:
        kw["softcap"] = softcap
    if alibi:
        slopes = (2.0 ** (-8.0 * np.arange(1, w.Hq + 1) / w.Hq)).astype(np.float32)
        kw["alibi_slopes"] = torch.from_numpy(slopes).cuda()
        om["alibi_slopes"] = slopes
    if docs:
        # each row's document starts somewhere in its context (inside a shared range too)
        starts = np.array([int(rng.integers(0, max(1, n))) for n in w.context_lens], np.int32)
        kw["doc_starts"] = torch.from_numpy(starts).cuda()
        om["doc_starts"] = starts
    return kw, oracle.ScoreMods(**om)


MOD_CASES = {
    "window_cuts_prefix": dict(window=150),
    "alibi": dict(alibi=True),
    "documents": dict(docs=True),
    "all": dict(window=333, softcap=3.0, alibi=True, docs=True),
}


@pytest.mark.parametrize("mods", sorted(MOD_CASES))
def test_cascade_mods_single_level(gpu_lib, mods):
    c = dict(CASES["mixed"])
    groups, private, cuts = c.pop("groups"), c.pop("private"), c.pop("cuts")
    w, starts, prefix = grouped(760, groups, private, cuts, **c)
    kw, om = _mods_for(w, 761, **MOD_CASES[mods])
    got = gpu_cascade(gpu_lib, w, starts, prefix, **kw)
    assert_close(got, oracle_out(w, om), "bf16")


@pytest.mark.parametrize("mods", ["window_cuts_prefix", "all"])
def test_cascade_mods_nested(gpu_lib, mods):
    c = dict(NESTED["two_levels"])
    specs, private, cuts = c.pop("specs"), c.pop("private"), c.pop("cuts")
    w, lv = nested(770, specs, private, cuts, **c)
    kw, om = _mods_for(w, 771, **MOD_CASES[mods])
    levels = [device_level(gpu_lib, st, hi, lo) for st, hi, lo in lv]
    assert_close(gpu_cascade_levels(gpu_lib, w, levels, **kw), oracle_out(w, om), "bf16")


def _auto_and(lib, w, starts, prefix, other):
    """(bits of the default call, bits of ``other``: "plain" decode or forced "two_phase")."""
    t = upload(w)
    lib.kv_append(t["k_new"], t["v_new"], t["k_cache"], t["v_cache"], t["slot_mapping"])
    levels = [device_level(lib, starts, prefix)]
    out_a = torch.full_like(t["q"], float("nan"))
    out_b = torch.full_like(t["q"], float("nan"))
    lib.paged_attn_decode_cascade(out_a, t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                                  levels, w.scale, w.max_context_len)
    if other == "plain":
        lib.paged_attn_decode(out_b, t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                              w.scale, w.max_context_len, 0)
    else:
        lib.paged_attn_decode_cascade(out_b, t["q"], t["k_cache"], t["v_cache"], t["block_tables"],
                                      t["context_lens"], levels, w.scale, w.max_context_len, mode="two_phase")
    torch.cuda.synchronize()
    return to_numpy_bits(out_a), to_numpy_bits(out_b)


def test_cascade_default_runs_the_plain_decode_on_the_shared_prefix_batch(gpu_lib):
    """16 sequences behind a 1,024-token prompt with 256 own tokens each: 84 MB
    of logical K+V, below the 256 MiB where the two-phase decode pays off, so
    the default call runs the plain decode (same bits) -- never slower."""
    from workloads import named_workload
    w = named_workload("shared_prefix_decode_bf16")
    starts, prefix = np.array([0, w.B], np.int32), np.array([1024], np.int32)
    assert gpu_lib.decode_cascade_plan(w.B, [device_level(gpu_lib, starts, prefix)], w.Hq, w.Hkv, w.D,
                                       w.max_context_len) == 0
    a, b = _auto_and(gpu_lib, w, starts, prefix, "plain")
    assert np.array_equal(a, b)
    assert_close(a, oracle_out(w), "bf16")


def test_cascade_default_runs_two_phase_on_large_batches(gpu_lib):
    """64 sequences behind one 1,024-token prompt, 256 own tokens each (335 MB
    logical): the default call is the two-phase decode (same bits)."""
    private = np.full(64, 256)
    w, starts, prefix = grouped(715, [(64, 64)], private, [0])
    assert gpu_lib.decode_cascade_plan(w.B, [device_level(gpu_lib, starts, prefix)], w.Hq, w.Hkv, w.D,
                                       w.max_context_len) == 1
    a, b = _auto_and(gpu_lib, w, starts, prefix, "two_phase")
    assert np.array_equal(a, b)
    seqs = [0, 31, 63]
    assert_close(a, oracle_out(w, seqs=seqs), "bf16", rows=seqs)

"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances (max-abs error of the output against the fp64 oracle): 2e-2 for
bf16 inputs with fp32 accumulation, 1e-4 for fp32; kv_append is bit-exact
over the whole pool.  Invariances that the pages state (scattered placement
and shared blocks give the same result) are checked bit for bit.
"""

import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
from oracle.paged import bits_to_f64
from workloads import bf16_round_bits, build_workload, named_workload
from workloads.device import to_numpy_bits, to_tensor, upload

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}


# ------------------------------------------------------------------------------------------
# helpers
# ------------------------------------------------------------------------------------------

def appended_pools(w):
    if len(w.slot_mapping) == 0:
        return w.k_pool, w.v_pool
    return oracle.kv_append(w.k_pool, w.v_pool, w.k_new, w.v_new, w.slot_mapping, w.bs)


def oracle_out(w, mods=None, seqs=None, causal=None):
    kp, vp = appended_pools(w)
    m = mods or oracle.ScoreMods()
    if causal is not None:
        m = dataclasses.replace(m, causal=causal)
    return oracle.paged_attention(w.q, kp, vp, w.block_table, w.context_lens, w.cu_q_lens, w.scale, w.bs,
                                  w.dtype, m, seqs=seqs)


def gpu_decode(lib, w, t=None, split=0, phase="both", **mods):
    t = t or upload(w)
    if len(w.slot_mapping):
        lib.kv_append(t["k_new"], t["v_new"], t["k_cache"], t["v_cache"], t["slot_mapping"])
    out = torch.empty_like(t["q"])
    if phase == "both":
        lib.paged_attn_decode(out, t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                              w.scale, w.max_context_len, split, **mods)
    else:
        ws = lib.decode_workspace(t["q"], w.Hkv, w.max_context_len, split)
        lib.paged_attn_decode(out, t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                              w.scale, w.max_context_len, split, workspace=ws, phase="partials", **mods)
        lib.paged_attn_decode(out, t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                              w.scale, w.max_context_len, split, workspace=ws, phase="merge", **mods)
    torch.cuda.synchronize()
    return to_numpy_bits(out)


def gpu_prefill(lib, w, t=None, causal=True, **mods):
    t = t or upload(w)
    if len(w.slot_mapping):
        lib.kv_append(t["k_new"], t["v_new"], t["k_cache"], t["v_cache"], t["slot_mapping"])
    out = torch.empty_like(t["q"])
    lib.paged_attn_prefill(out, t["q"], t["cu_q_lens"], t["k_cache"], t["v_cache"], t["block_tables"],
                           t["context_lens"], w.scale, w.max_q_len, causal, **mods)
    torch.cuda.synchronize()
    return to_numpy_bits(out)


def assert_close(gpu_bits, ref, dtype, rows=None, tol=None):
    got = bits_to_f64(gpu_bits, dtype)
    if rows is not None:
        got, ref = got[rows], ref[rows]
    assert np.all(np.isfinite(got)), "non-finite output"
    err = np.max(np.abs(got - ref)) if got.size else 0.0
    assert err <= (tol or TOL[dtype]), f"max abs err {err}"
    return err


def small(kind="decode", seed=100, dtype="bf16", ctx=(37, 300, 1000), Hq=32, Hkv=8, D=128, bs=16, q_lens=None,
          append=None, causal=False, shared=0, NB=None):
    return build_workload(name="t", seed=seed, kind=kind, dtype=dtype, Hq=Hq, Hkv=Hkv, D=D, bs=bs,
                          context_lens=list(ctx), q_lens=q_lens, append_lens=append, causal=causal,
                          shared_prefix_blocks=shared, NB=NB)


# ------------------------------------------------------------------------------------------
# kv_append
# ------------------------------------------------------------------------------------------

@pytest.mark.parametrize("case", ["gqa_decode", "chunked_prefill", "bs64_f32", "negative_slots",
                                  "mixed_runs_bf16_d64"])
def test_kv_append_bit_exact(gpu_lib, case):
    if case == "gqa_decode":
        w = named_workload("gqa_decode_bf16")
    elif case == "mixed_runs_bf16_d64":
        # runs of 16 new tokens that are one V sub-slab, that start inside one,
        # and that straddle two sequences
        w = small(ctx=(48, 100, 300), append=[40, 100, 37], D=64, Hq=8, Hkv=4, bs=32)
    elif case == "chunked_prefill":
        w = named_workload("chunked_prefill_bf16")
    elif case == "bs64_f32":
        w = small(dtype="f32", bs=64, ctx=(200, 129), append=[70, 129], D=64, Hq=8, Hkv=2)
    else:
        w = small(ctx=(40, 50), append=[5, 9])
        w.slot_mapping[::3] = -1
    t = upload(w)
    gpu_lib.kv_append(t["k_new"], t["v_new"], t["k_cache"], t["v_cache"], t["slot_mapping"])
    torch.cuda.synchronize()
    kp, vp = oracle.kv_append(w.k_pool, w.v_pool, w.k_new, w.v_new, w.slot_mapping, w.bs)
    ik = np.uint16 if w.dtype == "bf16" else np.uint32
    assert np.array_equal(to_numpy_bits(t["k_cache"]).view(ik), kp.view(ik))
    assert np.array_equal(to_numpy_bits(t["v_cache"]).view(ik), vp.view(ik))


# ------------------------------------------------------------------------------------------
# the reference workloads
# ------------------------------------------------------------------------------------------

def test_single_decode_f32(gpu_lib):
    w = named_workload("single_decode_f32")
    for split in (0, -2, -1, 16):
        assert_close(gpu_decode(gpu_lib, w, split=split), oracle_out(w), "f32")


def test_gqa_decode_with_append(gpu_lib):
    w = named_workload("gqa_decode_bf16")
    ref = oracle_out(w)
    for split in (0, -2, 512, -1):
        assert_close(gpu_decode(gpu_lib, w, split=split), ref, "bf16")


def test_chunked_prefill(gpu_lib):
    w = named_workload("chunked_prefill_bf16")
    assert_close(gpu_prefill(gpu_lib, w), oracle_out(w, causal=True), "bf16")


def test_shared_prefix_decode(gpu_lib):
    w = named_workload("shared_prefix_decode_bf16")
    assert_close(gpu_decode(gpu_lib, w), oracle_out(w), "bf16")


def test_long_decode_subset(gpu_lib):
    w = named_workload("long_decode_bf16", batch=6)
    assert_close(gpu_decode(gpu_lib, w, split=512), oracle_out(w), "bf16")


@pytest.mark.parametrize("bs", [32, 64, 128, 256])
def test_long_decode_page_size_variants_subset(gpu_lib, bs):
    w = named_workload("long_decode_bf16", bs=bs, batch=4)
    assert_close(gpu_decode(gpu_lib, w, split=512), oracle_out(w), "bf16")


def oracle_decode_compact(w):
    """The oracle's decode of every sequence, each on a compact copy of its
    own blocks (append included), so that a multi-GB pool is never copied
    whole; the same result as ``oracle_out`` (block placement does not change
    it)."""
    ref = np.full(bits_to_f64(w.q, w.dtype).shape, np.nan)
    for b in range(w.B):
        n = int(w.context_lens[b])
        nb = (n + w.bs - 1) // w.bs
        ids = w.block_table[b, :nb].astype(np.int64)
        kp, vp = w.k_pool[ids], w.v_pool[ids]
        # appended tokens that land in this sequence's blocks, re-addressed to the copy
        rows = [t for t in range(len(w.slot_mapping)) if w.slot_mapping[t] >= 0 and
                np.any(ids == w.slot_mapping[t] // w.bs)]
        slots = np.array([int(np.nonzero(ids == w.slot_mapping[t] // w.bs)[0][0]) * w.bs + w.slot_mapping[t] % w.bs
                          for t in rows], np.int32)
        if rows:
            kp, vp = oracle.kv_append(kp, vp, w.k_new[rows], w.v_new[rows], slots, w.bs)
        ref[b:b + 1] = oracle.paged_attention(w.q[b:b + 1], kp, vp, np.arange(nb, dtype=np.int32)[None],
                                              w.context_lens[b:b + 1], np.array([0, 1]), w.scale, w.bs, w.dtype)
    return ref


@pytest.mark.parametrize("split", [0, 512])
def test_long_decode_full_size_every_row(gpu_lib, split):
    """The full 64-sequence long-context batch (686,305 tokens) with the
    benchmarked launch (the balanced split, 0) and the fixed 512-token split
    measured beside it; every row against the oracle."""
    w = named_workload("long_decode_bf16")
    got = gpu_decode(gpu_lib, w, split=split)
    assert_close(got, oracle_decode_compact(w), "bf16")


@pytest.mark.parametrize("bs", [32, 64, 128, 256])
def test_long_decode_page_sizes_full_size_every_row(gpu_lib, bs):
    """The full long-context batch at each power-of-two page size with the
    balanced split that the page-size sweep times; every row."""
    w = named_workload("long_decode_bf16", bs=bs)
    got = gpu_decode(gpu_lib, w, split=0)
    assert_close(got, oracle_decode_compact(w), "bf16")


# ------------------------------------------------------------------------------------------
# invariances and special cases on the GPU
# ------------------------------------------------------------------------------------------

def test_block_permutation_bit_identical(gpu_lib):
    w = small(ctx=(700, 45, 1300), append=[1, 1, 1])
    base = gpu_decode(gpu_lib, w)
    perm = np.random.default_rng(1).permutation(w.NB)
    for pool in ("k_pool", "v_pool"):
        p = np.empty_like(getattr(w, pool))
        p[perm] = getattr(w, pool)
        setattr(w, pool, p)
    w.block_table = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], -1).astype(np.int32)
    w.slot_mapping = (perm[w.slot_mapping // w.bs] * w.bs + w.slot_mapping % w.bs).astype(np.int32)
    assert np.array_equal(gpu_decode(gpu_lib, w), base)


def test_prefill_block_permutation_bit_identical(gpu_lib):
    w = small("prefill", ctx=(300, 520), q_lens=[77, 130], causal=True)
    base = gpu_prefill(gpu_lib, w)
    perm = np.random.default_rng(2).permutation(w.NB)
    for pool in ("k_pool", "v_pool"):
        p = np.empty_like(getattr(w, pool))
        p[perm] = getattr(w, pool)
        setattr(w, pool, p)
    w.block_table = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], -1).astype(np.int32)
    assert np.array_equal(gpu_prefill(gpu_lib, w), base)


def test_shared_prefix_equals_private_copies(gpu_lib):
    w = named_workload("shared_prefix_decode_bf16", batch=4)
    base = gpu_decode(gpu_lib, w)
    S = int(w.meta["shared_prefix_blocks"])
    kp = np.concatenate([w.k_pool, w.k_pool[w.block_table[:, :S].ravel()]])
    vp = np.concatenate([w.v_pool, w.v_pool[w.block_table[:, :S].ravel()]])
    table = w.block_table.copy()
    table[:, :S] = (w.NB + np.arange(w.B * S)).reshape(w.B, S)
    w.k_pool, w.v_pool, w.block_table, w.NB = kp, vp, table.astype(np.int32), kp.shape[0]
    assert np.array_equal(gpu_decode(gpu_lib, w), base)


@pytest.mark.parametrize("kind", ["prefill", "decode"])
def test_running_max_moves_many_times(gpu_lib, kind):
    """Two fresh sequences (every key arrives through kv_append, in position
    order) whose key magnitudes grow up to 15-fold along the batch, with the
    queries doubled: later tiles keep raising each row's maximum past the lazy
    rescale threshold, so O and l are rescaled many times per row.  V is
    scaled by 0.4 so that outputs stay below 2 in magnitude, where the
    absolute bound is not dominated by the bf16 rounding of the output itself
    (half an ulp is at most 1/256 there, 1/64 at 4)."""
    prefill = kind == "prefill"
    w = small(kind, ctx=(1100, 400), q_lens=[1100, 400] if prefill else None, append=[1100, 400], causal=prefill,
              seed=5)
    k = bits_to_f64(w.k_new, "bf16")
    grow = 1.0 + np.arange(k.shape[0], dtype=np.float64) / 100.0
    w.k_new = bf16_round_bits((k * grow[:, None, None]).astype(np.float32))
    w.v_new = bf16_round_bits((bits_to_f64(w.v_new, "bf16") * 0.4).astype(np.float32))
    w.q = bf16_round_bits((bits_to_f64(w.q, "bf16") * 2.0).astype(np.float32))
    if prefill:
        assert_close(gpu_prefill(gpu_lib, w), oracle_out(w, causal=True), "bf16")
    else:
        for split in (0, -2, 64, -1):
            assert_close(gpu_decode(gpu_lib, w, split=split), oracle_out(w), "bf16")


def test_decode_merge_of_more_than_32_partials(gpu_lib):
    """Rows of 3,000 and 2,500 fresh keys whose magnitudes grow along the row,
    at 64-key partitions: 47 and 40 partial states, which the merge reads in
    two batches (32, then the rest); the second batch holds the larger maxima
    and rescales what the first summed.  Also at 128 keys (24 and 20 states,
    one batch) and with the balanced split."""
    w = small(ctx=(3000, 2500), append=[3000, 2500], Hq=8, Hkv=2, seed=23)
    k = bits_to_f64(w.k_new, "bf16")
    grow = 1.0 + np.arange(k.shape[0], dtype=np.float64) / 400.0
    w.k_new = bf16_round_bits((k * grow[:, None, None]).astype(np.float32))
    w.q = bf16_round_bits((bits_to_f64(w.q, "bf16") * 2.0).astype(np.float32))
    ref = oracle_out(w)
    for split in (64, 128, -2):
        assert_close(gpu_decode(gpu_lib, w, split=split), ref, "bf16")
        assert_close(gpu_decode(gpu_lib, w, split=split, phase="partials+merge"), ref, "bf16")


@pytest.mark.parametrize("kind", ["prefill", "decode"])
def test_running_max_moves_many_times_unscaled_values(gpu_lib, kind):
    """The growing-keys batch above with V ~ N(0,1) left as drawn, so peaked
    rows have outputs of magnitude 2-5, where bf16 output rounding alone
    spends up to 2^-8 |o| of the bound."""
    prefill = kind == "prefill"
    w = small(kind, ctx=(1100, 400), q_lens=[1100, 400] if prefill else None, append=[1100, 400], causal=prefill,
              seed=5)
    k = bits_to_f64(w.k_new, "bf16")
    grow = 1.0 + np.arange(k.shape[0], dtype=np.float64) / 100.0
    w.k_new = bf16_round_bits((k * grow[:, None, None]).astype(np.float32))
    w.q = bf16_round_bits((bits_to_f64(w.q, "bf16") * 2.0).astype(np.float32))
    ref = oracle_out(w, causal=prefill)
    assert np.max(np.abs(ref)) > 2.0
    if prefill:
        assert_close(gpu_prefill(gpu_lib, w), ref, "bf16")
    else:
        for split in (0, -2, 64, -1):
            assert_close(gpu_decode(gpu_lib, w, split=split), ref, "bf16")


def test_prefill_peaked_rows_unscaled_values(gpu_lib):
    """The chunked-prefill batch with queries scaled 16-fold: scores have a
    standard deviation of 16, so most rows put almost all their weight on one
    key and the output is close to that key's V row (N(0,1), up to ~5 in
    magnitude).  The decode batch the same way."""
    w = named_workload("chunked_prefill_bf16")
    w.q = bf16_round_bits((bits_to_f64(w.q, "bf16") * 16.0).astype(np.float32))
    ref = oracle_out(w, causal=True)
    assert np.max(np.abs(ref)) > 4.0
    assert_close(gpu_prefill(gpu_lib, w), ref, "bf16")
    wd = named_workload("gqa_decode_bf16")
    wd.q = bf16_round_bits((bits_to_f64(wd.q, "bf16") * 16.0).astype(np.float32))
    refd = oracle_out(wd)
    for split in (0, -2, 64, -1):
        assert_close(gpu_decode(gpu_lib, wd, split=split), refd, "bf16")


def test_one_token_context_returns_v_row_exactly(gpu_lib):
    w = small(ctx=(1, 1, 1), append=[1, 1, 1])
    got = gpu_decode(gpu_lib, w)
    g = w.Hq // w.Hkv
    for b in range(w.B):
        assert np.array_equal(got[b], np.repeat(w.v_new[b], g, axis=0))


def test_deterministic_bits(gpu_lib):
    w = named_workload("gqa_decode_bf16")
    t = upload(w)
    a = gpu_decode(gpu_lib, w, t=t)
    b = gpu_decode(gpu_lib, w, t=t)
    assert np.array_equal(a, b)
    w3 = named_workload("chunked_prefill_bf16", batch=2)
    t3 = upload(w3)
    assert np.array_equal(gpu_prefill(gpu_lib, w3, t=t3), gpu_prefill(gpu_lib, w3, t=t3))


@pytest.mark.parametrize("split", [0, -2, -1, 16, 64, 512])
def test_split_invariance(gpu_lib, split):
    w = small(ctx=(1500, 333, 2048, 17), append=[1, 1, 1, 1])
    assert_close(gpu_decode(gpu_lib, w, split=split), oracle_out(w), "bf16")


@pytest.mark.parametrize("split", [0, -2, 64])
def test_two_phase_calls_equal_single_call(gpu_lib, split):
    w = small(ctx=(1500, 333, 2048, 17), append=[1, 1, 1, 1])
    assert np.array_equal(gpu_decode(gpu_lib, w, split=split, phase="two"), gpu_decode(gpu_lib, w, split=split))


def test_decode_equals_prefill_with_one_row(gpu_lib):
    w = small(ctx=(900, 31, 256), append=[1, 1, 1])
    dec = gpu_decode(gpu_lib, w)
    wp = small(ctx=(900, 31, 256), append=[1, 1, 1])
    wp.kind = "prefill"
    pre = gpu_prefill(gpu_lib, wp, causal=True)
    assert np.max(np.abs(bits_to_f64(dec, "bf16") - bits_to_f64(pre, "bf16"))) <= 2e-2


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 4), (16, 4), (32, 8), (64, 8), (128, 8), (24, 8)])
def test_gqa_group_sizes(gpu_lib, Hq, Hkv):
    w = small(ctx=(129, 700), Hq=Hq, Hkv=Hkv, append=[1, 1])
    assert_close(gpu_decode(gpu_lib, w), oracle_out(w), "bf16")
    wp = small("prefill", ctx=(129, 300), q_lens=[40, 129], Hq=Hq, Hkv=Hkv, causal=True)
    assert_close(gpu_prefill(gpu_lib, wp), oracle_out(wp, causal=True), "bf16")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
def test_head_dims_and_dtypes(gpu_lib, dtype, D):
    w = small(dtype=dtype, D=D, ctx=(77, 640), append=[1, 1])
    assert_close(gpu_decode(gpu_lib, w), oracle_out(w), dtype)
    wp = small("prefill", dtype=dtype, D=D, ctx=(64, 200), q_lens=[64, 57], causal=True)
    assert_close(gpu_prefill(gpu_lib, wp), oracle_out(wp, causal=True), dtype)


@pytest.mark.parametrize("bs", [16, 32, 64, 128, 256])
def test_block_sizes_ragged(gpu_lib, bs):
    w = small(bs=bs, ctx=(1, 15, 16, 17, 255, 257, 1000), append=[1] * 7)
    assert_close(gpu_decode(gpu_lib, w), oracle_out(w), "bf16")
    wp = small("prefill", bs=bs, ctx=(1, 65, 300), q_lens=[1, 65, 99], causal=True)
    assert_close(gpu_prefill(gpu_lib, wp), oracle_out(wp, causal=True), "bf16")


@pytest.mark.parametrize("split", [0, -2, -1, 64, 512])
def test_empty_context_gives_zero(gpu_lib, split):
    w = small(ctx=(0, 5, 0))
    got = bits_to_f64(gpu_decode(gpu_lib, w, split=split), "bf16")
    assert np.all(got[0] == 0) and np.all(got[2] == 0)
    assert_close(gpu_decode(gpu_lib, w, split=split), oracle_out(w), "bf16")


# rows whose partitions hold fewer chunks than a work-group has wavefronts,
# ragged tails inside a chunk, empty rows
RAGGED_CTX = (0, 1, 15, 16, 17, 33, 63, 64, 65, 100, 130, 255, 256, 257, 700)


@pytest.mark.parametrize("mods", [False, True])
@pytest.mark.parametrize("split", [64, 128, 512, -1])
@pytest.mark.parametrize("copies", [1, 20])
def test_fixed_partitions_as_work_groups_and_as_wavefronts(gpu_lib, copies, split, mods):
    """Fixed partitions run as 4-wavefront work-groups that merge their states
    in LDS when the whole grid fits on the chip at once (15 rows, 2 kv-heads:
    at most 330 partitions) and as one wavefront per partition on a larger grid
    (the same rows 20 times: 600 to 6,600 partitions); both against the oracle,
    with and without score mods."""
    ctx = RAGGED_CTX * copies
    w = small(seed=140 + copies, ctx=ctx, Hq=8, Hkv=2)
    kw, om = {}, {}
    if mods:
        slopes = (2.0 ** -np.arange(1, 9) * 0.5).astype(np.float32)
        kw = {"window": 100, "softcap": 0.5, "alibi_slopes": torch.from_numpy(slopes).cuda()}
        om = {"window": 100, "softcap": 0.5, "alibi_slopes": slopes.astype(np.float64)}
    assert_close(gpu_decode(gpu_lib, w, split=split, **kw), oracle_out(w, oracle.ScoreMods(**om)), "bf16")


def test_non_causal_prefill(gpu_lib):
    wp = small("prefill", ctx=(100, 300), q_lens=[30, 300])
    assert_close(gpu_prefill(gpu_lib, wp, causal=False), oracle_out(wp, causal=False), "bf16")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("g", [1, 2, 8, 16, 32])
def test_prefill_group_sizes_ragged_chunks(gpu_lib, g, D):
    """The matrix-core prefill at every group size it takes beside 4 (a work-group holds 128/g query
    positions x the g heads of one kv-head, and its output rows leave in (position, head) order): chunks
    that end inside a query tile, a single-row chunk, a fresh prompt, causal."""
    Hkv = 2 if g <= 16 else 1
    wp = small("prefill", seed=300 + g + D, ctx=(90, 333, 700), q_lens=[90, 1, 141], Hq=g * Hkv, Hkv=Hkv, D=D,
               causal=True)
    assert_close(gpu_prefill(gpu_lib, wp), oracle_out(wp, causal=True), "bf16")


def test_chunk_rows_equal_full_prefill_rows(gpu_lib):
    full = small("prefill", ctx=(600,), q_lens=[600], causal=True, seed=7)
    chunk = small("prefill", ctx=(600,), q_lens=[200], causal=True, seed=7)
    assert np.array_equal(chunk.k_pool, full.k_pool)
    chunk.q = full.q[400:]
    a = bits_to_f64(gpu_prefill(gpu_lib, full), "bf16")[400:]
    b = bits_to_f64(gpu_prefill(gpu_lib, chunk), "bf16")
    assert np.max(np.abs(a - b)) <= 2e-2


@pytest.mark.parametrize("mods", ["window", "softcap", "alibi", "all"])
def test_score_mods(gpu_lib, mods):
    Hq, Hkv = 16, 4
    slopes = (2.0 ** -np.arange(1, Hq + 1) * 0.5).astype(np.float32)
    kw, om = {}, {}
    if mods in ("window", "all"):
        kw["window"] = om["window"] = 100
    if mods in ("softcap", "all"):
        kw["softcap"] = om["softcap"] = 0.5
    if mods in ("alibi", "all"):
        kw["alibi_slopes"] = torch.from_numpy(slopes).cuda()
        om["alibi_slopes"] = slopes.astype(np.float64)
    w = small(ctx=(90, 700, 1300), Hq=Hq, Hkv=Hkv, append=[1, 1, 1])
    assert_close(gpu_decode(gpu_lib, w, **kw), oracle_out(w, oracle.ScoreMods(**om)), "bf16")
    wp = small("prefill", ctx=(150, 400), q_lens=[150, 170], Hq=Hq, Hkv=Hkv, causal=True)
    assert_close(gpu_prefill(gpu_lib, wp, **kw), oracle_out(wp, oracle.ScoreMods(causal=True, **om)), "bf16")
    wf = small("prefill", dtype="f32", ctx=(150, 400), q_lens=[150, 170], Hq=Hq, Hkv=Hkv, causal=True)
    assert_close(gpu_prefill(gpu_lib, wf, **kw), oracle_out(wf, oracle.ScoreMods(causal=True, **om)), "f32")


@pytest.mark.parametrize("scale", [0.0, -0.08])
@pytest.mark.parametrize("bs", [16, 64])
def test_zero_and_negative_scale(gpu_lib, scale, bs):
    """A scale that is not positive cannot be folded into the bf16 prefill's
    exponent: those calls take its linear score-mod instance (and, with a soft
    cap, the soft-capped one).  Scale 0 gives every admissible key the same
    weight.  Decode in two split modes and both prefill paths, against the
    oracle."""
    w = small(ctx=(90, 700, 1300), Hq=16, Hkv=4, append=[1, 1, 1], bs=bs)
    w.scale = scale
    for split in (0, -1):
        assert_close(gpu_decode(gpu_lib, w, split=split), oracle_out(w), "bf16")
    for dtype in ("bf16", "f32"):
        wp = small("prefill", dtype=dtype, ctx=(150, 400, 333), q_lens=[150, 170, 90], Hq=16, Hkv=4, causal=True,
                   bs=bs)
        wp.scale = scale
        assert_close(gpu_prefill(gpu_lib, wp), oracle_out(wp, causal=True), dtype)
        assert_close(gpu_prefill(gpu_lib, wp, softcap=0.5), oracle_out(wp, oracle.ScoreMods(causal=True, softcap=0.5)),
                     dtype)


def test_pool_beyond_4gib(gpu_lib):
    """Block ids whose byte offsets exceed 32 bits (64-bit addressing)."""
    w = small(ctx=(300, 1000), append=[1, 1])
    base = gpu_decode(gpu_lib, w)
    NB_big = (5 << 30) // (w.Hkv * w.bs * w.D * 2) + 64  # > 5 GiB per pool
    used = np.unique(w.block_table[w.block_table >= 0])
    new_ids = NB_big - 1 - np.arange(len(used))
    remap = np.full(w.NB, -1, np.int64)
    remap[used] = new_ids
    t = upload(w)
    kb = torch.full((NB_big, w.Hkv, w.bs, w.D), float("nan"), dtype=torch.bfloat16, device="cuda")
    vb = torch.full((NB_big,) + tuple(t["v_cache"].shape[1:]), float("nan"), dtype=torch.bfloat16, device="cuda")
    idx_new = torch.from_numpy(new_ids).cuda()
    idx_old = torch.from_numpy(used.astype(np.int64)).cuda()
    kb[idx_new] = t["k_cache"][idx_old]
    vb[idx_new] = t["v_cache"][idx_old]
    t["k_cache"], t["v_cache"] = kb, vb
    table = np.where(w.block_table >= 0, remap[np.maximum(w.block_table, 0)], -1).astype(np.int32)
    t["block_tables"] = to_tensor(table, "i32", "cuda")
    slots = (remap[w.slot_mapping // w.bs] * w.bs + w.slot_mapping % w.bs).astype(np.int32)
    t["slot_mapping"] = to_tensor(slots, "i32", "cuda")
    got = gpu_decode(gpu_lib, w, t=t)
    del kb, vb
    assert np.array_equal(got, base)


def test_poisoned_table_tail_entries_ignored(gpu_lib):
    w = small(ctx=(33, 100), append=[1, 1])
    w.block_table = np.concatenate([w.block_table, np.full((w.B, 8), 2 ** 30, np.int32)], axis=1)
    w.block_table[w.block_table == -1] = 2 ** 30
    assert_close(gpu_decode(gpu_lib, w), oracle_out(w), "bf16")


def test_balanced_split_workspace_reuse_across_batches(gpu_lib):
    """One workspace buffer, sized for the larger batch, serves balanced-split
    decode calls of different batches in turn; every result matches the oracle."""
    import torch

    big = named_workload("long_decode_bf16", batch=6)
    small_w = small(ctx=(37, 300, 1000, 2500), append=[1, 1, 1, 1])
    sizes = [gpu_lib.decode_workspace_size(w.B, w.Hq, w.Hkv, w.D, w.max_context_len, -2) for w in (big, small_w)]
    ws = torch.empty(max(sizes) // 4 + 64, dtype=torch.float32, device="cuda")
    for w in (big, small_w, big, small_w):
        t = upload(w)
        gpu_lib.kv_append(t["k_new"], t["v_new"], t["k_cache"], t["v_cache"], t["slot_mapping"])
        out = torch.empty_like(t["q"])
        gpu_lib.paged_attn_decode(out, t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                                  w.scale, w.max_context_len, -2, workspace=ws)
        torch.cuda.synchronize()
        assert_close(to_numpy_bits(out), oracle_out(w), "bf16")


def _doc_starts(w, rng, docs_per_seq=3):
    """Per query row: the start of its document, for `docs_per_seq` documents
    cut at random points of each sequence (rows at positions n - Lq + i)."""
    out = []
    for b in range(w.B):
        n = int(w.context_lens[b])
        L = int(w.q_lens[b]) if w.kind == "prefill" else 1
        cuts = np.sort(rng.choice(np.arange(1, n), size=min(docs_per_seq - 1, max(n - 1, 0)), replace=False))
        starts = np.concatenate([[0], cuts])
        for pos in range(n - L, n):
            out.append(int(starts[np.searchsorted(starts, pos, side="right") - 1]))
    return np.array(out, dtype=np.int32)


@pytest.mark.parametrize("case", ["prefix", "docs", "prefix_docs_window", "docs_mods"])
def test_prefix_lm_and_document_masks(gpu_lib, case):
    rng = np.random.default_rng(77)
    Hq, Hkv = 16, 4
    wp = small("prefill", ctx=(150, 400, 700), q_lens=[150, 170, 300], Hq=Hq, Hkv=Hkv, causal=True)
    wd = small(ctx=(90, 700, 1300), Hq=Hq, Hkv=Hkv, append=[1, 1, 1])
    for w, is_prefill in ((wp, True), (wd, False)):
        kw, om = {}, {}
        if "prefix" in case:
            pl = np.array([min(int(n), 64 + 97 * i) for i, n in enumerate(w.context_lens)], dtype=np.int32)
            kw["prefix_lens"] = torch.from_numpy(pl).cuda()
            om["prefix_lens"] = pl
        if "docs" in case:
            ds = _doc_starts(w, rng)
            kw["doc_starts"] = torch.from_numpy(ds).cuda()
            om["doc_starts"] = ds
        if "window" in case:
            kw["window"] = om["window"] = 200
        if case == "docs_mods":
            kw["softcap"] = om["softcap"] = 0.5
        if is_prefill:
            ref = oracle_out(w, oracle.ScoreMods(causal=True, **om))
            assert_close(gpu_prefill(gpu_lib, w, **kw), ref, "bf16")
        else:
            ref = oracle_out(w, oracle.ScoreMods(**om))
            for split in (0, -2, 64, -1):
                assert_close(gpu_decode(gpu_lib, w, split=split, **kw), ref, "bf16")
    wf = small("prefill", dtype="f32", ctx=(150, 400), q_lens=[150, 170], Hq=Hq, Hkv=Hkv, causal=True)
    ds = _doc_starts(wf, rng)
    assert_close(gpu_prefill(gpu_lib, wf, doc_starts=torch.from_numpy(ds).cuda()),
                 oracle_out(wf, oracle.ScoreMods(causal=True, doc_starts=ds)), "f32")


# ------------------------------------------------------------------------------------------
# large sizes, checked on sampled rows
# ------------------------------------------------------------------------------------------

def test_decode_of_a_131072_token_row(gpu_lib):
    """One 128K-token row beside short ones (balanced split: the long row is
    cut into many pieces); the oracle checks the long row and a short one."""
    w = build_workload(name="long_row", seed=950, kind="decode", dtype="bf16", Hq=64, Hkv=8, D=128, bs=16,
                       context_lens=[131072, 40, 3000], append_lens=[1, 1, 1], pool_slack=1.1)
    ref = oracle_out(w, seqs=[0, 1])
    for split in (-2, 0):
        assert_close(gpu_decode(gpu_lib, w, split=split), ref, "bf16", rows=[0, 1])


@pytest.mark.parametrize("B,max_q", [(16, 1024), (27, 608)])
def test_prefill_tile_order_at_the_residency_limit(gpu_lib, B, max_q):
    """The bf16 prefill grid has sequences x kv-heads x query tiles work-groups
    (one kv-head here, 4 heads per kv-head, so 32 query rows per tile): 16 x 32
    = 512 fits two per compute unit on a 256-CU chip, and the launcher pairs
    long and short tiles; 27 x 19 = 513 does not, and the order stays longest
    first.  Both must cover every (row, head) once: the output starts as NaN,
    and every row is compared with the oracle.  Chunk lengths are ragged (one
    chunk of max_q rows, the rest random), contexts extend the chunks."""
    rng = np.random.default_rng(7000 + B)
    q = [max_q] + [int(rng.integers(1, max_q + 1)) for _ in range(B - 1)]
    ctx = [n + int(rng.integers(0, 400)) for n in q]
    w = build_workload(name=f"order{B}", seed=7000 + B, kind="prefill", dtype="bf16", Hq=4, Hkv=1, D=64, bs=16,
                       context_lens=ctx, q_lens=q, append_lens=q, causal=True)
    assert w.B * 1 * -(-w.max_q_len // 32) == {16: 512, 27: 513}[B]
    t = upload(w)
    gpu_lib.kv_append(t["k_new"], t["v_new"], t["k_cache"], t["v_cache"], t["slot_mapping"])
    out = torch.full_like(t["q"], float("nan"))
    gpu_lib.paged_attn_prefill(out, t["q"], t["cu_q_lens"], t["k_cache"], t["v_cache"], t["block_tables"],
                               t["context_lens"], w.scale, w.max_q_len, True)
    torch.cuda.synchronize()
    assert_close(to_numpy_bits(out), oracle_out(w, causal=True), "bf16")


@pytest.mark.parametrize("B", [4096, 4097])
def test_batch_size_limit_of_the_balanced_split(gpu_lib, B):
    """4,096 sequences are the most the balanced split takes (its per-row
    chunk prefix lives in LDS); one more and a request for it falls back to
    fixed partitions.  The same limit holds for the persistent walk over
    fixed partitions (its per-row partition prefix lives in LDS too; past it,
    one wavefront per partition).  Both sides of both, with rows just past
    the unsplit cutoff, against the oracle on every row."""
    rng = np.random.default_rng(B)
    w = build_workload(name=f"many{B}", seed=B, kind="decode", dtype="bf16", Hq=8, Hkv=1, D=64, bs=16,
                       context_lens=rng.integers(257, 420, size=B), append_lens=[1] * B, pool_slack=1.1)
    split = gpu_lib.decode_split_tokens(B, 1, int(w.max_context_len), -2)
    assert split == 0 if B <= 4096 else split > 0     # balanced split / fixed partitions
    ref = oracle_out(w)
    for split in (-2, 64):
        assert_close(gpu_decode(gpu_lib, w, split=split), ref, "bf16")


def test_long_prefill_chunks_sampled_rows(gpu_lib):
    """Two 2048-row causal chunks after 6144 and 2048 existing tokens, page 64;
    the oracle (the definition over the gathered keys) checks 96 sampled rows."""
    w = build_workload(name="long_prefill", seed=951, kind="prefill", dtype="bf16", Hq=32, Hkv=8, D=128,
                       bs=64, context_lens=[8192, 4096], q_lens=[2048, 2048], append_lens=[2048, 2048],
                       causal=True, pool_slack=1.1)
    got = bits_to_f64(gpu_prefill(gpu_lib, w), "bf16")
    kp, vp = appended_pools(w)
    rng = np.random.default_rng(951)
    for b in range(w.B):
        n = int(w.context_lens[b])
        r0, r1 = int(w.cu_q_lens[b]), int(w.cu_q_lens[b + 1])
        rows = np.sort(rng.choice(np.arange(r0, r1), size=48, replace=False))
        rows[0], rows[-1] = r0, r1 - 1                       # first and last row of the chunk
        K, V = oracle.gather_sequence(kp, vp, w.block_table[b], n, w.bs)
        K, V = bits_to_f64(K, "bf16"), bits_to_f64(V, "bf16")
        Q = bits_to_f64(w.q[rows], "bf16")
        pos = n - (r1 - r0) + (rows - r0)
        ref = oracle.attention_dense(Q, K, V, float(w.scale), pos, oracle.ScoreMods(causal=True))
        err = np.max(np.abs(got[rows] - ref))
        assert np.all(np.isfinite(got[rows])) and err <= TOL["bf16"], (b, err)

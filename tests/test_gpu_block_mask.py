"""GPU parity of FlexAttention-style block masks against the fp64 oracle.

A block mask admits, per sequence and query block (logical positions), a set
of key blocks; the other masks still apply inside them.  The bf16 prefill
visits only the 64-key tiles some row of a work-group admits (its list of
tiles is built in LDS, 2,048 tiles at a time), the decode and the fp32 path
skip the 16-token chunks a row does not admit.  Pools are poisoned with NaN in
blocks no visited tile touches, so any read of a skipped block shows.
Tolerances as for the other parity tests.
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import build_workload
from workloads.device import upload

from tests.test_gpu_parity import TOL, appended_pools, assert_close, gpu_decode, gpu_prefill
from tests.test_oracle import pack_block_mask

pytestmark = pytest.mark.gpu


def device_mask(lib, bm):
    """oracle.BlockMask -> the binding's block mask (int32 tensor [B, rows, words])."""
    rows = bm.rows_per_seq
    bits = np.ascontiguousarray(bm.bits.view(np.int32)).reshape(-1, rows, bm.bits.shape[1])
    return lib.block_mask(torch.from_numpy(bits).cuda(), bm.q_block, bm.kv_block)


def oracle_with(w, **mods):
    kp, vp = appended_pools(w)
    return oracle.paged_attention(w.q, kp, vp, w.block_table, w.context_lens, w.cu_q_lens, w.scale, w.bs, w.dtype,
                                  oracle.ScoreMods(**mods))


def random_dense(rng, w, q_block, kv_block, density, per_row=True):
    n_max = int(w.context_lens.max())
    qbn = (n_max + q_block - 1) // q_block
    kbn = (n_max + kv_block - 1) // kv_block
    if per_row:
        return rng.random((w.B, qbn, kbn)) < density
    seq = rng.random((w.B, 1, kbn)) < density
    return np.broadcast_to(seq, (w.B, qbn, kbn)).copy()


def poison_unadmitted(w, dense, kv_block):
    """NaN into every pool block of a sequence whose keys lie only in key
    blocks no query block of that sequence admits (after the append)."""
    kp, vp = appended_pools(w)
    any_row = dense.any(axis=1)  # [B, kbn]
    for b in range(w.B):
        n = int(w.context_lens[b])
        for j in range((n + w.bs - 1) // w.bs):
            keys = np.arange(j * w.bs, min(n, (j + 1) * w.bs))
            if not any_row[b][keys // kv_block].any():
                blk = int(w.block_table[b, j])
                kp[blk] = np.uint16(0x7FC0) if w.dtype == "bf16" else np.float32("nan")
                vp[blk] = np.uint16(0x7FC0) if w.dtype == "bf16" else np.float32("nan")
    w.k_pool, w.v_pool = kp, vp
    w.k_new = w.k_new[:0]
    w.v_new = w.v_new[:0]
    w.slot_mapping = w.slot_mapping[:0]


PREFILL_CASES = {
    # q_block, kv_block, causal, density, per-row masks, extra mods
    "q16_kv64_causal": (16, 64, True, 0.5, True, {}),
    "q1_kv128_causal": (1, 128, True, 0.6, True, {}),
    "q128_kv256_full": (128, 256, False, 0.5, True, {}),
    "q64_kv64_window_alibi": (64, 64, True, 0.7, True, {"window": 700}),
    "q32_kv64_softcap_docs": (32, 64, True, 0.6, True, {"softcap": 20.0}),
}


@pytest.mark.parametrize("case", sorted(PREFILL_CASES))
def test_prefill_block_mask(gpu_lib, case):
    q_block, kv_block, causal, density, per_row, extra = PREFILL_CASES[case]
    rng = np.random.default_rng(abs(hash(case)) % 2**32)
    w = build_workload(name="bm", seed=810 + len(case), kind="prefill", dtype="bf16", Hq=32, Hkv=8, D=128, bs=16,
                       context_lens=[1000, 1300, 400], q_lens=[300, 1300, 77], append_lens=[300, 1300, 77],
                       causal=causal)
    bm = pack_block_mask(random_dense(rng, w, q_block, kv_block, density, per_row), q_block, kv_block)
    kw, om = {}, {}
    if "window" in extra:
        kw["window"] = om["window"] = extra["window"]
        slopes = (2.0 ** -np.arange(1, 33)).astype(np.float32)
        kw["alibi_slopes"] = torch.from_numpy(slopes).cuda()
        om["alibi_slopes"] = slopes
    if "softcap" in extra:
        kw["softcap"] = om["softcap"] = extra["softcap"]
        docs = np.concatenate([np.full(int(q), max(0, int(n) - int(q) - 200 * k)) for k, (q, n) in
                               enumerate(zip(w.q_lens, w.context_lens))]).astype(np.int32)
        kw["doc_starts"] = torch.from_numpy(docs).cuda()
        om["doc_starts"] = docs
    ref = oracle_with(w, causal=causal, block_mask=bm, **om)
    got = gpu_prefill(gpu_lib, w, causal=causal, block_mask=device_mask(gpu_lib, bm), **kw)
    assert_close(got, ref, "bf16")


@pytest.mark.parametrize("kind,dtype", [("prefill", "bf16"), ("prefill", "f32"), ("decode", "bf16"),
                                        ("decode", "f32")])
def test_unadmitted_blocks_are_never_read(gpu_lib, kind, dtype):
    """Masks equal over a sequence's query blocks, NaN in every pool block
    that only unadmitted key blocks cover: the output must stay finite and
    match the oracle (which never reads them either)."""
    rng = np.random.default_rng(901)
    ctx = [900, 1500, 130, 2100]
    w = build_workload(name="bmp", seed=902, kind=kind, dtype=dtype, Hq=16, Hkv=4, D=128 if dtype == "bf16" else 64,
                       bs=16, context_lens=ctx, q_lens=[64, 200, 130, 33] if kind == "prefill" else None,
                       append_lens=None, causal=kind == "prefill")
    dense = random_dense(rng, w, 64, 64, 0.4, per_row=False)
    dense[2] = False  # one sequence admits nothing: zero rows
    poison_unadmitted(w, dense, 64)
    bm = pack_block_mask(dense, 64, 64)
    ref = oracle_with(w, causal=kind == "prefill", block_mask=bm)
    dm = device_mask(gpu_lib, bm)
    if kind == "prefill":
        got = gpu_prefill(gpu_lib, w, causal=True, block_mask=dm)
        assert_close(got, ref, dtype)
    else:
        for split in (0, -2, 64, -1):
            assert_close(gpu_decode(gpu_lib, w, split=split, block_mask=dm), ref, dtype)


@pytest.mark.parametrize("split", [0, -2, 64, -1])
def test_decode_block_mask_per_sequence(gpu_lib, split):
    rng = np.random.default_rng(903)
    w = build_workload(name="bmd", seed=903, kind="decode", dtype="bf16", Hq=64, Hkv=8, D=128, bs=32,
                       context_lens=rng.integers(100, 5000, size=12), append_lens=[1] * 12)
    q_block = 1 << 20  # one bitmap row per sequence
    bm = pack_block_mask(random_dense(rng, w, q_block, 128, 0.5), q_block, 128)
    ref = oracle_with(w, block_mask=bm)
    assert_close(gpu_decode(gpu_lib, w, split=split, block_mask=device_mask(gpu_lib, bm)), ref, "bf16")


@pytest.mark.parametrize("split", [64, -2])
def test_decode_merge_with_leading_empty_partials(gpu_lib, split):
    """A 3,000-key row whose mask admits only its last 7 key blocks of 64: at
    64-key partitions the first 32 partial states (the merge's first batch)
    are all empty and the rest hold every key; a second row admits every
    block."""
    w = build_workload(name="bme", seed=907, kind="decode", dtype="bf16", Hq=16, Hkv=2, D=128, bs=16,
                       context_lens=[3000, 900], append_lens=[1, 1])
    kbn = (3000 + 63) // 64
    dense = np.zeros((2, 1, kbn), dtype=bool)
    dense[0, 0, kbn - 7:] = True
    dense[1, 0, :] = True
    bm = pack_block_mask(dense, 1 << 20, 64)
    ref = oracle_with(w, block_mask=bm)
    assert_close(gpu_decode(gpu_lib, w, split=split, block_mask=device_mask(gpu_lib, bm)), ref, "bf16")


def test_block_mask_all_ones_equals_no_mask(gpu_lib):
    w = build_workload(name="bm1", seed=904, kind="prefill", dtype="bf16", Hq=32, Hkv=8, D=128, bs=16,
                       context_lens=[700, 333], q_lens=[200, 333], append_lens=[200, 333], causal=True)
    ones = np.ones((w.B, 700, 12), dtype=bool)
    bm = pack_block_mask(ones, 1, 64)
    ref = oracle_with(w, causal=True)
    assert_close(gpu_prefill(gpu_lib, w, causal=True, block_mask=device_mask(gpu_lib, bm)), ref, "bf16")


def test_prefill_block_mask_over_several_tile_lists(gpu_lib):
    """A 140,000-key sequence (2,188 tiles of 64 keys): the work-group builds
    its list of admitted tiles in two segments."""
    rng = np.random.default_rng(905)
    w = build_workload(name="bml", seed=905, kind="prefill", dtype="bf16", Hq=8, Hkv=2, D=128, bs=64,
                       context_lens=[140000], q_lens=[64], append_lens=[64], causal=True, pool_slack=1.02)
    dense = random_dense(rng, w, 64, 64, 0.3)
    dense[0, :, -1] = True  # the last block (the rows' own keys)
    bm = pack_block_mask(dense, 64, 64)
    ref = oracle_with(w, causal=True, block_mask=bm)
    assert_close(gpu_prefill(gpu_lib, w, causal=True, block_mask=device_mask(gpu_lib, bm)), ref, "bf16")


def test_cascade_with_block_mask(gpu_lib):
    """The shared-prefix call takes a block mask through the plain decode;
    the forced two-phase call refuses it."""
    from tests.test_gpu_cascade import device_level, grouped
    w, starts, prefix = grouped(906, [(4, 8)], [40, 1, 300, 17], [0])
    t = upload(w)
    gpu_lib.kv_append(t["k_new"], t["v_new"], t["k_cache"], t["v_cache"], t["slot_mapping"])
    rng = np.random.default_rng(906)
    bm = pack_block_mask(random_dense(rng, w, 1 << 20, 64, 0.6), 1 << 20, 64)
    levels = [device_level(gpu_lib, starts, prefix)]
    out = torch.empty_like(t["q"])
    gpu_lib.paged_attn_decode_cascade(out, t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                                      levels, w.scale, w.max_context_len, block_mask=device_mask(gpu_lib, bm))
    torch.cuda.synchronize()
    from workloads.device import to_numpy_bits
    assert_close(to_numpy_bits(out), oracle_with(w, block_mask=bm), "bf16")
    with pytest.raises(ValueError):
        gpu_lib.paged_attn_decode_cascade(out, t["q"], t["k_cache"], t["v_cache"], t["block_tables"],
                                          t["context_lens"], levels, w.scale, w.max_context_len,
                                          block_mask=device_mask(gpu_lib, bm), mode="two_phase")

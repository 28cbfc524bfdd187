"""Randomized parity sweep through the C ABI.

Each seeded case draws a batch size, kv-head count, group size (including a
3 that does not divide the tile), head dim, page size, dtype, per-sequence
context lengths (1, block boundaries and their neighbours, random), query
chunks (single rows, partial chunks, whole fresh prompts) and a random
subset of score mods (a block mask among them).  It checks kv_append bit for
bit over the whole pool, then decode in four split modes or prefill (causal
or not; also through the key-split entry) against the fp64 oracle, with the
tolerances of the other parity tests (2e-2 max-abs for bf16, 1e-4 for fp32).
Sizes stay small enough for the oracle to finish in about a second per case.
"""

import os

import numpy as np
import pytest
import torch

import oracle
from tests.test_gpu_parity import TOL, _doc_starts, appended_pools, assert_close, gpu_decode, gpu_prefill
from workloads import build_workload
from workloads.device import to_numpy_bits, upload

pytestmark = pytest.mark.gpu


def _lengths(rng, n, bs, cap):
    special = [1, bs - 1, bs, bs + 1, 2 * bs, 3 * bs - 1]
    out = []
    for _ in range(n):
        out.append(int(rng.choice(special)) if rng.random() < 0.4 else int(rng.integers(1, cap + 1)))
    return out


def draw(seed):
    rng = np.random.default_rng(seed)
    c = {}
    c["dtype"] = str(rng.choice(["bf16", "f32"], p=[0.75, 0.25]))
    c["D"] = int(rng.choice([64, 128]))
    c["Hkv"] = int(rng.choice([1, 2, 4, 8]))
    c["g"] = int(rng.choice([1, 2, 3, 4, 8, 16]))
    c["bs"] = int(rng.choice([16, 32, 64, 128, 256]))
    c["B"] = int(rng.integers(1, 6))
    c["kind"] = str(rng.choice(["decode", "prefill"]))
    if c["kind"] == "decode":
        c["ctx"] = _lengths(rng, c["B"], c["bs"], 1500)
        c["q"] = None
        c["append"] = [1] * c["B"]
        c["causal"] = False
    else:
        if c["g"] > 4:
            c["g"] = 4  # keep the fp64 oracle quick
        ctx = _lengths(rng, c["B"], c["bs"], 700)
        q = []
        for n in ctx:
            r = rng.random()
            q.append(n if r < 0.3 else (1 if r < 0.45 else int(rng.integers(1, min(n, 200) + 1))))
        c["ctx"], c["q"], c["append"] = ctx, q, list(q)
        c["causal"] = bool(rng.random() < 0.8)
    mods = {}
    if rng.random() < 0.3:
        mods["window"] = int(rng.integers(1, 400))
    if rng.random() < 0.25:
        mods["softcap"] = float(rng.choice([0.5, 5.0, 30.0]))
    if rng.random() < 0.25:
        mods["alibi"] = True
    if rng.random() < 0.2:
        mods["docs"] = True
    if c["kind"] == "prefill" and c["causal"] and rng.random() < 0.2:
        mods["prefix"] = True
    if rng.random() < 0.25:
        mods["blockmask"] = (int(rng.choice([1, 16, 64, 1 << 20])), int(rng.choice([64, 128, 256])),
                             float(rng.uniform(0.4, 0.95)))
    c["mods"] = mods
    return c


def _seeds(var, default):
    """Seed range from the environment ("first:last+1", e.g. PA_SWEEP_SEEDS=5000:6000)
    for longer runs of the same generators; the default otherwise."""
    spec = os.environ.get(var)
    if not spec:
        return default
    a, b = (int(x) for x in spec.split(":"))
    return list(range(a, b))


SEEDS = _seeds("PA_SWEEP_SEEDS", list(range(1000, 1096)))


@pytest.mark.parametrize("seed", SEEDS)
def test_random_case(gpu_lib, seed):
    c = draw(seed)
    print(f"case {seed}: {c}", flush=True)
    Hq = c["Hkv"] * c["g"]
    w = build_workload(name=f"sweep{seed}", seed=seed, kind=c["kind"], dtype=c["dtype"], Hq=Hq, Hkv=c["Hkv"],
                       D=c["D"], bs=c["bs"], context_lens=c["ctx"], q_lens=c["q"], append_lens=c["append"],
                       causal=c["causal"])
    # kv_append: bit-exact over the whole pool
    t = upload(w)
    gpu_lib.kv_append(t["k_new"], t["v_new"], t["k_cache"], t["v_cache"], t["slot_mapping"])
    torch.cuda.synchronize()
    kp, vp = appended_pools(w)
    assert np.array_equal(to_numpy_bits(t["k_cache"]).view(np.uint8), np.ascontiguousarray(kp).view(np.uint8))
    assert np.array_equal(to_numpy_bits(t["v_cache"]).view(np.uint8), np.ascontiguousarray(vp).view(np.uint8))

    rng = np.random.default_rng(seed + 1)
    kw, om = {}, {}
    m = c["mods"]
    if "window" in m:
        kw["window"] = om["window"] = m["window"]
    if "softcap" in m:
        kw["softcap"] = om["softcap"] = m["softcap"]
    if "alibi" in m:
        slopes = (2.0 ** -np.arange(1, Hq + 1) * 0.5).astype(np.float32)
        kw["alibi_slopes"] = torch.from_numpy(slopes).cuda()
        om["alibi_slopes"] = slopes.astype(np.float64)
    if "blockmask" in m:
        from tests.test_gpu_block_mask import device_mask, random_dense
        from tests.test_oracle import pack_block_mask
        qb, kvb, density = m["blockmask"]
        bm = pack_block_mask(random_dense(np.random.default_rng(seed + 2), w, qb, kvb, density), qb, kvb)
        kw["block_mask"] = device_mask(gpu_lib, bm)
        om["block_mask"] = bm
    if "docs" in m:
        ds = _doc_starts(w, rng)
        kw["doc_starts"] = torch.from_numpy(ds).cuda()
        om["doc_starts"] = ds
    if "prefix" in m:
        pl = np.array([int(rng.integers(0, n + 1)) for n in w.context_lens], dtype=np.int32)
        kw["prefix_lens"] = torch.from_numpy(pl).cuda()
        om["prefix_lens"] = pl
    ref = oracle.paged_attention(w.q, kp, vp, w.block_table, w.context_lens, w.cu_q_lens, w.scale, w.bs, w.dtype,
                                 oracle.ScoreMods(causal=c["causal"], **om))
    if c["kind"] == "decode":
        errs = [assert_close(gpu_decode(gpu_lib, w, t=t, split=split, **kw), ref, w.dtype, tol=TOL[w.dtype])
                for split in (0, -2, -1, 64)]
    else:
        errs = [assert_close(gpu_prefill(gpu_lib, w, t=t, causal=c["causal"], **kw), ref, w.dtype, tol=TOL[w.dtype])]
        # the same rows through the key-split entry: ranges of 64 or 128 keys,
        # or the library's choice under a context bound 4x the longest context
        ks = int(np.random.default_rng(seed + 3).choice([64, 128, 0]))
        max_ctx = int(w.context_lens.max()) * (4 if ks == 0 else 1)
        out = torch.empty_like(t["q"])
        gpu_lib.paged_attn_prefill(out, t["q"], t["cu_q_lens"], t["k_cache"], t["v_cache"], t["block_tables"],
                                   t["context_lens"], w.scale, w.max_q_len, c["causal"], max_context_len=max_ctx,
                                   key_split=ks, **kw)
        torch.cuda.synchronize()
        errs.append(assert_close(to_numpy_bits(out), ref, w.dtype, tol=TOL[w.dtype]))
    print(f"case {seed}: max abs err {max(errs):.3e} (tolerance {TOL[w.dtype]})", flush=True)


FORK_SEEDS = _seeds("PA_FORK_SEEDS", list(range(2000, 2016)))


@pytest.mark.parametrize("seed", FORK_SEEDS)
def test_random_fork_tree_two_phase(gpu_lib, seed):
    """Random fork trees kept by the block manager with random page rules
    (pages of one size or doubling, up to 16 blocks), random appends with the
    copy-on-write they cause, and a random subset of score mods: the
    manager's prefix levels drive the two-phase decode, which must match the
    oracle, as the plain decode must."""
    from tests.test_block_manager import copy_blocks_reference
    from workloads import bf16_round_bits

    rng = np.random.default_rng(seed)
    Hkv = int(rng.choice([2, 4, 8]))
    g = int(rng.choice([1, 4, 8]))
    D = int(rng.choice([64, 128]))
    Hq, BS_, nb = Hkv * g, 16, 1280
    bm = gpu_lib.BlockManager(nb, BS_, 16)
    kp = np.full((nb, Hkv, BS_, D), 0x7FC0, np.uint16)
    vp = np.full((nb, Hkv, 1, D, 16), 0x7FC0, np.uint16)
    gk = torch.from_numpy(kp.view(np.int16)).cuda().view(torch.bfloat16)
    gv = torch.from_numpy(vp.view(np.int16)).cuda().view(torch.bfloat16)
    to_dev = lambda x: torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)  # noqa: E731
    rules = [(1, 1), (4, 4), (16, 16), (1, 16), (2, 8)]

    def append(s, n):
        nonlocal kp, vp
        slots, copies = bm.append(s, n)
        copy_blocks_reference(kp, vp, copies)
        if copies:
            gpu_lib.kv_copy_blocks(gk, gv, torch.tensor([c[0] for c in copies], dtype=torch.int32, device="cuda"),
                                   torch.tensor([c[1] for c in copies], dtype=torch.int32, device="cuda"))
        kn = bf16_round_bits(rng.standard_normal((n, Hkv, D)).astype(np.float32))
        vn = bf16_round_bits(rng.standard_normal((n, Hkv, D)).astype(np.float32))
        kp, vp = oracle.kv_append(kp, vp, kn, vn, np.array(slots, np.int32), BS_)
        gpu_lib.kv_append(to_dev(kn), to_dev(vn), gk, gv, torch.tensor(slots, dtype=torch.int32, device="cuda"))

    # a forest: roots with random rules, children forked at random depths; the
    # batch lists each tree depth-first, so forks sit next to their relatives
    order = []
    for _ in range(int(rng.integers(1, 4))):
        root = bm.new_sequence(*rules[rng.integers(len(rules))])
        append(root, int(rng.integers(1, 900)))
        tree = [root]
        for _ in range(int(rng.integers(0, 7))):
            parent = tree[rng.integers(len(tree))]
            child = bm.fork(parent)
            tree.insert(tree.index(parent) + 1, child)
            append(child, int(rng.integers(0, 300)) or 1)
        order += tree
    for s in order:
        append(s, 1)                                 # this step's token
    rows = [bm.table(s) for s in order]
    W = max(len(t) for t, _ in rows)
    table = np.zeros((len(order), W), np.int32)
    for i, (t, _) in enumerate(rows):
        table[i, :len(t)] = t
    lens = np.array([n for _, n in rows], np.int32)
    scale = np.float32(1 / np.sqrt(D))
    kw, om = {}, {}
    if rng.random() < 0.3:
        kw["window"] = om["window"] = int(rng.integers(16, 600))
    if rng.random() < 0.3:
        kw["softcap"] = om["softcap"] = float(rng.choice([1.0, 10.0]))
    if rng.random() < 0.3:
        slopes = (2.0 ** -np.arange(1, Hq + 1) * 0.25).astype(np.float32)
        kw["alibi_slopes"] = torch.from_numpy(slopes).cuda()
        om["alibi_slopes"] = slopes.astype(np.float64)
    print(f"fork case {seed}: Hkv {Hkv} g {g} D {D} lens {lens.tolist()} mods {sorted(om)}", flush=True)
    q = bf16_round_bits(rng.standard_normal((len(order), Hq, D)).astype(np.float32))
    ref = oracle.paged_attention(q, kp, vp, table, lens, np.arange(len(order) + 1), scale, BS_, "bf16",
                                 oracle.ScoreMods(**om))
    qd, tt, tl = to_dev(q), torch.from_numpy(table).cuda(), torch.from_numpy(lens).cuda()
    out = torch.empty_like(qd)
    gpu_lib.paged_attn_decode(out, qd, gk, gv, tt, tl, float(scale), int(lens.max()), 0, **kw)
    torch.cuda.synchronize()
    assert_close(to_numpy_bits(out), ref, "bf16")
    levels_host = bm.prefix_levels(order)
    if not levels_host:
        return  # nothing shared (e.g. one sequence): the plain decode is the call
    levels = [gpu_lib.prefix_level(torch.from_numpy(st).cuda(), torch.from_numpy(hi).cuda(),
                                   int(np.max(np.diff(st))), int(max(1, np.max(hi - lo))), torch.from_numpy(lo).cuda())
              for st, lo, hi in levels_host]
    out = torch.empty_like(qd)
    gpu_lib.paged_attn_decode_cascade(out, qd, gk, gv, tt, tl, levels, float(scale), int(lens.max()),
                                      mode="two_phase", **kw)
    torch.cuda.synchronize()
    err = assert_close(to_numpy_bits(out), ref, "bf16")
    print(f"fork case {seed}: {len(levels_host)} levels, two-phase max abs err {err:.3e}", flush=True)

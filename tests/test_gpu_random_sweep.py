"""Randomized parity sweep through the C ABI.

Each seeded case draws a batch size, kv-head count, group size (including a
3 that does not divide the tile), head dim, page size, dtype, per-sequence
context lengths (1, block boundaries and their neighbours, random), query
chunks (single rows, partial chunks, whole fresh prompts) and a random
subset of score mods.  It checks kv_append bit for bit over the whole pool,
then decode in three split modes or prefill (causal or not) against the
fp64 oracle, with the tolerances of the other parity tests (2e-2 max-abs for
bf16, 1e-4 for fp32).  Sizes stay small enough for the oracle to finish in
about a second per case.
"""

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
    c["mods"] = mods
    return c


SEEDS = list(range(1000, 1096))


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
                for split in (0, -1, 64)]
    else:
        errs = [assert_close(gpu_prefill(gpu_lib, w, t=t, causal=c["causal"], **kw), ref, w.dtype, tol=TOL[w.dtype])]
    print(f"case {seed}: max abs err {max(errs):.3e} (tolerance {TOL[w.dtype]})", flush=True)

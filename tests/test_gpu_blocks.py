"""kv_copy_blocks on the GPU (bit-exact against a plain slab copy), and the
host block manager driving real pools: fork, copy-on-write and appends on the
GPU read back exactly, and decode over the resulting tables matches the oracle."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from tests.test_block_manager import Replay, copy_blocks_reference  # noqa: E402
from workloads import bf16_round_bits  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,D,bs", [("bf16", 128, 16), ("f32", 64, 32), ("bf16", 64, 256)])
def test_copy_blocks_bit_exact(gpu_lib, dtype, D, bs):
    rng = np.random.default_rng(5)
    NB, Hkv = 40, 4
    if dtype == "bf16":
        k = bf16_round_bits(rng.standard_normal((NB, Hkv, bs, D)).astype(np.float32))
        v = bf16_round_bits(rng.standard_normal((NB, Hkv, bs // 16, D, 16)).astype(np.float32))
        tk, tv = (torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda() for x in (k, v))
    else:
        k = rng.standard_normal((NB, Hkv, bs, D)).astype(np.float32)
        v = rng.standard_normal((NB, Hkv, bs // 16, D, 16)).astype(np.float32)
        tk, tv = torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda()
    pairs = [(3, 17), (0, 39), (25, 2), (11, 8)]
    src = torch.tensor([p[0] for p in pairs], dtype=torch.int32, device="cuda")
    dst = torch.tensor([p[1] for p in pairs], dtype=torch.int32, device="cuda")
    gpu_lib.kv_copy_blocks(tk, tv, src, dst)
    torch.cuda.synchronize()
    copy_blocks_reference(k, v, pairs)
    gk = tk.view(torch.int16).cpu().numpy() if dtype == "bf16" else tk.cpu().numpy()
    gv = tv.view(torch.int16).cpu().numpy() if dtype == "bf16" else tv.cpu().numpy()
    assert np.array_equal(gk.view(np.uint8), k.view(np.uint8))
    assert np.array_equal(gv.view(np.uint8), v.view(np.uint8))


def test_manager_driven_pools_and_decode(gpu_lib):
    """Replay a fork / copy-on-write workload on GPU pools (fp32, bs 16, D 8 is
    not a kernel shape, so this uses D 64) and compare with the numpy replay."""
    import tests.test_block_manager as tbm

    old = (tbm.HKV, tbm.D)
    tbm.HKV, tbm.D = 2, 64
    try:
        r = Replay(9, nb=64)
        gk = torch.full(r.k.shape, float("nan"), dtype=torch.float32, device="cuda")
        gv = torch.full(r.v.shape, float("nan"), dtype=torch.float32, device="cuda")

        def gpu_append(s, n):
            hk0 = len(r.hist[s][0])
            slots, copies = r.append(s, n)  # numpy replay (draws the new rows)
            if copies:
                src = torch.tensor([c[0] for c in copies], dtype=torch.int32, device="cuda")
                dst = torch.tensor([c[1] for c in copies], dtype=torch.int32, device="cuda")
                gpu_lib.kv_copy_blocks(gk, gv, src, dst)
            kn = torch.from_numpy(np.ascontiguousarray(r.hist[s][0][hk0:])).cuda()
            vn = torch.from_numpy(np.ascontiguousarray(r.hist[s][1][hk0:])).cuda()
            gpu_lib.kv_append(kn, vn, gk, gv, torch.tensor(slots, dtype=torch.int32, device="cuda"))

        a = r.new()
        gpu_append(a, 37)
        b = r.fork(a)
        gpu_append(b, 5)
        c = r.fork(a)
        gpu_append(a, 20)
        gpu_append(c, 16)
        r.free(b)
        d = r.fork(c)
        gpu_append(d, 2)
        torch.cuda.synchronize()
        r.check()
        assert np.array_equal(gk.cpu().numpy(), r.k, equal_nan=True)
        assert np.array_equal(gv.cpu().numpy(), r.v, equal_nan=True)

        # decode over the live sequences' tables
        seqs = sorted(r.hist)
        rows = [r.bm.table(s) for s in seqs]
        W = max(len(t) for t, _ in rows)
        table = np.zeros((len(seqs), W), np.int32)
        for i, (t, _) in enumerate(rows):
            table[i, :len(t)] = t
        lens = np.array([n for _, n in rows], np.int32)
        Hq = 4
        q = np.random.default_rng(2).standard_normal((len(seqs), Hq, 64)).astype(np.float32)
        out = torch.empty((len(seqs), Hq, 64), dtype=torch.float32, device="cuda")
        scale = np.float32(0.125)
        gpu_lib.paged_attn_decode(out, torch.from_numpy(q).cuda(), gk, gv, torch.from_numpy(table).cuda(),
                                  torch.from_numpy(lens).cuda(), float(scale), int(lens.max()), 0)
        torch.cuda.synchronize()
        ref = oracle.paged_attention(q, r.k, r.v, table, lens, np.arange(len(seqs) + 1), scale, 16, "f32")
        assert np.max(np.abs(out.cpu().numpy() - ref)) <= 1e-4
    finally:
        tbm.HKV, tbm.D = old


def test_manager_prefix_levels_drive_the_two_phase_decode(gpu_lib):
    """A fork tree of bf16 sequences (prompt, beams, sub-beams) kept by the
    manager on GPU pools; the manager's prefix levels of the batch drive the
    two-phase decode, which must match the oracle over the same tables."""
    HKV_, D_, HQ_, BS_ = 8, 128, 32, 16
    rng = np.random.default_rng(77)
    nb = 600
    bm = gpu_lib.BlockManager(nb, BS_)
    kp = np.full((nb, HKV_, BS_, D_), 0x7FC0, np.uint16)
    vp = np.full((nb, HKV_, BS_ // 16, D_, 16), 0x7FC0, np.uint16)
    gk = torch.from_numpy(kp.view(np.int16)).cuda().view(torch.bfloat16)
    gv = torch.from_numpy(vp.view(np.int16)).cuda().view(torch.bfloat16)

    def append(s, n):
        nonlocal kp, vp
        slots, copies = bm.append(s, n)
        copy_blocks_reference(kp, vp, copies)
        if copies:
            src = torch.tensor([c[0] for c in copies], dtype=torch.int32, device="cuda")
            dst = torch.tensor([c[1] for c in copies], dtype=torch.int32, device="cuda")
            gpu_lib.kv_copy_blocks(gk, gv, src, dst)
        kn = bf16_round_bits(rng.standard_normal((n, HKV_, D_)).astype(np.float32))
        vn = bf16_round_bits(rng.standard_normal((n, HKV_, D_)).astype(np.float32))
        kp, vp = oracle.kv_append(kp, vp, kn, vn, np.array(slots, np.int32), BS_)
        to_dev = lambda x: torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)  # noqa: E731
        gpu_lib.kv_append(to_dev(kn), to_dev(vn), gk, gv, torch.tensor(slots, dtype=torch.int32, device="cuda"))

    prompt = bm.new_sequence()
    append(prompt, 300)                          # shared system prompt (18 full blocks + 12)
    order = {prompt: (0,)}
    beams = [prompt]
    for i in range(3):
        c = bm.fork(prompt)
        order[c] = (0, i + 1)
        beams.append(c)
    for s in beams:
        append(s, int(rng.integers(40, 200)))    # each conversation's own history
    for s in list(beams[1:3]):
        for j in range(2):
            c = bm.fork(s)
            order[c] = order[s] + (j + 1,)
            beams.append(c)
    for s in beams:
        append(s, int(rng.integers(1, 30)))      # the newest tokens (decode step included)
    other = bm.new_sequence()
    append(other, 77)
    order[other] = (9,)
    beams.append(other)
    seqs = sorted(beams, key=lambda s: order[s])
    levels_host = bm.prefix_levels(seqs)
    assert len(levels_host) >= 2
    rows = [bm.table(s) for s in seqs]
    W = max(len(t) for t, _ in rows)
    table = np.zeros((len(seqs), W), np.int32)
    for i, (t, _) in enumerate(rows):
        table[i, :len(t)] = t
    lens = np.array([n for _, n in rows], np.int32)
    q = bf16_round_bits(rng.standard_normal((len(seqs), HQ_, D_)).astype(np.float32))
    scale = np.float32(1 / np.sqrt(D_))
    levels = [gpu_lib.prefix_level(torch.from_numpy(st).cuda(), torch.from_numpy(hi).cuda(),
                                   int(np.max(np.diff(st))), int(np.max(hi - lo)), torch.from_numpy(lo).cuda())
              for st, lo, hi in levels_host]
    qd = torch.from_numpy(q.view(np.int16)).cuda().view(torch.bfloat16)
    out = torch.empty_like(qd)
    gpu_lib.paged_attn_decode_cascade(out, qd, gk, gv, torch.from_numpy(table).cuda(), torch.from_numpy(lens).cuda(),
                                      levels, float(scale), int(lens.max()), mode="two_phase")
    torch.cuda.synchronize()
    ref = oracle.paged_attention(q, kp, vp, table, lens, np.arange(len(seqs) + 1), scale, BS_, "bf16")
    got = oracle.bits_to_f64(out.view(torch.int16).cpu().numpy().view(np.uint16), "bf16")
    assert np.max(np.abs(got - ref)) <= 2e-2


def test_mixed_page_sizes_in_one_pool_drive_decode_prefill_and_two_phase(gpu_lib):
    """One bf16 pool kept by the manager with pages of 1-16 blocks: fixed
    page sizes, pages doubling along a sequence, forks whose copy-on-write
    moves multi-block pages.  Decode, chunked prefill and the two-phase
    decode read the tables (block resolution) and must match the oracle."""
    HKV_, D_, HQ_, BS_ = 8, 128, 32, 16
    rng = np.random.default_rng(91)
    nb = 1024
    bm = gpu_lib.BlockManager(nb, BS_, 16)
    kp = np.full((nb, HKV_, BS_, D_), 0x7FC0, np.uint16)
    vp = np.full((nb, HKV_, BS_ // 16, D_, 16), 0x7FC0, np.uint16)
    gk = torch.from_numpy(kp.view(np.int16)).cuda().view(torch.bfloat16)
    gv = torch.from_numpy(vp.view(np.int16)).cuda().view(torch.bfloat16)
    to_dev = lambda x: torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)  # noqa: E731

    def append(s, n):
        nonlocal kp, vp
        slots, copies = bm.append(s, n)
        copy_blocks_reference(kp, vp, copies)
        if copies:
            src = torch.tensor([c[0] for c in copies], dtype=torch.int32, device="cuda")
            dst = torch.tensor([c[1] for c in copies], dtype=torch.int32, device="cuda")
            gpu_lib.kv_copy_blocks(gk, gv, src, dst)
        kn = bf16_round_bits(rng.standard_normal((n, HKV_, D_)).astype(np.float32))
        vn = bf16_round_bits(rng.standard_normal((n, HKV_, D_)).astype(np.float32))
        kp, vp = oracle.kv_append(kp, vp, kn, vn, np.array(slots, np.int32), BS_)
        gpu_lib.kv_append(to_dev(kn), to_dev(vn), gk, gv, torch.tensor(slots, dtype=torch.int32, device="cuda"))
        return copies

    prompt = bm.new_sequence(4, 4)
    append(prompt, 700)                              # 4-block pages; the last one part-filled
    beams = [prompt] + [bm.fork(prompt) for _ in range(3)]
    moved = [append(s, int(rng.integers(30, 300))) for s in beams[1:]]
    assert all(len(c) > 1 for c in moved)            # copy-on-write moved a page of several blocks
    others = [bm.new_sequence(1, 16), bm.new_sequence(16, 16), bm.new_sequence(1, 1), bm.new_sequence(2, 8)]
    for s in others:
        append(s, int(rng.integers(200, 1500)))
    for s in beams + others:
        append(s, 1)                                 # this step's token
    seqs = beams + others
    assert {n for s in seqs for _, n in bm.pages(s)} >= {1, 2, 4, 8, 16}
    rows = [bm.table(s) for s in seqs]
    W = max(len(t) for t, _ in rows)
    table = np.zeros((len(seqs), W), np.int32)
    for i, (t, _) in enumerate(rows):
        table[i, :len(t)] = t
    lens = np.array([n for _, n in rows], np.int32)
    scale = np.float32(1 / np.sqrt(D_))
    tt, tl = torch.from_numpy(table).cuda(), torch.from_numpy(lens).cuda()

    # decode, and the two-phase decode over the manager's prefix levels
    q = bf16_round_bits(rng.standard_normal((len(seqs), HQ_, D_)).astype(np.float32))
    ref = oracle.paged_attention(q, kp, vp, table, lens, np.arange(len(seqs) + 1), scale, BS_, "bf16")
    qd = to_dev(q)
    for split in (0, -2, 64):
        out = torch.empty_like(qd)
        gpu_lib.paged_attn_decode(out, qd, gk, gv, tt, tl, float(scale), int(lens.max()), split)
        torch.cuda.synchronize()
        got = oracle.bits_to_f64(out.view(torch.int16).cpu().numpy().view(np.uint16), "bf16")
        assert np.max(np.abs(got - ref)) <= 2e-2, split
    levels_host = bm.prefix_levels(seqs)
    assert levels_host
    levels = [gpu_lib.prefix_level(torch.from_numpy(st).cuda(), torch.from_numpy(hi).cuda(),
                                   int(np.max(np.diff(st))), int(np.max(hi - lo)), torch.from_numpy(lo).cuda())
              for st, lo, hi in levels_host]
    out = torch.empty_like(qd)
    gpu_lib.paged_attn_decode_cascade(out, qd, gk, gv, tt, tl, levels, float(scale), int(lens.max()), mode="two_phase")
    torch.cuda.synchronize()
    got = oracle.bits_to_f64(out.view(torch.int16).cpu().numpy().view(np.uint16), "bf16")
    assert np.max(np.abs(got - ref)) <= 2e-2

    # chunked prefill: the last 150 tokens of every sequence as query rows
    L = 150
    qp = bf16_round_bits(rng.standard_normal((len(seqs) * L, HQ_, D_)).astype(np.float32))
    cu = np.arange(len(seqs) + 1, dtype=np.int32) * L
    refp = oracle.paged_attention(qp, kp, vp, table, lens, cu, scale, BS_, "bf16", oracle.ScoreMods(causal=True))
    outp = torch.empty((len(seqs) * L, HQ_, D_), dtype=torch.bfloat16, device="cuda")
    gpu_lib.paged_attn_prefill(outp, to_dev(qp), torch.from_numpy(cu).cuda(), gk, gv, tt, tl, float(scale), L, True)
    torch.cuda.synchronize()
    got = oracle.bits_to_f64(outp.view(torch.int16).cpu().numpy().view(np.uint16), "bf16")
    assert np.max(np.abs(got - refp)) <= 2e-2

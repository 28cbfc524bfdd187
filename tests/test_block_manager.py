"""The host block manager (include/pagedattn_blocks.h): allocation, fork by
sharing, copy-on-write.  A random workload is replayed on numpy pools with
the oracle's kv_append and a plain block copy; every live sequence must read
back exactly its own token history through its table, and the counts must
add up.  Runs on the CPU (the manager never touches device memory)."""

import ctypes

import numpy as np
import pytest

import oracle
from paged_kv_cache_attn_amd import binding

BS, HKV, D, NB = 16, 2, 8, 48


def copy_blocks_reference(k_pool, v_pool, pairs):
    """Definition of kv_copy_blocks: whole (block, kv-head) slabs, bit for bit."""
    for src, dst in pairs:
        k_pool[dst] = k_pool[src]
        v_pool[dst] = v_pool[src]


class Replay:
    """Manager + numpy pools + each sequence's token history."""

    def __init__(self, seed, nb=NB, max_page=1):
        self.rng = np.random.default_rng(seed)
        self.bm = binding.BlockManager(nb, BS, max_page)
        self.nb = nb
        self.k = np.full((nb, HKV, BS, D), np.nan, np.float32)
        self.v = np.full((nb, HKV, BS // min(BS, 16), D, min(BS, 16)), np.nan, np.float32)
        self.hist = {}

    def new(self, min_page=1, max_page=None):
        s = self.bm.new_sequence(min_page, max_page)
        self.hist[s] = (np.zeros((0, HKV, D), np.float32), np.zeros((0, HKV, D), np.float32))
        return s

    def fork(self, s):
        c = self.bm.fork(s)
        self.hist[c] = tuple(x.copy() for x in self.hist[s])
        return c

    def free(self, s):
        self.bm.free(s)
        del self.hist[s]

    def append(self, s, n):
        slots, copies = self.bm.append(s, n)
        copy_blocks_reference(self.k, self.v, copies)
        kn = self.rng.standard_normal((n, HKV, D)).astype(np.float32)
        vn = self.rng.standard_normal((n, HKV, D)).astype(np.float32)
        self.k, self.v = oracle.kv_append(self.k, self.v, kn, vn, np.array(slots, np.int32), BS)
        hk, hv = self.hist[s]
        self.hist[s] = (np.concatenate([hk, kn]), np.concatenate([hv, vn]))
        return slots, copies

    def check(self):
        refs = np.zeros(self.nb, np.int64)
        waste = {}
        pages = {}  # first block -> size, over every live sequence
        for s, (hk, hv) in self.hist.items():
            row, n = self.bm.table(s)
            assert n == len(hk)
            # the table is the pages expanded; pages are aligned runs of 2^k blocks,
            # the last one holding the last token
            pg = self.bm.pages(s)
            assert row == [b for st, nb in pg for b in range(st, st + nb)]
            assert all(nb & (nb - 1) == 0 and st % nb == 0 for st, nb in pg)
            assert len(row) >= (n + BS - 1) // BS and (not pg or len(row) - pg[-1][1] < max(n, 1) / BS)
            for st, nb in pg:
                assert pages.setdefault(st, nb) == nb
            K, V = oracle.gather_sequence(self.k, self.v, np.array(row), n, BS)
            assert np.array_equal(K.transpose(1, 0, 2), hk) and np.array_equal(V.transpose(1, 0, 2), hv)
            for j, b in enumerate(row):
                refs[b] += 1
                waste[b] = min(waste.get(b, BS), BS - max(0, min(BS, n - j * BS)))
        # pages of different sequences are the same page or disjoint
        spans = sorted(pages.items())
        assert all(a + na <= b for (a, na), (b, _) in zip(spans, spans[1:]))
        for b in range(self.nb):
            assert self.bm.refcount(b) == refs[b], b
        free, used, w = self.bm.stats()
        assert used == int((refs > 0).sum()) and free + used == self.nb
        assert w == sum(waste.values())


def test_fork_and_copy_on_write():
    r = Replay(1)
    a = r.new()
    r.append(a, 20)            # blocks 0 (full) and 1 (4 tokens)
    b = r.fork(a)              # shares both
    _, copies = r.append(b, 3)  # the shared, partial last block is copied first
    assert len(copies) == 1 and copies[0][0] == r.bm.table(a)[0][1]
    _, copies = r.append(a, 1)  # a's last block is its own again: written in place
    assert copies == []
    r.check()
    c = r.fork(b)
    r.append(c, 13)            # fills b's copy of the last block, then a new one (copy first)
    r.free(b)
    r.check()
    r.free(a)
    r.free(c)
    assert r.bm.stats() == (NB, 0, 0)


@pytest.mark.parametrize("seed", range(6))
def test_random_workload_replays_exactly(seed):
    r = Replay(100 + seed)
    live = [r.new()]
    for _ in range(60):
        op = r.rng.random()
        if op < 0.5 and live:
            s = live[r.rng.integers(len(live))]
            n = int(r.rng.integers(1, 40))
            try:
                r.append(s, n)
            except ValueError:
                pass  # pool exhausted: nothing changed
        elif op < 0.7 and live:
            live.append(r.fork(live[r.rng.integers(len(live))]))
        elif op < 0.85 and len(live) > 1:
            r.free(live.pop(r.rng.integers(len(live))))
        else:
            live.append(r.new())
        r.check()


def test_exhaustion_changes_nothing_and_ids_are_checked():
    r = Replay(3, nb=4)
    a = r.new()
    r.append(a, 60)                      # 4 blocks
    before = r.bm.table(a), r.bm.stats()
    with pytest.raises(ValueError, match="no free block"):
        r.bm.append(a, 10)
    assert (r.bm.table(a), r.bm.stats()) == before
    b = r.fork(a)
    with pytest.raises(ValueError, match="no free block"):  # copy-on-write needs a block too
        r.bm.append(b, 1)
    r.free(b)
    with pytest.raises(ValueError, match="sequence"):
        r.bm.append(b, 1)
    with pytest.raises(ValueError, match="sequence"):
        r.bm.fork(12345)
    r.check()


# ---- pages of several blocks (power-of-two sizes, buddy allocation) ----

def test_pages_double_along_a_sequence():
    r = Replay(7, nb=200, max_page=8)
    a = r.new(1, 8)
    for _ in range(53):
        r.append(a, 7)                   # 371 tokens: capacity 1+2+4+8+8 = 23 blocks = 368 < 371
    assert [n for _, n in r.bm.pages(a)] == [1, 2, 4, 8, 8, 8]
    r.check()


def test_page_sizes_mix_in_one_pool():
    r = Replay(8, nb=640, max_page=16)
    seqs = [r.new(k, k) for k in (1, 2, 4, 8, 16)] + [r.new(1, 16), r.new(2, 4)]
    for _ in range(25):
        for q in seqs:
            r.append(q, int(r.rng.integers(1, 40)))
    for q, k in zip(seqs, (1, 2, 4, 8, 16)):
        assert {n for _, n in r.bm.pages(q)} == {k}
    r.check()


def test_copy_on_write_copies_the_filled_blocks_of_a_shared_page():
    r = Replay(9, nb=64, max_page=4)
    a = r.new(4, 4)
    r.append(a, 40)                      # one 4-block page; blocks 0..2 hold tokens
    b = r.fork(a)
    _, copies = r.append(b, 5)           # the shared page has room: b continues in a fresh page
    (pa_start, _), (pb_start, _) = r.bm.pages(a)[0], r.bm.pages(b)[0]
    assert copies == [(pa_start + i, pb_start + i) for i in range(3)]
    assert r.bm.refcount(pa_start) == 1 and r.bm.refcount(pb_start + 3) == 1
    _, copies = r.append(a, 30)          # a's page is its own again: written in place, then a new page
    assert copies == []
    r.check()
    c = r.fork(b)
    r.append(c, 100)
    r.free(b)
    r.check()
    r.free(a)
    r.free(c)
    assert r.bm.stats() == (64, 0, 0)


def test_buddies_merge_back_on_release():
    bm = binding.BlockManager(64, BS, 16)          # four aligned 16-block pages
    seqs = [bm.new_sequence(1, 16) for _ in range(6)]
    for q in seqs:
        bm.append(q, 16 * 5)                      # pages of 1, 2 and 4 blocks each
    for q in seqs:
        bm.free(q)
    big = [bm.new_sequence(16, 16) for _ in range(4)]
    for q in big:
        bm.append(q, 16 * 16)
    assert sorted(st for q in big for st, _ in bm.pages(q)) == [0, 16, 32, 48]
    assert bm.stats() == (0, 64, 0)


def test_smaller_pages_stand_in_when_the_pool_is_fragmented():
    bm = binding.BlockManager(16, BS, 8)
    ones = [bm.new_sequence() for _ in range(16)]
    for q in ones:
        bm.append(q, 1)
    for q in ones[1::2]:
        bm.free(q)                                # every other block free: no 2-block page left
    big = bm.new_sequence(8, 8)
    bm.append(big, 16 * 8)
    assert [n for _, n in bm.pages(big)] == [1] * 8
    assert bm.stats()[0] == 0


def test_paged_exhaustion_changes_nothing_and_arguments_are_checked():
    r = Replay(10, nb=12, max_page=4)
    a = r.new(4, 4)
    r.append(a, 16 * 8)                  # two full 4-block pages
    b = r.fork(a)
    r.append(b, 16)                      # a third page for b alone (its last page was full)
    before = [r.bm.stats(), r.bm.table(a), r.bm.table(b), r.bm.pages(b)]
    with pytest.raises(ValueError, match="no free block"):
        r.bm.append(b, 16 * 4)           # needs one more page
    c = r.fork(b)
    with pytest.raises(ValueError, match="no free block"):
        r.bm.append(c, 1)                # copy-on-write of the shared, part-filled page needs a page too
    r.free(c)
    assert [r.bm.stats(), r.bm.table(a), r.bm.table(b), r.bm.pages(b)] == before
    r.check()
    for lo, hi in ((3, 4), (4, 2), (8, 8), (0, 1)):
        with pytest.raises(ValueError):
            r.bm.new_sequence(lo, hi)     # not powers of two, min > max, or beyond the manager's pages
    with pytest.raises(ValueError):
        binding.BlockManager(8, BS, 3)
    with pytest.raises(ValueError):
        binding.BlockManager(8, BS, 8192)
    with pytest.raises(ValueError, match="too large"):
        binding.BlockManager((1 << 31) // BS, BS)   # slots past 2^31 - 1 would not fit kv_append's int32


@pytest.mark.parametrize("seed", range(6))
def test_random_paged_workload_replays_exactly(seed):
    r = Replay(200 + seed, nb=96, max_page=8)
    policies = [(1, 1), (2, 2), (8, 8), (1, 8), (2, 4)]

    def new():
        return r.new(*policies[r.rng.integers(len(policies))])

    live = [new()]
    for _ in range(80):
        op = r.rng.random()
        if op < 0.5 and live:
            q = live[r.rng.integers(len(live))]
            try:
                r.append(q, int(r.rng.integers(1, 60)))
            except ValueError:
                pass  # pool exhausted: nothing changed
        elif op < 0.7 and live:
            live.append(r.fork(live[r.rng.integers(len(live))]))
        elif op < 0.85 and len(live) > 1:
            r.free(live.pop(r.rng.integers(len(live))))
        else:
            live.append(new())
        r.check()
    for q in live:
        r.free(q)
    assert r.bm.stats() == (96, 0, 0)


def test_fragmentation_matches_the_arithmetic():
    r = Replay(4)
    lens = [1, 15, 16, 17, 33, 40]
    for n in lens:
        r.append(r.new(), n)
    free, used, waste = r.bm.stats()
    held = sum((n + BS - 1) // BS * BS for n in lens)
    assert used * BS == held and waste == held - sum(lens)


# ------------------------------------------------------------------------------------------
# shared prefixes of a decode batch (levels for the two-phase decode)
# ------------------------------------------------------------------------------------------

def _shared_tokens(r, s, t):
    """Leading full blocks that two sequences' tables both name, in tokens."""
    (ra, na), (rb, nb) = r.bm.table(s), r.bm.table(t)
    j = 0
    while j < min(na, nb) // BS and ra[j] == rb[j]:
        j += 1
    return j * BS


def check_levels(r, seqs, levels):
    n = len(seqs)
    prev = np.zeros(n, np.int64)
    for starts, lo, hi in levels:
        assert starts[0] == 0 and starts[-1] == n and np.all(np.diff(starts) >= 1)
        assert np.any(hi > lo), "a level with nothing shared"
        for g in range(len(lo)):
            mem = list(range(starts[g], starts[g + 1]))
            rows = [r.bm.table(seqs[i]) for i in mem]
            for i in mem:
                assert lo[g] == prev[i]                       # ranges chain per sequence
                prev[i] = hi[g]
            assert lo[g] <= hi[g] <= min(ln for _, ln in rows)
            nbk = (int(hi[g]) + BS - 1) // BS                # the range's blocks are the same ids
            for row, _ in rows:
                assert list(row[:nbk]) == list(rows[0][0][:nbk])
    return prev


def test_prefix_levels_by_hand():
    r = Replay(21, nb=64)
    a = r.new()
    r.append(a, 48)                      # 3 full blocks
    b, c = r.fork(a), r.fork(a)
    r.append(a, 20)
    r.append(b, 20)
    r.append(c, 20)                      # c: 4 full blocks + 4 tokens
    d = r.fork(c)
    r.append(d, 5)                       # copy-on-write of c's partly filled 5th block
    e = r.new()
    r.append(e, 30)
    seqs = [a, b, c, d, e]
    levels = r.bm.prefix_levels(seqs)
    assert len(levels) == 2
    (s0, lo0, hi0), (s1, lo1, hi1) = levels
    assert list(s0) == [0, 4, 5] and list(lo0) == [0, 0] and list(hi0) == [48, 0]
    assert list(s1) == [0, 1, 2, 4, 5] and list(lo1) == [48, 48, 48, 0] and list(hi1) == [48, 48, 64, 0]
    check_levels(r, seqs, levels)
    one = r.bm.prefix_levels(seqs, max_levels=1)
    assert len(one) == 1 and all(np.array_equal(x, y) for x, y in zip(one[0], levels[0]))
    assert r.bm.prefix_levels([a, e]) == []                 # neighbours that share nothing
    assert r.bm.prefix_levels([]) == []


@pytest.mark.parametrize("seed", [3, 4, 5])
def test_prefix_levels_of_random_fork_trees(seed):
    rng = np.random.default_rng(seed)
    r = Replay(seed, nb=400)
    roots = [r.new() for _ in range(3)]
    for s in roots:
        r.append(s, int(rng.integers(1, 80)))
    live = list(roots)
    order = {s: (i,) for i, s in enumerate(roots)}      # fork-tree path: keeps forks adjacent
    for _ in range(25):
        p = live[int(rng.integers(len(live)))]
        c = r.fork(p)
        order[c] = order[p] + (len(order),)
        live.append(c)
        for s in (p, c):
            r.append(s, int(rng.integers(0, 40)))
    seqs = sorted(live, key=lambda s: order[s])
    levels = r.bm.prefix_levels(seqs)
    ends = check_levels(r, seqs, levels)
    # with enough levels, every neighbour pair's shared blocks are grouped exactly
    assert len(levels) < 8
    for i in range(len(seqs) - 1):
        want = _shared_tokens(r, seqs[i], seqs[i + 1])
        got = 0
        for starts, lo, hi in levels:
            g = np.searchsorted(starts, i, side="right") - 1
            if starts[g + 1] > i + 1:
                got = max(got, int(hi[g]))
        assert got == want, (i, got, want)
    assert np.all(ends <= np.array([r.bm.table(s)[1] for s in seqs]))


def test_prefix_levels_argument_checks():
    r = Replay(22)
    a = r.new()
    L = binding.lib()
    ids = (ctypes.c_int32 * 1)(a)
    buf = (ctypes.c_int32 * 64)()
    nl = ctypes.c_int32()
    assert L.pa_bm_prefix_levels(r.bm._h, ids, 1, 0, buf, buf, buf, buf, ctypes.byref(nl)) == -2
    assert L.pa_bm_prefix_levels(r.bm._h, ids, 1, 9, buf, buf, buf, buf, ctypes.byref(nl)) == -2
    assert L.pa_bm_prefix_levels(r.bm._h, ids, -1, 1, buf, buf, buf, buf, ctypes.byref(nl)) == -2
    bad = (ctypes.c_int32 * 1)(12345)
    assert L.pa_bm_prefix_levels(r.bm._h, bad, 1, 1, buf, buf, buf, buf, ctypes.byref(nl)) == -13
    assert L.pa_bm_prefix_levels(r.bm._h, ids, 1, 1, None, buf, buf, buf, ctypes.byref(nl)) == -1

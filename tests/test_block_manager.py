"""The host block manager (include/pagedattn_blocks.h): allocation, fork by
sharing, copy-on-write.  A random workload is replayed on numpy pools with
the oracle's kv_append and a plain block copy; every live sequence must read
back exactly its own token history through its table, and the counts must
add up.  Runs on the CPU (the manager never touches device memory)."""

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

    def __init__(self, seed, nb=NB):
        self.rng = np.random.default_rng(seed)
        self.bm = binding.BlockManager(nb, BS)
        self.nb = nb
        self.k = np.full((nb, HKV, BS, D), np.nan, np.float32)
        self.v = np.full((nb, HKV, BS // min(BS, 16), D, min(BS, 16)), np.nan, np.float32)
        self.hist = {}

    def new(self):
        s = self.bm.new_sequence()
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
        for s, (hk, hv) in self.hist.items():
            row, n = self.bm.table(s)
            assert n == len(hk)
            assert len(row) == (n + BS - 1) // BS
            K, V = oracle.gather_sequence(self.k, self.v, np.array(row), n, BS)
            assert np.array_equal(K.transpose(1, 0, 2), hk) and np.array_equal(V.transpose(1, 0, 2), hv)
            for j, b in enumerate(row):
                refs[b] += 1
                waste[b] = min(waste.get(b, BS), BS - min(BS, n - j * BS))
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


def test_fragmentation_matches_the_arithmetic():
    r = Replay(4)
    lens = [1, 15, 16, 17, 33, 40]
    for n in lens:
        r.append(r.new(), n)
    free, used, waste = r.bm.stats()
    held = sum((n + BS - 1) // BS * BS for n in lens)
    assert used * BS == held and waste == held - sum(lens)

"""Seeded synthetic paged-KV workloads.

Everything here is input construction: random draws, rounding of those draws
to the storage dtype, and placement of the drawn rows in a shared block pool
whose blocks are handed to sequences in a random order (the block table).  No
attention arithmetic lives here.

Storage format (the contract the library, the oracle and these generators
share):

* ``k_pool``: ``[NB, Hkv, bs, D]`` -- one (block, kv-head) slab holds ``bs``
  key rows of ``D`` elements each (token-major).
* ``v_pool``: ``[NB, Hkv, bs/S, D, S]`` with ``S = min(bs, 16)`` -- one
  (block, kv-head) slab holds ``bs/S`` sub-slabs of ``S`` tokens, each ``D``
  rows of ``S`` tokens (dimension-major, token-minor); token ``o`` of a block
  is column ``o % S`` of sub-slab ``o // S``.
* ``block_table``: int32 ``[B, W]``; entry ``[b, j]`` is the physical block
  that holds logical tokens ``[j*bs, (j+1)*bs)`` of sequence ``b``; entries
  past ``ceil(context_lens[b] / bs)`` are -1 and never read.
* bf16 tensors are carried as their uint16 bit patterns; fp32 as float32.

Pool slots that no sequence references, tail slots past a sequence's length
and the slots that the step's ``kv_append`` is about to fill are set to NaN, so
any read of them shows up in the output.

Draws: numpy PCG64 through ``SeedSequence(seed)``.  Child stream 0 draws the
structure (lengths, block permutation), 1 the queries, 2 the appended tokens,
3 the pool contents (spawned again per range of physical blocks so that the
pool can be filled by several threads and still be identical bit for bit).
"""

from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

BF16_NAN_BITS = np.uint16(0x7FC0)
F32_NAN_BITS = np.uint32(0x7FC00000)

# Consecutive physical blocks per independently seeded draw range when filling a pool.
_POOL_GROUP_BLOCKS = 256


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """float32 values -> bf16 bit patterns (uint16), round to nearest even.

    Inputs are finite normal draws, so no NaN/Inf handling is needed.
    """
    b = np.array(x, dtype=np.float32, copy=True).view(np.uint32)
    b += np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return (b >> np.uint32(16)).astype(np.uint16)


def _normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return bf16_round_bits(x) if dtype == "bf16" else x


def _nan_fill(shape, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return np.full(shape, BF16_NAN_BITS, dtype=np.uint16)
    return np.full(shape, F32_NAN_BITS, dtype=np.uint32).view(np.float32)


def _nan_value(dtype: str):
    return BF16_NAN_BITS if dtype == "bf16" else F32_NAN_BITS.view(np.float32)


@dataclasses.dataclass
class Workload:
    """One batch of paged-attention inputs (host arrays)."""

    name: str
    kind: str  # "decode" (one query row per sequence) or "prefill"
    dtype: str  # "f32" or "bf16"
    B: int
    Hq: int
    Hkv: int
    D: int
    bs: int
    NB: int
    scale: np.float32
    causal: bool
    context_lens: np.ndarray  # int32 [B], keys per sequence incl. appended
    block_table: np.ndarray  # int32 [B, W]
    q: np.ndarray  # [sum(q_lens), Hq, D]
    q_lens: np.ndarray  # int32 [B]
    cu_q_lens: np.ndarray  # int32 [B + 1]
    k_pool: np.ndarray  # [NB, Hkv, bs, D]   (state before kv_append)
    v_pool: np.ndarray  # [NB, Hkv, bs/S, D, S], S = min(bs, 16)   (state before kv_append)
    k_new: np.ndarray  # [T, Hkv, D]
    v_new: np.ndarray  # [T, Hkv, D]
    slot_mapping: np.ndarray  # int32 [T]
    meta: dict = dataclasses.field(default_factory=dict)

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.B else 0

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens.max()) if self.B else 0

    @property
    def esize(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def kv_bytes(self) -> int:
        """K+V bytes that one pass over every sequence's context reads."""
        return int(self.context_lens.astype(np.int64).sum()) * self.Hkv * self.D * 2 * self.esize

    def unique_kv_bytes(self) -> int:
        """K+V bytes of the distinct physical slots referenced by the tables."""
        seen = {}
        for b in range(self.B):
            n = int(self.context_lens[b])
            for j in range((n + self.bs - 1) // self.bs):
                pb = int(self.block_table[b, j])
                seen[pb] = max(seen.get(pb, 0), min(self.bs, n - j * self.bs))
        return sum(seen.values()) * self.Hkv * self.D * 2 * self.esize


def _fill_pools(ss: np.random.SeedSequence, NB, Hkv, D, bs, live, dtype, threads):
    """Pools of NaN with N(0,1) rows in the live slots.

    ``live[pb]`` is the number of leading live token slots of physical block
    ``pb`` (-1: not referenced).  The pool is processed in ranges of
    consecutive physical blocks, each with its own child stream (so the
    result does not depend on the thread count); inside a range the
    referenced blocks are drawn in ascending physical order.
    """
    S = min(bs, 16)
    vshape = (Hkv, bs // S, D, S)
    if dtype == "bf16":
        k_pool = np.empty((NB, Hkv, bs, D), np.uint16)
        v_pool = np.empty((NB,) + vshape, np.uint16)
    else:
        k_pool = np.empty((NB, Hkv, bs, D), np.float32)
        v_pool = np.empty((NB,) + vshape, np.float32)
    ranges = [(i, min(NB, i + _POOL_GROUP_BLOCKS)) for i in range(0, NB, _POOL_GROUP_BLOCKS)]
    children = ss.spawn(len(ranges))
    nan = _nan_value(dtype)

    def work(ri):
        c0, c1 = ranges[ri]
        lv = live[c0:c1]
        ref = np.nonzero(lv >= 0)[0]
        k_pool[c0:c1][lv < 0] = nan
        v_pool[c0:c1][lv < 0] = nan
        if len(ref) == 0:
            return
        rng = np.random.default_rng(children[ri])
        kv = _normal(rng, (len(ref), Hkv, bs, D), dtype)
        vv = _normal(rng, (len(ref),) + vshape, dtype)
        lr = lv[ref]
        for i in np.nonzero(lr < bs)[0]:
            kv[i, :, lr[i]:, :] = nan
            tail = np.arange(lr[i], bs)
            vv[i, :, tail // S, :, tail % S] = nan
        k_pool[c0 + ref] = kv
        v_pool[c0 + ref] = vv

    nthreads = max(1, min(threads or os.cpu_count() or 1, 16, len(ranges) or 1))
    if nthreads == 1:
        for ri in range(len(ranges)):
            work(ri)
    else:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(work, range(len(ranges))))
    return k_pool, v_pool


def build_workload(
    *,
    name: str,
    seed: int,
    kind: str,
    dtype: str,
    Hq: int,
    Hkv: int,
    D: int,
    bs: int,
    context_lens,
    q_lens=None,
    append_lens=None,
    NB: int | None = None,
    pool_slack: float = 2.0,
    shared_prefix_blocks: int = 0,
    prefix_groups=None,
    causal: bool = False,
    scale: float | None = None,
    table_width: int | None = None,
    structure_rng: np.random.Generator | None = None,
    threads: int | None = None,
) -> Workload:
    """Lay out a batch of sequences in a randomly permuted block pool.

    ``context_lens[b]`` counts every key of sequence ``b`` after this step's
    append; the last ``append_lens[b]`` of them are not in the pool yet but
    arrive through ``k_new``/``v_new``/``slot_mapping``.  ``q_lens[b]`` query
    rows sit at the last ``q_lens[b]`` positions of the sequence.  The first
    ``shared_prefix_blocks`` logical blocks of every sequence map to the same
    physical blocks.  ``prefix_groups`` -- a list of (members, blocks) that
    covers the batch in order -- instead makes each run of ``members``
    consecutive sequences share their first ``blocks`` physical blocks.
    """
    ss = np.random.SeedSequence(seed)
    c_struct, c_q, c_new, c_pool = ss.spawn(4)
    rng = structure_rng if structure_rng is not None else np.random.default_rng(c_struct)

    ctx = np.asarray(context_lens, dtype=np.int64)
    B = len(ctx)
    if q_lens is None:
        q_lens = np.ones(B, np.int64) if kind == "decode" else ctx.copy()
    q_lens = np.asarray(q_lens, dtype=np.int64)
    if append_lens is None:
        append_lens = np.zeros(B, np.int64)
    append_lens = np.asarray(append_lens, dtype=np.int64)
    assert (kind == "decode" or np.all(q_lens <= ctx)) and np.all(append_lens <= ctx)
    if kind == "decode":
        assert np.all(q_lens == 1)

    nblk = (ctx + bs - 1) // bs
    if prefix_groups is None:
        groups = [(B, int(shared_prefix_blocks))]
    else:
        assert shared_prefix_blocks == 0
        groups = [(int(m), int(s)) for m, s in prefix_groups]
        assert sum(m for m, _ in groups) == B
    S_b = np.repeat(np.array([s for _, s in groups], np.int64), [m for m, _ in groups])
    assert np.all(nblk >= S_b)
    # shared blocks must be full and present in every sequence
    assert np.all((S_b == 0) | (ctx - append_lens >= S_b * bs))
    unique_needed = int(sum(s for _, s in groups) + (nblk - S_b).sum())
    if NB is None:
        NB = max(1, int(math.ceil(pool_slack * unique_needed)))
    assert NB >= unique_needed
    W = int(table_width if table_width is not None else max(1, int(nblk.max(initial=0))))
    perm = rng.permutation(NB).astype(np.int64)

    table = np.full((B, W), -1, dtype=np.int32)
    live = np.full(NB, -1, dtype=np.int64)
    cursor = 0
    shared_ids = []
    for _, s in groups:
        shared_ids.append(perm[cursor:cursor + s])
        cursor += s
    group_of = np.repeat(np.arange(len(groups)), [m for m, _ in groups])
    for b in range(B):
        S = int(S_b[b])
        priv = perm[cursor:cursor + nblk[b] - S]
        cursor += nblk[b] - S
        ids = np.concatenate([shared_ids[group_of[b]], priv])
        table[b, :nblk[b]] = ids
        present = ctx[b] - append_lens[b]
        for j, pb in enumerate(ids):
            n_live = int(min(bs, max(0, present - j * bs)))
            live[pb] = max(live[pb], n_live)

    k_pool, v_pool = _fill_pools(c_pool, NB, Hkv, D, bs, live, dtype, threads)

    q = _normal(np.random.default_rng(c_q), (int(q_lens.sum()), Hq, D), dtype)

    T = int(append_lens.sum())
    rng_new = np.random.default_rng(c_new)
    k_new = _normal(rng_new, (T, Hkv, D), dtype)
    v_new = _normal(rng_new, (T, Hkv, D), dtype)
    slots = np.empty(T, dtype=np.int32)
    t = 0
    for b in range(B):
        for p in range(int(ctx[b] - append_lens[b]), int(ctx[b])):
            slots[t] = table[b, p // bs] * bs + p % bs
            t += 1

    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(q_lens)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return Workload(
        name=name, kind=kind, dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, D=D, bs=bs, NB=NB,
        scale=np.float32(scale), causal=bool(causal),
        context_lens=ctx.astype(np.int32), block_table=table, q=q,
        q_lens=q_lens.astype(np.int32), cu_q_lens=cu, k_pool=k_pool, v_pool=v_pool,
        k_new=k_new, v_new=v_new, slot_mapping=slots,
        meta={"seed": seed, "unique_blocks": unique_needed, "shared_prefix_blocks": int(shared_prefix_blocks),
              "prefix_groups": groups},
    )


# The reference workloads: name -> (seed, description).
WORKLOADS = {
    "single_decode_f32": (1, "decode, fp32, 1 sequence of 128 tokens, 4 heads (no GQA), head_dim 64, "
                             "8 blocks of 16 in a 64-block pool"),
    "gqa_decode_bf16": (2, "decode, bf16, 8 sequences of 128..2048 tokens, 32/8 heads, head_dim 128, "
                           "block 16, pool 2x the needed blocks, one appended token per sequence"),
    "chunked_prefill_bf16": (3, "causal chunked prefill, bf16, 4 sequences: 512-token chunk after 1536 "
                                "tokens, 32/8 heads, head_dim 128, block 16"),
    "shared_prefix_decode_bf16": (4, "decode, bf16, 16 sequences sharing 64 physical blocks (1024-token "
                                     "prefix) plus 256 private tokens each, 32/8 heads, head_dim 128"),
    "long_decode_bf16": (5, "decode, bf16, 64 sequences, log-normal lengths (median 8192, clipped to "
                            "2048..32768), 64/8 heads, head_dim 128, block 16, one appended token each"),
}


def named_workload(name: str, bs: int | None = None, threads: int | None = None,
                   batch: int | None = None, tp: int = 1) -> Workload:
    """One of the reference workloads (seeded; see ``WORKLOADS``).

    ``bs`` overrides the page size (power-of-two page-size variants);
    ``batch`` keeps only the first ``batch`` sequences (same draws);
    ``tp`` keeps 1/tp of the query and kv heads: one GPU's share when the
    heads are split over tp GPUs (same lengths and tables).
    """
    i = WORKLOADS[name][0]
    ss = np.random.SeedSequence(i)
    rng = np.random.default_rng(ss.spawn(1)[0])  # same stream as build's c_struct
    common = dict(seed=i, structure_rng=rng, threads=threads)
    if tp != 1:
        full = {"single_decode_f32": (4, 4), "gqa_decode_bf16": (32, 8), "chunked_prefill_bf16": (32, 8),
                "shared_prefix_decode_bf16": (32, 8), "long_decode_bf16": (64, 8)}[name]
        if tp < 1 or full[0] % tp or full[1] % tp:
            raise ValueError(f"{name}: {full[0]}/{full[1]} heads do not split {tp} ways")
    hq = lambda n: n // tp
    if name == "single_decode_f32":
        return build_workload(name=name, kind="decode", dtype="f32", Hq=hq(4), Hkv=hq(4),
                              D=64, bs=bs or 16, context_lens=[128], NB=64, **common)
    if name == "gqa_decode_bf16":
        ctx = rng.integers(128, 2049, size=8)
        ctx = ctx[:batch] if batch else ctx
        return build_workload(name=name, kind="decode", dtype="bf16", Hq=hq(32), Hkv=hq(8),
                              D=128, bs=bs or 16, context_lens=ctx,
                              append_lens=np.ones(len(ctx), np.int64), **common)
    if name == "chunked_prefill_bf16":
        n = (batch or 4)
        return build_workload(name=name, kind="prefill", dtype="bf16", Hq=hq(32), Hkv=hq(8),
                              D=128, bs=bs or 16, context_lens=[2048] * n, q_lens=[512] * n,
                              append_lens=[512] * n, causal=True, **common)
    if name == "shared_prefix_decode_bf16":
        n = (batch or 16)
        bsz = bs or 16
        return build_workload(name=name, kind="decode", dtype="bf16", Hq=hq(32), Hkv=hq(8),
                              D=128, bs=bsz, context_lens=[1280] * n,
                              shared_prefix_blocks=1024 // bsz, **common)
    if name == "long_decode_bf16":
        ctx = np.rint(rng.lognormal(mean=math.log(8192), sigma=math.log(2), size=64))
        ctx = np.clip(ctx, 2048, 32768).astype(np.int64)
        ctx = ctx[:batch] if batch else ctx
        return build_workload(name=name, kind="decode", dtype="bf16", Hq=hq(64), Hkv=hq(8),
                              D=128, bs=bs or 16, context_lens=ctx,
                              append_lens=np.ones(len(ctx), np.int64), **common)
    raise ValueError(f"no workload {name}")

"""Plain fp64 statement of paged KV-cache attention (the oracle).

TEST INFRASTRUCTURE ONLY -- imported by ``tests/``, ``__graft_entry__.smoke()``
and ``bench.py``'s ``cpu_baseline`` leg, never by the product path.

What is computed, and where it comes from:

* Paged KV storage.  The KV cache is cut into fixed-size blocks (16 tokens by
  default), each sequence owns a list of physical blocks that a block table
  maps from logical positions, and placement of the blocks in memory does not
  change the result ("Ultimate Guide to PagedAttention", newline: the parts on
  KV blocks, the block table and non-contiguous storage; Kwon et al.,
  "Efficient Memory Management for Large Language Model Serving with
  PagedAttention", abstract).  Here that is :func:`gather_sequence`: look up
  each logical block in the table and read its rows.
* Exact attention.  Paged attention is exact softmax attention over the
  gathered keys/values, only computed without a contiguous copy (Dao et al.,
  "FlashAttention: Fast and Memory-Efficient Exact Attention with
  IO-Awareness", abstract: tiling is an IO technique for an exact result).
  Here that is :func:`attention_dense`: ``softmax(Q K^T * scale + mods) V`` in
  fp64, which is that definition written out.
* Mask / score modification in the style of PyTorch FlexAttention (Joshi et
  al., "Paged Attention Meets FlexAttention", abstract and summary): the page
  names the integration but not its mods; the mods offered here act on
  logical positions only (:class:`ScoreMods`).
* KV append.  New tokens' key/value vectors are stored into the cache as they
  are produced, growing a sequence by writing into (possibly new) blocks
  without moving existing data ("Ultimate Guide to PagedAttention": the parts
  on the KV cache and on dynamic growth).  Here that is :func:`kv_append`, a
  raw-bits scatter to the slots a slot mapping names.

Readings where the pages are silent (each is listed in the design notes):
query row ``i`` of a sequence with ``n`` keys and ``Lq`` query rows sits at
logical position ``n - Lq + i`` (bottom-right causal alignment; decode is
``Lq = 1``); query head ``h`` reads kv-head ``h // (Hq / Hkv)``; a row with no
admissible key outputs zeros; inside a (block, kv-head) the K slab is
token-major ``[bs, D]`` and the V slab is ``bs / S`` dimension-major sub-slabs
``[D, S]`` of ``S = min(bs, 16)`` tokens each (:func:`v_group`), so the V pool
is ``[NB, Hkv, bs / S, D, S]``.
"""

from __future__ import annotations

import dataclasses

import numpy as np


def bits_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Storage values -> fp64, exactly (bf16 bits shifted into an fp32)."""
    if dtype == "bf16":
        return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
            np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


@dataclasses.dataclass
class BlockMask:
    """Block-sparse mask in the manner of FlexAttention's block mask: which
    key blocks each query block may see at all (Joshi et al., "Paged
    Attention Meets FlexAttention", abstract: the paged kernel keeps
    FlexAttention's programmable masks; skipping whole blocks is how a block
    mask saves work).

    ``bits`` is uint32 ``[num_seqs * rows_per_seq, words]``.  For sequence
    ``b`` and a query at logical position ``p`` the row is
    ``b * rows_per_seq + p // q_block``; key ``j`` is admissible only if bit
    ``(j // kv_block) % 32`` of word ``(j // kv_block) // 32`` of that row is
    set (bit 0 = least significant).  Other masks still apply inside the
    admitted blocks.
    """

    bits: np.ndarray
    q_block: int
    kv_block: int
    rows_per_seq: int

    def keys_allowed(self, b, q_pos, n):
        """Boolean ``[len(q_pos), n]``: the block mask for these query positions."""
        q_pos = np.asarray(q_pos, dtype=np.int64)
        rows = b * self.rows_per_seq + q_pos // self.q_block
        kb = np.arange(n, dtype=np.int64) // self.kv_block
        words = np.asarray(self.bits, dtype=np.uint64)[rows][:, kb // 32]  # [Lq, n]
        return ((words >> (kb % 32).astype(np.uint64)[None, :]) & np.uint64(1)).astype(bool)


@dataclasses.dataclass
class ScoreMods:
    """FlexAttention-style modifications, all on logical positions.

    Applied to ``s = scale * q.k`` in this order:
      softcap > 0     : s <- softcap * tanh(s / softcap)
      alibi_slopes    : s <- s + slope[h] * (kv_pos - q_pos)
    then masks (a key is admissible only if all hold):
      kv_pos < n      (the sequence's keys; always)
      causal          : kv_pos <= q_pos, or kv_pos < prefix_lens[b] when
                        prefix lengths are given (prefix-LM: the prefix is
                        seen by every row of the sequence)
      window > 0      : q_pos - kv_pos < window
      doc_starts      : kv_pos >= doc_starts[row] (document masking of packed
                        sequences: a row sees nothing before its document)
      block_mask      : the key's block is admitted for the query's block
                        (:class:`BlockMask`)
    ``prefix_lens`` is per sequence ``[B]``; ``doc_starts`` per query row
    ``[sum Lq]`` (decode: one per sequence).
    """

    causal: bool = False
    window: int = 0
    softcap: float = 0.0
    alibi_slopes: np.ndarray | None = None
    prefix_lens: np.ndarray | None = None
    doc_starts: np.ndarray | None = None
    block_mask: BlockMask | None = None


def v_group(bs):
    """Tokens per V sub-slab: ``min(bs, 16)``."""
    return min(int(bs), 16)


def _check_pools(k_pool, v_pool, bs):
    S = v_group(bs)
    NB, Hkv, kbs, D = k_pool.shape
    if kbs != bs or tuple(v_pool.shape) != (NB, Hkv, bs // S, D, S):
        raise ValueError(f"pools {k_pool.shape} / {v_pool.shape} do not match block size {bs}")


def kv_append(k_pool, v_pool, k_new, v_new, slot_mapping, bs):
    """Write token ``t``'s rows into slot ``slot_mapping[t]``; return new pools.

    Slot ``s`` is block ``s // bs``, offset ``o = s % bs``.  K goes to
    ``k_pool[block, :, o, :]``, V to ``v_pool[block, :, o // S, :, o % S]``
    (``S = v_group(bs)``).
    Negative slots are skipped.  The copy is of raw bits (no conversion).
    Duplicate non-negative slots within one call have no defined result and
    are rejected here.
    """
    _check_pools(k_pool, v_pool, bs)
    S = v_group(bs)
    kp = np.array(k_pool, copy=True)
    vp = np.array(v_pool, copy=True)
    seen = set()
    for t, s in enumerate(np.asarray(slot_mapping).tolist()):
        if s < 0:
            continue
        if s in seen:
            raise ValueError(f"slot {s} written twice in one append")
        seen.add(s)
        blk, off = divmod(s, bs)
        kp[blk, :, off, :] = k_new[t]
        vp[blk, :, off // S, :, off % S] = v_new[t]
    return kp, vp


def gather_sequence(k_pool, v_pool, table_row, n, bs):
    """Logical keys/values of one sequence, ``[Hkv, n, D]`` each (storage dtype).

    Logical block ``j`` of the sequence is physical block ``table_row[j]``;
    only the first ``ceil(n / bs)`` entries are read and only the first ``n``
    token rows are kept.
    """
    _check_pools(k_pool, v_pool, bs)
    nb = (n + bs - 1) // bs
    phys = np.asarray(table_row[:nb], dtype=np.int64)
    Hkv, D = k_pool.shape[1], k_pool.shape[3]
    K = k_pool[phys]  # [nb, Hkv, bs, D]
    V = v_pool[phys]  # [nb, Hkv, bs/S, D, S]
    K = K.transpose(1, 0, 2, 3).reshape(Hkv, nb * bs, D)[:, :n]
    V = V.transpose(1, 0, 2, 4, 3).reshape(Hkv, nb * bs, D)[:, :n]  # token = sub-slab * S + column
    return K, V


def attention_dense(Q, K, V, scale, q_pos, mods: ScoreMods | None = None, prefix_len=0, doc_start=None,
                    keys_allowed=None):
    """Exact attention of query rows at logical positions ``q_pos``.

    ``Q`` ``[Lq, Hq, D]``, ``K``/``V`` ``[Hkv, n, D]`` (fp64), key ``j`` sits at
    logical position ``j``.  Query head ``h`` uses kv-head ``h // (Hq/Hkv)``.
    ``prefix_len`` (this sequence's prefix-LM length) and ``doc_start``
    (``[Lq]``, each row's document start) are the per-sequence and per-row
    values of ``mods.prefix_lens`` / ``mods.doc_starts``; ``keys_allowed``
    (boolean ``[Lq, n]``) is this sequence's block mask, if any.
    Returns fp64 ``[Lq, Hq, D]``; rows with no admissible key are zero.
    """
    mods = mods or ScoreMods()
    Lq, Hq, D = Q.shape
    Hkv, n = K.shape[0], K.shape[1]
    g = Hq // Hkv
    O = np.zeros((Lq, Hq, D), dtype=np.float64)
    if Lq == 0 or n == 0:
        return O
    qp = np.asarray(q_pos, dtype=np.int64)[:, None]
    kp = np.arange(n, dtype=np.int64)[None, :]
    allowed = np.ones((Lq, n), dtype=bool)
    if mods.causal:
        allowed &= (kp <= qp) | (kp < int(prefix_len))
    if mods.window > 0:
        allowed &= (qp - kp) < mods.window
    if doc_start is not None:
        allowed &= kp >= np.asarray(doc_start, dtype=np.int64)[:, None]
    if keys_allowed is not None:
        allowed &= np.asarray(keys_allowed, dtype=bool)
    for h in range(Hq):
        kvh = h // g
        S = (Q[:, h, :] @ K[kvh].T) * float(scale)
        if mods.softcap > 0:
            S = mods.softcap * np.tanh(S / mods.softcap)
        if mods.alibi_slopes is not None:
            S = S + float(mods.alibi_slopes[h]) * (kp - qp)
        S = np.where(allowed, S, -np.inf)
        m = S.max(axis=1, keepdims=True)
        has_key = np.isfinite(m[:, 0])
        m = np.where(np.isfinite(m), m, 0.0)
        P = np.exp(S - m)
        denom = P.sum(axis=1, keepdims=True)
        P = np.divide(P, denom, out=np.zeros_like(P), where=denom > 0)
        # the sum runs over keys some row admits (a key no row admits takes no
        # part, whatever its stored values; elsewhere its weight is exactly 0)
        cols = allowed.any(axis=0)
        O[:, h, :] = np.where(has_key[:, None], P[:, cols] @ V[kvh][cols], 0.0)
    return O


def paged_attention(q, k_pool, v_pool, block_table, context_lens, cu_q_lens, scale, bs,
                    dtype, mods: ScoreMods | None = None, seqs=None):
    """Paged attention over a batch, fp64 ``[sum Lq, Hq, D]``.

    Sequence ``b`` owns query rows ``cu_q_lens[b]:cu_q_lens[b+1]`` (decode:
    one row per sequence) and ``context_lens[b]`` keys found through
    ``block_table[b]``.  ``scale`` is used at the precision it is given in
    (the float32 value the kernel receives, widened).  ``seqs`` restricts the
    work to some sequences; rows of the others are left NaN.
    """
    q64 = bits_to_f64(q, dtype)
    cu = np.asarray(cu_q_lens, dtype=np.int64)
    out = np.full(q64.shape, np.nan, dtype=np.float64)
    B = len(context_lens)
    for b in (range(B) if seqs is None else seqs):
        n = int(context_lens[b])
        r0, r1 = int(cu[b]), int(cu[b + 1])
        Kb, Vb = gather_sequence(k_pool, v_pool, block_table[b], n, bs)
        Kb = bits_to_f64(Kb, dtype)
        Vb = bits_to_f64(Vb, dtype)
        Lq = r1 - r0
        q_pos = np.arange(n - Lq, n)
        prefix = 0 if mods is None or mods.prefix_lens is None else int(mods.prefix_lens[b])
        docs = None if mods is None or mods.doc_starts is None else np.asarray(mods.doc_starts)[r0:r1]
        blocks = None if mods is None or mods.block_mask is None else mods.block_mask.keys_allowed(b, q_pos, n)
        out[r0:r1] = attention_dense(q64[r0:r1], Kb, Vb, float(np.float32(scale)), q_pos, mods, prefix, docs,
                                     blocks)
    return out


def decode_positions(context_lens):
    """cu_q_lens for one query row per sequence (decode)."""
    B = len(context_lens)
    return np.arange(B + 1, dtype=np.int64)


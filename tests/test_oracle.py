"""Pins for the fp64 oracle: it is checked against things other than itself.

* worked examples derived in closed form (tests/golden/worked_examples.json),
* a brute-force loop that walks the block table token by token,
* torch's own scaled_dot_product_attention on an identity block table,
* invariances the pages state: scattered placement and shared blocks do not
  change the result,
* closed forms (one key, equal keys, zero query, constant values, GQA head
  mapping), and
* planted mistakes in the oracle that at least one pin must catch.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import paged as opa
from workloads import build_workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")
NAN = float("nan")


def _load_golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _nanify(x):
    return np.array(json.loads(json.dumps(x).replace("null", "NaN")), dtype=np.float64)


def contiguous_to_pool(K, V, bs):
    """Contiguous per-kv-head K/V ``[Hkv, n, D]`` -> pools with an identity table.

    The pool formats are the storage contract: K ``[NB, Hkv, bs, D]``, V
    ``[NB, Hkv, bs/S, D, S]`` (sub-slabs of ``S = min(bs, 16)`` tokens);
    tail slots are NaN.
    """
    Hkv, n, D = K.shape
    NB = max(1, (n + bs - 1) // bs)
    S = min(bs, 16)
    Kp = np.full((Hkv, NB * bs, D), NAN, np.float32)
    Vp = np.full((Hkv, NB * bs, D), NAN, np.float32)
    Kp[:, :n] = K
    Vp[:, :n] = V
    k_pool = Kp.reshape(Hkv, NB, bs, D).transpose(1, 0, 2, 3).copy()
    v_pool = Vp.reshape(Hkv, NB, bs // S, S, D).transpose(1, 0, 2, 4, 3).copy()
    table = np.arange(NB, dtype=np.int32)[None, :]
    return k_pool, v_pool, table


def run_dense_case(Q, K, V, scale, bs=16, mods=None):
    """Oracle on one sequence given contiguous Q ``[Lq,Hq,D]`` and K/V ``[Hkv,n,D]``."""
    k_pool, v_pool, table = contiguous_to_pool(K, V, bs)
    n = K.shape[1]
    Lq = Q.shape[0]
    return oracle.paged_attention(Q.astype(np.float32), k_pool, v_pool, table, [n], [0, Lq],
                                  np.float32(scale), bs, "f32", mods)


# --------------------------------------------------------------------------------------
# worked examples
# --------------------------------------------------------------------------------------

def check_golden():
    g = _load_golden()
    for name in ["two_token_logistic", "softcap_two_token", "alibi_three_keys", "sliding_window"]:
        c = g[name]
        K = np.array(c["K"], np.float32)[None]
        V = np.array(c["V"], np.float32)[None]
        q = np.array(c["q"], np.float32)[None, None]
        mods = oracle.ScoreMods(window=c.get("window", 0), softcap=c.get("softcap", 0.0),
                                alibi_slopes=np.array([c["alibi_slope"]]) if "alibi_slope" in c else None)
        out = run_dense_case(q, K, V, c["scale"], c["bs"], mods)
        np.testing.assert_allclose(out[0, 0], c["expected"], rtol=0, atol=1e-12, err_msg=name)
    c = g["causal_chunk_bottom_right"]
    out = run_dense_case(np.array(c["Q"], np.float32)[:, None], np.array(c["K"], np.float32)[None],
                         np.array(c["V"], np.float32)[None], c["scale"], c["bs"],
                         oracle.ScoreMods(causal=True))
    np.testing.assert_allclose(out[:, 0], c["expected"], rtol=0, atol=1e-12)
    c = g["paged_scattered_blocks"]
    k_pool = _nanify(c["k_pool"]).astype(np.float32)
    v_pool = _nanify(c["v_pool"]).astype(np.float32)[:, :, None]  # bs <= 16: one [D, bs] sub-slab
    out = oracle.paged_attention(np.array(c["q"], np.float32)[None, None], k_pool, v_pool,
                                 np.array([c["table"]], np.int32), [c["n"]], [0, 1],
                                 np.float32(c["scale"]), c["bs"], "f32")
    np.testing.assert_allclose(out[0, 0], c["expected"], rtol=0, atol=1e-12)
    c = g["kv_append_bs4"]
    shape_k = (c["NB"], c["Hkv"], c["bs"], c["D"])
    shape_v = (c["NB"], c["Hkv"], 1, c["D"], c["bs"])  # bs <= 16: one [D, bs] sub-slab
    kp, vp = oracle.kv_append(np.zeros(shape_k, np.float32), np.zeros(shape_v, np.float32),
                              np.array(c["k_new"], np.float32), np.array(c["v_new"], np.float32),
                              np.array(c["slot_mapping"], np.int32), c["bs"])
    np.testing.assert_array_equal(kp, np.array(c["expected_k_pool"], np.float32))
    np.testing.assert_array_equal(vp[:, :, 0], np.array(c["expected_v_pool"], np.float32))


def test_golden_worked_examples():
    check_golden()


# --------------------------------------------------------------------------------------
# brute force: walk the block table token by token in plain Python
# --------------------------------------------------------------------------------------

def bf16_value(bits):
    """A bfloat16 bit pattern's value from the format itself: 1 sign bit, 8
    exponent bits with bias 127, 7 fraction bits; exponent 0 is subnormal
    (no implicit leading 1), exponent 255 is inf / NaN."""
    bits = int(bits)
    sign = -1.0 if bits & 0x8000 else 1.0
    e = (bits >> 7) & 0xFF
    f = bits & 0x7F
    if e == 0xFF:
        return sign * math.inf if f == 0 else math.nan
    if e == 0:
        return sign * math.ldexp(f, -126 - 7)
    return sign * math.ldexp(128 + f, e - 127 - 7)


_BF16_BY_FORMAT = None


def decode_storage(a, dtype):
    """Stored values -> fp64 without the oracle's routine: bf16 through
    :func:`bf16_value`, fp32 by numpy's exact widening."""
    global _BF16_BY_FORMAT
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if _BF16_BY_FORMAT is None:
        _BF16_BY_FORMAT = np.array([bf16_value(i) for i in range(1 << 16)], dtype=np.float64)
    return _BF16_BY_FORMAT[np.asarray(a, dtype=np.uint16).astype(np.int64)]


# (bit pattern, value) written out by hand from the bfloat16 format
BF16_HAND = [
    (0x3F80, 1.0), (0xBF80, -1.0), (0xC040, -3.0), (0x3F81, 1.0078125), (0x4049, 3.140625),
    (0x3F00, 0.5), (0x4300, 128.0), (0x0080, 2.0 ** -126), (0x0001, 2.0 ** -133), (0x007F, 127 * 2.0 ** -133),
    (0x7F7F, (2 - 2.0 ** -7) * 2.0 ** 127), (0x0000, 0.0), (0x8000, -0.0), (0x7F80, math.inf),
    (0xFF80, -math.inf),
]


def check_bf16_decode():
    bits = np.array([b for b, _ in BF16_HAND], dtype=np.uint16)
    got = opa.bits_to_f64(bits, "bf16")
    for (b, v), x in zip(BF16_HAND, got.tolist()):
        assert x == v and math.copysign(1.0, x) == math.copysign(1.0, v), (hex(b), x, v)
    nan = opa.bits_to_f64(np.array([0x7FC0, 0xFFC1, 0x7F81], dtype=np.uint16), "bf16")
    assert np.all(np.isnan(nan))


def test_bf16_decode_hand_values():
    check_bf16_decode()


def test_bf16_decode_every_pattern():
    """All 65,536 patterns: the oracle's decode equals the format's definition
    and torch's own bfloat16 -> float64 conversion, sign of zero and NaNs
    included."""
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = opa.bits_to_f64(allbits, "bf16")
    by_format = decode_storage(allbits, "bf16")
    by_torch = torch.from_numpy(allbits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    for ref in (by_format, by_torch):
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan)
        assert np.array_equal(got[~nan], ref[~nan])
        assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def brute_force(w, mods, block_dense=None, q_block=1, kv_block=1):
    """Two-pass softmax with math.exp, reading each key through its table
    entry; stored values are decoded by :func:`decode_storage`, not by the
    oracle.  ``block_dense[b][p // q_block][j // kv_block]`` (booleans, not the
    packed bitmap) admits key j for the query at position p."""
    q = decode_storage(w.q, w.dtype)
    kp = decode_storage(w.k_pool, w.dtype)
    vp = decode_storage(w.v_pool, w.dtype)
    S = min(w.bs, 16)  # V: token o of a block is column o % S of sub-slab o // S
    g = w.Hq // w.Hkv
    out = np.zeros(q.shape)
    for b in range(w.B):
        n = int(w.context_lens[b])
        r0, r1 = int(w.cu_q_lens[b]), int(w.cu_q_lens[b + 1])
        for r in range(r0, r1):
            pos = n - (r1 - r0) + (r - r0)
            for h in range(w.Hq):
                c = h // g
                scores = []
                prefix = 0 if mods.prefix_lens is None else int(mods.prefix_lens[b])
                doc = 0 if mods.doc_starts is None else int(mods.doc_starts[r])
                for j in range(n):
                    if mods.causal and j > pos and j >= prefix:
                        continue
                    if mods.window and pos - j >= mods.window:
                        continue
                    if j < doc:
                        continue
                    if block_dense is not None and not block_dense[b][pos // q_block][j // kv_block]:
                        continue
                    blk = int(w.block_table[b][j // w.bs])
                    off = j % w.bs
                    s = 0.0
                    for d in range(w.D):
                        s += q[r, h, d] * kp[blk, c, off, d]
                    s *= float(w.scale)
                    if mods.softcap:
                        s = mods.softcap * math.tanh(s / mods.softcap)
                    if mods.alibi_slopes is not None:
                        s += float(mods.alibi_slopes[h]) * (j - pos)
                    scores.append((j, blk, off, s))
                if not scores:
                    continue
                m = max(s for _, _, _, s in scores)
                den = sum(math.exp(s - m) for _, _, _, s in scores)
                for d in range(w.D):
                    acc = 0.0
                    for _, blk, off, s in scores:
                        acc += math.exp(s - m) * vp[blk, c, off // S, d, off % S]
                    out[r, h, d] = acc / den
    return out


def _tiny(kind, seed, bs=4, dtype="f32", ctx=(13, 40), q_lens=None, Hq=4, Hkv=2, D=8, causal=False):
    return build_workload(name="tiny", seed=seed, kind=kind, dtype=dtype, Hq=Hq, Hkv=Hkv, D=D, bs=bs,
                          context_lens=list(ctx), q_lens=q_lens, causal=causal, threads=1)


def check_brute_force_large_pages(bs):
    """Pages of several V sub-slabs (bs 32, 48-token contexts end inside one)."""
    w = _tiny("prefill", 12, bs=bs, ctx=(45, 77), q_lens=[3, 9], causal=True)
    mods = oracle.ScoreMods(causal=True)
    np.testing.assert_allclose(_run(w, mods), brute_force(w, mods), rtol=0, atol=1e-12)


@pytest.mark.parametrize("bs", [32, 64])
def test_brute_force_large_pages(bs):
    check_brute_force_large_pages(bs)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("kind", ["decode", "prefill"])
def test_brute_force_loops(kind, dtype):
    w = _tiny(kind, 11, dtype=dtype, q_lens=None if kind == "decode" else [5, 7], causal=kind == "prefill")
    mods = oracle.ScoreMods(causal=w.causal)
    got = oracle.paged_attention(w.q, w.k_pool, w.v_pool, w.block_table, w.context_lens, w.cu_q_lens,
                                 w.scale, w.bs, w.dtype, mods)
    np.testing.assert_allclose(got, brute_force(w, mods), rtol=0, atol=1e-12)


def test_brute_force_with_mods():
    w = _tiny("prefill", 12, ctx=(9, 33), q_lens=[4, 6], causal=True)
    mods = oracle.ScoreMods(causal=True, window=5, softcap=0.7,
                            alibi_slopes=np.array([0.5, 0.25, 0.125, 0.0625]))
    got = oracle.paged_attention(w.q, w.k_pool, w.v_pool, w.block_table, w.context_lens, w.cu_q_lens,
                                 w.scale, w.bs, w.dtype, mods)
    np.testing.assert_allclose(got, brute_force(w, mods), rtol=0, atol=1e-12)


def test_brute_force_with_prefix_and_documents():
    w = _tiny("prefill", 13, ctx=(11, 30), q_lens=[6, 9], causal=True)
    mods = oracle.ScoreMods(causal=True, window=7, prefix_lens=np.array([8, 25]),
                            doc_starts=np.array([0, 0, 3, 3, 6, 6, 0, 12, 12, 21, 21, 21, 25, 25, 27]))
    got = _run(w, mods)
    np.testing.assert_allclose(got, brute_force(w, mods), rtol=0, atol=1e-12)


def test_prefix_lm_limits():
    """prefix 0 is plain causal; a prefix covering the context is no mask."""
    w = _tiny("prefill", 14, ctx=(17, 26), q_lens=[7, 10], causal=True)
    causal = _run(w, oracle.ScoreMods(causal=True))
    full = _run(w, oracle.ScoreMods(causal=False))
    np.testing.assert_allclose(_run(w, oracle.ScoreMods(causal=True, prefix_lens=np.array([0, 0]))), causal,
                               rtol=0, atol=0)
    np.testing.assert_allclose(_run(w, oracle.ScoreMods(causal=True, prefix_lens=w.context_lens)), full,
                               rtol=0, atol=0)


def test_document_rows_equal_the_document_alone():
    """A packed sequence of documents [0, a) and [a, n): a row of the second
    document with doc_start a gives what that document alone gives, its keys
    re-based to position 0 (causal holds relative positions)."""
    rng = np.random.default_rng(15)
    n, a, Lq, Hq, Hkv, D = 29, 12, 9, 4, 2, 8
    Q = rng.standard_normal((Lq, Hq, D))
    K = rng.standard_normal((Hkv, n, D))
    V = rng.standard_normal((Hkv, n, D))
    q_pos = np.arange(n - Lq, n)
    mods = oracle.ScoreMods(causal=True)
    packed = opa.attention_dense(Q, K, V, 0.3, q_pos, mods, doc_start=np.full(Lq, a))
    alone = opa.attention_dense(Q, K[:, a:], V[:, a:], 0.3, q_pos - a, mods)
    np.testing.assert_allclose(packed, alone, rtol=0, atol=1e-13)
    # doc_start 0 everywhere is no document mask
    np.testing.assert_allclose(opa.attention_dense(Q, K, V, 0.3, q_pos, mods, doc_start=np.zeros(Lq, int)),
                               opa.attention_dense(Q, K, V, 0.3, q_pos, mods), rtol=0, atol=0)


# --------------------------------------------------------------------------------------
# library special case: identity table == torch SDPA (fp64, CPU)
# --------------------------------------------------------------------------------------

def check_sdpa(n=37, Lq=9, Hq=8, Hkv=2, D=16, bs=16, alibi=False, seed=3):
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((Lq, Hq, D)).astype(np.float32)
    K = rng.standard_normal((Hkv, n, D)).astype(np.float32)
    V = rng.standard_normal((Hkv, n, D)).astype(np.float32)
    scale = np.float32(1 / math.sqrt(D))
    slopes = 2.0 ** -np.arange(1, Hq + 1) if alibi else None
    got = run_dense_case(Q, K, V, scale, bs, oracle.ScoreMods(causal=True, alibi_slopes=slopes))
    qt = torch.from_numpy(Q.astype(np.float64)).permute(1, 0, 2)[None]  # [1, Hq, Lq, D]
    kt = torch.from_numpy(K.astype(np.float64))[None]
    vt = torch.from_numpy(V.astype(np.float64))[None]
    pos = torch.arange(n - Lq, n)[:, None]
    kv = torch.arange(n)[None, :]
    allowed = kv <= pos
    if alibi:
        bias = torch.from_numpy(slopes)[:, None, None] * (kv - pos).to(torch.float64)[None]
        mask = torch.where(allowed[None], bias, torch.tensor(-math.inf, dtype=torch.float64))[None]
    else:
        mask = allowed
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask,
                                                           scale=float(scale), enable_gqa=True)
    ref = ref[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_identity_table_matches_torch_sdpa():
    check_sdpa()
    check_sdpa(n=1, Lq=1, Hq=4, Hkv=4, D=8, bs=16)
    check_sdpa(n=64, Lq=1, Hq=8, Hkv=1, D=32, bs=32)


def test_alibi_matches_torch_sdpa_bias():
    check_sdpa(alibi=True)


# --------------------------------------------------------------------------------------
# invariances stated on the pages
# --------------------------------------------------------------------------------------

def _run(w, mods=None, **over):
    a = dict(q=w.q, k_pool=w.k_pool, v_pool=w.v_pool, block_table=w.block_table,
             context_lens=w.context_lens, cu_q_lens=w.cu_q_lens, scale=w.scale, bs=w.bs, dtype=w.dtype)
    a.update(over)
    return oracle.paged_attention(mods=mods or oracle.ScoreMods(causal=w.causal), **a)


def check_permutation_invariance(dtype="bf16"):
    w = _tiny("prefill", 21, bs=16, dtype=dtype, ctx=(50, 100), q_lens=[3, 17], causal=True)
    base = _run(w)
    perm = np.random.default_rng(5).permutation(w.NB)
    kp = np.empty_like(w.k_pool)
    vp = np.empty_like(w.v_pool)
    kp[perm] = w.k_pool
    vp[perm] = w.v_pool
    table = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], -1).astype(np.int32)
    got = _run(w, k_pool=kp, v_pool=vp, block_table=table)
    assert np.array_equal(got, base)


def test_block_permutation_invariance():
    check_permutation_invariance("bf16")
    check_permutation_invariance("f32")


def test_shared_prefix_equals_private_copies():
    w = build_workload(name="shared", seed=4, kind="decode", dtype="bf16", Hq=8, Hkv=2, D=32, bs=16,
                       context_lens=[80, 80, 80], shared_prefix_blocks=3, threads=1)
    base = _run(w)
    # give every sequence private copies of the shared blocks
    S = 3
    extra = w.B * S
    kp = np.concatenate([w.k_pool, np.zeros((extra,) + w.k_pool.shape[1:], w.k_pool.dtype)])
    vp = np.concatenate([w.v_pool, np.zeros((extra,) + w.v_pool.shape[1:], w.v_pool.dtype)])
    table = w.block_table.copy()
    nxt = w.NB
    for b in range(w.B):
        for j in range(S):
            kp[nxt] = w.k_pool[w.block_table[b, j]]
            vp[nxt] = w.v_pool[w.block_table[b, j]]
            table[b, j] = nxt
            nxt += 1
    assert len({tuple(r[:S]) for r in table}) == w.B
    assert np.array_equal(_run(w, k_pool=kp, v_pool=vp, block_table=table), base)


# --------------------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------------------

def test_one_token_context_returns_v_row():
    w = _tiny("decode", 31, bs=16, dtype="bf16", ctx=(1, 1))
    got = _run(w)
    for b in range(w.B):
        pb = w.block_table[b, 0]
        v = opa.bits_to_f64(w.v_pool[pb, :, 0, :, 0], "bf16")  # token 0: sub-slab 0, column 0 -> [Hkv, D]
        assert np.array_equal(got[b], np.repeat(v, w.Hq // w.Hkv, axis=0))


def test_equal_tokens_and_zero_query_and_constant_v():
    rng = np.random.default_rng(9)
    n, D, Hq, Hkv = 29, 8, 4, 2
    k = rng.standard_normal(D).astype(np.float32)
    v = rng.standard_normal(D).astype(np.float32)
    Q = rng.standard_normal((1, Hq, D)).astype(np.float32)
    K = np.broadcast_to(k, (Hkv, n, D)).copy()
    V = np.broadcast_to(v, (Hkv, n, D)).copy()
    out = run_dense_case(Q, K, V, 0.3)
    np.testing.assert_allclose(out[0], np.broadcast_to(v, (Hq, D)), rtol=0, atol=1e-12)
    # zero query (or zero scale): plain mean of the value rows
    K = rng.standard_normal((Hkv, n, D)).astype(np.float32)
    V = rng.standard_normal((Hkv, n, D)).astype(np.float32)
    out = run_dense_case(np.zeros((1, Hq, D), np.float32), K, V, 0.3)
    mean = V.astype(np.float64).mean(axis=1)
    np.testing.assert_allclose(out[0], np.repeat(mean, Hq // Hkv, axis=0), rtol=0, atol=1e-12)
    out = run_dense_case(Q, K, V, 0.0)
    np.testing.assert_allclose(out[0], np.repeat(mean, Hq // Hkv, axis=0), rtol=0, atol=1e-12)
    # constant value rows: that constant whatever the scores
    V = np.full((Hkv, n, D), 0.75, np.float32)
    out = run_dense_case(Q, K, V, 5.0)
    np.testing.assert_allclose(out, 0.75, rtol=0, atol=1e-12)


def test_gqa_head_mapping_consecutive_groups():
    rng = np.random.default_rng(2)
    n, D, Hq, Hkv = 20, 4, 8, 2
    K = rng.standard_normal((Hkv, n, D)).astype(np.float32)
    V = np.stack([np.full((n, D), c + 1.0, np.float32) for c in range(Hkv)])
    out = run_dense_case(rng.standard_normal((1, Hq, D)).astype(np.float32), K, V, 0.5)
    for h in range(Hq):
        np.testing.assert_allclose(out[0, h], h // (Hq // Hkv) + 1.0, rtol=0, atol=1e-12)


def test_chunk_rows_equal_truncated_decode():
    w = _tiny("prefill", 41, bs=16, ctx=(70,), q_lens=[9], causal=True)
    chunk = _run(w)
    n = int(w.context_lens[0])
    for i in range(9):
        pos = n - 9 + i
        dec = _run(w, q=w.q[i:i + 1], context_lens=np.array([pos + 1], np.int32), cu_q_lens=np.array([0, 1]),
                   mods=oracle.ScoreMods())
        np.testing.assert_allclose(chunk[i], dec[0], rtol=0, atol=1e-12)


def test_window_equals_truncated_context():
    rng = np.random.default_rng(8)
    n, D, W = 50, 8, 7
    Q = rng.standard_normal((1, 2, D)).astype(np.float32)
    K = rng.standard_normal((2, n, D)).astype(np.float32)
    V = rng.standard_normal((2, n, D)).astype(np.float32)
    win = run_dense_case(Q, K, V, 0.4, mods=oracle.ScoreMods(window=W))
    ref = run_dense_case(Q, K[:, n - W:], V[:, n - W:], 0.4)
    np.testing.assert_allclose(win, ref, rtol=0, atol=1e-12)


def test_large_softcap_is_identity():
    rng = np.random.default_rng(6)
    Q = rng.standard_normal((1, 2, 8)).astype(np.float32)
    K = rng.standard_normal((2, 30, 8)).astype(np.float32)
    V = rng.standard_normal((2, 30, 8)).astype(np.float32)
    a = run_dense_case(Q, K, V, 0.3, mods=oracle.ScoreMods(softcap=1e7))
    b = run_dense_case(Q, K, V, 0.3)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-9)


def test_empty_context_outputs_zero():
    w = _tiny("decode", 51, bs=16, ctx=(0, 5))
    out = _run(w)
    assert np.all(out[0] == 0.0) and np.all(np.isfinite(out[1]))


def test_poisoned_slots_never_read():
    for kind in ["decode", "prefill"]:
        w = _tiny(kind, 61, bs=16, ctx=(33, 47), q_lens=None if kind == "decode" else [4, 4],
                  causal=kind == "prefill")
        assert np.isnan(opa.bits_to_f64(w.k_pool, "f32")).any()
        assert np.all(np.isfinite(_run(w)))


# --------------------------------------------------------------------------------------
# kv_append
# --------------------------------------------------------------------------------------

def test_kv_append_roundtrip_through_block_table():
    w = build_workload(name="app", seed=7, kind="decode", dtype="bf16", Hq=4, Hkv=2, D=16, bs=16,
                       context_lens=[40, 17], append_lens=[20, 17], threads=1)
    kp, vp = oracle.kv_append(w.k_pool, w.v_pool, w.k_new, w.v_new, w.slot_mapping, w.bs)
    t = 0
    for b in range(w.B):
        n = int(w.context_lens[b])
        K, V = oracle.gather_sequence(kp, vp, w.block_table[b], n, w.bs)
        for p in range(n - 20 if b == 0 else 0, n):
            assert np.array_equal(K[:, p], w.k_new[t]) and np.array_equal(V[:, p], w.v_new[t])
            t += 1
        K0, _ = oracle.gather_sequence(w.k_pool, w.v_pool, w.block_table[b], n, w.bs)
        keep = n - (20 if b == 0 else 17)
        assert np.array_equal(K[:, :keep], K0[:, :keep])
    changed = np.nonzero((kp != w.k_pool).any(axis=(1, 2, 3)))[0]
    assert set(changed.tolist()) <= set(w.block_table[w.block_table >= 0].tolist())


def test_v_sub_slab_layout_by_hand():
    """V of a 48-token block sits in three [D, 16] sub-slabs: token o of the
    block is column o % 16 of sub-slab o // 16 (indices written out by hand),
    K stays token-major, and gather reads the tokens back in logical order."""
    bs, D = 48, 3
    kp = np.zeros((2, 1, bs, D), np.float32)
    vp = np.zeros((2, 1, 3, D, 16), np.float32)
    slots = np.array([48 + 0, 48 + 15, 48 + 16, 48 + 33, 48 + 47], np.int32)  # block 1
    vals = np.arange(1, 6, dtype=np.float32)
    new = (vals[:, None, None] * np.array([1.0, 10.0, 100.0], np.float32)).astype(np.float32)
    kp2, vp2 = oracle.kv_append(kp, vp, new, new, slots, bs)
    expect = {(0, 0): 1, (0, 15): 2, (1, 0): 3, (2, 1): 4, (2, 15): 5}
    for (sub, col), v in expect.items():
        np.testing.assert_array_equal(vp2[1, 0, sub, :, col], [v, 10 * v, 100 * v])
    assert np.count_nonzero(vp2) == 3 * len(expect)
    np.testing.assert_array_equal(kp2[1, 0, [0, 15, 16, 33, 47], 0], vals)
    K, V = oracle.gather_sequence(kp2, vp2, np.array([1]), bs, bs)
    for o, v in zip([0, 15, 16, 33, 47], vals):
        np.testing.assert_array_equal(V[0, o], [v, 10 * v, 100 * v])
        np.testing.assert_array_equal(K[0, o], [v, 10 * v, 100 * v])
    with pytest.raises(ValueError):  # a [D, bs] V pool is not the format for bs > 16
        oracle.kv_append(kp, np.zeros((2, 1, D, bs), np.float32), new, new, slots, bs)


def test_kv_append_rejects_duplicates_and_skips_negative():
    z = np.zeros((2, 1, 4, 2), np.float32)
    zv = np.zeros((2, 1, 1, 2, 4), np.float32)
    new = np.ones((2, 1, 2), np.float32)
    with pytest.raises(ValueError):
        oracle.kv_append(z, zv, new, new, np.array([3, 3]), 4)
    kp, vp = oracle.kv_append(z, zv, new, new, np.array([-1, -7]), 4)
    assert not kp.any() and not vp.any()


# --------------------------------------------------------------------------------------
# block masks (FlexAttention-style block sparsity)
# --------------------------------------------------------------------------------------

def pack_block_mask(dense, q_block, kv_block):
    """Dense booleans [B, q_blocks, kv_blocks] -> oracle.BlockMask, packed with
    numpy's little-endian bit order (bit i of the little-endian uint32 word is
    block 32 * word + i)."""
    dense = np.asarray(dense, dtype=bool)
    B, QBn, KBn = dense.shape
    words = (KBn + 31) // 32
    padded = np.zeros((B * QBn, words * 32), dtype=bool)
    padded[:, :KBn] = dense.reshape(B * QBn, KBn)
    packed = np.packbits(padded, axis=1, bitorder="little").view("<u4")
    return oracle.BlockMask(bits=np.ascontiguousarray(packed.astype(np.uint32)), q_block=q_block,
                            kv_block=kv_block, rows_per_seq=QBn)


def _random_blocks(rng, B, n_max, q_block, kv_block, density=0.5):
    QBn = (n_max + q_block - 1) // q_block
    KBn = (n_max + kv_block - 1) // kv_block
    return rng.random((B, QBn, KBn)) < density


def check_block_mask_equals_removing_keys(kind="prefill", q_block=4, kv_block=8, seed=41):
    """Non-causal attention under a block mask equals attention over only the
    admitted keys, gathered row by row (no positional mod, so removing keys is
    all a mask does).  The bitmap is packed by numpy, the keys picked from the
    dense booleans."""
    rng = np.random.default_rng(seed)
    w = _tiny(kind, seed, bs=4, ctx=(37, 50), q_lens=None if kind == "decode" else [9, 13])
    dense = _random_blocks(rng, w.B, int(w.context_lens.max()), q_block, kv_block, 0.6)
    bm = pack_block_mask(dense, q_block, kv_block)
    got = _run(w, oracle.ScoreMods(block_mask=bm))
    kp, vp = w.k_pool, w.v_pool
    for b in range(w.B):
        n = int(w.context_lens[b])
        r0, r1 = int(w.cu_q_lens[b]), int(w.cu_q_lens[b + 1])
        K, V = opa.gather_sequence(kp, vp, w.block_table[b], n, w.bs)
        K, V = opa.bits_to_f64(K, w.dtype), opa.bits_to_f64(V, w.dtype)
        for r in range(r0, r1):
            pos = n - (r1 - r0) + (r - r0)
            keep = [j for j in range(n) if dense[b][pos // q_block][j // kv_block]]
            Q = opa.bits_to_f64(w.q[r:r + 1], w.dtype)
            ref = opa.attention_dense(Q, K[:, keep], V[:, keep], float(np.float32(w.scale)), [len(keep)])
            np.testing.assert_allclose(got[r:r + 1], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("kind", ["decode", "prefill"])
@pytest.mark.parametrize("q_block,kv_block", [(1, 4), (4, 8), (8, 32)])
def test_block_mask_equals_removing_keys(kind, q_block, kv_block):
    check_block_mask_equals_removing_keys(kind, q_block, kv_block)


def test_block_mask_brute_force_with_causal_and_window():
    w = _tiny("prefill", 43, bs=4, ctx=(29, 46), q_lens=[11, 17], causal=True)
    dense = _random_blocks(np.random.default_rng(43), w.B, 46, 4, 8, 0.5)
    mods = oracle.ScoreMods(causal=True, window=19, block_mask=pack_block_mask(dense, 4, 8))
    np.testing.assert_allclose(_run(w, mods), brute_force(w, mods, dense, 4, 8), rtol=0, atol=1e-12)


def test_block_mask_all_ones_and_block_causal():
    """Every bit set is no mask at all; with q_block == kv_block, the
    block-causal mask (key block <= query block) under causal masking is
    causal masking alone (it removes only keys causal removes anyway)."""
    w = _tiny("prefill", 44, bs=4, ctx=(33, 40), q_lens=[10, 12], causal=True)
    plain = _run(w, oracle.ScoreMods(causal=True))
    ones = np.ones((w.B, 40, 40), dtype=bool)
    assert np.array_equal(_run(w, oracle.ScoreMods(causal=True, block_mask=pack_block_mask(ones, 1, 1))), plain)
    qb = 8
    nb = (40 + qb - 1) // qb
    tri = np.broadcast_to(np.tril(np.ones((nb, nb), dtype=bool)), (w.B, nb, nb))
    got = _run(w, oracle.ScoreMods(causal=True, block_mask=pack_block_mask(tri, qb, qb)))
    assert np.array_equal(got, plain)
    # and without causal masking the block-causal mask admits whole diagonal blocks
    nc = _run(w, oracle.ScoreMods(causal=False, block_mask=pack_block_mask(tri, qb, qb)))
    assert not np.allclose(nc, plain)


def test_block_mask_row_without_blocks_is_zero():
    w = _tiny("decode", 45, bs=4, ctx=(20, 9))
    dense = np.ones((w.B, 1, 5), dtype=bool)
    dense[1] = False
    got = _run(w, oracle.ScoreMods(block_mask=pack_block_mask(dense, 64, 4)))
    assert np.all(got[1] == 0) and np.all(np.isfinite(got[0])) and np.any(got[0] != 0)


# --------------------------------------------------------------------------------------
# planted mistakes: each must make at least one pin fail
# --------------------------------------------------------------------------------------

def _all_pins():
    check_bf16_decode()
    check_golden()
    check_sdpa()
    check_permutation_invariance("f32")
    test_gqa_head_mapping_consecutive_groups()
    test_chunk_rows_equal_truncated_decode()
    w = _tiny("prefill", 11, q_lens=[5, 7], causal=True)
    mods = oracle.ScoreMods(causal=True)
    np.testing.assert_allclose(_run(w, mods), brute_force(w, mods), rtol=0, atol=1e-12)
    test_brute_force_with_prefix_and_documents()
    check_brute_force_large_pages(32)
    wb = _tiny("prefill", 11, dtype="bf16", q_lens=[5, 7], causal=True)
    np.testing.assert_allclose(_run(wb, mods), brute_force(wb, mods), rtol=0, atol=1e-12)
    check_block_mask_equals_removing_keys("prefill", 4, 8)


def _mutant_gather_v_not_transposed(k_pool, v_pool, table_row, n, bs):
    nb = (n + bs - 1) // bs
    phys = np.asarray(table_row[:nb], dtype=np.int64)
    Hkv, D = k_pool.shape[1], k_pool.shape[3]
    K = k_pool[phys].transpose(1, 0, 2, 3).reshape(Hkv, nb * bs, D)[:, :n]
    V = v_pool[phys].transpose(1, 0, 2, 3, 4).reshape(Hkv, nb * bs, D)[:, :n]  # wrong: sub-slabs are [D, S]
    return K, V


def _mutant_gather_v_whole_slab(k_pool, v_pool, table_row, n, bs):
    nb = (n + bs - 1) // bs
    phys = np.asarray(table_row[:nb], dtype=np.int64)
    Hkv, D = k_pool.shape[1], k_pool.shape[3]
    K = k_pool[phys].transpose(1, 0, 2, 3).reshape(Hkv, nb * bs, D)[:, :n]
    # wrong: reads the block's V as one [D, bs] slab instead of [D, 16] sub-slabs
    V = v_pool[phys].reshape(nb, Hkv, D, bs).transpose(1, 0, 3, 2).reshape(Hkv, nb * bs, D)[:, :n]
    return K, V


def _mutant_gather_ignores_table(k_pool, v_pool, table_row, n, bs):
    return opa.__dict__["_orig_gather"](k_pool, v_pool, np.arange(len(table_row)), n, bs)


def _mutant_bf16_low_bit_dropped(a, dtype):
    """bf16 decode that loses the last fraction bit (a plausible masking slip)."""
    if dtype == "bf16":
        a = np.asarray(a, dtype=np.uint16) & np.uint16(0xFFFE)
    return opa.__dict__["_orig_bits"](a, dtype)


def _mutant_block_rows_by_chunk_row(self, b, q_pos, n):
    """Block-mask rows indexed by the row's place in the chunk, not its position."""
    q_pos = np.asarray(q_pos, dtype=np.int64)
    return opa.__dict__["_orig_keys_allowed"](self, b, q_pos - q_pos[0], n)


def _mutant_block_bits_msb_first(self, b, q_pos, n):
    """Bits of each word read from the most significant end."""
    q_pos = np.asarray(q_pos, dtype=np.int64)
    rows = b * self.rows_per_seq + q_pos // self.q_block
    kb = np.arange(n, dtype=np.int64) // self.kv_block
    words = np.asarray(self.bits, dtype=np.uint64)[rows][:, kb // 32]
    return ((words >> (31 - kb % 32).astype(np.uint64)[None, :]) & np.uint64(1)).astype(bool)


def _make_attention_mutant(kind):
    orig = opa.__dict__["_orig_attention"]

    def mutant(Q, K, V, scale, q_pos, mods=None, prefix_len=0, doc_start=None, keys_allowed=None):
        mods = mods or oracle.ScoreMods()
        if kind == "no_scale":
            return orig(Q, K, V, 1.0, q_pos, mods, prefix_len, doc_start, keys_allowed)
        if kind == "top_left_causal":
            return orig(Q, K, V, scale, np.arange(len(q_pos)), mods, prefix_len, doc_start, keys_allowed)
        if kind == "gqa_modulo":
            Hq, Hkv = Q.shape[1], K.shape[0]
            idx = np.arange(Hq) % Hkv  # wrong grouping
            Kx = K[idx]
            Vx = V[idx]
            return orig(Q, Kx, Vx, scale, q_pos, mods, prefix_len, doc_start, keys_allowed)
        if kind == "no_max_sub_sign":
            return orig(Q, K, V, -scale, q_pos, mods, prefix_len, doc_start, keys_allowed)
        if kind == "prefix_inclusive":  # key == prefix wrongly visible
            return orig(Q, K, V, scale, q_pos, mods, prefix_len + 1 if prefix_len else 0, doc_start, keys_allowed)
        if kind == "doc_exclusive":  # the document's first key wrongly hidden
            return orig(Q, K, V, scale, q_pos, mods, prefix_len, None if doc_start is None else doc_start + 1,
                        keys_allowed)
        raise AssertionError(kind)

    return mutant


@pytest.mark.parametrize("mutant", ["bf16_low_bit", "block_rows_by_chunk_row", "block_bits_msb_first", "v_layout", "v_whole_slab", "ignore_table", "no_scale", "top_left_causal",
                                    "gqa_modulo", "sign", "prefix_inclusive", "doc_exclusive"])
def test_planted_mistakes_are_caught(monkeypatch, mutant):
    monkeypatch.setitem(opa.__dict__, "_orig_gather", opa.gather_sequence)
    monkeypatch.setitem(opa.__dict__, "_orig_attention", opa.attention_dense)
    monkeypatch.setitem(opa.__dict__, "_orig_bits", opa.bits_to_f64)
    monkeypatch.setitem(opa.__dict__, "_orig_keys_allowed", opa.BlockMask.keys_allowed)
    if mutant == "bf16_low_bit":
        monkeypatch.setattr(opa, "bits_to_f64", _mutant_bf16_low_bit_dropped)
    elif mutant == "block_rows_by_chunk_row":
        monkeypatch.setattr(opa.BlockMask, "keys_allowed", _mutant_block_rows_by_chunk_row)
    elif mutant == "block_bits_msb_first":
        monkeypatch.setattr(opa.BlockMask, "keys_allowed", _mutant_block_bits_msb_first)
    elif mutant == "v_layout":
        monkeypatch.setattr(opa, "gather_sequence", _mutant_gather_v_not_transposed)
    elif mutant == "v_whole_slab":
        monkeypatch.setattr(opa, "gather_sequence", _mutant_gather_v_whole_slab)
    elif mutant == "ignore_table":
        monkeypatch.setattr(opa, "gather_sequence", _mutant_gather_ignores_table)
    else:
        kind = {"no_scale": "no_scale", "top_left_causal": "top_left_causal",
                "gqa_modulo": "gqa_modulo", "sign": "no_max_sub_sign",
                "prefix_inclusive": "prefix_inclusive", "doc_exclusive": "doc_exclusive"}[mutant]
        monkeypatch.setattr(opa, "attention_dense", _make_attention_mutant(kind))
    with pytest.raises(AssertionError):
        _all_pins()

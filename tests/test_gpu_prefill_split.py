"""GPU parity of the key-split prefill (paged_attn_prefill_split) against the
fp64 oracle.

Each key range computes exact attention over its keys as a normalised fp32
output and its log-sum-exp; the merge weights the ranges by those
exponentials, which is the softmax over the whole range.  The bf16 tolerance
of the other prefill tests applies (2e-2 max-abs).  Calls that do not split
(key_split -1, a single range, a grid that fills the device, a block mask)
must equal paged_attn_prefill bit for bit.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle.paged import bits_to_f64
from paged_kv_cache_attn_amd import binding
from workloads import named_workload
from workloads.device import to_numpy_bits, upload

from tests.test_gpu_parity import assert_close, gpu_prefill, oracle_out, small

pytestmark = pytest.mark.gpu


def split_prefill(lib, w, key_split=0, max_ctx=None, causal=True, workspace=None, **mods):
    t = upload(w)
    if len(w.slot_mapping):
        lib.kv_append(t["k_new"], t["v_new"], t["k_cache"], t["v_cache"], t["slot_mapping"])
    out = torch.empty_like(t["q"])
    lib.paged_attn_prefill(out, t["q"], t["cu_q_lens"], t["k_cache"], t["v_cache"], t["block_tables"],
                           t["context_lens"], w.scale, w.max_q_len, causal,
                           max_context_len=int(w.context_lens.max()) if max_ctx is None else max_ctx,
                           key_split=key_split, workspace=workspace, **mods)
    torch.cuda.synchronize()
    return to_numpy_bits(out)


def splits(w, key_split=0, max_ctx=None):
    """Bytes of workspace the library asks for (0: it does not split)."""
    return binding.prefill_workspace_size(w.B, int(w.q_lens.sum()), w.max_q_len, w.Hq, w.Hkv, w.D,
                                          int(w.context_lens.max()) if max_ctx is None else max_ctx, key_split)


def ragged(seed=300, **kw):
    # a fresh prompt, a chunk after a long context, a short sequence whose
    # later key ranges are empty, and a single row
    a = dict(ctx=(150, 1300, 200, 33), q_lens=[150, 170, 90, 1], Hq=8, Hkv=2, causal=True)
    a.update(kw)
    return small("prefill", seed=seed, **a)


def test_head_shard_of_the_chunked_prefill(gpu_lib):
    """One GPU's share of an 8-way head split (4 sequences x 512 rows after
    1,536 tokens, 4/1 heads): 64 work-groups, so the library splits the keys
    (4 ranges of 512 keys on 256 compute units)."""
    w = named_workload("chunked_prefill_bf16", tp=8)
    assert splits(w) > 0
    assert_close(split_prefill(gpu_lib, w), oracle_out(w, causal=True), "bf16")


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("key_split", [64, 128, 320, 1024])
def test_explicit_key_ranges(gpu_lib, key_split, causal):
    w = ragged(causal=causal)
    assert splits(w, key_split) > 0
    assert_close(split_prefill(gpu_lib, w, key_split, causal=causal), oracle_out(w, causal=causal), "bf16")


@pytest.mark.parametrize("mods", ["window_alibi", "softcap_docs", "prefix_lm", "zero_scale", "negative_scale"])
def test_score_mods_over_key_ranges(gpu_lib, mods):
    w = ragged(seed=310)
    kw, om = {}, {}
    if mods == "window_alibi":
        slopes = (2.0 ** -np.arange(1, w.Hq + 1) * 0.5).astype(np.float32)
        kw = {"window": 300, "alibi_slopes": torch.from_numpy(slopes).cuda()}
        om = {"window": 300, "alibi_slopes": slopes.astype(np.float64)}
    elif mods == "softcap_docs":
        docs = np.concatenate([np.full(int(q), max(0, int(n) - int(q) - 100 * k)) for k, (q, n) in
                               enumerate(zip(w.q_lens, w.context_lens))]).astype(np.int32)
        kw = {"softcap": 0.5, "doc_starts": torch.from_numpy(docs).cuda()}
        om = {"softcap": 0.5, "doc_starts": docs}
    elif mods == "prefix_lm":
        pl = np.array([100, 1200, 150, 10], np.int32)
        kw = {"prefix_lens": torch.from_numpy(pl).cuda()}
        om = {"prefix_lens": pl}
    else:
        w.scale = 0.0 if mods == "zero_scale" else -0.06
    ref = oracle_out(w, oracle.ScoreMods(causal=True, **om))
    assert_close(split_prefill(gpu_lib, w, 128, **kw), ref, "bf16")


@pytest.mark.parametrize("D,bs", [(64, 16), (128, 64), (64, 256)])
def test_head_dims_and_page_sizes(gpu_lib, D, bs):
    w = ragged(seed=320, D=D, bs=bs, Hq=16, Hkv=2)
    assert_close(split_prefill(gpu_lib, w, 192), oracle_out(w, causal=True), "bf16")


def test_loose_context_bound_and_sequences_without_rows(gpu_lib):
    """max_context_len 4x the longest context (most ranges empty for every
    row) and a sequence with no query rows between two with rows."""
    w = small("prefill", seed=330, ctx=(300, 500, 700), q_lens=[300, 0, 64], Hq=8, Hkv=1, causal=True)
    assert_close(split_prefill(gpu_lib, w, 0, max_ctx=2800), oracle_out(w, causal=True), "bf16")
    assert splits(w, 0, 2800) > 0


def test_calls_that_do_not_split_equal_the_plain_prefill(gpu_lib):
    w = ragged(seed=340)
    plain = gpu_prefill(gpu_lib, w)
    assert splits(w, -1) == 0 and splits(w, 2048) == 0
    assert np.array_equal(split_prefill(gpu_lib, w, -1), plain)
    assert np.array_equal(split_prefill(gpu_lib, w, 2048), plain)  # one range holds every key
    full = named_workload("chunked_prefill_bf16")  # 512 work-groups fill the device
    assert splits(full) == 0
    assert np.array_equal(split_prefill(gpu_lib, full), gpu_prefill(gpu_lib, full))


def test_block_mask_keeps_the_unsplit_path(gpu_lib):
    from tests.test_gpu_block_mask import device_mask, random_dense
    from tests.test_oracle import pack_block_mask
    w = ragged(seed=350)
    rng = np.random.default_rng(350)
    bm = pack_block_mask(random_dense(rng, w, 16, 64, 0.5), 16, 64)
    dm = device_mask(gpu_lib, bm)
    got = split_prefill(gpu_lib, w, 128, block_mask=dm)
    assert np.array_equal(got, gpu_prefill(gpu_lib, w, block_mask=dm))
    assert_close(got, oracle_out(w, oracle.ScoreMods(causal=True, block_mask=bm)), "bf16")


def test_split_close_to_unsplit_and_small_workspace_refused(gpu_lib):
    w = ragged(seed=360)
    a = bits_to_f64(split_prefill(gpu_lib, w, 64), "bf16")
    b = bits_to_f64(gpu_prefill(gpu_lib, w), "bf16")
    assert np.max(np.abs(a - b)) <= 2e-2
    need = splits(w, 64)
    short = torch.empty(need // 4 - 1, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        split_prefill(gpu_lib, w, 64, workspace=short)

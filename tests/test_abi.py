"""The C-ABI library on the host: it loads, exports what the header declares,
and rejects invalid arguments with the documented codes before any HIP call.
No compute is launched here (no GPU needed)."""

import ctypes
import os
import re

import pytest

from paged_kv_cache_attn_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]

FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first
NULL = None


def declared_functions():
    names = []
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "defined")))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["kv_append", "paged_attn_decode", "paged_attn_prefill", "paged_attn_decode_partials",
              "paged_attn_decode_merge", "paged_attn_decode_workspace_size", "paged_attn_decode_split_tokens",
              "paged_attn_status_string", "pa_bench_stream_read", "pa_bench_fill"]:
        assert n in names, n
    assert set(names) == set(binding.SIGNATURES), names


def test_library_exports_every_declared_symbol():
    L = binding.lib()
    for n in declared_functions():
        assert hasattr(L, n), n
    out = os.popen(f"nm -D --defined-only {binding.lib_path()}").read()
    exported = set(re.findall(r" T (\w+)$", out, flags=re.M))
    assert set(declared_functions()) <= exported


def test_status_strings():
    assert binding.status_string(0) == "ok"
    for code in range(-15, 0):
        s = binding.status_string(code)
        assert s and s != "unknown status", code
    assert binding.status_string(-99) == "unknown status"


def _append(**over):
    a = dict(k_new=FAKE, v_new=FAKE, k_cache=FAKE, v_cache=FAKE, slots=FAKE, T=4, Hkv=8, D=128, bs=16, NB=10,
             dtype=1)
    a.update(over)
    return binding.lib().kv_append(a["k_new"], a["v_new"], a["k_cache"], a["v_cache"], a["slots"], a["T"],
                                   a["Hkv"], a["D"], a["bs"], a["NB"], a["dtype"], None)


def test_kv_append_validation():
    assert _append(dtype=2) == -8
    assert _append(T=-1) == -2
    assert _append(NB=-1) == -2
    assert _append(Hkv=0) == -3
    assert _append(D=96) == -4
    assert _append(bs=8) == -5
    assert _append(bs=24) == -5
    assert _append(bs=512) == -5
    assert _append(k_cache=NULL) == -1
    assert _append(slots=NULL) == -1
    assert _append(T=0, k_new=NULL, v_new=NULL, k_cache=NULL, v_cache=NULL, slots=NULL) == 0  # no-op
    assert _append(v_cache=ctypes.c_void_p(0x1002)) == -14   # not 16-byte aligned
    assert _append(k_new=ctypes.c_void_p(0x1008)) == -14


def _decode(fn="paged_attn_decode", **over):
    a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, bt=FAKE, stride=4, ctx=FAKE, B=2, Hq=32, Hkv=8, D=128, bs=16, NB=100,
             max_ctx=64, scale=0.1, split=0, mods=None, ws=FAKE, ws_bytes=1 << 40, dtype=1)
    a.update(over)
    L = binding.lib()
    if fn == "paged_attn_decode_merge":
        return L.paged_attn_decode_merge(a["out"], a["ctx"], a["B"], a["Hq"], a["Hkv"], a["D"], a["max_ctx"],
                                         a["split"], a["mods"], a["ws"], a["ws_bytes"], a["dtype"], None)
    return getattr(L, fn)(a["out"], a["q"], a["k"], a["v"], a["bt"], a["stride"], a["ctx"], a["B"], a["Hq"],
                          a["Hkv"], a["D"], a["bs"], a["NB"], a["max_ctx"], a["scale"], a["split"], a["mods"],
                          a["ws"], a["ws_bytes"], a["dtype"], None)


def _decode_noalloc(**over):
    a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, bt=FAKE, stride=4, ctx=FAKE, B=2, Hq=32, Hkv=8, D=128, bs=16, NB=100,
             max_ctx=64, scale=0.1, split=0, mods=None, dtype=1)
    a.update(over)
    return binding.lib().paged_attn_decode_noalloc(a["out"], a["q"], a["k"], a["v"], a["bt"], a["stride"], a["ctx"],
                                                   a["B"], a["Hq"], a["Hkv"], a["D"], a["bs"], a["NB"], a["max_ctx"],
                                                   a["scale"], a["split"], a["mods"], a["dtype"], None)


def test_block_mask_validation():
    """Block-mask fields are checked on the host: NULL bits, block sizes that
    are not powers of two, key blocks below one 64-key tile, empty rows,
    misaligned bits."""
    def call(**bm_over):
        f = dict(bits=0x10000, q_block=16, kv_block=128, rows_per_seq=4, words_per_row=2)
        f.update(bm_over)
        bm = binding.BlockMaskStruct(f["bits"], f["q_block"], f["kv_block"], f["rows_per_seq"], f["words_per_row"])
        m = binding.ScoreMods(0, 0.0, None, None, None, ctypes.pointer(bm))
        return _decode(mods=ctypes.pointer(m)), _prefill(mods=ctypes.pointer(m))
    assert call(bits=None) == (-1, -1)
    assert call(q_block=12) == (-10, -10)
    assert call(kv_block=32) == (-10, -10)
    assert call(kv_block=96) == (-10, -10)
    assert call(rows_per_seq=0) == (-10, -10)
    assert call(words_per_row=0) == (-10, -10)
    assert call(bits=0x10002) == (-14, -14)


def test_decode_noalloc_validation():
    """The allocation-free decode checks its arguments like the decode and
    refuses sizes whose workspace exceeds the library's 16 MiB scratch (all
    before any device work)."""
    assert _decode_noalloc(dtype=5) == -8
    assert _decode_noalloc(D=96) == -4
    assert _decode_noalloc(split=100) == -6
    assert _decode_noalloc(q=NULL) == -1
    assert _decode_noalloc(out=ctypes.c_void_p(0x1008)) == -14
    assert _decode_noalloc(B=0) == 0
    big = dict(B=4000, Hq=64, Hkv=8, max_ctx=32768, stride=2048)
    assert binding.decode_workspace_size(4000, 64, 8, 128, 32768, 0) > binding.DECODE_SCRATCH_BYTES
    assert _decode_noalloc(**big) == -15
    assert _decode_noalloc(**big, split=512) == -15
    # the long-context batch fits
    assert binding.decode_workspace_size(64, 64, 8, 128, 32768, 0) <= binding.DECODE_SCRATCH_BYTES


@pytest.mark.parametrize("fn", ["paged_attn_decode", "paged_attn_decode_partials"])
def test_decode_validation(fn):
    assert _decode(fn, dtype=5) == -8
    assert _decode(fn, B=-1) == -2
    assert _decode(fn, max_ctx=-3) == -2
    assert _decode(fn, Hq=30) == -3
    assert _decode(fn, Hkv=0) == -3
    assert _decode(fn, D=256) == -4
    assert _decode(fn, bs=48) == -5
    assert _decode(fn, split=100) == -6
    assert _decode(fn, split=8) == -6
    assert _decode(fn, split=-3) == -6
    assert _decode(fn, stride=0) == -11
    assert _decode(fn, q=NULL) == -1
    assert _decode(fn, bt=NULL) == -1
    assert _decode(fn, max_ctx=4096, ws=NULL) == -7
    assert _decode(fn, max_ctx=4096, ws_bytes=16) == -7
    bad = binding.ScoreMods(-1, 0.0, None)
    assert _decode(fn, mods=ctypes.pointer(bad)) == -10
    bad = binding.ScoreMods(0, float("nan"), None)
    assert _decode(fn, mods=ctypes.pointer(bad)) == -10
    bad = binding.ScoreMods(0, float("inf"), None)
    assert _decode(fn, mods=ctypes.pointer(bad)) == -10
    assert _decode(fn, B=0) == 0  # nothing to do, nothing launched
    assert _decode(fn, q=ctypes.c_void_p(0x1004)) == -14
    assert _decode(fn, ws=ctypes.c_void_p(0x1010 + 8)) == -14


def test_merge_validation():
    assert _decode("paged_attn_decode_merge", dtype=9) == -8
    assert _decode("paged_attn_decode_merge", out=NULL) == -1
    assert _decode("paged_attn_decode_merge", max_ctx=4096, ws=NULL) == -7


def _prefill(**over):
    a = dict(out=FAKE, q=FAKE, cu=FAKE, k=FAKE, v=FAKE, bt=FAKE, stride=4, ctx=FAKE, B=2, maxq=16, Hq=32, Hkv=8,
             D=128, bs=16, NB=100, scale=0.1, causal=1, mods=None, dtype=1)
    a.update(over)
    return binding.lib().paged_attn_prefill(a["out"], a["q"], a["cu"], a["k"], a["v"], a["bt"], a["stride"],
                                            a["ctx"], a["B"], a["maxq"], a["Hq"], a["Hkv"], a["D"], a["bs"], a["NB"],
                                            a["scale"], a["causal"], a["mods"], a["dtype"], None)


def test_prefill_validation():
    assert _prefill(dtype=3) == -8
    assert _prefill(B=-2) == -2
    assert _prefill(maxq=-1) == -2
    assert _prefill(Hq=12, Hkv=8) == -3
    assert _prefill(D=32) == -4
    assert _prefill(bs=1024) == -5
    assert _prefill(causal=2) == -9
    assert _prefill(stride=0) == -11
    assert _prefill(cu=NULL) == -1
    assert _prefill(v=NULL) == -1
    bad = binding.ScoreMods(0, -1.0, None)
    assert _prefill(mods=ctypes.pointer(bad)) == -10
    assert _prefill(out=ctypes.c_void_p(0x1001)) == -14
    assert _prefill(maxq=0) == 0
    assert _prefill(B=0) == 0


def _prefill_split(**over):
    a = dict(out=FAKE, q=FAKE, cu=FAKE, total_q=64, k=FAKE, v=FAKE, bt=FAKE, stride=128, ctx=FAKE, B=1, maxq=64,
             Hq=4, Hkv=1, D=128, bs=16, NB=200, max_ctx=2048, key_split=0, scale=0.1, causal=1, mods=None, ws=None,
             ws_bytes=0, dtype=1)
    a.update(over)
    return binding.lib().paged_attn_prefill_split(
        a["out"], a["q"], a["cu"], a["total_q"], a["k"], a["v"], a["bt"], a["stride"], a["ctx"], a["B"], a["maxq"],
        a["Hq"], a["Hkv"], a["D"], a["bs"], a["NB"], a["max_ctx"], a["key_split"], a["scale"], a["causal"],
        a["mods"], a["ws"], a["ws_bytes"], a["dtype"], None)


def test_prefill_split_validation():
    # the checks of paged_attn_prefill, then the split's own
    assert _prefill_split(dtype=3) == -8
    assert _prefill_split(Hq=12, Hkv=8) == -3
    assert _prefill_split(cu=NULL) == -1
    for bad in (100, 32, -2, -64):
        assert _prefill_split(key_split=bad) == -6, bad
    assert _prefill_split(total_q=-1) == -2
    assert _prefill_split(max_ctx=-1) == -2
    # a 2-work-group grid over 2,048 keys is split (no device is visible
    # here, so CUs = 256): the workspace is required
    assert _prefill_split() == -7
    assert _prefill_split(ws=FAKE, ws_bytes=1000) == -7
    assert _prefill_split(key_split=1024) == -7
    # nothing to do, or arguments the split does not read
    assert _prefill_split(total_q=0) == 0
    assert _prefill_split(maxq=0) == 0
    assert _prefill_split(B=0) == 0
    assert _prefill_split(key_split=-1, total_q=-1, max_ctx=-1, out=ctypes.c_void_p(0x1001)) == -14


def test_prefill_split_plan_and_workspace_size():
    ws = binding.prefill_workspace_size
    # one GPU's share of an 8-way head split of the chunked prefill: 4 sequences
    # x 1 kv-head x 16 query tiles = 64 work-groups on 256 units -> min(512 / 64,
    # 2048 / 512) = 4 ranges of 512 keys; part_o 4 x 2048 x 4 x 128 fp32, then
    # part_lse 4 x 2048 x 4 fp32
    assert ws(4, 2048, 512, 4, 1, 128, 2048) == 4 * 2048 * 4 * 128 * 4 + 4 * 2048 * 4 * 4
    # the whole batch (512 work-groups) fills the device: no split
    assert ws(4, 2048, 512, 32, 8, 128, 2048) == 0
    # explicit ranges: 1,024 keys of 2,048 -> 2 ranges; one range -> no split
    assert ws(4, 2048, 512, 32, 8, 128, 2048, 1024) == 2 * 2048 * 32 * 128 * 4 + 2 * 2048 * 32 * 4
    assert ws(4, 2048, 512, 32, 8, 128, 2048, 2048) == 0
    assert ws(4, 2048, 512, 4, 1, 128, 2048, -1) == 0
    # ranges of at least 512 keys: 700 keys are not split; 64 work-groups at
    # 1,500 keys -> min(512 / 64, 1500 // 512) = 2 ranges of 768 keys (750
    # rounded up to whole 64-key tiles)
    assert ws(1, 64, 64, 4, 1, 128, 700) == 0
    assert ws(4, 2048, 512, 4, 1, 128, 1500) == 2 * 2048 * 4 * 128 * 4 + 2 * 2048 * 4 * 4
    # D 64, 4 ranges of 1,024 keys, 3 rows of 1 head: part_o 4 x 3 x 64 fp32,
    # part_lse 4 x 3 fp32
    assert ws(1, 3, 3, 1, 1, 64, 4096, 1024) == 4 * 3 * 64 * 4 + 4 * 3 * 4
    # fp32, group sizes that do not divide 128, invalid key_split: no workspace
    assert ws(4, 2048, 512, 4, 1, 128, 2048, 0, binding.PA_F32) == 0
    assert ws(4, 2048, 512, 24, 8, 128, 2048) == 0
    assert ws(4, 2048, 512, 4, 1, 128, 2048, 100) == 0


def test_split_resolution_and_workspace_size():
    # explicit split sizes are taken as given; -1 never splits; -2 = balanced split;
    # 0 = the library's choice (no device is visible here, so CUs = 256)
    assert binding.decode_split_tokens(64, 8, 32768, 512) == 512
    assert binding.decode_split_tokens(64, 8, 32768, -1) == -1
    assert binding.decode_split_tokens(64, 8, 32768, 100) == 0  # invalid
    assert binding.decode_split_tokens(64, 8, 32768, -3) == 0  # invalid
    assert binding.decode_split_tokens(64, 8, 32768) == 0
    assert binding.decode_split_tokens(8, 8, 2048, -2) == 0
    # small batches: 512-key pieces while B * Hkv * ceil(max_ctx / 512) <= 16 per unit
    assert binding.decode_split_tokens(8, 8, 2048) == 512
    assert binding.decode_split_tokens(64, 8, 4096) == 512  # 4096 pieces
    assert binding.decode_split_tokens(64, 8, 4097) == 0    # 4608 pieces: balanced split
    # longer pieces once a row would hold more than 32 of 512 keys: at most 32
    # partial states per row (ceil(log2 max_ctx) - 5, at least 9)
    assert binding.decode_split_tokens(2, 8, 16384) == 512
    assert binding.decode_split_tokens(2, 8, 16385) == 1024
    assert binding.decode_split_tokens(1, 8, 32768) == 1024
    assert binding.decode_split_tokens(1, 8, 65536) == 2048
    assert binding.decode_split_tokens(1, 8, 131072) == 4096
    assert binding.decode_workspace_size(1, 64, 8, 128, 32768, 0) == 1 * 8 * 8 * 32 * 130 * 4
    # more than 4096 sequences: the balanced split is not available; fixed pieces
    assert binding.decode_split_tokens(5000, 8, 32768, -2) > 0
    # rows of at most 256 keys are never split by default: no workspace, no merge
    assert binding.decode_split_tokens(8, 8, 256) == -1
    assert binding.decode_split_tokens(8, 8, 257) == 512
    assert binding.decode_workspace_size(8, 32, 8, 128, 256, 0) == 0
    # fixed partitions: B * Hkv * ceil(g/GP)*GP * P * (D + 2) * 4 bytes, 0 when unsplit
    assert binding.decode_workspace_size(64, 64, 8, 128, 32768, 512) == 64 * 8 * 8 * 64 * 130 * 4
    assert binding.decode_workspace_size(8, 32, 8, 128, 2048, 512) == 8 * 8 * 4 * 4 * 130 * 4
    assert binding.decode_workspace_size(8, 32, 8, 128, 2048, -1) == 0
    assert binding.decode_workspace_size(8, 32, 8, 128, 512, 512) == 0
    assert binding.decode_workspace_size(1, 4, 4, 64, 128, 64) == 1 * 4 * 1 * 4 * 2 * 66 * 4
    assert binding.decode_workspace_size(8, 30, 8, 128, 2048, 0) == 0  # invalid heads
    # balanced split: (W + items) * GP * (D + 2) * 4 + items * 8 bytes, items =
    # B * Hkv * ceil(g/GP), W = min(8 * CUs, chunks / 8), chunks = items *
    # (ceil(max_ctx/16) + 1); no device is visible here, so CUs = 256
    assert binding.decode_workspace_size(64, 64, 8, 128, 32768, 0) == (2048 + 512) * 8 * 130 * 4 + 512 * 8
    assert binding.decode_workspace_size(8, 32, 8, 128, 2048, -2) == (1032 + 64) * 4 * 130 * 4 + 64 * 8
    # the default on a small batch: 512-key pieces
    assert binding.decode_workspace_size(8, 32, 8, 128, 2048, 0) == 8 * 8 * 4 * 4 * 130 * 4


def _lv(G=2, maxg=4, maxp=512, gs=FAKE, pe=FAKE, ps=None):
    return binding.PrefixLevel(gs, ps, pe, G, maxg, maxp)


def _cascade(levels=None, fn="paged_attn_decode_cascade", **over):
    a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, bt=FAKE, stride=4, ctx=FAKE, B=8, L=None, Hq=32, Hkv=8, D=128, bs=16,
             NB=100, max_ctx=1024, scale=0.1, mods=None, ws=FAKE, ws_bytes=1 << 40, dtype=1)
    a.update(over)
    lv = [_lv()] if levels is None else levels
    arr = (binding.PrefixLevel * max(1, len(lv)))(*lv)
    return getattr(binding.lib(), fn)(
        a["out"], a["q"], a["k"], a["v"], a["bt"], a["stride"], a["ctx"], a["B"], arr,
        len(lv) if a["L"] is None else a["L"], a["Hq"], a["Hkv"], a["D"], a["bs"], a["NB"], a["max_ctx"], a["scale"],
        a["mods"], a["ws"], a["ws_bytes"], a["dtype"], None)


def test_cascade_plan_picks_the_plain_decode_for_small_batches():
    """The two-phase decode runs from 256 MiB of logical K+V up (host bound:
    sequences x max context x kv-heads x D x 2 x 2 bytes); below, the plain
    decode is faster (a 16 x 1,280-token batch: 84 MB)."""
    lv = [_lv(G=1, maxg=16, maxp=1024)]
    assert binding.decode_cascade_plan(16, lv, 32, 8, 128, 1280) == 0          # 84 MB
    assert binding.decode_cascade_plan(64, lv, 32, 8, 128, 1280) == 1          # 335 MB
    assert binding.decode_cascade_plan(64, [_lv(G=1, maxg=64, maxp=16384)], 64, 8, 128, 17408) == 1
    assert binding.decode_cascade_plan(16, lv, 30, 8, 128, 1 << 20) == 0       # invalid heads
    assert binding.decode_cascade_plan(-1, lv, 32, 8, 128, 1280) == 0


@pytest.mark.parametrize("fn", ["paged_attn_decode_cascade", "paged_attn_decode_cascade_two_phase"])
def test_cascade_validation_both_entries(fn):
    assert _cascade(fn=fn, dtype=0) == -8
    assert _cascade(fn=fn, B=-1) == -2
    assert _cascade(fn=fn, Hq=24, Hkv=8) == -3 or _cascade(fn=fn, Hq=24, Hkv=8) < 0
    assert _cascade(fn=fn, q=NULL) == -1
    assert _cascade(fn=fn, ws=NULL) == -7
    assert _cascade(fn=fn, levels=[_lv(G=0)]) == -2


def test_cascade_validation():
    assert _cascade(dtype=0) == -8          # bf16 only
    assert _cascade(dtype=4) == -8
    assert _cascade(B=-1) == -2
    assert _cascade(levels=[_lv(G=0)]) == -2           # a non-empty batch needs a group per level
    assert _cascade(levels=[_lv(maxg=0)]) == -2
    assert _cascade(levels=[_lv(maxp=-1)]) == -2
    assert _cascade(levels=[_lv(), _lv(G=0)]) == -2
    assert _cascade(L=0) == -2                          # at least one level
    assert _cascade(levels=[_lv()] * 9) == -2           # at most eight
    assert _cascade(Hq=24, Hkv=8) == -3      # group of 3 does not divide 128
    assert _cascade(D=96) == -4
    assert _cascade(bs=8) == -5
    assert _cascade(stride=0) == -11
    assert _cascade(levels=[_lv(gs=NULL)]) == -1
    assert _cascade(levels=[_lv(), _lv(pe=NULL)]) == -1
    assert _cascade(q=NULL) == -1
    assert _cascade(ws=NULL) == -7
    assert _cascade(ws_bytes=1024) == -7
    assert _cascade(ws=ctypes.c_void_p(0x1008)) == -7  # not 16-byte aligned
    assert _cascade(k=ctypes.c_void_p(0x1008)) == -14
    assert _cascade(mods=ctypes.pointer(binding.ScoreMods(0, -2.0, None))) == -10
    assert _cascade(mods=ctypes.pointer(binding.ScoreMods(-3, 0.0, None))) == -10
    assert _cascade(B=0, L=0) == 0   # nothing to do, nothing launched


def _ws(B, levels, Hq, Hkv, D, ctx):
    arr = (binding.PrefixLevel * max(1, len(levels)))(*levels)
    return binding.lib().paged_attn_decode_cascade_workspace_size(B, arr, len(levels), Hq, Hkv, D, ctx)


def test_cascade_workspace_size():
    # key-range states [ranges, B*Hq, D + 1] fp32 over all levels, the suffix
    # state [B*Hq, D + 1], B key starts, then the balanced decode's workspace;
    # each piece 256-byte aligned
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    B, Hq, Hkv, D, ctx = 64, 64, 8, 128, 17408
    dec = binding.decode_workspace_size(B, Hq, Hkv, D, ctx, 0)

    def want(ranges):
        return (al(ranges * B * Hq * D * 4) + al(ranges * B * Hq * 4) + al(B * Hq * D * 4) + al(B * Hq * 4)
                + al(B * 4) + al(dec))
    # one group of 64: 1 group x 8 kv-heads x 4 query tiles = 32 work-groups per
    # key range; 512 wanted (2 per compute unit, 256 units) -> 16 ranges of 16 tiles
    assert _ws(B, [_lv(G=1, maxg=64, maxp=16384)], Hq, Hkv, D, ctx) == want(16)
    # a short prefix keeps at least 4 tiles per range: 300 keys -> 5 tiles -> 1 range
    assert _ws(B, [_lv(G=1, maxg=64, maxp=300)], Hq, Hkv, D, ctx) == want(1)
    # two levels add their ranges: 16 + (8 groups of 8 -> 64 work-groups -> 8 ranges of 4096/8)
    assert _ws(B, [_lv(G=1, maxg=64, maxp=16384), _lv(G=8, maxg=8, maxp=4096)], Hq, Hkv, D, ctx) == want(16 + 8)
    assert _ws(B, [_lv(G=0, maxg=64, maxp=16384)], Hq, Hkv, D, ctx) == 0  # invalid
    assert _ws(B, [], Hq, Hkv, D, ctx) == 0
    assert _ws(B, [_lv(G=1, maxg=64, maxp=16384)], 24, 8, D, ctx) == 0
    assert _ws(0, [_lv(G=1, maxg=64, maxp=16384)], Hq, Hkv, D, ctx) == 0


def test_bench_util_validation():
    L = binding.lib()
    sink = ctypes.c_void_p(0x2000)
    assert L.pa_bench_stream_read(NULL, 16, sink, None) == -1
    assert L.pa_bench_stream_read(FAKE, 16, NULL, None) == -1
    assert L.pa_bench_stream_read(FAKE, 17, sink, None) == -2          # size not a multiple of 16
    assert L.pa_bench_stream_read(ctypes.c_void_p(0x1004), 16, sink, None) == -2  # misaligned
    assert L.pa_bench_stream_read(FAKE, 0, sink, None) == 0             # nothing to do
    assert L.pa_bench_fill(NULL, 16, 0, None) == -1
    assert L.pa_bench_fill(FAKE, 24, 0, None) == -2
    assert L.pa_bench_fill(FAKE, 0, 0, None) == 0


def test_copy_blocks_validation():
    L = binding.lib()
    assert L.kv_copy_blocks(FAKE, FAKE, FAKE, FAKE, -1, 8, 128, 16, 10, 1, None) == -2
    assert L.kv_copy_blocks(FAKE, FAKE, FAKE, FAKE, 2, 0, 128, 16, 10, 1, None) == -3
    assert L.kv_copy_blocks(FAKE, FAKE, FAKE, FAKE, 2, 8, 96, 16, 10, 1, None) == -4
    assert L.kv_copy_blocks(FAKE, FAKE, FAKE, FAKE, 2, 8, 128, 24, 10, 1, None) == -5
    assert L.kv_copy_blocks(FAKE, FAKE, FAKE, FAKE, 2, 8, 128, 16, 10, 7, None) == -8
    assert L.kv_copy_blocks(NULL, FAKE, FAKE, FAKE, 2, 8, 128, 16, 10, 1, None) == -1
    assert L.kv_copy_blocks(NULL, NULL, NULL, NULL, 0, 8, 128, 16, 10, 1, None) == 0  # nothing to do
    assert L.kv_copy_blocks(FAKE, ctypes.c_void_p(0x1004), FAKE, FAKE, 2, 8, 128, 16, 10, 1, None) == -14


def test_block_manager_argument_checks():
    L = binding.lib()
    h = ctypes.c_void_p()
    assert L.pa_bm_create(10, 24, ctypes.byref(h)) == -5
    assert L.pa_bm_create(-1, 16, ctypes.byref(h)) == -2
    assert L.pa_bm_create(10, 16, None) == -1
    assert binding.status_string(-12).startswith("block manager")
    assert binding.status_string(-13).startswith("block manager")


def test_debug_check_build_exports_the_same_symbols():
    debug = os.path.join(os.path.dirname(binding.lib_path()), "libpagedattn_debug.so")
    assert os.path.exists(debug), "build() also builds the PA_DEBUG_CHECKS library"
    out = os.popen(f"nm -D --defined-only {debug}").read()
    exported = set(re.findall(r" T (\w+)$", out, flags=re.M))
    assert set(declared_functions()) <= exported


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """No fallback: without the built library every call raises."""
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "_LIB_PATH", str(tmp_path / "libpagedattn.so"))
    with pytest.raises(RuntimeError, match="missing"):
        binding.lib()
    with pytest.raises(RuntimeError, match="missing"):
        binding.decode_workspace_size(8, 32, 8, 128, 2048)

"""Thin Python binding of ``libpagedattn.so`` (ctypes, same names as the C ABI).

Marshalling only: tensors are checked for device, dtype, shape and
contiguity, their device pointers and torch's current HIP stream are passed
to the C entry points, and status codes become exceptions (negative codes
-> ``ValueError``, positive hip errors -> ``RuntimeError``).  Every step of the
computation runs in the library's gfx950 kernels; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

# PAGEDATTN_DEBUG_CHECKS=1 selects the build whose kernels trap on a broken
# device-side caller contract (block ids out of range, lengths past the table).
_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                         "libpagedattn_debug.so" if os.environ.get("PAGEDATTN_DEBUG_CHECKS") == "1"
                         else "libpagedattn.so")

PA_F32 = 0
PA_BF16 = 1
_DTYPES = {torch.float32: PA_F32, torch.bfloat16: PA_BF16}


class BlockMaskStruct(ctypes.Structure):
    """``pa_block_mask``: bitmap rows of admitted key blocks per query block."""

    _fields_ = [("bits", ctypes.c_void_p), ("q_block", ctypes.c_int32), ("kv_block", ctypes.c_int32),
                ("rows_per_seq", ctypes.c_int32), ("words_per_row", ctypes.c_int32)]


class ScoreMods(ctypes.Structure):
    """``pa_score_mods``: window (0 = none), softcap (0 = none), alibi slopes,
    prefix-LM lengths per sequence, document starts per query row, block mask."""

    _fields_ = [("window", ctypes.c_int32), ("softcap", ctypes.c_float),
                ("alibi_slopes", ctypes.c_void_p), ("prefix_lens", ctypes.c_void_p),
                ("doc_starts", ctypes.c_void_p), ("block_mask", ctypes.POINTER(BlockMaskStruct))]


class PrefixLevel(ctypes.Structure):
    """``pa_prefix_level``: one depth of shared prefixes for the two-phase decode."""

    _fields_ = [("group_starts", ctypes.c_void_p), ("prefix_starts", ctypes.c_void_p),
                ("prefix_ends", ctypes.c_void_p), ("num_groups", ctypes.c_int32),
                ("max_group_size", ctypes.c_int32), ("max_prefix_len", ctypes.c_int32)]


_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_f32 = ctypes.c_float
_sz = ctypes.c_size_t
_mods_p = ctypes.POINTER(ScoreMods)

# name -> (restype, argtypes), mirroring include/pagedattn.h
SIGNATURES = {
    "kv_append": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i64, _i32, _vp]),
    "paged_attn_decode_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "paged_attn_decode_split_tokens": (_i32, [_i32, _i32, _i32, _i32]),
    "paged_attn_decode": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _i64,
                                 _i32, _f32, _i32, _mods_p, _vp, _sz, _i32, _vp]),
    "paged_attn_decode_noalloc": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _i64,
                                         _i32, _f32, _i32, _mods_p, _i32, _vp]),
    "paged_attn_decode_partials": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32,
                                          _i64, _i32, _f32, _i32, _mods_p, _vp, _sz, _i32, _vp]),
    "paged_attn_decode_merge": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _mods_p, _vp, _sz, _i32,
                                       _vp]),
    "paged_attn_prefill": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                  _i64, _f32, _i32, _mods_p, _i32, _vp]),
    "paged_attn_prefill_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "paged_attn_prefill_split": (_i32, [_vp, _vp, _vp, _i32, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32,
                                        _i32, _i64, _i32, _i32, _f32, _i32, _mods_p, _vp, _sz, _i32, _vp]),
    "paged_attn_decode_cascade_workspace_size": (_sz, [_i32, ctypes.POINTER(PrefixLevel), _i32, _i32, _i32, _i32,
                                                        _i32]),
    "paged_attn_decode_cascade": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, ctypes.POINTER(PrefixLevel), _i32,
                                         _i32, _i32, _i32, _i32, _i64, _i32, _f32, _mods_p, _vp, _sz, _i32, _vp]),
    "paged_attn_decode_cascade_two_phase": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32,
                                                   ctypes.POINTER(PrefixLevel), _i32, _i32, _i32, _i32, _i32, _i64,
                                                   _i32, _f32, _mods_p, _vp, _sz, _i32, _vp]),
    "paged_attn_decode_cascade_plan": (_i32, [_i32, ctypes.POINTER(PrefixLevel), _i32, _i32, _i32, _i32, _i32]),
    "paged_attn_status_string": (ctypes.c_char_p, [_i32]),
    "kv_copy_blocks": (_i32, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i64, _i32, _vp]),
    # include/pagedattn_blocks.h (host block manager)
    "pa_bm_create": (_i32, [_i64, _i32, ctypes.POINTER(_vp)]),
    "pa_bm_create_paged": (_i32, [_i64, _i32, _i32, ctypes.POINTER(_vp)]),
    "pa_bm_new_sequence_paged": (_i32, [_vp, _i32, _i32, ctypes.POINTER(_i32)]),
    "pa_bm_pages": (_i32, [_vp, _i32, ctypes.POINTER(_i32), ctypes.POINTER(_i32), _i32, ctypes.POINTER(_i32)]),
    "pa_bm_destroy": (None, [_vp]),
    "pa_bm_new_sequence": (_i32, [_vp, ctypes.POINTER(_i32)]),
    "pa_bm_fork": (_i32, [_vp, _i32, ctypes.POINTER(_i32)]),
    "pa_bm_free_sequence": (_i32, [_vp, _i32]),
    "pa_bm_append": (_i32, [_vp, _i32, _i32, ctypes.POINTER(_i32), ctypes.POINTER(_i32), ctypes.POINTER(_i32), _i32,
                            ctypes.POINTER(_i32)]),
    "pa_bm_table": (_i32, [_vp, _i32, ctypes.POINTER(_i32), _i32, ctypes.POINTER(_i32), ctypes.POINTER(_i64)]),
    "pa_bm_stats": (_i32, [_vp, ctypes.POINTER(_i64), ctypes.POINTER(_i64), ctypes.POINTER(_i64)]),
    "pa_bm_block_refcount": (_i32, [_vp, _i32, ctypes.POINTER(_i32)]),
    "pa_bm_prefix_levels": (_i32, [_vp, ctypes.POINTER(_i32), _i32, _i32, ctypes.POINTER(_i32),
                                   ctypes.POINTER(_i32), ctypes.POINTER(_i32), ctypes.POINTER(_i32),
                                   ctypes.POINTER(_i32)]),
    # include/pagedattn_bench.h (measurement support)
    "pa_bench_stream_read": (_i32, [_vp, _sz, _vp, _vp]),
    "pa_bench_fill": (_i32, [_vp, _sz, ctypes.c_uint32, _vp]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load the library (built beforehand by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def lib_path() -> str:
    return _LIB_PATH


def status_string(code: int) -> str:
    return lib().paged_attn_status_string(int(code)).decode()


def _check(code: int, what: str):
    if code == 0:
        return
    msg = f"{what}: {status_string(code)} (status {code})"
    if code < 0:
        raise ValueError(msg)
    raise RuntimeError(msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t: torch.Tensor, name: str, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {t.dtype}")
    return _DTYPES[t.dtype]


def block_mask(bits, q_block, kv_block):
    """A block mask for the calls' ``block_mask=`` argument.

    ``bits``: int32 device tensor ``[num_seqs, rows_per_seq, words]`` holding
    uint32 bit patterns; row ``p // q_block`` of sequence ``b`` admits key
    ``j`` when bit ``(j // kv_block) % 32`` of word ``(j // kv_block) // 32``
    is set (``pa_block_mask``)."""
    _need(bits, "block mask bits", torch.int32, 3)
    return {"bits": bits, "q_block": int(q_block), "kv_block": int(kv_block)}


def _mods(window=0, softcap=0.0, alibi_slopes=None, prefix_lens=None, doc_starts=None, block_mask=None):
    if (not window and not softcap and alibi_slopes is None and prefix_lens is None and doc_starts is None
            and block_mask is None):
        return None, None
    if alibi_slopes is not None:
        _need(alibi_slopes, "alibi_slopes", torch.float32, 1)
    if prefix_lens is not None:
        _need(prefix_lens, "prefix_lens", torch.int32, 1)
    if doc_starts is not None:
        _need(doc_starts, "doc_starts", torch.int32, 1)
    ptr = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    bm = None
    if block_mask is not None:
        bits = block_mask["bits"]
        bm = BlockMaskStruct(bits.data_ptr(), block_mask["q_block"], block_mask["kv_block"], bits.shape[1],
                             bits.shape[2])
    m = ScoreMods(int(window), float(softcap), ptr(alibi_slopes), ptr(prefix_lens), ptr(doc_starts),
                  None if bm is None else ctypes.pointer(bm))
    return ctypes.pointer(m), (m, bm)


def _pool_dims(k_cache, v_cache):
    """K pool ``[NB, Hkv, bs, D]``; V pool ``[NB, Hkv, bs/S, D, S]``, S = min(bs, 16)."""
    _need(k_cache, "k_cache", ndim=4)
    _need(v_cache, "v_cache", ndim=5)
    NB, Hkv, bs, D = k_cache.shape
    S = min(bs, 16)
    if tuple(v_cache.shape) != (NB, Hkv, bs // S, D, S) or v_cache.dtype != k_cache.dtype:
        raise ValueError("v_cache must be [num_blocks, num_kv_heads, block_size/S, head_dim, S], "
                         "S = min(block_size, 16), of k_cache's dtype")
    return NB, Hkv, bs, D


def kv_append(k_new, v_new, k_cache, v_cache, slot_mapping):
    """Write ``k_new/v_new [T, Hkv, D]`` into the slots ``slot_mapping [T]`` (int32)."""
    NB, Hkv, bs, D = _pool_dims(k_cache, v_cache)
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _need(t, n, k_cache.dtype, 3)
    _need(slot_mapping, "slot_mapping", torch.int32, 1)
    T = slot_mapping.shape[0]
    if tuple(k_new.shape) != (T, Hkv, D) or tuple(v_new.shape) != (T, Hkv, D):
        raise ValueError("k_new/v_new must be [T, num_kv_heads, head_dim]")
    code = lib().kv_append(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(slot_mapping), T, Hkv,
                           D, bs, NB, _dtype_code(k_cache), _stream())
    _check(code, "kv_append")


def decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim, max_context_len, split_tokens=0) -> int:
    return int(lib().paged_attn_decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim,
                                                      max_context_len, split_tokens))


def decode_split_tokens(num_seqs, num_kv_heads, max_context_len, split_tokens=0) -> int:
    return int(lib().paged_attn_decode_split_tokens(num_seqs, num_kv_heads, max_context_len, split_tokens))


def decode_workspace(q, num_kv_heads, max_context_len, split_tokens=0):
    """A decode workspace for these sizes."""
    B, Hq, D = q.shape
    n = decode_workspace_size(B, Hq, num_kv_heads, D, max_context_len, split_tokens)
    return torch.empty(max(n, 4) // 4, dtype=torch.float32, device=q.device)


def _decode_args(out, q, k_cache, v_cache, block_tables, context_lens):
    NB, Hkv, bs, D = _pool_dims(k_cache, v_cache)
    _need(q, "q", k_cache.dtype, 3)
    _need(out, "out", k_cache.dtype, 3)
    _need(block_tables, "block_tables", torch.int32, 2)
    _need(context_lens, "context_lens", torch.int32, 1)
    B, Hq, Dq = q.shape
    if Dq != D or tuple(out.shape) != tuple(q.shape) or block_tables.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("shape mismatch between q/out/block_tables/context_lens/pools")
    return NB, Hkv, bs, D, B, Hq


def paged_attn_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
                      split_tokens=0, workspace=None, window=0, softcap=0.0, alibi_slopes=None, phase="both",
                      prefix_lens=None, doc_starts=None, block_mask=None):
    """One query row per sequence; writes ``out [B, Hq, D]``.

    ``phase`` selects ``paged_attn_decode`` ("both"), ``..._partials`` or
    ``..._merge``.  ``workspace`` defaults to a fresh buffer of the size the
    library asks for.
    """
    NB, Hkv, bs, D, B, Hq = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens)
    if workspace is None:
        workspace = decode_workspace(q, Hkv, max_context_len, split_tokens)
    _need(workspace, "workspace")
    mp, _keep = _mods(window, softcap, alibi_slopes, prefix_lens, doc_starts, block_mask)
    ws_bytes = workspace.numel() * workspace.element_size()
    L = lib()
    if phase == "merge":
        code = L.paged_attn_decode_merge(_ptr(out), _ptr(context_lens), B, Hq, Hkv, D, int(max_context_len),
                                         int(split_tokens), mp, _ptr(workspace), ws_bytes, _dtype_code(q),
                                         _stream())
    else:
        fn = L.paged_attn_decode if phase == "both" else L.paged_attn_decode_partials
        code = fn(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), block_tables.shape[1],
                  _ptr(context_lens), B, Hq, Hkv, D, bs, NB, int(max_context_len), float(scale), int(split_tokens),
                  mp, _ptr(workspace), ws_bytes, _dtype_code(q), _stream())
    _check(code, f"paged_attn_decode[{phase}]")
    return out


def paged_attn_decode_noalloc(out, q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
                              split_tokens=0, window=0, softcap=0.0, alibi_slopes=None, prefix_lens=None,
                              doc_starts=None, block_mask=None):
    """``paged_attn_decode`` on the library's own per-device scratch: takes no
    workspace and allocates nothing (the call fails with ``ValueError`` when
    the sizes need more than ``PA_DECODE_SCRATCH_BYTES``).  Calls that overlap
    on one device race on that scratch."""
    NB, Hkv, bs, D, B, Hq = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens)
    mp, _keep = _mods(window, softcap, alibi_slopes, prefix_lens, doc_starts, block_mask)
    code = lib().paged_attn_decode_noalloc(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                           block_tables.shape[1], _ptr(context_lens), B, Hq, Hkv, D, bs, NB,
                                           int(max_context_len), float(scale), int(split_tokens), mp,
                                           _dtype_code(q), _stream())
    _check(code, "paged_attn_decode_noalloc")
    return out


DECODE_SCRATCH_BYTES = 16 << 20  # PA_DECODE_SCRATCH_BYTES


def prefix_level(group_starts, prefix_ends, max_group_size, max_prefix_len, prefix_starts=None):
    """One depth of shared prefixes: int32 device tensors ``group_starts [G+1]``,
    ``prefix_ends [G]`` and optionally ``prefix_starts [G]`` (None: all 0),
    with host bounds on group members and range lengths."""
    _need(group_starts, "group_starts", torch.int32, 1)
    _need(prefix_ends, "prefix_ends", torch.int32, 1)
    G = prefix_ends.shape[0]
    if group_starts.shape[0] != G + 1:
        raise ValueError("group_starts must hold num_groups + 1 entries")
    if prefix_starts is not None:
        _need(prefix_starts, "prefix_starts", torch.int32, 1)
        if prefix_starts.shape[0] != G:
            raise ValueError("prefix_starts must hold num_groups entries")
    return {"group_starts": group_starts, "prefix_starts": prefix_starts, "prefix_ends": prefix_ends,
            "num_groups": G, "max_group_size": int(max_group_size), "max_prefix_len": int(max_prefix_len)}


def _levels_array(levels):
    arr = (PrefixLevel * max(1, len(levels)))()
    for i, v in enumerate(levels):
        if isinstance(v, PrefixLevel):  # already a pa_prefix_level
            arr[i] = v
            continue
        arr[i] = PrefixLevel(v["group_starts"].data_ptr(),
                             None if v["prefix_starts"] is None else v["prefix_starts"].data_ptr(),
                             v["prefix_ends"].data_ptr(), v["num_groups"], v["max_group_size"], v["max_prefix_len"])
    return arr


def decode_cascade_workspace_size(num_seqs, levels, num_heads, num_kv_heads, head_dim, max_context_len) -> int:
    return int(lib().paged_attn_decode_cascade_workspace_size(num_seqs, _levels_array(levels), len(levels),
                                                              num_heads, num_kv_heads, head_dim, max_context_len))


def decode_cascade_workspace(q, num_kv_heads, levels, max_context_len):
    """A two-phase decode workspace for these sizes."""
    B, Hq, D = q.shape
    n = decode_cascade_workspace_size(B, levels, Hq, num_kv_heads, D, max_context_len)
    return torch.empty(max(n, 4) // 4, dtype=torch.float32, device=q.device)


def decode_cascade_plan(num_seqs, levels, num_heads, num_kv_heads, head_dim, max_context_len) -> int:
    """1 if ``paged_attn_decode_cascade`` runs the two-phase decode for these sizes, 0 if the plain decode."""
    return int(lib().paged_attn_decode_cascade_plan(int(num_seqs), _levels_array(levels), len(levels),
                                                    int(num_heads), int(num_kv_heads), int(head_dim),
                                                    int(max_context_len)))


def paged_attn_decode_cascade(out, q, k_cache, v_cache, block_tables, context_lens, levels, scale,
                              max_context_len, workspace=None, softcap=0.0, window=0, alibi_slopes=None,
                              prefix_lens=None, doc_starts=None, mode="auto", block_mask=None):
    """Decode where sequences share (possibly nested) prefixes.

    ``levels``: a list of :func:`prefix_level`, outermost first.  Writes
    ``out [B, Hq, D]``.  ``mode`` "auto" calls ``paged_attn_decode_cascade``
    (the library runs the plain decode where that is faster), "two_phase"
    calls ``paged_attn_decode_cascade_two_phase``.
    """
    NB, Hkv, bs, D, B, Hq = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens)
    if workspace is None:
        workspace = decode_cascade_workspace(q, Hkv, levels, max_context_len)
    _need(workspace, "workspace")
    mp, _keep = _mods(window, softcap, alibi_slopes, prefix_lens, doc_starts, block_mask)
    arr = _levels_array(levels)
    if mode not in ("auto", "two_phase"):
        raise ValueError(f"mode must be 'auto' or 'two_phase', not {mode!r}")
    fn = lib().paged_attn_decode_cascade if mode == "auto" else lib().paged_attn_decode_cascade_two_phase
    code = fn(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), block_tables.shape[1],
        _ptr(context_lens), B, arr, len(levels), Hq, Hkv, D, bs, NB, int(max_context_len), float(scale), mp,
        _ptr(workspace), workspace.numel() * workspace.element_size(), _dtype_code(q), _stream())
    _check(code, f"paged_attn_decode_cascade[{mode}]")
    return out


def prefill_workspace_size(num_seqs, total_q, max_q_len, num_heads, num_kv_heads, head_dim, max_context_len,
                           key_split=0, dtype=PA_BF16) -> int:
    return int(lib().paged_attn_prefill_workspace_size(num_seqs, total_q, int(max_q_len), num_heads, num_kv_heads,
                                                       head_dim, int(max_context_len), int(key_split), dtype))


def prefill_workspace(q, num_seqs, num_kv_heads, max_q_len, max_context_len, key_split=0):
    """A workspace for ``paged_attn_prefill(..., max_context_len=...)``, or
    None when the library does not split these sizes."""
    total_q, Hq, D = q.shape
    n = prefill_workspace_size(num_seqs, total_q, max_q_len, Hq, num_kv_heads, D, max_context_len, key_split,
                               _dtype_code(q))
    return torch.empty(n // 4, dtype=torch.float32, device=q.device) if n > 0 else None


def paged_attn_prefill(out, q, cu_q_lens, k_cache, v_cache, block_tables, context_lens, scale, max_q_len,
                       causal=True, window=0, softcap=0.0, alibi_slopes=None, prefix_lens=None, doc_starts=None,
                       block_mask=None, max_context_len=None, key_split=0, workspace=None):
    """Query rows ``q [total_q, Hq, D]`` grouped by ``cu_q_lens [B+1]``; writes ``out``.

    With ``max_context_len`` (a host-side bound of ``context_lens``) the call
    goes through ``paged_attn_prefill_split``, which may split the key range
    of a small grid (``key_split``: 0 library choice, -1 never, or keys per
    range); ``workspace`` then defaults to a fresh buffer of the size asked for.
    """
    NB, Hkv, bs, D = _pool_dims(k_cache, v_cache)
    _need(q, "q", k_cache.dtype, 3)
    _need(out, "out", k_cache.dtype, 3)
    _need(cu_q_lens, "cu_q_lens", torch.int32, 1)
    _need(block_tables, "block_tables", torch.int32, 2)
    _need(context_lens, "context_lens", torch.int32, 1)
    B = context_lens.shape[0]
    if cu_q_lens.shape[0] != B + 1 or block_tables.shape[0] != B or tuple(out.shape) != tuple(q.shape) \
            or q.shape[2] != D:
        raise ValueError("shape mismatch between q/out/cu_q_lens/block_tables/context_lens/pools")
    mp, _keep = _mods(window, softcap, alibi_slopes, prefix_lens, doc_starts, block_mask)
    if max_context_len is None:
        code = lib().paged_attn_prefill(_ptr(out), _ptr(q), _ptr(cu_q_lens), _ptr(k_cache), _ptr(v_cache),
                                        _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), B,
                                        int(max_q_len), q.shape[1], Hkv, D, bs, NB, float(scale), int(bool(causal)),
                                        mp, _dtype_code(q), _stream())
        _check(code, "paged_attn_prefill")
        return out
    if workspace is None:
        workspace = prefill_workspace(q, B, Hkv, max_q_len, max_context_len, key_split)
    if workspace is not None:
        _need(workspace, "workspace")
    ws_ptr = _ptr(workspace) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    code = lib().paged_attn_prefill_split(_ptr(out), _ptr(q), _ptr(cu_q_lens), q.shape[0], _ptr(k_cache),
                                          _ptr(v_cache), _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
                                          B, int(max_q_len), q.shape[1], Hkv, D, bs, NB, int(max_context_len),
                                          int(key_split), float(scale), int(bool(causal)), mp, ws_ptr, ws_bytes,
                                          _dtype_code(q), _stream())
    _check(code, "paged_attn_prefill_split")
    return out


def bench_stream_read(src: torch.Tensor, sink: torch.Tensor):
    """Measurement support: read every byte of ``src`` once (streaming, non-temporal);
    the XOR of its 32-bit words is XOR-ed into ``sink`` (one int32, caller-zeroed)."""
    _need(src, "src")
    _need(sink, "sink", torch.int32, 1)
    code = lib().pa_bench_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink), _stream())
    _check(code, "pa_bench_stream_read")


def bench_fill(dst: torch.Tensor, value: int = 0):
    """Measurement support: overwrite ``dst`` with a 32-bit pattern (evicts the caches)."""
    _need(dst, "dst")
    code = lib().pa_bench_fill(_ptr(dst), dst.numel() * dst.element_size(), int(value) & 0xFFFFFFFF, _stream())
    _check(code, "pa_bench_fill")


def kv_copy_blocks(k_cache, v_cache, src_blocks, dst_blocks):
    """Copy whole physical blocks ``src_blocks[i] -> dst_blocks[i]`` (int32 device tensors) in both pools."""
    NB, Hkv, bs, D = _pool_dims(k_cache, v_cache)
    _need(src_blocks, "src_blocks", torch.int32, 1)
    _need(dst_blocks, "dst_blocks", torch.int32, 1)
    if src_blocks.shape != dst_blocks.shape:
        raise ValueError("src_blocks and dst_blocks must have the same length")
    code = lib().kv_copy_blocks(_ptr(k_cache), _ptr(v_cache), _ptr(src_blocks), _ptr(dst_blocks),
                                src_blocks.shape[0], Hkv, D, bs, NB, _dtype_code(k_cache), _stream())
    _check(code, "kv_copy_blocks")


class BlockManager:
    """Host block manager (``include/pagedattn_blocks.h``): allocation of
    power-of-two pages of blocks, fork by sharing, copy-on-write.  Thin
    wrapper; all bookkeeping is in the library.  ``max_page_blocks`` > 1 lets
    sequences take pages of several blocks (``new_sequence``'s bounds)."""

    def __init__(self, num_blocks: int, block_size: int, max_page_blocks: int = 1):
        h = ctypes.c_void_p()
        _check(lib().pa_bm_create_paged(int(num_blocks), int(block_size), int(max_page_blocks), ctypes.byref(h)),
               "pa_bm_create_paged")
        self._h = h
        self.block_size = int(block_size)
        self.max_page_blocks = int(max_page_blocks)

    def close(self):
        if self._h:
            lib().pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def new_sequence(self, min_page_blocks: int = 1, max_page_blocks: int | None = None) -> int:
        """A new sequence whose page k has min(min_page_blocks << k,
        max_page_blocks) blocks (max_page_blocks defaults to min_page_blocks:
        one page size)."""
        hi = min_page_blocks if max_page_blocks is None else max_page_blocks
        s = ctypes.c_int32()
        _check(lib().pa_bm_new_sequence_paged(self._h, int(min_page_blocks), int(hi), ctypes.byref(s)),
               "pa_bm_new_sequence_paged")
        return s.value

    def fork(self, parent: int) -> int:
        c = ctypes.c_int32()
        _check(lib().pa_bm_fork(self._h, int(parent), ctypes.byref(c)), "pa_bm_fork")
        return c.value

    def free(self, seq: int):
        _check(lib().pa_bm_free_sequence(self._h, int(seq)), "pa_bm_free_sequence")

    def append(self, seq: int, ntok: int):
        """Slots for ``ntok`` new tokens and the (src, dst) block copies to run first."""
        slots = (ctypes.c_int32 * max(1, ntok))()
        cap = self.max_page_blocks
        src = (ctypes.c_int32 * cap)()
        dst = (ctypes.c_int32 * cap)()
        n = ctypes.c_int32()
        _check(lib().pa_bm_append(self._h, int(seq), int(ntok), slots, src, dst, cap, ctypes.byref(n)),
               "pa_bm_append")
        return list(slots[:ntok]), [(src[i], dst[i]) for i in range(n.value)]

    def table(self, seq: int):
        """(block-table row, token count) of a sequence."""
        nb = ctypes.c_int32()
        ln = ctypes.c_int64()
        _check(lib().pa_bm_table(self._h, int(seq), None, 0, ctypes.byref(nb), ctypes.byref(ln)), "pa_bm_table")
        row = (ctypes.c_int32 * max(1, nb.value))()
        _check(lib().pa_bm_table(self._h, int(seq), row, nb.value, ctypes.byref(nb), ctypes.byref(ln)),
               "pa_bm_table")
        return list(row[:nb.value]), ln.value

    def pages(self, seq: int):
        """The sequence's pages in order, as (first block, blocks) pairs."""
        n = ctypes.c_int32()
        _check(lib().pa_bm_pages(self._h, int(seq), None, None, 0, ctypes.byref(n)), "pa_bm_pages")
        st = (ctypes.c_int32 * max(1, n.value))()
        nb = (ctypes.c_int32 * max(1, n.value))()
        _check(lib().pa_bm_pages(self._h, int(seq), st, nb, n.value, ctypes.byref(n)), "pa_bm_pages")
        return [(st[i], nb[i]) for i in range(n.value)]

    def stats(self):
        """(free blocks, used blocks, empty slots in used blocks)."""
        f, u, w = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        _check(lib().pa_bm_stats(self._h, ctypes.byref(f), ctypes.byref(u), ctypes.byref(w)), "pa_bm_stats")
        return f.value, u.value, w.value

    def refcount(self, block: int) -> int:
        c = ctypes.c_int32()
        _check(lib().pa_bm_block_refcount(self._h, int(block), ctypes.byref(c)), "pa_bm_block_refcount")
        return c.value

    def prefix_levels(self, seqs, max_levels: int = 8):
        """Shared prefixes of the batch ``seqs`` (in this order) as a list of
        (group_starts, prefix_starts, prefix_ends) int32 arrays, outermost
        level first; empty when neighbours share nothing."""
        n = len(seqs)
        ids = (ctypes.c_int32 * max(1, n))(*[int(x) for x in seqs])
        gs = (ctypes.c_int32 * (max_levels * (n + 1)))()
        ps = (ctypes.c_int32 * max(1, max_levels * n))()
        pe = (ctypes.c_int32 * max(1, max_levels * n))()
        ng = (ctypes.c_int32 * max_levels)()
        nl = ctypes.c_int32()
        _check(lib().pa_bm_prefix_levels(self._h, ids, n, int(max_levels), gs, ps, pe, ng, ctypes.byref(nl)),
               "pa_bm_prefix_levels")
        out = []
        for lvl in range(nl.value):
            G = ng[lvl]
            out.append((np.array(gs[lvl * (n + 1): lvl * (n + 1) + G + 1], np.int32),
                        np.array(ps[lvl * n: lvl * n + G], np.int32),
                        np.array(pe[lvl * n: lvl * n + G], np.int32)))
        return out

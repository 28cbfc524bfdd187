"""Run with PAGEDATTN_DEBUG_CHECKS=1: append, block copy, decode (four
splits), prefill (unsplit and over key ranges) and the two-phase decode
through the debug-check build on valid inputs; every result must match the
oracle (the checks never fire).  Exit status 0 = pass."""

import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from oracle.paged import bits_to_f64  # noqa: E402
from paged_kv_cache_attn_amd import binding  # noqa: E402
from workloads import build_workload  # noqa: E402
from workloads.device import to_numpy_bits, upload  # noqa: E402


def main():
    assert binding.lib_path().endswith("libpagedattn_debug.so"), binding.lib_path()
    worst = 0.0
    w = build_workload(name="dbg", seed=31, kind="decode", dtype="bf16", Hq=32, Hkv=8, D=128, bs=16,
                       context_lens=[37, 300, 1000], append_lens=[1, 1, 1], threads=1)
    kp, vp = oracle.kv_append(w.k_pool, w.v_pool, w.k_new, w.v_new, w.slot_mapping, w.bs)
    ref = oracle.paged_attention(w.q, kp, vp, w.block_table, w.context_lens, w.cu_q_lens, w.scale, w.bs,
                                 w.dtype)
    for split in (0, -2, 64, -1):
        t = upload(w)
        binding.kv_append(t["k_new"], t["v_new"], t["k_cache"], t["v_cache"], t["slot_mapping"])
        out = torch.empty_like(t["q"])
        binding.paged_attn_decode(out, t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                                  w.scale, w.max_context_len, split)
        torch.cuda.synchronize()
        worst = max(worst, float(np.max(np.abs(bits_to_f64(to_numpy_bits(out), "bf16") - ref))))
        if split > 0:
            # the same decode as two calls: partials, then the merge alone (the
            # merge-only call has no block table; rows longer than one block)
            out2 = torch.full_like(t["q"], float("nan"))
            ws = binding.decode_workspace(t["q"], w.Hkv, w.max_context_len, split)
            for phase in ("partials", "merge"):
                binding.paged_attn_decode(out2, t["q"], t["k_cache"], t["v_cache"], t["block_tables"],
                                          t["context_lens"], w.scale, w.max_context_len, split, workspace=ws,
                                          phase=phase)
            torch.cuda.synchronize()
            worst = max(worst, float(np.max(np.abs(bits_to_f64(to_numpy_bits(out2), "bf16") - ref))))
        # block copy of two unused blocks onto two others, then nothing referenced changed
        used = set(np.asarray(w.block_table[w.block_table >= 0]).tolist())
        free = [b for b in range(w.NB) if b not in used][:4]
        binding.kv_copy_blocks(t["k_cache"], t["v_cache"], torch.tensor(free[:2], dtype=torch.int32, device="cuda"),
                               torch.tensor(free[2:], dtype=torch.int32, device="cuda"))
        torch.cuda.synchronize()
    wp = build_workload(name="dbgp", seed=32, kind="prefill", dtype="bf16", Hq=32, Hkv=8, D=128, bs=16,
                        context_lens=[150, 400], q_lens=[150, 170], append_lens=[150, 170], causal=True,
                        threads=1)
    kp, vp = oracle.kv_append(wp.k_pool, wp.v_pool, wp.k_new, wp.v_new, wp.slot_mapping, wp.bs)
    ref = oracle.paged_attention(wp.q, kp, vp, wp.block_table, wp.context_lens, wp.cu_q_lens, wp.scale, wp.bs,
                                 wp.dtype, oracle.ScoreMods(causal=True))
    t = upload(wp)
    binding.kv_append(t["k_new"], t["v_new"], t["k_cache"], t["v_cache"], t["slot_mapping"])
    out = torch.empty_like(t["q"])
    binding.paged_attn_prefill(out, t["q"], t["cu_q_lens"], t["k_cache"], t["v_cache"], t["block_tables"],
                               t["context_lens"], wp.scale, wp.max_q_len, True)
    torch.cuda.synchronize()
    worst = max(worst, float(np.max(np.abs(bits_to_f64(to_numpy_bits(out), "bf16") - ref))))
    # the same rows with their keys split into ranges of 64 and 192 keys
    # (total_q and the context bound are checked on the device), and a
    # context bound four times the longest context (the library's own split)
    for key_split, max_ctx in ((64, 400), (192, 400), (0, 1600)):
        out = torch.full_like(t["q"], float("nan"))
        binding.paged_attn_prefill(out, t["q"], t["cu_q_lens"], t["k_cache"], t["v_cache"], t["block_tables"],
                                   t["context_lens"], wp.scale, wp.max_q_len, True, max_context_len=max_ctx,
                                   key_split=key_split)
        torch.cuda.synchronize()
        worst = max(worst, float(np.max(np.abs(bits_to_f64(to_numpy_bits(out), "bf16") - ref))))
    # two-phase decode: three groups (one of a single empty sequence), a
    # prefix that ends inside a block, a sequence with no own keys
    wc = build_workload(name="dbgc", seed=33, kind="decode", dtype="bf16", Hq=32, Hkv=8, D=128, bs=16,
                        context_lens=[16 * 6 + 9, 16 * 6, 16 * 6 + 300, 0, 16 * 2 + 1, 16 * 2 + 40],
                        append_lens=[1, 0, 1, 0, 1, 1], prefix_groups=[(3, 6), (1, 0), (2, 2)], threads=1)
    kp, vp = oracle.kv_append(wc.k_pool, wc.v_pool, wc.k_new, wc.v_new, wc.slot_mapping, wc.bs)
    ref = oracle.paged_attention(wc.q, kp, vp, wc.block_table, wc.context_lens, wc.cu_q_lens, wc.scale, wc.bs,
                                 wc.dtype)
    t = upload(wc)
    binding.kv_append(t["k_new"], t["v_new"], t["k_cache"], t["v_cache"], t["slot_mapping"])
    out = torch.empty_like(t["q"])
    # two levels: the groups above, then the first group split in (2, 1) with
    # 3 more shared keys for the pair (inside the shared sixth block)
    starts = torch.tensor([0, 3, 4, 6], dtype=torch.int32, device="cuda")
    prefix = torch.tensor([16 * 6 - 5, 0, 32], dtype=torch.int32, device="cuda")
    starts2 = torch.tensor([0, 2, 3, 4, 6], dtype=torch.int32, device="cuda")
    lo2 = torch.tensor([16 * 6 - 5, 16 * 6 - 5, 0, 32], dtype=torch.int32, device="cuda")
    hi2 = torch.tensor([16 * 6 - 2, 16 * 6 - 5, 0, 32], dtype=torch.int32, device="cuda")
    levels = [binding.prefix_level(starts, prefix, 3, 96), binding.prefix_level(starts2, hi2, 2, 3, lo2)]
    binding.paged_attn_decode_cascade(out, t["q"], t["k_cache"], t["v_cache"], t["block_tables"],
                                      t["context_lens"], levels, wc.scale, wc.max_context_len, mode="two_phase")
    torch.cuda.synchronize()
    worst = max(worst, float(np.max(np.abs(bits_to_f64(to_numpy_bits(out), "bf16") - ref))))
    print(f"debug-check build: max abs err {worst:.3e}", flush=True)
    return 0 if worst <= 2e-2 else 1


if __name__ == "__main__":
    sys.exit(main())

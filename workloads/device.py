"""Upload a host :class:`~workloads.synth.Workload` to torch device tensors.

Plumbing only: bf16 bit patterns are reinterpreted (never converted) as
``torch.bfloat16``; every other array is copied as is.
"""

from __future__ import annotations

import numpy as np
import torch


def to_tensor(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Storage array -> tensor with the same bits (uint16 bf16 bits -> bfloat16)."""
    a = np.ascontiguousarray(a)
    if dtype == "bf16" and a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    if a.dtype == np.float32:
        return torch.from_numpy(a).to(device)
    if a.dtype == np.int32:
        return torch.from_numpy(a).to(device)
    raise TypeError(a.dtype)


def to_numpy_bits(t: torch.Tensor) -> np.ndarray:
    """Tensor -> host array of the same bits (bfloat16 -> uint16, float32 -> float32)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def upload(w, device="cuda"):
    """All inputs of ``w`` on ``device``; pools are fresh copies (kv_append writes them)."""
    d = w.dtype
    return {
        "q": to_tensor(w.q, d, device),
        "k_cache": to_tensor(w.k_pool, d, device),
        "v_cache": to_tensor(w.v_pool, d, device),
        "k_new": to_tensor(w.k_new, d, device),
        "v_new": to_tensor(w.v_new, d, device),
        "slot_mapping": to_tensor(w.slot_mapping, "i32", device),
        "block_tables": to_tensor(w.block_table, "i32", device),
        "context_lens": to_tensor(w.context_lens, "i32", device),
        "cu_q_lens": to_tensor(w.cu_q_lens, "i32", device),
    }

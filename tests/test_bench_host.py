"""Host-side logic of bench.py (no GPU): the command-line contract, the
algorithmic flop count of the chunked prefill, the fragmentation arithmetic
and the staleness rule of the stored HBM-traffic record."""

import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import named_workload  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_chunked_prefill_flops_by_hand():
    # 512 causal rows after 1536 keys: row i sees 1536 + i + 1 keys, so
    # sum_i (1537 + i) = 512 * 1536 + 512 * 513 / 2 = 917,760 pairs per
    # (sequence, head); 4 sequences x 32 heads x 4 * 128 flops per pair
    w = named_workload("chunked_prefill_bf16")
    assert bench.prefill_flops(w) == 4 * 128 * 32 * 4 * 917_760 == 60_146_319_360


def test_head_shard_keeps_lengths_tables_and_one_eighth_of_the_heads():
    """One GPU's share of an 8-way head split: the same lengths and block
    tables, Hq/8 and Hkv/8 heads, 1/8 of the algorithmic flops; a split that
    does not divide the heads is refused."""
    import pytest
    full = named_workload("chunked_prefill_bf16")
    part = named_workload("chunked_prefill_bf16", tp=8)
    assert (part.Hq, part.Hkv) == (4, 1)
    assert np.array_equal(part.context_lens, full.context_lens)
    assert np.array_equal(part.block_table, full.block_table)
    assert bench.prefill_flops(part) * 8 == bench.prefill_flops(full)
    with pytest.raises(ValueError):
        named_workload("chunked_prefill_bf16", tp=3)


def test_fragmentation_arithmetic():
    # lengths 1, 16, 17: slots held at page 16 are 16 + 16 + 32 = 64, unused
    # 15 + 0 + 15 = 30; at page 32: 32 * 3 = 96 held, 31 + 16 + 15 = 62 unused
    f = bench.fragmentation(np.array([1, 16, 17]))
    assert f["16"] == round(30 / 64, 5)
    assert f["32"] == round(62 / 96, 5)
    assert set(f) == {"16", "32", "64", "128", "256", "doubling_16_256"}
    # pages doubling from 16 to 256 tokens: capacities 16, 48, 112, 240, 496, 752, ...
    # lengths 1, 16, 17, 500 hold 16, 16, 48, 752 slots, 15 + 0 + 31 + 252 unused
    g = bench.fragmentation(np.array([1, 16, 17, 500]))
    assert g["doubling_16_256"] == round(298 / 832, 5)


def test_traffic_record_only_for_the_current_kernel_source(tmp_path, monkeypatch):
    rec = {"kernel_source_sha256_16": bench.kernel_source_hash(), "hbm_bytes_per_launch": 1}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.traffic_record()["hbm_bytes_per_launch"] == 1
    rec["kernel_source_sha256_16"] = "0" * 16
    path.write_text(json.dumps(rec))
    assert bench.traffic_record() is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.traffic_record() is None

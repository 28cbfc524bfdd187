"""Benchmark of the paged-attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  1. kv_append of one new token per sequence of the long-context decode batch
     (64 sequences, log-normal contexts around 8192 tokens, 64 query / 8 KV
     heads, head_dim 128, bf16, 16-token blocks scattered in a ~5.6 GB pool),
  2. paged decode of that batch with split-KV (partition kernel, then the
     merge kernel); by default the library's balanced split, which gives every
     wavefront an equal share of the batch's 16-token chunks; ``--split 512``
     selects fixed 512-token partitions instead (also measured and reported
     under ``decode_fixed_split``),
  3. kv_append of a 512-token chunk for each of 4 sequences, and
  4. causal chunked prefill of those chunks after their 1536-token contexts
     (32 query / 8 KV heads, head_dim 128, bf16, matrix cores).

The headline ``value`` is the decode KV-read bandwidth: bytes of K and V the
decode batch must read (sum of context lengths x 8 kv-heads x 128 x 2 x 2)
divided by the measured time of the decode call (both kernels).  The prefill
throughput is reported beside it.  Inputs are resident in HBM before timing.
Before every step a 512 MiB buffer is overwritten (evicting L2 and the
last-level cache; not part of any phase).  Per-kernel times come from HIP
events recorded on the stream the kernels run on.  Every output row of the
timed step (all decode rows, all prefill rows) is compared with the fp64 CPU
oracle afterwards: the max-abs errors go into ``parity`` and the run fails
(exit status 3) above 2e-2.  ``cpu_baseline`` times that oracle on a bounded
sample of the same workload.

Beside the step it reports: the achievable HBM read bandwidth of a plain
streaming-read kernel (a second denominator), the decode of the other
workloads (GQA batch, shared-prefix batch with logical and unique bytes), the
two-phase decode of two shared-prefix batches beside their plain decode, a
context sweep of the GQA shape, the pool's internal fragmentation per
workload and page size (arithmetic only), and one GPU's share of an 8-way
head split (the decode, and the prefill unsplit and over key ranges).

Prints one JSON line.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PARITY_TOL = 2e-2           # max-abs error bar for bf16 inputs, fp32 accumulation
METRIC = "paged decode KV-read GB/s (% of HBM peak) + paged prefill TFLOP/s, 1 MI355X"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_partials_traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "paged_kv_cache_attn_amd", "csrc", f)
                  for f in ("decode.hip", "pa_device.h", "pa_kernels.h")]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def prefill_flops(w) -> float:
    """4*D flops (q.k and p.v) per admissible (query row, key) pair, every head."""
    total = 0
    for b in range(w.B):
        n = int(w.context_lens[b])
        L = int(w.q_lens[b])
        pos = np.arange(n - L, n)
        keys = np.minimum(n, pos + 1) if w.causal else np.full(L, n)
        total += int(keys.sum())
    return 4.0 * w.D * w.Hq * total


def traffic_record():
    """HBM bytes per launch of the partition kernel measured with rocprofv3
    counters, if they were taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec


def oracle_reference(w5, w3, budget_s):
    """The fp64 oracle over every row the step computes: all decode rows of
    the long batch (append + attention, each sequence on a compact copy of
    its blocks, so the multi-GB pool is never widened) and every chunked-
    prefill row.  Returns the reference outputs and, as ``cpu_baseline``, the
    oracle's own speed on the host: the decode sequences done within
    ``budget_s`` seconds (0: none timed) and the prefill batch."""
    import threadpoolctl

    import oracle

    info = threadpoolctl.threadpool_info()
    cores = max([i.get("num_threads", 1) for i in info] + [1])

    ref5 = np.full(w5.q.shape, np.nan, dtype=np.float64)
    timed, t_dec, bytes_dec = [], 0.0, 0
    for b in range(w5.B):
        nb = (int(w5.context_lens[b]) + w5.bs - 1) // w5.bs
        ids = w5.block_table[b, :nb].astype(np.int64)
        kp, vp = w5.k_pool[ids], w5.v_pool[ids]
        table = np.arange(nb, dtype=np.int32)[None]
        s = int(w5.slot_mapping[b])
        slot = np.array([int(np.nonzero(ids == s // w5.bs)[0][0]) * w5.bs + s % w5.bs], np.int32)
        t0 = time.perf_counter()
        kp2, vp2 = oracle.kv_append(kp, vp, w5.k_new[b:b + 1], w5.v_new[b:b + 1], slot, w5.bs)
        ref5[b:b + 1] = oracle.paged_attention(w5.q[b:b + 1], kp2, vp2, table, w5.context_lens[b:b + 1],
                                               np.array([0, 1]), w5.scale, w5.bs, w5.dtype)
        dt = time.perf_counter() - t0
        if t_dec < budget_s * 0.6:
            t_dec += dt
            timed.append(b)
            bytes_dec += int(w5.context_lens[b]) * w5.Hkv * w5.D * 2 * 2
    t0 = time.perf_counter()
    kp, vp = oracle.kv_append(w3.k_pool, w3.v_pool, w3.k_new, w3.v_new, w3.slot_mapping, w3.bs)
    ref3 = oracle.paged_attention(w3.q, kp, vp, w3.block_table, w3.context_lens, w3.cu_q_lens,
                                  w3.scale, w3.bs, w3.dtype, oracle.ScoreMods(causal=True))
    t_pre = time.perf_counter() - t0
    base = None
    if timed:
        base = {
            "value": round(bytes_dec / t_dec / 1e9, 4),
            "unit": "GB/s",
            "cores": int(cores),
            "kind": "oracle",
            "sample": (f"decode: {len(timed)} of {w5.B} sequences of the long-context batch "
                       f"({sum(int(w5.context_lens[b]) for b in timed)} tokens, kv_append + fp64 attention) in "
                       f"{t_dec:.2f} s; prefill: all {w3.B} chunked-prefill sequences (append + fp64 attention) "
                       f"in {t_pre:.2f} s"),
            "prefill_tflops": round(prefill_flops(w3) / t_pre / 1e12, 6),
        }
    return ref5, ref3, base


def max_abs_err(out, ref):
    """Largest |GPU - oracle| over every element (bf16 output read exactly)."""
    from oracle.paged import bits_to_f64
    from workloads.device import to_numpy_bits
    return float(np.max(np.abs(bits_to_f64(to_numpy_bits(out), "bf16") - ref)))


PAGE_SIZES = (16, 32, 64, 128, 256)


def fragmentation(context_lens):
    """Internal fragmentation of a paged pool: unused slots of every sequence's
    last page over all slots it holds (pure arithmetic), per fixed page size,
    and for pages that double along each sequence from 16 to 256 tokens
    (the block manager's 1..16-block pages on 16-token blocks: power-of-two
    growth)."""
    n = np.asarray(context_lens, dtype=np.int64)
    out = {}
    for bs in PAGE_SIZES:
        held = ((n + bs - 1) // bs) * bs
        out[str(bs)] = round(float((held - n).sum() / held.sum()), 5)
    page, held = 16, np.zeros_like(n)
    while np.any(held < n):
        held = np.where(held < n, held + page, held)
        page = min(2 * page, 256)
    out["doubling_16_256"] = round(float((held - n).sum() / max(held.sum(), 1)), 5)
    return out


class _HipTimer:
    """HIP events made with hipEventDisableSystemFence: recording one writes a
    timestamp without the system-scope cache write-back and invalidation a
    default event performs, which adds several microseconds between
    consecutive kernels (the runtime's own note on the flag: it improves the
    accuracy of timing).  Bound through ctypes to the HIP runtime torch has
    already loaded, so the events live on the same runtime and stream as the
    kernels."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            raise RuntimeError("the HIP runtime is not loaded")
        self.c = ctypes
        L = ctypes.CDLL(path)
        L.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        L.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        L.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.L = L

    def event(self):
        return _HipEvent(self)


class _HipEvent:
    def __init__(self, timer):
        self.t = timer
        self.h = timer.c.c_void_p()
        if timer.L.hipEventCreateWithFlags(timer.c.byref(self.h), _HipTimer.DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")

    def record(self, stream):
        if self.t.L.hipEventRecord(self.h, self.t.c.c_void_p(stream.cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_time(self, other):
        ms = self.t.c.c_float()
        if self.t.L.hipEventElapsedTime(self.t.c.byref(ms), self.h, other.h) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def __del__(self):
        try:
            self.t.L.hipEventDestroy(self.h)
        except Exception:
            pass


_TIMER = None


def new_event(torch):
    """A timing event on the kernels' stream: fence-free HIP event by default,
    torch's (default HIP flags) with --event-fence system."""
    if _TIMER is None:
        return torch.cuda.Event(enable_timing=True)
    return _TIMER.event()


def time_calls(torch, fn, flush, reps, warm=3):
    """Median GPU time (ms) of ``fn``, each call after a cache-evicting flush;
    events bracket only the call, and the flush keeps the GPU busy while the
    host enqueues it."""
    stream = torch.cuda.current_stream()
    for _ in range(warm):
        flush()
        fn()
    evs = []
    for _ in range(reps):
        flush()
        a = new_event(torch)
        b = new_event(torch)
        a.record(stream)
        fn()
        b.record(stream)
        evs.append((a, b))
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in evs]))


def calibration_copy(args, torch, dev):
    """One plain device copy of --calibration-copy-mib MiB: a known-size
    reference for the HBM traffic counters."""
    if args.calibration_copy_mib > 0:
        nbytes = args.calibration_copy_mib << 20
        src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"calibration copy of {args.calibration_copy_mib} MiB done")


def shared_prefix_long():
    """64 sequences behind one 16384-token prompt (1024 shared 16-token
    blocks) with 1024 own tokens each (the last appended this step), 64/8
    heads, d128, bf16."""
    from workloads import build_workload
    return build_workload(name="shared_prefix_16k_b64", seed=6, kind="decode", dtype="bf16", Hq=64, Hkv=8, D=128,
                          bs=16, context_lens=[16384 + 1024] * 64, append_lens=[1] * 64,
                          shared_prefix_blocks=16384 // 16, pool_slack=1.05)


def two_phase_call(pa, torch, dev, w, t, out, pre, mode="two_phase"):
    """(workspace, call) of the shared-prefix decode of a batch that is one
    group sharing its first ``pre`` tokens: forced two-phase, or the library's
    default choice (``mode="auto"``)."""
    gs = torch.tensor([0, w.B], dtype=torch.int32, device=dev)
    pl = torch.tensor([pre], dtype=torch.int32, device=dev)
    levels = [pa.prefix_level(gs, pl, w.B, pre)]
    ws2 = pa.decode_cascade_workspace(t["q"], w.Hkv, levels, w.max_context_len)

    def call():
        pa.paged_attn_decode_cascade(out, t["q"], t["k_cache"], t["v_cache"], t["block_tables"],
                                     t["context_lens"], levels, w.scale, w.max_context_len, workspace=ws2, mode=mode)
    call.plan = pa.decode_cascade_plan(w.B, levels, w.Hq, w.Hkv, w.D, w.max_context_len)
    return ws2, call


def two_phase_main(args, pa, torch, dev):
    """``--path two_phase``: the two-phase decode of the long shared-prompt
    batch as the step (its own JSON line; the plain decode of the same batch
    is timed beside it)."""
    from workloads.device import upload
    w = shared_prefix_long()
    t = upload(w, dev)
    pa.kv_append(t["k_new"], t["v_new"], t["k_cache"], t["v_cache"], t["slot_mapping"])
    out = torch.empty_like(t["q"])
    flush_buf = torch.empty(max(1, args.flush_mib) << 18, dtype=torch.int32, device=dev)

    def flush():
        if args.flush_mib > 0:
            pa.bench_fill(flush_buf, 0)
    calibration_copy(args, torch, dev)
    ws2, call = two_phase_call(pa, torch, dev, w, t, out, 16384)
    ws = pa.decode_workspace(t["q"], w.Hkv, w.max_context_len, 0)

    def plain():
        pa.paged_attn_decode(out, t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                             w.scale, w.max_context_len, 0, workspace=ws)
    ms_plain = time_calls(torch, plain, flush, reps=5)
    for _ in range(args.warmup):
        flush()
        call()
    ms = time_calls(torch, call, flush, reps=args.steps, warm=0)
    unique = w.unique_kv_bytes()
    print(json.dumps({
        "metric": "two-phase shared-prefix decode: unique KV-read GB/s, 1 MI355X", "value": round(
            unique / (ms * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "shared_prefix_16k_b64: 64 sequences, 16384 shared + 1024 own tokens, h64x8, d128, "
                               "block 16, one group", "kv_bytes": int(w.kv_bytes()), "unique_kv_bytes": int(unique),
                   "prefix_flops": 4.0 * w.B * w.Hq * 16384 * w.D},
        "plain_decode_ms": round(ms_plain, 5), "speedup_vs_plain_decode": round(ms_plain / ms, 3)}), flush=True)


def small_decode_main(args, pa, torch, dev):
    """``--path small_decode``: the decode of the three small workloads alone
    (single-sequence fp32, GQA batch with its append, shared-prefix batch
    plain, two-phase and default), ``--steps`` calls each after a
    cache-evicting write; one JSON line.  Made for kernel traces of these
    workloads."""
    from workloads import named_workload
    from workloads.device import upload
    flush_buf = torch.empty(max(1, args.flush_mib) << 18, dtype=torch.int32, device=dev)

    def flush():
        if args.flush_mib > 0:
            pa.bench_fill(flush_buf, 0)
    res = {}
    for name in ("single_decode_f32", "gqa_decode_bf16", "shared_prefix_decode_bf16"):
        w = named_workload(name)
        t = upload(w, dev)
        out = torch.empty_like(t["q"])
        ws = pa.decode_workspace(t["q"], w.Hkv, w.max_context_len, 0)
        has_append = len(w.slot_mapping) > 0

        def append():
            if has_append:
                pa.kv_append(t["k_new"], t["v_new"], t["k_cache"], t["v_cache"], t["slot_mapping"])

        def decode(split=0, ws=ws):
            pa.paged_attn_decode(out, t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                                 w.scale, w.max_context_len, split, workspace=ws)
        append()
        entry = {"kv_bytes": int(w.kv_bytes()),
                 "append_ms": round(time_calls(torch, append, flush, reps=args.steps), 5) if has_append else None,
                 "decode_ms": round(time_calls(torch, decode, flush, reps=args.steps), 5),
                 "decode_split": int(pa.decode_split_tokens(w.B, w.Hkv, w.max_context_len, 0))}
        entry["decode_gbs"] = round(w.kv_bytes() / (entry["decode_ms"] * 1e-3) / 1e9, 2)
        ws_f = pa.decode_workspace(t["q"], w.Hkv, w.max_context_len, 512)
        entry["fixed_512_split_ms"] = round(time_calls(torch, lambda: decode(512, ws_f), flush, reps=args.steps), 5)
        if name == "shared_prefix_decode_bf16":
            for mode in ("two_phase", "auto"):
                _, call = two_phase_call(pa, torch, dev, w, t, out, 1024, mode=mode)
                entry[f"{mode}_ms"] = round(time_calls(torch, call, flush, reps=args.steps), 5)
            entry["unique_kv_bytes"] = int(w.unique_kv_bytes())
        res[name] = entry
        log(f"{name}: {entry}")
        del t, out, ws
    print(json.dumps({"metric": "small-batch paged decode latency, 1 MI355X", "unit": "ms", "n_gpus": 1,
                      "steps": args.steps, "higher_is_better": False, "data": "synthetic", "dtype": "bf16/f32",
                      "workloads": res}), flush=True)


def extra_measurements(pa, torch, dev, flush, args):
    from workloads import build_workload, named_workload
    from workloads.device import upload

    res = {}
    # achievable HBM read bandwidth: one streaming read of 4 GiB (16x the last-level cache)
    src = torch.ones(1 << 30, dtype=torch.int32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    ms = time_calls(torch, lambda: pa.bench_stream_read(src, sink), flush, reps=7)
    res["achievable_hbm"] = {"value": round(src.numel() * 4 / (ms * 1e-3) / 1e9, 2), "unit": "GB/s",
                             "kernel": "stream_read_kernel (measurement support), 4 GiB, 16-byte non-temporal loads",
                             "ms": round(ms, 5)}
    del src, sink
    log(f"achievable HBM read: {res['achievable_hbm']['value']} GB/s")

    def decode_fn(w, t, out, ws):
        def f():
            pa.paged_attn_decode(out, t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                                 w.scale, w.max_context_len, 0, workspace=ws)
        return f

    def prepared(w):
        t = upload(w, dev)
        if len(w.slot_mapping):
            pa.kv_append(t["k_new"], t["v_new"], t["k_cache"], t["v_cache"], t["slot_mapping"])
        out = torch.empty_like(t["q"])
        ws = pa.decode_workspace(t["q"], w.Hkv, w.max_context_len, 0)
        return t, out, ws

    workloads = {}
    frag = {}
    for name in ("single_decode_f32", "gqa_decode_bf16", "shared_prefix_decode_bf16"):
        w = named_workload(name)
        frag[name] = fragmentation(w.context_lens)
        t, out, ws = prepared(w)
        ms = time_calls(torch, decode_fn(w, t, out, ws), flush, reps=20)
        logical = w.kv_bytes()
        entry = {"ms": round(ms, 5), "kv_bytes": int(logical), "gbs": round(logical / (ms * 1e-3) / 1e9, 2)}
        if name == "shared_prefix_decode_bf16":
            unique = w.unique_kv_bytes()
            entry.update({"unique_kv_bytes": int(unique),
                          "unique_gbs": round(unique / (ms * 1e-3) / 1e9, 2),
                          "pct_hbm_peak_unique": round(100.0 * unique / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)})
        workloads[name] = entry
        del t, out, ws
    res["decode_workloads"] = workloads
    res["fragmentation"] = frag
    log("other workloads measured")

    # two-phase decode of batches that share a prefix, beside the plain decode
    # of the same batch: the shared-prefix workload (16 sequences, 1024 shared
    # + 256 own tokens, 32/8 heads) and a long shared prompt (64 sequences,
    # 16384 shared + 1024 own tokens, 64/8 heads), d128, bf16, block 16
    two = {}
    for name, w, pre in (("shared_prefix_decode_bf16", named_workload("shared_prefix_decode_bf16"), 1024),
                         ("shared_prefix_16k_b64", shared_prefix_long(), 16384)):
        t, out, ws = prepared(w)
        ms_plain = time_calls(torch, decode_fn(w, t, out, ws), flush, reps=20)
        ws2, two_phase = two_phase_call(pa, torch, dev, w, t, out, pre)
        ms_two = time_calls(torch, two_phase, flush, reps=20)
        ws3, auto = two_phase_call(pa, torch, dev, w, t, out, pre, mode="auto")
        ms_auto = time_calls(torch, auto, flush, reps=20)
        unique = w.unique_kv_bytes()
        prefix_flops = 4.0 * w.B * w.Hq * pre * w.D
        two[name] = {"plain_ms": round(ms_plain, 5), "two_phase_ms": round(ms_two, 5),
                     "speedup": round(ms_plain / ms_two, 3),
                     "default_call": "two_phase" if auto.plan else "plain decode",
                     "default_call_ms": round(ms_auto, 5), "default_speedup": round(ms_plain / ms_auto, 3),
                     "kv_bytes": int(w.kv_bytes()),
                     "unique_kv_bytes": int(unique),
                     "two_phase_unique_gbs": round(unique / (ms_two * 1e-3) / 1e9, 2),
                     "prefix_flops": prefix_flops}
        del t, out, ws, ws2, ws3
    res["shared_prefix_two_phase"] = two
    log("two-phase decode measured")

    # block-sparse chunked prefill: the chunked-prefill batch under seeded
    # block masks of 64-position query blocks x 128-key blocks (each query
    # block keeps its own diagonal block); work counted on admitted pairs
    w3 = named_workload("chunked_prefill_bf16")
    t3 = upload(w3, dev)
    pa.kv_append(t3["k_new"], t3["v_new"], t3["k_cache"], t3["v_cache"], t3["slot_mapping"])
    out3 = torch.empty_like(t3["q"])
    sparse = {}
    for density in (1.0, 0.5, 0.25):
        rng = np.random.default_rng(77)
        qb, kvb, n = 64, 128, int(w3.context_lens.max())
        dense = rng.random((w3.B, n // qb, n // kvb)) < density
        for r in range(n // qb):
            dense[:, r, (r * qb) // kvb] = True
        words = (n // kvb + 31) // 32
        padded = np.zeros((w3.B * (n // qb), words * 32), dtype=bool)
        padded[:, :n // kvb] = dense.reshape(w3.B * (n // qb), -1)
        bits = np.packbits(padded, axis=1, bitorder="little").view("<i4").reshape(w3.B, n // qb, words)
        bm = pa.block_mask(torch.from_numpy(np.ascontiguousarray(bits)).to(dev), qb, kvb)
        pairs = 0
        for b in range(w3.B):
            L = int(w3.q_lens[b])
            pos = np.arange(n - L, n)
            keys = np.arange(n)
            ok = (keys[None, :] <= pos[:, None]) & dense[b][pos // qb][:, keys // kvb]
            pairs += int(ok.sum())

        def call(bm=bm):
            pa.paged_attn_prefill(out3, t3["q"], t3["cu_q_lens"], t3["k_cache"], t3["v_cache"], t3["block_tables"],
                                  t3["context_lens"], w3.scale, w3.max_q_len, causal=True, block_mask=bm)
        ms = time_calls(torch, call, flush, reps=20)
        fl = 4.0 * w3.D * w3.Hq * pairs
        sparse[str(density)] = {"ms": round(ms, 5), "admitted_flops": fl, "tflops": round(fl / (ms * 1e-3) / 1e12, 2)}
    res["block_mask_prefill"] = {"workload": "chunked_prefill_bf16, block mask 64-position query blocks x 128-key "
                                             "blocks, seeded, diagonal blocks kept", "density": sparse}
    del t3, out3
    log("block-sparse prefill measured")

    # context sweep of the GQA decode shape (8 sequences, 32/8 heads, d128, bf16, block 16)
    sweep = {}
    base = None
    for ctx in (128, 256, 512, 1024, 2048):
        w = build_workload(name=f"sweep{ctx}", seed=200 + ctx, kind="decode", dtype="bf16", Hq=32, Hkv=8, D=128,
                           bs=16, context_lens=[ctx] * 8, append_lens=[1] * 8)
        t, out, ws = prepared(w)
        ms = time_calls(torch, decode_fn(w, t, out, ws), flush, reps=20)
        base = base or ms
        sweep[str(ctx)] = {"us": round(ms * 1e3, 2), "vs_128": round(ms / base, 3),
                           "gbs": round(w.kv_bytes() / (ms * 1e-3) / 1e9, 2)}
        del t, out, ws
    res["context_sweep_gqa_decode"] = sweep
    log("context sweep measured")

    # one GPU's share of an 8-way split over heads: the long-context batch
    # with 8/1 heads and the chunked prefill with 4/1 heads (same lengths
    # and tables); the exchange between GPUs is not part of it
    shard = {}
    w = named_workload("long_decode_bf16", tp=8)
    t, out, ws = prepared(w)
    ms = time_calls(torch, decode_fn(w, t, out, ws), flush, reps=10)
    shard["long_decode_bf16"] = {"heads": f"{w.Hq}/{w.Hkv}", "ms": round(ms, 5), "kv_bytes": int(w.kv_bytes()),
                                 "gbs": round(w.kv_bytes() / (ms * 1e-3) / 1e9, 2)}
    del t, out, ws, w
    w = named_workload("chunked_prefill_bf16", tp=8)
    t = upload(w, dev)
    pa.kv_append(t["k_new"], t["v_new"], t["k_cache"], t["v_cache"], t["slot_mapping"])
    out = torch.empty_like(t["q"])

    max_ctx = int(w.context_lens.max())
    ws = pa.prefill_workspace(t["q"], w.B, w.Hkv, w.max_q_len, max_ctx)

    def prefill_call(split):
        kw = {"max_context_len": max_ctx, "workspace": ws} if split else {}
        return lambda: pa.paged_attn_prefill(out, t["q"], t["cu_q_lens"], t["k_cache"], t["v_cache"],
                                             t["block_tables"], t["context_lens"], w.scale, w.max_q_len, causal=True,
                                             **kw)
    fl = prefill_flops(w)
    entry = {"heads": f"{w.Hq}/{w.Hkv}", "flops": fl}
    for label, split in (("unsplit", False), ("key_split", True)):
        ms = time_calls(torch, prefill_call(split), flush, reps=20)
        entry[label] = {"ms": round(ms, 5), "tflops": round(fl / (ms * 1e-3) / 1e12, 2)}
    entry["key_split"]["workspace_bytes"] = 0 if ws is None else int(ws.numel() * 4)
    shard["chunked_prefill_bf16"] = entry
    del t, out, w, ws
    res["tp8_shard"] = shard
    log("8-way head shard measured")
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--page-size", type=int, default=16, help="block size of the decode pool (16..256)")
    ap.add_argument("--split", type=int, default=0,
                    help="decode split-KV: 0 balanced (default), -1 unsplit, else fixed partition length")
    ap.add_argument("--fixed-split", type=int, default=512,
                    help="fixed partition length measured beside the default (0: skip)")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (a known-size reference for "
                         "HBM traffic counters)")
    ap.add_argument("--cpu-baseline-seconds", type=float, default=15.0,
                    help="time budget of the oracle baseline's decode sample (0: no baseline)")
    ap.add_argument("--parity", type=int, default=1,
                    help="1: check every output row of the timed step against the fp64 oracle and fail "
                         "above the tolerance (0: skip)")
    ap.add_argument("--flush-mib", type=int, default=512,
                    help="cache-evicting write before every timed call (0: none)")
    ap.add_argument("--path", choices=("step", "two_phase", "small_decode"), default="step",
                    help="step: the hot-path step (default); two_phase: the two-phase decode of a "
                         "long shared-prompt batch; small_decode: the decode of the three small workloads")
    ap.add_argument("--event-fence", choices=("none", "system"), default="none",
                    help="timing events: none = HIP events without the system-scope fence (default); "
                         "system = torch's events with HIP's default flags")
    ap.add_argument("--extras", type=int, default=1,
                    help="1: also measure achievable HBM, the other workloads and the context sweep")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_kv_cache_attn_amd as pa
    from workloads import named_workload
    from workloads.device import upload

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pa.lib()
    global _TIMER
    if args.event_fence == "none":
        torch.zeros(1, device=dev)  # the HIP runtime is loaded and initialised
        _TIMER = _HipTimer()
    if args.path == "two_phase":
        two_phase_main(args, pa, torch, dev)
        return
    if args.path == "small_decode":
        small_decode_main(args, pa, torch, dev)
        return

    log("generating long-context decode batch")
    t0 = time.time()
    w5 = named_workload("long_decode_bf16", bs=args.page_size)
    w3 = named_workload("chunked_prefill_bf16")
    log(f"inputs generated in {time.time() - t0:.1f} s; uploading")
    t5 = upload(w5, dev)
    t3 = upload(w3, dev)
    out5 = torch.empty_like(t5["q"])
    out3 = torch.empty_like(t3["q"])
    ws = pa.decode_workspace(t5["q"], w5.Hkv, w5.max_context_len, args.split)
    torch.cuda.synchronize()
    log("inputs resident on the GPU")

    stream = torch.cuda.current_stream()
    flush_buf = (torch.empty(args.flush_mib << 18, dtype=torch.int32, device=dev)
                 if args.flush_mib > 0 else None)

    def flush():
        if flush_buf is not None:
            pa.bench_fill(flush_buf, 0)

    def step(ev=None):
        flush()
        if ev is not None:
            ev[0].record(stream)
        pa.kv_append(t5["k_new"], t5["v_new"], t5["k_cache"], t5["v_cache"], t5["slot_mapping"])
        if ev is not None:
            ev[1].record(stream)
        pa.paged_attn_decode(out5, t5["q"], t5["k_cache"], t5["v_cache"], t5["block_tables"], t5["context_lens"],
                             w5.scale, w5.max_context_len, args.split, workspace=ws, phase="partials")
        if ev is not None:
            ev[2].record(stream)
        pa.paged_attn_decode(out5, t5["q"], t5["k_cache"], t5["v_cache"], t5["block_tables"], t5["context_lens"],
                             w5.scale, w5.max_context_len, args.split, workspace=ws, phase="merge")
        if ev is not None:
            ev[3].record(stream)
        pa.kv_append(t3["k_new"], t3["v_new"], t3["k_cache"], t3["v_cache"], t3["slot_mapping"])
        if ev is not None:
            ev[4].record(stream)
        pa.paged_attn_prefill(out3, t3["q"], t3["cu_q_lens"], t3["k_cache"], t3["v_cache"], t3["block_tables"],
                              t3["context_lens"], w3.scale, w3.max_q_len, causal=True)
        if ev is not None:
            ev[5].record(stream)

    calibration_copy(args, torch, dev)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")

    events = [[new_event(torch) for _ in range(6)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_begin = time.perf_counter()
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    t_end = time.perf_counter()
    log(f"timed {args.steps} steps")
    # the timed step's outputs, kept for the parity check against the oracle
    out5_step, out3_step = out5.clone(), out3.clone()

    def phase_ms(i, j):
        return float(np.mean([e[i].elapsed_time(e[j]) for e in events]))

    ms_append5 = phase_ms(0, 1)
    ms_partials = phase_ms(1, 2)
    ms_merge = phase_ms(2, 3)
    ms_append3 = phase_ms(3, 4)
    ms_prefill = phase_ms(4, 5)
    ms_step = (t_end - t_begin) * 1e3 / args.steps
    ms_decode = ms_partials + ms_merge

    kv_bytes = w5.kv_bytes()
    decode_gbs = kv_bytes / (ms_decode * 1e-3) / 1e9
    partials_gbs = kv_bytes / (ms_partials * 1e-3) / 1e9
    flops = prefill_flops(w3)
    prefill_tflops = flops / (ms_prefill * 1e-3) / 1e12
    append_bytes5 = 2 * 2 * w5.k_new.size * 2  # read new + write pool, K and V
    append_bytes3 = 2 * 2 * w3.k_new.size * 2

    fixed = None
    if args.fixed_split > 0 and args.fixed_split != args.split:
        ws_f = pa.decode_workspace(t5["q"], w5.Hkv, w5.max_context_len, args.fixed_split)
        evs = []
        for k in range(args.warmup + args.steps):
            e = [new_event(torch) for _ in range(3)]
            e[0].record(stream)
            pa.paged_attn_decode(out5, t5["q"], t5["k_cache"], t5["v_cache"], t5["block_tables"],
                                 t5["context_lens"], w5.scale, w5.max_context_len, args.fixed_split, workspace=ws_f,
                                 phase="partials")
            e[1].record(stream)
            pa.paged_attn_decode(out5, t5["q"], t5["k_cache"], t5["v_cache"], t5["block_tables"],
                                 t5["context_lens"], w5.scale, w5.max_context_len, args.fixed_split, workspace=ws_f,
                                 phase="merge")
            e[2].record(stream)
            if k >= args.warmup:
                evs.append(e)
        torch.cuda.synchronize()
        out5_fixed = out5.clone()
        f_part = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
        f_merge = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
        fixed = {
            "split_tokens": args.fixed_split,
            "value": round(w5.kv_bytes() / ((f_part + f_merge) * 1e-3) / 1e9, 2),
            "unit": "GB/s",
            "partitions_ms": round(f_part, 5),
            "merge_ms": round(f_merge, 5),
        }
        del ws_f

    traffic = None
    rec = traffic_record()
    if rec is not None:
        traffic = rec["hbm_bytes_per_launch"]

    result = {
        "metric": METRIC,
        "value": round(decode_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "long_decode_bf16_b64_lognormal8192_h64x8_d128"
            + ("" if args.page_size == 16 else f"_bs{args.page_size}")
            + " + chunked_prefill_bf16_b4_ctx1536+512_h32x8_d128_causal",
            "decode_batch": w5.B,
            "decode_context_tokens": int(w5.context_lens.sum()),
            "decode_kv_bytes": int(kv_bytes),
            "heads_q_kv": [w5.Hq, w5.Hkv],
            "head_dim": w5.D,
            "block_size": w5.bs,
            "split_tokens": int(pa.decode_split_tokens(w5.B, w5.Hkv, w5.max_context_len, args.split)),
            "prefill_batch": w3.B,
            "prefill_rows": int(w3.q_lens.sum()),
            "prefill_flops": flops,
            "parallelism": "single GPU",
        },
        "decode_pct_hbm_peak": round(100.0 * decode_gbs / HBM_PEAK_GBS, 2),
        "roofline": {
            "kernel": ("decode_stream_kernel<BF16,128,8>" if args.split == 0 else "row_partials_kernel<BF16,128,8>")
            + " (decode partitions)",
            "bound": "hbm",
            "achieved": round(partials_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(partials_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "avg_launch_ms": round(ms_partials, 5),
            "algorithmic_bytes_per_launch": int(kv_bytes),
        },
        "prefill": {
            "value": round(prefill_tflops, 2),
            "unit": "TFLOP/s",
            "ms": round(ms_prefill, 5),
            "roofline": {
                "kernel": "prefill_mfma_kernel<128> (chunked prefill)",
                "bound": "mfma",
                "achieved": round(prefill_tflops, 2),
                "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s",
                "frac": round(prefill_tflops / BF16_PEAK_TFLOPS, 4),
                "algorithmic_flops_per_launch": flops,
            },
        },
        "timing_events": ("HIP events created with hipEventDisableSystemFence (no cache write-back between "
                          "kernels)" if args.event_fence == "none" else "torch.cuda.Event (HIP default flags)"),
        "phases_ms": {
            "kv_append_decode_batch": round(ms_append5, 5),
            "decode_partitions": round(ms_partials, 5),
            "decode_merge": round(ms_merge, 5),
            "kv_append_prefill_chunks": round(ms_append3, 5),
            "prefill": round(ms_prefill, 5),
        },
        "decode_fixed_split": fixed,
        "kv_append_gbs": {
            "decode_batch": round(append_bytes5 / (ms_append5 * 1e-3) / 1e9, 2),
            "prefill_chunks": round(append_bytes3 / (ms_append3 * 1e-3) / 1e9, 2),
        },
    }
    if args.extras:
        extra = extra_measurements(pa, torch, dev, flush, args)
        result["roofline"]["achievable_peak"] = extra["achievable_hbm"]["value"]
        result["roofline"]["frac_of_achievable"] = round(partials_gbs / extra["achievable_hbm"]["value"], 4)
        result.update(extra)
        result["fragmentation"]["long_decode_bf16"] = fragmentation(w5.context_lens)
        result["fragmentation"]["chunked_prefill_bf16"] = fragmentation(w3.context_lens)
    failed = False
    if args.parity:
        log("fp64 oracle on the host: every decode and prefill row of the step")
        ref5, ref3, base = oracle_reference(w5, w3, args.cpu_baseline_seconds)
        result["cpu_baseline"] = base
        par = {"tolerance": PARITY_TOL, "decode_rows": int(w5.B), "prefill_rows": int(w3.q_lens.sum()),
               "decode_max_abs_err": max_abs_err(out5_step, ref5),
               "prefill_max_abs_err": max_abs_err(out3_step, ref3)}
        if fixed is not None:
            fixed["max_abs_err"] = max_abs_err(out5_fixed, ref5)
            par["decode_fixed_split_max_abs_err"] = fixed["max_abs_err"]
        result["parity"] = par
        errs = [v for k, v in par.items() if k.endswith("max_abs_err")]
        failed = not all(e <= PARITY_TOL for e in errs)
        log(f"parity vs the oracle: {par}")
    else:
        result["cpu_baseline"] = None
        result["parity"] = None
    print(json.dumps(result), flush=True)
    if failed:
        print(f"bench.py: the timed step's outputs differ from the oracle by more than {PARITY_TOL}",
              file=sys.stderr)
        sys.exit(3)


if __name__ == "__main__":
    main()

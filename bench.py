#!/usr/bin/env python3
"""Benchmark of paged MLA decode on one MI355X.

One step = the whole hot path on one batch: the split metadata, the decode
kernel and the combine kernel (mla_get_split_metadata + mla_decode_fwd).
Inputs are seeded synthetic workloads, resident in HBM before timing. The
KV cache is replicated so consecutive steps read different copies (>= 1 GiB
in rotation), so no step finds the previous step's pages in the 256 MB
last-level cache.

Prints one JSON line per workload (default: the memory-bound workload).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from workloads import (ABSORB_WORKLOADS, APPEND_WORKLOADS, MHA_WORKLOADS, MI355X_BF16_TFLOPS,  # noqa: E402
                       MI355X_HBM_GBPS, make_mha_workload, visible_lengths,
                       WORKLOADS, algorithmic_bytes, algorithmic_bytes_fp8, algorithmic_flops,
                       make_absorb_workload, make_append_workload, make_fp8_cache, make_workload_inputs,
                       pack_fp8_pages)

METRIC = "MLA paged decode: achieved HBM GB/s and TFLOP/s (% of MI355X peak)"
DEFAULT_WORKLOAD = "memory_bound"
CSRC = os.path.join(ROOT, "mla_paged_kv_02_amd", "csrc")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


# Sources of the ops beside decode; the decode path's digest leaves their
# kernels out, so that changing one op does not void another's counter figures.
OP_SOURCES = {"kv_append": ("mla_kv_append.hip", "mla_common.h"),
              "absorb": ("mla_absorb.hip", "mla_common.h"),
              "mha": ("mla_mha_decode.hip", "mla_common.h"),
              "check": ("mla_check.hip",)}


def kernel_digest(op: str = "decode") -> str:
    """Digest of the library sources an op's kernels are built from: for
    decode every source but the other ops' kernels, for another op its kernel
    file and the shared helpers."""
    own_files = {srcs[0] for srcs in OP_SOURCES.values()}
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if op != "decode" and f not in OP_SOURCES[op]:
            continue
        if op == "decode" and f in own_files:
            continue
        if f.endswith((".hip", ".h", ".cpp")):
            h.update(f.encode())
            with open(os.path.join(CSRC, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def counter_entry(workload: str):
    """The committed rocprofv3 counter figures of `workload` (HBM bytes and
    MFMA ops per decode call), or None when absent or taken on different
    kernel sources."""
    try:
        with open(COUNTERS_FILE) as f:
            doc = json.load(f)
    except (OSError, ValueError):
        return None
    entry = doc.get("workloads", {}).get(workload)
    if not entry or entry.get("kernel_digest") != kernel_digest(_op_of(workload)):
        return None
    return entry


def _op_of(workload: str) -> str:
    if workload in APPEND_WORKLOADS or workload.replace("_fp8", "") in APPEND_WORKLOADS:
        return "kv_append"
    if workload in MHA_WORKLOADS:
        return "mha"
    if workload in ABSORB_WORKLOADS:
        return "absorb"
    return "decode"


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def streaming_context(nbytes: int = 1 << 30, reps: int = 10):
    """What plain torch kernels reach on this GPU, as context next to the
    datasheet peak: a full reduction that reads `nbytes` once, and a copy of
    `nbytes` (read + write). Median over `reps` event-timed runs."""
    import torch
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    s = torch.empty((), dtype=torch.float32, device="cuda:0")

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts)) * 1e-3

    t_read = timed(lambda: torch.sum(x, dim=0, out=s))
    t_copy = timed(lambda: y.copy_(x))
    del x, y
    return {"bytes": nbytes, "torch_sum_read_gbps": round(nbytes / t_read / 1e9, 1),
            "torch_copy_gbps": round(2 * nbytes / t_copy / 1e9, 1)}


def _oracle_sample(inp, budget_s: float):
    """Whole sequences through the oracle, in order and wrapping round the
    batch, until ~budget_s of wall time: (sequence indices, seconds)."""
    import oracle
    t0 = time.perf_counter()
    done = []
    while True:
        b = len(done) % inp.batch
        oracle.mla_decode_ref(inp.q_bits, inp.kv_bits, inp.block_table, inp.seqlens, inp.scale,
                              inp.causal, seqs=[b])
        done.append(b)
        if time.perf_counter() - t0 >= budget_s:
            break
    return done, time.perf_counter() - t0


def cpu_baseline(workload: str, inp, budget_s: float):
    """The FP64 oracle, untuned, on a bounded sample of the same workload,
    with the BLAS threads the host gives it and again with one thread (a
    third of the budget). Reported in the workload's algorithmic GB/s."""
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads, threadpool_limits = 1, None
    w = WORKLOADS[workload]
    done, dt = _oracle_sample(inp, budget_s)
    nbytes = algorithmic_bytes(inp.seqlens[done], w.s_q, w.h_q)
    passes = len(done) / inp.batch
    res = {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": int(threads),
           "kind": "oracle",
           "sample": f"{len(done)} sequence decodes ({passes:.2f} passes over the {inp.batch}-sequence "
                     f"batch, {int(inp.seqlens[done].sum())} tokens) in {dt:.1f} s; numpy FP64 "
                     f"two-pass softmax per sequence, GB/s from the same algorithmic-bytes formula",
           "seconds": round(dt, 2),
           "cpu_model": cpu_model(),
           "host_cpus": len(os.sched_getaffinity(0))}
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            done1, dt1 = _oracle_sample(inp, budget_s / 3)
        res["single_thread"] = {"value": round(algorithmic_bytes(inp.seqlens[done1], w.s_q, w.h_q) / dt1 / 1e9, 4),
                                "unit": "GB/s", "cores": 1, "sequences": len(done1),
                                "seconds": round(dt1, 2)}
    # the pure-Python definition (exactly rounded sums) on the tiny decode only
    import oracle
    tiny = make_workload_inputs("tiny")
    t0 = time.perf_counter()
    oracle.mla_decode_bruteforce(oracle.bf16_bits_to_f64(tiny.q_bits), oracle.bf16_bits_to_f64(tiny.kv_bits),
                                 tiny.block_table, tiny.seqlens, tiny.scale, tiny.causal)
    res["bruteforce_tiny_seconds"] = round(time.perf_counter() - t0, 3)
    return res


def run_workload(name: str, steps: int, warmup: int, cpu_budget: float, rotate_bytes: int,
                 num_partitions: int = 0, fp8: bool = False):
    """`fp8`: the same workload over an FP8 latent cache (mla_decode_fwd_fp8),
    its latent values drawn at the same scale as the BF16 rows."""
    import torch
    import mla_paged_kv_02_amd as mla

    w = WORKLOADS[name]
    inp = make_workload_inputs(name)
    dev = torch.device("cuda:0")
    q = torch.from_numpy(inp.q_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    if fp8:
        kv0 = torch.from_numpy(pack_fp8_pages(*make_fp8_cache(inp, seed=w.seed + 100))).to(dev)
        decode = mla.decode_fwd_fp8
    else:
        kv0 = torch.from_numpy(inp.kv_bits.view(np.int16)).view(torch.bfloat16).to(dev)
        decode = mla.decode_fwd
    bt = torch.from_numpy(inp.block_table).to(dev)
    sl = torch.from_numpy(inp.seqlens).to(dev)
    kv_bytes = kv0.numel() * kv0.element_size()
    copies = max(1, min(16, math.ceil(rotate_bytes / max(kv_bytes, 1))))
    kvs = [kv0] + [kv0.clone() for _ in range(copies - 1)]
    out = torch.empty((inp.batch, w.s_q, w.h_q, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((inp.batch, w.s_q, w.h_q), dtype=torch.float32, device=dev)
    ws = torch.empty(mla.workspace_bytes(inp.batch, w.h_q, w.s_q, num_partitions),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(i, ev=None):
        if ev is not None:
            ev[2].record(stream)
        meta = mla.get_split_metadata(sl, w.h_q, w.s_q, num_partitions, fp8=fp8)
        if ev is not None:
            ev[0].record(stream)
        decode(q, kvs[i % copies], bt, sl, inp.scale, inp.causal, meta=meta, out=out,
               lse=lse, workspace=ws)
        if ev is not None:
            ev[1].record(stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # (1) whole-step throughput: K steps between two events, nothing else
    # recorded in between
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for i in range(steps):
        step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / steps
    # (2) per-kernel durations: the library records HIP events on this stream
    # around each decode and each combine kernel; torch events bracket each
    # decode_fwd call. A separate pass, since the markers add dispatch gaps.
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(steps)]
    mla.timing_enable(True)
    for i in range(steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    dec_ms_sum, comb_ms_sum, ncalls = mla.timing_collect()
    mla.timing_enable(False)
    assert ncalls == steps, f"timed {ncalls} calls, expected {steps}"
    call_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    meta_ms = np.array([e[2].elapsed_time(e[0]) for e in evs])
    call_ms_mean = float(call_ms.mean())
    dec_ms = dec_ms_sum / steps
    comb_ms = comb_ms_sum / steps
    # (3) per layer: the attention call alone, back to back over the rotated
    # caches with one plan (a decode step builds it once for every layer),
    # between two events, all launches queued behind a device-side spin so
    # that the host's launch cost stays out
    meta = mla.get_split_metadata(sl, w.h_q, w.s_q, num_partitions, fp8=fp8)
    for i in range(2):
        decode(q, kvs[i % copies], bt, sl, inp.scale, inp.causal, meta=meta, out=out, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    l0, l1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    hold_queue(0.1 * steps + 0.5)
    l0.record(stream)
    for i in range(steps):
        decode(q, kvs[i % copies], bt, sl, inp.scale, inp.causal, meta=meta, out=out, lse=lse, workspace=ws)
    l1.record(stream)
    torch.cuda.synchronize()
    layer_ms = l0.elapsed_time(l1) / steps

    nbytes = (algorithmic_bytes_fp8 if fp8 else algorithmic_bytes)(inp.seqlens, w.s_q, w.h_q)
    flops = algorithmic_flops(inp.seqlens, w.s_q, w.h_q, w.causal)
    gbps = nbytes / (ms_step * 1e-3) / 1e9
    tflops = flops / (ms_step * 1e-3) / 1e12
    # one layer = the attention call (decode + combine), without the plan,
    # which a decode step builds once for all its layers
    layer_s = layer_ms * 1e-3
    # roofline of the dominant kernel (the decode kernel): algorithmic bytes
    # or FLOPs of one call over that kernel's mean event-timed duration
    dec_gbps = nbytes / (dec_ms * 1e-3) / 1e9
    dec_tflops = flops / (dec_ms * 1e-3) / 1e12
    hbm_bound = nbytes * 1.0 / (MI355X_HBM_GBPS * 1e9) >= flops * 1.0 / (MI355X_BF16_TFLOPS * 1e12)
    cnt = counter_entry(name + "_fp8" if fp8 else name)
    traffic = cnt.get("bytes_per_call") if cnt else None
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": round(dec_gbps, 1), "peak": MI355X_HBM_GBPS,
                "unit": "GB/s", "frac": round(dec_gbps / MI355X_HBM_GBPS, 4),
                "traffic": traffic}
    else:
        roof = {"bound": "mfma", "achieved": round(dec_tflops, 2), "peak": MI355X_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(dec_tflops / MI355X_BF16_TFLOPS, 4),
                "traffic": traffic}
    line = {
        "metric": METRIC if not fp8 else "MLA paged decode over an FP8 latent cache: achieved HBM GB/s",
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if not fp8 else "fp8-e4m3 cache, bf16 arithmetic",
        "data": ("synthetic (seeded; BF16 N(0,1) query and cache, shuffled block table)" if not fp8 else
                 "synthetic (seeded; BF16 N(0,1) query; E4M3 latent values ~N(0,1) at per-token scales, "
                 "BF16 rotary part; shuffled block table)"),
        "config": {"workload": f"{name}{'_fp8' if fp8 else ''}: {w.description}, d=576, dv=512, page 64, "
                               f"{'fp8 latent cache, ' if fp8 else ''}{'causal' if w.causal else 'non-causal'}",
                   "batch": inp.batch, "s_q": w.s_q, "h_q": w.h_q,
                   "total_tokens": int(inp.seqlens.sum()), "seed": w.seed},
        "tflops": round(tflops, 2),
        "hbm_frac_of_peak": round(gbps / MI355X_HBM_GBPS, 4),
        "mfma_frac_of_peak": round(tflops / MI355X_BF16_TFLOPS, 4),
        "decode_call_us": round(call_ms_mean * 1e3, 2),
        "decode_call_us_median": round(float(np.median(call_ms)) * 1e3, 2),
        "decode_call_us_min": round(float(call_ms.min()) * 1e3, 2),
        "decode_call_us_p90": round(float(np.percentile(call_ms, 90)) * 1e3, 2),
        "metadata_us_median": round(float(np.median(meta_ms)) * 1e3, 2),
        "decode_kernel_us": round(dec_ms * 1e3, 2),
        "combine_kernel_us": round(comb_ms * 1e3, 2),
        "layer": {"what": "one attention call per layer (decode + combine kernels) with a plan built "
                          "once, back to back between two events; the per-step plan is timed apart "
                          "(metadata_us_median)",
                  "us": round(layer_ms * 1e3, 2),
                  "gbps": round(nbytes / layer_s / 1e9, 1), "tflops": round(flops / layer_s / 1e12, 2),
                  "hbm_frac": round(nbytes / layer_s / 1e9 / MI355X_HBM_GBPS, 4),
                  "mfma_frac": round(flops / layer_s / 1e12 / MI355X_BF16_TFLOPS, 4)},
        "roofline_kernel": decode_kernel_name(fp8, w.h_q * w.s_q),
        "roofline_scope": "the decode kernel alone: algorithmic bytes (or FLOPs) of one call over its "
                          "mean event-timed duration",
        "algorithmic_bytes": nbytes,
        "algorithmic_flops": flops,
        "kv_copies_rotated": copies,
        "roofline": roof,
        "kernel_digest": kernel_digest(),
    }
    if cnt:
        c = {"hbm_bytes_per_call": traffic,
             "bytes_over_algorithmic": round(traffic / nbytes, 3) if traffic else None}
        if cnt.get("mfma_mops_bf16_per_call"):
            mf = cnt["mfma_mops_bf16_per_call"] * 512
            c.update({"mfma_flops_per_call": mf, "flops_over_algorithmic": round(mf / flops, 3)})
        line["counters"] = c
    if cpu_budget > 0:
        line["cpu_baseline"] = cpu_baseline(name, inp, cpu_budget)
    return line


# the decode kernel the roofline is taken on, by (FP8 cache, >= 64 rows)
# the decode organisation forced with --decode-kernel (None: the plan's own choice)
FORCED_KERNEL = None


def decode_kernel_name(fp8: bool, rows: int) -> str:
    """The decode kernel a plan of `rows` query rows per sequence runs: over
    the BF16 cache the library picks 16-row blocks below 64 rows and 64-row
    score/value blocks from there; over the FP8 cache score/value blocks of
    16, 32 or 64 rows (--decode-kernel forces one)."""
    if fp8:
        kind = FORCED_KERNEL or "ws"
        if kind == "rows16":
            return "mla_decode_rows16_fp8_kernel"
        return f"mla_decode_ws_kernel<{1 if rows <= 16 else 2 if rows <= 32 else 4}, true>"
    kind = FORCED_KERNEL or ("rows16" if rows < 64 else "ws")
    return {"rows16": "mla_decode_rows16_kernel", "ws": "mla_decode_ws_kernel",
            "fw": "mla_decode_fw_kernel"}[kind]


def workload_summary(line: dict) -> dict:
    """The figures of one workload's bench line that go into the headline
    line's `workloads` object."""
    keys = ("ms_per_step", "value", "tflops", "hbm_frac_of_peak", "mfma_frac_of_peak", "decode_kernel_us",
            "combine_kernel_us", "metadata_us_median", "decode_call_us", "layer", "roofline",
            "roofline_kernel", "counters", "algorithmic_bytes", "algorithmic_flops")
    out = {k: line[k] for k in keys if k in line}
    out["config"] = line["config"]["workload"]
    return out


_SLEEP_CYCLES_PER_MS = None


def hold_queue(ms: float):
    """Enqueue a device-side spin of about `ms` on the current stream, so that
    the calls that follow are all queued before the GPU reaches them. The
    events around them then time device work only: these ops run for a few
    microseconds, less than one Python-side launch takes on the host."""
    import torch
    global _SLEEP_CYCLES_PER_MS
    if _SLEEP_CYCLES_PER_MS is None:   # calibrate the spin's counter rate once
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        torch.cuda._sleep(1_000_000)
        b.record()
        torch.cuda.synchronize()
        _SLEEP_CYCLES_PER_MS = 1_000_000 / max(a.elapsed_time(b), 1e-3)
    torch.cuda._sleep(int(ms * _SLEEP_CYCLES_PER_MS))


def append_bytes(inp, fp8: bool = False) -> int:
    """Algorithmic bytes of one cache append: each placed token's row read once
    (1152 B) and written once (1152 B, or 644 B into an FP8 cache), one
    block-table entry per (sequence, page) touched, and the lengths."""
    s_new = inp.s_new
    rows, pages = 0, 0
    for n in inp.seqlens:
        n = int(n)
        lo, hi = max(0, n - s_new), n
        if hi > lo:
            rows += hi - lo
            pages += (hi - 1) // 64 - lo // 64 + 1
    return (1152 + (644 if fp8 else 1152)) * rows + 4 * pages + 4 * inp.batch


def run_append(name: str, steps: int, warmup: int, fp8: bool = False, rotate_bytes: int = 1 << 30):
    """One step = one mla_kv_append call on the workload's new rows. Each call
    writes the same rows (idempotent), timed call by call with HIP events on
    the launch stream, behind a device-side spin that keeps the host's launch
    cost out of the events. The cache and the new rows are replicated so
    consecutive calls use different copies (>= rotate_bytes in rotation), so
    no call finds the previous one's rows or pages in the 256 MB MALL."""
    import torch
    import mla_paged_kv_02_amd as mla

    inp = make_append_workload(name)
    dev = torch.device("cuda:0")

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    if fp8:
        kv = torch.from_numpy(pack_fp8_pages(*make_fp8_cache(inp, seed=APPEND_WORKLOADS[name]["seed"] + 100))).to(dev)
        append = mla.kv_append_fp8
    else:
        kv = to_dev(inp.kv_bits)
        append = mla.kv_append
    new = to_dev(inp.new_bits)
    bt = torch.from_numpy(inp.block_table).to(dev)
    sl = torch.from_numpy(inp.seqlens).to(dev)
    set_bytes = kv.numel() * kv.element_size() + new.numel() * new.element_size()
    copies = max(1, min(64, math.ceil(rotate_bytes / set_bytes)))
    sets = [(new, kv)] + [(new.clone(), kv.clone()) for _ in range(copies - 1)]
    stream = torch.cuda.current_stream(dev)
    for i in range(warmup):
        append(sets[i % copies][0], sl, bt, sets[i % copies][1])
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    hold_queue(0.1 * steps)
    t0.record(stream)
    for i in range(steps):
        append(sets[i % copies][0], sl, bt, sets[i % copies][1])
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    hold_queue(0.1 * steps)
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        append(sets[i % copies][0], sl, bt, sets[i % copies][1])
        b.record(stream)
    torch.cuda.synchronize()
    call_ms = np.array([a.elapsed_time(b) for a, b in evs])
    nbytes = append_bytes(inp, fp8)
    gbps = nbytes / (ms_step * 1e-3) / 1e9
    # the kernel's duration for the roofline: the back-to-back average (an
    # event pair around every call adds a few microseconds of its own, which
    # is most of a one-decode-step append)
    kern_gbps = gbps
    cnt = counter_entry(name + "_fp8" if fp8 else name)
    traffic = cnt.get("bytes_per_call") if cnt else None
    w = APPEND_WORKLOADS[name]
    return {
        "metric": "paged latent-cache append" + (" into an FP8 cache (quantising)" if fp8 else "")
                  + ": achieved HBM GB/s",
        "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; BF16 N(0,1) new rows, shuffled block table)",
        "config": {"workload": f"{name}{'_fp8' if fp8 else ''}: batch {inp.batch}, {w['s_new']} new tokens per sequence, "
                               f"final lengths U[{w['lengths'][2]},{w['lengths'][3]}], rows of 576 bf16, page 64",
                   "batch": inp.batch, "s_new": inp.s_new, "seed": w["seed"]},
        "append_kernel_us_avg": round(ms_step * 1e3, 2),
        "copies_rotated": copies,
        "append_call_us_median": round(float(np.median(call_ms)) * 1e3, 2),
        "append_call_us_min": round(float(call_ms.min()) * 1e3, 2),
        "append_call_us_p90": round(float(np.percentile(call_ms, 90)) * 1e3, 2),
        "algorithmic_bytes": nbytes,
        "roofline": {"bound": "hbm", "achieved": round(kern_gbps, 1), "peak": MI355X_HBM_GBPS,
                     "unit": "GB/s", "frac": round(kern_gbps / MI355X_HBM_GBPS, 4), "traffic": traffic},
        "kernel_digest": kernel_digest("kv_append"),
    }


def absorb_work(w: dict):
    """Algorithmic bytes and FLOPs of absorb_q and absorb_o: every operand
    read once and every result written once; 2 FLOPs per multiply-add."""
    t, h, dn, dv = w["tokens"], w["heads"], w["d_nope"], w["d_v"]
    q_bytes = 2 * (t * h * dn + t * h * 64 + h * 512 * dn + t * h * 576)
    o_bytes = 2 * (t * h * 512 + h * 512 * dv + t * h * dv)
    return q_bytes, 2 * t * h * 512 * dn, o_bytes, 2 * t * h * 512 * dv


def run_absorb(name: str, steps: int, warmup: int, rotate_bytes: int):
    """One step = mla_absorb_q then mla_absorb_o for one decode step's tokens.
    Inputs and weights are replicated so consecutive steps read different
    copies (>= rotate_bytes in rotation, so weights do not stay in the MALL);
    each kernel is also timed call by call with HIP events on its stream.
    Both timed passes start behind a device-side spin that keeps the host's
    launch cost out of the events."""
    import torch
    import mla_paged_kv_02_amd as mla

    w = ABSORB_WORKLOADS[name]
    inp = make_absorb_workload(name)
    dev = torch.device("cuda:0")

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    base = [to_dev(inp.q_nope), to_dev(inp.q_rope), to_dev(inp.w_uk), to_dev(inp.o_lat),
            to_dev(np.ascontiguousarray(inp.w_uv.transpose(0, 2, 1)))]
    set_bytes = sum(t.numel() * 2 for t in base)
    copies = max(1, min(32, math.ceil(rotate_bytes / set_bytes)))
    sets = [base] + [[t.clone() for t in base] for _ in range(copies - 1)]
    q_abs = torch.empty((w["tokens"], w["heads"], 576), dtype=torch.bfloat16, device=dev)
    out = torch.empty((w["tokens"], w["heads"], w["d_v"]), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(i, ev=None):
        qn, qr, wuk, ol, wuv = sets[i % copies]
        if ev:
            ev[0].record(stream)
        mla.absorb_q(qn, qr, wuk, out=q_abs)
        if ev:
            ev[1].record(stream)
        mla.absorb_o(ol, wuv, out=out)
        if ev:
            ev[2].record(stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    hold_queue(0.2 * steps)
    t0.record(stream)
    for i in range(steps):
        step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / steps
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(steps)]
    hold_queue(0.2 * steps)
    for i in range(steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    q_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    o_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])

    def batch_avg_ms(call):
        # one kernel back to back over the rotated copies, one event pair
        # around the batch: its average duration for the roofline (an event
        # pair around every call adds a few microseconds of its own)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        hold_queue(0.1 * steps)
        a.record(stream)
        for i in range(steps):
            call(sets[i % copies])
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    q_avg = batch_avg_ms(lambda st: mla.absorb_q(st[0], st[1], st[2], out=q_abs))
    o_avg = batch_avg_ms(lambda st: mla.absorb_o(st[3], st[4], out=out))
    qb, qf, ob, of = absorb_work(w)
    q_gbps = qb / (q_avg * 1e-3) / 1e9
    o_gbps = ob / (o_avg * 1e-3) / 1e9
    cnt = counter_entry(name)

    def roof(gbps, key):
        return {"bound": "hbm", "achieved": round(gbps, 1), "peak": MI355X_HBM_GBPS, "unit": "GB/s",
                "frac": round(gbps / MI355X_HBM_GBPS, 4),
                "traffic": (cnt or {}).get(key)}

    return {
        "metric": "MLA absorption products (absorb_q + absorb_o): achieved HBM GB/s",
        "value": round((qb + ob) / (ms_step * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; BF16 N(0,1) activations, N(0,1/K) weights)",
        "config": {"workload": f"{name}: {w['tokens']} tokens, {w['heads']} heads, d_nope {w['d_nope']}, "
                               f"d_v {w['d_v']}, latent 512", **{k: w[k] for k in ("tokens", "heads", "d_nope", "d_v")}},
        "tflops": round((qf + of) / (ms_step * 1e-3) / 1e12, 2),
        "absorb_q_kernel_us_avg": round(q_avg * 1e3, 2),
        "absorb_o_kernel_us_avg": round(o_avg * 1e3, 2),
        "absorb_q_us_median": round(float(np.median(q_ms)) * 1e3, 2),
        "absorb_q_us_p90": round(float(np.percentile(q_ms, 90)) * 1e3, 2),
        "absorb_o_us_median": round(float(np.median(o_ms)) * 1e3, 2),
        "absorb_o_us_p90": round(float(np.percentile(o_ms, 90)) * 1e3, 2),
        "algorithmic_bytes": {"absorb_q": qb, "absorb_o": ob},
        "algorithmic_flops": {"absorb_q": qf, "absorb_o": of},
        "copies_rotated": copies,
        "roofline": roof(q_gbps, "bytes_per_call"),
        "roofline_absorb_o": roof(o_gbps, "absorb_o_bytes_per_call"),
        "kernel_digest": kernel_digest("absorb"),
    }


def run_mha(name: str, steps: int, warmup: int):
    """One step = one paged grouped-query MHA decode call over the contrast
    workload (the memory-bound sequences with 8 KV heads of 128 values:
    a 1.09 GB K+V cache, so no step finds the previous one's data in the
    MALL). Timed back to back between two events behind a device-side spin."""
    import torch
    import mla_paged_kv_02_amd as mla

    w = MHA_WORKLOADS[name]
    inp = make_mha_workload(name)
    dev = torch.device("cuda:0")

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = to_dev(inp.q_bits), to_dev(inp.k_bits), to_dev(inp.v_bits)
    bt = torch.from_numpy(inp.block_table).to(dev)
    sl = torch.from_numpy(inp.seqlens).to(dev)
    out = torch.empty((inp.batch, w["s_q"], w["h_q"], w["d"]), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((inp.batch, w["s_q"], w["h_q"]), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    for _ in range(warmup):
        mla.mha_decode_fwd(q, k, v, bt, sl, inp.scale, inp.causal, out=out, lse=lse)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    hold_queue(0.1 * steps)
    t0.record(stream)
    for _ in range(steps):
        mla.mha_decode_fwd(q, k, v, bt, sl, inp.scale, inp.causal, out=out, lse=lse)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    n = inp.seqlens.astype(np.int64)
    rows = inp.batch * w["s_q"] * w["h_q"]
    kv_bytes = 2 * w["h_kv"] * w["d"] * 2 * int(n.sum())
    nbytes = kv_bytes + 2 * 2 * rows * w["d"] + 4 * rows + 4 * int(((n + 63) // 64).sum()) + 4 * inp.batch
    flops = 2 * 2 * w["d"] * w["h_q"] * int(visible_lengths(n, w["s_q"], False).sum())
    gbps = nbytes / (ms * 1e-3) / 1e9
    mla_bytes = algorithmic_bytes(inp.seqlens, w["s_q"], w["h_q"])
    cnt = counter_entry(name)
    return {
        "metric": "paged GQA MHA decode (contrast to MLA): achieved HBM GB/s",
        "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded; BF16 N(0,1) query, keys and values, shuffled block table)",
        "config": {"workload": f"{name}: batch {inp.batch}, seqlens U[{w['lengths'][0]},{w['lengths'][1]}], "
                               f"s_q={w['s_q']}, h_q={w['h_q']}, h_kv={w['h_kv']}, d={w['d']}, page 64",
                   "batch": inp.batch, "total_tokens": int(n.sum()), "seed": w["seed"]},
        "mha_kernel_us_avg": round(ms * 1e3, 2),
        "algorithmic_bytes": nbytes,
        "algorithmic_flops": flops,
        "kv_bytes_per_token": 2 * w["h_kv"] * w["d"] * 2,
        "mla_kv_bytes_per_token": 1152,
        "mla_algorithmic_bytes_same_sequences": mla_bytes,
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": MI355X_HBM_GBPS, "unit": "GB/s",
                     "frac": round(gbps / MI355X_HBM_GBPS, 4),
                     "traffic": cnt.get("bytes_per_call") if cnt else None},
        "kernel_digest": kernel_digest("mha"),
    }


def copy_calibration(nbytes: int = 1 << 30, reps: int = 5):
    """A plain device-to-device copy of known size, to calibrate the HBM
    byte counters (FETCH_SIZE / WRITE_SIZE) read by rocprofv3."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps}), flush=True)


def _counter_rows(run_dir: str):
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {run_dir}")
    rows = []
    for f in files:
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def _per_dispatch_mean(run_dir: str, kernel_substr: str, counter: str):
    vals = [float(r["Counter_Value"]) for r in _counter_rows(run_dir)
            if kernel_substr in r["Kernel_Name"] and r["Counter_Name"] == counter]
    if not vals:
        raise SystemExit(f"no {counter} rows for kernel '{kernel_substr}' in {run_dir}")
    return float(np.mean(vals)), len(vals)


def ingest_counters(workload: str, kernel: str, fetch_dir: str, write_dir: str,
                    cal_fetch_dir: str, cal_write_dir: str, command: str, key: str = ""):
    """Turn four rocprofv3 --pmc runs (FETCH_SIZE and WRITE_SIZE of the bench on
    `workload`, and of --copy-calibration) into HBM bytes per dispatch of
    `kernel`, scaled so that the 1 GiB copy reads and writes 1 GiB, and store
    them in profiles/hbm_traffic.json under the current kernel digest. With
    `key`, the figures of a second kernel of the same workload are added to
    its entry as `<key>` and `<key>_bytes_per_call`."""
    cal_bytes = 1 << 30
    cf, _ = _per_dispatch_mean(cal_fetch_dir, "copyBuffer", "FETCH_SIZE")
    cw, _ = _per_dispatch_mean(cal_write_dir, "copyBuffer", "WRITE_SIZE")
    fetch_scale = cal_bytes / (cf * 1024.0)
    write_scale = cal_bytes / (cw * 1024.0)
    f, nf = _per_dispatch_mean(fetch_dir, kernel, "FETCH_SIZE")
    wr, nw = _per_dispatch_mean(write_dir, kernel, "WRITE_SIZE")
    entry = {
        "kernel": kernel,
        "kernel_digest": kernel_digest(_op_of(workload)),
        "fetch_kib_per_dispatch": round(f, 1), "dispatches_fetch": nf,
        "write_kib_per_dispatch": round(wr, 1), "dispatches_write": nw,
        "fetch_scale": round(fetch_scale, 4), "write_scale": round(write_scale, 4),
        "copy_fetch_kib_per_gib": round(cf, 1), "copy_write_kib_per_gib": round(cw, 1),
        "bytes_per_call": int(round(f * 1024.0 * fetch_scale + wr * 1024.0 * write_scale)),
        "command": command,
    }
    try:
        with open(COUNTERS_FILE) as fh:
            doc = json.load(fh)
    except (OSError, ValueError):
        doc = {}
    if key:
        main = doc.get("workloads", {}).get(workload)
        if not main or main.get("kernel_digest") != entry["kernel_digest"]:
            raise SystemExit(f"no entry for {workload} on the current sources; ingest its first kernel first")
        main[key] = entry
        main[key + "_bytes_per_call"] = entry["bytes_per_call"]
        entry = main
    doc.setdefault("workloads", {})[workload] = entry
    with open(COUNTERS_FILE, "w") as fh:
        json.dump(doc, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(json.dumps({workload: entry}))


def ingest_mfma(workload: str, kernel: str, mfma_dir: str, command: str):
    """Add the MFMA BF16 op count of one rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16
    run (ops in units of 512 FLOPs, per dispatch of `kernel`) to the workload's
    entry in profiles/hbm_traffic.json, taken on the same kernel sources."""
    v, n = _per_dispatch_mean(mfma_dir, kernel, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    with open(COUNTERS_FILE) as fh:
        doc = json.load(fh)
    entry = doc.get("workloads", {}).get(workload)
    if not entry or entry.get("kernel_digest") != kernel_digest(_op_of(workload)):
        raise SystemExit(f"no byte-counter entry for {workload} on the current sources; ingest those first")
    entry.update({"mfma_mops_bf16_per_call": int(round(v)), "dispatches_mfma": n, "mfma_command": command})
    with open(COUNTERS_FILE, "w") as fh:
        json.dump(doc, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(json.dumps({workload: entry}))


def summarize_trace(trace_dir: str, command: str, bench_log: str = "", op: str = "decode") -> str:
    """Text summary of a rocprofv3 --kernel-trace --stats run (kernel stats CSV),
    with the bench JSON line of the same run when its log is given."""
    import csv
    import glob
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *kernel_stats.csv under {trace_dir}")
    with open(files[0]) as fh:
        rows = list(csv.DictReader(fh))
    out = [f"command: {command}", f"kernel sources digest: {kernel_digest(op)}", "",
           f"{'kernel':58s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'share':>7s}"]
    for r in rows:
        name = r["Name"].replace("(anonymous namespace)::", "")[:58]
        out.append(f"{name:58s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.2f} "
                   f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f} "
                   f"{float(r['Percentage']):6.1f}%")
    if bench_log:
        for line in open(bench_log):
            if line.startswith("{"):
                d = json.loads(line)
                out += ["", "bench.py line of the same run (under the profiler):",
                        "  " + json.dumps({k: d[k] for k in ("decode_kernel_us", "combine_kernel_us",
                                                              "decode_call_us", "ms_per_step",
                                                              "roofline") if k in d})]
    return "\n".join(out) + "\n"


def main():
    global FORCED_KERNEL
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    help="one of %s, or 'all'; with --op kv_append one of %s or 'all'"
                         % (", ".join(WORKLOADS), ", ".join(APPEND_WORKLOADS)))
    ap.add_argument("--op", default="decode",
                    choices=("decode", "decode_fp8", "kv_append", "kv_append_fp8", "absorb", "mha"),
                    help="decode (the hot path; default), decode over an FP8 latent cache, the paged "
                         "cache append, the absorption products, or the MHA comparison decode")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle CPU time for the cpu_baseline sample (0 = skip)")
    ap.add_argument("--rotate-gib", type=float, default=1.0)
    ap.add_argument("--num-partitions", type=int, default=0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a 1 GiB device copy (counter calibration)")
    ap.add_argument("--ingest-counters", nargs=4, metavar=("FETCH", "WRITE", "CAL_FETCH", "CAL_WRITE"),
                    help="rocprofv3 --pmc output dirs: write profiles/hbm_traffic.json for --workload "
                         "(no GPU needed)")
    ap.add_argument("--ingest-mfma", metavar="MFMA_DIR",
                    help="rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16 output dir: add the MFMA op count "
                         "to profiles/hbm_traffic.json for --workload (no GPU needed)")
    ap.add_argument("--decode-kernel", default=None, choices=("rows16", "ws", "fw"),
                    help="force one decode organisation for BF16 plans (mla_set_plan_override)")
    ap.add_argument("--merge", default=None, choices=("kernel", "fused"),
                    help="force where split sequences are merged (mla_set_plan_override)")
    ap.add_argument("--only", action="store_true",
                    help="decode: time only --workload (by default the memory-bound line also carries "
                         "every other workload under 'workloads')")
    ap.add_argument("--no-stream-context", action="store_true",
                    help="skip the torch streaming-read / copy bandwidth context")
    ap.add_argument("--kernel", default="mla_decode_rows16_kernel",
                    help="kernel name substring for --ingest-counters")
    ap.add_argument("--command", default="", help="profiling command recorded by --ingest-counters")
    ap.add_argument("--counter-key", default="",
                    help="with --ingest-counters: add a second kernel's bytes to the workload's entry "
                         "under this key")
    ap.add_argument("--summarize-trace", nargs="+", metavar=("TRACE_DIR", "BENCH_LOG"),
                    help="print a text summary of a rocprofv3 --kernel-trace --stats run (no GPU)")
    args = ap.parse_args()
    if args.summarize_trace:
        sys.stdout.write(summarize_trace(args.summarize_trace[0], args.command,
                                         args.summarize_trace[1] if len(args.summarize_trace) > 1 else "",
                                         _op_of(args.workload)))
        return
    if args.ingest_counters:
        ingest_counters(args.workload, args.kernel, *args.ingest_counters, command=args.command,
                        key=args.counter_key)
        return
    if args.ingest_mfma:
        ingest_mfma(args.workload, args.kernel, args.ingest_mfma, command=args.command)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: the decode library runs on one GPU (it has no multi-GPU path); use --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.op == "mha":
        names = list(MHA_WORKLOADS) if args.workload in ("all", DEFAULT_WORKLOAD) else [args.workload]
        for name in names:
            print(json.dumps(run_mha(name, args.steps, args.warmup)), flush=True)
        return
    if args.op == "absorb":
        names = list(ABSORB_WORKLOADS) if args.workload in ("all", DEFAULT_WORKLOAD) else [args.workload]
        for name in names:
            print(json.dumps(run_absorb(name, args.steps, args.warmup, int(args.rotate_gib * (1 << 30)))),
                  flush=True)
        return
    if args.op in ("kv_append", "kv_append_fp8"):
        names = list(APPEND_WORKLOADS) if args.workload in ("all", DEFAULT_WORKLOAD) else [args.workload]
        for name in names:
            print(json.dumps(run_append(name, args.steps, args.warmup, fp8=args.op == "kv_append_fp8",
                                        rotate_bytes=int(args.rotate_gib * (1 << 30)))), flush=True)
        return
    fp8 = args.op == "decode_fp8"
    if args.decode_kernel or args.merge:
        import mla_paged_kv_02_amd as mla
        mla.set_plan_override(kernel=args.decode_kernel, merge=args.merge)
        FORCED_KERNEL = args.decode_kernel
    names = list(WORKLOADS) if args.workload == "all" else [args.workload]
    ctx = None if args.no_stream_context else streaming_context()
    rotate = int(args.rotate_gib * (1 << 30))
    for name in names:
        line = run_workload(name, args.steps, args.warmup,
                            args.cpu_budget if (name == DEFAULT_WORKLOAD or args.workload != "all") and not fp8
                            else 0,
                            rotate, args.num_partitions, fp8=fp8)
        if ctx:
            line["achievable_context"] = ctx
        if args.workload == DEFAULT_WORKLOAD and not args.only:
            # the other workloads, timed the same way, in the same line: the
            # 128-head ones carry the MFMA half of the metric
            import torch
            others = {}
            for other in WORKLOADS:
                if other == name:
                    continue
                torch.cuda.empty_cache()
                others[other] = workload_summary(run_workload(other, args.steps, args.warmup, 0, rotate,
                                                              args.num_partitions, fp8=fp8))
            line["workloads"] = {name: workload_summary(line), **others}
        print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

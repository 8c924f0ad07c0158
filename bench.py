#!/usr/bin/env python3
"""Benchmark of the paged K8/V4 decode step on one MI355X.

A step is one pass of the whole hot path over one batch: one ``kvq_decode_step`` call, which
quantizes the step's new tokens into their slots and runs split-KV attention over every
sequence, query head and query row (one launch), then merges the splits (a second, small
launch).  ``--unfused`` times ``kvq_append`` followed by ``kvq_decode_attn`` instead.  The default workload is the 184,320-token KV
pool shared by two 92,160-token sequences (4 KV heads, 24 query heads, head_dim 256, page 64,
interleaved random page tables), the shape of the forum post "3090 单卡跑 Qwen3.8-27B：NInfer
上机实测（180K 上下文 / C2 并发 / 4bit KV）" (一、部署, launch-flag table: 184,320-token pool,
concurrency 2, rk8v4 KV).

Cold cache: the pool is replicated into ``--copies`` copies (default 8, 2.4 GB at the default
workload) and step k uses copy k mod copies, so no pool byte is still in the 256 MB Infinity
Cache or the L2s when it is read again.  Inputs are resident in HBM before the timed region.

Prints one JSON line (rank 0, N = 1).  Progress goes to stderr.
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
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth, 8 TB/s


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def library_hash() -> str:
    """Hash of the built library the bench loads (the build is deterministic, so an edit that
    changes no code keeps it): counters taken on other code are not reported as traffic."""
    from long_context_decode_flash_amd import kvq
    h = hashlib.sha256()
    with open(kvq.LIB_PATH, "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def token_bytes(head_dim: int, vbits: int = 4) -> int:
    """Stored bytes per token per KV head: K codes + K scale + V codes + V scales."""
    return head_dim + 2 + head_dim * vbits // 8 + 2 * (head_dim // 32)


def attended_range(L: int, n_rows: int, window: int):
    """First and one-past-last token some row of a sequence of L tokens sees."""
    return (max(0, L - n_rows - window + 1) if window > 0 else 0), L


def decode_algorithmic_bytes(wl, seq_lens, vbits: int = 4, window: int = 0) -> int:
    """Bytes the method itself must move per decode call: every cached K/V byte of every
    attended token once (with a window, the tokens some row's window covers), the queries, the
    page-table entries used, the outputs (+ lse)."""
    D = wl.head_dim
    spans = [attended_range(int(L), wl.n_rows, window) for L in seq_lens]
    kv = sum(t1 - t0 for t0, t1 in spans) * wl.num_kv_heads * token_bytes(D, vbits)
    q = wl.n_seq * wl.n_rows * wl.n_q_heads * D * 2
    pt = sum((t1 - 1) // wl.page_size - t0 // wl.page_size + 1 for t0, t1 in spans) * 4
    out = wl.n_seq * wl.n_rows * wl.n_q_heads * (D + 1) * 4
    return kv + q + pt + out


def prefill_attn_flops(seq_lens, chunk: int, n_q_heads: int, head_dim: int) -> int:
    """FLOPs of one chunked-prefill call: position i of a chunk at the end of a context of L
    tokens attends L - chunk + i + 1 tokens (none below zero), each costing 2D for Q K^T and 2D
    for P V per query head."""
    seen = 0
    for L in seq_lens:
        lo = int(L) - chunk + 1
        seen += sum(max(lo + i, 0) for i in range(chunk))
    return seen * n_q_heads * 4 * head_dim


def append_algorithmic_bytes(wl, vbits: int = 4) -> int:
    n = wl.n_seq * wl.n_new
    return n * wl.num_kv_heads * (2 * wl.head_dim * 4 + token_bytes(wl.head_dim, vbits)) + n * 4


def cpu_baseline(wl, inp, min_seconds=10.0, window=0, kv_format=0):
    """The oracle, as it is, on full steps of the workload on the host cores, repeated until
    min_seconds have passed (the step's append writes the same slots each time).  Returns the
    mean seconds per step, the steps run and the threads used."""
    import oracle
    pool = oracle.new_pool(wl.pool_pages, wl.page_size, wl.num_kv_heads, wl.head_dim,
                           4 if kv_format == 0 else 8)
    t0 = time.perf_counter()
    oracle.append(pool, wl.pool_pages, wl.page_size, wl.num_kv_heads, wl.head_dim,
                  *inp.prefill(), kv_format=kv_format)
    log(f"[cpu] oracle prefill {time.perf_counter() - t0:.1f}s (not timed)")
    steps = 0
    t0 = time.perf_counter()
    while True:
        oracle.append(pool, wl.pool_pages, wl.page_size, wl.num_kv_heads, wl.head_dim,
                      *inp.step_tokens(), kv_format=kv_format)
        oracle.decode_attn(pool, wl.pool_pages, wl.page_size, wl.num_kv_heads, wl.head_dim,
                           inp.q_bits, inp.page_table, inp.seq_lens, wl.n_rows, wl.n_q_heads,
                           window=window, kv_format=kv_format)
        steps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            return dt / steps, steps, oracle.num_threads()


def cpu_baseline_one_thread(wl, inp, rows=6, window=0, kv_format=0):
    """The oracle on one host thread, over a bounded sample: `rows` of the step's output rows
    (the first query row of the first heads of sequence 0), scaled to a whole step by the row
    count; the step's append (a few tokens) is negligible beside the attention.  Returns
    (seconds per step, sample description)."""
    import oracle
    pool = oracle.new_pool(wl.pool_pages, wl.page_size, wl.num_kv_heads, wl.head_dim,
                           4 if kv_format == 0 else 8)
    oracle.append(pool, wl.pool_pages, wl.page_size, wl.num_kv_heads, wl.head_dim,
                  *inp.all_tokens(), kv_format=kv_format)
    total = wl.n_seq * wl.n_rows * wl.n_q_heads
    rows = min(rows, total)
    sel = [(0, 0, hq) for hq in range(rows)]
    before = oracle.num_threads()
    oracle.set_num_threads(1)
    try:
        t0 = time.perf_counter()
        oracle.decode_attn(pool, wl.pool_pages, wl.page_size, wl.num_kv_heads, wl.head_dim,
                           inp.q_bits, inp.page_table, inp.seq_lens, wl.n_rows, wl.n_q_heads,
                           select=sel, window=window, kv_format=kv_format)
        dt = time.perf_counter() - t0
    finally:
        oracle.set_num_threads(before)
    return dt * total / rows, (f"{rows} of the step's {total} output rows on 1 thread "
                               f"({dt:.1f} s), scaled by {total}/{rows}")


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def read_telemetry() -> dict:
    """GPU clocks, power and power cap as the driver reports them.  The firmware's metrics table
    refreshes about every 100 ms, so a reading describes the state around the timed region,
    not inside it."""
    t = {}
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        h = amdsmi.amdsmi_get_processor_handles()[0]
        m = amdsmi.amdsmi_get_gpu_metrics_info(h)
        for k in ("current_gfxclk", "current_gfxclks", "current_uclk", "current_socclk",
                  "current_socket_power", "temperature_hotspot", "temperature_mem",
                  "average_gfx_activity", "average_umc_activity"):
            if k in m:
                t[k] = m[k]
        t["power_cap_w"] = amdsmi.amdsmi_get_power_cap_info(h)["power_cap"] / 1e6
    except Exception as e:  # telemetry is informative only
        t["amdsmi_error"] = str(e)[:120]
    import glob
    for name in ("pp_dpm_sclk", "pp_dpm_mclk"):
        paths = sorted(glob.glob(f"/sys/class/drm/card*/device/{name}"))
        try:
            with open(paths[0]) as f:
                cur = [l.strip() for l in f if "*" in l]
            t[name] = cur[0] if cur else None
        except (OSError, IndexError):
            t[name] = None
    return t


class ShaderClock:
    """Reads the shader clock on the GPU itself (kvq_probe_clock: shader-clock cycles against the
    constant-rate counter over a 20 us spin in 256 one-wave workgroups).  The driver's metrics
    table refreshes about every 100 ms and cannot resolve a millisecond-long timed region; this
    probe is enqueued on the stream right beside it.  enqueue() queues a reading into the next
    slot; read() returns every queued reading (mean MHz and the slowest and fastest XCD)."""

    WG = 256

    def __init__(self, kvq, torch, dev, stream, slots=64):
        self.torch = torch
        self.buf = torch.zeros((slots, 3 * self.WG), dtype=torch.int64, device=dev)
        self.calls = [kvq.prepare_clock_probe(self.buf[i], 2000, stream=stream) for i in range(slots)]
        self.khz = kvq.clock_counter_khz()
        self.n = 0

    def enqueue(self):
        self.calls[self.n]()
        self.n += 1
        return self.n - 1

    def read(self, i):
        v = self.buf[i].view(self.WG, 3).cpu().numpy()
        mhz = v[:, 0] / v[:, 1] * self.khz / 1000.0
        per = [float(mhz[v[:, 2] == x].mean()) for x in sorted(set(v[:, 2].tolist()))]
        return {"mhz": round(float(mhz.mean())), "xcd_min_mhz": round(min(per)),
                "xcd_max_mhz": round(max(per))}


def time_appends(kvq, torch, wl, inp, caches, apps, n_pre, D, vbits, dev_t, chunk_arg):
    """The prefill append (`reps` more passes of every sequence's kvq_append over its cached
    tokens, rewriting the same bytes) and one prefill chunk of one sequence (the engine's
    --prefill-chunk 1024 in the forum post, 一、部署: the last `chunk` cached tokens of
    sequence 0, rewritten in place), each event-timed over back-to-back calls."""
    from long_context_decode_flash_amd import workloads as W
    reps = 5
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for app in apps:
        app()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        for app in apps:
            app()
    e1.record()
    torch.cuda.synchronize()
    prefill_us = e0.elapsed_time(e1) * 1e3 / reps
    prefill_bytes = n_pre * wl.num_kv_heads * (2 * D * 4 + token_bytes(D, vbits)) + n_pre * 4
    log(f"[bench] prefill append of {n_pre} tokens: {prefill_us:.1f} us, "
        f"{prefill_bytes / prefill_us / 1e3:.0f} GB/s")
    chunk_n = min(chunk_arg or 1024, wl.seq_len - wl.n_new)
    c0 = wl.seq_len - wl.n_new - chunk_n
    ck = dev_t(inp.k[0, c0:c0 + chunk_n])
    cv = dev_t(inp.v[0, c0:c0 + chunk_n])
    cs = dev_t(W.slots_for(inp.page_table, wl.page_size, 0, c0, c0 + chunk_n))
    capp = kvq.prepare_append(caches[0], ck, cv, cs)
    capp()
    torch.cuda.synchronize()
    creps = 50
    e0.record()
    for _ in range(creps):
        capp()
    e1.record()
    torch.cuda.synchronize()
    chunk_us = e0.elapsed_time(e1) * 1e3 / creps
    chunk_bytes = chunk_n * wl.num_kv_heads * (2 * D * 4 + token_bytes(D, vbits)) + chunk_n * 4
    log(f"[bench] append of one {chunk_n}-token chunk: {chunk_us:.1f} us, "
        f"{chunk_bytes / chunk_us / 1e3:.0f} GB/s")
    return {
        "tokens": n_pre,
        "us": round(prefill_us, 1),
        "algorithmic_bytes": prefill_bytes,
        "GB_s": round(prefill_bytes / prefill_us / 1e3, 1),
        "frac_of_hbm_peak": round(prefill_bytes / prefill_us / 1e3 / HBM_PEAK_GBS, 4),
        "kernel": "kvq_append: append_kernel, one call per sequence over its cached tokens",
        "chunk": {"tokens": chunk_n, "us": round(chunk_us, 2), "algorithmic_bytes": chunk_bytes,
                  "GB_s": round(chunk_bytes / chunk_us / 1e3, 1),
                  "note": "one kvq_append of one sequence's chunk, back-to-back calls, event-timed"},
    }


def sustained_run(torch, stream, step, clk, n, group=50):
    """n more back-to-back steps (after the timed region, which they do not touch), timed in
    groups of `group` with a shader-clock reading after each group: how the step time follows
    the clock as the GPU's power management settles under a continuous decode load."""
    groups = []
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * (n // group))]
    idx = []
    for g in range(n // group):
        ev[2 * g].record(stream)
        for i in range(group):
            step(g * group + i)
        ev[2 * g + 1].record(stream)
        idx.append(clk.enqueue() if clk.n < len(clk.calls) else None)
    torch.cuda.synchronize()
    t0 = ev[0]
    for g in range(n // group):
        r = {"t_ms": round(t0.elapsed_time(ev[2 * g]), 2),
             "us_per_step": round(ev[2 * g].elapsed_time(ev[2 * g + 1]) * 1e3 / group, 2)}
        if idx[g] is not None:
            r.update(clk.read(idx[g]))
        groups.append(r)
    last = groups[len(groups) // 2:]
    med = sorted(x["us_per_step"] for x in last)[len(last) // 2]
    log(f"[bench] sustained: {n} more steps, first group {groups[0]['us_per_step']} us/step at "
        f"{groups[0].get('mhz')} MHz, median of the second half {med} us/step")
    return {"steps": n, "group": group, "groups": groups,
            "second_half_median_us_per_step": med,
            "note": "not the timed value: back-to-back steps after every timed measurement, "
                    "with the shader clock read after each group"}


def attainable_probe(kvq, torch, dev, stream, gib=2, reps=5):
    """The plain streaming read (kvq_probe_stream_read) over a `gib` GiB buffer in each load form
    and a few grid sizes, event-timed over `reps` calls each; returns the best and every
    result.  The sweep streams for a few tens of milliseconds; it runs after the timed decode
    steps, whose shader clock it would otherwise lower (the power management's answer to a
    sustained streaming load lasts some milliseconds after it)."""

    n = gib << 30
    buf = torch.empty(n, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    rows = []
    for mode, form in ((0, "16-byte register loads, nt"), (1, "16-byte register loads"),
                       (2, "direct-to-LDS 16-byte loads, nt")):
        for wgs in (256, 512, 1024, 2048):
            call = kvq.prepare_stream_probe(buf, mode, wgs, sink, stream=stream)
            call()
            e0.record(stream)
            for _ in range(reps):
                call()
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / reps
            rows.append({"mode": mode, "form": form, "workgroups": wgs, "us": round(us, 1),
                         "GB_s": round(n / us / 1e3, 1)})
    del buf
    best = max(rows, key=lambda r: r["GB_s"])
    log(f"[bench] attainable read: {best['GB_s']:.0f} GB/s ({best['form']}, "
        f"{best['workgroups']} workgroups, {gib} GiB)")
    return best, rows, n


def _counter_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def ingest_pmc(fetch_csv, write_csv, workload, probe_mib, commands):
    """Per-launch HBM traffic of the decode kernel from two rocprofv3 --pmc runs (FETCH_SIZE,
    WRITE_SIZE, KiB per dispatch), each scaled by what the same counter reads for a plain device
    copy of probe_mib MiB (the largest copyBuffer dispatches of the run)."""
    probe_kib = probe_mib * 1024.0
    out = {"workload": workload, "library_hash": library_hash(), "copy_probe_mib": probe_mib,
           "commands": commands}
    for key, path in (("fetch", fetch_csv), ("write", write_csv)):
        rows = _counter_rows(path)
        dec = [float(r["Counter_Value"]) for r in rows if "decode_kernel" in r["Kernel_Name"]]
        cps = sorted(float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"])
        probe = cps[-1]  # the probe copies are the largest copies of the run
        out[f"{key}_kib_per_dispatch"] = round(sum(dec) / len(dec), 1)
        out[f"{key}_copy_probe_kib"] = probe
        out[f"{key}_scale"] = round(probe_kib / probe, 4)
        out[f"{key}_dispatches"] = len(dec)
    out["hbm_bytes_per_launch"] = int(1024 * (out["fetch_kib_per_dispatch"] * out["fetch_scale"] +
                                              out["write_kib_per_dispatch"] * out["write_scale"]))
    return out


def ingest_trace(stats_csv, command, bench_log=None):
    """Markdown summary of a rocprofv3 --kernel-trace --stats run of bench.py, with the step time
    bench.py itself printed in that run (bench_log) beside the kernels' summed averages."""
    rows = _counter_rows(stats_csv)
    lines = ["# Kernel trace summary", "", "Command:", "", "```", command, "```", "",
             "| kernel | calls | average us | min us | max us | % of GPU time |",
             "|---|---:|---:|---:|---:|---:|"]
    for r in rows:
        name = r["Name"]
        short = name.replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0]
        lines.append(f"| {short} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.2f} |")
    js = []
    if bench_log:
        with open(bench_log) as f:
            js = [json.loads(x) for x in f if x.startswith("{")]
    pre = [r for r in rows if "prefill_kernel" in r["Name"]]
    if pre:
        # the merge launches of this run belong to both the decode steps and the prefill calls
        pre_us = sum(float(r["TotalDurationNs"]) for r in pre) / sum(int(r["Calls"]) for r in pre) / 1e3
        lines += ["", f"prefill_kernel average: {pre_us:.1f} us per call."]
        if js and "prefill_attn" in js[-1]:
            lines.append(f"bench.py's prefill_attn in the same profiled run: {js[-1]['prefill_attn']['us']:.1f} "
                         "us per call (prefill_kernel and its merge launch, event-timed).")
        return "\n".join(lines) + "\n"
    step_us = sum(float(r["AverageNs"]) / 1e3 for r in rows
                  if "decode_kernel" in r["Name"] or "merge_kernel" in r["Name"])
    lines += ["", f"Sum of the step's kernel averages over all calls, warm-up included (decode_kernel + "
              f"merge_kernel): {step_us:.2f} us."]
    trace_csv = os.path.join(os.path.dirname(stats_csv), os.path.basename(stats_csv).replace(
        "kernel_stats", "kernel_trace"))
    if js and os.path.exists(trace_csv):
        k = int(js[-1]["steps"])
        tr = _counter_rows(trace_csv)
        avg = {}
        lines += ["", f"Over the last {k} calls of each kernel (the timed steps):", "",
                  "| kernel | mean us | median us | p90 us | min us | max us |",
                  "|---|---:|---:|---:|---:|---:|"]
        for name in ("decode_kernel", "merge_kernel"):
            d = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in tr
                       if name in r["Kernel_Name"])[-k:]
            if not d:
                avg[name] = 0.0
                continue
            us = sorted((e - s) / 1e3 for s, e in d)
            avg[name] = sum(us) / len(us)
            med = us[len(us) // 2] if len(us) % 2 else 0.5 * (us[len(us) // 2 - 1] + us[len(us) // 2])
            p90 = us[min(len(us) - 1, int(0.9 * len(us)))]
            lines.append(f"| {name} | {avg[name]:.2f} | {med:.2f} | {p90:.2f} | {us[0]:.2f} | {us[-1]:.2f} |")
        lines += ["", f"Sum of the two means: {avg['decode_kernel'] + avg['merge_kernel']:.2f} us."]
    if js:
        lines.append(f"bench.py's own line in the same profiled run: {js[-1]['ms_per_step'] * 1e3:.2f} us "
                     "per step (kernel boundaries overlap slightly in the trace's timestamps).")
    return "\n".join(lines) + "\n"


def ingest_counters(dirs, command_lines, kernel_names, per_wave_units=None):
    """Markdown table of rocprofv3 --pmc counters per kernel: the mean per dispatch over all
    dispatches of each kernel in the runs (one run per counter set; the SQ counters are summed
    over the chip).  per_wave_units: {kernel substring: (units of work per wave, label)} adds
    per-unit figures (instructions of each kind per wave and unit)."""
    import collections
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for d in dirs:
        for root, _, files in os.walk(d):
            for fn in files:
                if fn.endswith("counter_collection.csv"):
                    for r in _counter_rows(os.path.join(root, fn)):
                        k = r["Kernel_Name"].replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0]
                        agg[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
    lines = ["# Hardware counters per kernel", "", "Commands (one rocprofv3 --pmc run per counter set):", "", "```"]
    lines += command_lines + ["```", ""]
    for k, cs in sorted(agg.items()):
        if not any(n in k for n in kernel_names):
            continue
        lines += [f"## {k}", "", "| counter | mean per dispatch | dispatches |", "|---|---:|---:|"]
        mean = {c: sum(v) / len(v) for c, v in cs.items()}
        for c in sorted(mean):
            lines.append(f"| {c} | {mean[c]:,.1f} | {len(cs[c])} |")
        waves = mean.get("SQ_WAVES")
        for sub, (units, label) in (per_wave_units or {}).items():
            if sub in k and waves:
                lines += ["", f"Per wave and {label} ({units:g} per wave):", ""]
                for c in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_INSTS_VMEM"):
                    if c in mean:
                        lines.append(f"- {c}: {mean[c] / waves / units:,.1f}")
                for c in ("SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_ANY", "SQ_WAIT_INST_ANY", "SQ_VALU_MFMA_BUSY_CYCLES"):
                    if c in mean and "SQ_WAVE_CYCLES" in mean:
                        lines.append(f"- {c} / SQ_WAVE_CYCLES: {mean[c] / mean['SQ_WAVE_CYCLES']:.3f}")
        lines.append("")
    return "\n".join(lines) + "\n"


MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix-core peak


def bench_prefill(kvq, torch, wl, inp, caches, stream, chunk, reps=5):
    """The chunked-prefill attention of the last `chunk` positions of every sequence of the
    workload (their tokens are already in the pool), event-timed over `reps` calls rotating the
    pool copies, against the fp16 matrix-core peak."""
    dev = caches[0].pool.device
    rng = np.random.default_rng(2024)
    q = torch.from_numpy(rng.standard_normal((wl.n_seq, chunk, wl.n_q_heads, wl.head_dim),
                                             dtype=np.float32).astype(np.float16)).to(dev)
    pt = torch.from_numpy(np.ascontiguousarray(inp.page_table)).to(dev)
    sl = torch.from_numpy(np.ascontiguousarray(inp.seq_lens)).to(dev)
    msl = int(wl.seq_len)
    splits = kvq.prefill_num_splits(wl.n_seq, chunk, wl.n_q_heads, wl.num_kv_heads, msl)
    ws = torch.empty(kvq.prefill_workspace_bytes(wl.n_seq, chunk, wl.n_q_heads, wl.num_kv_heads,
                                                 wl.head_dim, msl), dtype=torch.uint8, device=dev)
    out = torch.empty((wl.n_seq, chunk, wl.n_q_heads, wl.head_dim), dtype=torch.float32,
                      device=dev)
    lse = torch.empty((wl.n_seq, chunk, wl.n_q_heads), dtype=torch.float32, device=dev)
    calls = [kvq.prepare_prefill(c, q, pt, sl, msl, out, lse, ws, stream=stream) for c in caches]
    calls[0]()  # warm-up
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for r in range(reps):
        calls[(r + 1) % len(calls)]()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    flops = prefill_attn_flops(inp.seq_lens, chunk, wl.n_q_heads, wl.head_dim)
    tflops = flops / (us * 1e-6) / 1e12
    log(f"[bench] prefill attention, chunk {chunk}: {us:.1f} us, {tflops:.1f} TFLOP/s")
    return {
        "chunk": chunk,
        "us": round(us, 1),
        "flops": flops,
        "splits": splits,
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4)},
        "kernel": "kvq_prefill_attn: prefill_kernel (256-row tiles x context pieces) + merge_kernel",
    }


def ingest_settling(trace_csv, command, group=100):
    """Markdown summary of a rocprofv3 --kernel-trace run of many steps: the decode kernel's
    duration and the call period per group of calls, showing how the rate settles."""
    rows = _counter_rows(trace_csv)
    d = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in rows
               if "decode_kernel" in r["Kernel_Name"])
    m = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in rows
               if "merge_kernel" in r["Kernel_Name"])
    durs = [(e - s) / 1e3 for s, e in d]
    lines = ["# Decode kernel duration over a sustained run", "", "Command:", "", "```", command, "```", "",
             f"{len(d)} back-to-back decode steps. Per group of {group} calls: the decode kernel's mean, "
             "min and max duration, and the call period (start to start).", "",
             "| calls | t at first call (ms) | decode_kernel mean us | min us | max us | call period us |",
             "|---|---:|---:|---:|---:|---:|"]
    for i in range(0, len(d) - 1, group):
        ch = durs[i:i + group]
        j = min(i + group, len(d) - 1)
        per = (d[j][0] - d[i][0]) / 1e3 / (j - i)
        lines.append(f"| {i}-{i + len(ch) - 1} | {(d[i][0] - d[0][0]) / 1e6:.1f} | {sum(ch) / len(ch):.2f} | "
                     f"{min(ch):.2f} | {max(ch):.2f} | {per:.2f} |")
    settled = durs[len(durs) // 10:]
    mm = [(e - s) / 1e3 for s, e in m[len(m) // 10:]]
    lines += ["", f"After the first tenth of the calls: decode_kernel mean {sum(settled) / len(settled):.2f} us, "
              f"merge_kernel mean {sum(mm) / max(len(mm), 1):.2f} us (both under the profiler)."]
    return "\n".join(lines) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    # 400 warm-up steps (about 22 ms): the decode kernel runs about 6 us slower for the first
    # ~12 ms of a sustained run on this GPU, then settles (a kernel trace of 3,000 steps shows
    # it); the timed steps measure the settled rate
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--workload", default=None, help="name in workloads.WORKLOADS")
    ap.add_argument("--kv-format", default="k8v4", choices=["k8v4", "k8v8", "fp8"],
                    help="KV cache format: 4-bit (the headline) or 8-bit V codes")
    ap.add_argument("--copies", type=int, default=8, help="pool copies rotated for a cold cache")
    ap.add_argument("--splits", type=int, default=0, help="0 = automatic split plan")
    ap.add_argument("--window", type=int, default=0,
                    help="sliding window: each row sees only its last W tokens (0 = all)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sustained", type=int, default=600,
                    help="after everything timed, this many more back-to-back steps in groups of "
                         "50, each followed by a shader-clock reading (0: skip); reported apart "
                         "from the timed value")
    ap.add_argument("--no-attainable", action="store_true",
                    help="skip the streaming-read probe (it also runs right before the warm-up)")
    ap.add_argument("--prefill-chunk", type=int, default=1024,
                    help="positions of the chunked-prefill measurement (0: skip it)")
    ap.add_argument("--unfused", action="store_true",
                    help="time kvq_append + kvq_decode_attn instead of kvq_decode_step")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the per-launch HBM traffic of rocprofv3 counter CSVs to profiles/")
    ap.add_argument("--ingest-trace", metavar="KERNEL_STATS_CSV",
                    help="write a markdown summary of a rocprofv3 kernel-stats CSV to profiles/")
    ap.add_argument("--command", default="", help="command line recorded with an ingested profile")
    ap.add_argument("--ingest-settling", metavar="KERNEL_TRACE_CSV",
                    help="summarize a long --kernel-trace run: decode duration per group of calls")
    ap.add_argument("--ingest-out", default=None,
                    help="file name under profiles/ for --ingest-trace (default: the decode trace)")
    ap.add_argument("--ingest-counters", nargs="+", metavar="DIR",
                    help="summarize rocprofv3 --pmc runs (counter_collection.csv under each DIR) into "
                         "profiles/ (--ingest-out names the file)")
    ap.add_argument("--bench-log", default=None,
                    help="stdout of bench.py in the profiled run (its JSON line), for --ingest-trace")
    args = ap.parse_args(argv)

    if args.ingest_counters:
        from long_context_decode_flash_amd import workloads as W
        wl = W.WORKLOADS[args.workload or W.HEADLINE]
        splits = int(args.splits) or None
        units = {}
        if splits:
            blocks = -(-wl.seq_len // 32) * wl.n_seq * wl.num_kv_heads / (splits * wl.n_seq * wl.num_kv_heads * 4)
            units["decode_kernel"] = (blocks, "32-token block")
        path = os.path.join(ROOT, "profiles", args.ingest_out or f"counters_{args.workload or W.HEADLINE}.md")
        with open(path, "w") as f:
            f.write(ingest_counters(args.ingest_counters, args.command.split(" ;; ") if args.command else [],
                                    ["decode_kernel", "merge_kernel", "prefill_kernel", "append_kernel",
                                     "stream_read"], units))
        print(path)
        return 0

    if args.ingest_settling:
        from long_context_decode_flash_amd import workloads as W
        path = os.path.join(ROOT, "profiles", args.ingest_out or
                            f"decode_{args.workload or W.HEADLINE}_settling_trace.md")
        with open(path, "w") as f:
            f.write(ingest_settling(args.ingest_settling, args.command))
        print(path)
        return 0

    if args.ingest_pmc or args.ingest_trace:
        from long_context_decode_flash_amd import workloads as W
        name = args.workload or W.HEADLINE
        os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
        if args.ingest_pmc:
            res = ingest_pmc(*args.ingest_pmc, name, args.copy_probe_mib or 1024,
                             args.command.split(" ;; ") if args.command else [])
            path = os.path.join(ROOT, "profiles", f"decode_{name}_pmc.json")
            with open(path, "w") as f:
                json.dump(res, f, indent=1)
        else:
            path = os.path.join(ROOT, "profiles", args.ingest_out or f"decode_{name}_kernel_trace.md")
            with open(path, "w") as f:
                f.write(ingest_trace(args.ingest_trace, args.command, args.bench_log))
        print(path)
        return 0

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): there is no "
              "multi-GPU path here (the decode would shard by KV head or by sequence, with one "
              "partial per row exchanged only when a sequence is cut across GPUs).",
              file=sys.stderr)
        return 2

    import torch
    from long_context_decode_flash_amd import kvq
    from long_context_decode_flash_amd import workloads as W

    name = args.workload or W.HEADLINE
    wl = W.WORKLOADS[name]
    dev = torch.device("cuda:0")
    log(f"[bench] workload {name}: generating inputs")
    inp = W.generate(wl)
    D = wl.head_dim

    def dev_t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    fmt = kvq.FORMATS[args.kv_format]
    vbits = 4 if fmt == kvq.KVQ_FORMAT_K8V4 else 8  # fp8 codes use the 8-bit V layout
    caches = [kvq.PagedCache.allocate(wl.pool_pages, wl.page_size, wl.num_kv_heads, D, dev,
                                      kv_format=fmt)]
    k_pre, v_pre, s_pre = (dev_t(x) for x in inp.prefill())
    # The prefill append (one kvq_append call per sequence, over all its cached tokens, as an
    # engine's prefill writes them) fills the pool here; it is timed after the decode.
    n_pre = int(s_pre.numel())
    per = n_pre // wl.n_seq  # tokens are sequence-major, the same count per sequence
    apps = [kvq.prepare_append(caches[0], k_pre[i * per:(i + 1) * per], v_pre[i * per:(i + 1) * per],
                               s_pre[i * per:(i + 1) * per]) for i in range(wl.n_seq)]
    for app in apps:
        app()
    torch.cuda.synchronize()
    for _ in range(args.copies - 1):
        c = kvq.PagedCache.allocate(wl.pool_pages, wl.page_size, wl.num_kv_heads, D, dev,
                                    kv_format=fmt)
        c.pool.copy_(caches[0].pool)
        caches.append(c)
    k_new, v_new, s_new = (dev_t(x) for x in inp.step_tokens())
    q = dev_t(inp.q_bits).view(torch.float16)
    pt = dev_t(inp.page_table)
    sl = dev_t(inp.seq_lens)
    msl = int(wl.seq_len)
    win = args.window
    splits = kvq.decode_num_splits(wl.n_seq, wl.num_kv_heads, msl, args.splits, n_rows=wl.n_rows,
                                   window=win, kv_format=fmt)
    ws = torch.zeros(kvq.decode_workspace_bytes(wl.n_seq, wl.n_rows, wl.n_q_heads,
                                                wl.num_kv_heads, D, msl, args.splits, window=win),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((wl.n_seq, wl.n_rows, wl.n_q_heads, D), dtype=torch.float32, device=dev)
    lse = torch.empty((wl.n_seq, wl.n_rows, wl.n_q_heads), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize()
    log(f"[bench] pool {caches[0].pool.numel() / 1e6:.1f} MB x {len(caches)} copies, "
        f"splits {splits}")

    # One step is one kvq_decode_step call (the step's new tokens appended inside the decode
    # launch); --unfused times kvq_append + kvq_decode_attn instead.
    k_rows = torch.from_numpy(np.ascontiguousarray(inp.k[:, wl.seq_len - wl.n_new:])).to(dev)
    v_rows = torch.from_numpy(np.ascontiguousarray(inp.v[:, wl.seq_len - wl.n_new:])).to(dev)
    calls = []
    for c in caches:
        if args.unfused:
            app = kvq.prepare_append(c, k_new, v_new, s_new, stream=stream) if wl.n_new else None
            dec = kvq.prepare_decode_attn(c, q, pt, sl, msl, out, lse, ws,
                                          num_splits=args.splits, stream=stream, window=win)
            calls.append((lambda app=app, dec=dec: (app and app(), dec())))
        else:
            calls.append(kvq.prepare_decode_step(c, k_rows if wl.n_new else None,
                                                 v_rows if wl.n_new else None, q, pt, sl, msl,
                                                 out, lse, ws, num_splits=args.splits,
                                                 stream=stream, window=win))

    def step(i):
        calls[i % len(calls)]()

    # The timed decode comes first after the set-up: the other measurements (the attainable
    # streaming read, the append timings, the prefill attention) stream for tens of
    # milliseconds, and the GPU's power management answers such a load by lowering the shader
    # clock for some milliseconds after it (measured with kvq_probe_clock), which the timed
    # steps would otherwise inherit.
    telemetry = {"idle": read_telemetry()}
    clk = ShaderClock(kvq, torch, dev, stream)
    torch.cuda.synchronize()
    clk_at = {}

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} steps done; timing {args.steps} steps")

    # The timed region: K steps bracketed by two events.  No event sits between the calls: each
    # event record costs the stream a few microseconds of its own.
    # The shader clock is read right before the start event and right after the end event, on
    # the same stream, outside the timed region.
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    clk_at["before_timed_steps"] = clk.enqueue()
    t_wall = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        step(i)
    end.record(stream)
    clk_at["after_timed_steps"] = clk.enqueue()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    telemetry["after_timed_steps"] = read_telemetry()
    telemetry["shader_clock"] = {k: clk.read(i) for k, i in clk_at.items()}
    attainable = None
    if not args.no_attainable:
        attainable = attainable_probe(kvq, torch, dev, stream)
    append_res = time_appends(kvq, torch, wl, inp, caches, apps, n_pre, D, vbits, dev_t, args.prefill_chunk)
    del k_pre, v_pre, apps
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    log(f"[bench] {args.steps} steps in {total_ms:.2f} ms (wall {wall * 1e3:.1f} ms): "
        f"{ms_per_step * 1e3:.1f} us per step")

    dec_bytes = decode_algorithmic_bytes(wl, inp.seq_lens, vbits, win)
    step_bytes = dec_bytes + (append_algorithmic_bytes(wl, vbits) if wl.n_new else 0)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = value  # the step is one call: the attention launch (with the append) + the merge

    traffic = None
    pmc_file = os.path.join(ROOT, "profiles", f"decode_{name}_pmc.json")
    if os.path.exists(pmc_file):
        with open(pmc_file) as f:
            pmc = json.load(f)
        if (pmc.get("library_hash") == library_hash() and pmc.get("workload") == name and
                args.kv_format == "k8v4"):
            traffic = pmc.get("hbm_bytes_per_launch")

    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"[bench] copy probe: {args.copy_probe_mib} MiB device copy x3")

    res = {
        "metric": "decode-attn HBM GB/s (% of MI355X peak) + steps/s at 184K ctx, K8/V4 paged KV",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "steps_per_s": round(1e3 / ms_per_step, 1),
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": name + (f"_window{win}" if win else ""), "n_seq": wl.n_seq,
            "seq_len": wl.seq_len, "window": win,
            "kv_heads": wl.num_kv_heads, "q_heads": wl.n_q_heads, "head_dim": D,
            "page_size": wl.page_size, "pool_pages": wl.pool_pages,
            "page_order": wl.page_order, "query_rows": wl.n_rows, "new_tokens_per_seq": wl.n_new,
            "kv_format": {kvq.KVQ_FORMAT_K8V4: "K int8/token scale, V int4/32-dim scale",
                          kvq.KVQ_FORMAT_K8V8: "K int8/token scale, V int8/32-dim scale",
                          kvq.KVQ_FORMAT_FP8: "K e4m3/token scale, V e4m3/32-dim scale"}[fmt],
            "splits": splits,
            "pool_copies": len(caches), "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": ("kvq_append + kvq_decode_attn" if args.unfused else
                       "kvq_decode_step: decode_kernel (fused append + split-KV attention) + "
                       "merge_kernel (LSE merge of the splits)"),
            "algorithmic_bytes_per_launch": step_bytes,
            "launch_us_mean": round(ms_per_step * 1e3, 2),
        },
    }
    if attainable is not None:
        best, rows, nbytes = attainable
        res["roofline"]["attainable"] = best["GB_s"]
        res["roofline"]["frac_of_attainable"] = round(achieved / best["GB_s"], 4)
        res["attainable_read"] = {"best": best, "bytes": nbytes, "sweep": rows,
                                  "kernel": "kvq_probe_stream_read (plain streaming read)"}
    res["telemetry"] = telemetry
    if args.sustained > 0:
        res["sustained"] = sustained_run(torch, stream, step, clk, args.sustained)

    if args.prefill_chunk > 0 and not win:
        res["prefill_attn"] = bench_prefill(kvq, torch, wl, inp, caches, stream, args.prefill_chunk)

    res["prefill_append"] = append_res
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline: oracle on full steps, about 10 s")
        dt, n_cpu, cores = cpu_baseline(wl, inp, window=win, kv_format=fmt)
        res["cpu_baseline"] = {
            "value": round(step_bytes / dt / 1e9, 4),
            "unit": "GB/s",
            "cores": cores,
            "kind": "oracle",
            "sample": f"{n_cpu} full steps of {name} (each: append of {wl.n_seq * wl.n_new} "
                      f"tokens + attention of all {wl.n_seq * wl.n_rows * wl.n_q_heads} output rows "
                      f"over {min(wl.seq_len, win) if win else wl.seq_len} tokens each), fp64, "
                      f"{dt * n_cpu:.1f} s in all",
            "s_per_step": round(dt, 3),
            "cpu_model": cpu_model(),
        }
        log("[bench] cpu baseline: one-thread sample")
        dt1, sample1 = cpu_baseline_one_thread(wl, inp, window=win, kv_format=fmt)
        res["cpu_baseline"]["one_thread"] = {"s_per_step": round(dt1, 2),
                                             "value": round(step_bytes / dt1 / 1e9, 5),
                                             "sample": sample1}
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

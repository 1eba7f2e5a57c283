#!/usr/bin/env python3
"""CompKV decode-step benchmark on one MI355X.

One step = one layer's decode step for the workload's batch, through the
fused entry point cknv_decode_step: the streaming scoring pass over the
summaries with the append and the refresh of the block the token lands in
(score_kernel), then normalisers + selection + exact attention with Mean
compensation (step_kernel; when a unit's kept blocks are split over several
workgroups, the last of them merges the parts). Inputs are the seeded synthetic workload, resident in
HBM before timing. Steps rotate over R copies of the layer ("layers") at
distinct addresses so the per-step working set cannot stay in the 256 MB
Infinity Cache.

Prints ONE JSON line. `value` = steps/s from HIP-graph replay of whole layer
sweeps (HIP events around exactly K timed steps). `roofline` is for the
dominant kernel, the streaming score_kernel (issued alone by
cknv_decode_score): its algorithmic bytes per launch over its average
duration, measured with HIP events on the launch stream around sweeps of
back-to-back launches, one per layer. `cpu_baseline` times the fp64 oracle's per-step path on a bounded
sample on the host. The three-call path (cknv_append, cknv_score_select,
cknv_attend) and the dense baseline are reported beside it.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama8b_32k]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode steps/sec (1 layer, B=1) at 32K/128K ctx + achieved HBM GB/s vs peak"
PEAK_HBM_GBPS = 8000.0
MALL_BYTES = 256 * 2 ** 20
SCORE_SOURCES = ["block_sparse_kv_stats_amd/csrc/score.hip",
                 "block_sparse_kv_stats_amd/csrc/cknv_internal.h",
                 "block_sparse_kv_stats_amd/csrc/summary_core.h"]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def step_bytes(w, T: int):
    """Algorithmic HBM bytes of one fused step over all units, split by
    kernel (T = tokens after the step's append).
    score_kernel: k̄ + D̄ + |b| of every block closed before the step and v̄
    of those of them that are not kept; the append (the open block's cached
    BF16 tokens read, the token and its block's summary written);
    step_kernel: BF16 K and V of the kept blocks' tokens."""
    U = w.S * w.H
    NB = math.ceil(T / 16)
    closed = (T - 1) // 16
    kept = min(w.Kb, NB)
    kept_closed = kept - (NB - closed)  # the block holding the new token is always kept
    open_n = T - 16 * (NB - 1)
    append = (open_n - 1) * 2 * w.d * 2 + 2 * w.d * 2 + (2 * w.d + w.r + 1) * 4
    score = U * (closed * (w.d + w.r + 1) * 4 + (closed - kept_closed) * w.d * 4 + append)
    kept_tokens = (kept - 1) * 16 + open_n
    attend = U * kept_tokens * 2 * w.d * 2
    return score, attend


def dense_bytes(w, T: int) -> int:
    return w.S * w.H * T * 2 * w.d * 2


def build_bytes(w, T: int) -> int:
    """Algorithmic HBM bytes of one bulk summary build over T tokens per
    unit: the BF16 K and V read once, every block's summary written once."""
    NB = math.ceil(T / 16)
    return w.S * w.H * (T * 2 * w.d * 2 + NB * (2 * w.d + w.r + 1) * 4)


class Bench:
    def __init__(self, w, R, appends, stream):
        import numpy as np
        import torch
        from block_sparse_kv_stats_amd import cknv, synth

        self.w, self.R, self.stream = w, R, stream
        wl = w.replace(steps=max(w.steps, 1), extra_cap=appends + 16)
        log(f"generating {w.name}")
        data = synth.gen_layer(wl)
        T0 = w.prefill[0]
        cap_blocks = wl.cap_blocks
        self.max_blocks = math.ceil((T0 + appends) / 16)
        shape = cknv.make_shape(w.S, w.H, w.G, w.d, w.r, cap_blocks)
        self.shape = shape

        def dev_bf16(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)

        base = cknv.LayerCache.allocate(shape)
        kk = np.zeros((w.S, w.H, cap_blocks * 16, w.d), dtype=np.uint16)
        vv = np.zeros_like(kk)
        kk[:, :, :T0] = data["k"][:, :, :T0]
        vv[:, :, :T0] = data["v"][:, :, :T0]
        base.k.copy_(dev_bf16(kk))
        base.v.copy_(dev_bf16(vv))
        del kk, vv
        base.seq_len.fill_(T0)
        cknv.build_summaries(base, self.max_blocks)
        torch.cuda.synchronize()
        log(f"replicating {R} layers")
        self.layers = [base] + [cknv.LayerCache(shape, *(t.clone() for t in (
            base.k, base.v, base.kbar, base.dbar, base.cnt, base.vbar, base.seq_len)))
            for _ in range(R - 1)]
        nq = w.steps if w.steps > 1 else 1
        self.q = [torch.from_numpy(data["q"][i % nq]).cuda() for i in range(R)]
        self.new_k = dev_bf16(data["k"][:, :, T0])
        self.new_v = dev_bf16(data["v"][:, :, T0])
        self.ws = cknv.allocate_workspace(shape, self.max_blocks, w.budget, stream=stream)
        U = w.S * w.H
        self.sel = torch.zeros((U, w.Kb), dtype=torch.int32, device="cuda")
        self.n_sel = torch.zeros((U,), dtype=torch.int32, device="cuda")
        self.out = torch.zeros((w.S, w.H * w.G, w.d), dtype=torch.float32, device="cuda")
        self.lse = torch.zeros((w.S, w.H * w.G), dtype=torch.float32, device="cuda")
        self.bound = [cknv.BoundStep(L, self.max_blocks, w.budget, self.ws, self.sel, self.n_sel,
                                     self.out, self.lse, self.q[i], self.new_k, self.new_v, stream)
                      for i, L in enumerate(self.layers)]
        torch.cuda.synchronize()

    def seq_len(self):
        return int(self.layers[0].seq_len[0].item())


class Timer:
    """HIP-event timing on the launch stream. Before each measured region a
    spin kernel gives the host a head start, so the queued launches run back
    to back and host launch latency does not enter the intervals."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream
        e0, e1 = self.event(), self.event()
        with torch.cuda.stream(stream):
            torch.cuda._sleep(1000)
            e0.record(stream)
            torch.cuda._sleep(20_000_000)
            e1.record(stream)
        torch.cuda.synchronize()
        self.cycles_per_ms = 20_000_000 / max(e0.elapsed_time(e1), 1e-3)

    def event(self):
        return self.torch.cuda.Event(enable_timing=True)

    def head_start(self, ms):
        self.torch.cuda._sleep(int(self.cycles_per_ms * ms))


def capture(torch, stream, fn):
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=stream):
        fn()
    torch.cuda.synchronize()
    return g


def time_graph_steps(torch, timer, stream, bench, steps, which="step"):
    """ms per step over exactly `steps` steps, replaying captured layer sweeps."""
    R = bench.R
    full = capture(torch, stream, lambda: [getattr(b, which)() for b in bench.bound])
    rem = steps % R
    part = capture(torch, stream, lambda: [getattr(b, which)() for b in bench.bound[:rem]]) if rem else None
    e0, e1 = timer.event(), timer.event()
    with torch.cuda.stream(stream):
        timer.head_start(5.0 + 0.02 * (steps // R + 1))
        e0.record(stream)
        for _ in range(steps // R):
            full.replay()
        if part is not None:
            part.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def time_eager_steps(torch, timer, stream, bench, n):
    e0, e1 = timer.event(), timer.event()
    with torch.cuda.stream(stream):
        timer.head_start(5.0 + 0.08 * n)
        e0.record(stream)
        for i in range(n):
            bench.bound[i % bench.R].fused_step()
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def time_step_percentiles(torch, timer, stream, bench, n):
    """Per-step durations (ms) of eager fused steps, each between two HIP
    events on the launch stream (the launches queued behind a spin kernel,
    so host launch latency stays out): p10, median and p90."""
    evs = [(timer.event(), timer.event()) for _ in range(n)]
    with torch.cuda.stream(stream):
        timer.head_start(5.0 + 0.08 * n)
        for i in range(n):
            evs[i][0].record(stream)
            bench.bound[i % bench.R].fused_step()
            evs[i][1].record(stream)
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(c) for a, c in evs)
    pick = lambda f: ts[min(len(ts) - 1, int(f * len(ts)))]
    return pick(0.1), pick(0.5), pick(0.9)


def time_score_kernel(torch, timer, stream, bench, sweeps):
    """Average duration (ms) of the streaming score kernel: sweeps of
    back-to-back cknv_decode_score launches over the R layers, each sweep
    between two HIP events on the launch stream (a launch only rewrites the
    workspace, so repeating it leaves the layers unchanged). Returns the mean
    and the median over sweeps of the per-launch time."""
    evs = [(timer.event(), timer.event()) for _ in range(sweeps)]
    with torch.cuda.stream(stream):
        timer.head_start(5.0 + 0.03 * sweeps * bench.R)
        for i in range(sweeps):
            evs[i][0].record(stream)
            for b in bench.bound:
                b.decode_score()
            evs[i][1].record(stream)
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(c) / bench.R for a, c in evs)
    return sum(ts) / len(ts), ts[len(ts) // 2]


def time_kernel_events(torch, timer, stream, bench, n, which):
    """Average and median duration (ms) of one half of the fused step inside
    full eager steps, bracketed by HIP events on the launch stream."""
    evs = [(timer.event(), timer.event()) for _ in range(n)]
    with torch.cuda.stream(stream):
        timer.head_start(5.0 + 0.12 * n)
        for i in range(n):
            b = bench.bound[i % bench.R]
            if which == "decode_score":
                evs[i][0].record(stream)
                b.decode_score()
                evs[i][1].record(stream)
                b.decode_finish()
            else:
                b.decode_score()
                evs[i][0].record(stream)
                b.decode_finish()
                evs[i][1].record(stream)
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(c) for a, c in evs)
    return sum(ts) / len(ts), ts[len(ts) // 2]


def cpu_baseline(w, seconds: float):
    """The fp64 oracle's per-step path (open-block update, score, select,
    attend), single thread, on every (sequence, KV head) unit of sequence 0 in
    turn: each unit runs up to `seconds`/H of consecutive steps from the
    workload's context, and a step over all units costs the sum of the units'
    mean step times, scaled by S."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from block_sparse_kv_stats_amd import synth
    from oracle import compkv as ok

    n_max = 2500  # per unit: the context grows by at most this many tokens
    T0 = w.prefill[0]
    wl = w.replace(steps=max(w.steps, 1), extra_cap=n_max)
    per_step, steps, timed = 0.0, 0, 0.0
    with threadpool_limits(limits=1):
        for h in range(w.H):
            u = synth.gen_unit(wl, 0, h, ntok=T0 + n_max)
            q = u["q"][0]
            su = ok.StreamingUnit(u["k"], u["v"], T0, w.r, cap_tokens=T0 + n_max)
            t0 = time.perf_counter()
            n = 0
            while n < n_max:
                su.append(u["k"][T0 + n], u["v"][T0 + n])
                su.step(q, w.budget)
                n += 1
                if time.perf_counter() - t0 > seconds / w.H:
                    break
            dt = time.perf_counter() - t0
            per_step += dt / n
            steps += n
            timed += dt
    per_step *= w.S
    return {"value": 1.0 / per_step, "unit": "steps/s", "cores": 1, "kind": "oracle",
            "sample": f"{steps} steps over the {w.H} (sequence, KV head) units of sequence 0 of "
                      f"{w.name}, up to {n_max} consecutive steps each from {T0} tokens "
                      f"({timed:.1f} s, fp64 NumPy, 1 thread); a step is the sum of the units' "
                      f"mean step times" + (f", x{w.S} sequences" if w.S > 1 else "")}


def traffic_from_profile(workload):
    """HBM bytes per score_kernel launch from a committed rocprofv3 PMC
    summary, if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"score_kernel_{workload}_pmc.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != kernel_source_hash(SCORE_SOURCES):
        return None
    return rec.get("hbm_bytes_per_launch")


def run_workload(torch, timer, wname, args, stream, want_dense=True):
    from block_sparse_kv_stats_amd import synth

    w = synth.WORKLOADS[wname]
    sb, ab = step_bytes(w, w.prefill[0] + 1)
    R = args.layers or max(4, math.ceil(2 * MALL_BYTES / (sb + ab)))
    steps, warm = args.steps, args.warmup
    n_e = min(steps, 256)
    kernel_n = min(max(2 * R, 64), 256)
    appends = (math.ceil(warm / R) + math.ceil(steps / R) + 2 * math.ceil(n_e / R)
               + 2 * math.ceil(kernel_n / R) + math.ceil(max(R, steps // 4) / R) + 4)
    bench = Bench(w, R, appends, stream)
    log(f"{wname}: {R} layers, {warm} warm-up + {steps} timed steps")
    with torch.cuda.stream(stream):
        for i in range(warm):
            bench.bound[i % R].fused_step()
    torch.cuda.synchronize()
    ms_step = time_graph_steps(torch, timer, stream, bench, steps, which="fused_step")
    ms_eager = time_eager_steps(torch, timer, stream, bench, n_e)
    pct = time_step_percentiles(torch, timer, stream, bench, n_e)
    k_avg, k_med = time_score_kernel(torch, timer, stream, bench, max(8, 256 // R))
    f_avg, f_med = time_kernel_events(torch, timer, stream, bench, kernel_n, "decode_finish")
    ms_three = time_graph_steps(torch, timer, stream, bench, max(R, steps // 4), which="step")
    ms_build = time_build(torch, timer, stream, bench, max(2, 64 // R))
    T = bench.seq_len()
    sb, ab = step_bytes(w, T)
    res = {"w": w, "R": R, "steps": steps, "warmup": warm, "ms_step": ms_step,
           "ms_eager": ms_eager, "step_us_p10_p50_p90": [round(x * 1e3, 2) for x in pct], "T": T, "score_bytes": sb, "attend_bytes": ab,
           "score_ms": k_avg, "score_ms_median": k_med, "finish_ms": f_avg,
           "ms_three_calls": ms_three, "build_ms": ms_build, "build_bytes": build_bytes(w, T)}
    if want_dense:
        res["dense_ms_step"] = time_graph_steps(torch, timer, stream, bench, max(R, steps // 4),
                                                which="dense")
        res["dense_bytes"] = dense_bytes(w, bench.seq_len())
    del bench
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def time_build(torch, timer, stream, bench, sweeps):
    """Average duration (ms) of cknv_build_summaries over a whole layer
    (rebuilds what is there, so repeats are harmless), rotating the R layers so
    every launch reads its cache from HBM."""
    from block_sparse_kv_stats_amd import cknv
    e0, e1 = timer.event(), timer.event()
    with torch.cuda.stream(stream):
        timer.head_start(5.0 + 0.3 * sweeps * bench.R)
        e0.record(stream)
        for _ in range(sweeps):
            for L in bench.layers:
                cknv.build_summaries(L, bench.max_blocks, stream=stream)
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (sweeps * bench.R)


def copy_probe(nbytes: int, reps: int):
    """A plain device copy of known size (calibrates the rocprofv3 byte counters)."""
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "reps": reps}))


PROFILE_COMMANDS = {
    "trace": 'rocprofv3 --kernel-trace --stats -f csv -d $OUT/trace -o trace -- '
             'python3 bench.py --no-cpu --no-dense',
    "fetch": 'rocprofv3 --pmc FETCH_SIZE -f csv -d $OUT/fetch -o fetch -- '
             'python3 bench.py --steps 8 --warmup 2 --no-cpu --no-dense --also ""',
    "write": 'rocprofv3 --pmc WRITE_SIZE -f csv -d $OUT/write -o write -- '
             'python3 bench.py --steps 8 --warmup 2 --no-cpu --no-dense --also ""',
    "fetch128": 'rocprofv3 --pmc FETCH_SIZE -f csv -d $OUT/fetch128 -o fetch128 -- '
                'python3 bench.py --steps 8 --warmup 2 --no-cpu --no-dense --workload qwen8b_128k --also ""',
    "write128": 'rocprofv3 --pmc WRITE_SIZE -f csv -d $OUT/write128 -o write128 -- '
                'python3 bench.py --steps 8 --warmup 2 --no-cpu --no-dense --workload qwen8b_128k --also ""',
    "copy_fetch": 'rocprofv3 --pmc FETCH_SIZE -f csv -d $OUT/copy_fetch -o cf -- '
                  'python3 bench.py --copy-probe 268435456',
    "copy_write": 'rocprofv3 --pmc WRITE_SIZE -f csv -d $OUT/copy_write -o cw -- '
                  'python3 bench.py --copy-probe 268435456',
    "summary": 'python3 bench.py --summarize-profiles $OUT',
}
COPY_PROBE_BYTES = 268435456


def _csv_rows(directory, suffix):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True)):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _counter_per_dispatch(directory, counter, name_part, grid=None):
    """Per-dispatch values of one counter for kernels whose name contains name_part."""
    vals = []
    for r in _csv_rows(directory, "counter_collection.csv"):
        if name_part in r["Kernel_Name"] and r["Counter_Name"] == counter:
            if grid is None or int(r["Grid_Size"]) == grid:
                vals.append(float(r["Counter_Value"]))
    return vals


def summarize_profiles(out_dir):
    """Write profiles/ summaries from the rocprofv3 runs listed in
    PROFILE_COMMANDS (their CSV output under out_dir)."""
    import statistics
    from block_sparse_kv_stats_amd import synth
    prof = os.path.join(ROOT, "profiles")
    os.makedirs(prof, exist_ok=True)
    # ---- kernel trace: per (kernel, grid) duration statistics
    stats = {}
    for r in _csv_rows(os.path.join(out_dir, "trace"), "kernel_trace.csv"):
        name = r["Kernel_Name"]
        if "cknv" not in name:
            continue
        key = (name.split("(")[0].replace("void ", ""), int(r["Grid_Size_X"]))
        stats.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = ["# Kernel durations, bench.py default workloads (Llama-3.1-8B 32K, Qwen3-8B 128K)", "",
             "Command (from the repository root, OUT = an output directory):", "",
             "    " + PROFILE_COMMANDS["trace"], "    " + PROFILE_COMMANDS["summary"], "",
             "rocprofv3 kernel trace of every dispatch of the run (graph replays included),",
             "grouped by kernel and grid size (threads). Durations in microseconds.", "",
             "| kernel | grid threads | dispatches | avg us | median us | min us | max us |",
             "|---|---|---|---|---|---|---|"]
    for (name, grid), d in sorted(stats.items(), key=lambda kv: (kv[0][0], kv[0][1])):
        lines.append(f"| {name} | {grid} | {len(d)} | {statistics.mean(d):.2f} | "
                     f"{statistics.median(d):.2f} | {min(d):.2f} | {max(d):.2f} |")
    with open(os.path.join(prof, "kernels_llama8b_32k_qwen8b_128k_trace.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    # ---- HBM traffic of score_kernel per workload, calibrated on a plain copy
    cf = _counter_per_dispatch(os.path.join(out_dir, "copy_fetch"), "FETCH_SIZE", "copy")
    cw = _counter_per_dispatch(os.path.join(out_dir, "copy_write"), "WRITE_SIZE", "copy")
    if not (cf and cw):
        print("missing copy calibration data", file=sys.stderr)
        return
    kib = COPY_PROBE_BYTES / 1024.0
    f_cal = kib / statistics.median(cf)   # bytes per counted KiB, read side
    w_cal = kib / statistics.median(cw)   # ... write side
    for wname, kf, kw in (("llama8b_32k", "fetch", "write"), ("qwen8b_128k", "fetch128", "write128")):
        w = synth.WORKLOADS[wname]
        fetch = _counter_per_dispatch(os.path.join(out_dir, kf), "FETCH_SIZE", "score_kernel")
        write = _counter_per_dispatch(os.path.join(out_dir, kw), "WRITE_SIZE", "score_kernel")
        if not (fetch and write):
            print(f"missing counter data for {wname}", file=sys.stderr)
            continue
        fb = statistics.median(fetch) * 1024.0 * f_cal
        wb = statistics.median(write) * 1024.0 * w_cal
        T = w.prefill[0] + 1
        sb, _ = step_bytes(w, T)
        rec = {"kernel": "score_kernel", "workload": w.name,
               "source_hash": kernel_source_hash(SCORE_SOURCES),
               "fetch_KiB_per_dispatch_median": statistics.median(fetch),
               "write_KiB_per_dispatch_median": statistics.median(write),
               "dispatches": [len(fetch), len(write)],
               "copy_probe_bytes": COPY_PROBE_BYTES,
               "copy_fetch_KiB": statistics.median(cf), "copy_write_KiB": statistics.median(cw),
               "calibration_fetch": round(f_cal, 4), "calibration_write": round(w_cal, 4),
               "hbm_read_bytes_per_launch": int(fb), "hbm_write_bytes_per_launch": int(wb),
               "hbm_bytes_per_launch": int(fb + wb),
               "algorithmic_bytes_per_launch_first_step": sb,
               "commands": [PROFILE_COMMANDS[k] for k in (kf, kw, "copy_fetch", "copy_write",
                                                          "summary")]}
        with open(os.path.join(prof, f"score_kernel_{wname}_pmc.json"), "w") as f:
            json.dump(rec, f, indent=1)
        print(json.dumps(rec))


def build_line(res):
    gbps = res["build_bytes"] / (res["build_ms"] * 1e-3) / 1e9
    return {"kernel": "build_kernel (cknv_build_summaries)", "avg_us": round(res["build_ms"] * 1e3, 2),
            "algorithmic_bytes": res["build_bytes"], "GBps": round(gbps, 1),
            "frac": round(gbps / PEAK_HBM_GBPS, 4)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--workload", default="llama8b_32k")
    ap.add_argument("--also", default="qwen8b_128k", help="second workload reported beside ('' = none)")
    ap.add_argument("--layers", type=int, default=0, help="layer copies to rotate over (0 = auto)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, help="run only a device copy of this many bytes")
    ap.add_argument("--summarize-profiles", default="",
                    help="write profiles/ summaries from rocprofv3 output in this directory")
    args = ap.parse_args()
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (this build has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe:
        copy_probe(args.copy_probe, 5)
        return
    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    timer = Timer(torch, stream)

    main_res = run_workload(torch, timer, args.workload, args, stream, want_dense=not args.no_dense)
    extra = None
    if args.also and args.also != args.workload:
        extra = run_workload(torch, timer, args.also, args, stream, want_dense=not args.no_dense)

    w = main_res["w"]
    value = 1000.0 / main_res["ms_step"]
    score_gbps = main_res["score_bytes"] / (main_res["score_ms"] * 1e-3) / 1e9
    step_gbps = (main_res["score_bytes"] + main_res["attend_bytes"]) / (main_res["ms_step"] * 1e-3) / 1e9
    traffic = traffic_from_profile(args.workload)
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": main_res["steps"],
        "warmup": main_res["warmup"],
        "ms_per_step": round(main_res["ms_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 (bf16 KV, fp32 summaries)",
        "data": "synthetic (seeded generator: block-structured bf16 keys, 1% needles, N(0,1) values)",
        "config": {"workload": w.name, "S": w.S, "H": w.H, "G": w.G, "d": w.d, "r": w.r,
                   "context_tokens": main_res["T"], "budget_tokens": w.budget,
                   "layers_rotated": main_res["R"],
                   "launch": "hipGraph replay of layer sweeps of cknv_decode_step"},
        "step_GBps": round(step_gbps, 1),
        "eager_ms_per_step": round(main_res["ms_eager"], 5),
        "eager_step_us_p10_p50_p90": main_res["step_us_p10_p50_p90"],
        "roofline": {"bound": "hbm", "kernel": "score_kernel (cknv_decode_score)",
                     "achieved": round(score_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(score_gbps / PEAK_HBM_GBPS, 4),
                     "traffic": traffic,
                     "algorithmic_bytes_per_launch": main_res["score_bytes"],
                     "avg_launch_us": round(main_res["score_ms"] * 1e3, 3),
                     "median_sweep_us_per_launch": round(main_res["score_ms_median"] * 1e3, 3),
                     "timing": "HIP events around back-to-back launches (one per layer)"},
        "finish_kernels": {"kernels": "step_kernel (cknv_decode_finish)",
                           "avg_us": round(main_res["finish_ms"] * 1e3, 3),
                           "algorithmic_bytes": main_res["attend_bytes"]},
        "three_call_path": {"steps_per_s": round(1000.0 / main_res["ms_three_calls"], 2),
                            "calls": "cknv_append + cknv_score_select + cknv_attend"},
        "bulk_build": build_line(main_res),
    }
    if "dense_ms_step" in main_res:
        line["dense_baseline"] = {
            "steps_per_s": round(1000.0 / main_res["dense_ms_step"], 2),
            "GBps": round(main_res["dense_bytes"] / (main_res["dense_ms_step"] * 1e-3) / 1e9, 1),
            "speedup_of_compkv": round(main_res["dense_ms_step"] / main_res["ms_step"], 3)}
    if extra is not None:
        we = extra["w"]
        e_score = extra["score_bytes"] / (extra["score_ms"] * 1e-3) / 1e9
        line["also"] = {
            "workload": we.name, "steps_per_s": round(1000.0 / extra["ms_step"], 2),
            "ms_per_step": round(extra["ms_step"], 5), "context_tokens": extra["T"],
            "eager_step_us_p10_p50_p90": extra["step_us_p10_p50_p90"],
            "layers_rotated": extra["R"],
            "step_GBps": round((extra["score_bytes"] + extra["attend_bytes"]) / (extra["ms_step"] * 1e-3) / 1e9, 1),
            "score_kernel_GBps": round(e_score, 1), "score_frac": round(e_score / PEAK_HBM_GBPS, 4),
            "score_avg_launch_us": round(extra["score_ms"] * 1e3, 3),
            "score_traffic": traffic_from_profile(args.also),
            "finish_avg_us": round(extra["finish_ms"] * 1e3, 3),
            "three_call_steps_per_s": round(1000.0 / extra["ms_three_calls"], 2),
            "bulk_build": build_line(extra)}
        if "dense_ms_step" in extra:
            line["also"]["dense_steps_per_s"] = round(1000.0 / extra["dense_ms_step"], 2)
            line["also"]["speedup_of_compkv"] = round(extra["dense_ms_step"] / extra["ms_step"], 3)
    if not args.no_cpu:
        log("timing the CPU oracle")
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""CompKV decode-step benchmark on one MI355X.

One step = one layer's decode step for the workload's batch, through the
fused entry point cknv_decode_step (append the step's token, refresh its
block's summary, score every block, select, attend the kept blocks with Mean
compensation under one normaliser). Inputs are the seeded synthetic workload,
resident in HBM before timing. Steps rotate over R copies of the layer
("layers") at distinct addresses so the per-step working set cannot stay in
the 256 MB Infinity Cache; every timed region starts at the layer touched
least recently.

Prints ONE JSON line. `value` = steps/s from HIP-graph replay of layer sweeps
(HIP events around exactly K timed steps). `roofline` is for the dominant
kernel of the step by average duration, on that kernel's own algorithmic
bytes; `roofline_whole_step` puts all of the step's algorithmic bytes over
the measured step time; `kernels` lists every kernel of the step.
`cpu_baseline` times the fp64 oracle's per-step path on a bounded sample, on
one host thread and on a process pool over the layer's (sequence, KV head)
units (run before the first GPU call). The three-call path (cknv_append,
cknv_score_select, cknv_attend), the dense full-attention kernel and the
other workloads (64K r = 128, the 16-sequence ragged batch) are reported
beside it, and so is the host-offload placement (`host_offload`: the same
step and the dense baseline with the KV cache in pinned host memory, with
the bytes each step moves over the host link).

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
CSRC = "block_sparse_kv_stats_amd/csrc/"
KERNEL_SOURCES = {
    "score_kernel": [CSRC + f for f in ("score.hip", "cknv_internal.h", "summary_core.h")],
    "step_kernel": [CSRC + f for f in ("step.hip", "cknv_internal.h", "attend_core.h",
                                       "select_core.h", "step_config.h")],
}
POOL_MAX = 16  # worker processes for the all-cores CPU baseline (the GPU machine's CPU share)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash(paths) -> str:
    """Hash of a kernel's sources with comments and blank space removed, so
    that a profile stays valid across comment-only edits."""
    import re
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def _per_seq(w, T):
    return [int(T)] * w.S if isinstance(T, (int, float)) else [int(t) for t in T]


def step_bytes(w, T, budget=None):
    """Algorithmic HBM bytes of one fused step over all units, split into the
    streaming half (score_kernel) and the kept blocks' tokens (step_kernel).
    T = tokens of each sequence after the step's append (an int for every
    sequence, or one per sequence).
    score_kernel: k̄ + D̄ + |b| of every block closed before the step and v̄
    of those of them that are not kept; the append (the open block's cached
    BF16 tokens read, the token and its block's summary written);
    step_kernel: BF16 K and V of the kept blocks' tokens."""
    Kb = (budget or w.budget) // 16
    score = attend = 0
    for Ts in _per_seq(w, T):
        NB = math.ceil(Ts / 16)
        closed = (Ts - 1) // 16
        kept = min(Kb, NB)
        kept_closed = kept - (NB - closed)  # the block holding the new token is always kept
        open_n = Ts - 16 * (NB - 1)
        append = (open_n - 1) * 2 * w.d * 2 + 2 * w.d * 2 + (2 * w.d + w.r + 1) * 4
        score += w.H * (closed * (w.d + w.r + 1) * 4 + (closed - kept_closed) * w.d * 4 + append)
        attend += w.H * ((kept - 1) * 16 + open_n) * 2 * w.d * 2
    return score, attend


def host_link_bytes(w, T, budget=None) -> int:
    """Bytes one fused step moves over the host link when the KV cache lives
    in pinned host memory (summaries in HBM): the kept blocks' BF16 K and V
    read by step_kernel, the open block's cached tokens read for its
    summary, and the step's token written."""
    _, attend = step_bytes(w, T, budget)
    extra = 0
    for Ts in _per_seq(w, T):
        open_n = Ts - 16 * (math.ceil(Ts / 16) - 1)
        extra += w.H * ((open_n - 1) * 2 * w.d * 2 + 2 * w.d * 2)
    return attend + extra


def dense_bytes(w, T) -> int:
    return sum(w.H * Ts * 2 * w.d * 2 for Ts in _per_seq(w, T))


def build_bytes(w, T) -> int:
    """Algorithmic HBM bytes of one bulk summary build: the BF16 K and V read
    once, every block's summary written once."""
    return sum(w.H * (Ts * 2 * w.d * 2 + math.ceil(Ts / 16) * (2 * w.d + w.r + 1) * 4)
               for Ts in _per_seq(w, T))


# ---------------------------------------------------------------- CPU baseline
def host_cpu() -> dict:
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"model": model, "cpu_count": os.cpu_count(), "usable": usable}


def _oracle_unit(w, h, n_max, seconds, barrier=None, out=None):
    """Oracle per-step path of unit (0, h) from the workload's context: up to
    n_max steps or `seconds`, one BLAS thread. Returns (steps, seconds)."""
    from threadpoolctl import threadpool_limits

    from block_sparse_kv_stats_amd import synth
    from oracle import compkv as ok

    T0 = w.prefill[0]
    wl = w.replace(steps=max(w.steps, 1), extra_cap=n_max)
    with threadpool_limits(limits=1):
        u = synth.gen_unit(wl, 0, h, ntok=T0 + n_max)
        q = u["q"][0]
        su = ok.StreamingUnit(u["k"], u["v"], T0, w.r, cap_tokens=T0 + n_max)
        if barrier is not None:
            barrier.wait()
        t0 = time.perf_counter()
        n = 0
        while n < n_max:
            su.append(u["k"][T0 + n], u["v"][T0 + n])
            su.step(q, w.budget)
            n += 1
            if time.perf_counter() - t0 > seconds:
                break
        dt = time.perf_counter() - t0
    if out is not None:
        out.put((h, n, dt))
    return n, dt


def _pool_worker(w, h, n, barrier, out):
    os.environ["OMP_NUM_THREADS"] = "1"
    _oracle_unit(w, h, n, float("inf"), barrier, out)


def cpu_baseline(w, seconds: float, pool: bool = True):
    """The fp64 oracle's per-step path (open-block update, score, select,
    attend) on the H (sequence 0, KV head) units of the workload.
    Single thread: each unit in turn for about seconds/(2H) of consecutive
    steps; a layer step costs the sum of the units' mean step times (x S).
    Pool: one process per unit (at most POOL_MAX at once), all released
    together, each running the same number of steps; a layer step costs the
    slowest unit's mean step time. Must run before the process touches the
    GPU (the pool is started with spawn)."""
    n_max = 2500  # per unit: the context grows by at most this many tokens
    share = (seconds / 2 if pool else seconds) / w.H
    per_step, steps, timed = 0.0, 0, 0.0
    unit_step = []
    for h in range(w.H):
        n, dt = _oracle_unit(w, h, n_max, share)
        unit_step.append(dt / n)
        per_step += dt / n
        steps += n
        timed += dt
    per_step *= w.S
    hc = host_cpu()
    rec = {"value": 1.0 / per_step, "unit": "steps/s", "cores": 1, "kind": "oracle",
           "sample": f"{steps} steps over the {w.H} (sequence, KV head) units of sequence 0 of "
                     f"{w.name}, up to {n_max} consecutive steps each from {w.prefill[0]} tokens "
                     f"({timed:.1f} s, fp64 NumPy, 1 thread); a step is the sum of the units' "
                     f"mean step times" + (f", x{w.S} sequences" if w.S > 1 else ""),
           "host_cpu_model": hc["model"], "host_cpu_count": hc["cpu_count"],
           "host_cpus_usable": hc["usable"]}
    if not pool:
        return rec
    import multiprocessing as mp
    workers = max(1, min(w.H, POOL_MAX, hc["usable"] or 1))
    n = max(4, min(n_max, int((seconds / 2) / max(unit_step))))
    ctx = mp.get_context("spawn")
    done = {}
    for h0 in range(0, w.H, workers):
        hs = list(range(h0, min(w.H, h0 + workers)))
        barrier, out = ctx.Barrier(len(hs)), ctx.Queue()
        procs = [ctx.Process(target=_pool_worker, args=(w, h, n, barrier, out)) for h in hs]
        for p in procs:
            p.start()
        for _ in hs:
            h, nn, dt = out.get(timeout=600)
            done[h] = dt / nn
        for p in procs:
            p.join()
    rounds = math.ceil(w.H / workers)
    # units of one round run side by side; rounds follow each other
    batches = [max(done[h] for h in range(h0, min(w.H, h0 + workers)))
               for h0 in range(0, w.H, workers)]
    pool_step = sum(batches) * w.S
    single = rec["value"]
    rec.update({"value": 1.0 / pool_step, "cores": workers,
                "single_thread_steps_per_s": single,
                "sample": f"{n} consecutive steps from {w.prefill[0]} tokens on each of the {w.H} "
                          f"(sequence, KV head) units of sequence 0 of {w.name}, one spawned "
                          f"process per unit ({workers} at a time, {rounds} round(s)), fp64 "
                          f"NumPy with one BLAS thread each, released together; a layer step "
                          f"costs the slowest unit's mean step time" +
                          (f", x{w.S} sequences" if w.S > 1 else "") +
                          f". Single thread: {rec['sample']}"})
    return rec


# ---------------------------------------------------------------- GPU side
class Bench:
    def __init__(self, w, R, appends, stream, budgets=None, kv_on_host=False):
        import numpy as np
        import torch
        from block_sparse_kv_stats_amd import cknv, synth

        self.w, self.R, self.stream = w, R, stream
        budgets = budgets or [w.budget]
        wl = w.replace(steps=max(w.steps, 1), extra_cap=appends + 16)
        log(f"generating {w.name}")
        data = synth.gen_layer(wl, threads=min(16, w.S * w.H))
        pre = list(w.prefill)
        cap_blocks = wl.cap_blocks
        self.max_blocks = math.ceil((max(pre) + appends) / 16)
        shape = cknv.make_shape(w.S, w.H, w.G, w.d, w.r, cap_blocks)
        self.shape = shape

        def dev_bf16(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)

        base = cknv.LayerCache.allocate(shape, kv_on_host=kv_on_host)
        for s, T0 in enumerate(pre):  # each sequence's prefill, later slots zero
            base.k[s, :, :T0].copy_(dev_bf16(data["k"][s, :, :T0]))
            base.v[s, :, :T0].copy_(dev_bf16(data["v"][s, :, :T0]))
        base.seq_len.copy_(torch.tensor(pre, dtype=torch.int32))
        cknv.build_summaries(base, self.max_blocks)
        torch.cuda.synchronize()
        log(f"replicating {R} layers")
        self.layers = [base] + [base.replicate() for _ in range(R - 1)]
        nq = w.steps if w.steps > 1 else 1
        self.q = [torch.from_numpy(data["q"][i % nq]).cuda() for i in range(R)]
        tok = lambda a: np.stack([a[s, :, pre[s]] for s in range(w.S)])
        self.new_k = dev_bf16(tok(data["k"]))
        self.new_v = dev_bf16(tok(data["v"]))
        del data
        U = w.S * w.H
        self.sel = torch.zeros((U, max(budgets) // 16), dtype=torch.int32, device="cuda")
        self.n_sel = torch.zeros((U,), dtype=torch.int32, device="cuda")
        self.out = torch.zeros((w.S, w.H * w.G, w.d), dtype=torch.float32, device="cuda")
        self.lse = torch.zeros((w.S, w.H * w.G), dtype=torch.float32, device="cuda")
        # one workspace per layer, so that a layer's second half can be
        # repeated long after its first (the kernel-duration sweeps)
        self.ws, self.by_budget = {}, {}
        for b in budgets:
            self.ws[b] = [cknv.allocate_workspace(shape, self.max_blocks, b, stream=stream)
                          for _ in self.layers]
            self.by_budget[b] = [cknv.BoundStep(L, self.max_blocks, b, self.ws[b][i], self.sel,
                                                self.n_sel, self.out, self.lse, self.q[i],
                                                self.new_k, self.new_v, stream)
                                 for i, L in enumerate(self.layers)]
        self.bound = self.by_budget[budgets[0]]
        self.cursor = 0  # next layer to touch: the least recently used one
        torch.cuda.synchronize()

    def use_budget(self, b):
        self.bound = self.by_budget[b]

    def order(self, n):
        """Layer indices of the next n steps, starting at the least recently
        used layer; advances the cursor."""
        idx = [(self.cursor + i) % self.R for i in range(n)]
        self.cursor = (self.cursor + n) % self.R
        return idx

    def seq_lens(self):
        return [int(x) for x in self.layers[0].seq_len.cpu().tolist()]


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


def time_graph_steps(torch, timer, stream, bench, steps, which="fused_step"):
    """ms per step over exactly `steps` steps: graphs of whole layer sweeps
    (and one partial sweep), starting at the least recently used layer."""
    R = bench.R
    start = bench.order(steps)[0]
    seq = [bench.bound[(start + i) % R] for i in range(R)]
    full = capture(torch, stream, lambda: [getattr(b, which)() for b in seq])
    rem = steps % R
    part = capture(torch, stream, lambda: [getattr(b, which)() for b in seq[:rem]]) if rem else None
    e0, e1 = timer.event(), timer.event()
    with torch.cuda.stream(stream):
        timer.head_start(5.0 + 0.05 * (steps // R + 1))
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
    order = bench.order(n)
    with torch.cuda.stream(stream):
        timer.head_start(5.0 + 0.08 * n)
        e0.record(stream)
        for i in order:
            bench.bound[i].fused_step()
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def time_step_percentiles(torch, timer, stream, bench, n):
    """Per-step durations (ms) of eager fused steps, each between two HIP
    events on the launch stream (the launches queued behind a spin kernel,
    so host launch latency stays out): p10, median and p90."""
    evs = [(timer.event(), timer.event()) for _ in range(n)]
    order = bench.order(n)
    with torch.cuda.stream(stream):
        timer.head_start(5.0 + 0.08 * n)
        for i, li in enumerate(order):
            evs[i][0].record(stream)
            bench.bound[li].fused_step()
            evs[i][1].record(stream)
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(c) for a, c in evs)
    pick = lambda f: ts[min(len(ts) - 1, int(f * len(ts)))]
    return pick(0.1), pick(0.5), pick(0.9)


def time_score_kernel(torch, timer, stream, bench, sweeps):
    """Average duration (ms) of the streaming score kernel: sweeps of
    back-to-back cknv_decode_score launches over the R layers, each sweep
    between two HIP events on the launch stream (a launch only rewrites the
    workspace, so repeating it leaves the layers unchanged)."""
    evs = [(timer.event(), timer.event()) for _ in range(sweeps)]
    with torch.cuda.stream(stream):
        timer.head_start(5.0 + 0.03 * sweeps * bench.R)
        for i in range(sweeps):
            order = bench.order(bench.R)
            evs[i][0].record(stream)
            for li in order:
                bench.bound[li].decode_score()
            evs[i][1].record(stream)
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(c) / bench.R for a, c in evs)
    return sum(ts) / len(ts)


def time_finish_kernel(torch, timer, stream, bench, sweeps):
    """Average duration (ms) of the step kernel (cknv_decode_finish): one
    cknv_decode_score per layer (each layer has its own workspace), then
    sweeps of back-to-back decode_finish launches over the layers between HIP
    events. A repeated finish gives the same results: it sets seq_len to the
    same value, and its merging part resets the unit's count."""
    for li in bench.order(bench.R):
        bench.bound[li].decode_score()
    evs = [(timer.event(), timer.event()) for _ in range(sweeps)]
    with torch.cuda.stream(stream):
        timer.head_start(5.0 + 0.05 * sweeps * bench.R)
        for i in range(sweeps):
            order = bench.order(bench.R)
            evs[i][0].record(stream)
            for li in order:
                bench.bound[li].decode_finish()
            evs[i][1].record(stream)
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(c) / bench.R for a, c in evs)
    return sum(ts) / len(ts)


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
            for li in bench.order(bench.R):
                cknv.build_summaries(bench.layers[li], bench.max_blocks, stream=stream)
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (sweeps * bench.R)


def layers_for(step_total_bytes, args):
    """Layer copies so that R x per-step bytes exceeds twice the MALL."""
    if args.layers:
        return args.layers
    return max(2, math.ceil(2 * MALL_BYTES / step_total_bytes))


def run_workload(torch, timer, wname, args, stream, full=True, kv_on_host=False):
    """The main workload (full=True: every figure) or an extra one (steps/s,
    kernel durations and the dense baseline). kv_on_host: the KV cache in
    pinned host memory (the host-offload placement)."""
    from block_sparse_kv_stats_amd import synth

    w = synth.WORKLOADS[wname]
    budgets = [512, 1024, 2048] if wname == "ragged16" else [w.budget]
    T1 = [p + 1 for p in w.prefill]
    sb, ab = step_bytes(w, T1, min(budgets))
    R = layers_for(sb + ab, args)
    if wname == "ragged16":
        steps, warm = w.steps, min(args.warmup, 20)   # the workload's 256-step stream per budget
    else:
        steps, warm = args.steps, args.warmup
    n_e = min(steps, 256)
    sweeps = max(2, 64 // R)
    per_budget = (math.ceil(warm / R) + math.ceil(steps / R) + 2 * math.ceil(n_e / R)
                  + 2 * sweeps + math.ceil(max(R, steps // 4) / R) * (2 if full else 1) + 2)
    appends = per_budget * len(budgets) + 4
    bench = Bench(w, R, appends, stream, budgets, kv_on_host=kv_on_host)
    res = {"w": w, "R": R, "steps": steps, "warmup": warm, "by_budget": {}}
    for b in budgets:
        bench.use_budget(b)
        log(f"{wname} budget {b}: {R} layers, {warm} warm-up + {steps} timed steps"
            + (" (KV cache in pinned host memory)" if kv_on_host else ""))
        with torch.cuda.stream(stream):
            for li in bench.order(warm):
                bench.bound[li].fused_step()
        torch.cuda.synchronize()
        r = {"budget": b}
        r["ms_step"] = time_graph_steps(torch, timer, stream, bench, steps)
        T = bench.seq_lens()
        r["T"] = T
        r["score_bytes"], r["attend_bytes"] = step_bytes(w, T, b)
        r["ms_eager"] = time_eager_steps(torch, timer, stream, bench, n_e)
        r["pct"] = time_step_percentiles(torch, timer, stream, bench, n_e)
        r["score_ms"] = time_score_kernel(torch, timer, stream, bench, sweeps)
        r["finish_ms"] = time_finish_kernel(torch, timer, stream, bench, sweeps)
        if full:
            r["ms_three_calls"] = time_graph_steps(torch, timer, stream, bench, max(R, steps // 4),
                                                   which="step")
        if not args.no_dense:
            r["dense_ms"] = time_graph_steps(torch, timer, stream, bench, max(R, steps // 4),
                                             which="dense")
            r["dense_bytes"] = dense_bytes(w, bench.seq_lens())
        res["by_budget"][b] = r
    if full:
        res["build_ms"] = time_build(torch, timer, stream, bench, max(2, 64 // R))
        res["build_bytes"] = build_bytes(w, bench.seq_lens())
    del bench
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------- profiles
PROFILE_COMMANDS = {
    "trace": 'rocprofv3 --kernel-trace --stats -f csv -d $OUT/trace -o trace -- '
             'python3 bench.py --steps 64 --warmup 8 --no-cpu --no-host-offload --also qwen8b_128k',
    "fetch": 'rocprofv3 --pmc FETCH_SIZE -f csv -d $OUT/fetch -o fetch -- '
             'python3 bench.py --steps 8 --warmup 2 --no-cpu --no-dense --no-host-offload --also ""',
    "write": 'rocprofv3 --pmc WRITE_SIZE -f csv -d $OUT/write -o write -- '
             'python3 bench.py --steps 8 --warmup 2 --no-cpu --no-dense --no-host-offload --also ""',
    "fetch128": 'rocprofv3 --pmc FETCH_SIZE -f csv -d $OUT/fetch128 -o fetch128 -- '
                'python3 bench.py --steps 8 --warmup 2 --no-cpu --no-dense --no-host-offload --workload qwen8b_128k --also ""',
    "write128": 'rocprofv3 --pmc WRITE_SIZE -f csv -d $OUT/write128 -o write128 -- '
                'python3 bench.py --steps 8 --warmup 2 --no-cpu --no-dense --no-host-offload --workload qwen8b_128k --also ""',
    "copy_fetch": 'rocprofv3 --pmc FETCH_SIZE -f csv -d $OUT/copy_fetch -o cf -- '
                  'python3 bench.py --copy-probe 268435456',
    "copy_write": 'rocprofv3 --pmc WRITE_SIZE -f csv -d $OUT/copy_write -o cw -- '
                  'python3 bench.py --copy-probe 268435456',
    "summary": 'python3 bench.py --summarize-profiles $OUT',
}
COPY_PROBE_BYTES = 268435456
TRACE_SUMMARY = "kernels_llama8b_32k_qwen8b_128k_trace.md"


def copy_probe(nbytes: int, reps: int):
    """A plain device copy of known size (calibrates the rocprofv3 byte counters)."""
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "reps": reps}))


def device_copy_rate(torch, nbytes: int = 1 << 30, reps: int = 10) -> dict:
    """A plain device-to-device copy (torch's own copy kernel) of nbytes,
    timed with events: what a simple streaming kernel reaches on this GPU
    (read plus write bytes per second), a measured reference beside the
    nominal 8 TB/s."""
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b
    g = 2 * nbytes / (ms * 1e-3) / 1e9
    return {"kernel": "torch copy_ (device to device)", "bytes_read": nbytes, "bytes_written": nbytes,
            "avg_us": round(ms * 1e3, 1), "GBps": round(g, 1), "frac": round(g / PEAK_HBM_GBPS, 4)}


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


def pmc_path(kernel, workload):
    return os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.json")


def summarize_profiles(out_dir):
    """Write profiles/ summaries from the rocprofv3 runs listed in
    PROFILE_COMMANDS (their CSV output under out_dir)."""
    import statistics
    from block_sparse_kv_stats_amd import synth
    prof = os.path.join(ROOT, "profiles")
    os.makedirs(prof, exist_ok=True)
    stats = {}
    for r in _csv_rows(os.path.join(out_dir, "trace"), "kernel_trace.csv"):
        name = r["Kernel_Name"]
        if "cknv" not in name:
            continue
        key = (name.split("(")[0].replace("void ", ""), int(r["Grid_Size_X"]))
        stats.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    if stats:
        lines = ["# Kernel durations: Llama-3.1-8B layer at 32K (budget 512) and Qwen3-8B layer at "
                 "128K (budget 2048)", "",
                 "The fused step (score_kernel + step_kernel), the three-call path (append_kernel, "
                 "score_kernel, select_kernel, attend_kernel, merge_kernel), the dense baseline "
                 "(dense_kernel + merge_kernel) and the bulk build (build_kernel), as bench.py runs them.", "",
                 "Command (from the repository root, OUT = an output directory):", "",
                 "    " + PROFILE_COMMANDS["trace"], "    " + PROFILE_COMMANDS["summary"], "",
                 "rocprofv3 kernel trace of every dispatch of the run (graph replays included),",
                 "grouped by kernel and grid size (threads). Durations in microseconds.", "",
                 "| kernel | grid threads | dispatches | avg us | median us | min us | max us |",
                 "|---|---|---|---|---|---|---|"]
        for (name, grid), d in sorted(stats.items(), key=lambda kv: (kv[0][0], kv[0][1])):
            lines.append(f"| {name} | {grid} | {len(d)} | {statistics.mean(d):.2f} | "
                         f"{statistics.median(d):.2f} | {min(d):.2f} | {max(d):.2f} |")
        with open(os.path.join(prof, TRACE_SUMMARY), "w") as f:
            f.write("\n".join(lines) + "\n")
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
        T = [p + 1 for p in w.prefill]
        sb, ab = step_bytes(w, T)
        for kernel, alg in (("score_kernel", sb), ("step_kernel", ab)):
            fetch = _counter_per_dispatch(os.path.join(out_dir, kf), "FETCH_SIZE", kernel)
            write = _counter_per_dispatch(os.path.join(out_dir, kw), "WRITE_SIZE", kernel)
            if not (fetch and write):
                print(f"missing counter data for {kernel} {wname}", file=sys.stderr)
                continue
            fb = statistics.median(fetch) * 1024.0 * f_cal
            wb = statistics.median(write) * 1024.0 * w_cal
            rec = {"kernel": kernel, "workload": w.name,
                   "source_hash": kernel_source_hash(KERNEL_SOURCES[kernel]),
                   "fetch_KiB_per_dispatch_median": statistics.median(fetch),
                   "write_KiB_per_dispatch_median": statistics.median(write),
                   "dispatches": [len(fetch), len(write)],
                   "copy_probe_bytes": COPY_PROBE_BYTES,
                   "copy_fetch_KiB": statistics.median(cf), "copy_write_KiB": statistics.median(cw),
                   "calibration_fetch": round(f_cal, 4), "calibration_write": round(w_cal, 4),
                   "hbm_read_bytes_per_launch": int(fb), "hbm_write_bytes_per_launch": int(wb),
                   "hbm_bytes_per_launch": int(fb + wb),
                   "algorithmic_bytes_per_launch_first_step": alg,
                   "commands": [PROFILE_COMMANDS[k] for k in (kf, kw, "copy_fetch", "copy_write",
                                                              "summary")]}
            with open(pmc_path(kernel, wname), "w") as f:
                json.dump(rec, f, indent=1)
            print(json.dumps(rec))


def traffic_from_profile(kernel, workload):
    """HBM bytes per launch of `kernel` from a committed rocprofv3 PMC
    summary, if it was taken on the kernel's current source."""
    path = pmc_path(kernel, workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != kernel_source_hash(KERNEL_SOURCES[kernel]):
        return None
    return rec.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------- report
def gbps(nbytes, ms):
    return nbytes / (ms * 1e-3) / 1e9


def kernel_lines(r, wkey):
    ks = [("score_kernel", "cknv_decode_score: the append, its block's summary and the "
                           "streaming pass over the closed blocks' summaries",
           r["score_ms"], r["score_bytes"]),
          ("step_kernel", "cknv_decode_finish: normalisers, selection, exact attention of the "
                          "kept blocks, compensation and the merge of the parts",
           r["finish_ms"], r["attend_bytes"])]
    out = []
    for name, what, ms, nbytes in ks:
        g = gbps(nbytes, ms)
        out.append({"kernel": name, "does": what, "avg_us": round(ms * 1e3, 3),
                    "algorithmic_bytes": nbytes, "GBps": round(g, 1),
                    "frac": round(g / PEAK_HBM_GBPS, 4),
                    "traffic": traffic_from_profile(name, wkey)})
    return out


def roofline(kern):
    dom = max(kern, key=lambda k: k["avg_us"])
    return {"bound": "hbm", "kernel": dom["kernel"], "achieved": dom["GBps"], "peak": PEAK_HBM_GBPS,
            "unit": "GB/s", "frac": dom["frac"], "traffic": dom["traffic"],
            "algorithmic_bytes_per_launch": dom["algorithmic_bytes"], "avg_launch_us": dom["avg_us"],
            "timing": "HIP events on the launch stream around sweeps of back-to-back launches, "
                      "one per layer; the dominant kernel of the step by average duration"}


def whole_step(r):
    nbytes = r["score_bytes"] + r["attend_bytes"]
    g = gbps(nbytes, r["ms_step"])
    return {"achieved": round(g, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(g / PEAK_HBM_GBPS, 4), "algorithmic_bytes_per_step": nbytes,
            "us_per_step": round(r["ms_step"] * 1e3, 3)}


def extra_line(res, wkey):
    out = {"workload": res["w"].name, "layers_rotated": res["R"], "steps": res["steps"]}
    per = []
    for b, r in res["by_budget"].items():
        e = {"budget_tokens": b, "steps_per_s": round(1000.0 / r["ms_step"], 2),
             "us_per_step": round(r["ms_step"] * 1e3, 3),
             "context_tokens": r["T"] if len(r["T"]) > 1 else r["T"][0],
             "eager_step_us_p10_p50_p90": [round(x * 1e3, 2) for x in r["pct"]],
             "roofline_whole_step": whole_step(r), "kernels": kernel_lines(r, wkey)}
        if "ms_three_calls" in r:
            e["three_call_steps_per_s"] = round(1000.0 / r["ms_three_calls"], 2)
        if "dense_ms" in r:
            e["dense_steps_per_s"] = round(1000.0 / r["dense_ms"], 2)
            e["dense_GBps"] = round(gbps(r["dense_bytes"], r["dense_ms"]), 1)
            e["speedup_of_compkv"] = round(r["dense_ms"] / r["ms_step"], 3)
            e["speedup_vs_dense_at_0.7_peak"] = dense_bound_speedup(r)
        per.append(e)
    if len(per) == 1:
        out.update(per[0])
    else:
        out["by_budget"] = per
    if "build_ms" in res:
        out["bulk_build"] = build_line(res)
    return out


def dense_bound_speedup(r):
    """CompKV's speed-up over a dense step that streamed all of K/V at 0.7 of
    the HBM peak (a bound no measured dense kernel reaches): the ratio that
    does not depend on how well the dense baseline is tuned."""
    ideal_ms = r["dense_bytes"] / (0.7 * PEAK_HBM_GBPS * 1e9) * 1e3
    return round(ideal_ms / r["ms_step"], 3)


def host_line(res):
    """The host-offload placement's figures: the fused step and the dense
    baseline with the KV cache in pinned host memory."""
    w = res["w"]
    r = res["by_budget"][w.budget]
    link = host_link_bytes(w, r["T"], w.budget)
    out = {"workload": w.name, "budget_tokens": w.budget,
           "placement": "BF16 K/V in pinned host memory (torch pin_memory, i.e. hipHostMalloc), "
                        "mapped at the same address; summaries, workspace and outputs in HBM",
           "layers_rotated": res["R"], "steps": res["steps"],
           "steps_per_s": round(1000.0 / r["ms_step"], 2), "us_per_step": round(r["ms_step"] * 1e3, 3),
           "host_link_bytes_per_step": link,
           "host_link_GBps": round(gbps(link, r["ms_step"]), 2),
           "eager_step_us_p10_p50_p90": [round(x * 1e3, 2) for x in r["pct"]],
           "kernels_us": {"score_kernel": round(r["score_ms"] * 1e3, 3),
                          "step_kernel": round(r["finish_ms"] * 1e3, 3)}}
    if "dense_ms" in r:
        out["dense_steps_per_s"] = round(1000.0 / r["dense_ms"], 2)
        out["dense_host_link_GBps"] = round(gbps(r["dense_bytes"], r["dense_ms"]), 2)
        out["speedup_of_compkv"] = round(r["dense_ms"] / r["ms_step"], 3)
    return out


def build_line(res):
    g = gbps(res["build_bytes"], res["build_ms"])
    return {"kernel": "build_kernel (cknv_build_summaries)", "avg_us": round(res["build_ms"] * 1e3, 2),
            "algorithmic_bytes": res["build_bytes"], "GBps": round(g, 1),
            "frac": round(g / PEAK_HBM_GBPS, 4)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--workload", default="llama8b_32k")
    ap.add_argument("--also", default="qwen8b_128k,qwen32b_64k,ragged16",
                    help="other workloads reported beside (comma-separated; '' = none)")
    ap.add_argument("--layers", type=int, default=0, help="layer copies to rotate over (0 = auto)")
    ap.add_argument("--cpu-seconds", type=float, default=16.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-host-offload", action="store_true",
                    help="skip the host-offload placement (KV cache in pinned host memory)")
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
    from block_sparse_kv_stats_amd import synth
    if args.workload not in synth.WORKLOADS:
        print(f"unknown workload {args.workload}", file=sys.stderr)
        sys.exit(2)
    cpu = None
    if not args.no_cpu and not args.copy_probe:
        # before anything touches the GPU: the pool's processes are spawned
        log("timing the CPU oracle")
        cpu = cpu_baseline(synth.WORKLOADS[args.workload], args.cpu_seconds)
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

    main_res = run_workload(torch, timer, args.workload, args, stream, full=True)
    extras = [x for x in args.also.split(",") if x and x != args.workload]
    extra_res = {x: run_workload(torch, timer, x, args, stream, full=(x == "qwen8b_128k"))
                 for x in extras}
    copy_ref = device_copy_rate(torch)
    host_res = None
    if not args.no_host_offload:
        host_res = run_workload(torch, timer, args.workload, args, stream, full=False,
                                kv_on_host=True)

    w = main_res["w"]
    r = main_res["by_budget"][w.budget]
    kern = kernel_lines(r, args.workload)
    line = {
        "metric": METRIC,
        "value": round(1000.0 / r["ms_step"], 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": main_res["steps"],
        "warmup": main_res["warmup"],
        "ms_per_step": round(r["ms_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 (bf16 KV, fp32 summaries)",
        "data": "synthetic (seeded generator: block-structured bf16 keys, 1% needles, N(0,1) values)",
        "config": {"workload": w.name, "S": w.S, "H": w.H, "G": w.G, "d": w.d, "r": w.r,
                   "context_tokens": r["T"][0], "budget_tokens": w.budget,
                   "layers_rotated": main_res["R"],
                   "launch": "hipGraph replay of layer sweeps of cknv_decode_step"},
        "roofline": roofline(kern),
        "roofline_whole_step": whole_step(r),
        "kernels": kern,
        "eager_ms_per_step": round(r["ms_eager"], 5),
        "eager_step_us_p10_p50_p90": [round(x * 1e3, 2) for x in r["pct"]],
        "three_call_path": {"steps_per_s": round(1000.0 / r["ms_three_calls"], 2),
                            "calls": "cknv_append + cknv_score_select + cknv_attend"},
        "bulk_build": build_line(main_res),
        "device_copy": copy_ref,
    }
    if "dense_ms" in r:
        line["dense_baseline"] = {
            "steps_per_s": round(1000.0 / r["dense_ms"], 2),
            "GBps": round(gbps(r["dense_bytes"], r["dense_ms"]), 1),
            "frac": round(gbps(r["dense_bytes"], r["dense_ms"]) / PEAK_HBM_GBPS, 4),
            "speedup_of_compkv": round(r["dense_ms"] / r["ms_step"], 3),
            "speedup_vs_dense_at_0.7_peak": dense_bound_speedup(r)}
    if extra_res:
        line["also"] = {x: extra_line(res, x) for x, res in extra_res.items()}
    if host_res is not None:
        line["host_offload"] = host_line(host_res)
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

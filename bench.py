"""Benchmark of the tree-verification step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c4]

A step is one pass of the whole path over one batch of synthetic input:
tree_attn (prefix + tree-masked attention of every node) -> tree_verify ->
kv_commit, enqueued back to back on one stream with no host synchronisation.
Verification and commit run as one pass (tree_verify_commit: greedy = argmax
partials, then one launch that scans each tree and copies its accepted rows;
stochastic = the walk's workgroup copies them); --unfused times the two
separate calls instead.
The default workload is c4, the largest one that fits one GPU: the
long-context 70B-shaped layer (4 requests, 128-node merged trees, 64 query /
8 kv heads of 128, prefix 32768, vocabulary 32000, greedy).  Its attention
is bound by the matrix cores (about 1020 flop per KV byte against a bf16
ridge of about 312), so its roofline is reported against the MFMA peak, with
the KV GB/s beside it.
Inputs are resident in HBM before timing starts; each step reads a different
copy of them (enough copies to exceed twice the 256 MB last-level cache), so
the prefix KV and logits come from HBM, not from cache.

Exactly --steps steps are timed, each between two HIP events on the launch
stream; a short spin kernel ahead of them lets the host enqueue every step
before the first one runs, so the steps run back to back.  The events are
created with hipEventDisableSystemFence: recording an ordinary timing event
releases the caches to system scope, which measured 0.5-3 us per call on
MI355X (c2 attention 17.8 us per call against 15.2 us for 200 calls between
two events; 16.2 us with these events).  A step's kernels
are launched directly (measured on MI355X: a HIP-graph replay per step,
--graph, adds ~7 us of launch gap per replay: c5 109.5 vs 103.6 us per step,
the commit kernel alone 13.9 vs 6.4 us).  ms_per_step is the median step
time, ms_per_step_mean the mean over the same steps.

Prints one JSON line: value = verified tree-node queries per second (B*N per
step at the median step time); roofline = tree_attn's algorithmic work per
launch (flops for c4, KV bytes otherwise) over its average launch time (HIP
events on the launch stream); cpu_baseline = the CPU oracle timed on a
bounded sample of the same workload on all host cores and on one (the
oracle is test infrastructure; it is imported only here, for that leg).
warm_us: the medians of tree_attn and of the whole step on one input copy
run back to back (whatever of it fits stays in L2/MALL); the metric is the
rotated, cold measurement.
sub_workloads (--also, default c3,c5): the same measurement of the
HBM-bound workloads after the main one, compact (value, step and stage
medians, warm medians, roofline), without a CPU leg.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import platform
import subprocess
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
import token_tree_verification_attn_amd as ttv  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16
MALL_BYTES = 256 << 20
METRIC = "tree_attn KV HBM GB/s (% of peak) + verified tree-node queries/sec, 1 GPU"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Inputs:
    """One device copy of a workload's inputs plus preallocated outputs."""

    def __init__(self, d, dev):
        dt = torch.bfloat16 if d["dtype"] == "bf16" else torch.float32
        f = lambda k: torch.from_numpy(np.ascontiguousarray(d[k])).to(dev)
        self.q = f("q").to(dt)
        self.k_cache = f("k_cache").to(dt)
        self.v_cache = f("v_cache").to(dt)
        self.k_tree = f("k_tree").to(dt)
        self.v_tree = f("v_tree").to(dt)
        self.parents, self.tokens, self.cache_len = f("parents"), f("tokens"), f("cache_len")
        self.llm = f("llm")
        self.ssm = f("ssm") if "ssm" in d else None
        B, N, Hq, D = self.q.shape
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty((B, N, Hq), dtype=torch.float32, device=dev)
        self.st = torch.zeros(B, dtype=torch.int32, device=dev)
        self.path = torch.empty((B, N), dtype=torch.int32, device=dev)
        self.plen = torch.empty(B, dtype=torch.int32, device=dev)
        self.outt = torch.empty((B, N), dtype=torch.int32, device=dev)
        self.len_out = torch.empty(B, dtype=torch.int32, device=dev)
        self.src = torch.empty((B, N), dtype=torch.int32, device=dev)

    def nbytes(self):
        return sum(t.numel() * t.element_size() for t in
                   (self.q, self.k_cache, self.v_cache, self.k_tree, self.v_tree, self.llm)
                   + ((self.ssm,) if self.ssm is not None else ()))


class Step:
    def __init__(self, d, copies, dev, fuse=True):
        self.d = d
        self.copies = copies
        self.mode = ttv.GREEDY if d["mode"] == "greedy" else ttv.STOCHASTIC
        c = copies[0]
        B, N, Hq, D = c.q.shape
        dt = c.q.dtype
        self.ws_attn = torch.zeros(max(1, ttv.tree_attn_workspace_size(
            dt, B, N, Hq, d["Hkv"], D, d["Lmax"])), dtype=torch.uint8, device=dev)
        self.ws_ver = torch.empty(max(1, ttv.tree_verify_workspace_size(
            self.mode, B, N, d["V"])), dtype=torch.uint8, device=dev)
        self.fused = fuse  # one pass: verification + commit
        # stochastic draws: the workload's seed, step 0 (every timed step
        # verifies the same batch, so it draws the same uniforms)
        self.seed, self.step = d.get("seed", 0), d.get("step", 0)

    def attn(self, c):
        ttv.tree_attn(c.q, c.k_cache, c.v_cache, c.cache_len, c.k_tree, c.v_tree, c.parents,
                      self.d["Lmax"], scale=self.d["scale"], out=c.out, lse=c.lse,
                      dev_status=c.st, workspace=self.ws_attn)

    def verify(self, c):
        ttv.tree_verify(self.mode, c.parents, c.tokens, c.llm, c.ssm, seed=self.seed,
                        step=self.step, path=c.path, path_len=c.plen, out_tokens=c.outt,
                        dev_status=c.st, workspace=self.ws_ver)

    def commit(self, c):
        # lengths go to a separate array, so repeated steps rewrite the same rows
        ttv.kv_commit(c.k_tree, c.v_tree, c.k_cache, c.v_cache, c.cache_len, c.path, c.plen,
                      self.d["Lmax"], cache_len_out=c.len_out, committed_src=c.src,
                      dev_status=c.st)

    def verify_commit(self, c):
        ttv.tree_verify_commit(self.mode, c.parents, c.tokens, c.llm, c.k_tree, c.v_tree,
                               c.k_cache, c.v_cache, c.cache_len, self.d["Lmax"], ssm=c.ssm,
                               seed=self.seed, step=self.step, cache_len_out=c.len_out,
                               path=c.path, path_len=c.plen, out_tokens=c.outt,
                               committed_src=c.src, dev_status=c.st, workspace=self.ws_ver)


HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000
_hip = None


def hip_runtime():
    """The HIP runtime library (events are created through it directly:
    torch's events take no creation flags)."""
    global _hip
    if _hip is None:
        h = ctypes.CDLL("libamdhip64.so")
        vp, u = ctypes.c_void_p, ctypes.c_uint
        h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), u]
        h.hipEventRecord.argtypes = [vp, vp]
        h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
        h.hipEventDestroy.argtypes = [vp]
        for f in (h.hipEventCreateWithFlags, h.hipEventRecord, h.hipEventElapsedTime,
                  h.hipEventDestroy):
            f.restype = ctypes.c_int
        _hip = h
    return _hip


def hip_check(rc, what):
    if rc != 0:
        raise RuntimeError("%s failed with HIP error %d" % (what, rc))


def timed_steps(fns, n, stream, preroll=0):
    """Run fns[i % len(fns)]() for i = 0..n-1 on `stream`, each between two
    HIP events recorded on that stream; returns the n durations in ms.  A
    spin kernel enqueued first keeps the GPU busy while the host enqueues
    every step, so the steps run back to back as they would in a serving
    loop, not paced by the host.  `preroll` untimed calls of the same
    functions run between the spin and the first event: the spin leaves the
    GPU nearly idle, and its clocks take tens of milliseconds of real work to
    come back to their working level (measured on MI355X: c4 attention 600 us
    per call over 20-step batches, 520 us over 100-step ones, without them)."""
    h = hip_runtime()
    hs = ctypes.c_void_p(stream.cuda_stream)
    ev = []
    try:
        for _ in range(n + 1):
            e = ctypes.c_void_p()
            hip_check(h.hipEventCreateWithFlags(ctypes.byref(e), HIP_EVENT_DISABLE_SYSTEM_FENCE),
                      "hipEventCreateWithFlags")
            ev.append(e)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            torch.cuda._sleep(int(2e7))  # ~10 ms of clock cycles: the queue fills meanwhile
        for i in range(preroll):
            fns[i % len(fns)]()
        hip_check(h.hipEventRecord(ev[0], hs), "hipEventRecord")
        for i in range(n):
            fns[i % len(fns)]()
            hip_check(h.hipEventRecord(ev[i + 1], hs), "hipEventRecord")
        torch.cuda.synchronize()
        out = []
        for i in range(n):
            ms = ctypes.c_float()
            hip_check(h.hipEventElapsedTime(ctypes.byref(ms), ev[i], ev[i + 1]),
                      "hipEventElapsedTime")
            out.append(float(ms.value))
        return out
    finally:
        for e in ev:
            h.hipEventDestroy(e)


def summary(ms):
    a = np.asarray(ms, np.float64)
    return {"median": float(np.median(a)), "mean": float(a.mean()),
            "p10": float(np.percentile(a, 10)), "p90": float(np.percentile(a, 90))}


def capture(fn, dev):
    """Capture fn's launches into a HIP graph (None if capture fails)."""
    try:
        side = torch.cuda.Stream(dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g
    except Exception as e:  # pragma: no cover - reported, then direct launches
        log("graph capture failed (%s); timing direct launches" % e)
        return None


def tree_depths(par):
    depth = np.zeros_like(par)
    for i in range(1, par.shape[1]):
        depth[:, i] = depth[np.arange(par.shape[0]), par[:, i]] + 1
    return depth


def attn_work(d):
    """Algorithmic work of one tree_attn launch: bytes = every prefix and tree
    K/V element read once, sum_b (L_b + N) * Hkv * D * 2 * elt; flops = 4 * D
    per (query row, key it attends to), sum over rows of L_b + depth + 1."""
    elt = 2 if d["dtype"] == "bf16" else 4
    L = d["cache_len"].astype(np.int64)
    N, Hkv, Hq, D = d["N"], d["Hkv"], d["Hq"], d["D"]
    kv_bytes = int(((L + N) * Hkv * D * 2 * elt).sum())
    keys = (L[:, None] + tree_depths(d["parents"]) + 1).astype(np.int64)  # [B, N]
    flops = int(4 * D * Hq * keys.sum())
    return kv_bytes, flops


def source_hash():
    """Hash of the attention kernels' own sources, which a stored counter
    profile belongs to (the host-side entry points may change without
    changing what the kernels read and write)."""
    h = hashlib.sha256()
    for f in ("attn.hip", "attn_mfma.hip", "attn_plan.h", "ttv_common.h"):
        h.update(open(os.path.join(ROOT, "token_tree_verification_attn_amd", "csrc", f),
                      "rb").read())
    return h.hexdigest()[:16]


def stored_traffic(workload):
    """HBM bytes per tree_attn launch from the committed rocprofv3 counter
    summary, or None when there is none or the kernel changed since."""
    f = os.path.join(ROOT, "profiles", "tree_attn_%s_traffic.json" % workload)
    if not os.path.exists(f):
        return None
    rec = json.load(open(f))
    if rec.get("source_hash") != source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def host_cpu():
    """The host's logical CPU count and model name."""
    model = platform.processor() or "unknown"
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for ln in out.splitlines():
            if ln.lower().startswith("model name"):
                model = ln.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    return os.cpu_count() or 1, model


def cpu_step(d, budget_s, oracle):
    """Seconds of one full step of the oracle on the current thread count:
    verification of the whole batch, the commit of request 0 (time x B), and
    attention on a uniform sample of query rows sized to the time budget (all
    rows when they fit, time scaled to all rows), the whole repeated until
    about a quarter of the budget has passed.  Returns (step seconds,
    description of the sample)."""
    B, N, Hq = d["B"], d["N"], d["Hq"]
    rows_all = oracle.all_rows(B, N, Hq)
    rng = np.random.default_rng(0)
    attn = lambda rows: oracle.tree_attn_rows(d["q"], d["k_cache"], d["v_cache"], d["cache_len"],
                                              d["k_tree"], d["v_tree"], d["parents"], d["scale"],
                                              rows)
    probe = min(4 * oracle.max_threads(), len(rows_all))
    t0 = time.perf_counter()
    attn(rows_all[rng.choice(len(rows_all), size=probe, replace=False)])
    per_row = (time.perf_counter() - t0) / probe
    n = int(min(len(rows_all), max(probe, 0.6 * budget_s / per_row)))
    sample = rows_all if n >= len(rows_all) else \
        rows_all[rng.choice(len(rows_all), size=n, replace=False)]
    t_attn = t_verify = t_commit = 0.0
    reps = 0
    start = time.perf_counter()
    while reps == 0 or time.perf_counter() - start < 0.25 * budget_s:
        t0 = time.perf_counter()
        attn(sample)
        t1 = time.perf_counter()
        if d["mode"] == "greedy":
            path, plen, _, _ = oracle.verify_greedy(d["parents"], d["tokens"], d["llm"])
        else:
            path, plen, _, _ = oracle.verify_mss_seeded(d["parents"], d["tokens"], d["llm"],
                                                        d["ssm"], d["seed"], d["step"])
        t2 = time.perf_counter()
        oracle.kv_commit(d["k_tree"][:1], d["v_tree"][:1], d["k_cache"][:1], d["v_cache"][:1],
                         d["cache_len"][:1], path[:1], plen[:1], d["Lmax"])
        t3 = time.perf_counter()
        t_attn += (t1 - t0) * len(rows_all) / len(sample)
        t_verify += t2 - t1
        t_commit += (t3 - t2) * B
        reps += 1
    desc = ("%d step(s): attention on %d of %d query rows (uniform sample, time scaled to all "
            "rows), verify of the whole batch, commit of request 0 (time x B); %.1f s"
            % (reps, len(sample), len(rows_all), time.perf_counter() - start))
    return (t_attn + t_verify + t_commit) / reps, desc


def cpu_baseline(d, budget_s):
    """The CPU oracle on a bounded sample of the same workload, on every host
    core (OpenMP over rows and requests) and on one, as tree-node queries/s of
    one full step."""
    import oracle
    ncpu, model = host_cpu()
    B, N = d["B"], d["N"]
    oracle.set_threads(ncpu)
    threads = oracle.max_threads()
    step_all, desc_all = cpu_step(d, 0.7 * budget_s, oracle)
    oracle.set_threads(1)
    step_one, desc_one = cpu_step(d, 0.3 * budget_s, oracle)
    oracle.set_threads(ncpu)
    return {"value": B * N / step_all, "unit": "tree-node queries/s", "cores": threads,
            "kind": "oracle",
            "sample": "all %d threads: %s; one thread: %s" % (threads, desc_all, desc_one),
            "step_ms": step_all * 1e3, "value_1thread": B * N / step_one,
            "step_ms_1thread": step_one * 1e3, "nproc": ncpu, "cpu_model": model}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c4", choices=sorted(synth.WORKLOADS))
    ap.add_argument("--cpu-budget", type=float, default=16.0,
                    help="seconds of CPU oracle work for the baseline (0 = skip)")
    ap.add_argument("--graph", action="store_true",
                    help="replay each step (and stage) from a HIP graph instead of launching "
                         "its kernels directly")
    ap.add_argument("--warm", action="store_true",
                    help="reuse one input copy (cache-resident) instead of rotating copies")
    ap.add_argument("--unfused", action="store_true",
                    help="verification and commit as two calls instead of one pass")
    ap.add_argument("--also", default="c3,c5",
                    help="comma-separated workloads measured after the main one and reported "
                         "in compact form under sub_workloads ('' = none; no CPU leg)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)
    also = [w for w in args.also.split(",") if w and w != args.workload]
    for w in also:
        if w not in synth.WORKLOADS:
            print("--also: unknown workload %s" % w, file=sys.stderr)
            sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    res, d = measure(args.workload, args, dev)
    if also:
        res["sub_workloads"] = {}
        for w in also:
            torch.cuda.empty_cache()
            sub, _ = measure(w, args, dev)
            r = sub["roofline"]
            res["sub_workloads"][w] = {
                "value": sub["value"], "unit": sub["unit"], "ms_per_step": sub["ms_per_step"],
                "steps": sub["steps"], "config": sub["config"],
                "stage_us_median": {k: (v["median"] if v else None)
                                    for k, v in sub["stage_us"].items()},
                "warm_us": sub["warm_us"],
                "roofline": {k: r[k] for k in ("bound", "achieved", "peak", "unit", "frac",
                                               "traffic", "avg_launch_us")}}
    if args.cpu_budget > 0:
        res["cpu_baseline"] = cpu_baseline(d, args.cpu_budget)
    print(json.dumps(res), flush=True)


def measure(workload, args, dev):
    """One workload: its timed steps and per-entry-point stages, as the JSON
    record (without the CPU leg); returns (record, the workload's arrays)."""
    d = synth.make(workload)
    first = Inputs(d, dev)
    per_copy = first.nbytes()
    ncopies = 1 if args.warm else max(1, min(64, -(-2 * MALL_BYTES // per_copy)))
    copies = [first] + [Inputs(d, dev) for _ in range(ncopies - 1)]
    log("workload %s: %d input copies of %.1f MB" % (workload, ncopies, per_copy / 1e6))
    step = Step(d, copies, dev, fuse=not args.unfused)
    stream = torch.cuda.current_stream(dev)

    def launches(fn):
        """One callable per input copy: fn on that copy, or with --graph a
        replay of its HIP graph (direct launches when capture fails)."""
        out = []
        for c in copies:
            g = capture(lambda c=c: fn(c), dev) if args.graph else None
            out.append(g.replay if g is not None else (lambda c=c: fn(c)))
        return out

    def one_step(c):
        step.attn(c)
        if step.fused:
            step.verify_commit(c)
        else:
            step.verify(c)
            step.commit(c)

    for i in range(args.warmup):
        one_step(copies[i % ncopies])
    torch.cuda.synchronize()
    # untimed calls ahead of every timed batch: ~40 ms of GPU work, from one
    # step timed here (4..128 calls)
    t0 = time.perf_counter()
    one_step(copies[0])
    torch.cuda.synchronize()
    preroll = int(min(128, max(4, math.ceil(0.040 / max(time.perf_counter() - t0, 1e-6)))))
    step_fns = launches(one_step)
    graphed = args.graph and all(getattr(f, "__self__", None) is not None for f in step_fns)
    t_step = summary(timed_steps(step_fns, args.steps, stream, preroll))
    # per-entry-point times over the same rotation, launched the same way
    stage = lambda fn: summary(timed_steps(launches(fn), args.steps, stream, preroll))
    t_attn = stage(step.attn)
    t_verify = stage(step.verify)
    t_commit = stage(step.commit)
    t_fused = stage(step.verify_commit) if step.fused else None
    # warm: one input copy back to back (what of it fits stays in the caches)
    t_warm_attn = summary(timed_steps([lambda: step.attn(copies[0])], args.steps, stream, preroll))
    t_warm_step = summary(timed_steps([lambda: one_step(copies[0])], args.steps, stream, preroll))
    st = torch.stack([c.st for c in copies]).cpu()
    assert int(st.abs().sum()) == 0, "a request was rejected: %s" % st

    B, N = d["B"], d["N"]
    kv_bytes, flops = attn_work(d)
    ms_attn = t_attn["mean"]  # the roofline takes the average launch
    kv_gbs = kv_bytes / (ms_attn * 1e-3) / 1e9
    mfma_bound = workload == "c4"
    if mfma_bound:
        ach = flops / (ms_attn * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": ach, "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": ach / MFMA_BF16_PEAK_TFLOPS}
    else:
        roof = {"bound": "hbm", "achieved": kv_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": kv_gbs / HBM_PEAK_GBS}
    roof["traffic"] = stored_traffic(workload)
    roof["traffic_unit"] = "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, calibrated)"
    roof["kernel"] = "ttv_tree_attn (all kernels of one call)"
    roof["per_launch_algorithmic"] = flops if mfma_bound else kv_bytes
    roof["per_launch_algorithmic_unit"] = "flop" if mfma_bound else "byte"
    roof["avg_launch_us"] = ms_attn * 1e3
    roof["median_launch_us"] = t_attn["median"] * 1e3
    roof["kv_gbs"] = kv_gbs
    roof["kv_frac_of_hbm_peak"] = kv_gbs / HBM_PEAK_GBS

    ms_step = t_step["median"]
    us = lambda t: None if t is None else {k: v * 1e3 for k, v in t.items()}
    res = {
        "metric": METRIC,
        "value": B * N / (ms_step * 1e-3),
        "unit": "tree-node queries/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step,
        "ms_per_step_mean": t_step["mean"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": d["dtype"], "data": "synthetic",
        "config": {"workload": workload, "B": B, "N": N, "Hq": d["Hq"], "Hkv": d["Hkv"],
                   "D": d["D"], "prefix": synth.WORKLOADS[workload].L, "V": d["V"],
                   "verify": d["mode"],
                   "verify_commit": "one pass" if step.fused else "two calls",
                   "input_copies": ncopies,
                   "untimed_calls_before_each_timed_batch": preroll,
                   "launch": "hip graph replay per step" if graphed else "direct kernel launches",
                   "inputs": "rotated, HBM-resident" if ncopies > 1 else
                             ("one copy (warm)" if args.warm else
                              "one copy larger than twice the last-level cache, HBM-resident")},
        "tree_attn_kv_gbs": kv_gbs,
        "tree_attn_kv_frac_of_hbm_peak": kv_gbs / HBM_PEAK_GBS,
        "stage_us": {"tree_attn": us(t_attn), "tree_verify": us(t_verify),
                     "kv_commit": us(t_commit), "tree_verify_commit": us(t_fused)},
        "step_us": us(t_step),
        "warm_us": {"tree_attn_median": t_warm_attn["median"] * 1e3,
                    "step_median": t_warm_step["median"] * 1e3,
                    "inputs": "one copy, back to back (the metric is the rotated, cold one)"},
        "roofline": roof,
    }
    return res, d


if __name__ == "__main__":
    main()

"""rocprofv3 evidence for bench.py's roofline line (summaries to copy into profiles/).

    python bench_profile.py --workload c2

Runs, each as its own child process under rocprofv3 (the program follows
`--` directly; this script itself never touches the GPU):
  1. --kernel-trace --stats of `bench.py --workload W --steps S` -> per-kernel
     average durations (the tree_attn entry point = its kernels' sum);
  2. --pmc FETCH_SIZE, then --pmc WRITE_SIZE of the same bench (direct launches),
     one counter group per run -> KiB per dispatch of every tree_attn kernel;
  3. the same two counters on a plain device copy of known size (`--copy-ref`
     mode of this script), whose ratio to the true bytes calibrates them;
  4. one --pmc run of SQ counters plus GRBM_GUI_ACTIVE on the same bench ->
     matrix-core busy fraction and instruction mix of the attention kernels.
Writes tree_attn_W_kernels.md (durations, with the command),
tree_attn_W_traffic.json + .md (HBM bytes per tree_attn launch = calibrated
FETCH + WRITE, tagged with the kernel sources' hash; bench.py reports it only
while that hash matches) and tree_attn_W_counters.md to
gpurun_out/profile_W/summary/ -- the summaries that are kept are copied from
there into profiles/.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import shutil
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 256 << 20
CUS, SIMDS_PER_CU, XCDS = 256, 4, 8
# one pass: at most 8 SQ counters and 2 GRBM counters per run
SQ_COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES", "SQ_WAVE_CYCLES", "SQ_INSTS_MFMA",
               "SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_WAIT_INST_LDS", "SQ_LDS_BANK_CONFLICT"]


def copy_ref():
    import torch
    a = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()


def rocprof(outdir, args, prog, timeout):
    if os.path.exists(outdir):
        shutil.rmtree(outdir)
    cmd = ["rocprofv3"] + args + ["--output-format", "csv", "-d", outdir, "-o", "run", "--"] + prog
    t0 = time.time()
    res = subprocess.run(["timeout", "-s", "KILL", str(timeout)] + cmd, cwd="/tmp",
                         env=dict(os.environ, TMPDIR="/tmp"), capture_output=True, text=True)
    files = glob.glob(os.path.join(outdir, "**", "*.csv"), recursive=True)
    # rocprofv3 may end with a signal after writing complete results
    if not files:
        sys.stderr.write(res.stdout[-3000:] + res.stderr[-3000:])
        raise SystemExit("rocprofv3 produced no results (rc %d)" % res.returncode)
    print("  %.1f s: %s" % (time.time() - t0, " ".join(cmd)), flush=True)
    # the checkout's own path differs from machine to machine
    return {os.path.basename(f): f for f in files}, " ".join(cmd).replace(ROOT, "<repo>")


def counter_kib(files, counter, match):
    """Average per-dispatch value of `counter` over dispatches whose kernel
    name contains any of `match`, grouped by kernel."""
    f = [v for k, v in files.items() if k.endswith("counter_collection.csv")][0]
    per = {}
    for r in csv.DictReader(open(f)):
        if r["Counter_Name"] != counter or not any(m in r["Kernel_Name"] for m in match):
            continue
        per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in per.items()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="c2")
    # bench.py's own defaults, so that the traced average covers the same
    # number of launches as the live measurement it is compared with
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--copy-ref", action="store_true", help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.copy_ref:
        copy_ref()
        return
    sys.path.insert(0, ROOT)
    import bench
    w = args.workload
    out = os.path.join(ROOT, "gpurun_out", "profile_" + w)
    dest = os.path.join(out, "summary")
    os.makedirs(dest, exist_ok=True)
    bench_cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", w, "--steps",
                 str(args.steps), "--warmup", str(args.warmup), "--cpu-budget", "0", "--also", ""]

    # 1. kernel durations
    files, cmd_trace = rocprof(os.path.join(out, "trace"), ["--kernel-trace", "--stats"],
                               bench_cmd, 300)
    stats = list(csv.DictReader(open(files["run_kernel_stats.csv"])))
    rows = [(r["Name"], int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
             float(r["MaxNs"]) / 1e3) for r in stats if "ttv::" in r["Name"]]
    attn = [r for r in rows if "attn" in r[0]]
    with open(os.path.join(dest, "tree_attn_%s_kernels.md" % w), "w") as fh:
        fh.write("# Kernel durations, workload %s (rocprofv3 --kernel-trace --stats)\n\n" % w)
        fh.write("Command (run from /tmp with TMPDIR=/tmp):\n\n    %s\n\n" % cmd_trace)
        fh.write("| kernel | calls | avg us | min us | max us |\n|---|---|---|---|---|\n")
        for r in rows:
            fh.write("| `%s` | %d | %.2f | %.2f | %.2f |\n" % r)
        fh.write("\nOne ttv_tree_attn call = %s: %.2f us on average.\n"
                 % (" + ".join("`%s`" % r[0].split("(")[0] for r in attn),
                    sum(r[2] for r in attn)))

    # 2./3. HBM traffic
    tr = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        f, c = rocprof(os.path.join(out, ctr.lower()), ["--pmc", ctr], bench_cmd, 120)
        tr[ctr] = (counter_kib(f, ctr, ["attn_mfma2", "attn_fma", "attn_combine"]), c)
        f, c = rocprof(os.path.join(out, "copy_" + ctr.lower()), ["--pmc", ctr],
                       [sys.executable, os.path.abspath(__file__), "--copy-ref"], 120)
        ref = counter_kib(f, ctr, ["copy", "elementwise"])
        ref_kib = max(ref.values())  # the 256 MiB copy dispatch
        tr[ctr + "_ref"] = (ref_kib, c)
    fetch_factor = (COPY_BYTES / 1024) / tr["FETCH_SIZE_ref"][0]
    write_factor = (COPY_BYTES / 1024) / tr["WRITE_SIZE_ref"][0]
    fetch_kib = sum(tr["FETCH_SIZE"][0].values())
    write_kib = sum(tr["WRITE_SIZE"][0].values())
    hbm = fetch_kib * fetch_factor * 1024 + write_kib * write_factor * 1024
    import synth
    d = synth.make(w, with_verify=False)
    kv_bytes, flops = bench.attn_work(d)
    rec = {"workload": w, "source_hash": bench.source_hash(),
           "fetch_kib_per_launch": fetch_kib, "write_kib_per_launch": write_kib,
           "fetch_factor": fetch_factor, "write_factor": write_factor,
           "hbm_bytes_per_launch": hbm, "algorithmic_kv_bytes": kv_bytes,
           "per_kernel_fetch_kib": tr["FETCH_SIZE"][0], "per_kernel_write_kib": tr["WRITE_SIZE"][0],
           "commands": [tr[k][1] for k in ("FETCH_SIZE", "WRITE_SIZE", "FETCH_SIZE_ref",
                                            "WRITE_SIZE_ref")]}
    json.dump(rec, open(os.path.join(dest, "tree_attn_%s_traffic.json" % w), "w"), indent=1)
    with open(os.path.join(dest, "tree_attn_%s_traffic.md" % w), "w") as fh:
        fh.write("# HBM traffic of one ttv_tree_attn call, workload %s\n\n" % w)
        fh.write("FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each from its own rocprofv3 run, "
                 "summed over the call's kernels and scaled by what the same counter reads for "
                 "a plain %d MiB device copy.\n\n" % (COPY_BYTES >> 20))
        for k in ("FETCH_SIZE", "WRITE_SIZE"):
            for name, v in tr[k][0].items():
                fh.write("- %s `%s`: %.1f KiB\n" % (k, name.split("(")[0], v))
        fh.write("- copy reference: FETCH_SIZE %.1f KiB, WRITE_SIZE %.1f KiB for %d KiB moved "
                 "-> factors %.3f, %.3f\n" % (tr["FETCH_SIZE_ref"][0], tr["WRITE_SIZE_ref"][0],
                                               COPY_BYTES // 1024, fetch_factor, write_factor))
        fh.write("- HBM bytes per call: %.0f (algorithmic KV bytes %d, ratio %.3f)\n"
                 % (hbm, kv_bytes, hbm / kv_bytes))
        fh.write("\nCommands (run from /tmp with TMPDIR=/tmp):\n\n")
        for c in rec["commands"]:
            fh.write("    %s\n" % c)
    # 4. matrix-core busy fraction and instruction mix
    ctrs = SQ_COUNTERS + ["GRBM_GUI_ACTIVE"]
    f, c_sq = rocprof(os.path.join(out, "sq"), ["--pmc"] + ctrs, bench_cmd, 120)
    per = {k: counter_kib(f, k, ["attn_mfma2", "attn_fma"]) for k in ctrs}
    with open(os.path.join(dest, "tree_attn_%s_counters.md" % w), "w") as fh:
        fh.write("# SQ counters of the attention kernel, workload %s\n\n" % w)
        fh.write("One rocprofv3 --pmc run (averages per dispatch):\n\n    %s\n\n" % c_sq)
        fh.write("SQ_VALU_MFMA_BUSY_CYCLES sums the SIMDs' matrix-core busy cycles (16 per "
                 "v_mfma_f32_16x16x32_bf16) and GRBM_GUI_ACTIVE the %d XCDs' active cycles, so "
                 "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / %d x %d CUs x %d "
                 "SIMDs); VALU issue = 4 cycles per SQ_INSTS_VALU (wave64 on a 16-lane SIMD) over "
                 "the same SIMD-cycles.\n\n" % (XCDS, XCDS, CUS, SIMDS_PER_CU))
        fh.write("| kernel | MFMA busy | VALU issue | MFMA instr | VALU instr | LDS instr "
                 "| LDS wait / wave cycles | LDS bank conflicts | active cycles per XCD |\n"
                 "|---|---|---|---|---|---|---|---|---|\n")
        for name in per["SQ_INSTS_MFMA"]:
            g = {k: per[k].get(name, float("nan")) for k in ctrs}
            simd_cycles = g["GRBM_GUI_ACTIVE"] / XCDS * CUS * SIMDS_PER_CU
            fh.write("| `%s` | %.1f%% | %.1f%% | %.3g | %.3g | %.3g | %.1f%% | %.3g | %.3g |\n" % (
                name.split("(")[0], 100 * g["SQ_VALU_MFMA_BUSY_CYCLES"] / simd_cycles,
                100 * 4 * g["SQ_INSTS_VALU"] / simd_cycles, g["SQ_INSTS_MFMA"],
                g["SQ_INSTS_VALU"], g["SQ_INSTS_LDS"],
                100 * g["SQ_WAIT_INST_LDS"] / max(g["SQ_WAVE_CYCLES"], 1),
                g["SQ_LDS_BANK_CONFLICT"], g["GRBM_GUI_ACTIVE"] / XCDS))
    print(json.dumps({k: rec[k] for k in ("workload", "hbm_bytes_per_launch",
                                          "algorithmic_kv_bytes", "fetch_factor")}))


if __name__ == "__main__":
    main()

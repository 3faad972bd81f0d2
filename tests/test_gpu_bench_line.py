"""The JSON lines of short bench.py runs (the default long-context workload
and the stochastic one, with the one-pass verification + commit): one line on
stdout with the keys and units the measurement contract fixes, value = B*N
tree-node queries per step at the median step time, exactly the steps asked
for, a roofline for tree_attn (matrix-core peak for the long-context
workload, HBM peak otherwise), and the oracle's CPU baseline on all host
cores and on one."""
import json
import os
import subprocess
import sys

import pytest

from gpu_case import announce

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    announce("bench.py " + " ".join(args))
    res = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py")] + list(args),
                         capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-2000:]
    lines = [ln for ln in res.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1
    assert d["higher_is_better"] is True and d["vs_baseline"] is None
    assert d["dtype"] == "bf16" and d["data"] == "synthetic"
    c = d["config"]
    assert c["verify_commit"] == "one pass"
    assert d["value"] == pytest.approx(c["B"] * c["N"] / (d["ms_per_step"] * 1e-3), rel=1e-6)
    r = d["roofline"]
    assert 0 < r["frac"] < 1 and r["frac"] == pytest.approx(r["achieved"] / r["peak"])
    assert r["traffic"] is None or r["traffic"] > 0
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1
    assert cb["value_1thread"] > 0 and cb["nproc"] >= 1 and cb["cpu_model"]
    assert cb["unit"] == d["unit"] and isinstance(cb["sample"], str)
    return d


@pytest.mark.timeout(280)  # three workloads' inputs are built and measured
def test_default_bench_line():
    """The default line: the long-context workload, exactly the steps asked
    for, its roofline against the bf16 matrix-core peak with the KV GB/s
    beside it."""
    d = run_bench("--steps", "4", "--warmup", "2", "--cpu-budget", "0.5")
    assert d["steps"] == 4 and d["warmup"] == 2
    assert d["config"]["workload"] == "c4" and d["config"]["verify"] == "greedy"
    assert d["ms_per_step_mean"] > 0 and d["step_us"]["p10"] <= d["step_us"]["p90"]
    r = d["roofline"]
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2500.0
    assert r["per_launch_algorithmic_unit"] == "flop" and 0 < r["kv_frac_of_hbm_peak"] < 1
    # warm medians beside the cold metric
    assert d["warm_us"]["tree_attn_median"] > 0 and d["warm_us"]["step_median"] > 0
    # the HBM-bound workloads ride along in compact form
    assert sorted(d["sub_workloads"]) == ["c3", "c5"]
    for w, sub in d["sub_workloads"].items():
        assert sub["config"]["workload"] == w and sub["steps"] == 4
        c = sub["config"]
        assert sub["value"] == pytest.approx(c["B"] * c["N"] / (sub["ms_per_step"] * 1e-3), rel=1e-6)
        rs = sub["roofline"]
        assert rs["bound"] == "hbm" and 0 < rs["frac"] < 1 and rs["peak"] == 8000.0
        assert sub["warm_us"]["tree_attn_median"] > 0


def test_stochastic_bench_line():
    d = run_bench("--workload", "c5", "--steps", "3", "--warmup", "1", "--cpu-budget", "0.5",
                  "--also", "")
    assert "sub_workloads" not in d
    assert d["steps"] == 3 and d["config"]["workload"] == "c5"
    assert d["config"]["verify"] == "stochastic"
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0


@pytest.mark.parametrize("op", ["expand", "merge", "probs"])
def test_construction_bench_lines(op):
    """bench_expand.py's three operations each print one JSON line; the
    HBM-bound ones carry a roofline against the 8 TB/s peak."""
    announce("bench_expand.py --op %s --steps 8 --warmup 2" % op)
    res = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench_expand.py"), "--op", op,
                          "--steps", "8", "--warmup", "2", "--cpu-budget", "0.3"],
                         capture_output=True, text=True, timeout=110, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-2000:]
    lines = [ln for ln in res.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    assert d["value"] > 0 and d["n_gpus"] == 1 and d["ms_per_step"] > 0
    assert d["config"]["workload"] == op
    if op == "merge":
        assert d["roofline"] is None
    else:
        r = d["roofline"]
        assert r["bound"] == "hbm" and r["peak"] == 8000.0 and 0 < r["frac"] < 1
    if op == "expand":
        assert d["cpu_baseline"]["kind"] == "oracle" and d["cpu_baseline"]["value"] > 0

"""The JSON line of a short default bench.py run (the default workload, the
one-pass verification + commit): one line on stdout with the keys and units
the measurement contract fixes, value = B*N tree-node queries per step over
the measured step time, a roofline for tree_attn against the HBM peak, and
the oracle's CPU baseline."""
import json
import os
import subprocess
import sys

import pytest

from gpu_case import announce

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_default_bench_line():
    announce("bench.py --steps 4 --warmup 2 --cpu-budget 0.5")
    res = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "4",
                          "--warmup", "2", "--cpu-budget", "0.5"],
                         capture_output=True, text=True, timeout=110, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-2000:]
    lines = [ln for ln in res.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["warmup"] == 2 and d["steps"] >= 4
    assert d["higher_is_better"] is True and d["vs_baseline"] is None
    assert d["dtype"] == "bf16" and d["data"] == "synthetic"
    c = d["config"]
    assert c["workload"] == "c2" and c["verify_commit"] == "one pass"
    assert d["value"] == pytest.approx(c["B"] * c["N"] / (d["ms_per_step"] * 1e-3), rel=1e-6)
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert 0 < r["frac"] < 1 and r["frac"] == pytest.approx(r["achieved"] / r["peak"])
    assert r["traffic"] is None or r["traffic"] > r["per_launch_algorithmic"] * 0.5
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1
    assert cb["unit"] == d["unit"] and isinstance(cb["sample"], str)


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

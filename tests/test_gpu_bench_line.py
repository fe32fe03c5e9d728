"""The benchmark's one-line JSON record on a small run: the keys and types the
measurement contract names (throughput, roofline of the dominant call, the CPU
oracle baseline)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(300)
def test_bench_prints_one_complete_line():
    cmd = [sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--config", "c1", "--only", "--steps", "5",
           "--warmup", "2", "--cpu-seconds", "1"]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-4000:]
    lines = [ln for ln in res.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, res.stdout[-2000:]
    r = json.loads(lines[0])
    for k, t in (("metric", str), ("value", float), ("unit", str), ("n_gpus", int), ("steps", int),
                 ("warmup", int), ("ms_per_step", float), ("higher_is_better", bool), ("scaling", str),
                 ("dtype", str), ("data", str), ("config", dict), ("roofline", dict), ("cpu_baseline", dict)):
        assert isinstance(r[k], t), (k, r.get(k))
    assert r["n_gpus"] == 1 and r["steps"] == 5 and r["warmup"] == 2 and r["value"] > 0
    assert r["vs_baseline"] is None and r["higher_is_better"] is True
    assert r["config"]["workload"].startswith("c1:")
    roof = r["roofline"]
    assert roof["bound"] in ("hbm", "mfma") and roof["unit"] in ("GB/s", "TFLOP/s")
    assert roof["peak"] > 0 and abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert "traffic" in roof
    cb = r["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
    # the step's value is nodes per second of whole steps
    nodes = r["config"]["batch"] * r["config"]["draft_nodes"]
    assert abs(r["value"] - nodes / (r["ms_per_step"] / 1e3)) / r["value"] < 1e-3

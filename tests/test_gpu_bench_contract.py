"""bench.py's output contract on a GPU: one JSON line with the fields a
reader of the benchmark relies on, the roofline object for the dominant
kernel and the CPU oracle leg (a short run of the default workload)."""
import json
import os
import subprocess
import sys

import pytest

from tests.gpu_util import device

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_line():
    device()
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "2",
                        "--cold-launches", "2"], cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key, kind in (("metric", str), ("value", float), ("unit", str), ("n_gpus", int), ("steps", int),
                      ("warmup", int), ("ms_per_step", float), ("higher_is_better", bool), ("scaling", str),
                      ("dtype", str), ("data", str), ("config", dict), ("roofline", dict),
                      ("cpu_baseline", dict)):
        assert isinstance(d[key], kind), key
    assert "vs_baseline" in d
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 2 and d["value"] > 0
    assert "workload" in d["config"]
    roof = d["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert roof["achieved"] > 0 and abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert "traffic" in roof
    if roof["traffic"] is not None:
        assert "traffic_source" in roof
    # the other workloads of the hot path, measured by the same run
    assert set(d["configs"]) == {"square16384_plain", "moe16640", "moe16640_both", "kgroups", "experts16"}
    for name, e in d["configs"].items():
        assert e["kernel_us"] > 0 and 0 < e["frac"] < 1 and e["cold_us_median"] > 0, name
        # kernel_us is rounded to 0.01 us: compare relatively
        assert abs(e["achieved"] / (e["algorithmic_bytes"] / (e["kernel_us"] * 1e3)) - 1) < 1e-3, name
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["cores"] >= 1 and cpu["value"] > 0 and cpu["matches_gpu"] is True

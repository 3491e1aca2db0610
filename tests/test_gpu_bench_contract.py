"""The bench line's contract: one JSON line with the required keys, run as the
driver runs it (a child process), on the tiny workload so that it is quick."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_line_keys():
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny_fp32", "--steps", "3",
           "--warmup", "1", "--no-ceilings"]
    print("case bench contract", flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1
    j = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline", "stages_roofline"):
        assert key in j, key
    assert j["n_gpus"] == 1 and j["steps"] == 3 and j["warmup"] == 1
    assert j["value"] > 0 and j["ms_per_step"] > 0 and j["higher_is_better"] is True
    assert j["config"]["workload"] == "tiny_fp32" and j["dtype"] == "f32" and j["data"] == "synthetic"
    roof = j["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in roof, key
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"], abs=1e-3)
    cpu = j["cpu_baseline"]
    for key in ("value", "unit", "cores", "kind", "sample"):
        assert key in cpu, key
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1
    assert set(j["stages_roofline"]) <= {"gate", "topk", "dispatch", "fc1", "fc2", "combine"}

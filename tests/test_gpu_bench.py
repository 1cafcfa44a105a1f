"""bench.py end to end on the GPU, on the smallest workload (the residual block,
c1): the JSON line carries the fields the measurement contract names, and the
per-op profile (--per-op) covers every op of the plan with totals that add up
to the line's per-kernel times."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

from helpers import say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_line_and_per_op_profile(tmp_path):
    say("bench.py --workload c1 --steps 3 --per-op")
    ops_file = tmp_path / "ops.jsonl"
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "c1", "--steps", "3",
                        "--warmup", "1", "--videos", "0", "--no-cpu-baseline", "--per-op", str(ops_file)],
                       capture_output=True, text=True, timeout=280)
    assert r.returncode == 0, r.stderr[-3000:]
    line = json.loads(r.stdout.strip().splitlines()[-1])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "kernels"):
        assert key in line, key
    assert line["n_gpus"] == 1 and line["steps"] == 3 and line["value"] > 0
    roof = line["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in roof, key
    assert 0 < roof["frac"] < 1 and abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    rows = [json.loads(x) for x in open(ops_file)]
    # the residual block x + conv2(act2(conv1(act1(x)))): act1 as a norm op of
    # its own, act2 fused into conv1, the residual added by conv2
    assert [x["name"] for x in rows if x["part"] == "main"] == ["rb.act1", "rb.conv1", "rb.conv2"]
    assert all(x["launches"] == 3 and x["ms_per_launch"] > 0 for x in rows)
    per_kernel = {}
    for x in rows:
        per_kernel[x["kernel"]] = per_kernel.get(x["kernel"], 0.0) + x["ms_per_launch"] * x["launches"]
    assert set(per_kernel) == set(line["kernels"])
    for k, ms in per_kernel.items():
        assert abs(ms - line["kernels"][k]["ms"]) <= 0.01 * line["kernels"][k]["ms"] + 1e-3, k

"""bench.py end to end on a small workload: one JSON line with the fields
its consumers read, figures consistent with one another, and the oracle
baseline run on the same inputs."""

import json
import os
import subprocess
import sys

import pytest
import torch

from tests._gpu_util import say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


@pytest.mark.parametrize("args", [["--workload", "tiny_f32", "--window", "5", "--no-side"],
                                  ["--workload", "swa_mtp_bf16", "--flush", "--no-cpu-baseline",
                                   "--no-side"]])
def test_bench_line(args):
    say(f"[case] bench {' '.join(args)}")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "4",
                        "--warmup", "1", *args], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    res = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline"):
        assert key in res, key
    assert res["n_gpus"] == 1 and res["steps"] == 4 and res["warmup"] == 1
    assert res["value"] > 0 and res["higher_is_better"] is False
    assert abs(res["ms_per_step"] * 1e3 - res["value"]) < 1e-6 * max(1.0, res["value"]) + 0.01
    assert res["config"]["workload"] == args[1]
    roof = res["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert roof["traffic"] is None or roof["traffic"] > 0
    if "--no-cpu-baseline" in args:
        assert "cpu_baseline" not in res
    else:
        cb = res["cpu_baseline"]
        assert cb["kind"] == "oracle" and cb["cores"] >= 1 and cb["value"] > 0
        assert cb["parity_max_abs"] < 1e-4          # fp32 workload: the fp32 bar
        assert cb["cpu_model"] and "threads" in cb["sample"]
    pc = res["per_call"]
    assert pc["reps"] >= 50 and pc["p10"] <= pc["median"] <= pc["p90"]
    for key in ("copy_ceiling", "read_ceiling"):
        ce = res[key]
        assert ce["bytes"] > 0 and ce["us"] > 0 and 0 < ce["frac"] <= 1.05, (key, ce)
        assert abs(ce["gbps"] - ce["bytes"] / ce["us"] / 1e3) <= 0.1 + 1e-3 * ce["gbps"], (key, ce)
    assert res["read_ceiling"]["kernel_share"] > 0

"""The bench's output contract on the GPU: one JSON line with the metric, the
whole-job throughput, the roofline of the dominant kernel (its HBM traffic
from the committed counters) and the oracle's CPU rate, for a short run."""

import json
import os
import subprocess
import sys

import pytest
import torch

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_line():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3",
                        "--warmup", "1", "--no-backward", "--no-layer", "--no-c4", "--cpu-rows",
                        "32"],
                       capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["unit"] == "tokens/s" and d["higher_is_better"] is True
    assert d["dtype"] == "bf16" and d["data"] == "synthetic"
    assert d["config"]["workload"] == "block_bf16_64x64x64" and d["config"]["tokens"] == 262144
    # throughput is tokens over the measured step time
    assert abs(d["value"] - 262144 / (d["ms_per_step"] * 1e-3)) <= 1e-6 * d["value"]
    rf = d["roofline"]
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and rf["peak"] == 2500.0
    assert 0.0 < rf["frac"] < 1.0 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-9
    # HBM traffic from the committed counters, null when they belong to
    # another version of the kernel
    assert rf["traffic"] is None or rf["traffic"] > 1e9
    assert d["hbm_copy_probe"]["gbs"] > 1000
    assert d["ms_per_step"] > 0 and d["ms_per_step_mean"] > 0
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["unit"] == "tokens/s" and cb["value"] > 0
    assert cb["cores"] >= 1 and "32 of 262144" in cb["sample"]
    assert cb["cores"] <= cb["affinity_cores"] and cb["cpu_model"]

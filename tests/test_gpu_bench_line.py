"""bench.py's one-line JSON contract, checked on the GPU for the headline
workload (graph replay and host launches) and for the RMSNorm path."""
import json
import os
import subprocess
import sys

import pytest

from gpu_helpers import require_gpu

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _run(*args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                       timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    return json.loads(lines[0])


@pytest.mark.parametrize("graph", [True, False], ids=["graph", "host-launch"])
def test_headline_line(graph):
    args = ["--steps", "50", "--warmup", "5", "--no-cpu-baseline"] + ([] if graph else ["--no-graph"])
    d = _run(*args)
    assert d["metric"].startswith("GEMM TFLOP/s") and d["unit"] == "TFLOP/s"
    assert d["n_gpus"] == 1 and d["steps"] == 50 and d["warmup"] == 5
    assert d["higher_is_better"] is True and d["scaling"] == "weak" and d["vs_baseline"] is None
    assert d["dtype"] == "bf16" and d["data"].startswith("synthetic")
    assert d["config"]["M"] == 512 and d["config"]["N"] == 5632 and d["config"]["K"] == 2048
    assert "workload" in d["config"] and "model" not in d["config"]
    assert d["value"] > 0 and d["ms_per_step"] > 0
    # value is the wall-clock rate over the timed steps
    flop = 2 * 512 * 5632 * 2048
    assert abs(d["value"] - flop / (d["ms_per_step"] * 1e-3) / 1e12) <= 0.01 * d["value"]
    rl = d["roofline"]
    assert rl["bound"] == "mfma" and rl["unit"] == "TFLOP/s" and rl["peak"] == pytest.approx(2516.6)
    assert 0 < rl["frac"] < 1 and rl["frac"] == pytest.approx(rl["achieved"] / rl["peak"], rel=1e-3)
    # the kernel's own duration (HIP events on its stream) cannot exceed the wall-clock step
    assert rl["achieved"] >= 0.9 * d["value"]
    assert rl["traffic"] is None or rl["traffic"] > rl["algorithmic_bytes"] * 0.9
    assert "cpu_baseline" not in d


def test_rms_norm_line():
    d = _run("--workload", "rmsnorm_f32_65536x2048", "--steps", "20", "--warmup", "3", "--no-cpu-baseline")
    assert d["unit"] == "GB/s" and d["dtype"] == "f32" and d["value"] > 0
    rl = d["roofline"]
    assert rl["bound"] == "hbm" and rl["unit"] == "GB/s" and rl["peak"] == 8000
    assert 0 < rl["frac"] < 1

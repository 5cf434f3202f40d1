"""CPU tests of bench.py's host-side logic (nothing here touches a GPU)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from tiled_dense_gemm_mkl_amd import workloads  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_source_hashes_cover_the_device_code():
    h1 = bench.source_hash()
    h2 = bench.source_hash(bench.RMS_KERNEL_SOURCES)
    assert len(h1) == len(h2) == 16 and h1 != h2
    for rel in bench.KERNEL_SOURCES + bench.RMS_KERNEL_SOURCES:
        assert os.path.exists(os.path.join(ROOT, rel)), rel


def test_stored_traffic_only_for_matching_code_and_kernel():
    """profiles/hbm_traffic.json entries are reported only while the device
    code hash and the kernel configuration both match."""
    with open(os.path.join(ROOT, "profiles", "hbm_traffic.json")) as f:
        table = json.load(f)
    for key, e in table["workloads"].items():
        sources = bench.RMS_KERNEL_SOURCES if key.startswith("rmsnorm_") else None
        got = bench.measured_traffic(key, e["kernel"], sources)
        if e["source_hash"] == bench.source_hash(sources):
            assert got == e["bytes_per_launch"]
        else:
            assert got is None
        assert bench.measured_traffic(key, e["kernel"] + " other", sources) is None
    assert bench.measured_traffic("no_such_workload", "x") is None


def test_every_workload_key_is_known_to_one_bench_path():
    keys = list(workloads.WORKLOADS) + list(workloads.GROUPED_WORKLOADS) + list(workloads.RMSNORM_WORKLOADS)
    assert len(keys) == len(set(keys))
    assert workloads.HEADLINE in workloads.WORKLOADS


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
def test_cpu_baseline_is_a_bounded_oracle_sample():
    w = workloads.WORKLOADS["f32_128x128x128_identity"]
    A, B = workloads.make_inputs(w)
    r = bench.cpu_baseline(w, A, B, budget_s=0.5)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s" and r["value"] > 0 and r["cores"] >= 1
    assert "full workload" in r["sample"]

"""Host-side pieces of bench.py's output line: the refusal of several GPUs,
the oracle CPU baseline's fields, and the committed HBM-traffic records that
the roofline's `traffic` figure comes from."""

import json
import os
import subprocess
import sys

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stdout + r.stderr


def test_cpu_baseline_fields_on_the_small_workload():
    w, q, k, v, do, mask, scale = W.bsa_inputs(1)
    cb = bench.cpu_baseline_bsa((w, q, k, v, do, mask, scale, None), 0.2)
    assert cb["kind"] == "oracle" and cb["unit"] == "TFLOP/s"
    assert cb["value"] > 0 and cb["cores"] >= 1
    assert "Q blocks" in cb["sample"] and w["name"] in cb["sample"]


def test_traffic_records_name_their_kernel_sources():
    """Every record carries the hash of the sources it was measured on, and a
    record whose hash matches the tree gives bytes per launch (a stale one
    would give None, never an old figure)."""
    with open(bench.TRAFFIC_JSON) as f:
        t = json.load(f)
    cal = t["_calibration"]
    assert cal["fetch_factor"] > 0 and cal["write_factor"] > 0
    for workload, ents in t.items():
        if workload.startswith("_"):
            continue
        for kernel, e in ents.items():
            assert kernel in bench.KERNEL_SOURCES
            got = bench._traffic(workload, kernel)
            if e["src_hash"] == bench._src_hash(kernel):
                assert got == e["bytes_per_launch"] > 0
            else:
                assert got is None

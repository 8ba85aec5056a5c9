"""bench.py end to end on one GPU: the JSON line it prints carries the fields and the arithmetic it
promises (GPU)."""

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_line():
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1", "--secondary",
           "m_groups_tiny", "--cpu-seconds", "1", "--warm-ms", "1"]
    print("case bench line", " ".join(cmd[1:]), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-2000:]
    d = json.loads(res.stdout.strip().splitlines()[-1])

    assert d["unit"] == "GB/s" and d["higher_is_better"] is True and d["n_gpus"] == 1
    assert d["steps"] == 3 and d["warmup"] == 1 and d["data"] == "synthetic" and d["dtype"] == "u8"
    cfg = d["config"]
    assert cfg["workload"] == "k_groups_large" and cfg["scales_shape"] == [28672, 8192] and cfg["num_groups"] == 8
    assert cfg["bytes_per_step"] == 234881024 + 235798528
    # value, ms_per_step and the roofline's achieved rate come from one interval
    us = d["us_per_launch"]
    assert us > 0 and abs(d["ms_per_step"] * 1e3 - us) < 1e-3 * us + 1e-3
    assert abs(d["value"] - cfg["bytes_per_step"] / us / 1e3) < 1e-3 * d["value"] + 0.05
    roof = d["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert roof["achieved"] == d["value"] and abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert 0 < roof["frac"] < 1
    assert roof["traffic"] is None or roof["traffic"] > 0
    assert roof["launch_floor_us"] > 0 and 0 < roof["frac_ceiling"] <= 1
    # the other configuration and the secondary figures
    tiny = d["configs"]["m_groups_tiny"]
    assert tiny["steps"] == 200 and tiny["us_per_launch"] > 0 and tiny["bytes_per_step"] == 16384 + 24576
    for cold in (d["cold"], tiny["cold"]):
        assert 0 < cold["us_p10"] <= cold["us_median"] <= cold["us_p90"] and cold["flush_bytes"] == 512 << 20
    assert d["cold"]["launches"] == 50 and tiny["cold"]["launches"] == 200
    assert d["warm"]["us_per_launch"] > 0
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["unit"] == "GB/s" and cpu["value"] > 0 and cpu["cores"] == 1
    assert cpu["all_cores"]["value"] > 0 and cpu["all_cores"]["cores"] >= 1

"""bench.py's output contract: one GPU only, and one JSON line with the fields a reader of
the benchmark relies on (the metric, the step rate, the roofline of the dominant kernel and
the CPU baseline)."""

import json
import os
import subprocess
import sys

import pytest

from tests.conftest import gpu_available

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout.strip() == ""


@pytest.mark.gpu
@pytest.mark.timeout(600)
@pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")
def test_bench_json_line():
    cmd = [sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1",
           "--no-other-workloads", "--flushed-steps", "0", "--graph-steps", "0", "--cpu-seconds", "1",
           "--copy-calibration-mib", "64"]
    print("running", " ".join(cmd[1:]), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=540, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.strip().splitlines() if ln.strip()]
    assert len(lines) == 1, "bench.py prints exactly one line on stdout"
    d = json.loads(lines[0])
    for key, typ in (("metric", str), ("value", float), ("unit", str), ("n_gpus", int), ("steps", int),
                     ("warmup", int), ("ms_per_step", float), ("higher_is_better", bool), ("scaling", str),
                     ("dtype", str), ("data", str), ("config", dict), ("roofline", dict), ("cpu_baseline", dict)):
        assert isinstance(d[key], typ), key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1 and d["higher_is_better"] is True
    assert d["unit"] == "steps/s" and d["value"] > 0
    assert abs(d["value"] * d["ms_per_step"] - 1000.0) < 1.0
    assert "vs_baseline" in d and d["config"]["workload"] == "serving_b128_h64_l32768_bf16"
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert 0.0 < rf["frac"] < 1.0 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert "traffic" in rf
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] >= 1 and cb["value"] > 0 and cb["unit"] == "steps/s"
    assert isinstance(cb["sample"], str) and cb["sample"]
    host = d["host"]
    assert host["nproc"] >= 1 and "cpu_model" in host
    # the pool placement the value was measured on, and the same step with same-phase pools
    pp = d["pool_placement"]
    assert pp["v_minus_k_mod_1KiB"] == 256 and pp["min_minus_max_mod_1KiB"] == 256
    sp = pp["same_phase_pools"]
    assert sp["v_minus_k_mod_1KiB"] == 0 and sp["min_minus_max_mod_1KiB"] == 0 and sp["steps_per_s"] > 0

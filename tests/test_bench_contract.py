"""bench.py's command-line contract: one GPU only, the CPU baseline's fields,
and (on a GPU) the one JSON line with the roofline and the per-kernel lines."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True,
                       timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_cpu_baseline_fields():
    sys.path.insert(0, ROOT)
    import bench
    from scale_invariant_row_amd import inputs
    l2c = inputs.make("l2_rows_res_8192x4096")
    slc = inputs.make("slerp_rows_8192x4096")
    cb = bench.cpu_baseline(l2c, slc, rows=4)
    assert cb["kind"] == "oracle" and cb["unit"] == "GB/s" and cb["cores"] == 1
    assert cb["value"] > 0
    assert cb["sample"].startswith("first 4 of 8192 rows")


@pytest.mark.gpu
def test_json_line():
    """A short run prints one JSON line with the contract's fields."""
    r = subprocess.run([sys.executable, BENCH, "--steps", "3", "--warmup", "1", "--no-cpu"],
                       capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "ops"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["higher_is_better"] is True and d["unit"] == "GB/s"
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert "workload" in d["config"]
    rl = d["roofline"]
    assert rl["bound"] == "hbm" and rl["unit"] == "GB/s" and rl["peak"] == 8000.0
    assert 0 < rl["frac"] < 1
    assert abs(rl["frac"] - rl["achieved"] / rl["peak"]) < 1e-3
    # the step's two kernels and the stream reference are among the per-kernel lines
    for k in ("l2_rows_res_8192x4096", "slerp_rows_8192x4096", "stream_ceiling_8192x4096"):
        assert d["ops"][k]["us"] > 0

"""bench.py's output contract on the GPU: one JSON line with every field a
reader of the benchmark relies on, consistent with itself.

A short run of the default workload (the large-batch decode step) with a
one-second CPU baseline; the fields are checked for presence, type and
internal consistency (value = algorithmic bytes / step time, the roofline
fraction = achieved / peak), not for speed.
"""
import json
import os
import subprocess
import sys

import pytest

from gpu_util import note

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.gpu
def test_bench_prints_one_json_line_with_the_contract():
    note("bench.py: large_batch_decode, 3 steps, 1 s CPU baseline")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1",
                        "--cpu-budget", "1"], cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout[-3000:]
    d = json.loads(lines[0])

    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert (d["n_gpus"], d["steps"], d["warmup"]) == (1, 3, 1)
    assert d["unit"] == "GB/s" and d["higher_is_better"] is True and d["vs_baseline"] is None
    assert d["dtype"] == "f32" and d["cache_scrub"] is True
    assert d["config"]["workload"] == "large_batch_decode"
    assert "model" not in d["config"]
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert abs(d["value"] - d["algorithmic_bytes_per_step"] / (d["ms_per_step"] * 1e-3) / 1e9) <= 0.01 * d["value"]

    roof = d["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in roof, key
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert 0 < roof["frac"] < 1
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    # the dominant kernel's bytes over its own launch time
    dom = [k for k in d["kernels"] if k["name"] == roof["kernel"]][0]
    assert abs(roof["achieved"] - dom["algorithmic_bytes"] / (dom["us"] * 1e-6) / 1e9) <= 0.01 * roof["achieved"]
    assert roof["traffic"] is None or roof["traffic"] > 0
    cp = roof["copy_same_bytes"]
    assert cp["GB/s"] > 0 and cp["bytes_each_way"] > 0 and cp["kernel_frac_of_copy"] > 0

    cpu = d["cpu_baseline"]
    assert cpu["value"] > 0 and cpu["unit"] == "GB/s" and cpu["cores"] >= 1
    assert cpu["kind"] == "oracle" and isinstance(cpu["sample"], str) and cpu["sample"]

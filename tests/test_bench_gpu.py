"""bench.py end to end on the GPU (a few steps): the one JSON line has the
keys the benchmark contract names, its figures agree with each other
(value = counted flops / mean step time; each kernel's time inside the
timed steps adds up to the step; the roofline names the longest kernel and
rates it at its counted flops), and the kernels' per-row flag counts are
those of the workload."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_line_is_consistent():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1",
                        "--no-cpu-baseline"], capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    rec = json.loads(r.stdout.strip().splitlines()[-1])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "kernel_ms", "row_flags"):
        assert key in rec, key
    assert rec["n_gpus"] == 1 and rec["steps"] == 3 and rec["warmup"] == 1
    assert rec["unit"] == "TFLOP/s" and rec["dtype"] == "bf16" and rec["higher_is_better"] is True
    cfg = rec["config"]
    assert (cfg["batch"], cfg["heads_q"], cfg["seq_len"], cfg["head_dim"], cfg["causal"]) == (16, 12, 1024, 64, True)
    fl = cfg["flops_per_step"]
    assert fl == pytest.approx(7 * 2 * 16 * 12 * 1024 * 1024 * 64 / 2, rel=1e-9)
    ms = rec["ms_per_step"]
    assert rec["value"] == pytest.approx(fl / (ms * 1e-3) / 1e12, rel=1e-3)
    km = rec["kernel_ms"]
    assert set(km) == {"attn_fwd", "bwd_dq", "bwd_dkdv"}
    # the three launches fill the step (events between them, same steps)
    assert sum(km.values()) == pytest.approx(ms, rel=0.05)
    roof = rec["roofline"]
    assert roof["kernel"] == max(km, key=km.get)
    n_products = {"attn_fwd": 2, "bwd_dq": 3, "bwd_dkdv": 4}[roof["kernel"]]
    assert roof["achieved"] == pytest.approx(n_products * fl / 7 / (km[roof["kernel"]] * 1e-3) / 1e12, rel=1e-3)
    assert roof["peak"] == 2500.0 and roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s"
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"], abs=1e-4)
    assert 0.0 < roof["frac"] < 1.0
    flags = rec["row_flags"]
    assert flags["rows"] == 16 * 12 * 1024
    assert 0 < flags["tie_rows"] < flags["rows"] and flags["guard_applied_rows"] == flags["tie_rows"]

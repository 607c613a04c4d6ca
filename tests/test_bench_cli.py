"""bench.py's command line on the host: more than one GPU is refused with a
JSON error line and exit status 2 before anything touches a device."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2, (r.returncode, r.stderr[-500:])
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_measured_traffic_is_keyed_by_workload_and_sources():
    """roofline.traffic is reported only for the workload and the kernel
    sources the counters were taken on (host only: no device is touched)."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    m = b.MEASURED_TRAFFIC["bwd_dkdv"]
    t = b.measured_traffic("bwd_dkdv", m["workload"])
    if m["sources_sha256"] == b.kernel_sources_sha256("bwd_dkdv"):
        assert t == int(1024 * (m["fetch_kib"] * m["fetch_scale"] + m["write_kib"] * m["write_scale"]))
    else:
        assert t is None
    for other in ("gpt2m", "llama8b", "stress", "tiny"):
        assert b.measured_traffic("bwd_dkdv", other) is None
    assert b.measured_traffic("attn_fwd", m["workload"]) is None

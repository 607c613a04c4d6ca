"""The shader clock while each kernel of the step runs (a measurement,
reported; the assertions are sanity bounds only).

A monitor kernel (tests/probes/clock_probe.hip: 16 single waves on a second
stream, default priority) samples the constant 100 MHz counter and the
shader-clock counter every microsecond while one kernel is launched back to
back on the main stream for longer than the monitor runs.  The clock over a
window is the ratio of the two counters' advances.  Run with -s to see the
figures: at GPT-2 Small the three kernels run well below the 2.4 GHz peak
clock, which the peak matrix rate assumes, and the same dK/dV launch on
all-zero Q and dO (fewer switching bits) runs faster.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import flashattention_fa_fwd_amd as fa

from _util import dev, make, report

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "probes", "libisa_probe.so")
NWG, PERIOD = 16, 100          # monitor waves; ticks of the 100 MHz counter per sample (1 us)
WINDOW_US, SKIP_US = 3000, 300  # monitored span; samples before SKIP_US are not used


@pytest.fixture(scope="module")
def probe():
    if not os.path.exists(LIB):
        raise FileNotFoundError(f"{LIB} is not built (tests/probes/build_probe.py)")
    L = ctypes.CDLL(LIB)
    L.probe_clock_monitor.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_uint, ctypes.c_void_p]
    return L


def _monitored(probe, launch, per_launch_us):
    """Mean shader clock (MHz) per monitor wave while `launch` runs back to
    back on the current stream, from SKIP_US to WINDOW_US."""
    nsamp = WINDOW_US * 100 // PERIOD
    buf = torch.zeros(NWG * nsamp * 2, dtype=torch.int64, device="cuda")
    side = torch.cuda.Stream()
    n = int(1.5 * WINDOW_US / max(per_launch_us, 1.0)) + 2
    torch.cuda.synchronize()
    assert probe.probe_clock_monitor(buf.data_ptr(), NWG, nsamp, PERIOD, ctypes.c_void_p(side.cuda_stream)) == 0
    for _ in range(n):
        launch()
    torch.cuda.synchronize()
    s = buf.view(NWG, nsamp, 2).cpu().numpy().astype(np.float64)
    i0 = SKIP_US * 100 // PERIOD
    dr = s[:, -1, 0] - s[:, i0, 0]
    dc = s[:, -1, 1] - s[:, i0, 1]
    return dc / dr * 100.0


def _time_us(launch, n=20):
    for _ in range(3):
        launch()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        launch()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1000.0 / n


def test_shader_clock_per_kernel(probe):
    x = make("gpt2s")
    wl = x["workload"]
    q, k, v, do = dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["do"])
    kw = dict(causal=wl.causal, guard="beta")
    p = fa.make_params(wl.batch, wl.heads_q, wl.heads_kv, wl.seqlen, wl.head_dim, **kw)
    f0 = fa.attn_fwd(q, k, v, **kw)
    b0 = fa.attn_bwd(q, k, v, f0["o"], do, f0["row_m"], f0["row_l"], **kw)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty_like(f0["row_m"])
    zq, zdo = torch.zeros_like(q), torch.zeros_like(do)
    fo = {}
    kernels = {
        "attn_fwd": lambda: fa.attn_fwd(q, k, v, out=fo, **kw),
        "bwd_dq": lambda: fa.attn_bwd_dq(p, q, k, v, f0["o"], do, f0["row_m"], f0["row_l"], dq, delta),
        "bwd_dkdv": lambda: fa.attn_bwd_dkdv(p, q, k, v, do, f0["row_m"], f0["row_l"], b0["delta"], dk, dv),
        "bwd_dkdv, Q = dO = 0": lambda: fa.attn_bwd_dkdv(p, zq, k, v, zdo, f0["row_m"], f0["row_l"],
                                                         b0["delta"], dk, dv),
    }
    # the monitor alone (the card otherwise idle)
    idle = _monitored(probe, lambda: None, 1e9)
    report("shader clock, monitor alone", mean_mhz=f"{idle.mean():.0f}", min=f"{idle.min():.0f}",
           max=f"{idle.max():.0f}")
    for name, fn in kernels.items():
        us = _time_us(fn)
        mhz = _monitored(probe, fn, us)
        report(f"shader clock, GPT-2 Small {name}", us_per_launch=f"{us:.1f}", mean_mhz=f"{mhz.mean():.0f}",
               min=f"{mhz.min():.0f}", max=f"{mhz.max():.0f}")
        assert 100.0 < mhz.min() and mhz.max() < 2600.0
    assert 100.0 < idle.min() and idle.max() < 2600.0


def test_shader_clock_llama_dkdv(probe):
    """The d = 128 dK/dV kernel at the Llama-3.1-8B GQA shape (one workgroup
    of four waves per CU), for comparison with the GPT-2 Small kernels."""
    x = make("llama8b")
    wl = x["workload"]
    q, k, v, do = dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["do"])
    kw = dict(causal=wl.causal, guard="beta")
    p = fa.make_params(wl.batch, wl.heads_q, wl.heads_kv, wl.seqlen, wl.head_dim, **kw)
    f0 = fa.attn_fwd(q, k, v, **kw)
    b0 = fa.attn_bwd(q, k, v, f0["o"], do, f0["row_m"], f0["row_l"], **kw)
    dk, dv = torch.empty_like(k), torch.empty_like(v)
    fn = lambda: fa.attn_bwd_dkdv(p, q, k, v, do, f0["row_m"], f0["row_l"], b0["delta"], dk, dv)
    us = _time_us(fn, n=5)
    mhz = _monitored(probe, fn, us)
    report("shader clock, Llama-3.1-8B bwd_dkdv", us_per_launch=f"{us:.1f}", mean_mhz=f"{mhz.mean():.0f}",
           min=f"{mhz.min():.0f}", max=f"{mhz.max():.0f}")
    assert 100.0 < mhz.min() and mhz.max() < 2600.0

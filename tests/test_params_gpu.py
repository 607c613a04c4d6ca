"""Parity with the method's tunable parameters away from their defaults:
the tie window (tie_eps = 0, exact repeats only, and 0.05), the ε guard's
shift (2^-3), β = 4, and softmax scales other than 1/sqrt(d) (0.05, and 0.3,
which makes the logits larger).  Each on a ragged grouped shape at d = 64
(causal) and at d = 128 (non-causal): tie flags and certified bf16 Ō bit for
bit against the oracle's emulation run with the same parameters, O within
the stated bounds of FP64, and δ, dQ, dK, dV within the backward bounds."""
import numpy as np
import pytest
import torch

import flashattention_fa_fwd_amd as fa
import oracle as orc
from flashattention_fa_fwd_amd import workloads as W

from _util import GUARD, bits, check_o, dev, f32, report, schedule, threads
from test_bwd_gpu import _check, _floors

pytestmark = pytest.mark.gpu

CASES = [
    dict(guard="beta", tie_eps=0.0),
    dict(guard="beta", tie_eps=0.05),
    dict(guard="eps", shift_eps=2.0 ** -3),
    dict(guard="beta", beta=4.0),
    dict(guard="beta", softmax_scale=0.05),
    dict(guard="none", softmax_scale=0.3),
]
SHAPES = [(1, 4, 2, 300, 64, True), (1, 2, 1, 200, 128, False)]  # B, Hq, Hkv, N, d, causal


def _id(c):
    return "-".join(f"{k}={v:g}" if isinstance(v, float) else f"{v}" for k, v in c.items())


@pytest.mark.parametrize("shape", SHAPES, ids=["d64-causal", "d128-full"])
@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_parameters(case, shape):
    B, Hq, Hkv, N, d, causal = shape
    kw = dict(beta=2.0, tie_eps=1e-3, shift_eps=2.0 ** -5, softmax_scale=None)
    kw.update({k: v for k, v in case.items() if k != "guard"})
    guard = case["guard"]
    wl = W.Workload("params", B, Hq, Hkv, N, d, causal, 1.0, 1.0, "const", -0.3, 4.0, 0.1, 0.0, 16.0,
                    91 + d)
    x = W.make_custom(wl)
    alpha = None if kw["softmax_scale"] is None else float(np.float32(kw["softmax_scale"]))
    p = orc.Problem(B, Hq, Hkv, N, d, causal, GUARD[guard], alpha=alpha, beta=kw["beta"],
                    tie_eps=kw["tie_eps"], shift_eps=kw["shift_eps"])
    q, k, v, do = dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["do"])
    f = fa.attn_fwd(q, k, v, causal=causal, guard=guard, return_obar=True, **kw)
    b = fa.attn_bwd(q, k, v, f["o"], do, f["row_m"], f["row_l"], causal=causal, guard=guard, **kw)
    torch.cuda.synchronize()

    # forward: flags and certified bf16 Ō bits, O against FP64
    e = orc.fwd_emu(p, schedule(p), x["q"], x["k"], x["v"], nthreads=threads())
    o64, _ = orc.fwd_f64(p, x["q"], x["k"], x["v"], nthreads=threads())
    flags = f["row_flags"].cpu().numpy()
    fc = e["flag_cert"].astype(bool)
    assert np.array_equal(flags[fc], e["flags"][fc])
    out = check_o(f32(f["o"]), o64, e["o"], False)
    cert = e["obar_cert"].astype(bool)
    assert np.array_equal(bits(f["obar"])[cert], orc.bf16_from_f32(e["obar"].astype(np.float32))[cert])

    # backward against FP64, bounded by the method's own rounding points
    ref = orc.bwd_f64(p, x["q"], x["k"], x["v"], x["do"], nthreads=threads())
    fl = _floors(p, x, ref)
    for key in ("dq", "dk", "dv"):
        out.update(_check(key, f32(b[key]), ref[key], fl[key]))
    out.update(_check("delta", b["delta"].cpu().numpy(), ref["delta"], fl["delta"]))
    report(f"params {_id(case)} {shape}", ties=int((flags & 1).sum()), guarded=int(((flags & 4) != 0).sum()),
           flag_cert=f"{fc.mean():.3f}", obar_cert=f"{cert.mean():.3f}", **out)


@pytest.mark.parametrize("shape", SHAPES, ids=["d64-causal", "d128-full"])
@pytest.mark.parametrize("guard", ["beta", "eps"])
def test_negative_row_maxima(guard, shape):
    """Every logit moved down by about 30 (feature d-1 reserved: Q = 1 there
    and K = bf16(-30/alpha) for every key), so every row maximum is negative:
    the β guard's tie rows take the shift 0 instead of β·r, the ε guard's
    r + ε as before.  Flags and certified bf16 Ō bit for bit, O against FP64."""
    B, Hq, Hkv, N, d, causal = shape
    wl = W.Workload("negmax", B, Hq, Hkv, N, d, causal, 1.0, 1.0, "const", -0.3, 0.0, 0.1, 0.0, 8.0,
                    131 + d)
    x = W.make_custom(wl)
    one = W.to_bf16_bits(np.ones(1, np.float32))[0]
    low = W.to_bf16_bits(np.full(1, -30.0 / wl.alpha, np.float32))[0]
    x["q"][..., d - 1] = one
    x["k"][..., d - 1] = low
    p = orc.Problem(B, Hq, Hkv, N, d, causal, GUARD[guard])
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    f = fa.attn_fwd(q, k, v, causal=causal, guard=guard, return_obar=True, return_row_max=True)
    torch.cuda.synchronize()
    assert (f["row_max"].cpu().numpy() < 0).all()
    e = orc.fwd_emu(p, schedule(p), x["q"], x["k"], x["v"], nthreads=threads())
    o64, _ = orc.fwd_f64(p, x["q"], x["k"], x["v"], nthreads=threads())
    flags = f["row_flags"].cpu().numpy()
    fc = e["flag_cert"].astype(bool)
    assert np.array_equal(flags[fc], e["flags"][fc])
    tie = (flags & 1) != 0
    assert tie.sum() > 0
    m = f["row_m"].cpu().numpy()
    if guard == "beta":
        assert (m[tie] == 0.0).all()  # shift 0 for a non-positive repeated maximum
    out = check_o(f32(f["o"]), o64, e["o"], False)
    cert = e["obar_cert"].astype(bool)
    assert np.array_equal(bits(f["obar"])[cert], orc.bf16_from_f32(e["obar"].astype(np.float32))[cert])
    report(f"negative maxima {guard} {shape}", ties=int(tie.sum()), flag_cert=f"{fc.mean():.3f}",
           obar_cert=f"{cert.mean():.3f}", **out)

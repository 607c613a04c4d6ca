"""Parity over seeded random configurations: shape (batch, query and KV
heads, a sequence length anywhere up to past the 1024-key rounding point,
d = 64 or 128), causal or not, guard, Ō mode, delta mode, logit scale and
tie planting are drawn from a fixed-seed generator, so the cases are the
same on every run.  Each case checks, as the dedicated tests do: tie flags
on certified rows and certified bf16 Ō elements bit for bit against the
oracle's emulation, O against FP64 within the bound the method permits, and
delta, dQ, dK, dV against FP64 within the backward bound."""
import numpy as np
import pytest
import torch

import flashattention_fa_fwd_amd as fa
import oracle as orc
from flashattention_fa_fwd_amd import workloads as W

from _util import bits, check_o, dev, f32, problem, rel_errors, report, schedule, threads
from test_bwd_gpu import _check, _floors

pytestmark = pytest.mark.gpu

# keys per step and per Ō rounding of the streaming schedule: lengths next to
# their multiples are drawn more often
_EDGES = [1, 2, 63, 64, 65, 127, 128, 129, 511, 512, 513, 1023, 1024, 1025]


def _cases(n=30, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        d = int(rng.choice([64, 128]))
        hkv = int(rng.integers(1, 4))
        g = int(rng.choice([1, 2, 4]))
        b = int(rng.integers(1, 3))
        N = int(rng.choice(_EDGES)) if rng.random() < 0.5 else int(rng.integers(3, 1100))
        causal = bool(rng.random() < 0.6)
        guard = str(rng.choice(["none", "beta", "eps"]))
        obar_fp32 = bool(rng.random() < 0.25)
        delta = "dp_p" if rng.random() < 0.25 else "do_o"
        sigma = float(rng.choice([1.0, 1.5, 2.5]))
        tie_frac = float(rng.choice([0.05, 0.2]))
        lift = float(rng.choice([4.0, 8.0, 16.0]))
        out.append((c, b, hkv * g, hkv, N, d, causal, guard, obar_fp32, delta, sigma, tie_frac, lift))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"case{c[0]}")
def test_random_configuration(case):
    c, B, Hq, Hkv, N, d, causal, guard, obar_fp32, delta, sigma, tie_frac, lift = case
    wl = W.Workload(f"random{c}", B, Hq, Hkv, N, d, causal, sigma, sigma, "const", -0.3,
                    4.0 if N > 2 else 0.0, tie_frac, 0.2, lift, 5000 + c)
    x = W.make_custom(wl)
    p = problem(wl, guard)
    # forward
    e = orc.fwd_emu(p, schedule(p, obar_fp32), x["q"], x["k"], x["v"], nthreads=threads())
    o64, _ = orc.fwd_f64(p, x["q"], x["k"], x["v"], nthreads=threads())
    q, k, v, do = dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["do"])
    f = fa.attn_fwd(q, k, v, causal=causal, guard=guard, obar_fp32=obar_fp32, return_obar=True)
    b = fa.attn_bwd(q, k, v, None if delta == "dp_p" else f["o"], do, f["row_m"], f["row_l"],
                    causal=causal, guard=guard, delta=delta)
    torch.cuda.synchronize()
    flags = f["row_flags"].cpu().numpy()
    fc = e["flag_cert"].astype(bool)
    assert np.array_equal(flags[fc], e["flags"][fc])
    nan = np.isnan(e["o"]).any(-1)
    errs = check_o(f32(f["o"]), o64, e["o"], obar_fp32, rows=~nan)
    ncert = 0
    if not obar_fp32:
        ob_gpu = bits(f["obar"])
        ob_emu = orc.bf16_from_f32(e["obar"].astype(np.float32))
        cert = e["obar_cert"].astype(bool)
        assert np.array_equal(ob_gpu[cert], ob_emu[cert])
        ncert = int(cert.sum())
    # backward (rows whose denominator underflowed carry NaN by definition)
    ref = orc.bwd_f64(p, x["q"], x["k"], x["v"], x["do"], nthreads=threads())
    out = {}
    if not nan.any():
        fl = _floors(p, x, ref, obar_fp32, delta=delta)
        if N > 1:
            out.update(_check("dq", f32(b["dq"]), ref["dq"], fl["dq"]))
            out.update(_check("dk", f32(b["dk"]), ref["dk"], fl["dk"]))
        out.update(_check("dv", f32(b["dv"]), ref["dv"], fl["dv"]))
        if delta == "do_o":
            out.update(_check("delta", b["delta"].cpu().numpy(), ref["delta"], fl["delta"]))
        else:
            mx, mean = rel_errors(b["delta"].cpu().numpy(), ref["delta"])
            assert mx <= 1e-5 and mean <= 1e-5, (mx, mean)
    report(f"random case {c}: B{B} Hq{Hq} Hkv{Hkv} N{N} d{d} {'causal' if causal else 'full'} {guard} "
           f"{'fp32' if obar_fp32 else 'bf16'} Ō delta={delta}", ties=int((flags & 1).sum()),
           cert_elements=ncert, **errs, **out)

"""The pages' finding as a measured invariant of the kernels ([R] "Core idea",
equations, paper §3.3.2; [S] "Key claims"): on rows whose maximum repeats,
the bf16 rounding of Ō = P̄V is biased toward negative values on
negative-dominated features when P̄ = 1 at the repeated maximum (unguarded),
and the beta guard removes the bias.  fp32 Ō removes it too.  The eps
variant is measured and reported, not asserted.

Signed error of one element, in output units (independent of the shift):
    e = (Ō_gpu - Ō_64(m)) / ℓ_64(m)
with m the oracle's own final shift for the row (row statistics) and Ō_64,
ℓ_64 the exact unnormalised sums for that shift.  A feature is
negative-dominated when its V column has a negative mean over the keys.
"""
import numpy as np
import pytest
import torch

import flashattention_fa_fwd_amd as fa
import oracle as orc
from flashattention_fa_fwd_amd import workloads as W

from _util import dev, make, problem, report, schedule, threads

pytestmark = pytest.mark.gpu


def _signed_errors(name, guard, obar_fp32, heads, sched="stream"):
    x = make(name)
    wl = x["workload"]
    p = problem(wl, guard)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    r = fa.attn_fwd(q, k, v, causal=wl.causal, guard=guard, obar_fp32=obar_fp32, return_obar=True,
                    schedule=sched)
    torch.cuda.synchronize()
    ob = r["obar"].float().cpu().numpy().astype(np.float64)
    shp = (-1, wl.seqlen, wl.head_dim)
    ob = ob.reshape(shp)[heads]
    st = orc.row_stats(p, x["q"], x["k"], schedule(p, sched=sched), heads=heads, nthreads=threads())
    ob64, l64 = orc.obar_f64(p, x["q"], x["k"], x["v"], st["m"], heads=heads, nthreads=threads())
    ob64 = ob64.reshape(shp)[heads]
    l64 = l64.reshape(-1, wl.seqlen)[heads]
    err = (ob - ob64) / l64[..., None]
    tie = ((st["flags"] & orc.ROW_TIE) != 0).reshape(-1, wl.seqlen)[heads]
    cert = st["flag_cert"].reshape(-1, wl.seqlen)[heads].astype(bool)
    gpu_tie = ((r["row_flags"].cpu().numpy() & 1) != 0).reshape(-1, wl.seqlen)[heads]
    assert np.array_equal(gpu_tie[cert], tie[cert])
    # negative-dominated features: V column mean over the keys < 0
    g = wl.heads_q // wl.heads_kv
    vv = W.bits_to_f32(x["v"]).astype(np.float64).reshape(-1, wl.seqlen, wl.head_dim)
    kvh = [(h // wl.heads_q) * wl.heads_kv + (h % wl.heads_q) // g for h in heads]
    neg = vv[kvh].mean(axis=1) < 0  # [heads, d]
    return err, tie & cert, neg


def _stats(e):
    return float(e.mean()), float(e.std() / np.sqrt(max(e.size, 1))), int(e.size)


@pytest.mark.parametrize("name,heads", [("gpt2s", list(range(0, 192, 12))), ("gpt2m", list(range(0, 128, 8)))])
def test_bias_unguarded_negative_guarded_zero(name, heads):
    res = {}
    for guard, f32 in (("none", False), ("beta", False), ("eps", False), ("none", True), ("beta", True)):
        err, tie, neg = _signed_errors(name, guard, f32, heads)
        sel_neg = tie[..., None] & neg[:, None, :]
        sel_pos = tie[..., None] & ~neg[:, None, :]
        single = ~tie[..., None] & neg[:, None, :]
        res[(guard, f32)] = dict(neg=_stats(err[sel_neg]), pos=_stats(err[sel_pos]), single=_stats(err[single]))
    for (guard, f32), d in res.items():
        report(f"signed error {name} guard={guard} obar={'fp32' if f32 else 'bf16'}",
               **{k: f"{m:+.3e}±{se:.1e} (n={n})" for k, (m, se, n) in d.items()})
    m, se, n = res[("none", False)]["neg"]
    assert n > 10000 and m < -3 * se, "unguarded bf16 Ō should carry a negative bias on tie rows"
    assert abs(res[("beta", False)]["neg"][0]) <= 1e-4
    assert abs(res[("none", True)]["neg"][0]) <= 1e-4
    assert abs(res[("beta", True)]["neg"][0]) <= 1e-4


@pytest.mark.parametrize("sched", ["fa2_ops", "untiled"])
def test_bias_under_other_schedules(sched):
    """The same finding under the analysed implementation's schedule (FA2 as
    tensor operations, 512-key blocks, bf16 block product; [R] "Points to
    doubt") and without tiling ([S] "Key claims": disabling tiling still
    fails): unguarded bf16 Ō is biased negative on the negative-dominated
    features of tie rows, the beta guard removes it."""
    heads = list(range(0, 192, 12))
    res = {}
    for guard in ("none", "beta"):
        err, tie, neg = _signed_errors("gpt2s", guard, False, heads, sched)
        sel_neg = tie[..., None] & neg[:, None, :]
        res[guard] = _stats(err[sel_neg])
        report(f"signed error gpt2s schedule={sched} guard={guard}",
               neg=f"{res[guard][0]:+.3e}±{res[guard][1]:.1e} (n={res[guard][2]})")
    m, se, n = res["none"]
    assert n > 10000 and m < -3 * se
    assert abs(res["beta"][0]) <= 1e-4

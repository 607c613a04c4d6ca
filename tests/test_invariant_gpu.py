"""The pages' finding as a measured invariant of the kernels ([R] "Core idea",
equations, paper §3.3.2; [S] "Key claims"): on rows whose maximum repeats,
the bf16 rounding of Ō = P̄V is biased toward negative values on
negative-dominated features when P̄ = 1 at the repeated maximum (unguarded),
and the beta guard removes the bias.  fp32 Ō removes it too.  The eps
variant leaves a bias of the opposite sign whose size follows in closed form
from bf16(exp(-2^-5)) = 0.96875 (asserted below).

The pages locate the mechanism in the attention-sink regime (the repeated
maximum holds nearly all of the row's weight): the assertions run on the
``_sink`` workloads, whose planted pair sits 20 logits above the row.  The
configurations as stated (pair at a natural row maximum) are measured and
reported beside them.

Signed error of one element, in output units (independent of the shift):
    e = (Ō_gpu - Ō_64(m)) / ℓ_64(m)
with m the oracle's own final shift for the row (row statistics) and Ō_64,
ℓ_64 the exact unnormalised sums for that shift.  A feature is
negative-dominated when its V column has a negative mean over the keys.
Statistics: the errors of a row's selected features share that row's P̄
roundings, so each row contributes the mean over its selected features and
the standard error is taken over rows.
"""
import numpy as np
import pytest
import torch

import flashattention_fa_fwd_amd as fa
import oracle as orc
from flashattention_fa_fwd_amd import workloads as W

from _util import dev, make, problem, report, schedule, threads

pytestmark = pytest.mark.gpu

SHIFT_EPS = 2.0 ** -5


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
    gflags = r["row_flags"].cpu().numpy().reshape(-1, wl.seqlen)[heads]
    gpu_tie = (gflags & orc.ROW_TIE) != 0
    assert np.array_equal(gpu_tie[cert], tie[cert])
    # rows whose weights all underflowed (ℓ = 0: a tie at a maximum r above
    # ~88.7 under the beta guard, whose shift 2r puts every weight below
    # fp32's range), and rows where such a tie was broken later by a larger
    # key (the rescale exp(2 r_old - r_new) overflows and multiplies the
    # underflowed ℓ: NaN) carry no rounding bias; they are left out, counted
    # and reported
    gl = r["row_l"].float().cpu().numpy().reshape(-1, wl.seqlen)[heads]
    ok = np.isfinite(gl) & (gl > 0)
    live = cert & ok
    nz, nn = int((cert & (gl == 0)).sum()), int((cert & ~np.isfinite(gl)).sum())
    if nz or nn:
        report(f"rows left out, {name} guard={guard} obar={'fp32' if obar_fp32 else 'bf16'}",
               zero_denominator=nz, non_finite=nn, tie_rows=int((tie & cert).sum()))
    # negative-dominated features: V column mean over the keys < 0
    g = wl.heads_q // wl.heads_kv
    vv = W.bits_to_f32(x["v"]).astype(np.float64).reshape(-1, wl.seqlen, wl.head_dim)
    kvh = [(h // wl.heads_q) * wl.heads_kv + (h % wl.heads_q) // g for h in heads]
    neg = vv[kvh].mean(axis=1) < 0  # [heads, d]
    return err, tie & live, ~tie & live, neg, l64


def _row_stats(err, sel):
    """Mean over rows of each row's mean over its selected elements, its
    standard error over rows, and the number of rows."""
    cnt = sel.sum(-1)
    rows = cnt > 0
    rm = np.where(sel, err, 0.0).sum(-1)[rows] / cnt[rows]
    n = int(rm.size)
    if n == 0:
        return float("nan"), float("nan"), 0
    return float(rm.mean()), float(rm.std() / np.sqrt(max(n - 1, 1))), n


def _measure(name, heads):
    res = {}
    for guard, f32 in (("none", False), ("beta", False), ("eps", False), ("none", True), ("beta", True)):
        err, tie, other, neg, _ = _signed_errors(name, guard, f32, heads)
        sel_neg = tie[..., None] & neg[:, None, :]
        sel_pos = tie[..., None] & ~neg[:, None, :]
        single = other[..., None] & neg[:, None, :]
        res[(guard, f32)] = dict(neg=_row_stats(err, sel_neg), pos=_row_stats(err, sel_pos),
                                 single=_row_stats(err, single))
    for (guard, f32), d in res.items():
        report(f"signed error {name} guard={guard} obar={'fp32' if f32 else 'bf16'}",
               **{k: f"{m:+.3e}±{se:.1e} (rows={n})" for k, (m, se, n) in d.items()})
    return res


@pytest.mark.parametrize("name,heads", [("gpt2s_sink", list(range(0, 192, 12))),
                                        ("gpt2m_sink", list(range(0, 128, 8)))])
def test_bias_unguarded_negative_guarded_zero(name, heads):
    res = _measure(name, heads)
    m, se, n = res[("none", False)]["neg"]
    assert n > 300 and m < -3 * se, "unguarded bf16 Ō should carry a negative bias on tie rows"
    assert abs(res[("beta", False)]["neg"][0]) <= 1e-4
    assert abs(res[("none", True)]["neg"][0]) <= 1e-4
    assert abs(res[("beta", True)]["neg"][0]) <= 1e-4


@pytest.mark.parametrize("name,heads", [("gpt2s", list(range(0, 192, 12))), ("gpt2m", list(range(0, 128, 8)))])
def test_bias_on_the_stated_configurations(name, heads):
    """The same measurement where the repeated maximum sits at a natural row
    maximum (the configurations as stated): reported; the guarded and fp32
    figures must still meet the bound."""
    res = _measure(name, heads)
    assert abs(res[("beta", False)]["neg"][0]) <= 1e-4
    assert abs(res[("none", True)]["neg"][0]) <= 1e-4


def test_eps_guard_bias_closed_form():
    """Under the eps guard a tie row's shift is r + 2^-5, so a tied key takes
    P̄ = exp(-2^-5) = 0.969233 in fp32 and bf16(0.969233) = 0.96875 as the
    matrix operand, while ℓ sums the fp32 value.  A tied key reached after
    the step that detects the tie therefore weighs 0.96875/0.969233 of its
    due in Ō; the first occurrence of a pair split over two 64-key steps was
    taken at P̄ = 1 (no tie yet) and carries its full weight through the
    fp32 rescale.  In the sink regime the pair holds nearly all of ℓ, so
    per row and feature  e = (0.96875 - exp(-2^-5)) * sum_late V_j / ℓ_64.
    The measured mean on negative-dominated features of rows before key 512
    must match that prediction to within 15 % plus three standard errors
    (the rest is the rounding of the other P̄ and of Ō itself)."""
    name, heads = "gpt2s_sink", list(range(0, 192, 12))
    x = make(name)
    wl = x["workload"]
    err, tie, _, neg, l64 = _signed_errors(name, "eps", False, heads)
    w_dev = float(np.float32(0.96875)) - float(np.exp(np.float32(-SHIFT_EPS)).astype(np.float64))
    vv = W.bits_to_f32(x["v"]).astype(np.float64)
    pred = np.full(err.shape, np.nan)
    hidx = {h: n for n, h in enumerate(heads)}
    step = schedule(problem(wl, "eps"))
    bn = step.block_n
    for (b, hk, i, a, bb) in x["planted"]:
        h = b * wl.heads_q + hk  # heads_q == heads_kv here
        if h not in hidx or not tie[hidx[h], i]:
            continue
        lo, hi = min(a, bb), max(a, bb)
        late = [hi] if lo // bn != hi // bn else [lo, hi]
        pred[hidx[h], i] = w_dev * vv[b, hk, late].sum(0) / l64[hidx[h], i]
    have = ~np.isnan(pred[..., 0])
    early = np.arange(wl.seqlen) < 512  # rows whose Ō is rounded once (at their end)
    out = {}
    for tag, rows in (("rows<512", early), ("rows>=512", ~early)):
        sel = (have & rows[None, :])[..., None] & neg[:, None, :]
        m_meas, se_meas, n = _row_stats(err, sel)
        m_pred, _, _ = _row_stats(np.nan_to_num(pred), sel)
        out[tag] = (m_meas, se_meas, n, m_pred)
        report(f"eps guard bias, gpt2s_sink, {tag}", measured=f"{m_meas:+.3e}±{se_meas:.1e}",
               predicted=f"{m_pred:+.3e}", rows=n)
    # Rows past key 512 also lose the later keys' small contributions to the
    # intermediate bf16 rounding of Ō (a property of the 512-key schedule,
    # of either sign guard); the closed form is asserted where Ō is rounded
    # once.
    m_meas, se_meas, n, m_pred = out["rows<512"]
    assert n > 150 and m_pred > 0
    assert abs(m_meas - m_pred) <= 0.15 * abs(m_pred) + 3 * se_meas


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
        err, tie, _, neg, _ = _signed_errors("gpt2s_sink", guard, False, heads, sched)
        sel_neg = tie[..., None] & neg[:, None, :]
        res[guard] = _row_stats(err, sel_neg)
        report(f"signed error gpt2s_sink schedule={sched} guard={guard}",
               neg=f"{res[guard][0]:+.3e}±{res[guard][1]:.1e} (rows={res[guard][2]})")
    m, se, n = res["none"]
    assert n > 300 and m < -3 * se
    assert abs(res["beta"][0]) <= 1e-4


@pytest.mark.parametrize("name,heads", [("gpt2s_dup", list(range(0, 192, 12))), ("stress", list(range(0, 32, 4)))])
def test_bias_key_duplication_and_large_logits(name, heads):
    """Two more inputs, measured and reported: keys duplicated without any
    lift of the query rows (the recipe as stated; a pair is a row's maximum
    only where the duplicated key happens to be one), and the large-logit
    shape (row maxima 30-60, d = 128, non-causal)."""
    res = _measure(name, heads)
    assert res[("none", False)]["neg"][2] > 50
    assert abs(res[("beta", False)]["neg"][0]) <= 1e-4
    assert abs(res[("none", True)]["neg"][0]) <= 1e-4

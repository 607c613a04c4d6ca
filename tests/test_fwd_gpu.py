"""Forward parity on the GPU: the HIP kernels (through the C ABI) against the
CPU oracle -- bit-exact tie flags and bf16 Ō where the oracle certifies them,
O within the stated tolerances of FP64, and the full-size workloads on
sampled heads."""
import numpy as np
import pytest
import torch

import flashattention_fa_fwd_amd as fa
import oracle as orc
from flashattention_fa_fwd_amd import workloads as W

from _util import GUARD, bits, check_o, dev, f32, make, problem, rel_errors, report, schedule, threads

pytestmark = pytest.mark.gpu


def _run_fwd(x, guard, obar_fp32=False, causal=None, beta=2.0):
    wl = x["workload"]
    c = wl.causal if causal is None else causal
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    r = fa.attn_fwd(q, k, v, causal=c, guard=guard, beta=beta, obar_fp32=obar_fp32,
                    return_obar=True, return_row_max=True)
    torch.cuda.synchronize()
    return r


@pytest.mark.parametrize("obar_fp32", [False, True])
@pytest.mark.parametrize("guard", ["none", "beta", "eps"])
def test_tiny_bit_exact(guard, obar_fp32):
    x = make("tiny")
    wl = x["workload"]
    p = problem(wl, guard)
    sc = schedule(p, obar_fp32)
    e = orc.fwd_emu(p, sc, x["q"], x["k"], x["v"], nthreads=threads())
    o64, _ = orc.fwd_f64(p, x["q"], x["k"], x["v"], nthreads=threads())
    r = _run_fwd(x, guard, obar_fp32)
    flags = r["row_flags"].cpu().numpy()
    fc = e["flag_cert"].astype(bool)
    # tie flags: bit-exact on every certified row; zero-denominator never here
    assert np.array_equal(flags[fc], e["flags"][fc])
    assert fc.all()  # every tie decision of this seed is certified
    # O against FP64 (bf16-Ō mode: against the method's own floor too)
    errs = check_o(f32(r["o"]), o64, e["o"], obar_fp32)
    # shift and denominator
    m_gpu = r["row_m"].cpu().numpy()
    assert np.allclose(m_gpu[fc], e["m"][fc], rtol=1e-6, atol=1e-6)
    assert np.allclose(r["row_l"].cpu().numpy(), e["l"], rtol=1e-4)
    n_unc = 0
    if not obar_fp32:
        ob_gpu = bits(r["obar"])
        ob_emu = orc.bf16_from_f32(e["obar"].astype(np.float32))
        cert = e["obar_cert"].astype(bool)
        assert np.array_equal(ob_gpu[cert], ob_emu[cert])
        # uncertified elements of certified rows: at most one bf16 step apart
        rows = np.broadcast_to(fc[..., None], cert.shape)
        unc = ~cert & rows
        n_unc = int(unc.sum())
        step = np.abs(ob_gpu[unc].astype(np.int32) - ob_emu[unc].astype(np.int32))
        assert np.all(step <= 1)
        n_diff = int((ob_gpu[unc] != ob_emu[unc]).sum())
    else:
        ob = r["obar"].cpu().numpy()
        obx, l64 = orc.obar_f64(p, x["q"], x["k"], x["v"], e["m"])
        err = np.abs(ob - obx) / l64[..., None]
        assert err[fc].max() < 2 ** -7
        n_diff = 0
    report(f"tiny {guard} {'fp32' if obar_fp32 else 'bf16'}", flag_rows_cert=int(fc.sum()),
           ties=int((flags & 1).sum()), obar_uncertified=n_unc, obar_uncertified_differing=n_diff,
           **errs)


SHAPES = [  # B, Hq, Hkv, N, d, causal
    (1, 1, 1, 1, 64, True), (1, 2, 1, 63, 64, True), (2, 4, 2, 65, 64, False),
    (1, 2, 2, 200, 64, True), (1, 4, 1, 257, 128, True), (2, 2, 1, 129, 128, False),
    (1, 1, 1, 384, 64, False), (1, 8, 2, 96, 128, True),
    # groups of 8 query heads on a KV head
    (1, 8, 1, 160, 64, True), (2, 16, 2, 100, 128, False),
    # past the 512-key rounding point of the streaming bf16 Ō (rounded after
    # keys 512 and 1024 and at the row's end)
    (1, 2, 1, 1100, 64, True), (1, 2, 2, 1100, 128, False), (1, 1, 1, 1537, 64, False),
    (1, 2, 1, 1537, 128, True),
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("guard", ["none", "beta", "eps"])
def test_ragged_and_grouped(shape, guard):
    B, Hq, Hkv, N, d, causal = shape
    wl = W.Workload("ragged", B, Hq, Hkv, N, d, causal, 1.0, 1.0, "const", -0.3,
                    4.0 if N > 2 else 0.0, 0.1, 0.0, 16.0, 77)
    x = W.make_custom(wl)
    p = problem(wl, guard)
    e = orc.fwd_emu(p, schedule(p), x["q"], x["k"], x["v"], nthreads=threads())
    o64, _ = orc.fwd_f64(p, x["q"], x["k"], x["v"], nthreads=threads())
    r = _run_fwd(x, guard)
    flags = r["row_flags"].cpu().numpy()
    fc = e["flag_cert"].astype(bool)
    assert np.array_equal(flags[fc], e["flags"][fc])
    errs = check_o(f32(r["o"]), o64, e["o"], False)
    ob_gpu = bits(r["obar"])
    ob_emu = orc.bf16_from_f32(e["obar"].astype(np.float32))
    cert = e["obar_cert"].astype(bool)
    assert np.array_equal(ob_gpu[cert], ob_emu[cert])
    report(f"ragged {shape} {guard}", ties=int((flags & 1).sum()), cert=f"{cert.mean():.3f}", **errs)


@pytest.mark.parametrize("name,guard,beta,heads", [
    ("gpt2s", "beta", 2.0, [0, 77, 191]), ("gpt2s", "none", 2.0, [5, 100]),
    ("gpt2m", "beta", 2.0, [0, 127]), ("llama8b", "beta", 2.0, [0, 13]),
    ("llama8b", "none", 2.0, [1, 30]),
    ("stress", "beta", 2.0, [0]), ("stress", "beta", 8.0, [31]), ("stress", "eps", 2.0, [7]),
])
def test_full_size_sampled(name, guard, beta, heads):
    """At the full workload sizes, in the launch configuration the benchmark
    times: O of sampled heads against FP64 (and against the emulated method),
    NaN rows (zero denominators, rescale overflow) where the emulation
    predicts them, tie flags of the sampled heads (all heads for the GPT-2
    shapes) against the oracle's certified row statistics."""
    x = make(name)
    wl = x["workload"]
    p = problem(wl, guard, beta=beta)
    r = _run_fwd(x, guard, beta=beta)
    shp = (-1, wl.seqlen, wl.head_dim)
    o_gpu = f32(r["o"]).reshape(shp)[heads]
    o64 = orc.fwd_f64(p, x["q"], x["k"], x["v"], heads=heads, nthreads=threads())[0].reshape(shp)[heads]
    e = orc.fwd_emu(p, schedule(p, certify=False), x["q"], x["k"], x["v"], heads=heads,
                    nthreads=threads())
    o_emu = e["o"].reshape(shp)[heads]
    flags = r["row_flags"].cpu().numpy().reshape(-1, wl.seqlen)
    nan_emu = np.isnan(o_emu).any(-1)
    nan_gpu = np.isnan(o_gpu).any(-1)
    assert np.array_equal(nan_gpu, nan_emu)
    zd_emu = (e["flags"].reshape(-1, wl.seqlen)[heads] & 2) != 0
    assert np.array_equal((flags[heads] & 2) != 0, zd_emu)
    errs = check_o(o_gpu, o64, o_emu, False, rows=~nan_emu)
    flag_heads = None if name in ("gpt2s", "gpt2m") else heads
    st = orc.row_stats(p, x["q"], x["k"], schedule(p), heads=flag_heads, nthreads=threads())
    sel = slice(None) if flag_heads is None else heads
    fst = st["flags"].reshape(-1, wl.seqlen)[sel]
    fc = st["flag_cert"].reshape(-1, wl.seqlen)[sel].astype(bool)
    tie_gpu = flags[sel] & 1
    assert np.array_equal(tie_gpu[fc], (fst & 1)[fc])
    report(f"{name} {guard} beta={beta}", tie_rate=f"{tie_gpu.mean():.4f}",
           flag_uncertified=int((~fc).sum()), zero_denom=int(zd_emu.sum()), nan_rows=int(nan_emu.sum()),
           **errs)


def test_repeat_is_deterministic():
    x = make("gpt2s")
    a = _run_fwd(x, "beta")
    b = _run_fwd(x, "beta")
    for key in ("o", "row_m", "row_l", "row_flags", "obar"):
        assert torch.equal(a[key], b[key]), key


# ---- the other rounding schedules: FA2 as tensor operations (512-key
# blocks, bf16 block product; [R] "Points to doubt") and no tiling (one
# block a row; [S] "Key claims"), against the oracle replaying the schedule
# that attn_schedule reports for them

SCHED_CASES = [  # name, shape (B, Hq, Hkv, N, d, causal) for the ragged ones
    ("tiny", None), ("ragged", (1, 2, 1, 1100, 64, True)), ("ragged", (2, 4, 2, 600, 128, False)),
    ("ragged", (1, 1, 1, 1, 64, True)),
]


@pytest.mark.parametrize("sched", ["fa2_ops", "untiled"])
@pytest.mark.parametrize("guard", ["none", "beta", "eps"])
@pytest.mark.parametrize("name,shape", SCHED_CASES)
def test_other_schedules_bit_exact(sched, guard, name, shape):
    if name == "ragged":
        B, Hq, Hkv, N, d, causal = shape
        wl = W.Workload("ragged", B, Hq, Hkv, N, d, causal, 1.0, 1.0, "const", -0.3,
                        4.0 if N > 2 else 0.0, 0.1, 0.0, 16.0, 81)
        x = W.make_custom(wl)
    else:
        x = make(name)
        wl = x["workload"]
    p = problem(wl, guard)
    sc = schedule(p, sched=sched)
    e = orc.fwd_emu(p, sc, x["q"], x["k"], x["v"], nthreads=threads())
    o64, _ = orc.fwd_f64(p, x["q"], x["k"], x["v"], nthreads=threads())
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    r = fa.attn_fwd(q, k, v, causal=wl.causal, guard=guard, schedule=sched, return_obar=True,
                    return_row_max=True)
    torch.cuda.synchronize()
    flags = r["row_flags"].cpu().numpy()
    fc = e["flag_cert"].astype(bool)
    assert np.array_equal(flags[fc], e["flags"][fc])
    errs = check_o(f32(r["o"]), o64, e["o"], False)
    assert np.allclose(r["row_m"].cpu().numpy()[fc], e["m"][fc], rtol=1e-6, atol=1e-6)
    ob_gpu = bits(r["obar"])
    ob_emu = orc.bf16_from_f32(e["obar"].astype(np.float32))
    cert = e["obar_cert"].astype(bool)
    assert np.array_equal(ob_gpu[cert], ob_emu[cert])
    rows = np.broadcast_to(fc[..., None], cert.shape)
    unc = ~cert & rows
    # uncertified elements: distance in bf16 steps at the larger magnitude
    a_, b_ = f32(r["obar"])[unc].astype(np.float64), e["obar"][unc]
    steps = np.abs(a_ - b_) / np.array([orc.bf16_ulp(max(abs(u), abs(w))) for u, w in zip(a_, b_)] or [1.0])
    if name == "tiny":  # one block: one (double) rounding apart at most
        assert np.all(steps <= 1.0 + 1e-9)
    report(f"schedule {sched} {name} {shape or ''} {guard}", ties=int((flags & 1).sum()),
           cert=f"{cert.mean():.3f}", uncertified_differing=int((ob_gpu[unc] != ob_emu[unc]).sum()),
           max_steps=f"{steps.max() if steps.size else 0:.0f}", **errs)


@pytest.mark.parametrize("sched", ["fa2_ops", "untiled"])
def test_other_schedules_full_size(sched):
    """GPT-2 Small, sampled heads: O against FP64 and the replayed schedule."""
    x = make("gpt2s")
    wl = x["workload"]
    p = problem(wl, "beta")
    heads = [1, 150]
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    r = fa.attn_fwd(q, k, v, causal=True, guard="beta", schedule=sched, return_obar=True)
    torch.cuda.synchronize()
    shp = (-1, wl.seqlen, wl.head_dim)
    e = orc.fwd_emu(p, schedule(p, sched=sched), x["q"], x["k"], x["v"], heads=heads,
                    nthreads=threads())
    o64 = orc.fwd_f64(p, x["q"], x["k"], x["v"], heads=heads, nthreads=threads())[0].reshape(shp)[heads]
    errs = check_o(f32(r["o"]).reshape(shp)[heads], o64, e["o"].reshape(shp)[heads], False)
    cert = e["obar_cert"].reshape(shp)[heads].astype(bool)
    ob_gpu = bits(r["obar"]).reshape(shp)[heads]
    ob_emu = orc.bf16_from_f32(e["obar"].astype(np.float32)).reshape(shp)[heads]
    assert np.array_equal(ob_gpu[cert], ob_emu[cert])
    report(f"schedule {sched} gpt2s beta", cert=f"{cert.mean():.3f}", **errs)


@pytest.mark.parametrize("obar_fp32", [True, False])
def test_output_is_the_ieee_quotient(obar_fp32):
    """O = bf16(fl32(Ō/ℓ)) bit for bit, from the kernel's own Ō (fp32 or bf16)
    and ℓ, with numpy's IEEE fp32 division: the epilogue's reciprocal-based
    quotient must equal it on every row (GPT-2 Small, every head)."""
    x = make("gpt2s")
    wl = x["workload"]
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    r = fa.attn_fwd(q, k, v, causal=True, guard="beta", obar_fp32=obar_fp32, return_obar=True)
    torch.cuda.synchronize()
    ob = f32(r["obar"]).astype(np.float32)
    l = r["row_l"].cpu().numpy().astype(np.float32)[..., None]
    want = orc.bf16_from_f32(np.ascontiguousarray(ob / l, dtype=np.float32))
    got = bits(r["o"])
    assert np.array_equal(got, want), int((got != want).sum())
    report(f"O = bf16(Ō/ℓ) {'fp32' if obar_fp32 else 'bf16'} Ō", elements=got.size)


def test_binding_rejects_mismatched_outputs():
    """Output and statistics tensors of the wrong shape or dtype are refused
    before the library is called (it would write past them)."""
    q = torch.zeros((1, 2, 64, 64), dtype=torch.bfloat16, device="cuda")
    r = fa.attn_fwd(q, q, q)
    bad = dict(r)
    bad["row_m"] = torch.empty((1, 2, 32), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        fa.attn_fwd(q, q, q, out=bad)
    with pytest.raises(TypeError):
        fa.attn_bwd(q, q, q, r["o"], q, r["row_m"].double(), r["row_l"])
    with pytest.raises(ValueError):
        fa.attn_bwd(q, q[:, :1].contiguous(), q, r["o"], q, r["row_m"], r["row_l"])
    with pytest.raises(ValueError):
        fa.attn_bwd(q, q, q, r["o"], q, r["row_m"][:, :1].contiguous(), r["row_l"])


@pytest.mark.parametrize("guard", ["none", "beta"])
def test_gpt2m_fp32_obar_every_head(guard):
    """GPT-2 Medium at full size with Ō kept in fp32 (the fix the pages
    report: [S] "Key claims", the QK-Guard abstract): O of every head against
    FP64 within the stated tolerances (max rel 1e-2, mean rel 2e-3), and the
    bf16-Ō run beside it for comparison."""
    x = make("gpt2m")
    wl = x["workload"]
    p = problem(wl, guard)
    o64, _ = orc.fwd_f64(p, x["q"], x["k"], x["v"], nthreads=threads())
    r32 = _run_fwd(x, guard, obar_fp32=True)
    mx, mean = rel_errors(f32(r32["o"]), o64)
    assert mx <= 1e-2 and mean <= 2e-3, (mx, mean)
    r16 = _run_fwd(x, guard, obar_fp32=False)
    mx16, mean16 = rel_errors(f32(r16["o"]), o64)
    report(f"gpt2m every head {guard}", fp32_obar=f"{mx:.2e}/{mean:.2e}", bf16_obar=f"{mx16:.2e}/{mean16:.2e}")

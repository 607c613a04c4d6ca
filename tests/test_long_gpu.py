"""Parity at sequence lengths past every configuration: N = 32768 at d = 64
(causal, β guard) and N = 16384 at d = 128 (non-causal, unguarded), one
batch, two query heads sharing one KV head.  These lengths take the
kernels' row offsets, their step loops and the forward's Ō rounding
schedule (every 512 keys) far past the configured shapes.

Checked: the tie flag of every row the oracle's row statistics certify,
bit for bit; O, δ and dQ of sampled rows against the FP64 single-row
backward (within the bounds the method's rounding points permit, from the
oracle's replay of those rows) and their zero-denominator bit against the
oracle's streaming emulation; O of the same rows with the fp32 Ō
accumulator against the stated bounds as written (at N = 16384 the bf16
roundings of Ō alone take the method past the stated max of 1e-2); and
Σ_j dV_j = Σ_i dO_i over the KV head, an exact identity (each row of P sums
to one) that covers every key's dV."""
import numpy as np
import pytest
import torch

import flashattention_fa_fwd_amd as fa
import oracle as orc
from flashattention_fa_fwd_amd import workloads as W

from _util import check_o, dev, f32, problem, rel_errors, report, schedule, threads
from test_bwd_gpu import _check

pytestmark = pytest.mark.gpu

CASES = [(64, True, 32768, "beta"), (128, False, 16384, "none")]


@pytest.mark.parametrize("d,causal,N,guard", CASES, ids=["d64-causal-32768", "d128-full-16384"])
def test_long_sequence(d, causal, N, guard):
    # Q, K ~ N(0,1), V ~ N(-0.3,1), a +6 sink on key 0, 2 % of rows with a
    # planted repeated maximum lifted 8 logits (the Llama-3.1-8B recipe)
    wl = W.Workload(f"long{d}", 1, 2, 1, N, d, causal, 1.0, 1.0, "const", -0.3, 6.0, 0.02, 0.0, 8.0,
                    7000 + d)
    x = W.make_custom(wl)
    p = problem(wl, guard)
    q, k, v, do = dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["do"])
    print(f"[long] N={N} d={d} causal={causal} guard={guard}", flush=True)
    f = fa.attn_fwd(q, k, v, causal=causal, guard=guard)
    b = fa.attn_bwd(q, k, v, f["o"], do, f["row_m"], f["row_l"], causal=causal, guard=guard)
    torch.cuda.synchronize()
    flags = f["row_flags"].cpu().numpy().reshape(-1, N)

    # tie flags of every certified row
    st = orc.row_stats(p, x["q"], x["k"], schedule(p), nthreads=threads())
    fc = st["flag_cert"].reshape(-1, N).astype(bool)
    fst = st["flags"].reshape(-1, N)
    assert fc.mean() > 0.999
    assert np.array_equal((flags & 1)[fc], (fst & 1)[fc])

    # sampled rows: O, delta, dQ against FP64; zero-denominator bit
    rng = np.random.default_rng(11)
    rows = np.concatenate([rng.integers(0, N, 32), [0, 1, 511, 512, 8191, N // 2, N - 2, N - 1]])
    qh = rng.integers(0, wl.heads_q, rows.size)
    ref = orc.bwd_rows_f64(p, x["q"], x["k"], x["v"], x["do"], qh, rows, nthreads=threads())
    em = orc.fwd_emu_rows(p, schedule(p, certify=False), x["q"], x["k"], x["v"], qh, rows,
                          nthreads=threads())
    rep = orc.bwd_rows_emu(p, x["q"], x["k"], x["v"], x["do"], qh, rows, o_in=em["o"],
                           round_ops=True, nthreads=threads())
    assert np.array_equal(flags[qh, rows] & 2, em["flags"] & 2)
    shp = (-1, N, d)
    out = check_o(f32(f["o"]).reshape(shp)[qh, rows], ref["o"], em["o"], False)
    out.update(_check("dq", f32(b["dq"]).reshape(shp)[qh, rows], ref["dq"],
                      rel_errors(rep["dq"], ref["dq"])))
    de = b["delta"].cpu().numpy().reshape(-1, N)[qh, rows]
    out.update(_check("delta", de, ref["delta"], rel_errors(rep["delta"], ref["delta"])))

    # fp32 Ō (no rounding of the running sum): the stated bounds as written
    f32o = fa.attn_fwd(q, k, v, causal=causal, guard=guard, obar_fp32=True)
    torch.cuda.synchronize()
    o32 = check_o(f32(f32o["o"]).reshape(shp)[qh, rows], ref["o"], None, True)
    out.update({"fp32_" + key: val for key, val in o32.items() if key.startswith("o_")})

    # every key's dV through sum_j dV_j = sum_i dO_i
    dv = f32(b["dv"]).astype(np.float64).reshape(N, d).sum(0)
    dos = W.bits_to_f32(x["do"]).astype(np.float64).reshape(-1, d).sum(0)
    out.update(_check("sum_dv", dv, dos))
    report(f"long N={N} d={d} {'causal' if causal else 'full'} {guard}",
           tie_rows=int((flags & 1).sum()), flag_uncertified=int((~fc).sum()), **out)

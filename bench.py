"""Benchmark: guarded BF16 attention forward+backward at the GPT-2 Small
attention shape (B=16, H=12, N=1024, d=64, causal, beta = 2 guard, bf16 Ō)
on one MI355X.

One step = attn_fwd + attn_bwd (every stage of the path) over one batch of
synthetic inputs that are resident in device memory before timing starts.
The headline value is measured with cold caches (a 1 GiB buffer written
before each timed step, outside the timed region); the warm, back-to-back
figure is reported beside it.  Inside the timed steps the backward is
called as its two stages (the work of attn_bwd), so that HIP events between
the launches time each kernel there; the roofline object uses the longest
kernel's mean duration over those steps.  Prints one JSON line (see the keys
below).  The CPU oracle's FP64 forward+backward of the same workload is timed
on the host as a baseline.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload gpt2s]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X published dense bf16 matrix peak
HBM_PEAK_GBS = 8000.0

# HBM traffic of a kernel per launch, from two rocprofv3 --pmc passes over
# `bench.py --steps 3 --warmup 1 --no-cpu-baseline --copy-calibration`
# (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled by what the
# counter reads for a plain device copy of 256 MiB (FETCH_SIZE reads half the
# bytes: x2.0; WRITE_SIZE all of them: x1.0).  Summary and commands:
# profiles/bwd_dkdv_gpt2s_hbm_traffic.md.  The figures hold only for the
# sources of that kernel they were taken on (SHA-256 over the files that
# define it and the build script that sets its compiler flags) and for the
# workload they were taken on; otherwise the report says null.
KERNEL_SOURCES = {"bwd_dkdv": ("attn_bwd_dkdv.hip", "attn_bwd_common.h", "attn_device.h", "attn_internal.h",
                               "../build_lib.py")}
MEASURED_TRAFFIC = {
    "bwd_dkdv": {
        "workload": "gpt2s",
        "sources_sha256": "b0c728845f4f53e0c53359e1be3bea77e8b317f2184290bdead1477d8ab2cc1b",
        "fetch_kib": 64566.5, "write_kib": 49780.75, "fetch_scale": 2.0, "write_scale": 1.0,
    },
}


def kernel_sources_sha256(kernel: str) -> str:
    import hashlib
    csrc = os.path.join(ROOT, "flashattention_fa_fwd_amd", "csrc")
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        h.update(f.encode())
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel: str, workload: str):
    m = MEASURED_TRAFFIC.get(kernel)
    if m is None or m["workload"] != workload or m["sources_sha256"] != kernel_sources_sha256(kernel):
        return None
    return int(1024 * (m["fetch_kib"] * m["fetch_scale"] + m["write_kib"] * m["write_scale"]))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gpt2s")
    ap.add_argument("--guard", default="beta", choices=["none", "beta", "eps"])
    ap.add_argument("--obar-fp32", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=0,
                    help="KV heads in the CPU oracle's sample (0: every head of the workload)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain device copy of known size (for counter scaling)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the attention path runs on one GPU (no cross-GPU sharding is implemented); --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import flashattention_fa_fwd_amd as fa
    from flashattention_fa_fwd_amd import workloads as W

    fa.lib()  # fails loudly when the HIP library is not built
    x = W.make(args.workload)
    wl = x["workload"]
    dev = "cuda"

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v, do = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), to_dev(x["do"])
    kw = dict(causal=wl.causal, guard=args.guard)
    p = fa.make_params(wl.batch, wl.heads_q, wl.heads_kv, wl.seqlen, wl.head_dim,
                       obar_fp32=args.obar_fp32, **kw)
    fout, bout = {}, {}
    fa.attn_fwd(q, k, v, obar_fp32=args.obar_fp32, out=fout, **kw)
    fa.attn_bwd(q, k, v, fout["o"], do, fout["row_m"], fout["row_l"], out=bout, **kw)
    torch.cuda.synchronize()

    def step():
        fa.attn_fwd(q, k, v, obar_fp32=args.obar_fp32, out=fout, **kw)
        fa.attn_bwd(q, k, v, fout["o"], do, fout["row_m"], fout["row_l"], out=bout, **kw)

    stream = torch.cuda.current_stream()

    def timed(fn, iters, warm):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(iters):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters  # ms

    # ---- the timed region: exactly K steps with cold caches.  Before each
    # step a 1 GiB buffer is written (more than the 8 XCDs' L2 and the
    # last-level cache hold together), so every step reads its inputs from
    # HBM; HIP events on the launch stream bracket the step alone (the fill
    # is outside them).  W untimed warm-up steps first; synchronised on both
    # sides.  ms_per_step = mean over the K steps.  The backward is called as
    # its two stages (the work of attn_bwd: dQ, then dK/dV) so that events
    # between the launches give each kernel's duration inside the step.
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    delta = bout["delta"]
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.steps):
        flush.fill_(i & 0xFF)
        evs[i][0].record(stream)
        fa.attn_fwd(q, k, v, obar_fp32=args.obar_fp32, out=fout, **kw)
        evs[i][1].record(stream)
        fa.attn_bwd_dq(p, q, k, v, fout["o"], do, fout["row_m"], fout["row_l"], bout["dq"], delta)
        evs[i][2].record(stream)
        fa.attn_bwd_dkdv(p, q, k, v, do, fout["row_m"], fout["row_l"], delta, bout["dk"], bout["dv"])
        evs[i][3].record(stream)
    torch.cuda.synchronize()
    cold_steps = [e[0].elapsed_time(e[3]) for e in evs]
    ms_step = float(np.mean(cold_steps))
    cold_fwd = float(np.median([e[0].elapsed_time(e[1]) for e in evs]))
    cold_bwd = float(np.median([e[1].elapsed_time(e[3]) for e in evs]))
    # each kernel's mean duration over the timed steps
    in_step = {"attn_fwd": float(np.mean([e[0].elapsed_time(e[1]) for e in evs])),
               "bwd_dq": float(np.mean([e[1].elapsed_time(e[2]) for e in evs])),
               "bwd_dkdv": float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))}
    del flush
    print(f"[bench] {args.steps} cold steps: mean {ms_step:.4f} ms/step (median {np.median(cold_steps):.4f}); "
          f"fwd {cold_fwd:.4f}, bwd {cold_bwd:.4f} ms (medians)", file=sys.stderr, flush=True)
    # the warm figure beside it: K steps back to back (inputs may stay in the
    # last-level cache from one step to the next)
    ms_warm = timed(step, args.steps, 3)
    print(f"[bench] {args.steps} warm steps back to back: {ms_warm:.4f} ms/step", file=sys.stderr, flush=True)
    # the kernel's own per-row flags of the timed workload
    fl = fout["row_flags"]
    flag_counts = {"rows": int(fl.numel()), "tie_rows": int(((fl & 1) != 0).sum().item()),
                   "zero_denominator_rows": int(((fl & 2) != 0).sum().item()),
                   "guard_applied_rows": int(((fl & 4) != 0).sum().item())}

    # ---- per-kernel durations beside them: each of the step's launches
    # repeated back to back between HIP events on the launch stream (the
    # clock under one kernel repeated differs from the mix of the step)
    n_rep = max(20, args.steps)
    ms_fwd = timed(lambda: fa.attn_fwd(q, k, v, obar_fp32=args.obar_fp32, out=fout, **kw), n_rep, 3)
    ms_dq = timed(lambda: fa.attn_bwd_dq(p, q, k, v, fout["o"], do, fout["row_m"], fout["row_l"],
                                         bout["dq"], delta), n_rep, 3)
    ms_dkdv = timed(lambda: fa.attn_bwd_dkdv(p, q, k, v, do, fout["row_m"], fout["row_l"], delta,
                                             bout["dk"], bout["dv"]), n_rep, 3)
    other = "none" if args.guard != "none" else "beta"
    fo2 = {}
    ms_fwd_other = timed(lambda: fa.attn_fwd(q, k, v, causal=wl.causal, guard=other, out=fo2), n_rep, 3)
    # the backward with delta = rowsum(dP∘P) (a first sweep over the keys in
    # the dQ kernel instead of rowsum(dO∘O)): its cost next to the default
    bo2 = {}
    ms_bwd_dp = timed(lambda: fa.attn_bwd(q, k, v, None, do, fout["row_m"], fout["row_l"],
                                          delta="dp_p", out=bo2, **kw), n_rep, 3)
    # the forward's study variants at the same shape: the FP8 product (row
    # or fixed operand scale), the MXFP4 product and the two other rounding
    # schedules
    variants = {}
    for name, vkw in (("pv_fp8_row", dict(pv_fp8="row")), ("pv_fp8_fixed", dict(pv_fp8="fixed")),
                      ("pv_mxfp4", dict(pv_mxfp4=True)),
                      ("sched_fa2_ops", dict(schedule="fa2_ops")), ("sched_untiled", dict(schedule="untiled"))):
        fo3 = {}
        variants[name] = round(timed(lambda: fa.attn_fwd(q, k, v, obar_fp32=args.obar_fp32, out=fo3, **vkw, **kw),
                                     n_rep, 3), 5)
    print(f"[bench] forward variants (ms): {variants}", file=sys.stderr, flush=True)
    print(f"[bench] in the timed steps (mean): fwd {in_step['attn_fwd']:.4f} ms, bwd_dq {in_step['bwd_dq']:.4f}, "
          f"bwd_dkdv {in_step['bwd_dkdv']:.4f}", file=sys.stderr, flush=True)
    print(f"[bench] back to back: fwd {ms_fwd:.4f} ms, bwd_dq {ms_dq:.4f}, bwd_dkdv {ms_dkdv:.4f}; "
          f"fwd with guard={other}: {ms_fwd_other:.4f}; bwd with delta=rowsum(dP*P): "
          f"{ms_bwd_dp:.4f}", file=sys.stderr, flush=True)

    if args.copy_calibration:
        src = torch.empty(256 * 1024 * 1024, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()

    # Algorithmic matrix flops (causal: the visible half): the forward's two
    # products (S = Q K^T, O = P V); the backward's five (S recomputed once,
    # dP, dV, dK, dQ).  Per kernel, the products it performs: bwd_dkdv S, dP,
    # dV, dK; bwd_dq S, dP, dQ (S and dP are recomputed by both kernels).
    fl_fwd = wl.flops_fwd()
    fl_gemm = fl_fwd / 2          # one [N x N x d] product
    fl_bwd = 5 * fl_gemm
    fl_step = fl_fwd + fl_bwd
    value = fl_step / (ms_step * 1e-3) / 1e12
    # the roofline kernel: the longest of the step's kernels, at its mean
    # duration inside the timed steps
    kernels = {
        "attn_fwd": (in_step["attn_fwd"], fl_fwd),
        "bwd_dkdv": (in_step["bwd_dkdv"], 4 * fl_gemm),
        "bwd_dq": (in_step["bwd_dq"], 3 * fl_gemm),
    }
    dom = max(kernels, key=lambda n: kernels[n][0])
    dms, dfl = kernels[dom]
    achieved = dfl / (dms * 1e-3) / 1e12
    rec = {
        "metric": "attn fwd+bwd TFLOP/s (BF16, guarded) at GPT-2 shape; % of MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": wl.description,
            "batch": wl.batch, "heads_q": wl.heads_q, "heads_kv": wl.heads_kv,
            "seq_len": wl.seqlen, "head_dim": wl.head_dim, "causal": wl.causal,
            "guard": args.guard, "beta": 2.0, "obar": "fp32" if args.obar_fp32 else "bf16",
            "flops_per_step": fl_step,
        },
        "pct_of_mfma_peak": round(100.0 * value / MFMA_BF16_PEAK_TFLOPS, 2),
        "fwd_tflops": round(fl_fwd / (in_step["attn_fwd"] * 1e-3) / 1e12, 2),
        "bwd_tflops": round(fl_bwd / ((in_step["bwd_dkdv"] + in_step["bwd_dq"]) * 1e-3) / 1e12, 2),
        "kernel_ms": {n: round(t, 5) for n, t in in_step.items()},
        "kernel_ms_timing": "mean over the K timed steps, HIP events between the step's launches",
        "kernel_ms_back_to_back": {"attn_fwd": round(ms_fwd, 5), "bwd_dq": round(ms_dq, 5),
                                   "bwd_dkdv": round(ms_dkdv, 5)},
        "fwd_ms_other_guard": {other: round(ms_fwd_other, 5)},
        "fwd_ms_variants": variants,
        "bwd_ms_delta": {"rowsum(dO*O)": round(ms_dq + ms_dkdv, 5), "rowsum(dP*P)": round(ms_bwd_dp, 5)},
        "timing": "cold caches: a 1 GiB buffer written before each timed step, HIP events around the step only",
        "cold": {"fwd_ms_median": round(cold_fwd, 5), "bwd_ms_median": round(cold_bwd, 5),
                 "step_ms_median": round(float(np.median(cold_steps)), 5), "flush_bytes": 1 << 30},
        "warm": {"ms_per_step": round(ms_warm, 5), "tflops": round(fl_step / (ms_warm * 1e-3) / 1e12, 2),
                 "timing": "K steps back to back between two synchronisations"},
        "row_flags": flag_counts,
        "roofline": {
            "kernel": dom,
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": measured_traffic(dom, args.workload),  # HBM bytes per launch
        },
    }

    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(x, wl, args)
        rec["cpu_emulation"] = cpu_emulation(args)
    print(json.dumps(rec), flush=True)


def cpu_baseline(x, wl, args):
    """The FP64 oracle (forward+backward of softmax attention) on the same
    workload (or its first --cpu-heads KV heads) on the host threads one GPU
    may use (at most 16).  Scaled to TFLOP/s with the same counted work per
    head."""
    import oracle as orc

    # one GPU's share of a shared host is 16 threads, whatever
    # os.cpu_count() reports; the visible count is printed beside it
    nthreads = min(16, os.cpu_count() or 1)
    nkv = wl.batch * wl.heads_kv
    heads = list(range(min(args.cpu_heads, nkv) if args.cpu_heads > 0 else nkv))
    p = orc.Problem(wl.batch, wl.heads_q, wl.heads_kv, wl.seqlen, wl.head_dim, wl.causal,
                    {"none": 0, "beta": 1, "eps": 2}[args.guard])
    t0 = time.perf_counter()
    orc.bwd_f64(p, x["q"], x["k"], x["v"], x["do"], kv_heads=heads, nthreads=nthreads)
    dt = time.perf_counter() - t0
    g = wl.heads_q // wl.heads_kv
    frac = len(heads) * g / (wl.batch * wl.heads_q)
    flops = 3.5 * wl.flops_fwd() * frac
    return {
        "value": round(flops / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": min(nthreads, len(heads)),
        "host_cpus_visible": os.cpu_count(),
        "kind": "oracle",
        "sample": f"FP64 forward+backward of {len(heads)} of {wl.batch * wl.heads_kv} KV heads "
                  f"({len(heads) * g} query heads) of the {wl.name} workload, {dt:.2f} s wall",
    }


def cpu_emulation(args):
    """The oracle's bit-level BF16 replay of the forward (with its rounding
    certification) on the tiny workload, one thread: the cost of the check
    that the bit-exact tests rest on."""
    import oracle as orc
    import flashattention_fa_fwd_amd as fa
    from flashattention_fa_fwd_amd import workloads as W

    xt = W.make("tiny")
    wt = xt["workload"]
    p = orc.Problem(wt.batch, wt.heads_q, wt.heads_kv, wt.seqlen, wt.head_dim, wt.causal,
                    {"none": 0, "beta": 1, "eps": 2}[args.guard])
    s = fa.attn_schedule(fa.make_params(wt.batch, wt.heads_q, wt.heads_kv, wt.seqlen, wt.head_dim,
                                        causal=wt.causal))
    sc = orc.Schedule(block_n=s["block_n"], round_n=s["round_n"], obar_fp32=False, chunk=s["chunk"],
                      certify=True, block_bf16=bool(s["block_bf16"]))
    t0 = time.perf_counter()
    orc.fwd_emu(p, sc, xt["q"], xt["k"], xt["v"], nthreads=1)
    dt = time.perf_counter() - t0
    return {"seconds": round(dt, 4), "threads": 1, "kind": "oracle",
            "sample": f"certified BF16 replay of the forward, {wt.description}"}


if __name__ == "__main__":
    main()

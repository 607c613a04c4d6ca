"""Shared helpers of the GPU parity tests (the HIP path is called through the
C ABI via the binding; the expected values come from the CPU oracle)."""
import os

import numpy as np
import torch

import flashattention_fa_fwd_amd as fa
import oracle as orc
from flashattention_fa_fwd_amd import workloads as W

GUARD = {"none": orc.GUARD_NONE, "beta": orc.GUARD_BETA, "eps": orc.GUARD_EPS}
# tolerances the target states for O, delta, dQ, dK, dV against FP64
MAX_REL, MEAN_REL = 1e-2, 2e-3
# In bf16-Ō mode the method itself rounds the numerator to bf16 (on top of
# the bf16 P̄ operand and the bf16 output); that floor is computed by the
# oracle's emulation of the same schedule and the kernel may add at most
# this much on top of it.
MEAN_EXCESS = 2e-4


_CACHE = {}


def make(name, **kw):
    """Seeded workload, generated once per test process."""
    key = (name, tuple(sorted(kw.items())))
    if key not in _CACHE:
        _CACHE[key] = W.make(name, **kw)
    return _CACHE[key]


def threads():
    return min(16, os.cpu_count() or 1)


def dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda")


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def f32(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return W.bits_to_f32(bits(t))
    return t.detach().cpu().float().numpy()


def rel_errors(x, ref, mask=None):
    """Normwise relative errors: max|x-ref|/max|ref| and mean|x-ref|/mean|ref|."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    if mask is not None:
        x, ref = x[mask], ref[mask]
    d = np.abs(x - ref)
    return float(d.max() / max(np.abs(ref).max(), 1e-300)), float(d.mean() / max(np.abs(ref).mean(), 1e-300))


def problem(wl_or_shape, guard="beta", beta=2.0, causal=None):
    if isinstance(wl_or_shape, W.Workload):
        w = wl_or_shape
        return orc.Problem(w.batch, w.heads_q, w.heads_kv, w.seqlen, w.head_dim,
                           w.causal if causal is None else causal, GUARD[guard], beta=beta)
    B, Hq, Hkv, N, d, c = wl_or_shape
    return orc.Problem(B, Hq, Hkv, N, d, c, GUARD[guard], beta=beta)


def schedule(p: orc.Problem, obar_fp32=False, certify=True, sched="stream", pv_fp8=False,
             pv_mxfp4=False) -> orc.Schedule:
    """The oracle replays the rounding schedule the library reports."""
    fp = fa.make_params(p.batch, p.heads_q, p.heads_kv, p.seqlen, p.head_dim, causal=p.causal,
                        schedule=sched, pv_fp8=pv_fp8, pv_mxfp4=pv_mxfp4)
    s = fa.attn_schedule(fp)
    return orc.Schedule(block_n=s["block_n"], round_n=s["round_n"], obar_fp32=obar_fp32,
                        chunk=s["chunk"], certify=certify, block_bf16=bool(s["block_bf16"]),
                        pv_fp8=pv_fp8, pv_mxfp4=pv_mxfp4, pv_chunk=s["pv_chunk"])


def check_o(o_gpu, o64, o_emu=None, obar_fp32=True, rows=None):
    """O against FP64: max rel <= 1e-2 and mean rel <= 2e-3.  In bf16-Ō mode
    the method's own roundings of Ō (one per 512 keys and one at the row's
    end) set a floor, taken from the emulation of those roundings on the same
    rows: the bounds are max(1e-2, 1.25 x the emulation's max) and max(2e-3,
    the emulation's mean + 2e-4).  The max floor binds only on long rows
    (N = 16384: about 1.1e-2).  Returns the numbers for the report."""
    sel = (slice(None),) if rows is None else (rows,)
    mx, mean = rel_errors(o_gpu[sel], o64[sel])
    emx = emean = float("nan")
    bound, bmax = MEAN_REL, MAX_REL
    if o_emu is not None:
        emx, emean = rel_errors(o_emu[sel], o64[sel])
        if not obar_fp32:
            bound = max(MEAN_REL, emean + MEAN_EXCESS)
            bmax = max(MAX_REL, 1.25 * emx)
    assert mx <= bmax, ("max rel", mx, "bound", bmax, "emulation", emx)
    assert mean <= bound, ("mean rel", mean, "bound", bound, "emulation", emean)
    return dict(o_max_rel=f"{mx:.2e}", o_mean_rel=f"{mean:.2e}", emu_max_rel=f"{emx:.2e}",
                emu_mean_rel=f"{emean:.2e}")


def report(tag, **kv):
    print(f"[parity] {tag}: " + " ".join(f"{k}={v}" for k, v in kv.items()), flush=True)

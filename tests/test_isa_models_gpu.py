"""The oracle's instruction models against the hardware itself: a test-only
probe (tests/probes/isa_probe.hip) runs v_mfma_f32_32x32x16_bf16 and
v_exp_f32 on chosen operands, and the oracle's bounds (chain_bound, the
exponential's relative error and its flush to zero below 2^-126) must cover
every returned value.  These are the models that decide which Ō elements the
parity tests claim bit-exact."""
import ctypes
import math
import os

import numpy as np
import pytest
import torch

import oracle as orc
from flashattention_fa_fwd_amd import workloads as W

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "probes", "libisa_probe.so")


@pytest.fixture(scope="module")
def probe():
    if not os.path.exists(LIB):
        raise FileNotFoundError(f"{LIB} is not built (tests/probes/build_probe.py)")
    L = ctypes.CDLL(LIB)
    L.probe_mfma_bf16.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int]
    L.probe_exp2.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
    L.probe_mfma_fp8.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int]
    L.probe_mfma_fp4.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_int]
    return L


def _bf16(x):
    return W.bits_to_f32(W.to_bf16_bits(np.asarray(x, np.float32))).astype(np.float64)


def _operands(rng, kind, n):
    if kind == "attention":   # P̄ = exp(-x) times V ~ N(mu, 1), C an Ō-like running sum
        a = _bf16(np.exp(-rng.uniform(0, 12, (n, 32, 16))))
        b = _bf16(rng.normal(rng.uniform(-1, 1, (n, 1, 32)), 1, (n, 16, 32)))
        c = rng.normal(0, 3, (n, 32, 32))
    elif kind == "scores":    # Q K^T pieces, C a partial score
        a = _bf16(rng.normal(0, 1.5, (n, 32, 16)))
        b = _bf16(rng.normal(0, 1.5, (n, 16, 32)))
        c = rng.normal(0, 8, (n, 32, 32))
    elif kind == "wide":      # exponents spread over 2^-20 .. 2^10, random signs
        a = _bf16(rng.choice([-1, 1], (n, 32, 16)) * 2.0 ** rng.uniform(-20, 10, (n, 32, 16)))
        b = _bf16(rng.choice([-1, 1], (n, 16, 32)) * 2.0 ** rng.uniform(-10, 5, (n, 16, 32)))
        c = rng.choice([0.0, 1.0], (n, 32, 32)) * rng.normal(0, 1e3, (n, 32, 32))
    else:                     # cancelling pairs along k plus a tiny residual in C
        a0 = _bf16(rng.normal(0, 1, (n, 32, 8)))
        a = np.concatenate([a0, -a0], axis=2)
        b0 = _bf16(rng.normal(0, 1, (n, 8, 32)))
        b = np.concatenate([b0, b0], axis=1)
        c = rng.normal(0, 1e-6, (n, 32, 32))
    return a, b, np.asarray(c, np.float32).astype(np.float64)


@pytest.mark.parametrize("kind", ["attention", "scores", "wide", "cancel"])
def test_bf16_matrix_instruction_within_the_oracle_bound(probe, orc, kind):
    rng = np.random.default_rng({"attention": 1, "scores": 2, "wide": 3, "cancel": 4}[kind])
    n = 96
    a, b, c = _operands(rng, kind, n)
    A = torch.from_numpy(W.to_bf16_bits(a.astype(np.float32)).view(np.int16)).cuda()
    B = torch.from_numpy(W.to_bf16_bits(b.astype(np.float32)).view(np.int16)).cuda()
    C = torch.from_numpy(c.astype(np.float32)).cuda()
    D = torch.empty_like(C)
    assert probe.probe_mfma_bf16(A.data_ptr(), B.data_ptr(), C.data_ptr(), D.data_ptr(), n) == 0
    torch.cuda.synchronize()
    d = D.cpu().numpy().astype(np.float64)
    sched = orc.Schedule(chunk=16, chunk_err=1.0)  # the bound without its safety factor
    worst, n_over = 0.0, 0
    for w in range(n):
        prods = a[w][:, None, :] * b[w].T[None, :, :]  # [m, n, k], exact
        for m in range(32):
            for col in range(32):
                terms = prods[m, col]
                exact = math.fsum([c[w, m, col], *terms])
                err = abs(d[w, m, col] - exact)
                bound = orc.chain_bound(sched, c[w, m, col], terms)
                if err > bound:
                    n_over += 1
                if bound > 0:
                    worst = max(worst, err / bound)
    print(f"[isa] bf16 mfma {kind}: worst error / bound = {worst:.3f}, over the bound: {n_over}")
    assert n_over == 0


def test_exp2_within_the_oracle_error_and_flush(probe):
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.uniform(-126, 0, 1 << 18), rng.uniform(-1, 1, 1 << 16),
                        rng.uniform(-140, -120, 1 << 14), rng.uniform(0, 60, 1 << 14)]).astype(np.float32)
    X = torch.from_numpy(x).cuda()
    Y = torch.empty_like(X)
    assert probe.probe_exp2(X.data_ptr(), Y.data_ptr(), x.size) == 0
    torch.cuda.synchronize()
    y = Y.cpu().numpy().astype(np.float64)
    ref = np.exp2(x.astype(np.float64))
    normal = ref >= 2.0 ** -126
    rel = np.abs(y[normal] - ref[normal]) / ref[normal]
    bound = orc.Schedule().exp_rel_err
    ulps = rel.max() / 2.0 ** -24
    print(f"[isa] exp2: max relative error {rel.max():.3e} ({ulps:.2f} half-ulps of 2^-23), bound {bound:.3e}")
    assert rel.max() <= bound
    # results that would be subnormal are flushed to zero (the oracle's ftz model)
    assert np.all(y[ref < 2.0 ** -126 * (1 - 2.0 ** -20)] == 0.0)


def _e4m3_bits(x):
    """E4M3 byte of each (already E4M3-valued) x, from the OCP layout."""
    x = np.asarray(x, np.float64)
    out = np.zeros(x.shape, np.uint8)
    s = (x < 0).astype(np.uint8) << 7
    ax = np.abs(x)
    nz = ax > 0
    e = np.floor(np.log2(np.where(nz, ax, 1.0))).astype(np.int64)
    sub = nz & (e < -6)
    norm = nz & ~sub
    mant_n = np.round((ax / np.exp2(e.astype(np.float64)) - 1.0) * 8).astype(np.int64)
    out[norm] = ((e[norm] + 7) << 3 | mant_n[norm]).astype(np.uint8)
    out[sub] = np.round(ax[sub] / 2.0 ** -9).astype(np.uint8)
    return out | s


def _e4m3_exp(x):
    _, e = np.frexp(np.where(x == 0, 1.0, np.abs(x)))
    return np.where(x == 0, 0, np.maximum(e - 1, -6))


@pytest.mark.parametrize("kind", ["attention", "normal", "subnormal"])
def test_fp8_matrix_instruction_within_the_oracle_bound(probe, orc, kind):
    """The 64-product scaled FP8 instruction (E4M3, unit scales) of the FP8
    P̄V variant against chain_bound_fp8 (without its safety factors)."""
    rng = np.random.default_rng({"attention": 7, "normal": 8, "subnormal": 9}[kind])
    n = 48
    if kind == "attention":
        a = orc.e4m3_array(np.exp(-rng.uniform(0, 6, (n, 32, 64))) * 2.0 ** 7)
        b = orc.e4m3_array(rng.normal(rng.uniform(-1, 1, (n, 1, 32)), 1, (n, 64, 32)))
        c = rng.normal(0, 300, (n, 32, 32))
    elif kind == "normal":
        a = orc.e4m3_array(rng.normal(0, 30, (n, 32, 64)))
        b = orc.e4m3_array(rng.normal(0, 2, (n, 64, 32)))
        c = rng.normal(0, 50, (n, 32, 32)) * 2.0 ** rng.integers(-8, 8, (n, 1, 1))
    else:
        a = orc.e4m3_array(rng.uniform(-1, 1, (n, 32, 64)) * 2.0 ** -6)
        b = orc.e4m3_array(rng.normal(0, 4, (n, 64, 32)))
        c = rng.normal(0, 1e-3, (n, 32, 32))
    c = c.astype(np.float32).astype(np.float64)
    A = torch.from_numpy(_e4m3_bits(a)).cuda()
    B = torch.from_numpy(_e4m3_bits(b)).cuda()
    # the byte layout decodes back to the same values (torch's E4M3 type)
    assert np.array_equal(A.view(torch.float8_e4m3fn).float().cpu().numpy().astype(np.float64), a)
    C = torch.from_numpy(c.astype(np.float32)).cuda()
    D = torch.empty_like(C)
    assert probe.probe_mfma_fp8(A.data_ptr(), B.data_ptr(), C.data_ptr(), D.data_ptr(), n) == 0
    torch.cuda.synchronize()
    d = D.cpu().numpy().astype(np.float64)
    sched = orc.Schedule(pv_chunk=64, chunk_err=0.5)  # the oracle doubles; 0.5 undoes that
    worst, n_over = 0.0, 0
    for w in range(n):
        prods = a[w][:, None, :] * b[w].T[None, :, :]
        es = (_e4m3_exp(a[w])[:, None, :] + _e4m3_exp(b[w]).T[None, :, :]).astype(np.int32)
        for m in range(32):
            for col in range(32):
                terms = prods[m, col]
                exact = math.fsum([c[w, m, col], *terms])
                err = abs(d[w, m, col] - exact)
                bound = orc.chain_bound_fp8(sched, c[w, m, col], terms, es[m, col], 0)
                n_over += err > bound
                if bound > 0:
                    worst = max(worst, err / bound)
    print(f"[isa] fp8 scaled mfma {kind}: worst error / bound = {worst:.3f}, over the bound: {n_over}")
    assert n_over == 0


E2M1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6])


@pytest.mark.parametrize("kind", ["unit", "attention", "wide"])
def test_fp4_matrix_instruction_within_the_oracle_bound(probe, orc, kind):
    """The scaled FP4 instruction of the MXFP4 variant (E2M1 codes, one E8M0
    scale per row / column and 32-element block) against chain_bound_mx
    (without its safety factor)."""
    rng = np.random.default_rng({"unit": 31, "attention": 32, "wide": 33}[kind])
    n = 48
    ca = rng.integers(0, 16, (n, 32, 64)).astype(np.uint8)
    cb = rng.integers(0, 16, (n, 64, 32)).astype(np.uint8)
    if kind == "unit":
        sa = np.full((n, 32, 2), 127, np.uint8); sb = np.full((n, 2, 32), 127, np.uint8)
        c = rng.normal(0, 50, (n, 32, 32))
    elif kind == "attention":   # P̄-like scales (2^-2 .. 2^-12) times V-like ones
        sa = rng.integers(115, 126, (n, 32, 2)).astype(np.uint8)
        sb = rng.integers(124, 128, (n, 2, 32)).astype(np.uint8)
        c = rng.normal(0, 1, (n, 32, 32))
    else:
        sa = rng.integers(100, 150, (n, 32, 2)).astype(np.uint8)
        sb = rng.integers(100, 150, (n, 2, 32)).astype(np.uint8)
        c = rng.normal(0, 1, (n, 32, 32)) * 2.0 ** rng.integers(-20, 20, (n, 1, 1))
    c = c.astype(np.float32).astype(np.float64)
    a = E2M1[ca] * np.exp2(np.repeat(sa.astype(np.float64) - 127, 32, axis=2))
    b = E2M1[cb] * np.exp2(np.repeat(sb.astype(np.float64) - 127, 32, axis=1))
    args = [torch.from_numpy(np.ascontiguousarray(t)).cuda() for t in (ca, cb, sa, sb)]
    C = torch.from_numpy(c.astype(np.float32)).cuda()
    D = torch.empty_like(C)
    assert probe.probe_mfma_fp4(*[t.data_ptr() for t in args], C.data_ptr(), D.data_ptr(), n) == 0
    torch.cuda.synchronize()
    d = D.cpu().numpy().astype(np.float64)
    sched = orc.Schedule(chunk_err=0.5)  # the oracle doubles; 0.5 undoes that
    worst, n_over = 0.0, 0
    for w in range(n):
        prods = a[w][:, None, :] * b[w].T[None, :, :]
        for m in range(32):
            for col in range(32):
                terms = prods[m, col]
                exact = math.fsum([c[w, m, col], *terms])
                err = abs(d[w, m, col] - exact)
                bound = orc.chain_bound_mx(sched, c[w, m, col], terms)
                n_over += err > bound
                if bound > 0:
                    worst = max(worst, err / bound)
    print(f"[isa] fp4 scaled mfma {kind}: worst error / bound = {worst:.3f}, over the bound: {n_over}")
    assert n_over == 0

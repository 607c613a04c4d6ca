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

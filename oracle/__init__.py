"""CPU oracle for guarded BF16 attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports it and shares no code with it.

This module is argument marshalling for ``liboracle.so`` (plain C, see
``oracle.h``).  Arrays are numpy; bf16 tensors travel as ``uint16`` bit
patterns in row-major [batch, heads, seqlen, head_dim] layout.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_LIB: another build of the same source (the sanitizer test builds
# one with AddressSanitizer / UndefinedBehaviorSanitizer)
_LIB_PATH = os.environ.get("ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

GUARD_NONE, GUARD_BETA, GUARD_EPS = 0, 1, 2
ROW_TIE, ROW_ZERO_DENOM, ROW_GUARD_APPLIED = 1, 2, 4
EX_PBAR_ONE_TIED, EX_ZERO_MAX_TIE, EX_SHIFT_DECREASED = 1, 2, 4
EX_RESCALE_OVERFLOW, EX_PBAR_ONE_PRE_TIE = 8, 16


class _Problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32),
        ("heads_kv", ctypes.c_int32), ("seqlen", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("causal", ctypes.c_int32),
        ("guard", ctypes.c_int32), ("alpha", ctypes.c_float),
        ("beta", ctypes.c_float), ("tie_eps", ctypes.c_float),
        ("shift_eps", ctypes.c_float),
    ]


_ORC_VERSION = 2  # the struct layouts below match oracle.h at this version


class _Schedule(ctypes.Structure):
    _fields_ = [
        ("block_n", ctypes.c_int32), ("round_n", ctypes.c_int32),
        ("obar_fp32", ctypes.c_int32), ("certify", ctypes.c_int32),
        ("ftz", ctypes.c_int32), ("chunk", ctypes.c_int32),
        ("chunk_err", ctypes.c_double), ("exp_rel_err", ctypes.c_double),
        ("block_bf16", ctypes.c_int32), ("pv_fp8", ctypes.c_int32), ("pv_mxfp4", ctypes.c_int32),
        ("pv_chunk", ctypes.c_int32),
    ]


@dataclass
class Problem:
    batch: int
    heads_q: int
    heads_kv: int
    seqlen: int
    head_dim: int
    causal: bool = True
    guard: int = GUARD_NONE
    alpha: float | None = None  # None: fl32(1/sqrt(head_dim))
    beta: float = 2.0
    tie_eps: float = 1e-3
    shift_eps: float = 2.0 ** -5

    def c(self) -> _Problem:
        a = self.alpha if self.alpha is not None else float(np.float32(1.0 / np.sqrt(self.head_dim)))
        return _Problem(self.batch, self.heads_q, self.heads_kv, self.seqlen,
                        self.head_dim, int(bool(self.causal)), int(self.guard),
                        a, self.beta, self.tie_eps, self.shift_eps)

    @property
    def q_rows(self) -> int:
        return self.batch * self.heads_q * self.seqlen


@dataclass
class Schedule:
    """Rounding points and error model of the kernel under test.

    block_n: keys per streaming step (tie decision and shift).
    round_n: bf16 mode rounds Ō after every round_n keys (0: block_n).
    certify: compute the certification (slow); False leaves every cert 0.
    ftz: the kernel's exp flushes results below 2^-126 to zero.
    chunk/chunk_err: sums run as chains of matrix instructions of `chunk`
    terms (error model in oracle.c, chain_bound), scaled by the safety factor
    chunk_err; chunk=0 falls back to the any-order fp32 bound.
    exp_rel_err: relative error bound of the kernel's exp.
    block_bf16: bf16 mode rounds each block's product sum to bf16 before it is
    added to Ō (FA2 as tensor operations; needs round_n == block_n).
    pv_fp8: the P̄V product in FP8 E4M3 (P̄ * 2^k and V rounded to E4M3):
        False, True / "row" (k per row and block: the row's largest P̄ in
        [128, 256)) or "fixed" (k = 8).
    pv_mxfp4: the P̄V product in MXFP4 (E2M1 elements, one E8M0 scale per 32
        consecutive keys: keys 0..31 and 32..63 of a 64-key step);
        True / "floor" (the OCP rule) or "ceil" (scale from ceil(log2 amax)).
    """
    block_n: int = 64
    round_n: int = 0
    obar_fp32: bool = False
    certify: bool = True
    ftz: bool = True
    chunk: int = 16
    chunk_err: float = 2.0
    exp_rel_err: float = 2.0 ** -22
    block_bf16: bool = False
    pv_fp8: bool | str = False
    pv_mxfp4: bool | str = False
    pv_chunk: int = 0

    def c(self) -> _Schedule:
        return _Schedule(self.block_n, self.round_n, int(bool(self.obar_fp32)),
                         int(bool(self.certify)), int(bool(self.ftz)),
                         self.chunk, self.chunk_err, self.exp_rel_err, int(bool(self.block_bf16)),
                         {False: 0, True: 1, "row": 1, "fixed": 2}[self.pv_fp8], {False: 0, True: 1, "floor": 1, "ceil": 2}[self.pv_mxfp4],
                         int(self.pv_chunk))


def build(verbose: bool = False) -> str:
    from .build_oracle import build as _build
    return _build(verbose)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.POINTER
        u16p, f32p, f64p = P(ctypes.c_uint16), P(ctypes.c_float), P(ctypes.c_double)
        u8p, i32p = P(ctypes.c_uint8), P(ctypes.c_int32)
        pp, sp = P(_Problem), P(_Schedule)
        L.orc_version.restype = ctypes.c_int
        if L.orc_version() != _ORC_VERSION:
            raise ImportError(f"{_LIB_PATH} is version {L.orc_version()}, this binding expects "
                              f"{_ORC_VERSION}: rebuild it (oracle.build())")
        L.orc_bf16_from_f32.argtypes = [ctypes.c_float]
        L.orc_bf16_from_f32.restype = ctypes.c_uint16
        L.orc_bf16_from_f64.argtypes = [ctypes.c_double]
        L.orc_bf16_from_f64.restype = ctypes.c_uint16
        L.orc_f32_from_bf16.argtypes = [ctypes.c_uint16]
        L.orc_f32_from_bf16.restype = ctypes.c_float
        L.orc_bf16_from_f32_array.argtypes = [f32p, u16p, ctypes.c_int64]
        L.orc_f32_from_bf16_array.argtypes = [u16p, f32p, ctypes.c_int64]
        L.orc_bf16_ulp.argtypes = [ctypes.c_double]
        L.orc_bf16_ulp.restype = ctypes.c_double
        L.orc_bf16_boundary_distance.argtypes = [ctypes.c_double]
        L.orc_bf16_boundary_distance.restype = ctypes.c_double
        L.orc_bf16_round_of_sum.argtypes = [f64p, ctypes.c_int32, f64p]
        L.orc_bf16_round_of_sum.restype = ctypes.c_uint16
        L.orc_fwd_f64.argtypes = [pp, u16p, u16p, u16p, i32p, ctypes.c_int32, f64p, f64p, ctypes.c_int32]
        L.orc_bwd_f64.argtypes = [pp, u16p, u16p, u16p, u16p, i32p, ctypes.c_int32,
                                  f64p, f64p, f64p, f64p, f64p, ctypes.c_int32]
        L.orc_bwd_rows_f64.argtypes = [pp, u16p, u16p, u16p, u16p, i32p, i32p, ctypes.c_int32,
                                       f64p, f64p, f64p, ctypes.c_int32]
        L.orc_bwd_emu.argtypes = [pp, u16p, u16p, u16p, u16p, i32p, ctypes.c_int32, f64p,
                                  ctypes.c_int32, f64p, f64p, f64p, f64p, ctypes.c_int32]
        L.orc_bwd_rows_emu.argtypes = [pp, u16p, u16p, u16p, u16p, i32p, i32p, ctypes.c_int32,
                                       f64p, ctypes.c_int32, f64p, f64p, ctypes.c_int32]
        for nm in ("orc_chain_bound", "orc_chain_bound_mx"):
            getattr(L, nm).argtypes = [ctypes.POINTER(_Schedule), ctypes.c_double, f64p, ctypes.c_int32]
            getattr(L, nm).restype = ctypes.c_double
        L.orc_chain_bound_fp8.argtypes = [ctypes.POINTER(_Schedule), ctypes.c_double, f64p, i32p,
                                          ctypes.c_int32, ctypes.c_int32]
        L.orc_chain_bound_fp8.restype = ctypes.c_double
        L.orc_bwd_kv_keys.argtypes = [pp, u16p, u16p, u16p, u16p, ctypes.c_int32, f64p, ctypes.c_int32,
                                      f64p, f64p, f64p, ctypes.c_int32]
        L.orc_delta_dp_rows_f64.argtypes = [pp, u16p, u16p, u16p, u16p, i32p, i32p, ctypes.c_int32,
                                            f64p, ctypes.c_int32]
        L.orc_dsum_rows_f64.argtypes = [pp, u16p, u16p, u16p, u16p, i32p, i32p, ctypes.c_int32,
                                        f64p, f64p, f64p, ctypes.c_int32]
        L.orc_fwd_emu_rows.argtypes = [pp, sp, u16p, u16p, u16p, i32p, i32p, ctypes.c_int32,
                                       f64p, f32p, f32p, u8p, ctypes.c_int32]
        L.orc_row_stats.argtypes = [pp, sp, u16p, u16p, i32p, ctypes.c_int32,
                                    f32p, f32p, f32p, u8p, u8p, ctypes.c_int32]
        L.orc_obar_f64.argtypes = [pp, u16p, u16p, u16p, f32p, i32p, ctypes.c_int32, f64p, f64p, ctypes.c_int32]
        L.orc_fwd_emu.argtypes = [pp, sp, u16p, u16p, u16p, i32p, ctypes.c_int32,
                                  f64p, u8p, f64p, f64p, f32p, f32p, u8p, u8p, u8p, ctypes.c_int32]
        L.orc_e4m3_round.argtypes = [ctypes.c_double]
        L.orc_e4m3_round.restype = ctypes.c_double
        L.orc_e4m3_ulp.argtypes = [ctypes.c_double]
        L.orc_e4m3_ulp.restype = ctypes.c_double
        L.orc_e4m3_boundary_distance.argtypes = [ctypes.c_double]
        L.orc_e4m3_boundary_distance.restype = ctypes.c_double
        for fn in ("orc_e2m1_round", "orc_e2m1_spacing", "orc_e2m1_boundary_distance"):
            getattr(L, fn).argtypes = [ctypes.c_double]
            getattr(L, fn).restype = ctypes.c_double
        for fn in ("orc_mx_scale_byte", "orc_mx_scale_byte_ceil"):
            getattr(L, fn).argtypes = [ctypes.c_double]
            getattr(L, fn).restype = ctypes.c_int
        for name in ("orc_fwd_f64", "orc_bwd_f64", "orc_bwd_rows_f64", "orc_row_stats",
                     "orc_obar_f64", "orc_fwd_emu", "orc_bwd_emu", "orc_bwd_rows_emu",
                     "orc_fwd_emu_rows", "orc_delta_dp_rows_f64", "orc_dsum_rows_f64", "orc_bwd_kv_keys"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a, ctype):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, "bf16 inputs are passed as uint16 bit patterns"
    return a


def _threads(n):
    return int(n) if n else (os.cpu_count() or 1)


def _heads_arg(heads):
    if heads is None:
        return None, 0
    h = np.ascontiguousarray(np.asarray(heads, dtype=np.int32))
    return h, int(h.size)


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"{name} rejected its arguments (code {rc})")


# ---- bf16 ---------------------------------------------------------------

def bf16_from_f32(x) -> np.ndarray:
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    out = np.empty(x.shape, dtype=np.uint16)
    lib().orc_bf16_from_f32_array(_ptr(x, ctypes.c_float), _ptr(out, ctypes.c_uint16), x.size)
    return out


def f32_from_bf16(h) -> np.ndarray:
    h = np.ascontiguousarray(np.asarray(h, dtype=np.uint16))
    out = np.empty(h.shape, dtype=np.float32)
    lib().orc_f32_from_bf16_array(_ptr(h, ctypes.c_uint16), _ptr(out, ctypes.c_float), h.size)
    return out


def bf16_from_f64(x: float) -> int:
    return int(lib().orc_bf16_from_f64(float(x)))


def bf16_value(bits: int) -> float:
    return float(lib().orc_f32_from_bf16(int(bits)))


def bf16_ulp(x: float) -> float:
    return float(lib().orc_bf16_ulp(float(x)))


def bf16_boundary_distance(x: float) -> float:
    return float(lib().orc_bf16_boundary_distance(float(x)))


def e4m3_round(x: float) -> float:
    """x rounded to OCP FP8 E4M3 (nearest, ties to even; NaN past 448)."""
    return float(lib().orc_e4m3_round(float(x)))


def e4m3_ulp(x: float) -> float:
    return float(lib().orc_e4m3_ulp(float(x)))


def e4m3_boundary_distance(x: float) -> float:
    return float(lib().orc_e4m3_boundary_distance(float(x)))


def e2m1_round(y: float) -> float:
    """y rounded to FP4 E2M1 (nearest, ties to even, saturating at +-6)."""
    return float(lib().orc_e2m1_round(float(y)))


def e2m1_boundary_distance(y: float) -> float:
    return float(lib().orc_e2m1_boundary_distance(float(y)))


def mx_scale_byte(amax: float) -> int:
    """E8M0 byte of the MX block scale 2^(floor(log2 amax) - 2) (>= 1)."""
    return int(lib().orc_mx_scale_byte(float(amax)))


def mx_scale_byte_ceil(amax: float) -> int:
    """E8M0 byte of the rounded-up MX scale 2^(ceil(log2 amax) - 2) (>= 1)."""
    return int(lib().orc_mx_scale_byte_ceil(float(amax)))


def e4m3_array(x):
    """Elementwise e4m3_round over an array (float64 result)."""
    x = np.asarray(x, dtype=np.float64)
    f = np.frompyfunc(lambda t: lib().orc_e4m3_round(float(t)), 1, 1)
    return f(x).astype(np.float64)


def bf16_round_of_sum(terms) -> tuple[int, float]:
    t = np.ascontiguousarray(np.asarray(terms, dtype=np.float64))
    ex = ctypes.c_double(0.0)
    bits = lib().orc_bf16_round_of_sum(_ptr(t, ctypes.c_double), int(t.size), ctypes.byref(ex))
    return int(bits), float(ex.value)


# ---- attention ------------------------------------------------------------

def fwd_f64(p: Problem, q, k, v, heads=None, nthreads=None):
    """O (double) and lse for the listed query heads (flattened b*Hq+h)."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    o = np.zeros(q.shape, dtype=np.float64)
    lse = np.zeros(q.shape[:-1], dtype=np.float64)
    h, nh = _heads_arg(heads)
    pc = p.c()
    _check(lib().orc_fwd_f64(ctypes.byref(pc), _ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16),
                             _ptr(v, ctypes.c_uint16), _ptr(h, ctypes.c_int32), nh,
                             _ptr(o, ctypes.c_double), _ptr(lse, ctypes.c_double), _threads(nthreads)),
           "orc_fwd_f64")
    return o, lse


def bwd_f64(p: Problem, q, k, v, dout, kv_heads=None, nthreads=None):
    """Dict with o, delta, dq (query heads of the listed KV heads), dk, dv."""
    q, k, v, dout = _u16(q), _u16(k), _u16(v), _u16(dout)
    o = np.zeros(q.shape, dtype=np.float64)
    delta = np.zeros(q.shape[:-1], dtype=np.float64)
    dq = np.zeros(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    h, nh = _heads_arg(kv_heads)
    pc = p.c()
    _check(lib().orc_bwd_f64(ctypes.byref(pc), _ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16),
                             _ptr(v, ctypes.c_uint16), _ptr(dout, ctypes.c_uint16),
                             _ptr(h, ctypes.c_int32), nh, _ptr(o, ctypes.c_double),
                             _ptr(delta, ctypes.c_double), _ptr(dq, ctypes.c_double),
                             _ptr(dk, ctypes.c_double), _ptr(dv, ctypes.c_double), _threads(nthreads)),
           "orc_bwd_f64")
    return dict(o=o, delta=delta, dq=dq, dk=dk, dv=dv)


def bwd_rows_f64(p: Problem, q, k, v, dout, qheads, rows, nthreads=None):
    """o, delta, dq (double) for single rows: row rows[i] of query head qheads[i]."""
    q, k, v, dout = _u16(q), _u16(k), _u16(v), _u16(dout)
    qh = np.ascontiguousarray(np.asarray(qheads, dtype=np.int32))
    rw = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
    n = int(qh.size)
    d = q.shape[-1]
    o = np.zeros((n, d), np.float64); delta = np.zeros(n, np.float64); dq = np.zeros((n, d), np.float64)
    pc = p.c()
    _check(lib().orc_bwd_rows_f64(ctypes.byref(pc), _ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16),
                                  _ptr(v, ctypes.c_uint16), _ptr(dout, ctypes.c_uint16),
                                  _ptr(qh, ctypes.c_int32), _ptr(rw, ctypes.c_int32), n,
                                  _ptr(o, ctypes.c_double), _ptr(delta, ctypes.c_double),
                                  _ptr(dq, ctypes.c_double), _threads(nthreads)), "orc_bwd_rows_f64")
    return dict(o=o, delta=delta, dq=dq)


def delta_dp_rows_f64(p: Problem, q, k, v, dout, qheads, rows, nthreads=None):
    """delta = rowsum(dP∘P) (double) for single rows: row rows[i] of query
    head qheads[i] ([R] method, paper §3.2)."""
    q, k, v, dout = _u16(q), _u16(k), _u16(v), _u16(dout)
    qh = np.ascontiguousarray(np.asarray(qheads, dtype=np.int32))
    rw = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
    n = int(qh.size)
    delta = np.zeros(n, np.float64)
    pc = p.c()
    _check(lib().orc_delta_dp_rows_f64(ctypes.byref(pc), _ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16),
                                       _ptr(v, ctypes.c_uint16), _ptr(dout, ctypes.c_uint16),
                                       _ptr(qh, ctypes.c_int32), _ptr(rw, ctypes.c_int32), n,
                                       _ptr(delta, ctypes.c_double), _threads(nthreads)),
           "orc_delta_dp_rows_f64")
    return delta


def dsum_rows_f64(p: Problem, q, k, v, dout, qheads, rows, delta_in, nthreads=None):
    """Row sums of dS for the given delta (double, without alpha): returns
    (sum_j P (dP - delta), sum_j P |dP - delta|) per row ([R] Eq. 1-2)."""
    q, k, v, dout = _u16(q), _u16(k), _u16(v), _u16(dout)
    qh = np.ascontiguousarray(np.asarray(qheads, dtype=np.int32))
    rw = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
    n = int(qh.size)
    di = np.ascontiguousarray(np.asarray(delta_in, np.float64).reshape(-1))
    assert di.size == n
    dsum = np.zeros(n, np.float64); wsum = np.zeros(n, np.float64)
    pc = p.c()
    _check(lib().orc_dsum_rows_f64(ctypes.byref(pc), _ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16),
                                   _ptr(v, ctypes.c_uint16), _ptr(dout, ctypes.c_uint16),
                                   _ptr(qh, ctypes.c_int32), _ptr(rw, ctypes.c_int32), n,
                                   _ptr(di, ctypes.c_double), _ptr(dsum, ctypes.c_double),
                                   _ptr(wsum, ctypes.c_double), _threads(nthreads)), "orc_dsum_rows_f64")
    return dsum, wsum


def bwd_emu(p: Problem, q, k, v, dout, o_in=None, round_ops=True, kv_heads=None, nthreads=None):
    """Backward replayed at the method's rounding points (see oracle.h):
    delta from o_in (None = exact O), bf16 P/dS operands when round_ops."""
    q, k, v, dout = _u16(q), _u16(k), _u16(v), _u16(dout)
    oi = None if o_in is None else np.ascontiguousarray(np.asarray(o_in, np.float64))
    if oi is not None:
        assert oi.shape == q.shape
    delta = np.zeros(q.shape[:-1], np.float64)
    dq = np.zeros(q.shape, np.float64); dk = np.zeros(k.shape, np.float64); dv = np.zeros(v.shape, np.float64)
    h, nh = _heads_arg(kv_heads)
    pc = p.c()
    _check(lib().orc_bwd_emu(ctypes.byref(pc), _ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16),
                             _ptr(v, ctypes.c_uint16), _ptr(dout, ctypes.c_uint16), _ptr(h, ctypes.c_int32),
                             nh, _ptr(oi, ctypes.c_double), int(bool(round_ops)),
                             _ptr(delta, ctypes.c_double), _ptr(dq, ctypes.c_double),
                             _ptr(dk, ctypes.c_double), _ptr(dv, ctypes.c_double), _threads(nthreads)),
           "orc_bwd_emu")
    return dict(delta=delta, dq=dq, dk=dk, dv=dv)


def bwd_kv_keys(p: Problem, q, k, v, dout, kv_head, o_in=None, round_ops=False, nthreads=None):
    """FP64 backward of one KV head, parallel over rows and key blocks: delta
    [g, N] of its g query heads and dk, dv [N, d] of its keys.  o_in [g, N, d]
    and round_ops as in bwd_emu (the method's rounding points)."""
    q, k, v, dout = _u16(q), _u16(k), _u16(v), _u16(dout)
    g = p.heads_q // p.heads_kv
    N, d = q.shape[-2], q.shape[-1]
    oi = None if o_in is None else np.ascontiguousarray(np.asarray(o_in, np.float64))
    if oi is not None:
        assert oi.shape == (g, N, d)
    delta = np.zeros((g, N), np.float64)
    dk = np.zeros((N, d), np.float64); dv = np.zeros((N, d), np.float64)
    pc = p.c()
    _check(lib().orc_bwd_kv_keys(ctypes.byref(pc), _ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16),
                                 _ptr(v, ctypes.c_uint16), _ptr(dout, ctypes.c_uint16), int(kv_head),
                                 _ptr(oi, ctypes.c_double), int(bool(round_ops)),
                                 _ptr(delta, ctypes.c_double), _ptr(dk, ctypes.c_double),
                                 _ptr(dv, ctypes.c_double), _threads(nthreads)), "orc_bwd_kv_keys")
    return dict(delta=delta, dk=dk, dv=dv)


def bwd_rows_emu(p: Problem, q, k, v, dout, qheads, rows, o_in=None, round_ops=True, nthreads=None):
    q, k, v, dout = _u16(q), _u16(k), _u16(v), _u16(dout)
    qh = np.ascontiguousarray(np.asarray(qheads, dtype=np.int32))
    rw = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
    n, d = int(qh.size), q.shape[-1]
    oi = None if o_in is None else np.ascontiguousarray(np.asarray(o_in, np.float64))
    if oi is not None:
        assert oi.shape == (n, d)
    delta = np.zeros(n, np.float64); dq = np.zeros((n, d), np.float64)
    pc = p.c()
    _check(lib().orc_bwd_rows_emu(ctypes.byref(pc), _ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16),
                                  _ptr(v, ctypes.c_uint16), _ptr(dout, ctypes.c_uint16),
                                  _ptr(qh, ctypes.c_int32), _ptr(rw, ctypes.c_int32), n,
                                  _ptr(oi, ctypes.c_double), int(bool(round_ops)),
                                  _ptr(delta, ctypes.c_double), _ptr(dq, ctypes.c_double),
                                  _threads(nthreads)), "orc_bwd_rows_emu")
    return dict(delta=delta, dq=dq)


def fwd_emu_rows(p: Problem, sched: Schedule, q, k, v, qheads, rows, nthreads=None):
    """Streaming emulation of listed rows only (no certification)."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    qh = np.ascontiguousarray(np.asarray(qheads, dtype=np.int32))
    rw = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
    n, d = int(qh.size), q.shape[-1]
    o = np.zeros((n, d), np.float64); m = np.zeros(n, np.float32); l = np.zeros(n, np.float32)
    fl = np.zeros(n, np.uint8)
    pc, sc = p.c(), sched.c()
    _check(lib().orc_fwd_emu_rows(ctypes.byref(pc), ctypes.byref(sc), _ptr(q, ctypes.c_uint16),
                                  _ptr(k, ctypes.c_uint16), _ptr(v, ctypes.c_uint16),
                                  _ptr(qh, ctypes.c_int32), _ptr(rw, ctypes.c_int32), n,
                                  _ptr(o, ctypes.c_double), _ptr(m, ctypes.c_float), _ptr(l, ctypes.c_float),
                                  _ptr(fl, ctypes.c_uint8), _threads(nthreads)), "orc_fwd_emu_rows")
    return dict(o=o, m=m, l=l, flags=fl)


def row_stats(p: Problem, q, k, sched: Schedule | None = None, heads=None, nthreads=None):
    """r, r2, m (fp32), flags, flag_cert (u8) per query row."""
    q, k = _u16(q), _u16(k)
    shp = q.shape[:-1]
    r = np.zeros(shp, np.float32); r2 = np.zeros(shp, np.float32); m = np.zeros(shp, np.float32)
    fl = np.zeros(shp, np.uint8); fc = np.zeros(shp, np.uint8)
    h, nh = _heads_arg(heads)
    pc = p.c()
    sc = (sched or Schedule()).c()
    _check(lib().orc_row_stats(ctypes.byref(pc), ctypes.byref(sc), _ptr(q, ctypes.c_uint16),
                               _ptr(k, ctypes.c_uint16), _ptr(h, ctypes.c_int32), nh,
                               _ptr(r, ctypes.c_float), _ptr(r2, ctypes.c_float), _ptr(m, ctypes.c_float),
                               _ptr(fl, ctypes.c_uint8), _ptr(fc, ctypes.c_uint8), _threads(nthreads)),
           "orc_row_stats")
    return dict(r=r, r2=r2, m=m, flags=fl, flag_cert=fc)


def obar_f64(p: Problem, q, k, v, m, heads=None, nthreads=None):
    """Ō(m) and ℓ(m) in double for a given per-row shift m (fp32)."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    m = np.ascontiguousarray(np.asarray(m, dtype=np.float32))
    ob = np.zeros(q.shape, np.float64)
    l = np.zeros(q.shape[:-1], np.float64)
    h, nh = _heads_arg(heads)
    pc = p.c()
    _check(lib().orc_obar_f64(ctypes.byref(pc), _ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16),
                              _ptr(v, ctypes.c_uint16), _ptr(m, ctypes.c_float), _ptr(h, ctypes.c_int32),
                              nh, _ptr(ob, ctypes.c_double), _ptr(l, ctypes.c_double), _threads(nthreads)),
           "orc_obar_f64")
    return ob, l


def fwd_emu(p: Problem, sched: Schedule, q, k, v, heads=None, nthreads=None):
    """Streaming bf16 emulation: dict of obar, obar_cert, obar_dev, o, m, l,
    flags, flag_cert, ex (see oracle.h)."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    shp = q.shape[:-1]
    ob = np.zeros(q.shape, np.float64); oc = np.zeros(q.shape, np.uint8)
    od = np.zeros(q.shape, np.float64)
    o = np.zeros(q.shape, np.float64)
    m = np.zeros(shp, np.float32); l = np.zeros(shp, np.float32)
    fl = np.zeros(shp, np.uint8); fc = np.zeros(shp, np.uint8); ex = np.zeros(shp, np.uint8)
    h, nh = _heads_arg(heads)
    pc, sc = p.c(), sched.c()
    _check(lib().orc_fwd_emu(ctypes.byref(pc), ctypes.byref(sc), _ptr(q, ctypes.c_uint16),
                             _ptr(k, ctypes.c_uint16), _ptr(v, ctypes.c_uint16), _ptr(h, ctypes.c_int32), nh,
                             _ptr(ob, ctypes.c_double), _ptr(oc, ctypes.c_uint8), _ptr(od, ctypes.c_double),
                             _ptr(o, ctypes.c_double),
                             _ptr(m, ctypes.c_float), _ptr(l, ctypes.c_float), _ptr(fl, ctypes.c_uint8),
                             _ptr(fc, ctypes.c_uint8), _ptr(ex, ctypes.c_uint8), _threads(nthreads)),
           "orc_fwd_emu")
    return dict(obar=ob, obar_cert=oc, obar_dev=od, o=o, m=m, l=l, flags=fl, flag_cert=fc, ex=ex)


def chain_bound(sched: Schedule, c0: float, terms) -> float:
    """Bound on |kernel sum - exact c0 + sum(terms)| for a chain of bf16
    matrix instructions of sched.chunk products (oracle.c, chain_bound)."""
    t = np.ascontiguousarray(np.asarray(terms, np.float64))
    sc = sched.c()
    return lib().orc_chain_bound(ctypes.byref(sc), float(c0), _ptr(t, ctypes.c_double), int(t.size))


def chain_bound_fp8(sched: Schedule, c0: float, terms, esum, shift=0) -> float:
    """The same for FP8 E4M3 products (esum: exponent sums of the operands)."""
    t = np.ascontiguousarray(np.asarray(terms, np.float64))
    e = np.ascontiguousarray(np.asarray(esum, np.int32))
    sc = sched.c()
    return lib().orc_chain_bound_fp8(ctypes.byref(sc), float(c0), _ptr(t, ctypes.c_double),
                                     _ptr(e, ctypes.c_int32), int(t.size), int(shift))


def chain_bound_mx(sched: Schedule, c0: float, terms) -> float:
    """The same for one scaled FP4 matrix instruction."""
    t = np.ascontiguousarray(np.asarray(terms, np.float64))
    sc = sched.c()
    return lib().orc_chain_bound_mx(ctypes.byref(sc), float(c0), _ptr(t, ctypes.c_double), int(t.size))

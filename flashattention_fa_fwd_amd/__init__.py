"""Guarded BF16 FlashAttention for MI355X (gfx950): Python binding.

Argument marshalling for the C ABI in ``include/attn.h`` (``libattn.so``):
every step of the computation runs in the library's HIP kernels.  PyTorch is
used only to own device memory and to name the current HIP stream.  There is
no fallback: if the library is missing or fails to load, every call raises.

The functions carry the C ABI's names: attn_fwd, attn_bwd (and its stages
attn_bwd_dq / attn_bwd_dkdv), attn_bwd_workspace_bytes, attn_schedule,
attn_strerror, attn_abi_version.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn.so")

CAUSAL = 0x1
GUARD_NONE, GUARD_BETA, GUARD_EPS = 0x0, 0x2, 0x4
OBAR_FP32 = 0x8
DELTA_DP = 0x10
SCHED_FA2_OPS = 0x20
SCHED_UNTILED = 0x40
_SCHEDULES = {"stream": 0, "fa2_ops": SCHED_FA2_OPS, "untiled": SCHED_UNTILED}
PV_FP8 = 0x80
PV_FP8_FIXED = 0x100
PV_MXFP4 = 0x200
PV_MX_CEIL = 0x400
_FP8 = {False: 0, None: 0, True: PV_FP8, "row": PV_FP8, "fixed": PV_FP8 | PV_FP8_FIXED}
ROW_TIE, ROW_ZERO_DENOM, ROW_GUARD_APPLIED = 0x1, 0x2, 0x4
_GUARDS = {"none": GUARD_NONE, "beta": GUARD_BETA, "eps": GUARD_EPS}


class AttnError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {attn_strerror(code)} (code {code})")
        self.code = code


class Strides(ctypes.Structure):
    """Element strides (batch, head, row) of one tensor; zeros = dense."""
    _fields_ = [("batch", ctypes.c_int64), ("head", ctypes.c_int64), ("row", ctypes.c_int64)]


_TENSORS = ("q", "k", "v", "o", "do", "dq", "dk", "dv")


class Params(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32),
        ("heads_kv", ctypes.c_int32), ("seqlen", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
        ("beta", ctypes.c_float), ("tie_eps", ctypes.c_float),
        ("shift_eps", ctypes.c_float), ("flags", ctypes.c_uint32),
    ] + [(f"{n}_stride", Strides) for n in _TENSORS]


_lib = None


def lib():
    """Load libattn.so (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run flashattention_fa_fwd_amd/build_lib.py")
        L = ctypes.CDLL(LIB_PATH)
        vp, fp, pp = ctypes.c_void_p, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(Params)
        u8p, i32p = ctypes.POINTER(ctypes.c_uint8), ctypes.POINTER(ctypes.c_int32)
        L.attn_abi_version.restype = ctypes.c_int
        L.attn_strerror.argtypes = [ctypes.c_int]
        L.attn_strerror.restype = ctypes.c_char_p
        L.attn_schedule.argtypes = [pp, i32p, i32p, i32p, i32p, i32p, i32p]
        L.attn_fwd.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.attn_bwd.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.attn_bwd_dkdv.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.attn_bwd_dq.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        for n in ("attn_schedule", "attn_fwd", "attn_bwd", "attn_bwd_dkdv", "attn_bwd_dq"):
            getattr(L, n).restype = ctypes.c_int
        L.attn_bwd_workspace_bytes.argtypes = [pp]
        L.attn_bwd_workspace_bytes.restype = ctypes.c_size_t
        _lib = L
    return _lib


def attn_abi_version() -> int:
    return lib().attn_abi_version()


def attn_strerror(code: int) -> str:
    return lib().attn_strerror(int(code)).decode()


def attn_bwd_workspace_bytes(p: "Params") -> int:
    """Device scratch attn_bwd needs for these params (always 0 for valid
    params; (size_t)-1 for params attn_bwd would reject)."""
    return int(lib().attn_bwd_workspace_bytes(ctypes.byref(_set_strides(p))))


def make_params(batch, heads_q, heads_kv, seqlen, head_dim, *, causal=True, guard="beta",
                beta=2.0, tie_eps=1e-3, shift_eps=2.0 ** -5, obar_fp32=False,
                softmax_scale=None, delta="do_o", schedule="stream", pv_fp8=False,
                pv_mxfp4=False) -> Params:
    """delta: "do_o" (rowsum(dO∘O), the default) or "dp_p" (rowsum(dP∘P)).
    schedule: the forward's rounding schedule, "stream" (default), "fa2_ops"
    (512-key blocks, bf16 block product) or "untiled" (one block a row).
    pv_fp8: the forward's P̄V product in FP8 E4M3 (streaming schedule):
    True or "row" (operand scale 2^k per row and block) or "fixed" (2^8).
    pv_mxfp4: the same product in MXFP4 (E2M1 with E8M0 scales per 32 keys):
    True or "floor" (the OCP scale rule) or "ceil" (scale rounded up)."""
    if pv_fp8 not in _FP8:
        raise ValueError(f"pv_fp8 must be False, True, 'row' or 'fixed', not {pv_fp8!r}")
    if delta not in ("do_o", "dp_p"):
        raise ValueError(f"delta must be 'do_o' or 'dp_p', not {delta!r}")
    if schedule not in _SCHEDULES:
        raise ValueError(f"schedule must be one of {sorted(_SCHEDULES)}, not {schedule!r}")
    flags = (CAUSAL if causal else 0) | _GUARDS[guard] | (OBAR_FP32 if obar_fp32 else 0)
    flags |= (DELTA_DP if delta == "dp_p" else 0) | _SCHEDULES[schedule] | _FP8[pv_fp8]
    if pv_mxfp4 not in (False, None, True, "floor", "ceil"):
        raise ValueError(f"pv_mxfp4 must be False, True, 'floor' or 'ceil', not {pv_mxfp4!r}")
    flags |= (PV_MXFP4 if pv_mxfp4 else 0) | (PV_MX_CEIL if pv_mxfp4 == "ceil" else 0)
    return Params(batch, heads_q, heads_kv, seqlen, head_dim,
                  0.0 if softmax_scale is None else float(softmax_scale),
                  float(beta), float(tie_eps), float(shift_eps), flags)


def _params_from(q, k, **kw) -> Params:
    B, Hq, N, d = q.shape
    return make_params(B, Hq, k.shape[1], N, d, **kw)


def _check(name, t, dtype, shape=None, device=None, strided=False):
    """The library reads and writes through raw device pointers sized from
    the parameters: every tensor must have exactly the expected dtype, shape
    and layout, on the device of q.  The [B,H,N,d] operands may be strided
    views (head_dim contiguous, strides multiples of 8 elements, checked
    again by the library); everything else must be contiguous."""
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or not t.is_cuda:
        raise TypeError(f"{name} must be a {dtype} tensor on a HIP device")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if strided:
        if t.dim() != 4 or t.stride(-1) != 1 or any(s < 0 or s % 8 for s in t.stride()[:3]):
            raise ValueError(f"{name} must be [batch, heads, seqlen, head_dim] with head_dim "
                             f"contiguous and other strides multiples of 8, not {t.stride()}")
        if t.stride(2) < t.shape[3] and t.shape[2] > 1:
            raise ValueError(f"{name}: rows overlap (row stride {t.stride(2)} < head_dim)")
    elif not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_bf16(name, t, shape=None, device=None):
    _check(name, t, torch.bfloat16, shape, device, strided=True)


def _set_strides(p: Params, **tensors) -> Params:
    """A copy of p with the element strides of the given [B,H,N,d] tensors
    (dense tensors get the dense strides; the library accepts both)."""
    p2 = Params.from_buffer_copy(p)
    for n, t in tensors.items():
        if t is None:
            continue
        sb, sh, sn, _ = t.stride()
        setattr(p2, f"{n}_stride", Strides(sb, sh, sn))
    return p2


def _stream(stream, device=None):
    s = torch.cuda.current_stream(device) if stream is None else stream
    if device is not None and s.device != device:
        raise ValueError(f"stream is on {s.device}, the tensors on {device}")
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _call(name, rc):
    if rc != 0:
        raise AttnError(rc, name)


def attn_schedule(p: Params):
    bm, bn, rn, ch, bb, pc = (ctypes.c_int32() for _ in range(6))
    _call("attn_schedule", lib().attn_schedule(ctypes.byref(p), ctypes.byref(bm), ctypes.byref(bn),
                                               ctypes.byref(rn), ctypes.byref(ch), ctypes.byref(bb),
                                               ctypes.byref(pc)))
    return dict(block_m=bm.value, block_n=bn.value, round_n=rn.value, chunk=ch.value,
                block_bf16=bb.value, pv_chunk=pc.value)


def attn_fwd(q, k, v, *, causal=True, guard="beta", beta=2.0, tie_eps=1e-3,
             shift_eps=2.0 ** -5, obar_fp32=False, softmax_scale=None, schedule="stream",
             pv_fp8=False, pv_mxfp4=False, return_obar=False, return_row_max=False, out=None,
             stream=None):
    """Guarded forward.  q [B,Hq,N,d], k/v [B,Hkv,N,d] bf16 (strided views
    with head_dim contiguous are passed as they are, e.g. head-transposed
    views of a fused QKV projection; outputs are allocated dense).  schedule:
    "stream" (the streaming kernel), "fa2_ops" or "untiled" (see make_params);
    pv_fp8: P̄V in FP8 E4M3 (streaming kernel only): True/"row" or "fixed";
    pv_mxfp4: P̄V in MXFP4 (streaming kernel only).
    Returns a dict: o, row_m, row_l, row_flags (+ obar, row_max on request)."""
    _check_bf16("q", q)
    if q.dim() != 4:
        raise ValueError(f"q must be [batch, heads, seqlen, head_dim], not {tuple(q.shape)}")
    B, Hq, N, d = q.shape
    dev = q.device
    _check_bf16("k", k, (B, k.shape[1], N, d) if k.dim() == 4 else None, dev)
    _check_bf16("v", v, k.shape, dev)
    p = _params_from(q, k, causal=causal, guard=guard, beta=beta, tie_eps=tie_eps,
                     shift_eps=shift_eps, obar_fp32=obar_fp32, softmax_scale=softmax_scale,
                     schedule=schedule, pv_fp8=pv_fp8, pv_mxfp4=pv_mxfp4)
    res = out if out is not None else {}
    if "o" not in res:
        res["o"] = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
        res["row_m"] = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
        res["row_l"] = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
        res["row_flags"] = torch.empty((B, Hq, N), dtype=torch.uint8, device=dev)
    if return_obar and "obar" not in res:
        res["obar"] = torch.empty(q.shape, dtype=torch.float32 if obar_fp32 else torch.bfloat16, device=dev)
    if return_row_max and "row_max" not in res:
        res["row_max"] = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    rows = (B, Hq, N)
    _check_bf16("o", res["o"], q.shape, dev)
    _check("row_m", res["row_m"], torch.float32, rows, dev)
    _check("row_l", res["row_l"], torch.float32, rows, dev)
    _check("row_flags", res["row_flags"], torch.uint8, rows, dev)
    if res.get("obar") is not None:
        _check("obar", res["obar"], torch.float32 if obar_fp32 else torch.bfloat16, q.shape, dev)
    if res.get("row_max") is not None:
        _check("row_max", res["row_max"], torch.float32, rows, dev)
    p = _set_strides(p, q=q, k=k, v=v, o=res["o"])
    _call("attn_fwd", lib().attn_fwd(
        ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(res["o"]), _ptr(res["row_m"]),
        _ptr(res["row_l"]), _ptr(res["row_flags"]), _ptr(res.get("obar")), _ptr(res.get("row_max")),
        _stream(stream, dev)))
    return res


def attn_bwd(q, k, v, o, dout, row_m, row_l, *, causal=True, guard="beta", beta=2.0,
             tie_eps=1e-3, shift_eps=2.0 ** -5, softmax_scale=None, delta="do_o",
             row_dsum=False, out=None, stream=None):
    """Backward.  Returns a dict: dq, dk, dv (bf16) and delta (fp32), and with
    row_dsum=True the row sums of dS (fp32, without alpha).  delta="dp_p"
    forms delta = rowsum(dP∘P) (o is then not read; it may be None)."""
    _check_bf16("q", q)
    if q.dim() != 4:
        raise ValueError(f"q must be [batch, heads, seqlen, head_dim], not {tuple(q.shape)}")
    B, Hq, N, d = q.shape
    dev = q.device
    _check_bf16("k", k, (B, k.shape[1], N, d) if k.dim() == 4 else None, dev)
    _check_bf16("v", v, k.shape, dev)
    if not (o is None and delta == "dp_p"):
        _check_bf16("o", o, q.shape, dev)
    _check_bf16("dout", dout, q.shape, dev)
    rows = (B, Hq, N)
    _check("row_m", row_m, torch.float32, rows, dev)
    _check("row_l", row_l, torch.float32, rows, dev)
    p = _params_from(q, k, causal=causal, guard=guard, beta=beta, tie_eps=tie_eps,
                     shift_eps=shift_eps, softmax_scale=softmax_scale, delta=delta)
    res = out if out is not None else {}
    if "dq" not in res:
        res["dq"] = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
        res["dk"] = torch.empty(k.shape, dtype=torch.bfloat16, device=dev)
        res["dv"] = torch.empty(k.shape, dtype=torch.bfloat16, device=dev)
        res["delta"] = torch.empty(rows, dtype=torch.float32, device=dev)
    if row_dsum and "row_dsum" not in res:
        res["row_dsum"] = torch.empty(rows, dtype=torch.float32, device=dev)
    _check_bf16("dq", res["dq"], q.shape, dev)
    _check_bf16("dk", res["dk"], k.shape, dev)
    _check_bf16("dv", res["dv"], k.shape, dev)
    _check("delta", res["delta"], torch.float32, rows, dev)
    if row_dsum:
        _check("row_dsum", res["row_dsum"], torch.float32, rows, dev)
    p = _set_strides(p, q=q, k=k, v=v, o=o, do=dout, dq=res["dq"], dk=res["dk"], dv=res["dv"])
    _call("attn_bwd", lib().attn_bwd(
        ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(row_m), _ptr(row_l),
        _ptr(res["dq"]), _ptr(res["dk"]), _ptr(res["dv"]), _ptr(res["delta"]),
        _ptr(res.get("row_dsum") if row_dsum else None), _stream(stream, dev)))
    return res


def _stage_shapes(p: Params):
    qs = (p.batch, p.heads_q, p.seqlen, p.head_dim)
    ks = (p.batch, p.heads_kv, p.seqlen, p.head_dim)
    return qs, ks, (p.batch, p.heads_q, p.seqlen)


def attn_bwd_dkdv(p: Params, q, k, v, dout, row_m, row_l, delta, dk, dv, stream=None):
    """The backward's dK/dV stage (delta from attn_bwd_dq)."""
    qs, ks, rows = _stage_shapes(p)
    dev = q.device if isinstance(q, torch.Tensor) else None
    for n_, t, sh in (("q", q, qs), ("k", k, ks), ("v", v, ks), ("dout", dout, qs), ("dk", dk, ks), ("dv", dv, ks)):
        _check_bf16(n_, t, sh, dev)
    for n_, t in (("row_m", row_m), ("row_l", row_l), ("delta", delta)):
        _check(n_, t, torch.float32, rows, dev)
    p = _set_strides(p, q=q, k=k, v=v, do=dout, dk=dk, dv=dv)
    _call("attn_bwd_dkdv", lib().attn_bwd_dkdv(
        ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(row_m), _ptr(row_l),
        _ptr(delta), _ptr(dk), _ptr(dv), _stream(stream, dev)))


def attn_bwd_dq(p: Params, q, k, v, o, dout, row_m, row_l, dq, delta, row_dsum=None, stream=None):
    """The backward's dQ stage; it also writes delta (o unused, may be None,
    when p.flags holds DELTA_DP)."""
    qs, ks, rows = _stage_shapes(p)
    dev = q.device if isinstance(q, torch.Tensor) else None
    for n_, t, sh in (("q", q, qs), ("k", k, ks), ("v", v, ks), ("dout", dout, qs), ("dq", dq, qs)):
        _check_bf16(n_, t, sh, dev)
    if not (o is None and p.flags & DELTA_DP):
        _check_bf16("o", o, qs, dev)
    for n_, t in (("row_m", row_m), ("row_l", row_l), ("delta", delta)):
        _check(n_, t, torch.float32, rows, dev)
    if row_dsum is not None:
        _check("row_dsum", row_dsum, torch.float32, rows, dev)
    p = _set_strides(p, q=q, k=k, v=v, o=o, do=dout, dq=dq)
    _call("attn_bwd_dq", lib().attn_bwd_dq(
        ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(row_m), _ptr(row_l),
        _ptr(dq), _ptr(delta), _ptr(row_dsum), _stream(stream, dev)))


def default_scale(head_dim: int) -> float:
    """fl32(1/sqrt(head_dim)), the scale the library uses when none is given."""
    return float(torch.tensor(1.0 / math.sqrt(head_dim), dtype=torch.float32))

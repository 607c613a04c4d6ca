"""The C-ABI library loads on the CPU host, exports every function that
include/attn.h declares, and rejects bad arguments before touching a GPU
(no compute call is made here)."""
import ctypes
import os
import re

import pytest

import flashattention_fa_fwd_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(fa.LIB_PATH):
        from flashattention_fa_fwd_amd import build_lib
        build_lib.build()
    return fa.lib()


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "attn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\**\s*(attn_[a-z_0-9]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_every_declared_symbol_is_exported(L):
    names = _declared_functions()
    assert {"attn_fwd", "attn_bwd", "attn_schedule", "attn_bwd_dkdv", "attn_bwd_dq"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_version_and_strings(L):
    assert fa.attn_abi_version() == 12
    for code in (0, -1, -2, -3, -4, -6):
        assert fa.attn_strerror(code) and fa.attn_strerror(code) != "unknown error code"
    assert fa.attn_strerror(-99) == "unknown error code"


def test_schedule(L):
    p = fa.make_params(1, 1, 1, 128, 64)
    assert fa.attn_schedule(p) == dict(block_m=128, block_n=64, round_n=512, chunk=16, block_bf16=0, pv_chunk=16)
    p = fa.make_params(1, 1, 1, 128, 64, schedule="fa2_ops")
    assert fa.attn_schedule(p) == dict(block_m=128, block_n=512, round_n=512, chunk=16, block_bf16=1, pv_chunk=16)
    p = fa.make_params(1, 1, 1, 128, 64, schedule="untiled")
    assert fa.attn_schedule(p) == dict(block_m=128, block_n=0, round_n=0, chunk=16, block_bf16=1, pv_chunk=16)
    p.flags |= fa.SCHED_FA2_OPS  # two schedules at once
    assert L.attn_schedule(ctypes.byref(p), None, None, None, None, None, None) == -4
    # the FP8 product: streaming schedule only
    p = fa.make_params(1, 1, 1, 128, 64, pv_fp8=True)
    assert fa.attn_schedule(p)["block_n"] == 64
    for sched in ("fa2_ops", "untiled"):
        for kw in (dict(pv_fp8=True), dict(pv_mxfp4=True)):
            p = fa.make_params(1, 1, 1, 128, 64, schedule=sched, **kw)
            assert L.attn_schedule(ctypes.byref(p), None, None, None, None, None, None) == -4
    p = fa.make_params(1, 1, 1, 128, 64, pv_mxfp4=True)
    assert fa.attn_schedule(p)["block_n"] == 64
    p = fa.make_params(1, 1, 1, 128, 64, pv_fp8=True, pv_mxfp4=True)  # two formats
    assert L.attn_schedule(ctypes.byref(p), None, None, None, None, None, None) == -4
    p = fa.make_params(1, 1, 1, 128, 64)
    p.flags |= fa.PV_FP8_FIXED  # the fixed FP8 scale without the FP8 product
    assert L.attn_schedule(ctypes.byref(p), None, None, None, None, None, None) == -4
    p = fa.make_params(1, 1, 1, 128, 64)
    p.flags |= fa.PV_MX_CEIL  # the MX rule without the MXFP4 product
    assert L.attn_schedule(ctypes.byref(p), None, None, None, None, None, None) == -4
    p = fa.make_params(1, 1, 1, 128, 64, pv_mxfp4="ceil")
    assert fa.attn_schedule(p)["block_n"] == 64
    with pytest.raises(ValueError):
        fa.make_params(1, 1, 1, 64, 64, schedule="blocked")


FAKE = 0x10000  # a 16-byte aligned non-null address; never dereferenced


def _fwd(L, p, ptrs=None, obar=None):
    ptrs = ptrs or [FAKE] * 7
    vp = [ctypes.c_void_p(x) for x in ptrs]
    return L.attn_fwd(ctypes.byref(p), *vp, ctypes.c_void_p(obar), None, None)


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), -2), (dict(heads_q=3, heads_kv=2), -2), (dict(seqlen=0), -2),
    (dict(head_dim=96), -3), (dict(head_dim=32), -3),
    # more workgroups of 128 rows than one launch can address (2^24 - 1)
    (dict(batch=1 << 16, heads_q=256, heads_kv=256, seqlen=129), -2),
])
def test_shape_errors(L, kw, code):
    args = dict(batch=1, heads_q=2, heads_kv=1, seqlen=64, head_dim=64)
    args.update(kw)
    p = fa.make_params(args["batch"], args["heads_q"], args["heads_kv"], args["seqlen"], args["head_dim"])
    assert _fwd(L, p) == code


def test_param_errors(L):
    p = fa.make_params(1, 1, 1, 64, 64, guard="beta", beta=1.0)
    assert _fwd(L, p) == -4
    p = fa.make_params(1, 1, 1, 64, 64, guard="eps", shift_eps=0.0)
    assert _fwd(L, p) == -4
    p = fa.make_params(1, 1, 1, 64, 64, tie_eps=-1.0)
    assert _fwd(L, p) == -4
    p = fa.make_params(1, 1, 1, 64, 64)
    p.flags = fa.GUARD_BETA | fa.GUARD_EPS
    assert _fwd(L, p) == -4
    p.flags = 0x100
    assert _fwd(L, p) == -4
    p = fa.make_params(1, 1, 1, 64, 64, softmax_scale=float("nan"))
    assert _fwd(L, p) == -4
    # beta is only checked when the beta guard is on
    p = fa.make_params(1, 1, 1, 64, 64, guard="none", beta=0.5)
    assert fa.attn_schedule(p)["block_n"] == 64


def test_null_and_alignment_errors(L):
    p = fa.make_params(1, 1, 1, 64, 64)
    assert L.attn_fwd(None, *([ctypes.c_void_p(FAKE)] * 7), None, None, None) == -1
    ptrs = [FAKE] * 7
    ptrs[0] = 0
    assert _fwd(L, p, ptrs) == -1
    ptrs = [FAKE] * 7
    ptrs[1] = FAKE + 2
    assert _fwd(L, p, ptrs) == -3
    assert _fwd(L, p, obar=FAKE + 8) == -3


def test_backward_argument_errors(L):
    """The backward stages validate before enqueueing anything (no GPU needed)."""
    vp = ctypes.c_void_p
    p = fa.make_params(2, 4, 2, 100, 64)
    args = [vp(FAKE)] * 11 + [None]  # ..., delta, row_dsum (optional)
    assert L.attn_bwd(ctypes.byref(p), *[None] + args[1:], None) == -1          # q missing
    assert L.attn_bwd(ctypes.byref(p), *[vp(FAKE + 2)] + args[1:], None) == -3  # misaligned
    assert L.attn_bwd_dkdv(ctypes.byref(p), *[vp(FAKE)] * 8, None, None) == -1  # dv missing
    assert L.attn_bwd_dq(ctypes.byref(p), *[vp(FAKE)] * 8, None, None, None) == -1  # delta missing
    assert L.attn_bwd_dq(ctypes.byref(p), *[vp(FAKE)] * 7, vp(FAKE + 8), vp(FAKE), None, None) == -3
    bad = fa.make_params(1, 3, 2, 10, 64)
    assert L.attn_bwd_dq(ctypes.byref(bad), *[vp(FAKE)] * 9, None, None) == -2
    huge = fa.make_params(1, 1, 1, 1 << 24, 64)  # one head past a 32-bit byte range
    assert L.attn_bwd_dkdv(ctypes.byref(huge), *[vp(FAKE)] * 9, None) == -2
    # O is required for delta = rowsum(dO∘O) only; when given it must be aligned
    no_o = [vp(FAKE)] * 4 + [None] + [vp(FAKE)] * 6 + [None]
    assert L.attn_bwd(ctypes.byref(p), *no_o, None) == -1
    dp = fa.make_params(2, 4, 2, 100, 64, delta="dp_p")
    assert dp.flags & fa.DELTA_DP
    bad_o = [vp(FAKE)] * 4 + [vp(FAKE + 8)] + [vp(FAKE)] * 6 + [None]
    assert L.attn_bwd(ctypes.byref(dp), *bad_o, None) == -3
    assert L.attn_bwd_dq(ctypes.byref(dp), *[vp(FAKE)] * 3, vp(FAKE + 8), *[vp(FAKE)] * 5, None, None) == -3
    with pytest.raises(ValueError):
        fa.make_params(1, 1, 1, 64, 64, delta="o")


def test_binding_has_no_fallback(monkeypatch, tmp_path):
    """Without the library the binding raises instead of computing anything."""
    monkeypatch.setattr(fa, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(fa, "_lib", None)
    with pytest.raises(ImportError):
        fa.lib()


def test_binding_rejects_host_and_mistyped_tensors():
    """The binding checks dtype, device and layout before any pointer reaches
    the library (host tensors here, so no library call is made)."""
    import torch
    q = torch.zeros((1, 1, 64, 64), dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        fa.attn_fwd(q, q, q)
    with pytest.raises(TypeError):
        fa.attn_fwd(q.float(), q, q)
    m = torch.zeros((1, 1, 64), dtype=torch.float32)
    with pytest.raises(TypeError):
        fa.attn_bwd(q, q, q, q, q, m, m)
    p = fa.make_params(1, 1, 1, 64, 64)
    with pytest.raises(TypeError):
        fa.attn_bwd_dkdv(p, q, q, q, q, m, m, m, q, q)


def test_stride_rules(L):
    """Per-tensor strides: zeros are the dense layout; negative strides,
    strides that are not multiples of 8 elements, overlapping rows and rows
    beyond a 32-bit byte range are refused before anything is enqueued."""
    B, H, N, d = 2, 3, 100, 64
    ok = fa.make_params(B, H, H, N, d)
    assert _fwd(L, ok) != -3 and fa.attn_schedule(ok)["block_n"] == 64
    fused = fa._set_strides(ok)
    # one third of a fused [B, N, 3, H, d] projection output, head-transposed
    for n in ("q", "k", "v"):
        setattr(fused, f"{n}_stride", fa.Strides(N * 3 * H * d, d, 3 * H * d))
    fused.o_stride = fa.Strides(N * H * d, d, H * d)  # O written as [B, N, H, d]
    assert fa.attn_schedule(fused)["block_n"] == 64
    cases = [
        ("q", fa.Strides(-8, d, 3 * H * d), -3),
        ("k", fa.Strides(N * H * d, 4, d), -3),          # head stride not a multiple of 8
        ("v", fa.Strides(N * H * d, d, 60), -3),         # row stride not a multiple of 8
        ("o", fa.Strides(N * H * d, d, 56), -3),         # rows overlap (56 < 64)
        ("dk", fa.Strides(N * H * d, d, 1 << 24), -2),   # (N + 256) rows past 2^31 bytes
    ]
    for name, st, code in cases:
        p = fa._set_strides(ok)
        setattr(p, f"{name}_stride", st)
        assert L.attn_schedule(ctypes.byref(p), None, None, None, None, None, None) == code, name
        assert _fwd(L, p) == code, name


def test_bwd_workspace_query(L):
    """The backward needs no workspace: 0 for valid params, (size_t)-1 for
    params the backward would reject."""
    import ctypes as C
    for args, kw in (((1, 1, 1, 64, 64), {}), ((2, 8, 2, 1000, 128), dict(causal=False)),
                     ((16, 12, 12, 1024, 64), dict(delta="dp_p"))):
        assert fa.attn_bwd_workspace_bytes(fa.make_params(*args, **kw)) == 0
    bad = fa.make_params(1, 3, 2, 64, 64)   # heads_q not a multiple of heads_kv
    assert fa.attn_bwd_workspace_bytes(bad) == C.c_size_t(-1).value
    assert L.attn_bwd_workspace_bytes(None) == C.c_size_t(-1).value

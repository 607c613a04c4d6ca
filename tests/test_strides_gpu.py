"""Strided operands through the C ABI: head-transposed views of a fused QKV
projection output (the layout of the GPT-2 attention layers the pages train,
[R] "Core idea" -> method, paper §3.1) and O / dO / dQ / dK / dV in the
[batch, seqlen, heads, head_dim] layout give bit for bit what the dense
call gives on the same values."""
import numpy as np
import pytest
import torch

import flashattention_fa_fwd_amd as fa
from flashattention_fa_fwd_amd import workloads as W

from _util import bits, dev, report

pytestmark = pytest.mark.gpu


def _fused(x, wl):
    """q, k, v as views of one [B, N, 3, H, d] buffer (H = heads_q; for GQA
    the K and V views take the first heads_kv heads of their thirds)."""
    B, Hq, Hkv, N, d = wl.batch, wl.heads_q, wl.heads_kv, wl.seqlen, wl.head_dim
    qkv = torch.zeros((B, N, 3, Hq, d), dtype=torch.bfloat16, device="cuda")
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    qkv[:, :, 0] = q.transpose(1, 2)
    qkv[:, :, 1, :Hkv] = k.transpose(1, 2)
    qkv[:, :, 2, :Hkv] = v.transpose(1, 2)
    qs = qkv[:, :, 0].transpose(1, 2)
    ks = qkv[:, :, 1, :Hkv].transpose(1, 2)
    vs = qkv[:, :, 2, :Hkv].transpose(1, 2)
    assert not qs.is_contiguous() and torch.equal(qs, q) and torch.equal(ks, k)
    return (q, k, v), (qs, ks, vs)


def _bnhd(shape):
    """An empty [B, H, N, d] tensor whose memory is [B, N, H, d]."""
    B, H, N, d = shape
    return torch.empty((B, N, H, d), dtype=torch.bfloat16, device="cuda").transpose(1, 2)


@pytest.mark.parametrize("shape", [(2, 4, 4, 200, 64, True), (1, 8, 2, 257, 128, True),
                                   (2, 2, 1, 130, 64, False)])
@pytest.mark.parametrize("guard", ["none", "beta"])
def test_fused_qkv_views_match_dense(shape, guard):
    B, Hq, Hkv, N, d, causal = shape
    wl = W.Workload("strided", B, Hq, Hkv, N, d, causal, 1.5, 1.5, "mu_uniform", 0.0, 4.0, 0.1,
                    0.0, 16.0, 4242)
    x = W.make_custom(wl)
    (q, k, v), (qs, ks, vs) = _fused(x, wl)
    do = dev(x["do"])
    f0 = fa.attn_fwd(q, k, v, causal=causal, guard=guard)
    f1 = fa.attn_fwd(qs, ks, vs, causal=causal, guard=guard, out={
        "o": _bnhd(q.shape),
        "row_m": torch.empty((B, Hq, N), dtype=torch.float32, device="cuda"),
        "row_l": torch.empty((B, Hq, N), dtype=torch.float32, device="cuda"),
        "row_flags": torch.empty((B, Hq, N), dtype=torch.uint8, device="cuda")})
    torch.cuda.synchronize()
    assert not f1["o"].is_contiguous()
    assert np.array_equal(bits(f0["o"]), bits(f1["o"]))
    for key in ("row_m", "row_l", "row_flags"):
        assert torch.equal(f0[key], f1[key]), key
    # backward: dO in the [B, N, H, d] layout, gradients written into a
    # fused [B, N, 3, H, d] buffer (the projection's gradient)
    dos = _bnhd(q.shape)
    dos.copy_(do)
    gqkv = torch.zeros((B, N, 3, Hq, d), dtype=torch.bfloat16, device="cuda")
    out = {"dq": gqkv[:, :, 0].transpose(1, 2), "dk": gqkv[:, :, 1, :Hkv].transpose(1, 2),
           "dv": gqkv[:, :, 2, :Hkv].transpose(1, 2),
           "delta": torch.empty((B, Hq, N), dtype=torch.float32, device="cuda")}
    b0 = fa.attn_bwd(q, k, v, f0["o"], do, f0["row_m"], f0["row_l"], causal=causal, guard=guard)
    b1 = fa.attn_bwd(qs, ks, vs, f1["o"], dos, f1["row_m"], f1["row_l"], causal=causal, guard=guard,
                     out=out)
    torch.cuda.synchronize()
    for key in ("dq", "dk", "dv"):
        assert np.array_equal(bits(b0[key]), bits(b1[key])), key
    assert torch.equal(b0["delta"], b1["delta"])
    # nothing outside the gradient views was written
    if Hkv < Hq:
        assert not gqkv[:, :, 1:, Hkv:].any()
    report(f"strided {shape} {guard}", o_bits="equal", grads="equal")

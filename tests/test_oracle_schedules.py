"""Pins of the oracle's streaming emulation under the other rounding
schedules: FA2 written as tensor operations, which keeps each block's
product P̄V in bf16 ([R] "Points to doubt": the analysed implementation,
block size 512), and no tiling (one block per row; [S] "Key claims":
disabling tiling still fails).

Closed form: with Q = 0 every logit is 0, so (no guard) every P̄ = exp(0 - 0)
is exactly 1 and Ō is a plain sequence of bf16 sums of V, which torch's own
bf16 conversion computes independently of the oracle."""
import numpy as np
import pytest
import torch

from flashattention_fa_fwd_amd import workloads as W


def _bf16(x64):
    """RNE to bf16 of a double that is exact in fp32 (checked), via torch."""
    x32 = np.float32(x64)
    assert float(x32) == x64, "intermediate sum not exact in fp32"
    return float(torch.tensor(x32).to(torch.bfloat16).float())


def _case(orc, N, d, seed):
    rng = np.random.default_rng(seed)
    q = np.zeros((1, 1, N, d), np.uint16)  # bf16 zero
    k = W.to_bf16_bits(rng.standard_normal((1, 1, N, d)).astype(np.float32))
    v = W.to_bf16_bits((rng.standard_normal((1, 1, N, d)) * 3.0).astype(np.float32))
    p = orc.Problem(1, 1, 1, N, d, False, 0)
    return p, q, k, v


@pytest.mark.parametrize("block", [1, 2, 4, 8])
def test_block_bf16_closed_form(orc, block):
    N, d = 8, 64
    p, q, k, v = _case(orc, N, d, 20 + block)
    vf = W.bits_to_f32(v[0, 0]).astype(np.float64)
    exp_blk = np.zeros(d)   # FA2 as tensor ops: bf16 block product, bf16 add
    exp_acc = np.zeros(d)   # default: the block adds into the fp32 sum, one rounding
    for j0 in range(0, N, block):
        for f in range(d):
            bsum = float(np.sum(vf[j0:j0 + block, f]))
            exp_blk[f] = _bf16(exp_blk[f] + _bf16(bsum))
            exp_acc[f] = _bf16(exp_acc[f] + bsum)
    for block_bf16, exp in ((True, exp_blk), (False, exp_acc)):
        s = orc.Schedule(block_n=block, round_n=block, block_bf16=block_bf16, certify=False)
        e = orc.fwd_emu(p, s, q, k, v)
        assert np.all(e["l"] == N)  # every P̄ is 1
        for i in range(N):
            assert np.array_equal(e["obar"][0, 0, i], exp), (block_bf16, i)
    if 1 < block < N:  # the two schedules differ somewhere on these inputs
        assert not np.array_equal(exp_blk, exp_acc)
    else:  # one key per block (already bf16) or one block (nothing to add to)
        assert np.array_equal(exp_blk, exp_acc)


def test_untiled_is_one_block(orc):
    """No tiling: one block per row, Ō = bf16(sum_j P̄_j V_j) with the final
    shift; block_bf16 changes nothing (bf16(0 + bf16(x)) = bf16(x))."""
    N, d = 8, 64
    p, q, k, v = _case(orc, N, d, 30)
    vf = W.bits_to_f32(v[0, 0]).astype(np.float64)
    exp = np.array([_bf16(float(np.sum(vf[:, f]))) for f in range(d)])
    for block_bf16 in (False, True):
        s = orc.Schedule(block_n=0, round_n=0, block_bf16=block_bf16, certify=False)
        e = orc.fwd_emu(p, s, q, k, v)
        for i in range(N):
            assert np.array_equal(e["obar"][0, 0, i], exp)

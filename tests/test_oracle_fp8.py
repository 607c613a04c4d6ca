"""Pins of the oracle's FP8 E4M3 arithmetic and of its emulation of the FP8
P̄V product (the pages' open question of the bias with fewer mantissa bits:
[R] "Open questions").

E4M3 is the OCP 8-bit format: sign, 4 exponent bits (bias 7), 3 mantissa
bits, subnormals k * 2^-9, largest finite 448, no infinities.  The rounding
is pinned against (1) a brute-force nearest search over the 254 finite codes
decoded from that bit layout and (2) torch's float8_e4m3fn conversion.  The
emulation is pinned against closed forms (Q = 0: every logit 0) and against
a direct numpy/torch evaluation of the single-block sum."""
import numpy as np
import pytest
import torch

from flashattention_fa_fwd_amd import workloads as W


def _decode(b):
    s = -1.0 if b & 0x80 else 1.0
    e, m = (b >> 3) & 15, b & 7
    if e == 15 and m == 7:
        return float("nan")
    return s * (m / 8 * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))


CODES = [(b, _decode(b)) for b in range(256) if not np.isnan(_decode(b))]


def _nearest(x):
    """Nearest finite code value; ties to the even code (mantissa LSB 0)."""
    best = None
    for b, v in CODES:
        d = abs(v - x)
        if best is None or d < best[0] or (d == best[0] and (b & 1) == 0):
            best = (d, b, v)
    return best[2]


def test_e4m3_decode_table():
    vals = sorted(v for _, v in CODES if v > 0)
    assert len(CODES) == 254 and vals[-1] == 448.0 and vals[0] == 2.0 ** -9 and len(vals) == 126
    assert _decode(0x38) == 1.0 and _decode(0x7E) == 448.0 and _decode(0x08) == 2.0 ** -6


def test_e4m3_round_brute_force(orc):
    pos = sorted(v for _, v in CODES if v > 0)
    xs = []
    for a, b in zip(pos[:-1], pos[1:]):  # each gap: ends, midpoint, quarters
        xs += [a, (a + b) / 2, a + (b - a) / 4, a + 3 * (b - a) / 4]
    xs += [448.0, 455.9, 2.0 ** -10, 2.0 ** -10 * 1.0001, 2.0 ** -11, 0.0]
    for x in xs:
        for sx in (x, -x):
            assert orc.e4m3_round(sx) == _nearest(sx), sx
    # past the largest finite value: 448 until the midpoint to the next
    # binade step (464), NaN from there (no infinities in the format)
    assert orc.e4m3_round(463.9) == 448.0
    assert np.isnan(orc.e4m3_round(464.5)) and np.isnan(orc.e4m3_round(float("inf")))


def test_e4m3_round_matches_torch(orc):
    rng = np.random.default_rng(5)
    x = rng.uniform(-1, 1, 20000) * 2.0 ** rng.uniform(-12, 8.7, 20000)
    x = x[np.abs(x) < 464]
    ref = torch.tensor(x, dtype=torch.float64).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = orc.e4m3_array(x)
    assert np.array_equal(got, ref)


def test_e4m3_ulp_and_boundary_distance(orc):
    assert orc.e4m3_ulp(1.0) == 0.125 and orc.e4m3_ulp(1.99) == 0.125
    assert orc.e4m3_ulp(256.0) == 32.0 and orc.e4m3_ulp(255.0) == 16.0
    assert orc.e4m3_ulp(2.0 ** -7) == 2.0 ** -9 and orc.e4m3_ulp(2.0 ** -6) == 2.0 ** -9
    assert orc.e4m3_boundary_distance(1.0625) == 0.0  # midpoint of 1 and 1.125
    assert orc.e4m3_boundary_distance(1.0) == 0.0625
    assert orc.e4m3_boundary_distance(248.0) == 0.0  # midpoint of 240 and 256


def _q0_case(orc, N, d, guard, seed, **kw):
    rng = np.random.default_rng(seed)
    q = np.zeros((1, 1, N, d), np.uint16)
    k = W.to_bf16_bits(rng.standard_normal((1, 1, N, d)).astype(np.float32))
    v = W.to_bf16_bits((rng.standard_normal((1, 1, N, d)) * 2.0).astype(np.float32))
    p = orc.Problem(1, 1, 1, N, d, False, guard, **kw)
    return p, q, k, v


def _torch_e4m3(x):
    return torch.tensor(np.asarray(x, np.float64)).to(torch.float8_e4m3fn).to(torch.float64).numpy()


def _bf16(x):
    return torch.tensor(np.asarray(x, np.float64)).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()


@pytest.mark.parametrize("guard", ["none", "eps"])
def test_fp8_q0_closed_form(orc, guard):
    """Q = 0: every logit is 0 and every row ties.  No guard: P̄ = 1 and
    2^8 P̄ = 256 is exact in E4M3, so Ō = sum_j e4m3(V_j) and ℓ = N.  The eps
    guard shifts by 2^-5: P̄ = exp(-2^-5) and 256 P̄ = 248.12 rounds up to
    256 in E4M3, so Ō is the same sum while ℓ = N exp(-2^-5): O comes out
    exp(2^-5) = 1.032 times too large (the bf16 path rounds P̄ to 0.96875
    and stays within 5e-4)."""
    N, d = 40, 64
    g = {"none": orc.GUARD_NONE, "eps": orc.GUARD_EPS}[guard]
    p, q, k, v = _q0_case(orc, N, d, g, 3)
    vf = W.bits_to_f32(v[0, 0]).astype(np.float64)
    v8 = _torch_e4m3(vf)
    sum8 = v8.sum(axis=0)  # exact in double (few, short mantissas)
    for obar_fp32 in (True, False):
        s = orc.Schedule(block_n=64, round_n=512, obar_fp32=obar_fp32, certify=False, pv_fp8="row")
        e = orc.fwd_emu(p, s, q, k, v)
        ob = e["obar"][0, 0]
        want = sum8 if obar_fp32 else _bf16(sum8)
        assert np.array_equal(ob, np.broadcast_to(want, ob.shape))
        pbar = 1.0 if guard == "none" else float(np.exp(-(2.0 ** -5)))
        l_want = np.float32(0)
        for _ in range(N):
            l_want = np.float32(l_want + np.float32(pbar))
        assert np.all(e["l"][0, 0] == l_want)
        o = e["o"][0, 0]
        o_want = _bf16(np.float32(want) / l_want)
        assert np.array_equal(o, np.broadcast_to(o_want, o.shape))
        if guard == "eps":  # the predicted factor exp(2^-5) over the exact mean
            ratio = (want / l_want) / (sum8 / N)
            assert np.allclose(ratio[np.abs(sum8) > 1.0], np.exp(2.0 ** -5), rtol=8e-3)
            assert np.all(e["ex"][0, 0] & orc.EX_PBAR_ONE_TIED)


@pytest.mark.parametrize("scale", ["row", "fixed"])
def test_fp8_single_block_direct(orc, scale):
    """One block (N <= 64), fp32 Ō: the emulated Ō is the exact sum
    sum_j e4m3(2^k exp(t_j - m)) / 2^k * e4m3(V_j), here evaluated with
    numpy and torch's float8 conversion from the row's final shift m and
    maximum r: k = 8 (fixed) or 7 - floor(fl32(fl32(r - m) * fl32(log2 e)))."""
    N, d = 56, 64
    rng = np.random.default_rng(17)
    q = W.to_bf16_bits(rng.standard_normal((1, 2, N, d)).astype(np.float32))
    k = W.to_bf16_bits(rng.standard_normal((1, 2, N, d)).astype(np.float32))
    v = W.to_bf16_bits((rng.standard_normal((1, 2, N, d)) * 1.5).astype(np.float32))
    for guard in (orc.GUARD_NONE, orc.GUARD_BETA, orc.GUARD_EPS):
        p = orc.Problem(1, 2, 2, N, d, True, guard, tie_eps=0.05)
        s = orc.Schedule(block_n=64, round_n=512, obar_fp32=True, certify=False, pv_fp8=scale)
        e = orc.fwd_emu(p, s, q, k, v)
        st = orc.row_stats(p, q, k, s)
        assert np.array_equal(st["m"], e["m"])
        alpha = float(np.float32(1.0 / np.sqrt(d)))
        checked = 0
        for h in range(2):
            qf = W.bits_to_f32(q[0, h]).astype(np.float64)
            kf = W.bits_to_f32(k[0, h]).astype(np.float64)
            v8 = _torch_e4m3(W.bits_to_f32(v[0, h]).astype(np.float64))
            for i in range(N):
                r, m = np.float32(st["r"][0, h, i]), np.float32(st["m"][0, h, i])
                ks = 8 if scale == "fixed" else 7 - int(np.floor(np.float32(np.float32(r - m) * np.float32(np.log2(np.e)))))
                t = alpha * (kf[: i + 1] @ qf[i])
                x = 2.0 ** ks * np.exp(t - float(m))
                if scale == "row":
                    assert 128.0 * (1 - 1e-6) <= x.max() < 256.0 * (1 + 1e-6)
                # skip rows with a value too close to an E4M3 rounding boundary
                # for the two evaluations of exp to agree on its side
                dist = np.array([orc.e4m3_boundary_distance(float(xx)) for xx in x])
                if np.any(dist <= 1e-9 * x):
                    continue
                want = (_torch_e4m3(x) / 2.0 ** ks) @ v8[: i + 1]
                assert np.allclose(e["obar"][0, h, i], want, rtol=1e-12, atol=1e-12)
                checked += 1
        assert checked > 0.9 * 2 * N


def test_fp8_beta_guard_underflow_closed_form(orc):
    """Every key identical, logit t0 = 14 on every key: the beta guard
    (beta = 2) shifts by 2 t0, so every P̄ = exp(-14) = 8.3e-7.  With the fixed
    scale 2^8 P̄ = 2.1e-4 is below half of E4M3's smallest subnormal 2^-9:
    every operand rounds to 0, Ō = 0 and O = 0 while ℓ = N exp(-14) > 0.
    With the row scale 2^k P̄ lands in [128, 256): O is mean(e4m3(V)) times
    e4m3(2^k P̄) / (2^k P̄), within 1/16 of it."""
    N, d = 24, 64
    qv = np.zeros((1, 1, N, d), np.float32); qv[..., 0] = 8.0
    kv = np.zeros((1, 1, N, d), np.float32); kv[..., 0] = 14.0  # t0 = 0.125 * 8 * 14
    rng = np.random.default_rng(4)
    v = W.to_bf16_bits(rng.standard_normal((1, 1, N, d)).astype(np.float32))
    q, k = W.to_bf16_bits(qv), W.to_bf16_bits(kv)
    p = orc.Problem(1, 1, 1, N, d, False, orc.GUARD_BETA, beta=2.0)
    pbar = np.exp(-14.0)
    v8 = _torch_e4m3(W.bits_to_f32(v[0, 0]).astype(np.float64))
    for scale in ("fixed", "row"):
        s = orc.Schedule(block_n=64, round_n=512, obar_fp32=True, certify=False, pv_fp8=scale)
        e = orc.fwd_emu(p, s, q, k, v)
        assert np.all(e["m"] == np.float32(28.0))
        assert np.allclose(e["l"], N * pbar, rtol=1e-5)
        if scale == "fixed":
            assert np.all(e["obar"] == 0.0) and np.all(e["o"] == 0.0)
        else:
            ks = 7 - int(np.floor(np.float32(np.float32(-14.0) * np.float32(np.log2(np.e)))))
            assert 128 <= 2.0 ** ks * pbar < 256
            f = float(_torch_e4m3(2.0 ** ks * pbar)) / (2.0 ** ks * pbar)
            assert abs(f - 1.0) <= 1.0 / 16
            want = v8.mean(axis=0) * f
            assert np.allclose(e["o"][0, 0], np.broadcast_to(want, (N, d)), rtol=2 ** -7, atol=1e-6)


def test_fp8_dev_bound_is_finite(orc):
    """The emulation's deviation bound: finite on rows with a certain shift
    decision, non-negative, and zero where every rounding is certified."""
    N, d = 100, 64
    rng = np.random.default_rng(9)
    q = W.to_bf16_bits(rng.standard_normal((1, 1, N, d)).astype(np.float32))
    k = W.to_bf16_bits(rng.standard_normal((1, 1, N, d)).astype(np.float32))
    v = W.to_bf16_bits(rng.standard_normal((1, 1, N, d)).astype(np.float32))
    p = orc.Problem(1, 1, 1, N, d, True, orc.GUARD_BETA)
    for fp8 in (False, True):
        s = orc.Schedule(block_n=64, round_n=512, chunk=16, pv_fp8=fp8)
        e = orc.fwd_emu(p, s, q, k, v)
        dev = e["obar_dev"][0, 0]
        fc = e["flag_cert"][0, 0].astype(bool)
        assert np.all(np.isfinite(dev[fc])) and np.all(dev >= 0)
        cert = e["obar_cert"][0, 0].astype(bool)
        assert np.all(dev[cert] == 0.0)


# ---- MXFP4 (OCP MX: E2M1 elements, one E8M0 scale per 32 values)

E2M1 = [(c, (-1.0 if c & 8 else 1.0) * [0, 0.5, 1, 1.5, 2, 3, 4, 6][c & 7]) for c in range(16)]


def _nearest_e2m1(y):
    """Brute force over the 16 codes: nearest after saturating at +-6, ties
    to the even code (mantissa bit 0)."""
    y = min(max(y, -6.0), 6.0)
    best = None
    for c, v in E2M1:
        d = abs(v - y)
        if best is None or d < best[0] or (d == best[0] and (c & 1) == 0):
            best = (d, c, v)
    return best[2]


def test_e2m1_round_brute_force(orc):
    mags = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    ys = []
    for a, b in zip(mags[:-1], mags[1:]):
        ys += [a, (a + b) / 2, a + (b - a) / 4, a + 3 * (b - a) / 4]
    ys += [6.0, 6.5, 7.0, 100.0, 0.1, 0.2499]
    for y in ys:
        for sy in (y, -y):
            assert orc.e2m1_round(sy) == abs(_nearest_e2m1(sy)) * (1 if sy >= 0 else -1) or \
                (orc.e2m1_round(sy) == 0.0 and _nearest_e2m1(sy) == 0.0), sy
    assert orc.e2m1_boundary_distance(1.75) == 0.0 and orc.e2m1_boundary_distance(6.0) == 1.0


def test_mx_scale_rule(orc):
    # X = 2^(floor(log2 amax) - 2): amax / X in [4, 8)
    for amax in (1.0, 0.969, 6.0, 7.99, 0.001, 3.0e-7, 255.0):
        b = orc.mx_scale_byte(amax)
        X = 2.0 ** (b - 127)
        assert 4.0 <= amax / X < 8.0, amax
    assert orc.mx_scale_byte(1.0) == 125 and orc.mx_scale_byte(0.969) == 124 and orc.mx_scale_byte(0.0) == 1
    # the rounded-up rule: amax / X in (2, 4], equal at powers of two
    for amax in (1.0, 0.969, 6.0, 7.99, 0.001, 3.0e-7, 255.0, 0.5):
        b = orc.mx_scale_byte_ceil(amax)
        X = 2.0 ** (b - 127)
        assert 2.0 < amax / X <= 4.0, amax
    assert orc.mx_scale_byte_ceil(1.0) == 125 and orc.mx_scale_byte_ceil(0.969) == 125


def _mx_quant(v, ceil=False):
    """numpy reference of one MX block: scale from the largest magnitude."""
    v = np.asarray(v, np.float64)
    amax = np.abs(v).max()
    rnd = np.ceil if ceil else np.floor
    X = 2.0 ** (rnd(np.log2(amax)) - 2) if amax > 0 else 2.0 ** -126
    return np.array([_nearest_e2m1(t / X) for t in v]) * X


@pytest.mark.parametrize("rule", ["floor", "ceil"])
@pytest.mark.parametrize("guard", ["none", "eps"])
def test_mxfp4_q0_closed_form(orc, guard, rule):
    """Q = 0: every P̄ of a row is equal.  No guard: P̄ = 1, X = 1/4, 4 is
    exact, Ō = sum_j q(V_j).  The eps guard: P̄ = exp(-2^-5) = 0.969, X =
    1/8, 0.969 * 8 = 7.75 saturates to 6: every operand is 0.75, so Ō is 0.75
    sum_j q(V_j) while ℓ = N exp(-2^-5) (O 23 % too small).  With the rule
    rounded up, X = 1/4 and 3.88 rounds to 4: every operand is 1, O 3.2 %
    too large, as with FP8.  V's blocks: per feature, keys 0..31 and 32..63
    of the 64-key step."""
    N, d = 40, 64
    g = {"none": orc.GUARD_NONE, "eps": orc.GUARD_EPS}[guard]
    p, q, k, v = _q0_case(orc, N, d, g, 5)
    vf = W.bits_to_f32(v[0, 0]).astype(np.float64)
    vq = np.zeros_like(vf)
    for f in range(d):
        for h in range(2):
            idx = [j for j in range(N) if (j >> 5) == h]
            vq[idx, f] = _mx_quant(vf[idx, f], ceil=rule == "ceil")
    pq = 1.0 if guard == "none" or rule == "ceil" else 0.75
    s = orc.Schedule(block_n=64, round_n=512, obar_fp32=True, certify=False, pv_mxfp4=rule)
    e = orc.fwd_emu(p, s, q, k, v)
    want = pq * vq.sum(axis=0)
    assert np.allclose(e["obar"][0, 0], np.broadcast_to(want, (N, d)), rtol=1e-12, atol=1e-12)
    if guard == "eps":
        cols = np.abs(vq.sum(axis=0)) > 1.0
        ratio = (want[cols] / e["l"][0, 0][:, None]) / (vq.sum(axis=0)[cols] / N)
        assert np.allclose(ratio, pq / np.exp(-(2.0 ** -5)), rtol=1e-5)


def test_mxfp4_single_block_direct(orc):
    """One 64-key step (N = 56), fp32 Ō: the emulation equals the MX
    quantization written out with numpy from the row's final shift."""
    N, d = 56, 64
    rng = np.random.default_rng(21)
    q = W.to_bf16_bits(rng.standard_normal((1, 1, N, d)).astype(np.float32))
    k = W.to_bf16_bits(rng.standard_normal((1, 1, N, d)).astype(np.float32))
    v = W.to_bf16_bits((rng.standard_normal((1, 1, N, d)) * 1.5).astype(np.float32))
    p = orc.Problem(1, 1, 1, N, d, True, orc.GUARD_BETA, tie_eps=0.05)
    s = orc.Schedule(block_n=64, round_n=512, obar_fp32=True, certify=False, pv_mxfp4=True)
    e = orc.fwd_emu(p, s, q, k, v)
    alpha = float(np.float32(1.0 / np.sqrt(d)))
    qf = W.bits_to_f32(q[0, 0]).astype(np.float64)
    kf = W.bits_to_f32(k[0, 0]).astype(np.float64)
    vf = W.bits_to_f32(v[0, 0]).astype(np.float64)
    vq = np.zeros_like(vf)  # V's blocks span every existing key of the step
    for f in range(d):
        for h in range(2):
            idx = [j for j in range(N) if (j >> 5) == h]
            vq[idx, f] = _mx_quant(vf[idx, f])
    checked = 0
    for i in range(N):
        t = alpha * (kf[: i + 1] @ qf[i])
        pbar = np.exp(t - float(e["m"][0, 0, i]))
        pq = np.zeros_like(pbar)
        ok = True
        for h in range(2):
            idx = [j for j in range(i + 1) if (j >> 5) == h]
            if not idx:
                continue
            amax = pbar[idx].max()
            X = 2.0 ** (np.floor(np.log2(amax)) - 2)
            y = pbar[idx] / X
            if np.any([orc.e2m1_boundary_distance(float(t)) <= 1e-9 * t for t in y]) or \
                    0 < abs(np.log2(amax) - np.round(np.log2(amax))) < 1e-9:
                ok = False
            pq[idx] = _mx_quant(pbar[idx])
        if not ok:
            continue
        assert np.allclose(e["obar"][0, 0, i], pq @ vq[: i + 1], rtol=1e-12, atol=1e-12)
        checked += 1
    assert checked > 0.8 * N

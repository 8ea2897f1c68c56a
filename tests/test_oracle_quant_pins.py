"""Pins for the oracle's dynamic-quant output (RMSNorm + per-row symmetric
quantisation, the Add + RmsNorm + DynamicQuant fusion the TileLang tutorial
ch. 02, section 4.2, cites from CANN).

The root r cancels out of the codes: with scale = r * max|x*w| / Q the codes
are q_j = round(Q * x_j * w_j / max_k |x_k * w_k|), an exact rational of the
inputs alone, so they can be checked exactly with Fractions -- independent of
any square root -- and the scale separately against r's closed forms.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests import exact
from tests.test_oracle_pins import bits_bf16, EPS5, EPS6

Q = {oracle.QUANT_INT8: 127, oracle.QUANT_FP8_E4M3: 448}


def _exact_codes(xv, wv, qtype):
    """Exact codes of one row from its exact input values; None where the exact
    quotient sits within 1e-9 (relative) of a rounding tie."""
    p = [a * b for a, b in zip(xv, wv)]
    m = max(abs(v) for v in p)
    out = []
    for v in p:
        t = Fraction(Q[qtype]) * v / m if m else Fraction(0)
        if qtype == oracle.QUANT_INT8:
            c = exact.round_half_even(t)
            c = max(-127, min(127, c))
            tie = abs((t - (t.numerator // t.denominator)) - Fraction(1, 2)) <= Fraction(1, 10 ** 9) * (abs(t) + 1)
            out.append(None if tie else c & 0xFF)
        else:
            c = exact.round_e4m3_exact(t)
            near = False
            a = abs(t)
            if 0 < a < 448:
                lo = c & 0x7F
                base = exact.e4m3_value(lo)
                for nb in (lo - 1, lo + 1):
                    if 0 <= nb <= 0x7E:
                        mid = (base + exact.e4m3_value(nb)) / 2
                        near |= abs(a - mid) <= Fraction(1, 10 ** 9) * a
            out.append(None if near else c)
    return out


def _check_row(q_row, xv, wv, qtype):
    want = _exact_codes(xv, wv, qtype)
    got = [int(v) & 0xFF for v in q_row]
    flagged = 0
    for g, w_ in zip(got, want):
        if w_ is None:
            flagged += 1
        else:
            assert g == w_, (got, want)
    return flagged


def test_e4m3_rounding_matches_exact_rational():
    rng = np.random.default_rng(20)
    vals = list(rng.standard_normal(3000) * np.exp(rng.uniform(-10, 7, 3000)))
    vals += [0.0, 448.0, 449.0, 470.0, 1e6, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -11, 2.0 ** -6, 232.0, 224.0, 240.0,
             1.0625, 1.0625 + 2 ** -30]
    for v in vals:
        want = exact.round_e4m3_exact(Fraction(v))
        if v == 0.0:
            want = 0
        assert oracle.round_e4m3(v) == want, (v, hex(oracle.round_e4m3(v)), hex(want))


def test_e4m3_ties_go_to_even():
    for code in (0x01, 0x02, 0x07, 0x08, 0x38, 0x39, 0x6A, 0x7D):
        mid = (exact.e4m3_value(code) + exact.e4m3_value(code + 1)) / 2
        want = code if code % 2 == 0 else code + 1
        assert oracle.round_e4m3(float(mid)) == want
        assert oracle.round_e4m3(-float(mid)) == (want | 0x80)


@pytest.mark.parametrize("qtype", [oracle.QUANT_INT8, oracle.QUANT_FP8_E4M3])
def test_hand_worked_codes(qtype):
    """x = [1, 2, 3, 5, 6, 7, 8, -8], w = 1: codes are round(Q*j/8); for int8
    127*j/8 = 15.875, 31.75, 47.625, 79.375, 95.25, 111.125, 127 ->
    16, 32, 48, 79, 95, 111, 127, -127 (no value near a tie)."""
    x = np.array([[1, 2, 3, 5, 6, 7, 8, -8]], np.float32)
    _, q, scale = oracle.rmsnorm_dynamic_quant_fwd(x, np.ones(8, np.float32), 0.0, qtype)
    if qtype == oracle.QUANT_INT8:
        assert list(q[0]) == [16, 32, 48, 79, 95, 111, 127, -127]
    else:
        # 448*j/8 = 56, 112, 168(tie), 280, 336(tie), 392, 448: check the non-tie ones
        got = [int(v) for v in q[0]]
        for idx, t in ((0, 56), (1, 112), (3, 280), (5, 392), (6, 448)):
            assert got[idx] == exact.round_e4m3_exact(t)
        assert got[7] == 0xFE  # -448
    # scale = r * max|y| / Q with r = 1/sqrt(mean(x^2)) and mean(x^2) = 252/8
    r = 1 / np.sqrt(252 / 8)
    assert abs(float(scale[0]) - r * 8 / Q[qtype]) <= 1e-7 * r * 8 / Q[qtype]


@pytest.mark.parametrize("qtype", [oracle.QUANT_INT8, oracle.QUANT_FP8_E4M3])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_codes_are_the_exact_rational_closed_form(qtype, dtype):
    """Random rows, random weights, eps > 0: codes equal the exact rounding of
    Q * x_j * w_j / max|x * w| (r cancels) except within 1e-9 of a tie."""
    rng = np.random.default_rng(21)
    x = (rng.standard_normal((6, 96)) * np.exp(rng.uniform(-4, 4, (6, 1)))).astype(np.float32)
    w = rng.uniform(-1.5, 1.5, 96).astype(np.float32)
    if dtype == "bf16":
        xs, ws = bits_bf16(x), bits_bf16(w)
        xv = [[exact.bf16_value(int(b)) for b in row] for row in xs]
        wv = [exact.bf16_value(int(b)) for b in ws]
    else:
        xs, ws = x, w
        xv = [[Fraction(float(v)) for v in row] for row in xs]
        wv = [Fraction(float(v)) for v in ws]
    _, q, _ = oracle.rmsnorm_dynamic_quant_fwd(xs, ws, 1e-5, qtype)
    flagged = sum(_check_row(q[i], xv[i], wv, qtype) for i in range(6))
    assert flagged <= 2


@pytest.mark.parametrize("qtype", [oracle.QUANT_INT8, oracle.QUANT_FP8_E4M3])
def test_scale_closed_form_constant_row(qtype):
    """Constant row c, weights w: r = 1/sqrt(c^2 + eps), max|y| = |c| r max|w|,
    scale = |c| max|w| / (Q sqrt(c^2 + eps)); eps comparable to c^2 matters."""
    c, eps = 1e-3, EPS6
    w = np.array([1.0, -2.0, 0.5, 1.5], np.float32)
    x = np.full((1, 4), c, np.float32)
    _, q, scale = oracle.rmsnorm_dynamic_quant_fwd(x, w, eps, qtype)
    cq = float(np.float32(c))
    want = abs(cq) * 2.0 / (Q[qtype] * np.sqrt(cq * cq + eps))
    assert abs(float(scale[0]) - want) <= 2e-7 * want
    # codes: Q * w_j / 2 * sign(c)
    for j in range(4):
        t = Fraction(Q[qtype]) * Fraction(float(w[j])) / 2
        wantc = exact.round_half_even(t) & 0xFF if qtype == oracle.QUANT_INT8 else exact.round_e4m3_exact(t)
        assert int(q[0, j]) & 0xFF == wantc


@pytest.mark.parametrize("qtype", [oracle.QUANT_INT8, oracle.QUANT_FP8_E4M3])
def test_row_max_maps_to_full_scale_and_zero_row(qtype):
    rng = np.random.default_rng(22)
    x = rng.standard_normal((4, 50)).astype(np.float32)
    x[2] = 0
    w = rng.uniform(0.5, 1.5, 50).astype(np.float32)
    _, q, scale = oracle.rmsnorm_dynamic_quant_fwd(x, w, 1e-5, qtype)
    for i in (0, 1, 3):
        k = int(np.argmax(np.abs(x[i].astype(np.float64) * w)))
        if qtype == oracle.QUANT_INT8:
            assert abs(int(q[i, k])) == 127
        else:
            assert int(q[i, k]) & 0x7F == 0x7E
    assert np.all(q[2] == 0) and scale[2] == 0


@pytest.mark.parametrize("qtype", [oracle.QUANT_INT8, oracle.QUANT_FP8_E4M3])
def test_dequantised_values_are_within_half_a_step(qtype):
    """|q * scale - y| is at most half a quantisation step (int8) or half an
    fp8 spacing at that magnitude -- for any correct quantiser."""
    rng = np.random.default_rng(23)
    x = bits_bf16(rng.standard_normal((8, 256)).astype(np.float32))
    w = bits_bf16(rng.uniform(0.5, 1.5, 256).astype(np.float32))
    _, q, scale = oracle.rmsnorm_dynamic_quant_fwd(x, w, 1e-5, qtype)
    y = oracle.rmsnorm_fwd(x, w, 1e-5)  # bf16-rounded y: allow its rounding too
    yv = (y.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for i in range(8):
        s = float(scale[i])
        if qtype == oracle.QUANT_INT8:
            deq = q[i].astype(np.float64) * s
            assert np.all(np.abs(deq - yv[i]) <= 0.5 * s * (1 + 1e-6) + np.abs(yv[i]) * 2 ** -8)
        else:
            deq = np.array([float(exact.e4m3_value(int(c))) for c in q[i]]) * s
            assert np.all(np.abs(deq - yv[i]) <= np.abs(yv[i]) * (2 ** -4 + 2 ** -8) + s * 2 ** -10)


@pytest.mark.parametrize("qtype", [oracle.QUANT_INT8, oracle.QUANT_FP8_E4M3])
def test_fused_quant_uses_the_rounded_sum(qtype):
    rng = np.random.default_rng(24)
    x = bits_bf16(rng.standard_normal((5, 64)).astype(np.float32))
    r = bits_bf16((rng.standard_normal((5, 64)) * 0.3).astype(np.float32))
    w = bits_bf16(rng.uniform(0.5, 1.5, 64).astype(np.float32))
    h, q, scale = oracle.rmsnorm_dynamic_quant_fwd(x, w, 1e-5, qtype, residual=r)
    h2, _ = oracle.rmsnorm_residual_fwd(x, r, w, 1e-5)
    assert np.array_equal(h, h2)
    _, q2, s2 = oracle.rmsnorm_dynamic_quant_fwd(h, w, 1e-5, qtype)
    assert np.array_equal(q, q2) and np.array_equal(scale, s2)


@pytest.mark.parametrize("qtype", [oracle.QUANT_INT8, oracle.QUANT_FP8_E4M3])
def test_scale_invariance_of_codes(qtype):
    """eps = 0: x -> 2^k x leaves codes and scale bitwise unchanged."""
    rng = np.random.default_rng(25)
    x = rng.standard_normal((3, 40)).astype(np.float32)
    w = rng.uniform(0.5, 1.5, 40).astype(np.float32)
    a = oracle.rmsnorm_dynamic_quant_fwd(x, w, 0.0, qtype)
    b = oracle.rmsnorm_dynamic_quant_fwd(x * np.float32(8.0), w, 0.0, qtype)
    assert np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2])

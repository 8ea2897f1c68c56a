"""Pins for the CPU oracle: closed forms, exact special cases, invariants and an
exact-arithmetic brute force.  None of these re-run the oracle's own formula at
the same precision; each is chosen so that a plausible slip in the oracle
(dropped or misplaced eps, wrong divisor, wrong sign, wrong or transposed index,
rounding twice or in the wrong mode, normalising the unrounded residual sum)
fails at least one of them.

Formula being pinned: y = x * rsqrt(mean(x^2) + eps) * w with eps inside the
root and mean = sum / hidden (xserv phase 4, csrc/normalization/rmsnorm.cu and
docs/04-transformer-kernels.md "RMSNorm"); fp32 math, one rounding at
write-back, never before the weight multiply (gollamago README, "RMSNorm 优化
（TileLang）").
"""
import math
import os
import struct
from decimal import Decimal
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests import exact

EPS5 = float(np.float32(1e-5))  # the fp32 value that actually crosses the ABI
EPS6 = float(np.float32(1e-6))
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16_row(vals):
    return np.array([[exact.round_bf16_exact(Fraction(v)) for v in vals]], dtype=np.uint16)


def f32_row(vals):
    return np.array([vals], dtype=np.float32)


def bf16_of(bits):
    return float(exact.bf16_value(int(bits)))


# ---------------------------------------------------------------- rounding


def test_round_bf16_matches_exact_rational_rounding():
    rng = np.random.default_rng(1)
    vals = list(rng.standard_normal(2000) * np.exp(rng.uniform(-30, 30, 2000)))
    vals += [0.0, -0.0, 1.0, -1.0, 3.3895313892515355e38, 3.4e38, -3.5e38, 1e-40, -1e-42,
             9.18e-41, 2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135, 1.0 + 2.0 ** -8,
             1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -40]
    for v in vals:
        want = exact.round_bf16_exact(Fraction(v))
        if v == 0.0 or want & 0x7FFF == 0:
            want |= 0x8000 if math.copysign(1.0, v) < 0 else 0  # Fraction drops the sign of zero
        got = oracle.round_bf16(v)
        assert got == want, (v, hex(got), hex(want))


def test_round_bf16_ties_go_to_even():
    # exact midpoints between consecutive bf16 values, in normal and subnormal range
    for base_bits in (0x3F80, 0x3F81, 0x4049, 0x0001, 0x0002, 0x7F7E, 0x00FF, 0x0100):
        lo = exact.bf16_value(base_bits)
        hi = exact.bf16_value(base_bits + 1)
        mid = (lo + hi) / 2
        want = base_bits if base_bits % 2 == 0 else base_bits + 1
        assert oracle.round_bf16(float(mid)) == want
        assert oracle.round_bf16(-float(mid)) == (want | 0x8000)
    # halfway past the largest finite value overflows; just below it does not
    top = exact.bf16_value(0x7F7F)
    spacing = top - exact.bf16_value(0x7F7E)
    assert oracle.round_bf16(float(top + spacing / 2)) == 0x7F80
    assert oracle.round_bf16(float(top + spacing / 2 - spacing / 64)) == 0x7F7F


def test_round_bf16_special_values():
    assert oracle.round_bf16(float("inf")) == 0x7F80
    assert oracle.round_bf16(float("-inf")) == 0xFF80
    assert oracle.round_bf16(float("nan")) & 0x7FFF > 0x7F80
    assert oracle.round_bf16(-0.0) == 0x8000


def test_round_f32_matches_exact_rational_rounding():
    rng = np.random.default_rng(2)
    vals = list(rng.standard_normal(500) * np.exp(rng.uniform(-80, 80, 500)))
    one = Fraction(1)
    vals += [float(one + Fraction(1, 2 ** 24)), float(one + Fraction(3, 2 ** 24)), 1e-45, 7e-46]
    for v in vals:
        want = exact.round_f32_exact(Fraction(v))
        if want & 0x7FFFFFFF == 0:
            want |= 0x80000000 if math.copysign(1.0, v) < 0 else 0
        got = exact.f32_bits(oracle.round_f32(v))
        assert got == want, v


# ---------------------------------------------------------------- closed forms


def test_hand_computed_four_element_example():
    """x = [1, 2, 3, 4], w = 1, eps = 0: mean(x^2) = 30/4 = 7.5, so
    y_j = x_j / sqrt(7.5) = x_j * sqrt(2/15).  Worked by hand; the test
    evaluates sqrt(2/15) to 80 digits and rounds exactly."""
    x = [1.0, 2.0, 3.0, 4.0]
    k = (Decimal(2) / Decimal(15)).sqrt()
    exact_y = [Decimal(v) * k for v in x]
    assert abs(exact_y[0] - Decimal("0.36514837167011074230")) < Decimal("1e-19")
    w = [1.0] * 4
    yb = oracle.rmsnorm_fwd(bf16_row(x), bf16_row(w)[0], 0.0)[0]
    assert [int(b) for b in yb] == [exact.round_bf16_exact(Fraction(v)) for v in exact_y]
    assert [int(b) for b in yb] == [0x3EBB, 0x3F3B, 0x3F8C, 0x3FBB]
    yf = oracle.rmsnorm_fwd(f32_row(x), np.ones(4, np.float32), 0.0)[0]
    assert [exact.f32_bits(float(v)) for v in yf] == [exact.round_f32_exact(Fraction(v)) for v in exact_y]
    # the same row with eps = fp32(1e-5): y_j = x_j / sqrt(7.5 + eps)
    k2 = 1 / (Decimal(7.5) + Decimal(Fraction(EPS5).numerator) / Decimal(Fraction(EPS5).denominator)).sqrt()
    yf2 = oracle.rmsnorm_fwd(f32_row(x), np.ones(4, np.float32), 1e-5)[0]
    assert [exact.f32_bits(float(v)) for v in yf2] == [
        exact.round_f32_exact(Fraction(Decimal(v) * k2)) for v in x]
    assert yf2[0] != yf[0]  # eps is not dropped


def test_exact_example_every_dtype_bitwise():
    """x = [2, -2, 2, -2]: mean(x^2) = 4, rsqrt = 1/2, so y = x * w / 2 exactly."""
    x = [2.0, -2.0, 2.0, -2.0]
    w = [0.5, 1.0, 1.5, 2.0]
    want = [0.5, -1.0, 1.5, -2.0]
    yb = oracle.rmsnorm_fwd(bf16_row(x), bf16_row(w)[0], 0.0)[0]
    assert [int(b) for b in yb] == [0x3F00, 0xBF80, 0x3FC0, 0xC000]
    yf = oracle.rmsnorm_fwd(f32_row(x), np.array(w, np.float32), 0.0)[0]
    assert list(yf) == want


@pytest.mark.parametrize("c,eps,dtype", [(3.0, EPS5, "bf16"), (3.0, EPS5, "f32"),
                                         (-0.5, EPS6, "f32"), (1e-3, EPS6, "f32"),
                                         (1e-3, EPS6, "bf16"), (0.0078125, EPS5, "f32")])
def test_constant_row_closed_form(c, eps, dtype):
    """A constant row c: mean(x^2) = c^2, so y_j = c / sqrt(c^2 + eps) * w_j.
    With eps comparable to c^2 (c = 1e-3, eps = 1e-6) the eps term changes the
    result by a factor 1/sqrt(2), so dropping or misplacing it fails."""
    w = [1.0, -1.0, 0.5, 2.0, 0.75, -1.25, 3.0, 0.125]
    H = len(w)
    if dtype == "bf16":
        xb = bf16_row([c] * H)
        wb = bf16_row(w)[0]
        cq = exact.bf16_value(int(xb[0, 0]))
        y = oracle.rmsnorm_fwd(xb, wb, eps)[0]
        ws = [exact.bf16_value(int(b)) for b in wb]
    else:
        cq = Fraction(float(np.float32(c)))
        y = oracle.rmsnorm_fwd(f32_row([c] * H), np.array(w, np.float32), eps)[0]
        ws = [Fraction(float(np.float32(v))) for v in w]
    dc = Decimal(cq.numerator) / Decimal(cq.denominator)
    de = Decimal(Fraction(eps).numerator) / Decimal(Fraction(eps).denominator)
    scale = dc / (dc * dc + de).sqrt()
    for j in range(H):
        q = Fraction(scale * Decimal(ws[j].numerator) / Decimal(ws[j].denominator))
        if dtype == "bf16":
            assert int(y[j]) == exact.round_bf16_exact(q)
        else:
            assert exact.f32_bits(float(y[j])) == exact.round_f32_exact(q)


def test_single_column_rows():
    """hidden = 1: y = x / sqrt(x^2 + eps) * w; for x = -0.5, eps = fp32(1e-6):
    -0.5 / sqrt(0.25 + 1e-6) = -0.999998000006..."""
    x = np.array([[-0.5], [0.25], [4.0]], np.float32)
    y = oracle.rmsnorm_fwd(x, np.array([1.0], np.float32), 1e-6)
    de = Decimal(Fraction(EPS6).numerator) / Decimal(Fraction(EPS6).denominator)
    for i in range(3):
        xv = Decimal(float(x[i, 0]))
        q = Fraction(xv / (xv * xv + de).sqrt())
        assert exact.f32_bits(float(y[i, 0])) == exact.round_f32_exact(q)
    assert abs(float(y[0, 0]) + 0.999998000006005) < 1e-7
    yb = oracle.rmsnorm_fwd(bf16_row([-0.5]).reshape(1, 1), bf16_row([1.0])[0], 1e-6)
    assert int(yb[0, 0]) == 0xBF80


# ---------------------------------------------------------------- invariants


@pytest.mark.parametrize("k", [-6, 3, 10])
def test_power_of_two_scale_invariance_bitwise(k):
    """With eps = 0 every step scales exactly under x -> 2^k x, so outputs are identical;
    with eps > 0, y(2^k x; eps) == y(x; eps / 4^k) exactly."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 77)).astype(np.float32)
    w = (1 + 0.1 * rng.standard_normal(77)).astype(np.float32)
    a = np.float32(2.0 ** k)
    assert np.array_equal(oracle.rmsnorm_fwd(x * a, w, 0.0), oracle.rmsnorm_fwd(x, w, 0.0))
    eps = 2.0 ** -14
    assert np.array_equal(oracle.rmsnorm_fwd(x * a, w, eps),
                          oracle.rmsnorm_fwd(x, w, eps / float(a) ** 2))
    xb = bits_bf16(x)
    wb = bits_bf16(w)
    xb2 = bits_bf16(x * a)
    assert np.array_equal(oracle.rmsnorm_fwd(xb2, wb, 0.0), oracle.rmsnorm_fwd(xb, wb, 0.0))


def bits_bf16(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_row_independence_and_layout():
    """Each output row depends on its own input row only (catches transposed or
    cross-row indexing): a stacked call equals per-row calls bitwise."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal((7, 33)).astype(np.float32) * np.arange(1, 8, dtype=np.float32)[:, None]
    w = rng.uniform(0.5, 1.5, 33).astype(np.float32)
    full = oracle.rmsnorm_fwd(x, w, 1e-5)
    for i in range(7):
        assert np.array_equal(full[i], oracle.rmsnorm_fwd(x[i:i + 1], w, 1e-5)[0])
    xb, wb = bits_bf16(x), bits_bf16(w)
    fullb = oracle.rmsnorm_fwd(xb, wb, 1e-5)
    for i in range(7):
        assert np.array_equal(fullb[i], oracle.rmsnorm_fwd(xb[i:i + 1], wb, 1e-5)[0])


def test_column_permutation_equivariance():
    """Permuting the columns of x and w together permutes y (bitwise except where the
    reordered fp64 sum moves a value across a rounding midpoint)."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((9, 300)).astype(np.float32)
    w = rng.uniform(0.5, 1.5, 300).astype(np.float32)
    perm = rng.permutation(300)
    y = oracle.rmsnorm_fwd(x, w, 1e-5)
    yp = oracle.rmsnorm_fwd(np.ascontiguousarray(x[:, perm]), np.ascontiguousarray(w[perm]), 1e-5)
    rel = np.abs(yp - y[:, perm]) / np.abs(y[:, perm])
    assert rel.max() <= 2.0 ** -23
    assert np.mean(yp == y[:, perm]) > 0.999


def test_rms_identity():
    """eps = 0: mean_j (y_j / w_j)^2 = 1 (exact in real arithmetic); fp32 outputs
    keep it to the size of one fp32 rounding."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal((4, 1000)).astype(np.float32) * 3
    w = rng.uniform(0.5, 1.5, 1000).astype(np.float32)
    y = oracle.rmsnorm_fwd(x, w, 0.0).astype(np.float64)
    m = np.mean((y / w.astype(np.float64)) ** 2, axis=1)
    assert np.all(np.abs(m - 1) < 2.5e-7)


def test_zero_row_and_signs():
    x = np.zeros((2, 16), np.float32)
    x[1] = np.linspace(-2, 2, 16, dtype=np.float32)
    w = np.linspace(-1, 1.5, 16).astype(np.float32)
    y = oracle.rmsnorm_fwd(x, w, 1e-5)
    assert np.all(y[0] == 0)
    prod = x[1].astype(np.float64) * w
    assert np.all(np.sign(y[1]) == np.sign(prod))


# ---------------------------------------------------------------- brute force


def _brute_force_check(xr, wr, eps, dtype, y):
    """Compare one oracle row against 80-digit arithmetic + exact rounding."""
    if dtype == "bf16":
        v = [exact.bf16_value(int(b)) for b in xr]
        ws = [exact.bf16_value(int(b)) for b in wr]
    else:
        v = [Fraction(float(a)) for a in xr]
        ws = [Fraction(float(a)) for a in wr]
    ref = exact.rmsnorm_decimal(v, ws, float(np.float32(eps)))
    flagged = 0
    for j, q in enumerate(ref):
        qf = Fraction(q)
        if dtype == "bf16":
            want = exact.round_bf16_exact(qf)
            got = int(y[j])
            if got != want:
                lo = exact.bf16_value(want)
                sp = abs(exact.bf16_value(want + 1) - lo) if want & 0x7FFF else Fraction(1, 2 ** 133)
                assert exact.near_midpoint(qf, lo, sp, 1e-12), (j, hex(got), hex(want))
                flagged += 1
        else:
            want = exact.round_f32_exact(qf)
            got = exact.f32_bits(float(y[j]))
            if got != want:
                lo = exact.f32_value(want)
                sp = abs(exact.f32_value(want + 1) - lo)
                assert exact.near_midpoint(qf, lo, sp, 1e-12), (j, hex(got), hex(want))
                flagged += 1
    return flagged


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_brute_force_tiny_rows(dtype):
    """Random tiny rows: the oracle agrees bitwise with 80-digit arithmetic followed
    by exact nearest-even rounding (a double rounding, e.g. rounding x*r before the
    weight multiply, would show up here)."""
    rng = np.random.default_rng(7 if dtype == "bf16" else 8)
    flagged = 0
    for H in (1, 2, 3, 5, 8, 13, 16):
        x = (rng.standard_normal((3, H)) * np.exp(rng.uniform(-3, 3, (3, 1)))).astype(np.float32)
        w = rng.uniform(-2, 2, H).astype(np.float32)
        for eps in (0.0, 1e-5, 0.5):
            if dtype == "bf16":
                xb, wb = bits_bf16(x), bits_bf16(w)
                if eps == 0.0 and np.any(np.all((xb & 0x7FFF) == 0, axis=1)):
                    continue
                y = oracle.rmsnorm_fwd(xb, wb, eps)
                for i in range(3):
                    flagged += _brute_force_check(xb[i], wb, eps, dtype, y[i])
            else:
                y = oracle.rmsnorm_fwd(x, w, eps)
                for i in range(3):
                    flagged += _brute_force_check(x[i], w, eps, dtype, y[i])
    assert flagged <= 1


def test_brute_force_detects_round_before_weight():
    """Sanity of the brute force itself: rounding x*r to bf16 first and then
    multiplying by w (the variant the gollamago README calls a precision loss)
    disagrees with the single rounding on a visible fraction of elements."""
    rng = np.random.default_rng(9)
    x = bits_bf16(rng.standard_normal((1, 64)).astype(np.float32))
    w = bits_bf16(rng.uniform(0.5, 1.5, 64).astype(np.float32))
    v = [exact.bf16_value(int(b)) for b in x[0]]
    ws = [exact.bf16_value(int(b)) for b in w]
    ref = exact.rmsnorm_decimal(v, [Fraction(1)] * 64, EPS5)
    twice = [exact.round_bf16_exact(exact.bf16_value(exact.round_bf16_exact(Fraction(q))) * ws[j])
             for j, q in enumerate(ref)]
    y = oracle.rmsnorm_fwd(x, w[0] if w.ndim == 2 else w.reshape(-1), 1e-5)[0]
    assert sum(int(a) != b for a, b in zip(y, twice)) >= 5


# ---------------------------------------------------------------- fused residual


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_residual_sum_rounded_once(dtype):
    """h = x + residual, rounded once from the exact sum (bitwise)."""
    rng = np.random.default_rng(10)
    x = (rng.standard_normal((6, 40)) * np.exp(rng.uniform(-8, 8, (6, 40)))).astype(np.float32)
    r = (rng.standard_normal((6, 40)) * np.exp(rng.uniform(-8, 8, (6, 40)))).astype(np.float32)
    w = rng.uniform(0.5, 1.5, 40).astype(np.float32)
    if dtype == "bf16":
        xb, rb, wb = bits_bf16(x), bits_bf16(r), bits_bf16(w)
        h, _ = oracle.rmsnorm_residual_fwd(xb, rb, wb, 1e-5)
        for i in range(6):
            for j in range(40):
                q = exact.bf16_value(int(xb[i, j])) + exact.bf16_value(int(rb[i, j]))
                assert int(h[i, j]) == exact.round_bf16_exact(q)
    else:
        h, _ = oracle.rmsnorm_residual_fwd(x, r, w, 1e-5)
        for i in range(6):
            for j in range(40):
                q = Fraction(float(x[i, j])) + Fraction(float(r[i, j]))
                assert exact.f32_bits(float(h[i, j])) == exact.round_f32_exact(q)


def test_residual_normalises_the_rounded_sum():
    """y is RMSNorm of the stored (rounded) h, checked against 80-digit arithmetic on
    the rounded h; the unrounded-sum variant differs on this data."""
    rng = np.random.default_rng(11)
    x = bits_bf16(rng.standard_normal((3, 16)).astype(np.float32))
    r = bits_bf16((rng.standard_normal((3, 16)) * 0.01).astype(np.float32))
    w = bits_bf16(rng.uniform(0.5, 1.5, 16).astype(np.float32))
    h, y = oracle.rmsnorm_residual_fwd(x, r, w, 1e-5)
    for i in range(3):
        assert _brute_force_check(h[i], w, 1e-5, "bf16", y[i]) == 0
    # normalising the exact (unrounded) sum instead gives different bits somewhere
    diffs = 0
    for i in range(3):
        v = [exact.bf16_value(int(a)) + exact.bf16_value(int(b)) for a, b in zip(x[i], r[i])]
        ref = exact.rmsnorm_decimal(v, [exact.bf16_value(int(b)) for b in w], EPS5)
        diffs += sum(exact.round_bf16_exact(Fraction(q)) != int(y[i, j]) for j, q in enumerate(ref))
    assert diffs > 0


def test_residual_special_cases_reduce_to_plain():
    rng = np.random.default_rng(12)
    x = bits_bf16(rng.standard_normal((4, 50)).astype(np.float32))
    w = bits_bf16(rng.uniform(0.5, 1.5, 50).astype(np.float32))
    zeros = np.zeros_like(x)
    h, y = oracle.rmsnorm_residual_fwd(x, zeros, w, 1e-5)
    assert np.array_equal(h, x)
    assert np.array_equal(y, oracle.rmsnorm_fwd(x, w, 1e-5))
    h2, y2 = oracle.rmsnorm_residual_fwd(zeros, x, w, 1e-5)
    assert np.array_equal(h2, x) and np.array_equal(y2, y)


# ---------------------------------------------------------------- the pages' own test


def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    return vals


def test_pages_rmsnorm_test_case():
    """The xserv RMSNorm tests' own data and tolerances (see the golden file):
    the oracle passes the same check the pages' GPU kernel passed against their
    f32 CPU reference, with an error of the order they printed."""
    g = _read_golden("xserv_rmsnorm_test.txt")
    rows, hidden, eps = int(g["rows"]), int(g["hidden"]), float(g["eps"])
    i = np.arange(rows * hidden)
    x = (((i % 17).astype(np.float32) - np.float32(8.0)) * np.float32(0.1)).reshape(rows, hidden)
    gamma = (np.float32(0.5) + (np.arange(hidden) % 3).astype(np.float32) * np.float32(0.2)).astype(np.float32)
    # the pages' CPU reference in f32: sequential sum, then 1/sqrt(sum/hidden + eps)
    ref = np.empty_like(x)
    for r in range(rows):
        s = np.float32(0.0)
        for v in x[r]:
            s = np.float32(s + v * v)
        inv = np.float32(1.0) / np.sqrt(np.float32(s / np.float32(hidden) + np.float32(eps)))
        ref[r] = x[r] * inv * gamma
    y32 = oracle.rmsnorm_fwd(x, gamma, eps)
    err32 = float(np.max(np.abs(y32 - ref)))
    assert err32 <= float(g["f32_atol"])
    assert err32 <= 10 * float(g["f32_printed_max_err"])
    yb = oracle.rmsnorm_fwd(bits_bf16(x), bits_bf16(gamma), eps)
    yb_f = np.array([bf16_of(b) for b in yb.reshape(-1)], np.float64).reshape(rows, hidden)
    errb = float(np.max(np.abs(yb_f - ref)))
    assert errb <= float(g["bf16_atol"])
    assert errb <= 2 * float(g["bf16_printed_max_err"])

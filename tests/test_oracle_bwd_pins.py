"""Pins for the oracle's RMSNorm backward (dx and dweight).

The pages name the norm backward only as part of a training step's backward
stage (TileLang tutorial ch. 02, section 1.1(b)) and print no formula, so the
oracle writes out the plain derivative.  None of the pins below restate that
derivative: they differentiate the forward numerically in 80-digit decimal
arithmetic, or check consequences of the forward's structure:
  * central differences of L = sum(dy * y) in exact-input decimal arithmetic,
    rounded once, must give the oracle's bits (except within 1e-9 of a tie);
  * hidden = 1 has the closed form dx = dy * w * eps / (x^2 + eps)^1.5;
  * at eps = 0 the forward is scale invariant, so <dx, x> = 0 per row and
    dx(2^k x) = 2^-k dx(x), dw(2^k x) = dw(x) bit for bit;
  * <dw, w> = sum(dy * y) (y is linear in w);
  * the map is linear in dy; rows are independent; dw sums over rows.
"""
from decimal import Decimal
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests import exact
from tests.test_oracle_pins import EPS5, EPS6

H = Decimal(10) ** -25  # finite-difference step (inputs are O(1); 80 digits carried)


def _rand(rows, hidden, dtype, rng, scale=1.0, loc=0.0):
    a = (rng.standard_normal((rows, hidden)) * scale + loc).astype(np.float32)
    if dtype == "f32":
        return a
    return np.array([[exact.round_bf16_exact(Fraction(float(v))) for v in row] for row in a], dtype=np.uint16)


def _value(bits, dtype) -> Fraction:
    return exact.bf16_value(int(bits)) if dtype == "bf16" else Fraction(float(bits))


def _dec(q: Fraction) -> Decimal:
    return Decimal(q.numerator) / Decimal(q.denominator)


def _loss_row(v, w, g, eps):
    """sum_j g_j * y_j of one row, decimal, from exact inputs."""
    y = exact.rmsnorm_decimal(v, w, eps)
    return sum(_dec(Fraction(a)) * b for a, b in zip(g, y))


def _round(q, dtype) -> int:
    return exact.round_bf16_exact(q) if dtype == "bf16" else exact.round_f32_exact(q)


def _pattern_value(b: int, dtype) -> Fraction:
    return exact.bf16_value(b) if dtype == "bf16" else exact.f32_value(b)


def _key(b: int, dtype) -> int:
    sign, mag = (0x8000, 0x7FFF) if dtype == "bf16" else (0x80000000, 0x7FFFFFFF)
    return -(b & mag) if b & sign else b & mag


def _bits(a, dtype):
    return [int(v) for v in a] if dtype == "bf16" else [exact.f32_bits(float(v)) for v in a]


def _check_rounded(got: int, exact_val: Decimal, dtype, what):
    """got must be the nearest-even pattern of the exact value, or its
    neighbour when the exact value is within 1e-9 (relative) of their midpoint."""
    q = Fraction(exact_val)
    want = _round(q, dtype)
    d = abs(_key(got, dtype) - _key(want, dtype))
    if d == 0:
        return
    if d == 1:
        mid = (_pattern_value(got, dtype) + _pattern_value(want, dtype)) / 2
        if abs(q - mid) <= Fraction(1, 10 ** 9) * abs(q):
            return
    raise AssertionError("%s: got 0x%x want 0x%x (exact %s)" % (what, got, want, exact_val))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("hidden", [2, 5, 8])
def test_matches_decimal_central_differences(dtype, hidden):
    rng = np.random.default_rng(100 + hidden)
    rows = 3
    x = _rand(rows, hidden, dtype, rng)
    dy = _rand(rows, hidden, dtype, rng)
    w = _rand(1, hidden, dtype, rng, 0.3, 1.0)[0]
    eps = EPS5 if hidden != 5 else 0.25  # a large eps makes its term visible
    dx, dw = oracle.rmsnorm_bwd(x, w, dy, eps)
    xv = [[_value(b, dtype) for b in row] for row in x]
    gv = [[_value(b, dtype) for b in row] for row in dy]
    wv = [_value(b, dtype) for b in w]
    dxb = [_bits(row, dtype) for row in dx]
    dwb = _bits(dw, dtype)
    for i in range(rows):
        for k in range(hidden):
            up = [_dec(v) for v in xv[i]]
            dn = list(up)
            up[k] += H
            dn[k] -= H
            d = (_loss_row(up, wv, gv[i], eps) - _loss_row(dn, wv, gv[i], eps)) / (2 * H)
            _check_rounded(dxb[i][k], d, dtype, "dx[%d,%d]" % (i, k))
    for k in range(hidden):
        up = [_dec(v) for v in wv]
        dn = list(up)
        up[k] += H
        dn[k] -= H
        d = sum(_loss_row(xv[i], up, gv[i], eps) - _loss_row(xv[i], dn, gv[i], eps) for i in range(rows)) / (2 * H)
        _check_rounded(dwb[k], d, dtype, "dw[%d]" % k)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_column_closed_form(dtype):
    rng = np.random.default_rng(7)
    rows = 12
    x = _rand(rows, 1, dtype, rng, 2.0)
    dy = _rand(rows, 1, dtype, rng)
    w = _rand(1, 1, dtype, rng, 0.3, 1.0)[0]
    eps = 0.0625
    dx, dw = oracle.rmsnorm_bwd(x, w, dy, eps)
    wv = _value(w[0], dtype)
    e = Decimal(eps)
    acc = Decimal(0)
    for i in range(rows):
        xv = _dec(_value(x[i, 0], dtype))
        gv = _dec(_value(dy[i, 0], dtype))
        den = (xv * xv + e).sqrt()
        _check_rounded(_bits(dx[i], dtype)[0], gv * _dec(wv) * e / (den * den * den), dtype, "dx[%d]" % i)
        acc += gv * xv / den
    _check_rounded(_bits(dw, dtype)[0], acc, dtype, "dw")


def test_orthogonal_to_x_without_eps():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((16, 1024)).astype(np.float32) * 3
    dy = rng.standard_normal((16, 1024)).astype(np.float32)
    w = (rng.standard_normal(1024) * 0.1 + 1).astype(np.float32)
    dx, _ = oracle.rmsnorm_bwd(x, w, dy, 0.0, want_dw=False)
    p = dx.astype(np.float64) * x.astype(np.float64)
    assert np.all(np.abs(p.sum(axis=1)) <= 2.0 ** -22 * np.abs(p).sum(axis=1))
    assert np.all(np.abs(p).sum(axis=1) > 0)


def test_eps_component_along_x():
    """With eps > 0 the radial part is what eps leaves: <dx, x> = sum(dy * y) * eps / (m + eps),
    m = mean(x^2) -- d/dt y(x(1+t)) at t = 0."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal((8, 256)).astype(np.float32) * 0.5
    dy = rng.standard_normal((8, 256)).astype(np.float32)
    w = (rng.standard_normal(256) * 0.1 + 1).astype(np.float32)
    eps = 0.125
    dx, _ = oracle.rmsnorm_bwd(x, w, dy, eps, want_dw=False)
    xd = x.astype(np.float64)
    m = (xd * xd).mean(axis=1)
    y = xd / np.sqrt(m + eps)[:, None] * w.astype(np.float64)
    want = (dy.astype(np.float64) * y).sum(axis=1) * eps / (m + eps)
    p = dx.astype(np.float64) * xd
    assert np.all(np.abs(p.sum(axis=1) - want) <= 2.0 ** -22 * np.abs(p).sum(axis=1))
    assert np.all(np.abs(want) > 1e-3 * np.abs(p).sum(axis=1))  # the eps term is not negligible here


@pytest.mark.parametrize("k", [-3, 5])
def test_power_of_two_scaling_without_eps(k):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((6, 96)).astype(np.float32)
    dy = rng.standard_normal((6, 96)).astype(np.float32)
    w = (rng.standard_normal(96) * 0.1 + 1).astype(np.float32)
    dx1, dw1 = oracle.rmsnorm_bwd(x, w, dy, 0.0)
    dx2, dw2 = oracle.rmsnorm_bwd(x * np.float32(2.0 ** k), w, dy, 0.0)
    assert np.array_equal(dx2, dx1 * np.float32(2.0 ** -k))
    assert np.array_equal(dw2, dw1)


def test_weight_gradient_identity():
    """y is linear in w, so <dw, w> = sum(dy * y) over all rows."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal((64, 300)).astype(np.float32)
    dy = rng.standard_normal((64, 300)).astype(np.float32)
    w = (rng.standard_normal(300) * 0.5 + 1).astype(np.float32)
    _, dw = oracle.rmsnorm_bwd(x, w, dy, EPS6)
    xd = x.astype(np.float64)
    y = xd / np.sqrt((xd * xd).mean(axis=1) + EPS6)[:, None] * w.astype(np.float64)
    want = (dy.astype(np.float64) * y).sum()
    got = (dw.astype(np.float64) * w.astype(np.float64)).sum()
    assert abs(got - want) <= 1e-6 * np.abs(dw.astype(np.float64) * w).sum()


def test_linear_in_dy_and_zero_gradient():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((5, 40)).astype(np.float32)
    dy = rng.standard_normal((5, 40)).astype(np.float32)
    w = (rng.standard_normal(40) * 0.1 + 1).astype(np.float32)
    dx1, dw1 = oracle.rmsnorm_bwd(x, w, dy, EPS5)
    dx2, dw2 = oracle.rmsnorm_bwd(x, w, dy * np.float32(4.0), EPS5)
    assert np.array_equal(dx2, dx1 * 4) and np.array_equal(dw2, dw1 * 4)
    dx0, dw0 = oracle.rmsnorm_bwd(x, w, np.zeros_like(dy), EPS5)
    assert not np.any(dx0) and not np.any(dw0)
    # the zero row: dx = dy * w / sqrt(eps), dw gets nothing from it
    xz = x.copy()
    xz[2] = 0
    dxz, _ = oracle.rmsnorm_bwd(xz, w, dy, 0.25)
    assert np.array_equal(dxz[2], (dy[2].astype(np.float64) * w / 0.5).astype(np.float32))


def test_rows_independent_and_dw_sums_rows():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((7, 33)).astype(np.float32)  # rows != hidden: catches a transposed index
    dy = rng.standard_normal((7, 33)).astype(np.float32)
    w = (rng.standard_normal(33) * 0.3 + 1).astype(np.float32)
    dx, dw = oracle.rmsnorm_bwd(x, w, dy, EPS5)
    parts = np.zeros(33)
    for i in range(7):
        dxi, dwi = oracle.rmsnorm_bwd(x[i:i + 1], w, dy[i:i + 1], EPS5)
        assert np.array_equal(dxi[0], dx[i])
        parts += dwi.astype(np.float64)
    assert np.allclose(dw, parts, rtol=1e-6, atol=1e-6)
    _, none = oracle.rmsnorm_bwd(x, w, dy, EPS5, want_dw=False)
    assert none is None
    e, ew = oracle.rmsnorm_bwd(x[:0], w, dy[:0], EPS5)
    assert e.shape == (0, 33) and not np.any(ew)

"""Pins for the oracle's LayerNorm (y = gamma * (x - mean) / sqrt(var + eps) + beta,
biased variance; xserv "phase 4: transformer core kernels",
csrc/normalization/layernorm.cu and docs/04-transformer-kernels.md "LayerNorm").

None of these re-runs the oracle's formula at its precision:
  * torch's own layer_norm in float64 on the CPU (a library routine), rounded
    once to the dtype, gives the oracle's bits except within 1e-9 of a tie;
  * hidden = 2 has the closed form y = +-d / sqrt(d^2 + eps) * gamma + beta,
    d = (a - b) / 2 (exactly +-gamma + beta at eps = 0, which pins the biased
    divisor);
  * constant rows and hidden = 1 give beta exactly;
  * adding a constant to a row (exactly representable) changes no bit, nor does
    a power-of-two scale at eps = 0, nor negating x with beta = 0 (sign);
  * with gamma = 1, beta = 0 the output has mean 0 and mean square
    var / (var + eps);
  * the pages' own test case passes the pages' tolerance with an error of the
    printed order.
"""
import os
from decimal import Decimal
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests import exact
from tests.test_oracle_pins import EPS5, bits_bf16, bf16_of, _read_golden


def _vals(a):
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _store(a: np.ndarray, dtype: str) -> np.ndarray:
    return a.astype(np.float32) if dtype == "f32" else bits_bf16(a.astype(np.float32))


def _round_bits(v: float, dtype: str) -> int:
    return exact.round_bf16_exact(Fraction(v)) if dtype == "bf16" else exact.round_f32_exact(Fraction(v))


def _bits(a, dtype):
    return [int(b) for b in a.reshape(-1)] if dtype == "bf16" else [exact.f32_bits(float(b)) for b in a.reshape(-1)]


def _close_to_tie(v: float, got: int, want: int, dtype: str) -> bool:
    val = exact.bf16_value if dtype == "bf16" else exact.f32_value
    mid = (val(got) + val(want)) / 2
    return abs(Fraction(v) - mid) <= Fraction(1, 10 ** 9) * abs(Fraction(v))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("with_beta", [True, False])
def test_matches_torch_layer_norm_in_float64(dtype, with_beta):
    rng = np.random.default_rng(11)
    rows, hidden = 24, 300
    x = _store(rng.standard_normal((rows, hidden)) * 2 + 0.5, dtype)
    g = _store(rng.standard_normal(hidden) * 0.2 + 1.0, dtype)
    b = _store(rng.standard_normal(hidden) * 0.1, dtype) if with_beta else None
    got = oracle.layernorm_fwd(x, g, b, EPS5)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(_vals(x)), (hidden,), torch.from_numpy(_vals(g)),
                                         torch.from_numpy(_vals(b)) if b is not None else None, EPS5).numpy()
    gb = _bits(got, dtype)
    for k, v in enumerate(ref.reshape(-1)):
        want = _round_bits(float(v), dtype)
        if gb[k] != want:
            assert _close_to_tie(float(v), gb[k], want, dtype), (k, v, gb[k], want)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_two_columns_closed_form(dtype):
    rng = np.random.default_rng(12)
    x = _store(rng.standard_normal((40, 2)) * 3, dtype)
    g = _store(np.array([1.25, -0.75]), dtype)
    b = _store(np.array([0.5, -0.25]), dtype)
    y0 = oracle.layernorm_fwd(x, g, b, 0.0)
    gv, bv = _vals(g), _vals(b)
    for i, (a, c) in enumerate(_vals(x)):
        if a == c:
            continue
        s = 1.0 if a > c else -1.0
        want = [_round_bits(s * gv[0] + bv[0], dtype), _round_bits(-s * gv[1] + bv[1], dtype)]
        assert _bits(y0[i], dtype) == want, i
    eps = 0.5
    y1 = oracle.layernorm_fwd(x, g, b, eps)
    for i, (a, c) in enumerate(_vals(x)):
        d = (Decimal(a) - Decimal(c)) / 2
        r = d / (d * d + Decimal(eps)).sqrt()
        for j, sign in ((0, 1), (1, -1)):
            v = Fraction(sign * r * Decimal(gv[j]) + Decimal(bv[j]))
            want = _round_bits(v, dtype)
            got = _bits(y1[i], dtype)[j]
            assert got == want or _close_to_tie(float(v), got, want, dtype), (i, j)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_constant_rows_and_single_column_give_beta(dtype):
    rng = np.random.default_rng(13)
    g = _store(rng.standard_normal(64) + 1, dtype)
    b = _store(rng.standard_normal(64), dtype)
    x = _store(np.repeat(rng.standard_normal((5, 1)) * 10, 64, axis=1), dtype)
    assert np.array_equal(oracle.layernorm_fwd(x, g, b, EPS5), np.tile(b, (5, 1)))
    x1 = _store(rng.standard_normal((7, 1)), dtype)
    assert np.array_equal(oracle.layernorm_fwd(x1, g[:1], b[:1], EPS5), np.tile(b[:1], (7, 1)))
    y = oracle.layernorm_fwd(x1, g[:1], None, EPS5)
    assert np.all(_vals(y) == 0)


def test_shift_invariance_bitwise():
    """x + c, with x + c exact in fp32 and every fp64 sum and the mean exact
    (values on a 1/64 grid, hidden a power of two): no bit changes."""
    rng = np.random.default_rng(14)
    x = (np.round(np.clip(rng.standard_normal((9, 256)), -7, 7) * 64) / 64).astype(np.float32)
    g = (rng.standard_normal(256) * 0.2 + 1).astype(np.float32)
    b = (rng.standard_normal(256) * 0.1).astype(np.float32)
    y = oracle.layernorm_fwd(x, g, b, EPS5)
    for c in (1.0, -37.5, 4096.0, 2.0 ** 14):
        xc = x + np.float32(c)
        assert np.array_equal(xc.astype(np.float64), x.astype(np.float64) + c)  # the shift is exact
        assert np.array_equal(oracle.layernorm_fwd(xc, g, b, EPS5), y), c


def test_scale_and_sign_invariance_bitwise():
    rng = np.random.default_rng(15)
    x = rng.standard_normal((6, 128)).astype(np.float32)
    g = (rng.standard_normal(128) * 0.2 + 1).astype(np.float32)
    b = (rng.standard_normal(128) * 0.1).astype(np.float32)
    y = oracle.layernorm_fwd(x, g, b, 0.0)
    for k in (-5, 3, 12):
        assert np.array_equal(oracle.layernorm_fwd(x * np.float32(2.0 ** k), g, b, 0.0), y)
    y0 = oracle.layernorm_fwd(x, g, None, EPS5)
    assert np.array_equal(oracle.layernorm_fwd(-x, g, None, EPS5), -y0)


def test_standardised_moments():
    rng = np.random.default_rng(16)
    x = (rng.standard_normal((8, 512)) * 0.3 + 2).astype(np.float32)
    ones = np.ones(512, np.float32)
    eps = 0.01
    y = oracle.layernorm_fwd(x, ones, None, eps).astype(np.float64)
    xd = x.astype(np.float64)
    var = ((xd - xd.mean(axis=1, keepdims=True)) ** 2).mean(axis=1)
    assert np.all(np.abs(y.mean(axis=1)) < 1e-6)
    assert np.allclose((y * y).mean(axis=1), var / (var + eps), rtol=1e-6)
    y0 = oracle.layernorm_fwd(x, ones, None, 0.0).astype(np.float64)
    assert np.allclose((y0 * y0).mean(axis=1), 1.0, rtol=1e-6)


def test_rows_independent_and_layout():
    rng = np.random.default_rng(17)
    x = rng.standard_normal((5, 33)).astype(np.float32)
    g = (rng.standard_normal(33) + 1).astype(np.float32)
    b = rng.standard_normal(33).astype(np.float32)
    y = oracle.layernorm_fwd(x, g, b, EPS5)
    for i in range(5):
        assert np.array_equal(oracle.layernorm_fwd(x[i:i + 1], g, b, EPS5)[0], y[i])
    assert oracle.layernorm_fwd(x[:0], g, b, EPS5).shape == (0, 33)


def test_pages_layernorm_test_case():
    """The xserv LayerNorm test's own data and tolerance (see the golden file):
    the oracle passes the check the pages' GPU kernel passed against their f32
    CPU reference, with an error of the printed order."""
    gd = _read_golden("xserv_layernorm_test.txt")
    rows, hidden, eps = int(gd["rows"]), int(gd["hidden"]), float(gd["eps"])
    i = np.arange(rows * hidden)
    x = (((i % 17).astype(np.float32) - np.float32(8.0)) * np.float32(0.1)).reshape(rows, hidden)
    j = np.arange(hidden)
    gamma = (np.float32(0.8) + (j % 5).astype(np.float32) * np.float32(0.1)).astype(np.float32)
    beta = (((j % 7).astype(np.float32) - np.float32(3.0)) * np.float32(0.01)).astype(np.float32)
    # the pages' CPU reference in f32: sequential sums for the mean and the
    # centred squares, then 1 / sqrt(var + eps)
    ref = np.empty_like(x)
    for r in range(rows):
        s = np.float32(0.0)
        for v in x[r]:
            s = np.float32(s + v)
        mean = np.float32(s / np.float32(hidden))
        q = np.float32(0.0)
        for v in x[r]:
            q = np.float32(q + (v - mean) * (v - mean))
        inv = np.float32(1.0) / np.sqrt(np.float32(q / np.float32(hidden)) + np.float32(eps))
        ref[r] = gamma * (x[r] - mean) * inv + beta
    y = oracle.layernorm_fwd(x, gamma, beta, eps)
    err = float(np.max(np.abs(y - ref)))
    assert err <= float(gd["f32_atol"])
    assert err <= 10 * float(gd["f32_printed_max_err"])

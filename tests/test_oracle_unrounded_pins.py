"""Pins for the oracle's unrounded outputs (the float64 value each output has
before its one rounding) and for its array roundings.

The GPU comparisons take the unrounded value e of every element and accept a
result only if it is a correct nearest-even rounding of some value within the
GPU's own evaluation error of e.  That is what tells round-to-nearest-even at
write-back (gollamago README, "RMSNorm 优化（TileLang）": round once, at the
end) apart from truncation or double rounding, so e itself has to be right:
each function's unrounded output is pinned here against closed forms worked
by hand and against 80-digit decimal arithmetic, never against the oracle's
own formula run again at the same precision.
"""
import math
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from memory_bound_rmsnorm_amd import inputs
from tests import exact

EPS5 = float(np.float32(1e-5))
EPS6 = float(np.float32(1e-6))

getcontext().prec = 80


def _bf16(a) -> np.ndarray:
    a = np.asarray(a, np.float32)
    return np.array([exact.round_bf16_exact(Fraction(float(v))) for v in a.reshape(-1)],
                    np.uint16).reshape(a.shape)


def _vals(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _dec(v) -> Decimal:
    q = Fraction(float(v))
    return Decimal(q.numerator) / Decimal(q.denominator)


def _close(got: float, want: Decimal, rel: float):
    w = float(want)
    assert abs(got - w) <= rel * abs(w) + 1e-300, (got, w)


# ---------------------------------------------------------------- array roundings


def test_round_arrays_match_exact_rational_rounding():
    rng = np.random.default_rng(21)
    v = rng.standard_normal(3000) * np.exp(rng.uniform(-40, 40, 3000))
    mids = [float((exact.bf16_value(b) + exact.bf16_value(b + 1)) / 2) for b in (0x3F80, 0x3F81, 0x0001, 0x4049)]
    # just past a midpoint by far less than a float32 ulp: rounding through
    # float32 first would land on the midpoint and tie to even instead
    near = [1.0 + 2.0 ** -8 + 2.0 ** -40, -(3.0 + 2.0 ** -7 + 2.0 ** -35), 1.0 + 3 * 2.0 ** -8 - 2.0 ** -41]
    v = np.concatenate([v, mids, [-m for m in mids], near, [0.0, 1.0, -2.5, 3.5e38, 1e-41]])
    b = oracle.round_bf16_array(v)
    f = oracle.round_f32_array(v)
    for k, val in enumerate(v):
        want = exact.round_bf16_exact(Fraction(float(val)))
        if val == 0.0 or want & 0x7FFF == 0:
            want |= 0x8000 if math.copysign(1.0, val) < 0 else 0
        assert int(b[k]) == want, (val, hex(int(b[k])), hex(want))
        assert exact.f32_bits(float(f[k])) == exact.round_f32_exact(Fraction(float(val))) or \
            (val == 0.0 and f[k] == 0.0), val


# ---------------------------------------------------------------- forward


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_unrounded_hand_example(dtype):
    """x = [1, 2, 3, 4], w = 1: mean(x^2) = 7.5, y = x / sqrt(7.5 + eps); the
    eps = 0 values are x * sqrt(2/15), worked by hand."""
    x = np.array([[1.0, 2.0, 3.0, 4.0]], np.float32)
    w = np.ones(4, np.float32)
    if dtype == "bf16":
        x, w = _bf16(x), _bf16(w)
    for eps in (0.0, EPS5):
        e = oracle.rmsnorm_fwd(x, w, eps, unrounded=True)
        assert e.dtype == np.float64
        k = 1 / (Decimal(15) / Decimal(2) + _dec(eps)).sqrt()
        for j, v in enumerate((1, 2, 3, 4)):
            _close(float(e[0, j]), v * k, 4e-16)
    e0 = oracle.rmsnorm_fwd(x, w, 0.0, unrounded=True)
    _close(float(e0[0, 0]), Decimal("0.36514837167011074230"), 4e-16)


@pytest.mark.parametrize("c,eps", [(3.0, EPS5), (-0.5, EPS6), (1e-3, EPS6), (0.0078125, EPS5)])
def test_unrounded_constant_rows(c, eps):
    """A constant row: y_j = c / sqrt(c^2 + eps) * w_j."""
    w = np.array([1.0, -1.0, 0.5, 2.0, 0.75, -1.25, 3.0, 0.125], np.float32)
    x = np.full((1, 8), c, np.float32)
    e = oracle.rmsnorm_fwd(x, w, eps, unrounded=True)[0]
    cd = _dec(np.float32(c))
    s = cd / (cd * cd + _dec(eps)).sqrt()
    for j in range(8):
        _close(float(e[j]), s * _dec(w[j]), 4e-16)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_unrounded_brute_force_tiny_rows(dtype):
    """Random tiny rows against 80-digit arithmetic: the fp64 evaluation stays
    within (H + 4) * 2^-53 relative of the exact value."""
    rng = np.random.default_rng(23)
    for H in (1, 2, 3, 5, 8, 13, 16):
        x = (rng.standard_normal((3, H)) * np.exp(rng.uniform(-3, 3, (3, 1)))).astype(np.float32)
        w = rng.uniform(-2, 2, H).astype(np.float32)
        if dtype == "bf16":
            x, w = _bf16(x), _bf16(w)
        for eps in (0.0, EPS5, 0.5):
            e = oracle.rmsnorm_fwd(x, w, eps, unrounded=True)
            for i in range(3):
                v = [Fraction(float(a)) for a in _vals(x[i])]
                if eps == 0.0 and all(q == 0 for q in v):
                    continue
                ref = exact.rmsnorm_decimal(v, [Fraction(float(a)) for a in _vals(w)], eps)
                for j in range(H):
                    _close(float(e[i, j]), ref[j], (H + 8) * 2.0 ** -53)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rounding_the_unrounded_output_gives_the_rounded_output(dtype):
    """The rounded entry point stores exactly the nearest-even rounding of the
    unrounded one (same arithmetic, then one rounding)."""
    w_ = inputs.custom(37, 777, dtype, True)
    t = inputs.make(w_, seed=5)
    xb, rb, wb = (inputs.bits(t[k]) for k in ("x", "residual", "weight"))
    rnd = oracle.round_bf16_array if dtype == "bf16" else oracle.round_f32_array
    assert np.array_equal(rnd(oracle.rmsnorm_fwd(xb, wb, 1e-5, unrounded=True)), oracle.rmsnorm_fwd(xb, wb, 1e-5))
    h, y = oracle.rmsnorm_residual_fwd(xb, rb, wb, 1e-5)
    h2, e = oracle.rmsnorm_residual_fwd(xb, rb, wb, 1e-5, unrounded=True)
    assert np.array_equal(h, h2)  # h is always rounded: the norm consumes it rounded
    assert np.array_equal(rnd(e), y)


def test_unrounded_fused_output_normalises_the_rounded_sum():
    rng = np.random.default_rng(24)
    x = _bf16(rng.standard_normal((3, 16)))
    r = _bf16(rng.standard_normal((3, 16)) * 0.01)
    w = _bf16(rng.uniform(0.5, 1.5, 16))
    h, e = oracle.rmsnorm_residual_fwd(x, r, w, EPS5, unrounded=True)
    for i in range(3):
        ref = exact.rmsnorm_decimal([Fraction(float(a)) for a in _vals(h[i])],
                                    [Fraction(float(a)) for a in _vals(w)], EPS5)
        for j in range(16):
            _close(float(e[i, j]), ref[j], 24 * 2.0 ** -53)


# ---------------------------------------------------------------- backward


def _loss_row(xr, wr, gr, eps):
    s = sum(v * v for v in xr)
    r = 1 / (s / len(xr) + _dec(eps)).sqrt()
    return sum(gr[j] * xr[j] * r * wr[j] for j in range(len(xr)))


def test_unrounded_backward_matches_decimal_central_differences():
    """dx and dw unrounded against 80-digit central differences of
    L = sum(dy * RMSNorm(x) * w), step 1e-30 (truncation error ~1e-60)."""
    rng = np.random.default_rng(25)
    rows, hidden = 3, 6
    x = rng.standard_normal((rows, hidden)).astype(np.float32)
    dy = rng.standard_normal((rows, hidden)).astype(np.float32)
    w = rng.uniform(0.3, 1.0, hidden).astype(np.float32)
    eps = 0.25
    dx, dw = oracle.rmsnorm_bwd(x, w, dy, eps, unrounded=True)
    assert dx.dtype == np.float64 and dw.dtype == np.float64
    step = Decimal("1e-30")
    xv = [[_dec(v) for v in row] for row in x]
    gv = [[_dec(v) for v in row] for row in dy]
    wv = [_dec(v) for v in w]
    scale = max(abs(float(v)) for v in dx.reshape(-1))
    for i in range(rows):
        for k in range(hidden):
            up, dn = list(xv[i]), list(xv[i])
            up[k] += step
            dn[k] -= step
            d = (_loss_row(up, wv, gv[i], eps) - _loss_row(dn, wv, gv[i], eps)) / (2 * step)
            assert abs(float(dx[i, k]) - float(d)) <= 1e-14 * scale, (i, k)
    for k in range(hidden):
        up, dn = list(wv), list(wv)
        up[k] += step
        dn[k] -= step
        d = sum(_loss_row(xv[i], up, gv[i], eps) - _loss_row(xv[i], dn, gv[i], eps) for i in range(rows)) / (2 * step)
        _close(float(dw[k]), d, 1e-14)


# ---------------------------------------------------------------- LayerNorm


@pytest.mark.parametrize("with_beta", [True, False])
def test_unrounded_layernorm_matches_torch_float64(with_beta):
    rng = np.random.default_rng(26)
    rows, hidden = 16, 300
    x = _bf16(rng.standard_normal((rows, hidden)) * 2 + 0.5)
    g = _bf16(rng.standard_normal(hidden) * 0.2 + 1.0)
    b = _bf16(rng.standard_normal(hidden) * 0.1) if with_beta else None
    e = oracle.layernorm_fwd(x, g, b, EPS5, unrounded=True)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(_vals(x)), (hidden,), torch.from_numpy(_vals(g)),
                                         torch.from_numpy(_vals(b)) if b is not None else None, EPS5).numpy()
    mag = np.abs(_vals(g))[None, :] * 4 + (np.abs(_vals(b))[None, :] if b is not None else 0)
    assert np.all(np.abs(e - ref) <= 1e-13 * mag)


def test_unrounded_layernorm_two_columns():
    """Two columns a, b: mean (a + b)/2, var ((a - b)/2)^2, so the normalised
    values are +-d / sqrt(d^2 + eps) with d = (a - b)/2."""
    x = np.array([[3.0, 1.0], [-2.0, 6.0]], np.float32)
    g = np.array([1.5, -0.5], np.float32)
    bt = np.array([0.25, 2.0], np.float32)
    e = oracle.layernorm_fwd(x, g, bt, EPS5, unrounded=True)
    for i in range(2):
        d = (_dec(x[i, 0]) - _dec(x[i, 1])) / 2
        s = d / (d * d + _dec(EPS5)).sqrt()
        _close(float(e[i, 0]), _dec(g[0]) * s + _dec(bt[0]), 4e-16)
        _close(float(e[i, 1]), -_dec(g[1]) * s + _dec(bt[1]), 4e-16)


# ---------------------------------------------------------------- KV RMSNorm + RoPE + cache


@pytest.mark.parametrize("style", [oracle.ROPE_HALVES, oracle.ROPE_PAIRS])
def test_unrounded_kv_parts(style):
    """Norm part: the forward's unrounded values; rotated part: the complex
    product (a + ib)(cos + i sin) in float64 (exact products, one addition)."""
    rng = np.random.default_rng(27)
    tokens, heads, dn, dr, max_pos, slots = 6, 2, 24, 8, 16, 20
    kv = _bf16(rng.standard_normal((tokens, heads, dn + dr)))
    g = _bf16(rng.standard_normal(dn) * 0.2 + 1)
    cos_t, sin_t = inputs.rope_tables(max_pos, dr)
    pos = rng.integers(0, max_pos, tokens).astype(np.int32)
    sl = rng.permutation(slots)[:tokens].astype(np.int64)
    nc = np.zeros((slots, heads, dn), np.float64)
    rc = np.zeros((slots, heads, dr), np.float64)
    oracle.kv_rmsnorm_rope_cache(kv, g, cos_t, sin_t, pos, sl, nc, rc, EPS5, style)
    want = oracle.rmsnorm_fwd(np.ascontiguousarray(kv[:, :, :dn].reshape(-1, dn)), g, EPS5, unrounded=True)
    assert np.array_equal(nc[sl].reshape(-1, dn), want)
    half = dr // 2
    xr = _vals(kv[:, :, dn:])
    ia = np.arange(half) * 2 if style == oracle.ROPE_PAIRS else np.arange(half)
    ib = ia + 1 if style == oracle.ROPE_PAIRS else ia + half
    c = cos_t[pos].astype(np.float64)[:, None, :]
    s = sin_t[pos].astype(np.float64)[:, None, :]
    re = xr[:, :, ia] * c - xr[:, :, ib] * s
    im = xr[:, :, ia] * s + xr[:, :, ib] * c
    got = rc[sl]
    tol = 2.0 ** -52 * (np.abs(xr[:, :, ia] * c) + np.abs(xr[:, :, ib] * s))
    assert np.all(np.abs(got[:, :, ia] - re) <= tol)
    tol = 2.0 ** -52 * (np.abs(xr[:, :, ia] * s) + np.abs(xr[:, :, ib] * c))
    assert np.all(np.abs(got[:, :, ib] - im) <= tol)

"""The GPU comparison itself, on the CPU: a simulated fp32 evaluation rounded
once to nearest-even passes, while the same values truncated, rounded twice,
or rounded before the weight multiply fail.  Also the fp32 form: an error
inside the stated 1e-5 but outside the evaluation bound fails.

The "GPU" results here are numpy float32 evaluations of the forward (a pairwise
fp32 sum of squares, a correctly rounded divide and square root, two fp32
products) -- a stand-in for the kernels' arithmetic, not a copy of it.
"""
import numpy as np
import pytest

import memory_bound_rmsnorm_amd as mbr
from memory_bound_rmsnorm_amd import inputs
from tests import parity

CFG = mbr.Config(mbr.PATH_VECTOR, 8, 2, 1, 0)  # chain 2 * 8 + 6 + 8 = 30 (bf16)


def _f32_eval(xb: np.ndarray, wb: np.ndarray, eps: float, round_before_weight=False):
    x = parity._values(xb).astype(np.float32)
    w = parity._values(wb).astype(np.float32)
    s = np.add.reduce(x * x, axis=1, dtype=np.float32)
    r = (np.float32(1) / np.sqrt(s / np.float32(x.shape[1]) + np.float32(eps))).astype(np.float32)
    xr = x * r[:, None]
    if round_before_weight:
        xr = _bf16_vals(_rne_bf16(xr)).astype(np.float32)
    return xr * w[None, :]


def _rne_bf16(f: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 nearest-even by the usual bias-and-truncate construction
    (add 0x7FFF plus the lowest kept bit, keep the top 16 bits); finite data."""
    u = np.ascontiguousarray(f, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _trunc_bf16(f: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(f, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _bf16_vals(b: np.ndarray) -> np.ndarray:
    return parity.bf16_to_f64(b)


@pytest.fixture(scope="module")
def case():
    w = inputs.custom(64, 8192, "bf16", False)
    t = inputs.make(w, seed=3)
    xb, wb = inputs.bits(t["x"]), inputs.bits(t["weight"])
    want, e = parity.oracle_fwd(xb, wb, w.eps, unrounded=True)
    return xb, wb, w.eps, want, e


def test_correct_rounding_passes(case):
    xb, wb, eps, want, e = case
    got = _rne_bf16(_f32_eval(xb, wb, eps))
    st = parity.compare(got, want, e, parity.fwd_gamma(CFG, 8192, True))
    assert st["max_ulp"] <= 1 and st["rounding"]["differ_from_nearest_even"] < 0.001 * got.size


@pytest.mark.parametrize("slip", ["truncated", "rounded before the weight multiply", "double rounding via fp16"])
def test_rounding_slips_fail(case, slip):
    xb, wb, eps, want, e = case
    if slip == "truncated":
        got = _trunc_bf16(_f32_eval(xb, wb, eps))
    elif slip == "rounded before the weight multiply":
        got = _rne_bf16(_f32_eval(xb, wb, eps, round_before_weight=True))
    else:
        # rounded to an 11-bit significand (fp16) first, then to bf16's 8
        got = _rne_bf16(_f32_eval(xb, wb, eps).astype(np.float16).astype(np.float32))
    # the stated 1-ulp tolerance alone lets every one of these through ...
    assert parity.compare_bf16(got, want)["max_ulp"] <= 1
    # ... the correct-rounding check does not
    with pytest.raises(AssertionError, match="not a nearest-even rounding"):
        parity.compare(got, want, e, parity.fwd_gamma(CFG, 8192, True))


def test_f32_error_inside_the_stated_tolerance_but_outside_the_bound_fails():
    w = inputs.custom(16, 4096, "f32", False)
    t = inputs.make(w, seed=4)
    x, wt = inputs.bits(t["x"]), inputs.bits(t["weight"])
    want, e = parity.oracle_fwd(x, wt, w.eps, unrounded=True)
    gamma = parity.fwd_gamma(mbr.Config(mbr.PATH_VECTOR, 4, 2, 1, 0), 4096, False)
    good = _f32_eval(x, wt, w.eps)
    parity.compare(good, want, e, gamma)
    sloppy = (good.astype(np.float64) * (1 + 5e-6)).astype(np.float32)  # e.g. a 5e-6 rsqrt
    assert parity.compare_f32(sloppy, want)["max_rel_err"] < 1e-5
    with pytest.raises(AssertionError, match="not a nearest-even rounding"):
        parity.compare(sloppy, want, e, gamma)


def test_magnitude_bound_rejects_truncation():
    """The cancellation-aware bound (backward, LayerNorm, RoPE) still demands a
    correct rounding: a truncated bf16 dx fails, the nearest-even one passes."""
    rng = np.random.default_rng(5)
    e = rng.standard_normal((32, 512))
    mag = np.abs(e) + 0.01
    stats = {}
    good = _rne_bf16(e.astype(np.float32))
    parity.check_magnitude(good, e, mag, 64 * parity.U, "dx", stats, 512)
    with pytest.raises(AssertionError):
        parity.check_magnitude(_trunc_bf16(e.astype(np.float32)), e, mag, 64 * parity.U, "dx", stats, 512)


def test_non_finite_values_must_match():
    e = np.array([[1.0, np.inf, np.nan, -np.inf]])
    got = _rne_bf16(np.array([[1.0, np.inf, np.nan, -np.inf]], np.float32))
    parity.check_rounded(got, e, 0.0, 4)
    bad = got.copy()
    bad[0, 1] = 0x7F7F  # largest finite in place of +inf
    with pytest.raises(AssertionError, match="infinities"):
        parity.check_rounded(bad, e, 0.0, 4)
    bad = got.copy()
    bad[0, 2] = 0x3F80  # a number in place of NaN
    with pytest.raises(AssertionError, match="NaN"):
        parity.check_rounded(bad, e, 0.0, 4)

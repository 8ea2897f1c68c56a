"""Comparison of HIP results with the CPU oracle (tests and smoke check only).

Tolerances:
  * bf16 outputs: at most 1 unit in the last place from the oracle's
    correctly rounded value, on the monotone integer line of bf16 patterns
    (+0 and -0 equal).  The fp32 evaluation on the GPU can land on the other
    side of a rounding midpoint when the exact value is that close to one; it
    can never move a result by two places.
  * fp32 outputs: |gpu - oracle| <= 1e-5 * |oracle|, and oracle == 0 implies
    gpu == 0.  Derivation: y = x * r * w, so the relative error of every
    element of a row is the relative error of r (half the relative error of
    the fp32 sum of squares, at most about (n_lane + 10) * 2^-24 / 2 for the
    longest per-lane chain n_lane <= 256, plus the rsqrt's) plus two fp32
    products -- below 1e-5 for every built configuration.
  * the fused residual sum h: bitwise equal (one rounding of an exact sum on
    both sides).
NaN positions must agree and are otherwise excluded.
"""
import concurrent.futures
import os

import numpy as np

import oracle

BF16_MAX_ULP = 1
F32_RTOL = 1e-5


def _bf16_key(bits: np.ndarray) -> np.ndarray:
    u = bits.astype(np.int32)
    return np.where(u & 0x8000, -(u & 0x7FFF), u)


def _bf16_is_nan(bits: np.ndarray) -> np.ndarray:
    return ((bits & 0x7F80) == 0x7F80) & ((bits & 0x007F) != 0)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def compare_bf16(got: np.ndarray, want: np.ndarray, max_ulp: int = BF16_MAX_ULP) -> dict:
    assert got.shape == want.shape and got.dtype == np.uint16 and want.dtype == np.uint16
    gn, wn = _bf16_is_nan(got), _bf16_is_nan(want)
    assert np.array_equal(gn, wn), "NaN positions differ"
    ok = ~wn
    d = np.abs(_bf16_key(got[ok]) - _bf16_key(want[ok]))
    err = np.abs(bf16_to_f64(got[ok]) - bf16_to_f64(want[ok]))
    stats = {"n": int(ok.sum()), "max_ulp": int(d.max()) if d.size else 0,
             "frac_bitwise_equal": float(np.mean(d == 0)) if d.size else 1.0,
             "n_one_ulp": int(np.sum(d == 1)), "max_abs_err": float(err.max()) if err.size else 0.0}
    if stats["max_ulp"] > max_ulp:
        idx = np.argmax(d)
        flat = np.flatnonzero(ok)[idx]
        raise AssertionError("bf16 mismatch of %d ulp at flat index %d: got 0x%04x want 0x%04x; %s"
                             % (stats["max_ulp"], flat, got.reshape(-1)[flat], want.reshape(-1)[flat], stats))
    return stats


def compare_f32(got: np.ndarray, want: np.ndarray, rtol: float = F32_RTOL) -> dict:
    assert got.shape == want.shape and got.dtype == np.float32 and want.dtype == np.float32
    gn, wn = np.isnan(got), np.isnan(want)
    assert np.array_equal(gn, wn), "NaN positions differ"
    ok = ~wn
    g = got[ok].astype(np.float64)
    w = want[ok].astype(np.float64)
    zero = w == 0
    assert np.all(g[zero] == 0), "oracle zero, GPU non-zero"
    rel = np.abs(g[~zero] - w[~zero]) / np.abs(w[~zero])
    stats = {"n": int(ok.sum()), "max_rel_err": float(rel.max()) if rel.size else 0.0,
             "max_abs_err": float(np.abs(g - w).max()) if g.size else 0.0,
             "frac_bitwise_equal": float(np.mean(got[ok] == want[ok])) if g.size else 1.0}
    if stats["max_rel_err"] > rtol:
        raise AssertionError("fp32 relative error %.3e > %.1e; %s" % (stats["max_rel_err"], rtol, stats))
    return stats


def compare(got: np.ndarray, want: np.ndarray) -> dict:
    return compare_bf16(got, want) if want.dtype == np.uint16 else compare_f32(got, want)


def _chunks(rows: int, n: int):
    step = max(1, (rows + n - 1) // n)
    return [(i, min(rows, i + step)) for i in range(0, rows, step)]


def threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def oracle_fwd(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """The oracle over all rows, rows split across host threads (the C code
    releases the GIL; each row is computed exactly as in a serial call)."""
    out = np.empty_like(x)
    with concurrent.futures.ThreadPoolExecutor(threads()) as ex:
        def job(r):
            out[r[0]:r[1]] = oracle.rmsnorm_fwd(x[r[0]:r[1]], w, eps)
        list(ex.map(job, _chunks(x.shape[0], 4 * threads())))
    return out


def oracle_residual(x: np.ndarray, res: np.ndarray, w: np.ndarray, eps: float):
    h = np.empty_like(x)
    y = np.empty_like(x)
    with concurrent.futures.ThreadPoolExecutor(threads()) as ex:
        def job(r):
            h[r[0]:r[1]], y[r[0]:r[1]] = oracle.rmsnorm_residual_fwd(x[r[0]:r[1]], res[r[0]:r[1]], w, eps)
        list(ex.map(job, _chunks(x.shape[0], 4 * threads())))
    return h, y

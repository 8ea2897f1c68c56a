"""Comparison of HIP results with the CPU oracle (tests and smoke check only).

Two layers of checks, both applied to every normalised output:

1. The stated tolerances.
   * bf16 outputs: at most 1 unit in the last place from the oracle's
     correctly rounded value, on the monotone integer line of bf16 patterns
     (+0 and -0 equal).
   * fp32 outputs: |gpu - oracle| <= 1e-5 * |oracle|, and oracle == 0 implies
     gpu == 0.
   * the fused residual sum h: bitwise equal (one rounding of an exact sum on
     both sides).

2. Correct rounding (check_rounded).  The kernels evaluate in fp32 and round
   once, to nearest-even, at write-back (gollamago README, "RMSNorm 优化
   （TileLang）").  With e the oracle's unrounded fp64 value of an element and
   t a bound on the GPU's fp32 evaluation error before that last rounding,
   the GPU result must be the nearest-even rounding of some value in
   [e - t, e + t]; since rounding is monotone, that is the set of patterns
   between RN(e - t) and RN(e + t).  For the forward t is about 1e-6 of |e|,
   far below half a bf16 ulp (2^-9 relative), so a result may differ from
   RN(e) only when e lies within t of a rounding midpoint -- a truncating
   conversion, a double rounding or a rounding before the weight multiply
   fails this on about half the elements.

   Bound for the RMSNorm forward (u = 2^-24, L = chain(cfg), the longest fp32
   summation chain of a row: terms per lane + 6 wave levels + one add per wave
   slot):
     * the sum of squares has only positive terms: relative error <= (L + 1)u;
     * / hidden and + eps (both rounded): 2u more, all terms positive;
     * v_rsq_f32 is accurate to 1 ulp (2u): r's relative error is at most
       (L + 3)u/2 + 2u;
     * (x * r) * w: two fp32 products, 2u;
   so |y_fp32 - e| <= (L/2 + 6)u |e| to first order.  check_rounded uses
   fwd_gamma = (L + 12)u, twice that, plus the oracle's own fp64 error
   (hidden + 8) 2^-53 |e|.  For fp32 outputs the last product's rounding is
   the output rounding itself, which the interval check already allows.
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


U = 2.0 ** -24
_CHUNK = 1 << 22


def _keys(a: np.ndarray) -> np.ndarray:
    """Monotone integer keys of bf16 patterns (uint16) or float32 values."""
    if a.dtype == np.uint16:
        return _bf16_key(a).astype(np.int64)
    u = a.view(np.uint32).astype(np.int64)
    return np.where(u & 0x80000000, -(u & 0x7FFFFFFF), u)


def _round_keys(v: np.ndarray, bf16: bool) -> np.ndarray:
    r = oracle.round_bf16_array(v) if bf16 else oracle.round_f32_array(v)
    return _keys(r)


def _half_ulp(v: np.ndarray, bf16: bool) -> np.ndarray:
    """Half the spacing of the output format at |v| (the spacing above v at a
    power of two), subnormals included."""
    mant, lo = (7, -133) if bf16 else (23, -149)
    a = np.abs(v)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return 0.5 * np.maximum(2.0 ** (e - mant), 2.0 ** lo)


def check_rounded(got: np.ndarray, exact: np.ndarray, tol, hidden: int, what: str = "y",
                  stats: dict = None) -> dict:
    """Every element of got (bf16 patterns or float32) must be the nearest-even
    rounding of some value within tol (absolute, scalar or per element) plus the
    oracle's own fp64 error of exact (the oracle's unrounded value).

    Besides the counts, the result reports max_bound_used: over all elements,
    how much of the bound the element needed, (|got - exact| - half an ulp of
    got) / bound, floored at 0 -- an element that is exactly the nearest-even
    rounding of exact needs none of it."""
    bf16 = got.dtype == np.uint16
    g = np.ascontiguousarray(got).reshape(-1)
    e = np.ascontiguousarray(exact, dtype=np.float64).reshape(-1)
    assert g.size == e.size, "%s: shape mismatch" % what
    t_all = np.broadcast_to(np.asarray(tol, dtype=np.float64), np.shape(exact)).reshape(-1)
    ora = (hidden + 8) * 2.0 ** -53
    n_bad = n_diff = 0
    first = None
    worst = 0.0
    used = 0.0
    for a in range(0, g.size, _CHUNK):
        gc, ec, tc = g[a:a + _CHUNK], e[a:a + _CHUNK], t_all[a:a + _CHUNK]
        gnan = _bf16_is_nan(gc) if bf16 else np.isnan(gc)
        enan = np.isnan(ec)
        assert np.array_equal(gnan, enan), "%s: NaN positions differ" % what
        einf = np.isinf(ec)
        assert np.array_equal(_keys(gc[einf]), _round_keys(ec[einf], bf16)), "%s: infinities differ" % what
        ok = ~enan & ~einf
        gc, ec, tc = gc[ok], ec[ok], tc[ok]
        t = tc + ora * np.abs(ec)
        with np.errstate(invalid="ignore", over="ignore"):
            lo = _round_keys(ec - t, bf16)
            hi = _round_keys(ec + t, bf16)
        kg = _keys(gc)
        kw = _round_keys(ec, bf16)
        bad = (kg < lo) | (kg > hi)
        n_diff += int(np.sum(kg != kw))
        if bad.any():
            n_bad += int(bad.sum())
            if first is None:
                i = int(np.flatnonzero(bad)[0])
                first = (a + int(np.flatnonzero(ok)[i]), gc[i], ec[i], t[i], int(kw[i]))
        with np.errstate(invalid="ignore", divide="ignore"):
            d = np.abs(kg - kw)
            worst = max(worst, float(d.max()) if d.size else 0.0)
            gv = _values(gc)
            need = np.maximum(np.abs(gv - ec) - _half_ulp(gv, bf16), 0.0)
            u = np.where(need > 0, need / np.where(t > 0, t, np.inf), 0.0)
            used = max(used, float(u.max()) if u.size else 0.0)
    res = {"n": int(g.size), "differ_from_nearest_even": n_diff, "max_ulp_from_nearest_even": int(worst),
           "max_bound_used": round(used, 4)}
    if stats is not None:
        stats[what + "_rounding"] = res
    if n_bad:
        i, gv, ev, tv, kw = first
        raise AssertionError("%s: %d elements are not a nearest-even rounding of a value within the fp32 "
                             "evaluation bound of the exact result; first at flat index %d: got %r, exact %r, "
                             "bound %.3e" % (what, n_bad, i, hex(int(gv)) if bf16 else float(gv), float(ev), tv))
    return res


def chain(cfg, hidden: int, bf16: bool) -> int:
    """Longest fp32 chain of a row sum for a launch configuration: the terms one
    lane adds, 6 wave levels, and one add per wave slot."""
    v = 8 if bf16 else 4
    wpr = cfg.waves_per_row
    if cfg.path == 1:      # vector (also rows narrower than a wave)
        per_lane = cfg.items_per_lane * v
    elif cfg.path == 2:    # element
        per_lane = cfg.items_per_lane
    elif cfg.path == 4:    # any alignment: the lane's vectors plus one tail element
        per_lane = cfg.items_per_lane * v + 1
    elif cfg.path == 5:    # register + LDS: the lane's register vectors plus its staged ones
        staged = hidden // v - 1024 * cfg.items_per_lane
        per_lane = (cfg.items_per_lane + -(-staged // 1024)) * v
    else:                  # two-pass: every lane strides over the row
        vec = hidden % v == 0
        units = hidden // v if vec else hidden
        per_lane = -(-units // (64 * wpr)) * (v if vec else 1)
    return per_lane + 6 + wpr


def fwd_gamma(cfg, hidden: int, bf16: bool) -> float:
    """Relative fp32 evaluation bound of the RMSNorm forward (see the module
    docstring): twice the first-order bound (L/2 + 6)u."""
    return (chain(cfg, hidden, bf16) + 12) * U


def compare(got: np.ndarray, want: np.ndarray, exact: np.ndarray, gamma: float) -> dict:
    """The stated tolerance, then correct rounding of a value within
    gamma * |exact| of the oracle's unrounded result."""
    stats = compare_bf16(got, want) if want.dtype == np.uint16 else compare_f32(got, want)
    hidden = want.shape[-1] if want.ndim else 1
    r = check_rounded(got, exact, gamma * np.abs(exact), hidden)
    stats["rounding"] = r
    return stats


def _chunks(rows: int, n: int):
    step = max(1, (rows + n - 1) // n)
    return [(i, min(rows, i + step)) for i in range(0, rows, step)]


def threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _round_like(e: np.ndarray, like: np.ndarray) -> np.ndarray:
    """The oracle's nearest-even rounding of unrounded values, rows across threads."""
    out = np.empty(e.shape, like.dtype)
    rnd = oracle.round_bf16_array if like.dtype == np.uint16 else oracle.round_f32_array
    with concurrent.futures.ThreadPoolExecutor(threads()) as ex:
        def job(r):
            out[r[0]:r[1]] = rnd(e[r[0]:r[1]])
        list(ex.map(job, _chunks(e.shape[0], 4 * threads())))
    return out


def oracle_fwd(x: np.ndarray, w: np.ndarray, eps: float, unrounded: bool = False):
    """The oracle over all rows, rows split across host threads (the C code
    releases the GIL; each row is computed exactly as in a serial call).
    Returns the rounded output, or (rounded, unrounded) with ``unrounded``;
    the rounded one is the oracle's rounding of the unrounded one."""
    e = np.empty(x.shape, np.float64)
    with concurrent.futures.ThreadPoolExecutor(threads()) as ex:
        def job(r):
            e[r[0]:r[1]] = oracle.rmsnorm_fwd(x[r[0]:r[1]], w, eps, unrounded=True)
        list(ex.map(job, _chunks(x.shape[0], 4 * threads())))
    want = _round_like(e, x)
    return (want, e) if unrounded else want


def oracle_residual(x: np.ndarray, res: np.ndarray, w: np.ndarray, eps: float, unrounded: bool = False):
    """(h, y), or (h, y, y_unrounded) with ``unrounded``."""
    h = np.empty_like(x)
    e = np.empty(x.shape, np.float64)
    with concurrent.futures.ThreadPoolExecutor(threads()) as ex:
        def job(r):
            h[r[0]:r[1]], e[r[0]:r[1]] = oracle.rmsnorm_residual_fwd(x[r[0]:r[1]], res[r[0]:r[1]], w, eps,
                                                                     unrounded=True)
        list(ex.map(job, _chunks(x.shape[0], 4 * threads())))
    y = _round_like(e, x)
    return (h, y, e) if unrounded else (h, y)


QMAX = {0: 127.0, 1: 448.0}


def _e4m3_table() -> np.ndarray:
    """Value of every e4m3fn code (NaN codes 0x7F/0xFF as NaN)."""
    v = np.empty(256)
    for c in range(256):
        e, m = (c >> 3) & 0xF, c & 7
        mag = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
        v[c] = np.nan if (c & 0x7F) == 0x7F else (-mag if c & 0x80 else mag)
    return v


E4M3 = _e4m3_table()


def quant_t(v_bits: np.ndarray, w_bits: np.ndarray, qtype: int) -> np.ndarray:
    """Q * v_j * w_j / max_k |v_k * w_k| per row in fp64 (products of two bf16 or
    fp32 values are exact in fp64): the quantity the codes round, with the
    root cancelled."""
    if v_bits.dtype == np.uint16:
        v = bf16_to_f64(v_bits)
        w = bf16_to_f64(w_bits)
    else:
        v = v_bits.astype(np.float64)
        w = w_bits.astype(np.float64)
    p = v * w[None, :]
    m = np.max(np.abs(p), axis=1, keepdims=True)
    with np.errstate(invalid="ignore", divide="ignore"):
        t = np.where(m > 0, QMAX[qtype] * p / m, 0.0)
    return t


def compare_quant(q_gpu, q_want, s_gpu, s_want, t, qtype, tie_tol=1e-5) -> dict:
    """Codes equal except where t lies within tie_tol (relative, int8: of 1)
    of the tie between the two codes involved; scales within 1e-5 relative."""
    s_g = s_gpu.astype(np.float64)
    s_w = s_want.astype(np.float64)
    assert np.all(s_g[s_w == 0] == 0), "zero scale expected"
    nz = s_w != 0
    srel = np.abs(s_g[nz] - s_w[nz]) / s_w[nz] if nz.any() else np.zeros(1)
    assert srel.max() <= F32_RTOL, "scale relative error %.3e" % srel.max()
    g = q_gpu.reshape(q_want.shape)
    diff = g != q_want
    n_diff = int(diff.sum())
    if n_diff:
        gi = g[diff]
        wi = q_want[diff]
        ti = t[diff]
        if qtype == 0:
            gi = gi.astype(np.int64)
            wi = wi.astype(np.int64)
            assert np.all(np.abs(gi - wi) == 1), "int8 codes differ by more than one"
            mid = (gi + wi) / 2.0
            assert np.all(np.abs(ti - mid) <= tie_tol * 127), "int8 code differs away from a tie"
        else:
            gu = gi.astype(np.uint8)
            wu = wi.astype(np.uint8)
            gv, wv = E4M3[gu], E4M3[wu]
            assert np.all(np.sign(gv) * np.sign(wv) >= 0), "fp8 codes differ in sign"
            key = lambda c: np.where(c & 0x80, -(c & 0x7F).astype(np.int64), (c & 0x7F).astype(np.int64))
            assert np.all(np.abs(key(gu) - key(wu)) == 1), "fp8 codes differ by more than one step"
            mid = (gv + wv) / 2.0
            assert np.all(np.abs(ti - mid) <= tie_tol * np.abs(ti) + 2.0 ** -12), "fp8 code differs away from a tie"
    return {"n": int(q_want.size), "codes_differing_at_ties": n_diff,
            "max_scale_rel_err": float(srel.max())}


def oracle_quant(x, w, eps, qtype, residual=None):
    """The oracle's dynamic-quant output over all rows, rows across threads."""
    rows = x.shape[0]
    h = np.empty_like(x) if residual is not None else None
    q = np.empty(x.shape, np.int8 if qtype == 0 else np.uint8)
    s = np.empty(rows, np.float32)
    with concurrent.futures.ThreadPoolExecutor(threads()) as ex:
        def job(r):
            a, b = r
            res = residual[a:b] if residual is not None else None
            hh, qq, ss = oracle.rmsnorm_dynamic_quant_fwd(x[a:b], w, eps, qtype, residual=res)
            if h is not None:
                h[a:b] = hh
            q[a:b] = qq
            s[a:b] = ss
        list(ex.map(job, _chunks(rows, 4 * threads())))
    return h, q, s


# ---------------------------------------------------------------- backward
#
# Tolerance derivation.  Let u = 2^-24 and L the longest fp32 chain of a row
# sum on the GPU (terms per lane + 6 wave levels + one add per wave slot).
#   * r = rsqrt(s/H + eps): s has all-positive terms, so its relative error is
#     <= L*u; r's is about half of that plus the rsqrt's and the divide's, below
#     (L/2 + 4)*u.
#   * c = sum(dy*w*x) has error <= (L + 2)*u * C_abs, C_abs = sum|dy*w*x|.
#   * dx_k = r*(dy_k*w_k - x_k*r^2*c/H) therefore has absolute error below
#     gamma * M_k with M_k = r*|dy_k*w_k| + |x_k|*r^3*C_abs/H and
#     gamma = (2L + 16)*u, before its one rounding to the dtype.  The two
#     terms can cancel, so the bound is on M_k, not on |dx_k|.
#   * dw_j = sum_i dy_ij*x_ij*r_i is summed per lane over ceil(ceil(rows/R)/G)
#     rows (R row slots per workgroup, G partial rows), the R slot sums are
#     added in slot order, then ceil(G/64) partial rows per slice and a 7-level
#     tree: absolute error below gamma_w * A_j, A_j = sum_i |dy_ij*x_ij|*r_i,
#     gamma_w = 2*(ceil(ceil(rows/R)/G) + R + ceil(G/64) + L/2 + 12)*u (factor
#     2 for the per-term errors and margin), before its one rounding.
# M and A are magnitudes computed here in fp64 for the bound only; the values
# compared against are the oracle's unrounded ones, and every GPU result must
# be a nearest-even rounding of a value within the bound (check_rounded).


def _values(a: np.ndarray) -> np.ndarray:
    return bf16_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


bwd_chain = chain


def _bwd_magnitudes(x, w, dy, eps, rows_chunk=2048):
    """(M, A): per-element dx magnitudes and per-column dw magnitudes, fp64."""
    rows, hidden = x.shape
    M = np.empty((rows, hidden))
    A = np.zeros(hidden)
    wd = _values(w)
    for a in range(0, rows, rows_chunk):
        xd = _values(x[a:a + rows_chunk])
        gd = _values(dy[a:a + rows_chunk])
        r = 1.0 / np.sqrt((xd * xd).mean(axis=1) + float(np.float32(eps)))
        gw = np.abs(gd * wd[None, :])
        cabs = (gw * np.abs(xd)).sum(axis=1)
        M[a:a + rows_chunk] = r[:, None] * gw + np.abs(xd) * (r ** 3 * cabs / hidden)[:, None]
        A += (np.abs(gd * xd) * r[:, None]).sum(axis=0)
    return M, A


def check_magnitude(got, exact, mag, gamma, what: str, stats: dict, sum_len: int):
    """got must be a nearest-even rounding of a value within gamma * mag of the
    oracle's unrounded values exact (sum_len: the oracle's longest fp64 sum)."""
    with np.errstate(invalid="ignore"):
        tol = gamma * np.where(np.isfinite(mag), mag, 0.0)
    return check_rounded(got, exact, tol, sum_len, what, stats)


def compare_bwd(dx_gpu, dw_gpu, dx_exact, dw_exact, x, w, dy, eps, cfg, n_part) -> dict:
    """dx (and dw unless dw_exact is None) against the oracle's unrounded
    values with the bounds above."""
    bf16 = x.dtype == np.uint16
    rows, hidden = x.shape
    L = bwd_chain(cfg, hidden, bf16)
    M, A = _bwd_magnitudes(x, w, dy, eps)
    stats = {"chain": L}
    check_magnitude(dx_gpu, dx_exact, M, (2 * L + 16) * U, "dx", stats, hidden)
    if dw_exact is not None:
        g = max(1, n_part)
        R = max(1, getattr(cfg, "rows_per_block", 1))
        gamma_w = 2 * (-(-(-(-rows // R)) // g) + R + -(-g // 64) + L / 2 + 12) * U
        check_magnitude(dw_gpu, dw_exact, A, gamma_w, "dw", stats, rows + hidden)
    return stats


def oracle_bwd(x: np.ndarray, w: np.ndarray, dy: np.ndarray, eps: float, want_dw: bool = True):
    """The oracle's unrounded dx over all rows (rows across host threads) and
    unrounded dw (one serial fp64 pass over all rows, as the oracle defines
    it), both float64."""
    dx = np.empty(x.shape, np.float64)
    with concurrent.futures.ThreadPoolExecutor(threads()) as ex:
        def job(r):
            dx[r[0]:r[1]] = oracle.rmsnorm_bwd(x[r[0]:r[1]], w, dy[r[0]:r[1]], eps, want_dw=False,
                                               unrounded=True)[0]
        fut = ex.submit(lambda: oracle.rmsnorm_bwd(x, w, dy, eps, want_dx=False, unrounded=True)[1]) \
            if want_dw else None
        list(ex.map(job, _chunks(x.shape[0], 4 * threads())))
        dw = fut.result() if fut is not None else None
    return dx, dw


# ---------------------------------------------------------------- LayerNorm
#
# y = gamma*(x - mu)*inv + beta on the GPU in fp32 with the same reduction as
# the RMSNorm kernels (chain length L as in bwd_chain), moments by the
# corrected two-pass scheme: m0 = fp32 mean, then c = sum(x - m0)/H and
# q = sum(x - m0)^2/H from the same values, output from (x - m0) - c.  The
# correction leaves a mean error below about L*u*sum|x - mu|/H (m0's own error
# cancels to first order), the differences add u*|x - mu|, inv's relative
# error is below (L/2 + 4)*u, and the affine step adds two roundings; so
# |y_gpu - y| <= (2L + 16)*u * M with M = |gamma|*inv*(|x - mu| + sum|x - mu|/H)
# + |beta| before the one rounding to the dtype, which check_rounded allows.
# gamma*(x - mu)*inv and beta can cancel, hence the bound on M; it does not
# grow with |mu|.


def _ln_magnitudes(x, g, b, eps, rows_chunk=2048):
    rows, hidden = x.shape
    M = np.empty((rows, hidden))
    gd = np.abs(_values(g))
    bd = np.abs(_values(b)) if b is not None else np.zeros(hidden)
    for a in range(0, rows, rows_chunk):
        xd = _values(x[a:a + rows_chunk])
        mu = xd.mean(axis=1, keepdims=True)
        var = ((xd - mu) ** 2).mean(axis=1, keepdims=True)
        inv = 1.0 / np.sqrt(var + float(np.float32(eps)))
        sabs = np.abs(xd - mu).mean(axis=1, keepdims=True)
        M[a:a + rows_chunk] = gd[None, :] * inv * (np.abs(xd - mu) + sabs) + bd[None, :]
    return M


def compare_ln(y_gpu, y_exact, x, g, b, eps, cfg) -> dict:
    """y against the oracle's unrounded LayerNorm with the bound above."""
    bf16 = x.dtype == np.uint16
    L = bwd_chain(cfg, x.shape[1], bf16)
    stats = {"chain": L}
    check_magnitude(y_gpu, y_exact, _ln_magnitudes(x, g, b, eps), (2 * L + 16) * U, "y", stats, 2 * x.shape[1])
    return stats


def oracle_ln(x, g, b, eps):
    """The oracle's unrounded LayerNorm (float64), rows across host threads."""
    out = np.empty(x.shape, np.float64)
    with concurrent.futures.ThreadPoolExecutor(threads()) as ex:
        def job(r):
            out[r[0]:r[1]] = oracle.layernorm_fwd(x[r[0]:r[1]], g, b, eps, unrounded=True)
        list(ex.map(job, _chunks(x.shape[0], 4 * threads())))
    return out

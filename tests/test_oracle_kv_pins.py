"""Pins for the oracle's KV RMSNorm + RoPE + cache scatter (the CANN
aclnnKvRmsNormRopeCache fusion the TileLang tutorial ch. 02, sections 1.2 and
4.2, describes; RoPE as xserv's rope.cu, phase 4).

  * the normalised part equals the (separately pinned) RMSNorm oracle applied to
    the left part of each row, bit for bit;
  * the rotated part equals a complex multiplication (a + ib)(cos + i sin) done
    by numpy in complex128 (a library routine), rounded once, except within
    1e-9 of a tie;
  * position 0 leaves the rotated part unchanged, bit for bit (xserv's
    "RoPE position=0" identity test);
  * a table whose only non-trivial entry is a quarter turn on one pair moves
    exactly that pair, (a, b) -> (-b, a): pins the pairing (adjacent pairs or
    halves) and the sign;
  * rotations preserve each pair's length;
  * every token lands at its slot, every other cache row is untouched, and
    tokens with a negative or out-of-range slot or position write nothing.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from memory_bound_rmsnorm_amd import inputs
from tests import exact
from tests.test_oracle_pins import EPS5, bits_bf16


def _vals(a):
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _store(a, dtype):
    a = np.asarray(a, dtype=np.float32)
    return a if dtype == "f32" else bits_bf16(a.reshape(-1)).reshape(a.shape)


def _case(dtype, tokens=6, heads=2, dn=24, dr=8, max_pos=16, slots=40, seed=0):
    rng = np.random.default_rng(seed)
    kv = _store(rng.standard_normal((tokens, heads, dn + dr)), dtype)
    g = _store(rng.standard_normal(dn) * 0.2 + 1, dtype)
    cos_t, sin_t = inputs.rope_tables(max_pos, dr)
    pos = rng.integers(0, max_pos, tokens).astype(np.int32)
    sl = rng.permutation(slots)[:tokens].astype(np.int64)
    nc = _store(rng.standard_normal((slots, heads, dn)), dtype)
    rc = _store(rng.standard_normal((slots, heads, dr)), dtype)
    return kv, g, cos_t, sin_t, pos, sl, nc, rc


def _run(kv, g, cos_t, sin_t, pos, sl, nc, rc, style, eps=EPS5):
    nc, rc = nc.copy(), rc.copy()
    oracle.kv_rmsnorm_rope_cache(kv, g, cos_t, sin_t, pos, sl, nc, rc, eps, style)
    return nc, rc


def _round(v, dtype):
    return exact.round_bf16_exact(Fraction(v)) if dtype == "bf16" else exact.f32_bits(float(np.float32(v)))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("style", [oracle.ROPE_HALVES, oracle.ROPE_PAIRS])
def test_norm_part_is_the_rmsnorm_oracle(dtype, style):
    kv, g, c, s, pos, sl, nc, rc = _case(dtype)
    nc2, _ = _run(kv, g, c, s, pos, sl, nc, rc, style)
    dn = g.shape[0]
    want = oracle.rmsnorm_fwd(np.ascontiguousarray(kv[:, :, :dn].reshape(-1, dn)), g, EPS5)
    assert np.array_equal(nc2[sl].reshape(-1, dn), want)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("style", [oracle.ROPE_HALVES, oracle.ROPE_PAIRS])
def test_rope_part_is_a_complex_multiplication(dtype, style):
    kv, g, c, s, pos, sl, nc, rc = _case(dtype, tokens=10, dr=16, max_pos=64, seed=3)
    _, rc2 = _run(kv, g, c, s, pos, sl, nc, rc, style)
    dn, dr = g.shape[0], rc.shape[2]
    half = dr // 2
    x = _vals(kv[:, :, dn:])
    ia = np.arange(half) * 2 if style == oracle.ROPE_PAIRS else np.arange(half)
    ib = ia + 1 if style == oracle.ROPE_PAIRS else ia + half
    z = (x[:, :, ia] + 1j * x[:, :, ib]) * (c[pos].astype(np.float64) + 1j * s[pos].astype(np.float64))[:, None, :]
    got = rc2[sl]
    for want_vals, idx in ((z.real, ia), (z.imag, ib)):
        for (t, h, j), v in np.ndenumerate(want_vals):
            gb = int(got[t, h, idx[j]]) if dtype == "bf16" else exact.f32_bits(float(got[t, h, idx[j]]))
            wb = exact.round_bf16_exact(Fraction(v)) if dtype == "bf16" else exact.round_f32_exact(Fraction(v))
            if gb != wb:
                val = exact.bf16_value if dtype == "bf16" else exact.f32_value
                mid = (val(gb) + val(wb)) / 2
                assert abs(Fraction(v) - mid) <= Fraction(1, 10 ** 9) * abs(Fraction(v)), (t, h, j)


@pytest.mark.parametrize("style", [oracle.ROPE_HALVES, oracle.ROPE_PAIRS])
def test_position_zero_is_the_identity(style):
    kv, g, c, s, pos, sl, nc, rc = _case("bf16", seed=4)
    pos[:] = 0
    _, rc2 = _run(kv, g, c, s, pos, sl, nc, rc, style)
    assert np.array_equal(rc2[sl], kv[:, :, g.shape[0]:])


@pytest.mark.parametrize("style", [oracle.ROPE_HALVES, oracle.ROPE_PAIRS])
def test_quarter_turn_moves_exactly_one_pair(style):
    kv, g, c, s, pos, sl, nc, rc = _case("f32", dr=8, seed=5)
    c = np.ones_like(c)
    s = np.zeros_like(s)
    c[:, 1] = 0.0
    s[:, 1] = 1.0  # pair 1 turns by +90 degrees at every position
    _, rc2 = _run(kv, g, c, s, pos, sl, nc, rc, style)
    x = kv[:, :, g.shape[0]:]
    a_i, b_i = (2, 3) if style == oracle.ROPE_PAIRS else (1, 5)
    want = x.copy()
    want[:, :, a_i] = -x[:, :, b_i]
    want[:, :, b_i] = x[:, :, a_i]
    assert np.array_equal(rc2[sl], want)


def test_rotation_preserves_pair_lengths():
    kv, g, c, s, pos, sl, nc, rc = _case("f32", tokens=20, dr=32, max_pos=4096, seed=6)
    pos = np.random.default_rng(7).integers(0, 4096, 20).astype(np.int32)
    _, rc2 = _run(kv, g, c, s, pos, sl, nc, rc, oracle.ROPE_PAIRS)
    x = _vals(kv[:, :, g.shape[0]:])
    y = _vals(rc2[sl])
    lx = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    ly = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    assert np.allclose(ly, lx, rtol=2e-6, atol=1e-12)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scatter_rows_and_skips(dtype):
    kv, g, c, s, pos, sl, nc, rc = _case(dtype, tokens=8, slots=30, max_pos=16, seed=8)
    sl[2] = -1          # padding token
    sl[5] = 30          # beyond the cache
    pos[6] = 16         # beyond the tables
    pos[7] = -3
    nc2, rc2 = _run(kv, g, c, s, pos, sl, nc, rc, oracle.ROPE_PAIRS)
    written = [t for t in range(8) if t not in (2, 5, 6, 7)]
    rows = set(int(sl[t]) for t in written)
    for r in range(30):
        if r not in rows:
            assert np.array_equal(nc2[r], nc[r]) and np.array_equal(rc2[r], rc[r]), r
    # each written row is the token's own result, head by head
    solo_n, solo_r = nc.copy(), rc.copy()
    for t in written:
        one_n, one_r = _run(kv[t:t + 1], g, c, s, pos[t:t + 1], np.array([0]), nc[:1], rc[:1], oracle.ROPE_PAIRS)
        assert np.array_equal(nc2[sl[t]], one_n[0]) and np.array_equal(rc2[sl[t]], one_r[0])
    assert not np.array_equal(nc2[sl[0]], nc[sl[0]])


def test_tables_follow_the_rope_cache_formula():
    """The input tables: angle = pos * theta^(-2i/d) (xserv compute_rope_cache)."""
    c, s = inputs.rope_tables(100, 64, 10000.0)
    assert c.shape == (100, 32) and c.dtype == np.float32
    assert np.all(c[0] == 1) and np.all(s[0] == 0)
    assert abs(float(c[1, 0]) - np.cos(1.0)) < 1e-7 and abs(float(s[99, 31]) - np.sin(99 * 10000.0 ** (-62 / 64))) < 1e-7

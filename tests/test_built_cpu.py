"""The built-configuration mirror (tests/built.py) against the library, and
the automatic choices against what is built -- on the CPU, with fake device
addresses that only ever reach argument validation: with no GPU visible, a
call whose configuration passes every check fails at the launch itself
(RMSNORM_ERR_RUNTIME), while a configuration that is not built is refused
before it (RMSNORM_ERR_INVALID_ARG)."""
import ctypes

import pytest
import torch

import memory_bound_rmsnorm_amd as mbr
from tests import built
from tests.test_abi_cpu import fake_only

INV, RT = mbr.RMSNORM_ERR_INVALID_ARG, mbr.RMSNORM_ERR_RUNTIME
# 64 GiB apart: the largest swept tensor (12289 x 2^20 fp32) is 48 GiB
A, R, W, B, H, O, S, DY, DW, WS = (0x700000000000 + i * (1 << 36) for i in range(10))
ROWS = 8


def _cfg(path, wpr, per):
    return ctypes.byref(mbr.Config(path, wpr, per, 1, 0))


def _fwd(path, dtype, wpr, per, hidden, off=0, fused=False, qt=None):
    L = mbr.lib()
    c = _cfg(path, wpr, per)
    if qt is not None:
        return L.rmsnorm_dynamic_quant_fwd_ex(A + off, R + off if fused else None, W, H + off if fused else None, O,
                                              S, ROWS, hidden, 1e-5, dtype, qt, c, None)
    if fused:
        return L.rmsnorm_residual_fwd_ex(A + off, R + off, W, H + off, O + off, ROWS, hidden, 1e-5, dtype, c, None)
    return L.rmsnorm_fwd_ex(A + off, W, O + off, ROWS, hidden, 1e-5, dtype, c, None)


def _bwd(path, dtype, wpr, per, hidden, off=0):
    return mbr.lib().rmsnorm_bwd_ex(A + off, W, DY + off, O + off, None, ROWS, hidden, 1e-5, dtype, None, 0,
                                    _cfg(path, wpr, per), None)


def _ln(path, dtype, wpr, per, hidden, off=0):
    return mbr.lib().layernorm_fwd_ex(A + off, W, B, O + off, ROWS, hidden, 1e-5, dtype, _cfg(path, wpr, per), None)


def _expect(ok, got, what):
    assert got == (RT if ok else INV), (what, got)


@fake_only
@pytest.mark.parametrize("dtype", [0, 1])
def test_forward_mirror(dtype):
    v = 8 if dtype == 1 else 4
    for fused in (False, True):
        for qt in (None, 0, 1):
            for wpr in built.WPR:
                for per in range(1, 17):
                    lanes = 64 * wpr
                    ok = (built.qvec(wpr, per) if qt is not None else built.vec(wpr, per, fused))
                    for nvec in {lanes * per, lanes * (per - 1) + 1}:
                        _expect(ok and per in built.VEC_VPL, _fwd(1, dtype, wpr, per, nvec * v, 0, fused, qt),
                                ("vector", dtype, fused, qt, wpr, per, nvec))
                    ok = built.qany(wpr, per) if qt is not None else built.any_(wpr, per, fused)
                    _expect(ok, _fwd(4, dtype, wpr, per, lanes * per * v + 1, 16 // v, fused, qt),
                            ("any", dtype, fused, qt, wpr, per))
                for epl in built.EPL:
                    hidden = min(64 * wpr * epl, v - 1)
                    _expect(built.elem(wpr, epl), _fwd(2, dtype, wpr, epl, hidden, 0, fused, qt),
                            ("element", dtype, fused, qt, wpr, epl))


@fake_only
@pytest.mark.parametrize("dtype", [0, 1])
def test_backward_and_layernorm_mirror(dtype):
    v = 8 if dtype == 1 else 4
    for wpr in built.WPR:
        lanes = 64 * wpr
        for per in range(1, 10):
            for nvec in {lanes * per, lanes * (per - 1) + 1}:
                _expect(built.bwd_vec(wpr, per), _bwd(1, dtype, wpr, per, nvec * v), ("bwd vector", wpr, per, nvec))
                _expect(built.ln_vec(wpr, per), _ln(1, dtype, wpr, per, nvec * v), ("ln vector", wpr, per, nvec))
            _expect(built.bwd_any(wpr, per), _bwd(4, dtype, wpr, per, lanes * per * v + 1, 16 // v), ("bwd any", wpr, per))
            _expect(built.ln_any(wpr, per), _ln(4, dtype, wpr, per, lanes * per * v + 1, 16 // v), ("ln any", wpr, per))
        for epl in (1, 2, 4, 8):
            hidden = min(64 * wpr * epl, v - 1)
            _expect(built.elem(wpr, epl), _bwd(2, dtype, wpr, epl, hidden), ("bwd element", wpr, epl))
            _expect(built.elem(wpr, epl), _ln(2, dtype, wpr, epl, hidden), ("ln element", wpr, epl))


def _widths():
    return sorted(set(range(1, 1100)) | set(range(1100, 20000, 37)) | set(range(20000, 170000, 1021))
                  | {2048, 4096, 5120, 6144, 7168, 8192, 16384, 32768, 65536, 81920, 81928, 131072, 131080,
                     163328, 163336, 1 << 20})


@fake_only
@pytest.mark.parametrize("rows", [1, 300, 1024, 2048, 4096, 12289])
def test_every_automatic_choice_is_built(rows):
    """The automatic choice of every entry point, over widths 1 .. 2^20 at both
    alignments, never names a configuration that is not built."""
    L = mbr.lib()
    n = 0
    for dtype in (0, 1):
        for hidden in _widths():
            for off in (0, 16 // (8 if dtype else 4)):  # 16-byte aligned, or one element past it
                for fn, args in (
                        (L.rmsnorm_fwd, (A + off, W, O + off, rows, hidden, 1e-5, dtype, None)),
                        (L.rmsnorm_residual_fwd, (A + off, R + off, W, H + off, O + off, rows, hidden, 1e-5, dtype,
                                                  None)),
                        (L.rmsnorm_dynamic_quant_fwd, (A + off, None, W, None, O, S, rows, hidden, 1e-5, dtype, 0,
                                                       None)),
                        (L.rmsnorm_dynamic_quant_fwd, (A + off, R + off, W, H + off, O, S, rows, hidden, 1e-5, dtype,
                                                       1, None)),
                        (L.rmsnorm_bwd, (A + off, W, DY + off, O + off, None, rows, hidden, 1e-5, dtype, None, 0,
                                         None)),
                        (L.layernorm_fwd, (A + off, W, B, O + off, rows, hidden, 1e-5, dtype, None))):
                    got = fn(*args)
                    assert got == RT, (fn.__name__, dtype, hidden, off, rows, got)
                    n += 1
                need = mbr.rmsnorm_bwd_workspace_size(rows, hidden, torch.bfloat16 if dtype else torch.float32)
                got = L.rmsnorm_bwd(A + off, W, DY + off, O + off, DW, rows, hidden, 1e-5, dtype, WS, need, None)
                assert got == RT, ("rmsnorm_bwd with dweight", dtype, hidden, off, rows, got)
    assert n > 40000

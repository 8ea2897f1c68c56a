"""CPU reference oracle for RMSNorm -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product (``memory_bound_rmsnorm_amd``)
never imports it and has no CPU fallback.

The arithmetic lives in ``rmsnorm_oracle.c`` (fp64, one rounding per output);
this module only moves numpy arrays in and out of it.  Arrays are row-major
``[rows, hidden]``; float32 data is ``np.float32`` and bfloat16 data is the raw
16-bit pattern in ``np.uint16``.

Pinning status: every function here is checked against closed forms,
bit-exact special cases and an exact-rational brute force --
``tests/test_oracle_pins.py`` (forward, fused residual),
``tests/test_oracle_quant_pins.py`` (dynamic quantisation) and
``tests/test_oracle_bwd_pins.py`` (backward: 80-digit central differences of
the forward, closed forms, invariants) and ``tests/test_oracle_ln_pins.py``
(LayerNorm: torch's float64 layer_norm, closed forms, exact invariances) and
``tests/test_oracle_kv_pins.py`` (KV RMSNorm + RoPE + cache scatter).
The only unpinned choice is which bf16 neighbour is returned when the exact
result lies within the fp64 evaluation error (about 1e-12 relative) of a
rounding midpoint.

``unrounded=True`` on the normalising functions returns the float64 value each
output has before its one rounding (the same arithmetic, stopped short of the
store).  Comparisons use it to check that a result is a correct rounding of a
value within the evaluation error of the exact one, which tells nearest-even
apart from truncation or double rounding; ``round_bf16_array`` and
``round_f32_array`` apply the oracle's roundings to such arrays.
"""
import ctypes
import os

import numpy as np

from . import build as _build

F32 = 0
BF16 = 1
F64 = 2  # output only: unrounded

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        vp, i64, f32, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
        lib.oracle_rmsnorm_fwd.argtypes = [vp, vp, vp, i64, i64, f32, i32, i32]
        lib.oracle_rmsnorm_fwd.restype = i32
        lib.oracle_rmsnorm_residual_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, f32, i32, i32]
        lib.oracle_rmsnorm_residual_fwd.restype = i32
        lib.oracle_round_bf16.argtypes = [ctypes.c_double]
        lib.oracle_round_bf16.restype = ctypes.c_uint16
        lib.oracle_round_f32.argtypes = [ctypes.c_double]
        lib.oracle_round_f32.restype = ctypes.c_float
        lib.oracle_round_e4m3.argtypes = [ctypes.c_double]
        lib.oracle_round_e4m3.restype = ctypes.c_uint8
        lib.oracle_round_bf16_n.argtypes = [vp, vp, i64]
        lib.oracle_round_bf16_n.restype = None
        lib.oracle_round_f32_n.argtypes = [vp, vp, i64]
        lib.oracle_round_f32_n.restype = None
        lib.oracle_rmsnorm_dynamic_quant_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, f32, i32, i32]
        lib.oracle_rmsnorm_dynamic_quant_fwd.restype = i32
        lib.oracle_rmsnorm_bwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, f32, i32, i32]
        lib.oracle_rmsnorm_bwd.restype = i32
        lib.oracle_layernorm_fwd.argtypes = [vp, vp, vp, vp, i64, i64, f32, i32, i32]
        lib.oracle_layernorm_fwd.restype = i32
        lib.oracle_kv_rmsnorm_rope_cache.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                                     f32, i32, i32, i32]
        lib.oracle_kv_rmsnorm_rope_cache.restype = i32
        _lib = lib
    return _lib


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError("oracle arrays must be float32 or uint16 (bf16 bits), got %s" % a.dtype)


def _check(a: np.ndarray, name: str) -> np.ndarray:
    if a.ndim != 2:
        raise ValueError("%s must be 2-D [rows, hidden]" % name)
    return np.ascontiguousarray(a)


def _out(like: np.ndarray, unrounded: bool) -> np.ndarray:
    return np.empty(like.shape, np.float64) if unrounded else np.empty_like(like)


def rmsnorm_fwd(x: np.ndarray, weight: np.ndarray, eps: float, unrounded: bool = False) -> np.ndarray:
    """RMSNorm of every row of ``x`` (float32 or bf16-bits), same dtype out
    (float64 before the rounding with ``unrounded``)."""
    x = _check(x, "x")
    weight = np.ascontiguousarray(weight).reshape(-1)
    code = _dtype_code(x)
    if weight.dtype != x.dtype or weight.shape[0] != x.shape[1]:
        raise ValueError("weight must be [hidden] with the dtype of x")
    out = _out(x, unrounded)
    rc = _load().oracle_rmsnorm_fwd(x.ctypes.data, weight.ctypes.data, out.ctypes.data,
                                    x.shape[0], x.shape[1], float(eps), code, F64 if unrounded else code)
    if rc != 0:
        raise RuntimeError("oracle_rmsnorm_fwd failed")
    return out


def rmsnorm_residual_fwd(x: np.ndarray, residual: np.ndarray, weight: np.ndarray, eps: float,
                         unrounded: bool = False):
    """Returns ``(h, y)``: h = round(x + residual), y = RMSNorm(h) (y in
    float64 before its rounding with ``unrounded``; h is always rounded)."""
    x = _check(x, "x")
    residual = _check(residual, "residual")
    weight = np.ascontiguousarray(weight).reshape(-1)
    code = _dtype_code(x)
    if residual.dtype != x.dtype or residual.shape != x.shape:
        raise ValueError("residual must match x")
    if weight.dtype != x.dtype or weight.shape[0] != x.shape[1]:
        raise ValueError("weight must be [hidden] with the dtype of x")
    h = np.empty_like(x)
    y = _out(x, unrounded)
    rc = _load().oracle_rmsnorm_residual_fwd(x.ctypes.data, residual.ctypes.data,
                                             weight.ctypes.data, h.ctypes.data, y.ctypes.data,
                                             x.shape[0], x.shape[1], float(eps), code, F64 if unrounded else code)
    if rc != 0:
        raise RuntimeError("oracle_rmsnorm_residual_fwd failed")
    return h, y


QUANT_INT8 = 0
QUANT_FP8_E4M3 = 1


def rmsnorm_dynamic_quant_fwd(x: np.ndarray, weight: np.ndarray, eps: float, qtype: int,
                              residual: np.ndarray = None):
    """Returns ``(h, q, scale)``: h = round(x + residual) (None without a
    residual), q the int8 codes (``np.int8``) or e4m3fn codes (``np.uint8``) of
    the RMSNorm output quantised per row, scale the per-row float32 scales."""
    x = _check(x, "x")
    weight = np.ascontiguousarray(weight).reshape(-1)
    code = _dtype_code(x)
    if weight.dtype != x.dtype or weight.shape[0] != x.shape[1]:
        raise ValueError("weight must be [hidden] with the dtype of x")
    h = None
    if residual is not None:
        residual = _check(residual, "residual")
        if residual.dtype != x.dtype or residual.shape != x.shape:
            raise ValueError("residual must match x")
        h = np.empty_like(x)
    q = np.empty(x.shape, dtype=np.int8 if qtype == QUANT_INT8 else np.uint8)
    scale = np.empty(x.shape[0], dtype=np.float32)
    rc = _load().oracle_rmsnorm_dynamic_quant_fwd(
        x.ctypes.data, residual.ctypes.data if residual is not None else None, weight.ctypes.data,
        h.ctypes.data if h is not None else None, q.ctypes.data, scale.ctypes.data,
        x.shape[0], x.shape[1], float(eps), code, int(qtype))
    if rc != 0:
        raise RuntimeError("oracle_rmsnorm_dynamic_quant_fwd failed")
    return h, q, scale


def rmsnorm_bwd(x: np.ndarray, weight: np.ndarray, dy: np.ndarray, eps: float, want_dw: bool = True,
                want_dx: bool = True, unrounded: bool = False):
    """Returns ``(dx, dw)`` of y = RMSNorm(x) * weight for upstream gradient dy
    (either is None when not wanted; float64 before the rounding with
    ``unrounded``)."""
    x = _check(x, "x")
    dy = _check(dy, "dy")
    weight = np.ascontiguousarray(weight).reshape(-1)
    code = _dtype_code(x)
    if dy.dtype != x.dtype or dy.shape != x.shape:
        raise ValueError("dy must match x")
    if weight.dtype != x.dtype or weight.shape[0] != x.shape[1]:
        raise ValueError("weight must be [hidden] with the dtype of x")
    dx = _out(x, unrounded) if want_dx else None
    dw = _out(weight, unrounded) if want_dw else None
    rc = _load().oracle_rmsnorm_bwd(x.ctypes.data, weight.ctypes.data, dy.ctypes.data,
                                    dx.ctypes.data if dx is not None else None,
                                    dw.ctypes.data if dw is not None else None, x.shape[0], x.shape[1],
                                    float(eps), code, F64 if unrounded else code)
    if rc != 0:
        raise RuntimeError("oracle_rmsnorm_bwd failed")
    return dx, dw


def layernorm_fwd(x: np.ndarray, gamma: np.ndarray, beta, eps: float, unrounded: bool = False) -> np.ndarray:
    """LayerNorm of every row of ``x``: gamma * (x - mean) / sqrt(var + eps) + beta
    (beta None: no bias), same dtype out (float64 before the rounding with
    ``unrounded``)."""
    x = _check(x, "x")
    gamma = np.ascontiguousarray(gamma).reshape(-1)
    code = _dtype_code(x)
    if gamma.dtype != x.dtype or gamma.shape[0] != x.shape[1]:
        raise ValueError("gamma must be [hidden] with the dtype of x")
    if beta is not None:
        beta = np.ascontiguousarray(beta).reshape(-1)
        if beta.dtype != x.dtype or beta.shape[0] != x.shape[1]:
            raise ValueError("beta must be [hidden] with the dtype of x")
    out = _out(x, unrounded)
    rc = _load().oracle_layernorm_fwd(x.ctypes.data, gamma.ctypes.data,
                                      beta.ctypes.data if beta is not None else None, out.ctypes.data,
                                      x.shape[0], x.shape[1], float(eps), code, F64 if unrounded else code)
    if rc != 0:
        raise RuntimeError("oracle_layernorm_fwd failed")
    return out


ROPE_HALVES = 0
ROPE_PAIRS = 1


def kv_rmsnorm_rope_cache(kv: np.ndarray, gamma: np.ndarray, cos_t: np.ndarray, sin_t: np.ndarray,
                          positions: np.ndarray, slots: np.ndarray, norm_cache: np.ndarray, rope_cache: np.ndarray,
                          eps: float, rope_style: int) -> None:
    """Writes RMSNorm(kv[..., :Dn]) * gamma into norm_cache[slot] and the RoPE of
    kv[..., Dn:] into rope_cache[slot], in place.  kv [tokens, heads, Dn + Dr];
    caches [num_slots, heads, Dn] and [num_slots, heads, Dr] (same dtype as kv,
    or both float64 for the values before their rounding);
    cos_t / sin_t float32 [max_pos, Dr / 2]; positions int32 [tokens]; slots
    int64 [tokens]."""
    if kv.ndim != 3 or norm_cache.ndim != 3 or rope_cache.ndim != 3:
        raise ValueError("kv and the caches must be 3-D")
    tokens, heads, d = kv.shape
    norm_dim, rope_dim = norm_cache.shape[2], rope_cache.shape[2]
    code = _dtype_code(kv)
    if norm_dim + rope_dim != d or norm_cache.shape[1] != heads or rope_cache.shape[1] != heads:
        raise ValueError("cache shapes do not match kv")
    if norm_cache.shape[0] != rope_cache.shape[0]:
        raise ValueError("the two caches must have the same number of slots")
    unrounded = norm_cache.dtype == np.float64
    for a in (norm_cache, rope_cache):
        if a.dtype != (np.float64 if unrounded else kv.dtype) or not a.flags.c_contiguous:
            raise ValueError("the caches must be contiguous, both with the dtype of kv or both float64")
    gamma = np.ascontiguousarray(gamma).reshape(-1)
    if gamma.dtype != kv.dtype or gamma.shape[0] != norm_dim:
        raise ValueError("gamma must be [norm_dim] with the dtype of kv")
    cos_t = np.ascontiguousarray(cos_t, dtype=np.float32)
    sin_t = np.ascontiguousarray(sin_t, dtype=np.float32)
    if cos_t.shape != sin_t.shape or cos_t.ndim != 2 or cos_t.shape[1] != rope_dim // 2:
        raise ValueError("tables must be [max_pos, rope_dim / 2]")
    positions = np.ascontiguousarray(positions, dtype=np.int32)
    slots = np.ascontiguousarray(slots, dtype=np.int64)
    if positions.shape != (tokens,) or slots.shape != (tokens,):
        raise ValueError("positions and slots must have one entry per token")
    kv = np.ascontiguousarray(kv)
    rc = _load().oracle_kv_rmsnorm_rope_cache(
        kv.ctypes.data, gamma.ctypes.data, cos_t.ctypes.data, sin_t.ctypes.data, positions.ctypes.data,
        slots.ctypes.data, norm_cache.ctypes.data, rope_cache.ctypes.data, tokens, heads, norm_dim, rope_dim,
        cos_t.shape[0], norm_cache.shape[0], float(eps), int(rope_style), code, F64 if unrounded else code)
    if rc != 0:
        raise RuntimeError("oracle_kv_rmsnorm_rope_cache failed")


def round_e4m3(v: float) -> int:
    """Nearest-even fp8 e4m3fn code of a Python float, saturating at 448."""
    return int(_load().oracle_round_e4m3(float(v)))


def round_bf16(v: float) -> int:
    """Nearest-even bf16 bit pattern of a Python float (fp64), one rounding."""
    return int(_load().oracle_round_bf16(float(v)))


def round_f32(v: float) -> float:
    return float(_load().oracle_round_f32(float(v)))


def round_bf16_array(v: np.ndarray) -> np.ndarray:
    """Nearest-even bf16 bit patterns of a float64 array, one rounding each."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, np.uint16)
    _load().oracle_round_bf16_n(v.ctypes.data, out.ctypes.data, v.size)
    return out


def round_f32_array(v: np.ndarray) -> np.ndarray:
    """Nearest-even float32 values of a float64 array."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, np.float32)
    _load().oracle_round_f32_n(v.ctypes.data, out.ctypes.data, v.size)
    return out

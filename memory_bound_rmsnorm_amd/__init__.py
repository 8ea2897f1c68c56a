"""Python binding of librmsnorm.so, the gfx950 RMSNorm library.

Argument marshalling only: every function takes torch CUDA (HIP) tensors,
passes their device pointers, sizes, dtype code and the current HIP stream to
the C ABI declared in include/rmsnorm.h, and turns a non-OK status into an
exception.  All arithmetic runs in the HIP kernels; there is no CPU path and no
fallback -- if the library is not built, every call raises.

    rmsnorm_fwd(x, weight, out, eps)                          -> out
    rmsnorm_residual_fwd(x, residual, weight, residual_out, out, eps) -> (residual_out, out)
    rmsnorm_fwd_ex / rmsnorm_residual_fwd_ex(..., config)      forced launch configuration
    rmsnorm_select_config(rows, hidden, dtype, vector_aligned, fused) -> Config
    rmsnorm_dynamic_quant_fwd(x, weight, q_out, scale_out, eps, qtype, residual, residual_out)
    rmsnorm_dynamic_quant_fwd_ex(..., config)                   forced launch configuration
    rmsnorm_select_quant_config(rows, hidden, dtype, vector_aligned, fused) -> Config
    rmsnorm_bwd(x, weight, dy, dx, dweight, eps, workspace)    -> (dx, dweight)
    rmsnorm_bwd_ex(..., config)                                forced launch configuration
    rmsnorm_bwd_workspace_size(rows, hidden, dtype, config)    -> bytes
    rmsnorm_select_bwd_config(rows, hidden, dtype, vector_aligned) -> Config
    rmsnorm_bwd_noalloc(x, weight, dy, dx, dweight, eps)       -> (dx, dweight), no workspace (fixed per-GPU scratch)
    layernorm_fwd(x, gamma, beta, out, eps)                    -> out (beta may be None)
    layernorm_fwd_ex(..., config)                              forced launch configuration
    layernorm_select_config(rows, hidden, dtype, vector_aligned) -> Config
    kv_rmsnorm_rope_cache(kv, gamma, cos, sin, positions, slots, norm_cache, rope_cache, eps, rope_style)
    kv_rmsnorm_rope_cache_ex(..., config), kv_select_config(...) forced / reported configuration
    rmsnorm_status_string(status)                              -> str
    hbm_copy(src, dst)                                         16-byte copy (libhbm_copy.so), the bandwidth ceiling

The backward's weight gradient needs a workspace; when none is passed, a
torch byte tensor of the queried size is allocated for the call (device
memory is the only thing torch provides here).
"""
import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librmsnorm.so")
COPY_LIB_PATH = os.path.join(_HERE, "libhbm_copy.so")

RMSNORM_OK = 0
RMSNORM_ERR_INVALID_ARG = 1
RMSNORM_ERR_UNSUPPORTED_DTYPE = 2
RMSNORM_ERR_RUNTIME = 3

DTYPE_F32 = 0
DTYPE_BF16 = 1

QUANT_INT8 = 0
QUANT_FP8_E4M3 = 1

PATH_AUTO = 0
PATH_VECTOR = 1
PATH_ELEMENT = 2
PATH_TWO_PASS = 3
PATH_VECTOR_ANY = 4
PATH_VECTOR_LDS = 5
PATH_NAMES = {PATH_AUTO: "auto", PATH_VECTOR: "vector", PATH_ELEMENT: "element", PATH_TWO_PASS: "two_pass",
              PATH_VECTOR_ANY: "vector_any", PATH_VECTOR_LDS: "vector_lds"}


class Config(ctypes.Structure):
    """rmsnorm_config_t."""
    _fields_ = [("path", ctypes.c_int32), ("waves_per_row", ctypes.c_int32),
                ("items_per_lane", ctypes.c_int32), ("rows_per_block", ctypes.c_int32),
                ("max_blocks", ctypes.c_int32), ("lanes_per_row", ctypes.c_int32),
                ("weight_lds", ctypes.c_int32)]

    def as_dict(self):
        d = {"path": PATH_NAMES.get(self.path, self.path), "waves_per_row": self.waves_per_row,
             "items_per_lane": self.items_per_lane, "rows_per_block": self.rows_per_block,
             "max_blocks": self.max_blocks}
        if self.lanes_per_row:
            d["lanes_per_row"] = self.lanes_per_row
        if self.weight_lds:
            d["weight_lds"] = self.weight_lds
        return d

    def __repr__(self):
        return "Config(%s)" % ", ".join("%s=%s" % kv for kv in self.as_dict().items())


class RmsnormError(RuntimeError):
    def __init__(self, status: int, fn: str):
        self.status = status
        super().__init__("%s: %s" % (fn, rmsnorm_status_string(status)))


_lib = None
_copy_lib = None


def lib() -> ctypes.CDLL:
    """The loaded librmsnorm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("librmsnorm.so is not built (%s); run `python -m memory_bound_rmsnorm_amd._build` "
                              "or __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, f32, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int32
        cfgp = ctypes.POINTER(Config)
        L.rmsnorm_fwd.argtypes = [vp, vp, vp, i64, i64, f32, i32, vp]
        L.rmsnorm_residual_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, f32, i32, vp]
        L.rmsnorm_fwd_ex.argtypes = [vp, vp, vp, i64, i64, f32, i32, cfgp, vp]
        L.rmsnorm_residual_fwd_ex.argtypes = [vp, vp, vp, vp, vp, i64, i64, f32, i32, cfgp, vp]
        L.rmsnorm_select_config.argtypes = [i64, i64, i32, i32, i32, cfgp]
        L.rmsnorm_select_quant_config.argtypes = [i64, i64, i32, i32, i32, cfgp]
        L.rmsnorm_dynamic_quant_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, f32, i32, i32, vp]
        L.rmsnorm_dynamic_quant_fwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, f32, i32, i32, cfgp, vp]
        L.rmsnorm_bwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, f32, i32, vp, ctypes.c_size_t, vp]
        L.rmsnorm_bwd_ex.argtypes = [vp, vp, vp, vp, vp, i64, i64, f32, i32, vp, ctypes.c_size_t, cfgp, vp]
        L.rmsnorm_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, f32, i32, vp]
        L.rmsnorm_bwd_workspace_size.argtypes = [i64, i64, i32, cfgp, ctypes.POINTER(ctypes.c_size_t)]
        L.rmsnorm_select_bwd_config.argtypes = [i64, i64, i32, i32, cfgp]
        L.layernorm_fwd.argtypes = [vp, vp, vp, vp, i64, i64, f32, i32, vp]
        L.layernorm_fwd_ex.argtypes = [vp, vp, vp, vp, i64, i64, f32, i32, cfgp, vp]
        L.layernorm_select_config.argtypes = [i64, i64, i32, i32, cfgp]
        L.kv_rmsnorm_rope_cache.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, f32, i32,
                                            i32, vp]
        L.kv_rmsnorm_rope_cache_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, f32,
                                               i32, i32, cfgp, vp]
        L.kv_select_config.argtypes = [i64, i64, i64, i64, i32, i32, i32, cfgp]
        L.rmsnorm_status_string.argtypes = [i32]
        L.rmsnorm_status_string.restype = ctypes.c_char_p
        for fn in (L.rmsnorm_fwd, L.rmsnorm_residual_fwd, L.rmsnorm_fwd_ex, L.rmsnorm_residual_fwd_ex,
                   L.rmsnorm_select_config, L.rmsnorm_select_quant_config, L.rmsnorm_dynamic_quant_fwd,
                   L.rmsnorm_dynamic_quant_fwd_ex, L.rmsnorm_bwd, L.rmsnorm_bwd_ex, L.rmsnorm_bwd_noalloc,
                   L.rmsnorm_bwd_workspace_size,
                   L.rmsnorm_select_bwd_config, L.layernorm_fwd, L.layernorm_fwd_ex, L.layernorm_select_config,
                   L.kv_rmsnorm_rope_cache, L.kv_rmsnorm_rope_cache_ex, L.kv_select_config):
            fn.restype = i32
        _lib = L
    return _lib


def copy_lib() -> ctypes.CDLL:
    """The loaded libhbm_copy.so (bandwidth ceiling and counter calibration)."""
    global _copy_lib
    if _copy_lib is None:
        if not os.path.exists(COPY_LIB_PATH):
            raise ImportError("libhbm_copy.so is not built (%s)" % COPY_LIB_PATH)
        L = ctypes.CDLL(COPY_LIB_PATH)
        L.hbm_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p]
        L.hbm_copy.restype = ctypes.c_int
        _copy_lib = L
    return _copy_lib


def rmsnorm_status_string(status: int) -> str:
    return lib().rmsnorm_status_string(int(status)).decode()


def dtype_code(dtype: torch.dtype) -> int:
    if dtype == torch.float32:
        return DTYPE_F32
    if dtype == torch.bfloat16:
        return DTYPE_BF16
    raise TypeError("RMSNorm supports torch.float32 and torch.bfloat16, not %s" % dtype)


def _device_tensor(t: torch.Tensor, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor; this library has no CPU path" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous (row-major)" % name)
    return t


# The current stream's raw handle without building a torch.cuda.Stream object
# (about 1.9 us per call that way, most of the binding's own cost); the public
# route when this torch has no such accessor.
_raw_current_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream, device) -> Optional[int]:
    if stream is None:
        if _raw_current_stream is not None and device.index is not None:
            return _raw_current_stream(device.index)
        return torch.cuda.current_stream(device).cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _shape(x: torch.Tensor, weight: torch.Tensor):
    if x.dim() < 1:
        raise ValueError("x must have at least one dimension")
    hidden = x.shape[-1]
    if weight.dim() != 1 or weight.shape[0] != hidden:
        raise ValueError("weight must have shape [hidden] = [%d]" % hidden)
    rows = x.numel() // hidden if hidden else 0
    return rows, hidden


def _check(status: int, fn: str):
    if status != RMSNORM_OK:
        raise RmsnormError(status, fn)


def rmsnorm_fwd_ex(x, weight, out, eps: float = 1e-5, config: Optional[Config] = None, stream=None):
    """out = RMSNorm(x) * weight over the last dimension, with a forced configuration."""
    for t, n in ((x, "x"), (weight, "weight"), (out, "out")):
        _device_tensor(t, n)
    if out.shape != x.shape or out.dtype != x.dtype or weight.dtype != x.dtype:
        raise ValueError("out must match x in shape and dtype; weight must match x in dtype")
    rows, hidden = _shape(x, weight)
    st = lib().rmsnorm_fwd_ex(x.data_ptr(), weight.data_ptr(), out.data_ptr(), rows, hidden, float(eps),
                              dtype_code(x.dtype), ctypes.byref(config) if config is not None else None,
                              _stream(stream, x.device))
    _check(st, "rmsnorm_fwd")
    return out


def rmsnorm_fwd(x, weight, out, eps: float = 1e-5, stream=None):
    """out = RMSNorm(x) * weight over the last dimension (C: rmsnorm_fwd)."""
    return rmsnorm_fwd_ex(x, weight, out, eps, None, stream)


def rmsnorm_residual_fwd_ex(x, residual, weight, residual_out, out, eps: float = 1e-5,
                            config: Optional[Config] = None, stream=None):
    for t, n in ((x, "x"), (residual, "residual"), (weight, "weight"), (residual_out, "residual_out"),
                 (out, "out")):
        _device_tensor(t, n)
    for t in (residual, residual_out, out):
        if t.shape != x.shape or t.dtype != x.dtype:
            raise ValueError("residual, residual_out and out must match x in shape and dtype")
    if weight.dtype != x.dtype:
        raise ValueError("weight must match x in dtype")
    rows, hidden = _shape(x, weight)
    st = lib().rmsnorm_residual_fwd_ex(x.data_ptr(), residual.data_ptr(), weight.data_ptr(),
                                       residual_out.data_ptr(), out.data_ptr(), rows, hidden, float(eps),
                                       dtype_code(x.dtype), ctypes.byref(config) if config is not None else None,
                                       _stream(stream, x.device))
    _check(st, "rmsnorm_residual_fwd")
    return residual_out, out


def rmsnorm_residual_fwd(x, residual, weight, residual_out, out, eps: float = 1e-5, stream=None):
    """residual_out = x + residual (rounded once); out = RMSNorm(residual_out) * weight
    (C: rmsnorm_residual_fwd)."""
    return rmsnorm_residual_fwd_ex(x, residual, weight, residual_out, out, eps, None, stream)


def rmsnorm_select_config(rows: int, hidden: int, dtype, vector_aligned: bool = True,
                          fused: bool = False) -> Config:
    """The configuration the automatic choice uses for this shape."""
    code = dtype_code(dtype) if isinstance(dtype, torch.dtype) else int(dtype)
    cfg = Config()
    _check(lib().rmsnorm_select_config(int(rows), int(hidden), code, int(bool(vector_aligned)),
                                       int(bool(fused)), ctypes.byref(cfg)), "rmsnorm_select_config")
    return cfg


def rmsnorm_dynamic_quant_fwd_ex(x, weight, q_out, scale_out, eps: float = 1e-5, qtype: int = QUANT_INT8,
                                 residual=None, residual_out=None, config: Optional[Config] = None, stream=None):
    """(residual add +) RMSNorm + per-row dynamic quantisation with a forced
    configuration.  q_out: one-byte tensor shaped like x (int8, uint8 or an
    fp8 dtype); scale_out: float32 tensor with one element per row."""
    for t, n in ((x, "x"), (weight, "weight"), (q_out, "q_out"), (scale_out, "scale_out")):
        _device_tensor(t, n)
    if (residual is None) != (residual_out is None):
        raise ValueError("residual and residual_out go together")
    if residual is not None:
        for t, n in ((residual, "residual"), (residual_out, "residual_out")):
            _device_tensor(t, n)
            if t.shape != x.shape or t.dtype != x.dtype:
                raise ValueError("%s must match x in shape and dtype" % n)
    if weight.dtype != x.dtype:
        raise ValueError("weight must match x in dtype")
    rows, hidden = _shape(x, weight)
    if q_out.shape != x.shape or q_out.element_size() != 1:
        raise ValueError("q_out must be a one-byte tensor shaped like x")
    if scale_out.dtype != torch.float32 or scale_out.numel() != rows:
        raise ValueError("scale_out must be float32 with one element per row")
    st = lib().rmsnorm_dynamic_quant_fwd_ex(
        x.data_ptr(), residual.data_ptr() if residual is not None else None, weight.data_ptr(),
        residual_out.data_ptr() if residual_out is not None else None, q_out.data_ptr(), scale_out.data_ptr(),
        rows, hidden, float(eps), dtype_code(x.dtype), int(qtype),
        ctypes.byref(config) if config is not None else None, _stream(stream, x.device))
    _check(st, "rmsnorm_dynamic_quant_fwd")
    return q_out, scale_out


def rmsnorm_dynamic_quant_fwd(x, weight, q_out, scale_out, eps: float = 1e-5, qtype: int = QUANT_INT8,
                              residual=None, residual_out=None, stream=None):
    """(residual add +) RMSNorm + per-row dynamic quantisation (C: rmsnorm_dynamic_quant_fwd)."""
    return rmsnorm_dynamic_quant_fwd_ex(x, weight, q_out, scale_out, eps, qtype, residual, residual_out, None, stream)


def rmsnorm_select_quant_config(rows: int, hidden: int, dtype, vector_aligned: bool = True,
                                fused: bool = False) -> Config:
    code = dtype_code(dtype) if isinstance(dtype, torch.dtype) else int(dtype)
    cfg = Config()
    _check(lib().rmsnorm_select_quant_config(int(rows), int(hidden), code, int(bool(vector_aligned)),
                                             int(bool(fused)), ctypes.byref(cfg)), "rmsnorm_select_quant_config")
    return cfg


def rmsnorm_bwd_workspace_size(rows: int, hidden: int, dtype, config: Optional[Config] = None) -> int:
    """Workspace bytes the backward needs for dweight (C: rmsnorm_bwd_workspace_size)."""
    code = dtype_code(dtype) if isinstance(dtype, torch.dtype) else int(dtype)
    n = ctypes.c_size_t()
    _check(lib().rmsnorm_bwd_workspace_size(int(rows), int(hidden), code,
                                            ctypes.byref(config) if config is not None else None,
                                            ctypes.byref(n)), "rmsnorm_bwd_workspace_size")
    return int(n.value)


def rmsnorm_select_bwd_config(rows: int, hidden: int, dtype, vector_aligned: bool = True) -> Config:
    code = dtype_code(dtype) if isinstance(dtype, torch.dtype) else int(dtype)
    cfg = Config()
    _check(lib().rmsnorm_select_bwd_config(int(rows), int(hidden), code, int(bool(vector_aligned)),
                                           ctypes.byref(cfg)), "rmsnorm_select_bwd_config")
    return cfg


def rmsnorm_bwd_ex(x, weight, dy, dx, dweight=None, eps: float = 1e-5, workspace=None,
                   config: Optional[Config] = None, stream=None):
    """dx (and dweight unless None) of y = RMSNorm(x) * weight for the upstream
    gradient dy, with a forced configuration.  workspace: a contiguous GPU
    tensor of at least rmsnorm_bwd_workspace_size bytes, or None."""
    for t, n in ((x, "x"), (weight, "weight"), (dy, "dy"), (dx, "dx")):
        _device_tensor(t, n)
    for t, n in ((dy, "dy"), (dx, "dx")):
        if t.shape != x.shape or t.dtype != x.dtype:
            raise ValueError("%s must match x in shape and dtype" % n)
    if weight.dtype != x.dtype:
        raise ValueError("weight must match x in dtype")
    rows, hidden = _shape(x, weight)
    ws_ptr, ws_bytes = None, 0
    if dweight is not None:
        _device_tensor(dweight, "dweight")
        if dweight.shape != weight.shape or dweight.dtype != x.dtype:
            raise ValueError("dweight must match weight in shape and dtype")
        if workspace is None:
            need = rmsnorm_bwd_workspace_size(rows, hidden, x.dtype, config)
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
            if stream is not None:  # freed on return: keep it from reuse until that stream has run
                workspace.record_stream(stream if isinstance(stream, torch.cuda.Stream)
                                        else torch.cuda.ExternalStream(int(stream)))
        _device_tensor(workspace, "workspace")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    st = lib().rmsnorm_bwd_ex(x.data_ptr(), weight.data_ptr(), dy.data_ptr(), dx.data_ptr(),
                              dweight.data_ptr() if dweight is not None else None, rows, hidden, float(eps),
                              dtype_code(x.dtype), ws_ptr, ws_bytes,
                              ctypes.byref(config) if config is not None else None, _stream(stream, x.device))
    _check(st, "rmsnorm_bwd")
    return dx, dweight


def rmsnorm_bwd(x, weight, dy, dx, dweight=None, eps: float = 1e-5, workspace=None, stream=None):
    """RMSNorm backward (C: rmsnorm_bwd)."""
    return rmsnorm_bwd_ex(x, weight, dy, dx, dweight, eps, workspace, None, stream)


def rmsnorm_bwd_noalloc(x, weight, dy, dx, dweight=None, eps: float = 1e-5, stream=None):
    """RMSNorm backward with no workspace and no allocation (C:
    rmsnorm_bwd_noalloc): the partial dweight rows live in the library's
    per-GPU scratch array, so calls on one GPU must not overlap in time."""
    for t, n in ((x, "x"), (weight, "weight"), (dy, "dy"), (dx, "dx")):
        _device_tensor(t, n)
    for t, n in ((dy, "dy"), (dx, "dx")):
        if t.shape != x.shape or t.dtype != x.dtype:
            raise ValueError("%s must match x in shape and dtype" % n)
    if weight.dtype != x.dtype:
        raise ValueError("weight must match x in dtype")
    rows, hidden = _shape(x, weight)
    if dweight is not None:
        _device_tensor(dweight, "dweight")
        if dweight.shape != weight.shape or dweight.dtype != x.dtype:
            raise ValueError("dweight must match weight in shape and dtype")
    st = lib().rmsnorm_bwd_noalloc(x.data_ptr(), weight.data_ptr(), dy.data_ptr(), dx.data_ptr(),
                                   dweight.data_ptr() if dweight is not None else None, rows, hidden, float(eps),
                                   dtype_code(x.dtype), _stream(stream, x.device))
    _check(st, "rmsnorm_bwd_noalloc")
    return dx, dweight


def layernorm_fwd_ex(x, gamma, beta, out, eps: float = 1e-5, config: Optional[Config] = None, stream=None):
    """out = LayerNorm(x) * gamma + beta over the last dimension (beta None: no
    bias), with a forced configuration."""
    for t, n in ((x, "x"), (gamma, "gamma"), (out, "out")):
        _device_tensor(t, n)
    if out.shape != x.shape or out.dtype != x.dtype or gamma.dtype != x.dtype:
        raise ValueError("out must match x in shape and dtype; gamma must match x in dtype")
    rows, hidden = _shape(x, gamma)
    if beta is not None:
        _device_tensor(beta, "beta")
        if beta.shape != gamma.shape or beta.dtype != x.dtype:
            raise ValueError("beta must match gamma in shape and dtype")
    st = lib().layernorm_fwd_ex(x.data_ptr(), gamma.data_ptr(), beta.data_ptr() if beta is not None else None,
                                out.data_ptr(), rows, hidden, float(eps), dtype_code(x.dtype),
                                ctypes.byref(config) if config is not None else None, _stream(stream, x.device))
    _check(st, "layernorm_fwd")
    return out


def layernorm_fwd(x, gamma, beta, out, eps: float = 1e-5, stream=None):
    """LayerNorm over the last dimension (C: layernorm_fwd)."""
    return layernorm_fwd_ex(x, gamma, beta, out, eps, None, stream)


def layernorm_select_config(rows: int, hidden: int, dtype, vector_aligned: bool = True) -> Config:
    code = dtype_code(dtype) if isinstance(dtype, torch.dtype) else int(dtype)
    cfg = Config()
    _check(lib().layernorm_select_config(int(rows), int(hidden), code, int(bool(vector_aligned)),
                                         ctypes.byref(cfg)), "layernorm_select_config")
    return cfg


ROPE_HALVES = 0
ROPE_PAIRS = 1


def kv_rmsnorm_rope_cache(kv, gamma, cos_table, sin_table, positions, slots, norm_cache, rope_cache,
                          eps: float = 1e-6, rope_style: int = ROPE_PAIRS, stream=None):
    """RMSNorm of kv[..., :norm_dim] into norm_cache[slot] and RoPE of
    kv[..., norm_dim:] into rope_cache[slot] (C: kv_rmsnorm_rope_cache).
    kv [tokens, heads, norm_dim + rope_dim]; caches [num_slots, heads, dim];
    tables float32 [max_pos, rope_dim / 2]; positions int32, slots int64."""
    return kv_rmsnorm_rope_cache_ex(kv, gamma, cos_table, sin_table, positions, slots, norm_cache, rope_cache,
                                    eps, rope_style, None, stream)


def kv_select_config(tokens: int, heads: int, norm_dim: int, rope_dim: int, rope_style: int, dtype,
                     vector_aligned: bool = True) -> Config:
    """The configuration kv_rmsnorm_rope_cache uses for this shape."""
    code = dtype_code(dtype) if isinstance(dtype, torch.dtype) else int(dtype)
    cfg = Config()
    _check(lib().kv_select_config(int(tokens), int(heads), int(norm_dim), int(rope_dim), int(rope_style), code,
                                  int(bool(vector_aligned)), ctypes.byref(cfg)), "kv_select_config")
    return cfg


def kv_rmsnorm_rope_cache_ex(kv, gamma, cos_table, sin_table, positions, slots, norm_cache, rope_cache,
                             eps: float = 1e-6, rope_style: int = ROPE_PAIRS, config: Optional[Config] = None,
                             stream=None):
    """kv_rmsnorm_rope_cache with a forced configuration (None: automatic)."""
    for t, n in ((kv, "kv"), (gamma, "gamma"), (positions, "positions"), (slots, "slots"),
                 (norm_cache, "norm_cache"), (rope_cache, "rope_cache"), (cos_table, "cos_table"),
                 (sin_table, "sin_table")):
        _device_tensor(t, n)
    if kv.dim() != 3 or norm_cache.dim() != 3 or rope_cache.dim() != 3:
        raise ValueError("kv and the caches must be 3-D")
    tokens, heads, d = kv.shape
    norm_dim, rope_dim = norm_cache.shape[2], rope_cache.shape[2]
    if norm_dim + rope_dim != d or norm_cache.shape[1] != heads or rope_cache.shape[1] != heads or \
            norm_cache.shape[0] != rope_cache.shape[0]:
        raise ValueError("cache shapes do not match kv")
    for t, n in ((gamma, "gamma"), (norm_cache, "norm_cache"), (rope_cache, "rope_cache")):
        if t.dtype != kv.dtype:
            raise ValueError("%s must have the dtype of kv" % n)
    if gamma.dim() != 1 or gamma.shape[0] != norm_dim:
        raise ValueError("gamma must be [norm_dim]")
    if cos_table.dtype != torch.float32 or sin_table.dtype != torch.float32 or cos_table.shape != sin_table.shape \
            or cos_table.dim() != 2 or cos_table.shape[1] != rope_dim // 2:
        raise ValueError("tables must be float32 [max_pos, rope_dim / 2]")
    if positions.dtype != torch.int32 or slots.dtype != torch.int64 or positions.numel() != tokens or \
            slots.numel() != tokens:
        raise ValueError("positions (int32) and slots (int64) need one entry per token")
    st = lib().kv_rmsnorm_rope_cache_ex(kv.data_ptr(), gamma.data_ptr(), cos_table.data_ptr(),
                                        sin_table.data_ptr(), positions.data_ptr(), slots.data_ptr(),
                                        norm_cache.data_ptr(), rope_cache.data_ptr(), tokens, heads, norm_dim,
                                        rope_dim, cos_table.shape[0], norm_cache.shape[0], float(eps),
                                        int(rope_style), dtype_code(kv.dtype),
                                        ctypes.byref(config) if config is not None else None,
                                        _stream(stream, kv.device))
    _check(st, "kv_rmsnorm_rope_cache")
    return norm_cache, rope_cache


def hbm_copy(src: torch.Tensor, dst: torch.Tensor, max_blocks: int = 0, stream=None):
    """Plain 16-byte-vector copy of src's bytes into dst (bandwidth ceiling)."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst too small")
    rc = copy_lib().hbm_copy(src.data_ptr(), dst.data_ptr(), nbytes, int(max_blocks), _stream(stream, src.device))
    if rc != 0:
        raise RuntimeError("hbm_copy failed with code %d" % rc)
    return dst

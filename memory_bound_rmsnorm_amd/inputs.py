"""Seeded synthetic inputs for the RMSNorm workloads.

This module only draws random numbers and stores them in the tensor dtype; it
contains no RMSNorm arithmetic, so both the HIP path's tests/benchmark and the
CPU oracle can take their inputs from here without sharing any of the method.

Recipe (one ``numpy.random.default_rng(seed)`` stream per workload):
  * draw order is x, then residual (fused workloads only) or the upstream
    gradient dy (backward workloads only), then weight (gamma), then beta
    (LayerNorm workloads only);
  * ``N(mu, sigma)`` means ``standard_normal(float32) * sigma + mu``
    (sigma is a standard deviation), ``U(a, b)`` means ``uniform(a, b)``
    cast to float32;
  * outlier channels, where a workload has them, are scaled before storing;
  * bf16 tensors are the float32 draws rounded once, to nearest-even, by
    torch's CPU conversion.

The shapes are the Llama-style activations the pages discuss: hidden 2048 at
the Llama-3.2-1B size used by the gollamago project (README, "性能测量", bf16
rows=4096 x columns=2048), a decode-sized batch, a large-hidden headline shape
and a fused residual shape with an odd row count.  Synthetic normal rows stand
in for real activations; no model weights or datasets are involved.
"""
from dataclasses import dataclass, field
from typing import Dict, Optional, Tuple

import numpy as np
import torch

# Eight fixed columns, one in each of the eight bf16 positions of a 16-byte
# vector (stride 1021), scaled x100 in the large-hidden workload.
OUTLIER_COLUMNS: Tuple[int, ...] = (13, 1034, 2055, 3076, 4097, 5118, 6139, 7160)


@dataclass(frozen=True)
class Dist:
    kind: str  # "normal" (a = mean, b = std) or "uniform" (a = low, b = high)
    a: float
    b: float


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str  # "f32" or "bf16"
    rows: int
    hidden: int
    eps: float
    fused: bool
    x: Dist
    weight: Dist
    residual: Optional[Dist] = None
    outlier_columns: Tuple[int, ...] = ()
    outlier_scale: float = 1.0
    quant: Optional[str] = None  # None: normalised output; "int8" / "fp8": codes + per-row scale
    grad: Optional[Dist] = None  # backward workloads: distribution of the upstream gradient dy
    beta: Optional[Dist] = None  # LayerNorm workloads: distribution of beta (weight is gamma)
    note: str = field(default="", compare=False)

    @property
    def layernorm(self) -> bool:
        return self.beta is not None

    @property
    def backward(self) -> bool:
        return self.grad is not None

    @property
    def elem_size(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def read_bytes(self) -> int:
        # forward: x (and residual) plus weight; backward: x and dy plus weight;
        # LayerNorm: x plus gamma and beta
        params = 2 if self.layernorm else 1
        return ((2 if self.fused or self.backward else 1) * self.rows * self.hidden
                + params * self.hidden) * self.elem_size

    @property
    def write_bytes(self) -> int:
        if self.backward:  # dx and dweight
            return (self.rows * self.hidden + self.hidden) * self.elem_size
        h = self.rows * self.hidden * self.elem_size if self.fused else 0
        if self.quant:
            return h + self.rows * self.hidden + 4 * self.rows
        return h + self.rows * self.hidden * self.elem_size

    @property
    def copy_bytes(self) -> int:
        """Size of the plain copy that moves the same traffic (read == written):
        the output bytes for the normalised forms, half the ledger (rounded
        down to 16 bytes) for the quantised and backward ones."""
        if self.quant or self.backward:
            return (self.algorithmic_bytes // 2) & ~15
        return self.write_bytes

    @property
    def algorithmic_bytes(self) -> int:
        """Each input read once, each output written once, weight once.

        Byte ledger rule: TileLang tutorial ch. 02, section 2.1 (every input
        stored tensor read once, every output written once, intermediates not
        counted)."""
        return self.read_bytes + self.write_bytes


N01 = Dist("normal", 0.0, 1.0)
W_N = Dist("normal", 1.0, 0.1)

WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("fp32_64x2048", "f32", 64, 2048, 1e-5, False, N01, W_N,
                 note="small fp32 case"),
        Workload("bf16_prefill_4096x2048", "bf16", 4096, 2048, 1e-5, False, N01, W_N,
                 note="Llama-1B prefill shape"),
        Workload("bf16_decode_256x4096", "bf16", 256, 4096, 1e-6, False,
                 Dist("normal", 0.0, 2.0), Dist("uniform", 0.5, 1.5),
                 note="decode shape; latency case"),
        Workload("bf16_16384x8192", "bf16", 16384, 8192, 1e-5, False, N01, W_N,
                 outlier_columns=OUTLIER_COLUMNS, outlier_scale=100.0,
                 note="large hidden, 8 outlier channels x100; headline bandwidth case"),
        Workload("bf16_residual_12289x5120", "bf16", 12289, 5120, 1e-5, True, N01, W_N,
                 residual=N01, note="fused residual add; odd row count"),
        Workload("bf16_shard_2048x8192", "bf16", 2048, 8192, 1e-5, False, N01, W_N,
                 outlier_columns=OUTLIER_COLUMNS, outlier_scale=100.0,
                 note="one GPU's rows of the 16384 x 8192 case split by tokens over 8 GPUs"),
    ]
}

HEADLINE = "bf16_16384x8192"

# The same inputs with the output quantised per row (int8 or fp8 e4m3fn codes
# plus one fp32 scale per row): the Add + RmsNorm + DynamicQuant fusion.
QUANT_WORKLOADS: Dict[str, Workload] = {}
for _base in ("bf16_16384x8192", "bf16_residual_12289x5120"):
    for _q in ("int8", "fp8"):
        _w = WORKLOADS[_base]
        _name = _base.replace("bf16_", "bf16_%s_" % _q, 1)
        QUANT_WORKLOADS[_name] = Workload(_name, _w.dtype, _w.rows, _w.hidden, _w.eps, _w.fused, _w.x, _w.weight,
                                          _w.residual, _w.outlier_columns, _w.outlier_scale, quant=_q,
                                          note=_w.note + "; %s output" % _q)
# Backward (dx and dweight) for an upstream gradient dy ~ N(0, 1): the
# large-hidden shape (same x recipe, outlier channels included), the Llama-1B
# prefill shape, and the small fp32 case.
BWD_WORKLOADS: Dict[str, Workload] = {}
for _base in ("bf16_16384x8192", "bf16_prefill_4096x2048", "fp32_64x2048"):
    _w = WORKLOADS[_base]
    _name = _base.replace("bf16_", "bf16_bwd_", 1).replace("fp32_", "fp32_bwd_", 1).replace("prefill_", "")
    BWD_WORKLOADS[_name] = Workload(_name, _w.dtype, _w.rows, _w.hidden, _w.eps, False, _w.x, _w.weight,
                                    outlier_columns=_w.outlier_columns, outlier_scale=_w.outlier_scale,
                                    grad=N01, note=_w.note + "; backward")
# LayerNorm: the pages' worked ledger example ([8192, 4096], fp16 there; bf16
# moves the same bytes), their exercise shape [4096, 4096], and a small fp32
# case at GPT-2's hidden size 768.
LN_WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("bf16_ln_8192x4096", "bf16", 8192, 4096, 1e-5, False, N01, W_N, beta=Dist("normal", 0.0, 0.1),
                 note="LayerNorm, the pages' ledger example shape"),
        Workload("bf16_ln_4096x4096", "bf16", 4096, 4096, 1e-5, False, N01, W_N, beta=Dist("normal", 0.0, 0.1),
                 note="LayerNorm, the pages' exercise shape"),
        Workload("fp32_ln_64x768", "f32", 64, 768, 1e-5, False, N01, W_N, beta=Dist("normal", 0.0, 0.1),
                 note="LayerNorm, small fp32 case at hidden 768"),
    ]
}
# Rows wider than the register path holds (131072 elements, 256 KiB per bf16
# row), plain and fused: the register + LDS path, read once.
WIDE_WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("bf16_wide_2048x131072", "bf16", 2048, 131072, 1e-5, False, N01, W_N,
                 note="rows past the register budget"),
        Workload("bf16_wide_residual_2048x131072", "bf16", 2048, 131072, 1e-5, True, N01, W_N, residual=N01,
                 note="fused rows past the register budget"),
    ]
}
# Two shapes that exercise the forward's other launch forms at full scale:
# per-head rows narrower than a wave (several rows share a wave in lane
# groups), and an odd width (16-byte vectors at the row's own alignment, every
# other row in the shifted frame, plus a tail element).
SHAPE_WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("bf16_narrow_262144x128", "bf16", 262144, 128, 1e-5, False, N01, W_N,
                 note="per-head width: rows narrower than a wave"),
        Workload("bf16_odd_16384x8191", "bf16", 16384, 8191, 1e-5, False, N01, W_N,
                 note="odd width: rows at any element alignment, tail element"),
    ]
}
ALL_WORKLOADS: Dict[str, Workload] = dict(WORKLOADS, **QUANT_WORKLOADS, **BWD_WORKLOADS, **LN_WORKLOADS,
                                          **WIDE_WORKLOADS, **SHAPE_WORKLOADS)


def _draw(rng: np.random.Generator, d: Dist, shape) -> np.ndarray:
    if d.kind == "normal":
        return rng.standard_normal(shape, dtype=np.float32) * np.float32(d.b) + np.float32(d.a)
    if d.kind == "uniform":
        return rng.uniform(d.a, d.b, shape).astype(np.float32)
    raise ValueError("unknown distribution %r" % d.kind)


def _store(a: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if dtype == "f32":
        return t
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    raise ValueError("dtype must be 'f32' or 'bf16'")


def make(w: Workload, seed: int = 0, rows: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """CPU tensors ``x``, ``weight`` (and ``residual`` when fused) for ``w``.

    ``rows`` overrides the row count (same per-row distribution); the draws for
    a smaller ``rows`` are not a prefix of the full-size draws."""
    r = w.rows if rows is None else rows
    rng = np.random.default_rng(seed)
    x = _draw(rng, w.x, (r, w.hidden))
    if w.outlier_columns:
        cols = [c for c in w.outlier_columns if c < w.hidden]
        x[:, cols] *= np.float32(w.outlier_scale)
    out = {"x": _store(x, w.dtype)}
    if w.fused:
        out["residual"] = _store(_draw(rng, w.residual or N01, (r, w.hidden)), w.dtype)
    if w.backward:
        out["dy"] = _store(_draw(rng, w.grad, (r, w.hidden)), w.dtype)
    out["weight"] = _store(_draw(rng, w.weight, (w.hidden,)), w.dtype)
    if w.layernorm:
        out["beta"] = _store(_draw(rng, w.beta, (w.hidden,)), w.dtype)
    return out


def custom(rows: int, hidden: int, dtype: str, fused: bool = False, eps: float = 1e-5,
           x: Dist = N01, weight: Dist = W_N, residual: Dist = N01, backward: bool = False,
           grad: Dist = N01, layernorm: bool = False, beta: Dist = Dist("normal", 0.0, 0.1)) -> Workload:
    """An ad-hoc workload (ragged widths, odd row counts, ...) with the same recipe."""
    return Workload("custom_%s_%dx%d%s%s%s" % (dtype, rows, hidden, "_res" if fused else "", "_bwd" if backward else "",
                                               "_ln" if layernorm else ""),
                    dtype, rows, hidden, eps, fused, x, weight,
                    residual if fused else None, grad=grad if backward else None,
                    beta=beta if layernorm else None)


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw storage of a CPU tensor as numpy: float32 values or bf16 bit patterns."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    raise TypeError("unsupported dtype %s" % t.dtype)


# ---------------------------------------------------------------- KV RMSNorm + RoPE + cache scatter
#
# kv rows [tokens, heads, norm_dim + rope_dim] drawn like x above; gamma like
# the weight; cos / sin tables [max_pos, rope_dim / 2] from the xserv rope
# cache formula (phase 4, csrc/embedding/rope.cu: angle = pos * theta^(-2i /
# rope_dim)), evaluated in float64 and stored as float32; a paged cache of
# num_blocks blocks of block_size rows, each sequence owning a random set of
# blocks listed in its block table (the block_table / cache_seqlens interface
# of the paged MLA decode kernel the TileLang tutorial ch. 02, section 1.2,
# points to); every token's slot is block_table[seq][pos // block_size] *
# block_size + pos % block_size.  The caches start filled with seeded values,
# so that rows a call must not touch can be checked.  The 512 + 64 split is the
# latent + rotary width of the MLA KV cache in that kernel's DeepSeek model
# family; the pages do not print it.


@dataclass(frozen=True)
class KvWorkload:
    name: str
    dtype: str
    seqs: int
    new_tokens: int        # tokens per sequence written by one call
    max_len: int           # cache length per sequence (decode: lengths drawn up to this)
    heads: int
    norm_dim: int
    rope_dim: int
    eps: float
    rope_style: int        # 1: adjacent pairs (xserv), 0: two halves
    decode: bool           # True: one new token per sequence at a random length
    block_size: int = 64
    theta: float = 10000.0
    note: str = field(default="", compare=False)

    @property
    def elem_size(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def tokens(self) -> int:
        return self.seqs * self.new_tokens

    @property
    def blocks_per_seq(self) -> int:
        return -(-self.max_len // self.block_size)

    @property
    def num_blocks(self) -> int:
        return 2 * self.seqs * self.blocks_per_seq  # half of the blocks stay free

    @property
    def num_slots(self) -> int:
        return self.num_blocks * self.block_size

    @property
    def max_pos(self) -> int:
        return self.max_len

    @property
    def read_bytes(self) -> int:
        """kv, the token's two table rows, its position and slot; gamma once."""
        d = self.norm_dim + self.rope_dim
        return self.tokens * (self.heads * d * self.elem_size + self.rope_dim * 4 + 4 + 8) + \
            self.norm_dim * self.elem_size

    @property
    def write_bytes(self) -> int:
        """Both cache rows of every token."""
        return self.tokens * self.heads * (self.norm_dim + self.rope_dim) * self.elem_size

    @property
    def algorithmic_bytes(self) -> int:
        return self.read_bytes + self.write_bytes

    @property
    def copy_bytes(self) -> int:
        return (self.algorithmic_bytes // 2) & ~15

    @property
    def cache_bytes(self) -> int:
        return self.num_slots * self.heads * (self.norm_dim + self.rope_dim) * self.elem_size


KV_WORKLOADS: Dict[str, KvWorkload] = {
    w.name: w
    for w in [
        KvWorkload("bf16_kv_prefill_4x4096_576", "bf16", 4, 4096, 4096, 1, 512, 64, 1e-6, 1, False,
                   note="prefill: 4 sequences x 4096 new tokens, MLA-style 512 + 64 split"),
        KvWorkload("bf16_kv_decode_256_576", "bf16", 256, 1, 4096, 1, 512, 64, 1e-6, 1, True,
                   note="decode: 256 sequences, one new token each at a random length"),
    ]
}


def rope_tables(max_pos: int, rope_dim: int, theta: float = 10000.0):
    """cos / sin tables [max_pos, rope_dim / 2], float32."""
    i = np.arange(rope_dim // 2, dtype=np.float64)
    freq = theta ** (-2.0 * i / rope_dim)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * freq[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def make_kv(w: KvWorkload, seed: int = 0) -> Dict[str, torch.Tensor]:
    """CPU tensors for one call: kv, gamma, cos, sin, positions (int32), slots
    (int64), block_table (int32) and cache_seqlens (int32).  The caches come
    from kv_caches()."""
    rng = np.random.default_rng(seed)
    d = w.norm_dim + w.rope_dim
    kv = _draw(rng, N01, (w.tokens, w.heads * d))
    gamma = _draw(rng, W_N, (w.norm_dim,))
    perm = rng.permutation(w.num_blocks)
    table = perm[: w.seqs * w.blocks_per_seq].reshape(w.seqs, w.blocks_per_seq).astype(np.int32)
    if w.decode:
        lens = rng.integers(1, w.max_len + 1, size=w.seqs).astype(np.int32)
        pos = (lens - 1).astype(np.int64)[:, None]
    else:
        lens = np.full(w.seqs, w.new_tokens, dtype=np.int32)
        pos = np.tile(np.arange(w.new_tokens, dtype=np.int64), (w.seqs, 1))
    seq = np.repeat(np.arange(w.seqs), w.new_tokens).reshape(w.seqs, w.new_tokens)
    slots = table[seq, pos // w.block_size].astype(np.int64) * w.block_size + pos % w.block_size
    cos_t, sin_t = rope_tables(w.max_pos, w.rope_dim, w.theta)
    return {
        "kv": _store(kv, w.dtype).reshape(w.tokens, w.heads, d),
        "gamma": _store(gamma, w.dtype),
        "cos": torch.from_numpy(cos_t), "sin": torch.from_numpy(sin_t),
        "positions": torch.from_numpy(pos.reshape(-1).astype(np.int32)),
        "slots": torch.from_numpy(slots.reshape(-1)),
        "block_table": torch.from_numpy(table), "cache_seqlens": torch.from_numpy(lens),
    }


def cache_pattern(rows: int, heads: int, dim: int, dtype: str, device="cpu", salt: int = 0) -> torch.Tensor:
    """Initial cache contents [rows, heads, dim]: a fixed pattern of small
    multiples of 1/64 (exact in bf16), so that untouched rows can be checked."""
    i = torch.arange(rows * heads * dim, device=device, dtype=torch.int64)
    v = (((i * 7 + salt) % 251) - 125).to(torch.float32) / 64.0
    return v.to(torch.float32 if dtype == "f32" else torch.bfloat16).reshape(rows, heads, dim)


def kv_caches(w: KvWorkload, device="cpu"):
    """(norm_cache, rope_cache) with their initial pattern."""
    return (cache_pattern(w.num_slots, w.heads, w.norm_dim, w.dtype, device, 1),
            cache_pattern(w.num_slots, w.heads, w.rope_dim, w.dtype, device, 2))


# Every workload bench.py can time, by name.
EVERY_WORKLOAD = dict(ALL_WORKLOADS, **KV_WORKLOADS)

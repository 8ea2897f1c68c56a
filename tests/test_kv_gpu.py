"""Parity of the HIP KV RMSNorm + RoPE + cache scatter (through the C ABI) with
the CPU oracle.

Normalised rows: bf16 within 1 ulp, fp32 within 1e-5 relative (the RMSNorm
bounds of tests/parity.py).  Rotated rows: |gpu - oracle| <= 4u*(|a*cos| +
|b*sin|) + 1 ulp per output (two fp32 products and a sum or difference, which
can cancel).  Every cache row that no valid token names must keep its initial
pattern.  Covered: the stated prefill and decode workloads at full size, both
pairings, both dtypes, vector and element kernels (widths that are not
multiples of the vector, misaligned buffers, rotated parts wider than 64
lanes), several heads, padding and out-of-range tokens, determinism and graph
replays.
"""
import sys

import numpy as np
import pytest
import torch

import memory_bound_rmsnorm_amd as mbr
import oracle
from memory_bound_rmsnorm_amd import inputs
from tests import parity

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bits(t):
    return inputs.bits(t.reshape(-1)).reshape(tuple(t.shape))


def run_gpu(t, nc, rc, eps, style, cfg=None):
    d = {k: v.cuda() for k, v in t.items() if k in ("kv", "gamma", "cos", "sin", "positions", "slots")}
    mbr.kv_rmsnorm_rope_cache_ex(d["kv"], d["gamma"], d["cos"], d["sin"], d["positions"], d["slots"], nc, rc, eps,
                                 style, cfg)
    torch.cuda.synchronize()


def check(t, eps, style, dtype, nc0, rc0, nc, rc, sample_untouched=None):
    """Compare the GPU caches nc, rc (device, after the call) with the oracle on
    the rows the call names, and the other rows with their initial contents
    nc0, rc0 (device)."""
    tokens, heads, d = t["kv"].shape
    dn = nc.shape[2]
    dr = d - dn
    num_slots = nc.shape[0]
    pos = t["positions"].numpy()
    sl = t["slots"].numpy()
    valid = (sl >= 0) & (sl < num_slots) & (pos >= 0) & (pos < t["cos"].shape[0])
    vt = np.flatnonzero(valid)
    # the oracle on compact caches: token k of the valid set writes row k
    compact = np.full(tokens, -1, np.int64)
    compact[vt] = np.arange(len(vt))
    kvb = bits(t["kv"])
    # the oracle's unrounded caches (float64); the rounded ones are its rounding of them
    onc = np.zeros((len(vt), heads, dn), np.float64)
    orc = np.zeros((len(vt), heads, dr), np.float64)
    oracle.kv_rmsnorm_rope_cache(kvb, bits(t["gamma"]), t["cos"].numpy(), t["sin"].numpy(), pos, compact, onc, orc,
                                 eps, style)
    rnd = oracle.round_bf16_array if dtype == "bf16" else oracle.round_f32_array
    rows = torch.from_numpy(sl[vt]).cuda()
    gnc = bits(nc[rows].cpu())
    grc = bits(rc[rows].cpu()) if dr else None
    # longest fp32 chain of a norm row: at most 64 terms per lane on the vector
    # paths (8 vectors of a 64-lane row, 2 of an 8-lane group), ceil(Dn/64) on
    # the element path, plus 6 wave levels and one slot add
    L = max(64, -(-dn // 64)) + 7
    stats = {"tokens_written": int(len(vt)),
             "norm": parity.compare(gnc.reshape(-1, dn), rnd(onc).reshape(-1, dn), onc.reshape(-1, dn),
                                    (L + 12) * U)}
    if dr:
        half = dr // 2
        x = parity._values(kvb[vt][:, :, dn:])
        c = t["cos"].numpy()[pos[vt]].astype(np.float64)[:, None, :]
        s = t["sin"].numpy()[pos[vt]].astype(np.float64)[:, None, :]
        ia = np.arange(half) * 2 if style == mbr.ROPE_PAIRS else np.arange(half)
        ib = ia + 1 if style == mbr.ROPE_PAIRS else ia + half
        mag = np.empty_like(x)
        mag[:, :, ia] = np.abs(x[:, :, ia] * c) + np.abs(x[:, :, ib] * s)
        mag[:, :, ib] = np.abs(x[:, :, ia] * s) + np.abs(x[:, :, ib] * c)
        parity.check_magnitude(grc, orc, mag, 4 * U, "rope", stats, 2)
    # untouched rows keep their initial contents
    mask = torch.ones(num_slots, dtype=torch.bool, device=nc.device)
    mask[rows] = False
    if sample_untouched is not None:
        keep = torch.zeros_like(mask)
        idx = torch.randint(0, num_slots, (sample_untouched,), device=nc.device)
        keep[idx] = True
        near = torch.cat([rows - 1, rows + 1]).clamp(0, num_slots - 1)
        keep[near] = True
        mask &= keep
    assert torch.equal(nc[mask], nc0[mask]), "a norm-cache row outside the named slots changed"
    if dr:
        assert torch.equal(rc[mask], rc0[mask]), "a rope-cache row outside the named slots changed"
    return stats


@pytest.mark.parametrize("name", list(inputs.KV_WORKLOADS))
def test_kv_workloads_full_size(name):
    w = inputs.KV_WORKLOADS[name]
    t = inputs.make_kv(w, seed=0)
    nc0, rc0 = inputs.kv_caches(w, "cuda")
    nc, rc = nc0.clone(), rc0.clone()
    say("kv workload", name, "tokens", w.tokens, "slots", w.num_slots)
    run_gpu(t, nc, rc, w.eps, w.rope_style)
    say(name, check(t, w.eps, w.rope_style, w.dtype, nc0, rc0, nc, rc,
                    sample_untouched=None if w.num_slots <= 1 << 16 else 1 << 16))


def _custom(dtype, tokens, heads, dn, dr, slots, max_pos, seed, style):
    w = inputs.KvWorkload("custom", dtype, 1, tokens, max_pos, heads, dn, dr, 1e-5, style, False)
    rng = np.random.default_rng(seed)
    kv = rng.standard_normal((tokens, heads, dn + dr)).astype(np.float32)
    g = (rng.standard_normal(dn) * 0.1 + 1).astype(np.float32)
    td = torch.float32 if dtype == "f32" else torch.bfloat16
    cos_t, sin_t = inputs.rope_tables(max_pos, dr)
    t = {"kv": torch.from_numpy(kv).to(td), "gamma": torch.from_numpy(g).to(td),
         "cos": torch.from_numpy(cos_t), "sin": torch.from_numpy(sin_t),
         "positions": torch.from_numpy(rng.integers(0, max_pos, tokens).astype(np.int32)),
         "slots": torch.from_numpy(rng.permutation(slots)[:tokens].astype(np.int64))}
    nc0 = inputs.cache_pattern(slots, heads, dn, dtype, "cuda", 1)
    rc0 = inputs.cache_pattern(slots, heads, dr, dtype, "cuda", 2)
    return w, t, nc0, rc0


SHAPES = [  # (dn, dr, heads): vector path, masked vector path, element fallbacks
    (512, 64, 1), (128, 64, 2), (8, 16, 3), (520, 32, 1), (1024, 128, 4), (2056, 64, 1), (4096, 512, 1),
    (4104, 64, 1), (512, 520, 1), (100, 30, 2), (64, 12, 1), (48, 24, 2), (512, 0, 1), (7, 2, 5),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("style", [mbr.ROPE_HALVES, mbr.ROPE_PAIRS])
@pytest.mark.parametrize("dn,dr,heads", SHAPES)
def test_kv_shapes(dn, dr, heads, style, dtype):
    w, t, nc0, rc0 = _custom(dtype, 37, heads, dn, dr, 101, 4096, dn + dr + heads, style)
    nc, rc = nc0.clone(), rc0.clone()
    say("kv shape", dtype, style, dn, dr, heads)
    run_gpu(t, nc, rc, 1e-5, style)
    check(t, 1e-5, style, dtype, nc0, rc0, nc, rc)


KV_CONFIGS = [(0, 1), (0, 2), (0, 4), (0, 8), (8, 1), (8, 2), (16, 1), (16, 2), (32, 1),
              (32, 2)]  # (lanes per row, vectors per lane)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("style", [mbr.ROPE_HALVES, mbr.ROPE_PAIRS])
@pytest.mark.parametrize("lpr,nvpl", KV_CONFIGS)
def test_kv_every_vector_config(lpr, nvpl, style, dtype):
    """Every built vector configuration, forced: full and masked norm parts,
    a rotated part filling the row's lanes or a few of them, none at all;
    rows that leave part of the last wave idle, several heads, and padding,
    out-of-range slots and positions among the tokens."""
    v = 8 if dtype == "bf16" else 4
    lanes = lpr or 64
    unit = v if style == mbr.ROPE_PAIRS else 2 * v
    n = 0
    for nv in sorted({lanes * nvpl, max(1, lanes * (nvpl - 1) + 3)}):
        for dr in sorted({0, unit, min(lanes, 16) * unit}):
            for tokens, heads in ((1, 1), (37, 2), (9, 3)):
                w, t, nc0, rc0 = _custom(dtype, tokens, heads, nv * v, dr, 101, 512, 100 * n + tokens, style)
                if tokens > 4:
                    t["slots"][1] = -1
                    t["slots"][3] = 101
                    t["positions"][2] = 512
                cfg = mbr.Config(mbr.PATH_VECTOR, 1, nvpl, 1, 0, lpr)
                nc, rc = nc0.clone(), rc0.clone()
                say("kv config", dtype, style, cfg.as_dict(), "dn", nv * v, "dr", dr, "tokens", tokens, "heads", heads)
                run_gpu(t, nc, rc, 1e-5, style, cfg)
                check(t, 1e-5, style, dtype, nc0, rc0, nc, rc)
                n += 1
    assert n >= 9


def test_kv_padding_and_out_of_range_tokens_write_nothing():
    w, t, nc0, rc0 = _custom("bf16", 40, 2, 512, 64, 64, 128, 3, mbr.ROPE_PAIRS)
    t["slots"][[1, 5]] = -1
    t["slots"][7] = 64            # == num_slots
    t["slots"][9] = 1 << 40
    t["positions"][[11, 12]] = torch.tensor([128, -1], dtype=torch.int32)
    nc, rc = nc0.clone(), rc0.clone()
    run_gpu(t, nc, rc, 1e-5, mbr.ROPE_PAIRS)
    st = check(t, 1e-5, mbr.ROPE_PAIRS, "bf16", nc0, rc0, nc, rc)
    assert st["tokens_written"] == 34


def test_kv_misaligned_buffers_take_the_element_kernel():
    w, t, nc0, rc0 = _custom("bf16", 20, 1, 512, 64, 50, 256, 4, mbr.ROPE_HALVES)
    kvbuf = torch.zeros(20 * 576 + 8, dtype=torch.bfloat16, device="cuda")
    kvbuf[1:1 + 20 * 576] = t["kv"].reshape(-1).cuda()
    kv = kvbuf[1:1 + 20 * 576].view(20, 1, 576)
    assert kv.data_ptr() % 16 != 0
    nc, rc = nc0.clone(), rc0.clone()
    d = {k: t[k].cuda() for k in ("gamma", "cos", "sin", "positions", "slots")}
    mbr.kv_rmsnorm_rope_cache(kv, d["gamma"], d["cos"], d["sin"], d["positions"], d["slots"], nc, rc, 1e-5,
                              mbr.ROPE_HALVES)
    torch.cuda.synchronize()
    check(t, 1e-5, mbr.ROPE_HALVES, "bf16", nc0, rc0, nc, rc)


def test_kv_deterministic_and_graph_replays():
    w = inputs.KV_WORKLOADS["bf16_kv_prefill_4x4096_576"]
    t = inputs.make_kv(w, seed=1)
    d = {k: v.cuda() for k, v in t.items()}
    nc0, rc0 = inputs.kv_caches(w, "cuda")
    a = (nc0.clone(), rc0.clone())
    mbr.kv_rmsnorm_rope_cache(d["kv"], d["gamma"], d["cos"], d["sin"], d["positions"], d["slots"], *a, w.eps,
                              w.rope_style)
    torch.cuda.synchronize()
    b = (nc0.clone(), rc0.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mbr.kv_rmsnorm_rope_cache(d["kv"], d["gamma"], d["cos"], d["sin"], d["positions"], d["slots"], *b, w.eps,
                                  w.rope_style)
    for rep in range(3):
        b[0].copy_(nc0)
        b[1].copy_(rc0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]), rep


def test_kv_overlap_rejected_on_device_buffers():
    w, t, nc0, rc0 = _custom("bf16", 4, 1, 64, 16, 8, 16, 5, mbr.ROPE_PAIRS)
    d = {k: v.cuda() for k, v in t.items()}
    L, s = mbr.lib(), torch.cuda.current_stream().cuda_stream
    args = [d["kv"].data_ptr(), d["gamma"].data_ptr(), d["cos"].data_ptr(), d["sin"].data_ptr(),
            d["positions"].data_ptr(), d["slots"].data_ptr(), nc0.data_ptr(), rc0.data_ptr(), 4, 1, 64, 16, 16, 8,
            1e-5, 1, 1, s]
    INV = mbr.RMSNORM_ERR_INVALID_ARG
    for i, bad in ((6, d["kv"].data_ptr()), (7, nc0.data_ptr() + 64), (6, d["cos"].data_ptr()),
                   (7, d["slots"].data_ptr())):
        a = list(args)
        a[i] = bad
        assert L.kv_rmsnorm_rope_cache(*a) == INV, i


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_kv_non_finite_values(dtype):
    """A NaN in a token's norm part makes that token's normalised row NaN and
    leaves its rotated part alone; an Inf in the rotated part propagates through
    the rotation of its own pair only."""
    w, t, nc0, rc0 = _custom(dtype, 16, 2, 512, 64, 40, 256, 6, mbr.ROPE_PAIRS)
    t["kv"][3, 1, 10] = float("nan")
    t["kv"][7, 0, 512 + 5] = float("inf")
    nc, rc = nc0.clone(), rc0.clone()
    run_gpu(t, nc, rc, 1e-5, mbr.ROPE_PAIRS)
    check(t, 1e-5, mbr.ROPE_PAIRS, dtype, nc0, rc0, nc, rc)

"""Parity of the HIP path (through the C ABI) with the CPU oracle, on the GPU.

Every test compares element by element on seeded inputs: bf16 within 1 ulp,
fp32 within 1e-5 relative, the fused residual sum h bitwise, and every output a
nearest-even rounding of a value within the launch configuration's fp32
evaluation bound of the oracle's unrounded result (tests/parity.py).
Covered: the five stated workloads at full size in the automatically chosen
launch configuration (the one bench.py times), every built kernel
configuration on shapes that span several workgroups and a partial last one,
ragged widths, odd row counts, misaligned and aliased buffers, the two-pass
fallback, the in-kernel row loop, determinism and degenerate rows.
"""
import ctypes
import os
import sys

import numpy as np
import pytest
import torch

import memory_bound_rmsnorm_amd as mbr
from memory_bound_rmsnorm_amd import inputs
from tests import parity
from tests import built

pytestmark = pytest.mark.gpu

BF16, F32 = torch.bfloat16, torch.float32


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def tdtype(w):
    return F32 if w.dtype == "f32" else BF16


def run_plain(x, w, eps, cfg=None, out=None):
    out = torch.empty_like(x) if out is None else out
    mbr.rmsnorm_fwd_ex(x, w, out, eps, cfg)
    torch.cuda.synchronize()
    return out


def run_fused(x, r, w, eps, cfg=None, h=None, out=None):
    h = torch.empty_like(x) if h is None else h
    out = torch.empty_like(x) if out is None else out
    mbr.rmsnorm_residual_fwd_ex(x, r, w, h, out, eps, cfg)
    torch.cuda.synchronize()
    return h, out


def auto(rows, hidden, td, aligned=True, fused=False):
    return mbr.rmsnorm_select_config(rows, hidden, td, aligned, fused)


def expect(xb, wb, eps, cfg, res=None):
    """(h, y, y unrounded, gamma): the oracle's residual sum (None without a
    residual), its rounded and unrounded output, and the relative fp32
    evaluation bound of the launch configuration cfg."""
    gamma = parity.fwd_gamma(cfg, xb.shape[1], xb.dtype == np.uint16)
    if res is None:
        want, e = parity.oracle_fwd(xb, wb, eps, unrounded=True)
        return None, want, e, gamma
    h, want, e = parity.oracle_residual(xb, res, wb, eps, unrounded=True)
    return h, want, e, gamma


def check_workload(w, t, cfg=None, eps=None):
    """Run workload tensors t (CPU) on the GPU and compare with the oracle."""
    eps = w.eps if eps is None else eps
    eff = cfg if cfg is not None else auto(w.rows, w.hidden, tdtype(w), True, w.fused)
    dev = {k: v.cuda() for k, v in t.items()}
    xb, wb = inputs.bits(t["x"]), inputs.bits(t["weight"])
    if w.fused:
        h, y = run_fused(dev["x"], dev["residual"], dev["weight"], eps, cfg)
        h_want, y_want, e, gamma = expect(xb, wb, eps, eff, inputs.bits(t["residual"]))
        assert np.array_equal(inputs.bits(h), h_want), "residual sum differs"
        return parity.compare(inputs.bits(y), y_want, e, gamma)
    y = run_plain(dev["x"], dev["weight"], eps, cfg)
    _, y_want, e, gamma = expect(xb, wb, eps, eff)
    return parity.compare(inputs.bits(y), y_want, e, gamma)


# ---------------------------------------------------------------- stated workloads


@pytest.mark.parametrize("name", list(inputs.WORKLOADS))
def test_stated_workloads_full_size(name):
    w = inputs.WORKLOADS[name]
    say("workload", name, "seed 0", "config", mbr.rmsnorm_select_config(w.rows, w.hidden, tdtype(w), True, w.fused))
    stats = check_workload(w, inputs.make(w, seed=0))
    say(name, stats)


@pytest.mark.parametrize("name", list(inputs.SHAPE_WORKLOADS))
def test_shape_workloads_full_size(name):
    """The narrow-row and odd-width shapes bench.py also times."""
    w = inputs.SHAPE_WORKLOADS[name]
    say("workload", name, "seed 0", "config", mbr.rmsnorm_select_config(w.rows, w.hidden, tdtype(w), True, w.fused))
    stats = check_workload(w, inputs.make(w, seed=0))
    say(name, stats)


@pytest.mark.parametrize("name", ["bf16_prefill_4096x2048", "bf16_residual_12289x5120"])
@pytest.mark.parametrize("seed", [1, 2])
def test_stated_workloads_other_seeds(name, seed):
    w = inputs.WORKLOADS[name]
    say("workload", name, "seed", seed)
    check_workload(w, inputs.make(w, seed=seed))


# ---------------------------------------------------------------- shapes


RAGGED = [(1, 1), (3, 3), (5, 7), (2, 8), (5, 9), (67, 127), (12, 769), (5, 2048), (3, 4095), (7, 5120),
          (5, 5121), (3, 8193), (9, 16384), (2, 20000), (3, 65536), (2, 81920), (2, 131080)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("rows,hidden", RAGGED)
def test_ragged_shapes(rows, hidden, dtype, fused):
    w = inputs.custom(rows, hidden, dtype, fused)
    cfg = mbr.rmsnorm_select_config(rows, hidden, BF16 if dtype == "bf16" else F32, True, fused)
    say("shape", rows, hidden, dtype, "fused" if fused else "plain", cfg)
    check_workload(w, inputs.make(w, seed=rows * 7 + hidden))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("fused", [False, True])
def test_odd_row_counts(dtype, fused):
    for rows in (1, 2, 3, 5, 12289):
        w = inputs.custom(rows, 2048, dtype, fused)
        say("rows", rows, dtype, fused)
        check_workload(w, inputs.make(w, seed=rows))


@pytest.mark.parametrize("subwave", [False, True])
def test_many_rows_in_kernel_loop(subwave):
    """More row groups than the largest grid (2^20 workgroups): workgroups loop
    over rows, with a whole wave per row and with 8 rows per wave."""
    if subwave:
        rows = (1 << 20) * 8 + 3
        cfg = mbr.rmsnorm_select_config(rows, 8, BF16)
        assert cfg.lanes_per_row == 8
    else:
        rows = (1 << 20) * 4 + 3
        cfg = mbr.Config(mbr.PATH_VECTOR, 1, 1, 1, 0)
    assert (rows + cfg.rows_per_block - 1) // cfg.rows_per_block > (1 << 20)
    w = inputs.custom(rows, 8, "bf16", False)
    say("many rows", rows, cfg)
    check_workload(w, inputs.make(w, seed=5), cfg)


# ---------------------------------------------------------------- every built configuration


def _configs(path, dtype, fused):
    vec = path == mbr.PATH_VECTOR
    for wpr in built.WPR:
        for per in (built.VEC_VPL if vec else built.EPL):
            if built.vec(wpr, per, fused) if vec else built.elem(wpr, per):
                yield wpr, per


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("fused", [False, True])
def test_every_vector_config(dtype, fused):
    vecw = 8 if dtype == "bf16" else 4
    n = 0
    for wpr, vpl in _configs(mbr.PATH_VECTOR, dtype, fused):
        lanes = 64 * wpr
        max_rpb = (1024 if wpr == 16 else 512) // lanes
        for nvec in sorted({lanes * vpl, max(1, lanes * vpl - 37), lanes * (vpl - 1) + 1}):
            for rpb in sorted({1, max_rpb}):
                # three row groups, the last one partial; with max_blocks 2 one
                # workgroup walks two groups (next-row prefetch path)
                rows = 2 * rpb + 1
                for mb in (0, 2):
                    cfg = mbr.Config(mbr.PATH_VECTOR, wpr, vpl, rpb, mb)
                    w = inputs.custom(rows, nvec * vecw, dtype, fused)
                    say("vector", dtype, fused, cfg, "hidden", nvec * vecw, "rows", rows)
                    check_workload(w, inputs.make(w, seed=n), cfg)
                    n += 1
    assert n > 100


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("fused", [False, True])
def test_every_element_config(dtype, fused):
    n = 0
    for wpr, epl in _configs(mbr.PATH_ELEMENT, dtype, fused):
        lanes = 64 * wpr
        max_rpb = (1024 if wpr == 16 else 512) // lanes
        # the one built element configuration: below one vector (as chosen)
        # and up to the whole wave it covers
        for hidden in (1, 2, 3, 5, 7, 33, 59, 64):
            rpb = max_rpb if n % 2 else 1
            rows = 2 * rpb + 1
            cfg = mbr.Config(mbr.PATH_ELEMENT, wpr, epl, rpb, 0)
            w = inputs.custom(rows, hidden, dtype, fused)
            say("element", dtype, fused, cfg, "hidden", hidden, "rows", rows)
            check_workload(w, inputs.make(w, seed=n), cfg)
            n += 1
    assert n == 8


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("fused", [False, True])
def test_every_two_pass_config(dtype, fused):
    for wpr in (1, 2, 4, 8, 16):
        for hidden in (4096, 4099, 12288 + 8):
            cfg = mbr.Config(mbr.PATH_TWO_PASS, wpr, 0, 1, 0)
            w = inputs.custom(5, hidden, dtype, fused)
            say("two-pass", dtype, fused, cfg, "hidden", hidden)
            check_workload(w, inputs.make(w, seed=wpr + hidden), cfg)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("fused", [False, True])
def test_weight_in_lds_matches_bitwise(dtype, fused):
    """weight_lds = 1 (the workgroup stages the weight in LDS once) on every
    built vector configuration, with one and with the most row slots, full and
    masked rows, and a capped grid whose workgroups walk several row groups:
    bitwise equal to the same configuration reading the weight from global
    memory, and within the oracle's bound."""
    vecw = 8 if dtype == "bf16" else 4
    n = 0
    for wpr, vpl in _configs(mbr.PATH_VECTOR, dtype, fused):
        lanes = 64 * wpr
        max_rpb = (1024 if wpr == 16 else 512) // lanes
        for nvec in sorted({lanes * vpl, max(1, lanes * vpl - 37)}):
            if nvec * 16 > 159 * 1024:
                continue
            for rpb, mb in sorted({(1, 0), (max_rpb, 0), (max_rpb, 2)}):
                rows = 2 * rpb + 1
                w = inputs.custom(rows, nvec * vecw, dtype, fused)
                t = inputs.make(w, seed=500 + n)
                dev = {k: v.cuda() for k, v in t.items()}
                on = mbr.Config(mbr.PATH_VECTOR, wpr, vpl, rpb, mb, 0, 1)
                off = mbr.Config(mbr.PATH_VECTOR, wpr, vpl, rpb, mb, 0, 0)
                say("weight in LDS", dtype, fused, on, "hidden", nvec * vecw, "rows", rows)
                if fused:
                    a = run_fused(dev["x"], dev["residual"], dev["weight"], w.eps, on)
                    b = run_fused(dev["x"], dev["residual"], dev["weight"], w.eps, off)
                    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
                else:
                    assert torch.equal(run_plain(dev["x"], dev["weight"], w.eps, on),
                                       run_plain(dev["x"], dev["weight"], w.eps, off))
                if n % 4 == 0:
                    check_workload(w, t, on)
                n += 1
    assert n > 60


@pytest.mark.parametrize("fused", [False, True])
def test_persistent_grid_matches_bitwise(fused):
    """Capping the grid (workgroups loop over row groups) changes nothing."""
    w = inputs.custom(1000, 4096, "bf16", fused)
    t = {k: v.cuda() for k, v in inputs.make(w, seed=3).items()}
    base = mbr.rmsnorm_select_config(1000, 4096, BF16, True, fused)
    capped = mbr.Config(base.path, base.waves_per_row, base.items_per_lane, base.rows_per_block, 37)
    if fused:
        a = run_fused(t["x"], t["residual"], t["weight"], 1e-5, base)
        b = run_fused(t["x"], t["residual"], t["weight"], 1e-5, capped)
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    else:
        assert torch.equal(run_plain(t["x"], t["weight"], 1e-5, base), run_plain(t["x"], t["weight"], 1e-5, capped))
    check_workload(w, inputs.make(w, seed=3), capped)


# ---------------------------------------------------------------- rows wider than the registers


STAGED_WIDTHS = [81928, 98304, 131072, 131080, 163328]


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("hidden", STAGED_WIDTHS)
def test_staged_rows_automatic(hidden, fused):
    """bf16 rows past the register budget: part in VGPRs, the rest in LDS, read
    once (fused rows past what registers plus LDS hold take two passes)."""
    rows = 37
    cfg = auto(rows, hidden, BF16, True, fused)
    say("staged", hidden, "fused" if fused else "plain", cfg)
    if not fused or hidden <= 138752:
        assert cfg.path == mbr.PATH_VECTOR_LDS
    check_workload(inputs.custom(rows, hidden, "bf16", fused), inputs.make(inputs.custom(rows, hidden, "bf16", fused),
                                                                            seed=hidden + fused))


def _staged_cases(dtype, fused):
    """(items_per_lane, staged vectors) for every built register + LDS kernel:
    one staged vector, a partial last slot, whole slots, and the LDS limit."""
    v = 8 if dtype == "bf16" else 4
    top = (160 * 1024 - 1024) // 16
    for rv in ((6, 7) if fused else (10,)):
        for staged in sorted({1, 1023, 1024, 1025, 5000, top - 1, top}):
            yield rv, (1024 * rv + staged) * v


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("fused", [False, True])
def test_every_staged_config(dtype, fused):
    """Forced register + LDS configurations at every staged-part shape, with a
    capped grid whose workgroups walk several rows (the LDS slots reused)."""
    n = 0
    for rv, hidden in _staged_cases(dtype, fused):
        for mb in (0, 2):
            rows = 5
            cfg = mbr.Config(mbr.PATH_VECTOR_LDS, 16, rv, 1, mb)
            w = inputs.custom(rows, hidden, dtype, fused)
            say("staged config", dtype, fused, cfg, "hidden", hidden)
            check_workload(w, inputs.make(w, seed=900 + n), cfg)
            n += 1
    assert n >= 14


def test_staged_in_place_and_rejections():
    """out == x and h == residual on the register + LDS path; configurations
    that would leave nothing for LDS, overflow it, or lack alignment are
    refused before launch."""
    rows, hidden = 9, 131072
    w = inputs.custom(rows, hidden, "bf16", True)
    t = inputs.make(w, seed=77)
    cfg = auto(rows, hidden, BF16, True, True)
    h_want, y_want, e, gamma = expect(inputs.bits(t["x"]), inputs.bits(t["weight"]), w.eps, cfg,
                                      inputs.bits(t["residual"]))
    x, r, wt = t["x"].cuda(), t["residual"].cuda(), t["weight"].cuda()
    run_fused(x, r, wt, w.eps, h=r, out=x)
    assert np.array_equal(inputs.bits(r), h_want)
    parity.compare(inputs.bits(x), y_want, e, gamma)
    x = torch.zeros(2, 81920, dtype=BF16, device="cuda")
    wt = torch.ones(81920, dtype=BF16, device="cuda")
    out = torch.empty_like(x)
    L, s = mbr.lib(), torch.cuda.current_stream().cuda_stream
    INV = mbr.RMSNORM_ERR_INVALID_ARG
    for c in (mbr.Config(mbr.PATH_VECTOR_LDS, 16, 10, 1, 0),     # nothing left for LDS
              mbr.Config(mbr.PATH_VECTOR_LDS, 16, 8, 1, 0),      # not built
              mbr.Config(mbr.PATH_VECTOR_LDS, 8, 10, 1, 0),      # 16 waves per row only
              mbr.Config(mbr.PATH_VECTOR_LDS, 16, 10, 2, 0)):    # one row per workgroup
        assert L.rmsnorm_fwd_ex(x.data_ptr(), wt.data_ptr(), out.data_ptr(), 2, 81920, 1e-5, 1, ctypes.byref(c),
                                s) == INV
    big = torch.zeros(1, 163336, dtype=BF16, device="cuda")
    wb = torch.ones(163336, dtype=BF16, device="cuda")
    ob = torch.empty_like(big)
    c = mbr.Config(mbr.PATH_VECTOR_LDS, 16, 10, 1, 0)  # one vector past the LDS limit
    assert L.rmsnorm_fwd_ex(big.data_ptr(), wb.data_ptr(), ob.data_ptr(), 1, 163336, 1e-5, 1, ctypes.byref(c),
                            s) == INV
    assert L.rmsnorm_fwd_ex(big.data_ptr() + 2, wb.data_ptr(), ob.data_ptr(), 1, 163328, 1e-5, 1, ctypes.byref(c),
                            s) == INV  # not 16-byte aligned
    torch.cuda.synchronize()


# ---------------------------------------------------------------- pointers


def _raw_plain(xp, wp, op, rows, hidden, eps, dt):
    st = mbr.lib().rmsnorm_fwd(xp, wp, op, rows, hidden, eps, dt, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return st


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("which", ["x", "weight", "out"])
def test_misaligned_pointers(dtype, which):
    """Element-aligned but not 16-byte-aligned buffers take the any-alignment
    vector path (full vectors at the buffer's own alignment)."""
    rows, hidden, eps = 33, 2048, 1e-5
    w = inputs.custom(rows, hidden, dtype, False)
    t = inputs.make(w, seed=11)
    td = BF16 if dtype == "bf16" else F32
    es = 2 if dtype == "bf16" else 4
    pad = 8
    xbuf = torch.zeros(rows * hidden + pad, dtype=td, device="cuda")
    wbuf = torch.zeros(hidden + pad, dtype=td, device="cuda")
    obuf = torch.zeros(rows * hidden + pad, dtype=td, device="cuda")
    off = {k: (1 if k == which else 0) for k in ("x", "weight", "out")}
    xbuf[off["x"]:off["x"] + rows * hidden] = t["x"].reshape(-1).cuda()
    wbuf[off["weight"]:off["weight"] + hidden] = t["weight"].cuda()
    st = _raw_plain(xbuf.data_ptr() + es * off["x"], wbuf.data_ptr() + es * off["weight"],
                    obuf.data_ptr() + es * off["out"], rows, hidden, eps, mbr.dtype_code(td))
    assert st == mbr.RMSNORM_OK
    got = inputs.bits(obuf[off["out"]:off["out"] + rows * hidden].reshape(rows, hidden).cpu())
    _, want, e, gamma = expect(inputs.bits(t["x"]), inputs.bits(t["weight"]), eps, auto(rows, hidden, td, False))
    parity.compare(got, want, e, gamma)
    # nothing outside the output was written
    assert torch.count_nonzero(obuf[:off["out"]]) == 0
    assert torch.count_nonzero(obuf[off["out"] + rows * hidden:]) == 0


def _run_any(dtype, rows, hidden, fused, cfg, off, seed):
    """Forced configuration on buffers that start `off` elements past a
    16-byte boundary, inside guard space: parity with the oracle, and no byte
    outside the outputs written."""
    w = inputs.custom(rows, hidden, dtype, fused)
    t = inputs.make(w, seed=seed)
    td = BF16 if dtype == "bf16" else F32
    es = 2 if dtype == "bf16" else 4
    n = rows * hidden
    g = 64  # guard elements around every region
    bases = [g + off + i * (n + 2 * g) for i in range(4)]  # x, residual, h, out
    # guard space holds a non-zero pattern, so that a stray write of a zero
    # (the value the shifted frame's slot before a row computes to) shows
    buf = torch.full((4 * (n + 2 * g) + 2 * g,), 1.0, dtype=td, device="cuda")
    buf[bases[0]:bases[0] + n] = t["x"].reshape(-1).cuda()
    if fused:
        buf[bases[1]:bases[1] + n] = t["residual"].reshape(-1).cuda()
    wt = t["weight"].cuda()
    p = buf.data_ptr()
    ptr = [p + es * b for b in bases]
    L = mbr.lib()
    stream = torch.cuda.current_stream().cuda_stream
    code = mbr.dtype_code(td)
    if fused:
        st = L.rmsnorm_residual_fwd_ex(ptr[0], ptr[1], wt.data_ptr(), ptr[2], ptr[3], rows, hidden, w.eps, code,
                                       ctypes.byref(cfg), stream)
    else:
        st = L.rmsnorm_fwd_ex(ptr[0], wt.data_ptr(), ptr[3], rows, hidden, w.eps, code, ctypes.byref(cfg), stream)
    torch.cuda.synchronize()
    assert st == mbr.RMSNORM_OK, mbr.rmsnorm_status_string(st)
    cpu = inputs.bits(buf.cpu())
    xb, wb = inputs.bits(t["x"]), inputs.bits(t["weight"])
    h_want, y_want, e, gamma = expect(xb, wb, w.eps, cfg, inputs.bits(t["residual"]) if fused else None)
    if fused:
        assert np.array_equal(cpu[bases[2]:bases[2] + n].reshape(rows, hidden), h_want), "residual sum differs"
    parity.compare(cpu[bases[3]:bases[3] + n].reshape(rows, hidden), y_want, e, gamma)
    written = np.zeros(cpu.shape, bool)
    for i in (0, 1, 2, 3) if fused else (0, 3):
        written[bases[i]:bases[i] + n] = True
    assert np.all(cpu[~written] == inputs.bits(torch.ones(1, dtype=td))[0]), "a byte outside the buffers changed"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("fused", [False, True])
def test_every_any_alignment_config(dtype, fused):
    """Every built any-alignment vector configuration, forced: full and
    masked vector sets, tails of 0, 1 and V - 1 elements, rows starting 0, 1
    and V - 1 elements past a 16-byte boundary."""
    v = 8 if dtype == "bf16" else 4
    n = 0
    for wpr in built.WPR:
        for vpl in built.ANY_VPL:
            if not built.any_(wpr, vpl, fused):
                continue
            lanes = 64 * wpr
            for nvec in sorted({lanes * vpl, max(1, lanes * (vpl - 1) + 3)}):
                tail = (0, 1, v - 1)[n % 3]
                off = (1, v - 1, 0)[n % 3]
                cfg = mbr.Config(mbr.PATH_VECTOR_ANY, wpr, vpl, 1, 2 if n % 4 == 3 else 0)
                say("any", dtype, fused, cfg, "hidden", nvec * v + tail, "offset", off)
                _run_any(dtype, 5, nvec * v + tail, fused, cfg, off, 4000 + n)
                n += 1
    assert n == (48 if fused else 52)


def _run_any_offsets(rows, hidden, fused, offs, cfg=None, inplace=False, seed=0):
    """bf16 rows through the any-alignment path with x, residual, h and out at
    their own element offsets past a 16-byte boundary (inplace: out = x and
    h = residual), automatic or forced configuration: parity with the oracle
    and no byte outside the outputs written."""
    w = inputs.custom(rows, hidden, "bf16", fused)
    t = inputs.make(w, seed=seed)
    n = rows * hidden
    g = 64
    bases = [g + offs[i] + i * (n + 2 * g) for i in range(4)]  # x, residual, h, out
    if inplace:
        bases[3], bases[2] = bases[0], bases[1]
    buf = torch.full((4 * (n + 2 * g) + 2 * g,), 1.0, dtype=BF16, device="cuda")  # non-zero guard pattern
    buf[bases[0]:bases[0] + n] = t["x"].reshape(-1).cuda()
    if fused:
        buf[bases[1]:bases[1] + n] = t["residual"].reshape(-1).cuda()
    wt = t["weight"].cuda()
    ptr = [buf.data_ptr() + 2 * b for b in bases]
    L = mbr.lib()
    stream = torch.cuda.current_stream().cuda_stream
    cfgp = ctypes.byref(cfg) if cfg is not None else None
    if fused:
        st = L.rmsnorm_residual_fwd_ex(ptr[0], ptr[1], wt.data_ptr(), ptr[2], ptr[3], rows, hidden, w.eps, 1, cfgp,
                                       stream)
    else:
        st = L.rmsnorm_fwd_ex(ptr[0], wt.data_ptr(), ptr[3], rows, hidden, w.eps, 1, cfgp, stream)
    torch.cuda.synchronize()
    assert st == mbr.RMSNORM_OK, mbr.rmsnorm_status_string(st)
    aligned = hidden % 8 == 0 and all(b % 8 == 0 for b in (bases if fused else bases[::3]))
    used = cfg if cfg is not None else mbr.rmsnorm_select_config(rows, hidden, BF16, aligned, fused)
    cpu = inputs.bits(buf.cpu())
    xb, wb = inputs.bits(t["x"]), inputs.bits(t["weight"])
    h_want, y_want, e, gamma = expect(xb, wb, w.eps, used, inputs.bits(t["residual"]) if fused else None)
    if fused:
        assert np.array_equal(cpu[bases[2]:bases[2] + n].reshape(rows, hidden), h_want), "residual sum differs"
    parity.compare(cpu[bases[3]:bases[3] + n].reshape(rows, hidden), y_want, e, gamma)
    written = np.zeros(cpu.shape, bool)
    for i in ((0, 1, 2, 3) if fused else (0, 3)):
        written[bases[i]:bases[i] + n] = True
    assert np.all(cpu[~written] == inputs.bits(torch.ones(1, dtype=BF16))[0]), "a byte outside the buffers changed"


# element offsets of (x, residual, h, out) past a 16-byte boundary: every row
# tensor 2 bytes past a 4-byte boundary (shifted frame), 4-byte aligned but
# not 16 (no shift), and mixed (x and out at different offsets modulo 4: the
# frame is off and rows move at their own alignment)
ANY_OFFSETS = [(0, 0, 0, 0), (1, 1, 1, 1), (3, 5, 7, 1), (2, 2, 6, 4), (1, 0, 0, 0), (0, 3, 1, 2), (5, 1, 1, 4)]


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("hidden", [9, 15, 17, 2049, 4095, 5121, 8191, 8193])
def test_any_alignment_shifted_frame(hidden, fused):
    """The any-alignment path's shifted frame: rows that start 2 bytes past a
    4-byte boundary move as the dword-aligned row one element earlier.  Odd
    widths (rows alternate between the two cases), every mix of tensor
    offsets, in place, the automatic choice and forced configurations that
    do and do not cover the longer shifted row."""
    rows = 7
    n = 0
    for offs in ANY_OFFSETS:
        say("any frame", hidden, fused, offs)
        _run_any_offsets(rows, hidden, fused, offs, seed=hidden + n)
        n += 1
    say("any frame in place", hidden, fused)
    _run_any_offsets(rows, hidden, fused, (1, 1, 1, 1), inplace=True, seed=hidden + 99)
    _run_any_offsets(rows, hidden, fused, (0, 2, 2, 0), inplace=True, seed=hidden + 98)
    nv = hidden // 8
    for wpr in (1, 2, 4):
        per = -(-nv // (64 * wpr))
        if per < 1 or not built.any_(wpr, per, fused):
            continue
        cfg = mbr.Config(mbr.PATH_VECTOR_ANY, wpr, per, 1, 2)
        say("any frame forced", hidden, fused, cfg)
        _run_any_offsets(rows, hidden, fused, (1, 1, 1, 1), cfg=cfg, seed=hidden + 50 + wpr)


def test_misaligned_fused():
    rows, hidden, eps = 17, 1024, 1e-5
    w = inputs.custom(rows, hidden, "bf16", True)
    t = inputs.make(w, seed=12)
    n = rows * hidden
    buf = torch.zeros(4 * n + 64, dtype=BF16, device="cuda")
    xo, ro, ho, oo = 1, n + 3, 2 * n + 5, 3 * n + 9
    buf[xo:xo + n] = t["x"].reshape(-1).cuda()
    buf[ro:ro + n] = t["residual"].reshape(-1).cuda()
    wt = t["weight"].cuda()
    p = buf.data_ptr()
    st = mbr.lib().rmsnorm_residual_fwd(p + 2 * xo, p + 2 * ro, wt.data_ptr(), p + 2 * ho, p + 2 * oo, rows, hidden,
                                        eps, 1, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == mbr.RMSNORM_OK
    h_want, y_want, e, gamma = expect(inputs.bits(t["x"]), inputs.bits(t["weight"]), eps,
                                      auto(rows, hidden, BF16, False, True), inputs.bits(t["residual"]))
    cpu = inputs.bits(buf.cpu())
    assert np.array_equal(cpu[ho:ho + n].reshape(rows, hidden), h_want)
    parity.compare(cpu[oo:oo + n].reshape(rows, hidden), y_want, e, gamma)


@pytest.mark.parametrize("hidden", [4096, 4100])
def test_in_place_plain(hidden):
    w = inputs.custom(300, hidden, "bf16", False)
    t = inputs.make(w, seed=13)
    _, want, e, gamma = expect(inputs.bits(t["x"]), inputs.bits(t["weight"]), 1e-5, auto(300, hidden, BF16))
    x = t["x"].cuda()
    run_plain(x, t["weight"].cuda(), 1e-5, out=x)
    parity.compare(inputs.bits(x), want, e, gamma)


@pytest.mark.parametrize("alias", ["h=residual", "h=x", "out=x", "out=residual", "h=x,out=residual"])
def test_in_place_fused(alias):
    w = inputs.custom(257, 5120, "bf16", True)
    t = inputs.make(w, seed=14)
    h_want, y_want, e, gamma = expect(inputs.bits(t["x"]), inputs.bits(t["weight"]), 1e-5,
                                      auto(257, 5120, BF16, True, True), inputs.bits(t["residual"]))
    x, r, wt = t["x"].cuda(), t["residual"].cuda(), t["weight"].cuda()
    named = {"x": x, "residual": r}
    h = torch.empty_like(x)
    out = torch.empty_like(x)
    for part in alias.split(","):
        k, v = part.split("=")
        if k == "h":
            h = named[v]
        else:
            out = named[v]
    run_fused(x, r, wt, 1e-5, h=h, out=out)
    assert np.array_equal(inputs.bits(h), h_want)
    parity.compare(inputs.bits(out), y_want, e, gamma)


def test_overlap_rejected_on_device_buffers():
    """Partial overlaps are refused (and nothing is launched) -- real buffers,
    so even a validation slip could not touch memory outside this allocation."""
    buf = torch.zeros(4 * 64 * 2, dtype=BF16, device="cuda")
    wt = torch.ones(64, dtype=BF16, device="cuda")
    p = buf.data_ptr()
    st = _raw_plain(p, wt.data_ptr(), p + 32, 2, 64, 1e-5, 1)
    assert st == mbr.RMSNORM_ERR_INVALID_ARG
    assert torch.count_nonzero(buf) == 0


def test_non_default_stream():
    w = inputs.WORKLOADS["bf16_prefill_4096x2048"]
    t = inputs.make(w, seed=15)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        x, wt = t["x"].cuda(), t["weight"].cuda()
        out = torch.empty_like(x)
        mbr.rmsnorm_fwd(x, wt, out, w.eps)
    s.synchronize()
    _, want, e, gamma = expect(inputs.bits(t["x"]), inputs.bits(t["weight"]), w.eps, auto(w.rows, w.hidden, BF16))
    parity.compare(inputs.bits(out), want, e, gamma)


# ---------------------------------------------------------------- determinism and degenerate rows


@pytest.mark.parametrize("name", [inputs.HEADLINE, "bf16_residual_12289x5120"])
def test_bitwise_deterministic(name):
    w = inputs.WORKLOADS[name]
    t = {k: v.cuda() for k, v in inputs.make(w, seed=0, rows=2048).items()}
    if w.fused:
        a = run_fused(t["x"], t["residual"], t["weight"], w.eps)
        b = run_fused(t["x"], t["residual"], t["weight"], w.eps)
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    else:
        assert torch.equal(run_plain(t["x"], t["weight"], w.eps), run_plain(t["x"], t["weight"], w.eps))


def test_row_batches_bitwise_equal_in_one_config():
    w = inputs.custom(4096, 8192, "bf16", False)
    t = {k: v.cuda() for k, v in inputs.make(w, seed=16).items()}
    cfg = mbr.rmsnorm_select_config(4096, 8192, BF16)
    full = run_plain(t["x"], t["weight"], 1e-5, cfg)
    top = run_plain(t["x"][:1000].contiguous(), t["weight"], 1e-5, cfg)
    bot = run_plain(t["x"][1000:].contiguous(), t["weight"], 1e-5, cfg)
    assert torch.equal(full, torch.cat([top, bot]))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_degenerate_rows(dtype):
    """A zero row gives zeros (eps > 0); NaN and Inf stay in their own rows;
    constant rows give c / sqrt(c^2 + eps) * w; eps = 0 works on non-zero rows."""
    td = BF16 if dtype == "bf16" else F32
    H = 4096
    x = torch.randn(6, H, generator=torch.Generator().manual_seed(0)).to(td)
    x[0] = 0
    x[1, 7] = float("nan")
    x[2, 9] = float("inf")
    x[3] = -3.0
    wt = (1 + 0.1 * torch.randn(H, generator=torch.Generator().manual_seed(1))).to(td)
    for eps in (1e-5, 0.0):
        xs = x if eps > 0 else x[1:]
        y = run_plain(xs.cuda(), wt.cuda(), eps)
        _, want, e, gamma = expect(inputs.bits(xs), inputs.bits(wt), eps, auto(xs.shape[0], H, td))
        got = inputs.bits(y)
        if eps > 0:
            assert np.all(got[0].astype(np.float64) == 0) if dtype == "f32" else np.all(got[0] & 0x7FFF == 0)
        parity.compare(got, want, e, gamma)


def test_pages_rmsnorm_test_case_on_gpu():
    """The xserv RMSNorm tests' data (rows 4, hidden 768, eps 1e-5) through the
    HIP path: parity with the oracle, and within the pages' tolerances of their
    f32 CPU reference computed from the unrounded inputs."""
    rows, hidden, eps = 4, 768, 1e-5
    i = np.arange(rows * hidden)
    x = (((i % 17).astype(np.float32) - np.float32(8.0)) * np.float32(0.1)).reshape(rows, hidden)
    g = (np.float32(0.5) + (np.arange(hidden) % 3).astype(np.float32) * np.float32(0.2)).astype(np.float32)
    ref = x.astype(np.float64) / np.sqrt(np.mean(x.astype(np.float64) ** 2, axis=1, keepdims=True) + eps) * g
    for td, tol in ((F32, 1e-4), (BF16, 0.05)):
        xt, gt = torch.from_numpy(x).to(td), torch.from_numpy(g).to(td)
        y = run_plain(xt.cuda(), gt.cuda(), eps)
        _, want, e, gamma = expect(inputs.bits(xt), inputs.bits(gt), eps, auto(rows, hidden, td))
        parity.compare(inputs.bits(y), want, e, gamma)
        err = float(np.max(np.abs(y.float().cpu().numpy() - ref)))
        say("pages' test case", td, "max_err vs f32 reference on unrounded inputs", err)
        assert err <= tol


@pytest.mark.parametrize("fused", [False, True])
def test_graph_capture_replays_match_eager(fused):
    """Both entry points captured in a HIP graph: every replay, with eager work
    and synchronisations in between, equals the eager result bitwise."""
    w = inputs.custom(3000, 5120, "bf16", fused)
    t = {k: v.cuda() for k, v in inputs.make(w, seed=17).items()}
    x, wt = t["x"], t["weight"]
    if fused:
        h_e, y_e = run_fused(x, t["residual"], wt, 1e-5)
    else:
        y_e = run_plain(x, wt, 1e-5)
    h_g = torch.empty_like(x)
    y_g = torch.empty_like(x)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        if fused:
            mbr.rmsnorm_residual_fwd(x, t["residual"], wt, h_g, y_g, 1e-5)
        else:
            mbr.rmsnorm_fwd(x, wt, y_g, 1e-5)
    for rep in range(3):
        y_g.zero_()
        h_g.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_g, y_e), "replay %d differs" % rep
        if fused:
            assert torch.equal(h_g, h_e), "replay %d differs (h)" % rep
        # eager work between replays
        run_plain(x, wt, 1e-5)


def test_hbm_copy_copies():
    src = torch.randint(0, 255, (3 * (1 << 20) + 13,), dtype=torch.uint8, device="cuda")
    dst = torch.zeros_like(src)
    mbr.hbm_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


# ---------------------------------------------------------------- rows narrower than a wave


def subwave_configs():
    """(lanes per row, vectors per lane, rows per workgroup) for every built
    sub-wave kernel, at the smallest and the largest workgroup."""
    out = []
    for lpr in (8, 16, 32):
        for vpl in (1, 2):
            for rpb in (64 // lpr, 512 // lpr):
                out.append((lpr, vpl, rpb))
    return out


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("fused", [False, True])
def test_every_subwave_config(dtype, fused):
    """Several rows per wave: exact and partial rows, a partial last group of
    rows, and a capped grid that walks row groups."""
    vecw = 8 if dtype == "bf16" else 4
    n = 0
    for lpr, vpl, rpb in subwave_configs():
        for nvec in sorted({lpr * vpl, max(1, lpr * vpl - 3), lpr * (vpl - 1) + 1}):
            for mb in (0, 2):
                rows = 2 * rpb + 3
                cfg = mbr.Config(mbr.PATH_VECTOR, 1, vpl, rpb, mb, lpr)
                w = inputs.custom(rows, nvec * vecw, dtype, fused)
                say("subwave", dtype, fused, cfg, "hidden", nvec * vecw, "rows", rows)
                check_workload(w, inputs.make(w, seed=n), cfg)
                n += 1
    assert n > 50


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("hidden", [8, 16, 64, 96, 128, 200, 256, 384, 512])
@pytest.mark.parametrize("fused", [False, True])
def test_narrow_rows_automatic(dtype, hidden, fused):
    """Narrow rows (per-head norms) at many rows take the sub-wave path."""
    rows = 20001
    cfg = mbr.rmsnorm_select_config(rows, hidden, BF16 if dtype == "bf16" else F32, True, fused)
    say("narrow", dtype, hidden, fused, cfg)
    w = inputs.custom(rows, hidden, dtype, fused)
    check_workload(w, inputs.make(w, seed=hidden))

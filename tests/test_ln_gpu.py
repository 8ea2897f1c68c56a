"""Parity of the HIP LayerNorm (through the C ABI) with the CPU oracle.

Outputs are compared element by element with the bound derived in
tests/parity.py (fp32 evaluation error scaled by the magnitude of the terms,
plus one unit in the last place).  Covered: the stated LayerNorm workloads at
full size in the automatic launch configuration (the one bench.py times),
every built vector / element / multi-pass configuration with partial last
vectors or lanes, ragged widths, rows with a large common offset (where
E[x^2] - mean^2 would cancel), no-bias calls, in-place output, misaligned
buffers, degenerate rows, determinism, streams, graph replays and the pages'
own LayerNorm test case.
"""
import sys

import numpy as np
import pytest
import torch

import memory_bound_rmsnorm_amd as mbr
from memory_bound_rmsnorm_amd import inputs
from tests import parity
from tests.test_oracle_pins import _read_golden
from tests import built

pytestmark = pytest.mark.gpu

BF16, F32 = torch.bfloat16, torch.float32


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def tdt(dtype):
    return BF16 if dtype == "bf16" else F32


def run_ln(x, g, b, eps, cfg=None, out=None):
    out = torch.empty_like(x) if out is None else out
    mbr.layernorm_fwd_ex(x, g, b, out, eps, cfg)
    torch.cuda.synchronize()
    return out


def check(w, t, cfg=None, eps=None, bias=True):
    eps = w.eps if eps is None else eps
    dev = {k: v.cuda() for k, v in t.items()}
    y = run_ln(dev["x"], dev["weight"], dev["beta"] if bias else None, eps, cfg)
    xb, gb = inputs.bits(t["x"]), inputs.bits(t["weight"])
    bb = inputs.bits(t["beta"]) if bias else None
    c = cfg if cfg is not None else mbr.layernorm_select_config(w.rows, w.hidden, tdt(w.dtype), True)
    return parity.compare_ln(inputs.bits(y.cpu()), parity.oracle_ln(xb, gb, bb, eps), xb, gb, bb, eps, c)


@pytest.mark.parametrize("name", list(inputs.LN_WORKLOADS))
def test_ln_workloads_full_size(name):
    w = inputs.LN_WORKLOADS[name]
    say("ln workload", name, mbr.layernorm_select_config(w.rows, w.hidden, tdt(w.dtype), True))
    say(name, check(w, inputs.make(w, seed=0)))


RAGGED = [(1, 1), (3, 3), (5, 7), (2, 8), (5, 9), (67, 127), (12, 769), (5, 2048), (3, 4095), (7, 5120),
          (5, 5121), (3, 8193), (9, 16384), (2, 20000), (3, 65536), (2, 81920), (2, 131080)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,hidden", RAGGED)
def test_ln_ragged_shapes(rows, hidden, dtype):
    w = inputs.custom(rows, hidden, dtype, layernorm=True)
    say("ln shape", rows, hidden, dtype, mbr.layernorm_select_config(rows, hidden, tdt(dtype), True))
    check(w, inputs.make(w, seed=rows * 3 + hidden), bias=(hidden % 2 == 0))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ln_every_vector_config(dtype):
    vecw = 8 if dtype == "bf16" else 4
    n = 0
    for wpr in built.WPR:
        for vpl in built.LN_VPL:
            if not built.ln_vec(wpr, vpl):
                continue
            lanes = 64 * wpr
            for nvec in sorted({lanes * vpl, max(1, lanes * vpl - 37), lanes * (vpl - 1) + 1}):
                cfg = mbr.Config(mbr.PATH_VECTOR, wpr, vpl, 1, 2 if n % 3 == 0 else 0)
                w = inputs.custom(5, nvec * vecw, dtype, layernorm=True)
                say("ln vector", dtype, cfg, "hidden", nvec * vecw)
                check(w, inputs.make(w, seed=n), cfg, bias=(n % 2 == 0))
                n += 1
    assert n > 100


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ln_gamma_beta_in_lds(dtype):
    """weight_lds = 1 (gamma and beta copied into LDS once per workgroup, which
    then holds rows_per_block row slots) on every built vector configuration:
    one slot and the most slots, full and masked rows, with and without beta,
    and a capped grid whose workgroups walk several row groups.  Bitwise equal
    to the per-row-load kernel, and within the oracle's bound."""
    vecw = 8 if dtype == "bf16" else 4
    n = 0
    for wpr in built.WPR:
        for vpl in built.LN_VPL:
            if not built.ln_vec(wpr, vpl):
                continue
            lanes = 64 * wpr
            max_rpb = (1024 if wpr == 16 else 512) // lanes
            for nvec in sorted({lanes * vpl, max(1, lanes * vpl - 37)}):
                for rpb, mb in sorted({(1, 0), (max_rpb, 0), (max_rpb, 2)}):
                    bias = n % 2 == 0
                    if nvec * 16 * (2 if bias else 1) > 159 * 1024:
                        continue
                    rows = 2 * rpb + 1
                    w = inputs.custom(rows, nvec * vecw, dtype, layernorm=True)
                    t = inputs.make(w, seed=700 + n)
                    on = mbr.Config(mbr.PATH_VECTOR, wpr, vpl, rpb, mb, 0, 1)
                    off = mbr.Config(mbr.PATH_VECTOR, wpr, vpl, 1, 0)
                    say("ln gamma/beta in LDS", dtype, on, "hidden", nvec * vecw, "bias", bias)
                    x, g = t["x"].cuda(), t["weight"].cuda()
                    b = t["beta"].cuda() if bias else None
                    assert torch.equal(run_ln(x, g, b, w.eps, on), run_ln(x, g, b, w.eps, off))
                    if n % 4 == 0:
                        check(w, t, on, bias=bias)
                    n += 1
    assert n > 60


NARROW = [(1024, 8), (1027, 64), (4096, 128), (3001, 256), (2050, 384), (1500, 512), (20000, 128), (9000, 24)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,hidden", NARROW)
def test_ln_narrow_rows_automatic(rows, hidden, dtype):
    """Per-head widths from 1024 rows take several rows per wave when they
    are whole vectors; checked through the automatic choice."""
    w = inputs.custom(rows, hidden, dtype, layernorm=True)
    cfg = mbr.layernorm_select_config(rows, hidden, tdt(dtype), True)
    say("ln narrow", rows, hidden, dtype, cfg.as_dict())
    if hidden % (8 if dtype == "bf16" else 4) == 0 and hidden // (8 if dtype == "bf16" else 4) <= 64:
        assert cfg.lanes_per_row in (8, 16, 32)
    check(w, inputs.make(w, seed=rows + 5 * hidden), bias=rows % 2 == 0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ln_subwave_configs(dtype):
    """Rows narrower than a wave (8, 16 or 32 lanes per row): one, two and
    eight waves per workgroup, full and masked rows, rows that leave part of
    a wave or of the last group idle, capped grids; without beta every third
    case."""
    vecw = 8 if dtype == "bf16" else 4
    n = 0
    for lpr in (8, 16, 32):
        for vpl in (1, 2):
            for rpb in (64 // lpr, 128 // lpr, 512 // lpr):
                for nvec in sorted({lpr * vpl, max(1, lpr * (vpl - 1) + 3)}):
                    for mb, rows in ((0, rpb + 1), (3, 7 * rpb + 5), (0, 3), (0, 1)):
                        cfg = mbr.Config(mbr.PATH_VECTOR, 1, vpl, rpb, mb, lpr)
                        w = inputs.custom(rows, nvec * vecw, dtype, layernorm=True)
                        say("ln sub-wave", dtype, cfg.as_dict(), "hidden", nvec * vecw, "rows", rows)
                        check(w, inputs.make(w, seed=3000 + n), cfg, bias=(n % 3 != 2))
                        n += 1
    assert n > 100


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ln_every_element_and_multipass_config(dtype):
    n = 0
    for wpr in built.WPR:
        for epl in built.LN_EPL:
            if not built.elem(wpr, epl):
                continue
            # the one built element configuration: below one vector (as
            # chosen) and up to the whole wave it covers
            for hidden in (1, 2, 3, 5, 7, 33, 59, 64):
                cfg = mbr.Config(mbr.PATH_ELEMENT, wpr, epl, 1, 2 if n % 2 else 0)
                w = inputs.custom(5, hidden, dtype, layernorm=True)
                say("ln element", dtype, cfg, "hidden", hidden)
                check(w, inputs.make(w, seed=n), cfg, bias=(n % 3 != 0))
                n += 1
        for hidden in (4096, 4099, 12288 + 8):
            cfg = mbr.Config(mbr.PATH_TWO_PASS, wpr, 0, 1, 2)
            w = inputs.custom(5, hidden, dtype, layernorm=True)
            say("ln multipass", dtype, cfg, "hidden", hidden)
            check(w, inputs.make(w, seed=wpr + hidden), cfg)


@pytest.mark.parametrize("dtype,offset", [("f32", 1000.0), ("f32", -3.0e4), ("bf16", 100.0)])
def test_ln_large_common_offset(dtype, offset):
    """Rows far from zero mean: the centred variance keeps full accuracy (a
    variance from E[x^2] - mean^2 in fp32 would lose it entirely here)."""
    for hidden in (4096, 5121, 81920):
        w = inputs.custom(6, hidden, dtype, layernorm=True, x=inputs.Dist("normal", offset, 1.0))
        st = check(w, inputs.make(w, seed=hidden))
        say("ln offset", dtype, offset, hidden, st)


def test_ln_in_place_and_degenerate_rows():
    w = inputs.custom(40, 4096, "bf16", layernorm=True)
    t = {k: v.cuda() for k, v in inputs.make(w, seed=8).items()}
    y = run_ln(t["x"], t["weight"], t["beta"], 1e-5)
    x2 = t["x"].clone()
    assert torch.equal(run_ln(x2, t["weight"], t["beta"], 1e-5, out=x2), y)
    # constant rows and hidden = 1 give beta exactly
    const = torch.full((3, 4096), 2.5, dtype=BF16, device="cuda")
    assert torch.equal(run_ln(const, t["weight"], t["beta"], 1e-5), t["beta"].expand(3, 4096))
    one = torch.randn(5, 1, device="cuda").to(BF16)
    assert torch.equal(run_ln(one, t["weight"][:1], t["beta"][:1], 1e-5), t["beta"][:1].expand(5, 1))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ln_misaligned_pointers(dtype):
    rows, hidden, eps = 33, 2048, 1e-5
    td = tdt(dtype)
    es = 2 if dtype == "bf16" else 4
    w = inputs.custom(rows, hidden, dtype, layernorm=True)
    t = inputs.make(w, seed=11)
    xbuf = torch.zeros(rows * hidden + 8, dtype=td, device="cuda")
    obuf = torch.zeros(rows * hidden + 8, dtype=td, device="cuda")
    gbuf = torch.zeros(hidden + 8, dtype=td, device="cuda")
    bbuf = torch.zeros(hidden + 8, dtype=td, device="cuda")
    xbuf[1:1 + rows * hidden] = t["x"].reshape(-1).cuda()
    gbuf[1:1 + hidden] = t["weight"].cuda()
    bbuf[1:1 + hidden] = t["beta"].cuda()
    st = mbr.lib().layernorm_fwd(xbuf.data_ptr() + es, gbuf.data_ptr() + es, bbuf.data_ptr() + es,
                                 obuf.data_ptr() + es, rows, hidden, eps, mbr.dtype_code(td),
                                 torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == mbr.RMSNORM_OK
    y = inputs.bits(obuf[1:1 + rows * hidden].reshape(rows, hidden).cpu())
    xb, gb, bb = inputs.bits(t["x"]), inputs.bits(t["weight"]), inputs.bits(t["beta"])
    cfg = mbr.layernorm_select_config(rows, hidden, td, False)
    assert cfg.path == mbr.PATH_VECTOR_ANY  # vectors at the buffers' own alignment
    parity.compare_ln(y, parity.oracle_ln(xb, gb, bb, eps), xb, gb, bb, eps, cfg)
    assert obuf[0].item() == 0 and torch.count_nonzero(obuf[1 + rows * hidden:]) == 0


def test_ln_overlap_rejected_on_device_buffers():
    x = torch.randn(8, 256, device="cuda")
    g, b = torch.ones(256, device="cuda"), torch.zeros(256, device="cuda")
    L, s = mbr.lib(), torch.cuda.current_stream().cuda_stream
    INV = mbr.RMSNORM_ERR_INVALID_ARG
    assert L.layernorm_fwd(x.data_ptr(), g.data_ptr(), b.data_ptr(), x.data_ptr() + 4, 8, 256, 1e-5, 0, s) == INV
    assert L.layernorm_fwd(x.data_ptr(), g.data_ptr(), b.data_ptr(), g.data_ptr(), 1, 256, 1e-5, 0, s) == INV
    assert L.layernorm_fwd(x.data_ptr(), g.data_ptr(), b.data_ptr(), b.data_ptr(), 1, 256, 1e-5, 0, s) == INV


def test_ln_deterministic_streams_and_graph_replays():
    w = inputs.LN_WORKLOADS["bf16_ln_8192x4096"]
    t = {k: v.cuda() for k, v in inputs.make(w, seed=0).items()}
    y = run_ln(t["x"], t["weight"], t["beta"], w.eps)
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        y2 = torch.empty_like(y)
        mbr.layernorm_fwd(t["x"], t["weight"], t["beta"], y2, w.eps, stream=st)
    st.synchronize()
    assert torch.equal(y, y2)
    yg = torch.empty_like(y)
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        mbr.layernorm_fwd(t["x"], t["weight"], t["beta"], yg, w.eps)
    for rep in range(3):
        yg.zero_()
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        assert torch.equal(yg, y), rep
        run_ln(t["x"], t["weight"], None, w.eps)


def test_pages_layernorm_test_case_on_gpu():
    gd = _read_golden("xserv_layernorm_test.txt")
    rows, hidden, eps = int(gd["rows"]), int(gd["hidden"]), float(gd["eps"])
    i = np.arange(rows * hidden)
    x = (((i % 17).astype(np.float32) - np.float32(8.0)) * np.float32(0.1)).reshape(rows, hidden)
    j = np.arange(hidden)
    g = (np.float32(0.8) + (j % 5).astype(np.float32) * np.float32(0.1)).astype(np.float32)
    b = (((j % 7).astype(np.float32) - np.float32(3.0)) * np.float32(0.01)).astype(np.float32)
    y = run_ln(torch.from_numpy(x).cuda(), torch.from_numpy(g).cuda(), torch.from_numpy(b).cuda(), eps).cpu().numpy()
    want = oracle_y = parity.oracle_ln(x, g, b, eps)
    parity.compare_ln(y, oracle_y, x, g, b, eps, mbr.layernorm_select_config(rows, hidden, F32, True))
    assert float(np.max(np.abs(y - want))) <= float(gd["f32_atol"])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ln_non_finite_rows(dtype):
    """A NaN or an Inf in a row makes that row NaN (as in the oracle: the mean
    and the variance are non-finite) and leaves the other rows alone."""
    w = inputs.custom(9, 4096, dtype, layernorm=True)
    for bad in (float("nan"), float("inf"), -float("inf")):
        t = inputs.make(w, seed=5)
        t["x"][4, 100] = bad
        say("ln non-finite", dtype, bad)
        check(w, t)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ln_every_any_alignment_config(dtype):
    """Every built any-alignment LayerNorm configuration, forced: full and
    masked vector sets, tails of 0, 1 and V - 1 elements, x and out starting
    0, 1 or V - 1 elements past a 16-byte boundary inside guard space, with
    and without beta; parity with the oracle and no byte outside out written."""
    import ctypes
    v = 8 if dtype == "bf16" else 4
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    es = 2 if dtype == "bf16" else 4
    L = mbr.lib()
    n = 0
    for wpr in built.WPR:
        for vpl in built.ANY_VPL:
            if not built.ln_any(wpr, vpl):
                continue
            lanes = 64 * wpr
            for nvec in sorted({lanes * vpl, max(1, lanes * (vpl - 1) + 3)}):
                tail = (0, 1, v - 1)[n % 3]
                off = (1, v - 1, 0)[n % 3]
                bias = n % 2 == 0
                rows, hidden = 5, nvec * v + tail
                w = inputs.custom(rows, hidden, dtype, layernorm=True)
                t = inputs.make(w, seed=5000 + n)
                cnt, g = rows * hidden, 64
                # non-zero guard pattern: a stray write of a zero would show
                buf = torch.full((2 * (cnt + 2 * g) + 2 * g,), 1.0, dtype=td, device="cuda")
                xb, ob = g + off, g + off + cnt + 2 * g
                buf[xb:xb + cnt] = t["x"].reshape(-1).cuda()
                gam, bet = t["weight"].cuda(), t["beta"].cuda()
                cfg = mbr.Config(mbr.PATH_VECTOR_ANY, wpr, vpl, 1, 2 if n % 4 == 3 else 0)
                say("ln any", dtype, cfg, "hidden", hidden, "offset", off, "bias", bias)
                p = buf.data_ptr()
                st = L.layernorm_fwd_ex(p + es * xb, gam.data_ptr(), bet.data_ptr() if bias else None, p + es * ob,
                                        rows, hidden, w.eps, mbr.dtype_code(td), ctypes.byref(cfg),
                                        torch.cuda.current_stream().cuda_stream)
                torch.cuda.synchronize()
                assert st == mbr.RMSNORM_OK
                cpu = inputs.bits(buf.cpu())
                xbits, gbits = inputs.bits(t["x"]), inputs.bits(t["weight"])
                bbits = inputs.bits(t["beta"]) if bias else None
                got = cpu[ob:ob + cnt].reshape(rows, hidden)
                parity.compare_ln(got, parity.oracle_ln(xbits, gbits, bbits, w.eps), xbits, gbits, bbits, w.eps, cfg)
                written = np.zeros(cpu.shape, bool)
                written[xb:xb + cnt] = True
                written[ob:ob + cnt] = True
                assert np.all(cpu[~written] == inputs.bits(torch.ones(1, dtype=td))[0]), \
                    "a byte outside the buffers changed"
                n += 1
    assert n == 70


@pytest.mark.parametrize("hidden", [9, 17, 2049, 4095, 4097, 8191])
def test_ln_any_alignment_offsets(hidden):
    """bf16 LayerNorm at odd widths through the automatic choice, x and out
    at several offsets past a 16-byte boundary (the same and different ones
    modulo 4 bytes), in place, with and without beta: parity with the oracle
    and a guard pattern that must stay untouched."""
    import ctypes
    L = mbr.lib()
    rows, g = 7, 64
    cnt = rows * hidden
    n = 0
    for xo, oo, inplace in ((1, 1, False), (3, 5, False), (1, 0, False), (2, 6, False), (0, 0, False), (1, 1, True),
                            (0, 0, True)):
        bias = n % 2 == 0
        w = inputs.custom(rows, hidden, "bf16", layernorm=True)
        t = inputs.make(w, seed=7000 + hidden + n)
        buf = torch.full((2 * (cnt + 2 * g) + 2 * g,), 1.0, dtype=torch.bfloat16, device="cuda")
        xb = g + xo
        ob = xb if inplace else g + oo + cnt + 2 * g
        buf[xb:xb + cnt] = t["x"].reshape(-1).cuda()
        gam, bet = t["weight"].cuda(), t["beta"].cuda()
        say("ln any offsets", hidden, xo, oo, inplace, bias)
        p = buf.data_ptr()
        st = L.layernorm_fwd(p + 2 * xb, gam.data_ptr(), bet.data_ptr() if bias else None, p + 2 * ob, rows, hidden,
                             w.eps, 1, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert st == mbr.RMSNORM_OK
        cfg = mbr.layernorm_select_config(rows, hidden, torch.bfloat16, False)
        cpu = inputs.bits(buf.cpu())
        xbits, gbits = inputs.bits(t["x"]), inputs.bits(t["weight"])
        bbits = inputs.bits(t["beta"]) if bias else None
        got = cpu[ob:ob + cnt].reshape(rows, hidden)
        parity.compare_ln(got, parity.oracle_ln(xbits, gbits, bbits, w.eps), xbits, gbits, bbits, w.eps, cfg)
        written = np.zeros(cpu.shape, bool)
        written[xb:xb + cnt] = True
        written[ob:ob + cnt] = True
        assert np.all(cpu[~written] == inputs.bits(torch.ones(1, dtype=torch.bfloat16))[0]), \
            "a byte outside the buffers changed"
        n += 1


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,hidden", [(300, 4097), (1027, 769), (64, 5121), (2000, 100), (5, 9)])
def test_ln_odd_widths_automatic(rows, hidden, dtype):
    """Widths that are not whole vectors take the any-alignment path."""
    w = inputs.custom(rows, hidden, dtype, layernorm=True)
    cfg = mbr.layernorm_select_config(rows, hidden, tdt(dtype), True)
    say("ln odd", rows, hidden, dtype, cfg)
    if hidden % (8 if dtype == "bf16" else 4):
        assert cfg.path == mbr.PATH_VECTOR_ANY
    check(w, inputs.make(w, seed=rows + hidden), bias=rows % 2 == 0)

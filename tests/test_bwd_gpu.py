"""Parity of the HIP RMSNorm backward (through the C ABI) with the CPU oracle.

dx and dweight are compared element by element with the bounds derived in
tests/parity.py (fp32 evaluation error scaled by the magnitudes of the terms,
plus one unit in the last place).  Covered: the stated backward workloads at
full size in the automatic launch configuration (the one bench.py times),
every built vector / element / two-pass configuration on shapes with a partial
last vector or lane, grid caps that make workgroups walk many rows, ragged
widths, rows == 0, dx-only calls, in-place dx, misaligned buffers, workspace
checks, determinism, non-finite rows and HIP-graph replays.
"""
import ctypes
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


def tdt(dtype):
    return BF16 if dtype == "bf16" else F32


def run_bwd(x, w, dy, eps, cfg=None, want_dw=True, dx=None, ws=None):
    dx = torch.empty_like(x) if dx is None else dx
    dw = torch.empty_like(w) if want_dw else None
    mbr.rmsnorm_bwd_ex(x, w, dy, dx, dw, eps, ws, cfg)
    torch.cuda.synchronize()
    return dx, dw


def effective_config(rows, hidden, dtype, cfg=None, aligned=True):
    return cfg if cfg is not None else mbr.rmsnorm_select_bwd_config(rows, hidden, tdt(dtype), aligned)


def n_partials(rows, cfg):
    cap = cfg.max_blocks if cfg.max_blocks > 0 else 1 << 20
    return min(-(-rows // max(1, cfg.rows_per_block)), cap)


def check(w, t, cfg=None, eps=None, want_dw=True):
    eps = w.eps if eps is None else eps
    dev = {k: v.cuda() for k, v in t.items()}
    dx, dw = run_bwd(dev["x"], dev["weight"], dev["dy"], eps, cfg, want_dw)
    xb, wb, gb = inputs.bits(t["x"]), inputs.bits(t["weight"]), inputs.bits(t["dy"])
    dx_want, dw_want = parity.oracle_bwd(xb, wb, gb, eps, want_dw)
    c = effective_config(w.rows, w.hidden, w.dtype, cfg)
    return parity.compare_bwd(inputs.bits(dx), inputs.bits(dw) if want_dw else None, dx_want, dw_want,
                              xb, wb, gb, eps, c, n_partials(w.rows, c))


# ---------------------------------------------------------------- stated workloads


@pytest.mark.parametrize("name", list(inputs.BWD_WORKLOADS))
def test_bwd_workloads_full_size(name):
    w = inputs.BWD_WORKLOADS[name]
    say("bwd workload", name, "seed 0", mbr.rmsnorm_select_bwd_config(w.rows, w.hidden, tdt(w.dtype), True))
    say(name, check(w, inputs.make(w, seed=0)))


@pytest.mark.parametrize("seed", [1, 2])
def test_bwd_prefill_other_seeds(seed):
    w = inputs.BWD_WORKLOADS["bf16_bwd_4096x2048"]
    say("bwd prefill seed", seed)
    check(w, inputs.make(w, seed=seed))


# ---------------------------------------------------------------- shapes and configurations


RAGGED = [(1, 1), (3, 3), (5, 7), (2, 8), (5, 9), (67, 127), (12, 769), (5, 2048), (3, 4095), (7, 5120),
          (5, 5121), (3, 8193), (9, 16384), (2, 20000), (3, 65536), (2, 81920), (2, 131080), (5000, 96)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,hidden", RAGGED)
def test_bwd_ragged_shapes(rows, hidden, dtype):
    w = inputs.custom(rows, hidden, dtype, backward=True)
    say("bwd shape", rows, hidden, dtype, effective_config(rows, hidden, dtype))
    check(w, inputs.make(w, seed=rows * 5 + hidden))


NARROW = [(1024, 8), (1027, 64), (4096, 128), (3001, 256), (2050, 384), (1500, 512), (20000, 128), (9000, 24)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,hidden", NARROW)
def test_bwd_narrow_rows_automatic(rows, hidden, dtype):
    """Per-head widths from 1024 rows take several rows per wave when they
    are whole vectors; checked through the automatic choice."""
    w = inputs.custom(rows, hidden, dtype, backward=True)
    cfg = effective_config(rows, hidden, dtype)
    say("bwd narrow", rows, hidden, dtype, cfg.as_dict())
    if hidden % (8 if dtype == "bf16" else 4) == 0 and hidden // (8 if dtype == "bf16" else 4) <= 64:
        assert cfg.lanes_per_row in (8, 16, 32)
    check(w, inputs.make(w, seed=rows + 3 * hidden))


def test_bwd_many_rows_per_workgroup():
    """Far more rows than partial rows: every workgroup walks ~100 rows."""
    w = inputs.custom(40000, 1024, "bf16", backward=True)
    cfg = effective_config(40000, 1024, "bf16")
    say("bwd many rows", cfg)
    assert n_partials(40000, cfg) < 40000 // 8
    check(w, inputs.make(w, seed=5))


def _built_vec():
    return [(wpr, vpl) for wpr in built.WPR for vpl in built.BWD_VPL if built.bwd_vec(wpr, vpl)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bwd_every_vector_config(dtype):
    vecw = 8 if dtype == "bf16" else 4
    n = 0
    for wpr, vpl in _built_vec():
        lanes = 64 * wpr
        for nvec in sorted({lanes * vpl, max(1, lanes * vpl - 37), lanes * (vpl - 1) + 1}):
            for mb, rows in ((0, 3), (2, 5)):
                cfg = mbr.Config(mbr.PATH_VECTOR, wpr, vpl, 1, mb)
                w = inputs.custom(rows, nvec * vecw, dtype, backward=True)
                say("bwd vector", dtype, cfg, "hidden", nvec * vecw, "rows", rows)
                check(w, inputs.make(w, seed=n), cfg, want_dw=(n % 3 != 2))
                n += 1
    assert n == 180


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bwd_rows_per_block_configs(dtype):
    """Several row slots per workgroup on every built vector configuration
    that fits the thread limit: rows not a multiple of the slot count, slots
    with no row at all, masked rows, and caps that make each workgroup walk
    several groups; dx-only calls every third case."""
    vecw = 8 if dtype == "bf16" else 4
    n = 0
    for wpr, vpl in _built_vec():
        for rpb in {1: (2, 3, 8), 2: (2, 4), 4: (2,)}.get(wpr, ()):
            lanes = 64 * wpr
            for nvec in sorted({lanes * vpl, max(1, lanes * (vpl - 1) + 3)}):
                if nvec * vecw * 4 > 159 * 1024:
                    continue  # the LDS combine limit (checked on the CPU)
                for mb, rows in ((0, rpb + 1), (2, 5 * rpb + 2), (0, 1)):
                    cfg = mbr.Config(mbr.PATH_VECTOR, wpr, vpl, rpb, mb)
                    w = inputs.custom(rows, nvec * vecw, dtype, backward=True)
                    say("bwd slots", dtype, cfg, "hidden", nvec * vecw, "rows", rows)
                    check(w, inputs.make(w, seed=1000 + n), cfg, want_dw=(n % 3 != 2))
                    n += 1
    assert n > 100


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bwd_subwave_configs(dtype):
    """Rows narrower than a wave (8, 16 or 32 lanes per row): one wave and
    several waves per workgroup, full and masked rows, rows that leave part
    of a wave or of the last group idle, capped grids; dx-only calls every
    third case."""
    vecw = 8 if dtype == "bf16" else 4
    n = 0
    for lpr in (8, 16, 32):
        for vpl in (1, 2):
            for rpb in (64 // lpr, 128 // lpr, 512 // lpr):
                for nvec in sorted({lpr * vpl, max(1, lpr * (vpl - 1) + 3)}):
                    for mb, rows in ((0, rpb + 1), (3, 7 * rpb + 5), (0, 3), (0, 1)):
                        cfg = mbr.Config(mbr.PATH_VECTOR, 1, vpl, rpb, mb, lpr)
                        w = inputs.custom(rows, nvec * vecw, dtype, backward=True)
                        say("bwd sub-wave", dtype, cfg.as_dict(), "hidden", nvec * vecw, "rows", rows)
                        check(w, inputs.make(w, seed=2000 + n), cfg, want_dw=(n % 3 != 2))
                        n += 1
    assert n > 100


def test_bwd_subwave_many_groups_deterministic():
    """Per-head rows (bf16, hidden 128) over a capped grid: parity, and the
    same bits on a second call."""
    w = inputs.custom(40000, 128, "bf16", backward=True)
    cfg = mbr.Config(mbr.PATH_VECTOR, 1, 1, 32, 64, 16)
    say("bwd sub-wave many groups", cfg.as_dict())
    t = inputs.make(w, seed=9)
    check(w, t, cfg)
    dev = {k: v.cuda() for k, v in t.items()}
    a = run_bwd(dev["x"], dev["weight"], dev["dy"], w.eps, cfg)
    b = run_bwd(dev["x"], dev["weight"], dev["dy"], w.eps, cfg)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_bwd_rows_per_block_many_groups_deterministic():
    """A capped grid over many rows with row slots: parity, and the same bits
    on a second call."""
    w = inputs.custom(20000, 2048, "bf16", backward=True)
    cfg = mbr.Config(mbr.PATH_VECTOR, 2, 2, 4, 128)
    say("bwd slots many groups", cfg)
    t = inputs.make(w, seed=7)
    check(w, t, cfg)
    dev = {k: v.cuda() for k, v in t.items()}
    a = run_bwd(dev["x"], dev["weight"], dev["dy"], w.eps, cfg)
    b = run_bwd(dev["x"], dev["weight"], dev["dy"], w.eps, cfg)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bwd_every_element_config(dtype):
    """The one built element configuration (one wave, one element per lane)
    at every width it covers that matters: below one vector, as chosen, and
    up to a whole wave."""
    n = 0
    for wpr in built.WPR:
        for epl in built.BWD_EPL:
            if not built.elem(wpr, epl):
                continue
            for hidden in (1, 2, 3, 5, 7, 33, 59, 64):
                cfg = mbr.Config(mbr.PATH_ELEMENT, wpr, epl, 1, 2 if n % 2 else 0)
                w = inputs.custom(5, hidden, dtype, backward=True)
                say("bwd element", dtype, cfg, "hidden", hidden)
                check(w, inputs.make(w, seed=n), cfg, want_dw=(n % 4 != 3))
                n += 1
    assert n == 8


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bwd_every_two_pass_config(dtype):
    for wpr in (1, 2, 4, 8, 16):
        for hidden in (4096, 4099, 12288 + 8):
            for mb in (0, 2):
                cfg = mbr.Config(mbr.PATH_TWO_PASS, wpr, 0, 1, mb)
                w = inputs.custom(5, hidden, dtype, backward=True)
                say("bwd two-pass", dtype, cfg, "hidden", hidden)
                check(w, inputs.make(w, seed=wpr + hidden + mb), cfg)


def test_bwd_large_eps_and_small_rows():
    """eps comparable to mean(x^2): a misplaced eps would show."""
    w = inputs.custom(300, 2048, "f32", eps=0.5, x=inputs.Dist("normal", 0.0, 0.5), backward=True)
    say("bwd eps 0.5")
    check(w, inputs.make(w, seed=9))


# ---------------------------------------------------------------- semantics


def test_bwd_dx_only_matches_and_grid_cap_changes_no_dx_bit():
    w = inputs.custom(3000, 4096, "bf16", backward=True)
    t = {k: v.cuda() for k, v in inputs.make(w, seed=3).items()}
    dx_a, dw_a = run_bwd(t["x"], t["weight"], t["dy"], 1e-5)
    dx_b, _ = run_bwd(t["x"], t["weight"], t["dy"], 1e-5, want_dw=False)
    assert torch.equal(dx_a, dx_b)
    base = effective_config(3000, 4096, "bf16")
    for mb in (1, 7, 3000):
        cfg = mbr.Config(base.path, base.waves_per_row, base.items_per_lane, 1, mb)
        dx_c, dw_c = run_bwd(t["x"], t["weight"], t["dy"], 1e-5, cfg)
        assert torch.equal(dx_a, dx_c), mb
        say("bwd grid cap", mb)
        xb, wb, gb = (inputs.bits(t[k].cpu()) for k in ("x", "weight", "dy"))
        dx_want, dw_want = parity.oracle_bwd(xb, wb, gb, 1e-5)
        parity.compare_bwd(inputs.bits(dx_c.cpu()), inputs.bits(dw_c.cpu()), dx_want, dw_want, xb, wb, gb, 1e-5,
                           cfg, n_partials(3000, cfg))


@pytest.mark.parametrize("alias", ["dx=dy", "dx=x"])
@pytest.mark.parametrize("hidden", [4096, 4100, 81920])
def test_bwd_in_place(alias, hidden):
    w = inputs.custom(37, hidden, "bf16", backward=True)
    t = {k: v.cuda() for k, v in inputs.make(w, seed=4).items()}
    dx_e, dw_e = run_bwd(t["x"], t["weight"], t["dy"], 1e-5)
    x, dy = t["x"].clone(), t["dy"].clone()
    dst = dy if alias == "dx=dy" else x
    dx_i, dw_i = run_bwd(x, t["weight"], dy, 1e-5, dx=dst)
    assert dx_i.data_ptr() == dst.data_ptr()
    assert torch.equal(dx_i, dx_e) and torch.equal(dw_i, dw_e)


def test_bwd_rows_zero_zeroes_dweight():
    wt = torch.randn(1000, device="cuda").to(BF16)
    x = torch.empty(0, 1000, dtype=BF16, device="cuda")
    dw = torch.full_like(wt, float("nan"))
    mbr.rmsnorm_bwd(x, wt, torch.empty_like(x), torch.empty_like(x), dw, 1e-5)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dw) == 0 and not torch.isnan(dw).any()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bwd_misaligned_pointers(dtype):
    rows, hidden, eps = 33, 2048, 1e-5
    td = tdt(dtype)
    es = 2 if dtype == "bf16" else 4
    w = inputs.custom(rows, hidden, dtype, backward=True)
    t = inputs.make(w, seed=11)
    bufs = {k: torch.zeros(rows * hidden + 8, dtype=td, device="cuda") for k in ("x", "dy", "dx")}
    wbuf = torch.zeros(hidden + 8, dtype=td, device="cuda")
    dwbuf = torch.zeros(hidden + 8, dtype=td, device="cuda")
    bufs["x"][1:1 + rows * hidden] = t["x"].reshape(-1).cuda()
    bufs["dy"][1:1 + rows * hidden] = t["dy"].reshape(-1).cuda()
    wbuf[1:1 + hidden] = t["weight"].cuda()
    nbytes = mbr.rmsnorm_bwd_workspace_size(rows, hidden, td)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    st = mbr.lib().rmsnorm_bwd(bufs["x"].data_ptr() + es, wbuf.data_ptr() + es, bufs["dy"].data_ptr() + es,
                               bufs["dx"].data_ptr() + es, dwbuf.data_ptr() + es, rows, hidden, eps,
                               mbr.dtype_code(td), ws.data_ptr(), nbytes, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == mbr.RMSNORM_OK
    dx = inputs.bits(bufs["dx"][1:1 + rows * hidden].reshape(rows, hidden).cpu())
    dw = inputs.bits(dwbuf[1:1 + hidden].cpu())
    xb, wb, gb = inputs.bits(t["x"]), inputs.bits(t["weight"]), inputs.bits(t["dy"])
    dx_want, dw_want = parity.oracle_bwd(xb, wb, gb, eps)
    cfg = effective_config(rows, hidden, dtype, aligned=False)
    assert cfg.path == mbr.PATH_VECTOR_ANY
    parity.compare_bwd(dx, dw, dx_want, dw_want, xb, wb, gb, eps, cfg, n_partials(rows, cfg))
    assert bufs["dx"][0].item() == 0 and torch.count_nonzero(bufs["dx"][1 + rows * hidden:]) == 0
    assert dwbuf[0].item() == 0 and torch.count_nonzero(dwbuf[1 + hidden:]) == 0


def test_bwd_workspace_checked_on_device_buffers():
    rows, hidden = 100, 1024
    x = torch.randn(rows, hidden, device="cuda").to(BF16)
    dy, dx = torch.randn_like(x), torch.empty_like(x)
    wt = torch.ones(hidden, dtype=BF16, device="cuda")
    dw = torch.empty_like(wt)
    need = mbr.rmsnorm_bwd_workspace_size(rows, hidden, BF16)
    cfg = effective_config(rows, hidden, "bf16")
    assert need == n_partials(rows, cfg) * 1024 * 4
    ws = torch.empty(need + 64, dtype=torch.uint8, device="cuda")
    L, s = mbr.lib(), torch.cuda.current_stream().cuda_stream
    args = (x.data_ptr(), wt.data_ptr(), dy.data_ptr(), dx.data_ptr(), dw.data_ptr(), rows, hidden, 1e-5, 1)
    INV = mbr.RMSNORM_ERR_INVALID_ARG
    assert L.rmsnorm_bwd(*args, ws.data_ptr(), need - 1, s) == INV
    assert L.rmsnorm_bwd(*args, None, need, s) == INV
    assert L.rmsnorm_bwd(*args, ws.data_ptr() + 8, need, s) == INV          # not 16-byte aligned
    assert L.rmsnorm_bwd(*args[:4], dx.data_ptr() + 64, *args[5:], ws.data_ptr(), need, s) == INV  # dw inside dx
    assert L.rmsnorm_bwd(*args, dx.data_ptr(), need, s) == INV              # workspace over dx
    assert L.rmsnorm_bwd(*args[:3], x.data_ptr() + 2, *args[4:], ws.data_ptr(), need, s) == INV  # partial overlap
    assert L.rmsnorm_bwd(*args[:3], wt.data_ptr(), *args[4:], ws.data_ptr(), need, s) == INV     # dx over weight
    assert L.rmsnorm_bwd(*args, ws.data_ptr(), need, s) == mbr.RMSNORM_OK
    torch.cuda.synchronize()


@pytest.mark.parametrize("name", ["bf16_bwd_16384x8192", "fp32_bwd_64x2048"])
def test_bwd_bitwise_deterministic(name):
    w = inputs.BWD_WORKLOADS[name]
    t = {k: v.cuda() for k, v in inputs.make(w, seed=0).items()}
    a = run_bwd(t["x"], t["weight"], t["dy"], w.eps)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        dx, dw = torch.empty_like(t["x"]), torch.empty_like(t["weight"])
        mbr.rmsnorm_bwd(t["x"], t["weight"], t["dy"], dx, dw, w.eps, stream=s)
    s.synchronize()
    assert torch.equal(a[0], dx) and torch.equal(a[1], dw)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bwd_non_finite_rows(dtype):
    """A NaN or Inf in one row of x makes that row's dx and every dweight NaN,
    as in the oracle; other rows' dx are untouched."""
    w = inputs.custom(9, 1024, dtype, backward=True)
    t = inputs.make(w, seed=2)
    t["x"][3, 17] = float("nan")
    say("bwd non-finite", dtype)
    check(w, t)
    t = inputs.make(w, seed=2)
    t["dy"][5, 3] = float("inf")
    check(w, t)


def test_bwd_graph_capture_replays_match_eager():
    w = inputs.custom(3000, 5120, "bf16", backward=True)
    t = {k: v.cuda() for k, v in inputs.make(w, seed=17).items()}
    dx_e, dw_e = run_bwd(t["x"], t["weight"], t["dy"], 1e-5)
    dx_g, dw_g = torch.empty_like(t["x"]), torch.empty_like(t["weight"])
    ws = torch.empty(mbr.rmsnorm_bwd_workspace_size(3000, 5120, BF16), dtype=torch.uint8, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mbr.rmsnorm_bwd(t["x"], t["weight"], t["dy"], dx_g, dw_g, 1e-5, ws)
    for rep in range(3):
        dx_g.zero_()
        dw_g.zero_()
        ws.fill_(0x7F)  # the workspace's contents on entry must not matter
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dx_g, dx_e) and torch.equal(dw_g, dw_e), "replay %d differs" % rep
        run_bwd(t["x"], t["weight"], t["dy"], 1e-5)


def _run_bwd_any(dtype, rows, hidden, cfg, off, woff, seed, want_dw=True):
    """Forced configuration with x, dy and dx starting `off` elements and the
    weight and dweight `woff` elements past a 16-byte boundary, inside guard
    space: parity with the oracle, and no element outside dx and dweight
    written."""
    w = inputs.custom(rows, hidden, dtype, backward=True)
    t = inputs.make(w, seed=seed)
    td = tdt(dtype)
    es = 2 if dtype == "bf16" else 4
    n, g = rows * hidden, 64
    bases = [g + off + i * (n + 2 * g) for i in range(3)]  # x, dy, dx
    buf = torch.zeros(3 * (n + 2 * g) + 2 * g, dtype=td, device="cuda")
    buf[bases[0]:bases[0] + n] = t["x"].reshape(-1).cuda()
    buf[bases[1]:bases[1] + n] = t["dy"].reshape(-1).cuda()
    wbuf = torch.zeros(2 * (hidden + 2 * g), dtype=td, device="cuda")  # weight, dweight
    wb0, wb1 = g + woff, hidden + 3 * g + woff
    wbuf[wb0:wb0 + hidden] = t["weight"].cuda()
    nbytes = mbr.rmsnorm_bwd_workspace_size(rows, hidden, td, cfg)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    p, q = buf.data_ptr(), wbuf.data_ptr()
    st = mbr.lib().rmsnorm_bwd_ex(p + es * bases[0], q + es * wb0, p + es * bases[1], p + es * bases[2],
                                  q + es * wb1 if want_dw else None, rows, hidden, w.eps, mbr.dtype_code(td),
                                  ws.data_ptr() if want_dw else None, nbytes if want_dw else 0,
                                  ctypes.byref(cfg), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == mbr.RMSNORM_OK, mbr.rmsnorm_status_string(st)
    cpu, wcpu = inputs.bits(buf.cpu()), inputs.bits(wbuf.cpu())
    xb, wb, gb = inputs.bits(t["x"]), inputs.bits(t["weight"]), inputs.bits(t["dy"])
    dx_want, dw_want = parity.oracle_bwd(xb, wb, gb, w.eps, want_dw)
    dx = cpu[bases[2]:bases[2] + n].reshape(rows, hidden)
    dw = wcpu[wb1:wb1 + hidden] if want_dw else None
    say(parity.compare_bwd(dx, dw, dx_want, dw_want, xb, wb, gb, w.eps, cfg, n_partials(rows, cfg)))
    written = np.zeros(cpu.shape, bool)
    for i in range(3):
        written[bases[i]:bases[i] + n] = True
    assert not np.any(cpu[~written] != 0), "an element outside x, dy and dx changed"
    wwritten = np.zeros(wcpu.shape, bool)
    wwritten[wb0:wb0 + hidden] = True
    if want_dw:
        wwritten[wb1:wb1 + hidden] = True
    assert not np.any(wcpu[~wwritten] != 0), "an element outside weight and dweight changed"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bwd_every_any_alignment_config(dtype):
    """Every built any-alignment backward configuration, forced: full and
    masked vector sets, tails of 0, 1 and V - 1 elements, buffers at several
    offsets from a 16-byte boundary, with and without dweight and a grid cap."""
    v = 8 if dtype == "bf16" else 4
    n = 0
    for wpr in built.WPR:
        for vpl in built.BWD_VPL:
            if not built.bwd_any(wpr, vpl):
                continue
            lanes = 64 * wpr
            for nvec in sorted({lanes * vpl, max(1, lanes * (vpl - 1) + 3)}):
                tail = (0, 1, v - 1)[n % 3]
                off = (1, v - 1, 0)[n % 3]
                woff = (0, 1, v - 1, 2)[n % 4]
                cfg = mbr.Config(mbr.PATH_VECTOR_ANY, wpr, vpl, 1, 2 if n % 4 == 3 else 0)
                say("bwd any", dtype, cfg.as_dict(), "hidden", nvec * v + tail, "offsets", off, woff)
                _run_bwd_any(dtype, 5, nvec * v + tail, cfg, off, woff, 6000 + n, want_dw=n % 5 != 4)
                n += 1
    assert n == 54


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,hidden", [(4096, 8191), (2048, 5121), (4096, 4097), (4096, 2049), (300, 1031)])
def test_bwd_odd_widths_automatic(rows, hidden, dtype):
    """Widths that are not whole vectors take the any-alignment path by themselves."""
    td = tdt(dtype)
    cfg = mbr.rmsnorm_select_bwd_config(rows, hidden, td, True)
    assert cfg.path == mbr.PATH_VECTOR_ANY
    say("bwd odd width", dtype, rows, hidden, cfg.as_dict())
    _run_bwd_any(dtype, rows, hidden, cfg, 1, 1, hidden)

"""rmsnorm_bwd_noalloc -- the backward for callers that cannot allocate -- on
the GPU, through the C ABI: its outputs against rmsnorm_bwd's (the entry point
with a caller workspace) and against the oracle, on consecutive calls with a
smaller input second, past the scratch array's partial-row cap, and replayed
from a HIP graph."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import memory_bound_rmsnorm_amd as mbr
from memory_bound_rmsnorm_amd import inputs
from tests import parity

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 16 << 20


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _tensors(rows, hidden, dtype, seed):
    w = inputs.custom(rows, hidden, dtype, backward=True)
    t = inputs.make(w, seed=seed)
    return w, t, {k: t[k].cuda() for k in ("x", "weight", "dy")}


def _with_workspace(d, eps, cfg=None):
    x, wt, dy = d["x"], d["weight"], d["dy"]
    dx, dw = torch.empty_like(x), torch.empty_like(wt)
    need = mbr.rmsnorm_bwd_workspace_size(x.shape[0], x.shape[1], x.dtype, cfg)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    L = mbr.lib()
    args = (x.data_ptr(), wt.data_ptr(), dy.data_ptr(), dx.data_ptr(), dw.data_ptr(), x.shape[0], x.shape[1], eps,
            mbr.dtype_code(x.dtype), ws.data_ptr(), ws.numel())
    s = torch.cuda.current_stream().cuda_stream
    st = L.rmsnorm_bwd_ex(*args, ctypes.byref(cfg), s) if cfg is not None else L.rmsnorm_bwd(*args, s)
    assert st == mbr.RMSNORM_OK, mbr.rmsnorm_status_string(st)
    torch.cuda.synchronize()
    return dx, dw


def _noalloc(d, eps, want_dw=True):
    x, wt, dy = d["x"], d["weight"], d["dy"]
    dx = torch.empty_like(x)
    dw = torch.empty_like(wt) if want_dw else None
    st = mbr.lib().rmsnorm_bwd_noalloc(x.data_ptr(), wt.data_ptr(), dy.data_ptr(), dx.data_ptr(),
                                       dw.data_ptr() if want_dw else None, x.shape[0], x.shape[1], eps,
                                       mbr.dtype_code(x.dtype), torch.cuda.current_stream().cuda_stream)
    assert st == mbr.RMSNORM_OK, mbr.rmsnorm_status_string(st)
    torch.cuda.synchronize()
    return dx, dw


def _oracle_check(w, t, dx, dw, cfg, n_part):
    xb, wb, gb = inputs.bits(t["x"]), inputs.bits(t["weight"]), inputs.bits(t["dy"])
    dx_e, dw_e = parity.oracle_bwd(xb, wb, gb, w.eps, dw is not None)
    return parity.compare_bwd(inputs.bits(dx), inputs.bits(dw) if dw is not None else None, dx_e, dw_e, xb, wb, gb,
                              w.eps, cfg, n_part)


def _n_part(rows, cfg):
    return min(-(-rows // max(1, cfg.rows_per_block)), cfg.max_blocks if cfg.max_blocks > 0 else 1 << 20)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_two_calls_in_a_row_match_the_workspace_entry_point(dtype):
    """A larger call, then a smaller one on the same scratch array: both equal
    rmsnorm_bwd bitwise (same configuration below the cap) and meet the
    oracle's bound."""
    for rows, hidden, seed in ((4096, 2048, 1), (300, 1024, 2)):
        w, t, d = _tensors(rows, hidden, dtype, seed)
        say("noalloc", dtype, rows, hidden)
        a = _with_workspace(d, w.eps)
        b = _noalloc(d, w.eps)
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
        cfg = mbr.rmsnorm_select_bwd_config(rows, hidden, d["x"].dtype, True)
        say(_oracle_check(w, t, b[0], b[1], cfg, _n_part(rows, cfg)))


def test_partial_rows_capped_by_the_scratch_array():
    """hidden 16384 with 8192 rows wants 512 partial rows (32 MiB): the entry
    point takes 256 (what 16 MiB holds), equal bitwise to rmsnorm_bwd_ex forced
    to that cap, and within the oracle's bound; then a small call after it."""
    rows, hidden = 8192, 16384
    w, t, d = _tensors(rows, hidden, "bf16", 3)
    auto = mbr.rmsnorm_select_bwd_config(rows, hidden, torch.bfloat16, True)
    cap = SCRATCH_BYTES // (((hidden + 63) // 64 * 64) * 4)
    assert _n_part(rows, auto) > cap
    capped = mbr.Config(auto.path, auto.waves_per_row, auto.items_per_lane, auto.rows_per_block, cap,
                        auto.lanes_per_row, auto.weight_lds)
    say("noalloc capped", capped)
    a = _with_workspace(d, w.eps, capped)
    b = _noalloc(d, w.eps)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    say(_oracle_check(w, t, b[0], b[1], capped, cap))
    w2, t2, d2 = _tensors(64, 512, "bf16", 4)
    c = _noalloc(d2, w2.eps)
    assert torch.equal(c[0], _with_workspace(d2, w2.eps)[0]) and torch.equal(c[1], _with_workspace(d2, w2.eps)[1])


def test_without_dweight_and_with_no_rows():
    w, t, d = _tensors(777, 4096, "bf16", 5)
    dx, _ = _noalloc(d, w.eps, want_dw=False)
    assert torch.equal(dx, _with_workspace(d, w.eps)[0])
    dw = torch.full((4096,), 3.0, dtype=torch.bfloat16, device="cuda")
    st = mbr.lib().rmsnorm_bwd_noalloc(None, None, None, None, dw.data_ptr(), 0, 4096, 1e-5, 1,
                                       torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == mbr.RMSNORM_OK and torch.count_nonzero(dw) == 0


def test_graph_replays_match_eager():
    """Captured in a HIP graph (the caller that cannot allocate): every replay,
    with eager work in between, equals the eager result bitwise."""
    w, t, d = _tensors(2048, 4096, "bf16", 6)
    e_dx, e_dw = _noalloc(d, w.eps)
    dx, dw = torch.empty_like(e_dx), torch.empty_like(e_dw)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mbr.rmsnorm_bwd_noalloc(d["x"], d["weight"], d["dy"], dx, dw, w.eps)
    for rep in range(3):
        dx.zero_()
        dw.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dx, e_dx) and torch.equal(dw, e_dw), rep
        _noalloc(d, w.eps)  # eager use of the same scratch array between replays

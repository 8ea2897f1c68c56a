"""C-ABI checks of the backward entry points that need no GPU: declarations,
argument validation before any HIP call, the workspace-size formula and the
automatic configuration choice."""
import ctypes

import pytest
import torch

import memory_bound_rmsnorm_amd as mbr
from tests.test_abi_cpu import HEADERS, _declared, fake_only
from tests import built

INV = mbr.RMSNORM_ERR_INVALID_ARG


def test_backward_declared():
    names = {n for h in HEADERS for n in _declared(h)}
    for n in ("rmsnorm_bwd", "rmsnorm_bwd_ex", "rmsnorm_bwd_workspace_size", "rmsnorm_select_bwd_config"):
        assert n in names


def test_rows_zero_without_dweight_needs_no_pointers():
    assert mbr.lib().rmsnorm_bwd(None, None, None, None, None, 0, 64, 1e-5, 1, None, 0, None) == mbr.RMSNORM_OK


@pytest.mark.parametrize("rows,hidden,eps,dtype,want", [
    (-1, 16, 1e-5, 1, INV), (4, 0, 1e-5, 1, INV), (4, 2 ** 31, 1e-5, 1, INV), (4, 16, -1.0, 1, INV),
    (4, 16, float("nan"), 0, INV), (4, 16, float("inf"), 0, INV), (4, 16, 1e-5, 2, mbr.RMSNORM_ERR_UNSUPPORTED_DTYPE),
    (2 ** 62, 16, 1e-5, 1, INV),
])
def test_bad_sizes_rejected(rows, hidden, eps, dtype, want):
    assert mbr.lib().rmsnorm_bwd(None, None, None, None, None, rows, hidden, eps, dtype, None, 0, None) == want
    n = ctypes.c_size_t()
    if want == INV and eps == 1e-5:
        assert mbr.lib().rmsnorm_bwd_workspace_size(rows, hidden, dtype, None, ctypes.byref(n)) == INV


def test_workspace_size_formula():
    for rows, hidden, dt in [(0, 64, torch.bfloat16), (1, 1, torch.float32), (100, 1000, torch.bfloat16),
                             (16384, 8192, torch.bfloat16), (5, 131080, torch.float32), (70000, 96, torch.float32)]:
        need = mbr.rmsnorm_bwd_workspace_size(rows, hidden, dt)
        ld = (hidden + 63) // 64 * 64
        cfgs = [mbr.rmsnorm_select_bwd_config(rows, hidden, dt, a) for a in (True, False)]
        assert need == max(min(-(-rows // c.rows_per_block), c.max_blocks) for c in cfgs) * ld * 4
        cfg = mbr.Config(mbr.PATH_ELEMENT, 4, 8, 1, 3)
        assert mbr.rmsnorm_bwd_workspace_size(rows, hidden, dt, cfg) == min(rows, 3) * ld * 4
        # row slots share a partial row: one per group of rows_per_block rows
        for rpb, mb, lpr in ((4, 3, 0), (4, 0, 0), (2, 1000, 0), (16, 7, 16), (8, 0, 8)):
            cfg = mbr.Config(mbr.PATH_VECTOR, 1 if lpr else 2, 2, rpb, mb, lpr)
            groups = -(-rows // rpb)
            assert mbr.rmsnorm_bwd_workspace_size(rows, hidden, dt, cfg) == (min(groups, mb) if mb else groups) * ld * 4
    assert mbr.lib().rmsnorm_bwd_workspace_size(4, 16, 1, None, None) == INV
    bad = mbr.Config(mbr.PATH_VECTOR, 4, 2, 1, -1)
    assert mbr.lib().rmsnorm_bwd_workspace_size(4, 16, 1, ctypes.byref(bad), ctypes.byref(ctypes.c_size_t())) == INV


def test_headline_choice():
    c = mbr.rmsnorm_select_bwd_config(16384, 8192, torch.bfloat16, True)
    assert (c.path, c.waves_per_row, c.items_per_lane, c.rows_per_block, c.max_blocks) == (mbr.PATH_VECTOR, 4, 4, 1, 512)
    # narrower rows: four vectors per lane, four row slots, 256 partial rows
    c = mbr.rmsnorm_select_bwd_config(4096, 2048, torch.bfloat16, True)
    assert (c.path, c.waves_per_row, c.items_per_lane, c.rows_per_block, c.max_blocks) == (mbr.PATH_VECTOR, 1, 4, 4, 256)
    c = mbr.rmsnorm_select_bwd_config(16384, 4096, torch.bfloat16, True)
    assert (c.path, c.waves_per_row, c.items_per_lane, c.rows_per_block, c.max_blocks) == (mbr.PATH_VECTOR, 2, 4, 2, 512)
    # few rows: one row per workgroup, spread over more waves
    c = mbr.rmsnorm_select_bwd_config(64, 2048, torch.float32, True)
    assert (c.path, c.waves_per_row, c.items_per_lane, c.rows_per_block) == (mbr.PATH_VECTOR, 8, 1, 1)
    # narrow rows: lane groups of 8, 16 or 32 with at most two vectors per lane,
    # four waves per workgroup (eight with one vector per lane), fewer slots
    # when the rows would make under 256 groups
    for rows, hidden, dt, want in [(262144, 128, torch.bfloat16, (8, 2, 32)), (262144, 64, torch.bfloat16, (8, 1, 64)),
                                   (131072, 256, torch.bfloat16, (16, 2, 16)), (65536, 512, torch.bfloat16, (32, 2, 8)),
                                   (131072, 128, torch.float32, (16, 2, 16)), (4096, 128, torch.bfloat16, (8, 2, 16)),
                                   (1024, 128, torch.bfloat16, (8, 2, 8)), (65536, 24, torch.bfloat16, (8, 1, 64))]:
        c = mbr.rmsnorm_select_bwd_config(rows, hidden, dt, True)
        assert (c.path, c.waves_per_row, c.max_blocks) == (mbr.PATH_VECTOR, 1, 512), (rows, hidden)
        assert (c.lanes_per_row, c.items_per_lane, c.rows_per_block) == want, (rows, hidden, c.as_dict())
    c = mbr.rmsnorm_select_bwd_config(1023, 128, torch.bfloat16, True)
    assert c.lanes_per_row == 0


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("aligned", [True, False])
@pytest.mark.parametrize("rows", [1, 100, 5000, 100000])
def test_choice_is_built_and_covering(dtype, aligned, rows):
    v = 8 if dtype == torch.bfloat16 else 4
    for hidden in [1, 7, 8, 64, 100, 1000, 2048, 4095, 4096, 5120, 8192, 16384, 32768, 32776, 65536, 131080]:
        c = mbr.rmsnorm_select_bwd_config(rows, hidden, dtype, aligned)
        lanes = c.lanes_per_row or 64 * c.waves_per_row
        assert c.max_blocks >= 1 and c.waves_per_row in (1, 2, 4, 8, 16)
        assert c.rows_per_block == 1 or (c.path == mbr.PATH_VECTOR and lanes * c.rows_per_block <= 512
                                         and hidden * 4 <= 159 * 1024)
        if c.lanes_per_row:  # rows narrower than a wave: whole waves per workgroup
            assert c.path == mbr.PATH_VECTOR and c.lanes_per_row in (8, 16, 32) and c.waves_per_row == 1
            assert c.items_per_lane in (1, 2) and lanes * c.rows_per_block % 64 == 0
            assert rows >= 1024 and hidden // v <= 64
        if c.path == mbr.PATH_VECTOR:
            assert aligned and hidden % v == 0
            assert c.lanes_per_row or built.bwd_vec(c.waves_per_row, c.items_per_lane)
            assert lanes * c.items_per_lane >= hidden // v
        elif c.path == mbr.PATH_VECTOR_ANY:
            assert (not aligned or hidden % v != 0) and hidden >= v and c.rows_per_block == 1
            assert built.bwd_any(c.waves_per_row, c.items_per_lane)
            assert lanes * c.items_per_lane >= hidden // v
        elif c.path == mbr.PATH_ELEMENT:
            assert built.elem(c.waves_per_row, c.items_per_lane) and lanes * c.items_per_lane >= hidden
            assert hidden < v
        else:
            assert c.path == mbr.PATH_TWO_PASS and hidden > 8 * 1024


@fake_only
def test_pointer_validation():
    L = mbr.lib()
    X, W, G, D, DW, WS = (0x7F0000000000 + i * 0x10000000 for i in range(6))
    rows, hidden = 4, 16
    need = mbr.rmsnorm_bwd_workspace_size(rows, hidden, torch.bfloat16)

    def call(x=X, w=W, g=G, d=D, dw=DW, ws=WS, nb=need, dt=1):
        return L.rmsnorm_bwd(x, w, g, d, dw, rows, hidden, 1e-5, dt, ws, nb, None)

    for kw in [dict(x=None), dict(w=None), dict(g=None), dict(d=None), dict(x=X + 1), dict(dw=DW + 1),
               dict(d=D + 2, dt=0), dict(ws=None), dict(ws=WS + 8), dict(nb=need - 1),
               dict(d=X + 2), dict(d=G + 32), dict(d=W), dict(dw=X + 4), dict(dw=D), dict(dw=W), dict(dw=G + 2),
               dict(ws=X), dict(ws=D + 16), dict(ws=DW - 16)]:
        assert call(**kw) == INV, kw


@fake_only
def test_bad_forced_configs():
    L = mbr.lib()
    X, W, G, D, DW, WS = (0x7F0000000000 + i * 0x10000000 for i in range(6))
    rows, hidden = 4, 4096
    for cfg in [mbr.Config(mbr.PATH_VECTOR, 3, 2, 1, 0), mbr.Config(mbr.PATH_VECTOR, 8, 2, 2, 0),
                mbr.Config(mbr.PATH_VECTOR, 8, 2, 1, -1), mbr.Config(mbr.PATH_VECTOR, 1, 2, 1, 0),
                mbr.Config(mbr.PATH_VECTOR, 16, 5, 1, 0), mbr.Config(mbr.PATH_VECTOR, 8, 9, 1, 0),
                mbr.Config(mbr.PATH_ELEMENT, 4, 3, 1, 0), mbr.Config(mbr.PATH_ELEMENT, 1, 8, 1, 0),
                mbr.Config(7, 8, 2, 1, 0), mbr.Config(mbr.PATH_VECTOR, 1, 1, 1, 0, 16),
                # row slots: vector path only, within the thread limit
                mbr.Config(mbr.PATH_VECTOR, 4, 2, 0, 0), mbr.Config(mbr.PATH_VECTOR, 4, 2, 3, 0),
                mbr.Config(mbr.PATH_VECTOR, 2, 4, 8, 0), mbr.Config(mbr.PATH_ELEMENT, 4, 8, 2, 0),
                mbr.Config(mbr.PATH_TWO_PASS, 16, 0, 2, 0),
                # any alignment: one row per workgroup, whole waves, built and covering
                mbr.Config(mbr.PATH_VECTOR_ANY, 1, 4, 2, 0), mbr.Config(mbr.PATH_VECTOR_ANY, 1, 4, 1, 0, 32),
                mbr.Config(mbr.PATH_VECTOR_ANY, 1, 2, 1, 0), mbr.Config(mbr.PATH_VECTOR_ANY, 1, 9, 1, 0)]:
        n = mbr.rmsnorm_bwd_workspace_size(rows, hidden, torch.bfloat16, cfg) if cfg.max_blocks >= 0 else 0
        st = L.rmsnorm_bwd_ex(X, W, G, D, DW, rows, hidden, 1e-5, 1, WS, n, ctypes.byref(cfg), None)
        assert st == INV, cfg
    # rows narrower than a wave: 8, 16 or 32 lanes, one wave per row group,
    # one or two vectors per lane covering the row, whole waves per workgroup
    for cfg in [mbr.Config(mbr.PATH_VECTOR, 2, 1, 8, 0, 16), mbr.Config(mbr.PATH_VECTOR, 1, 3, 4, 0, 16),
                mbr.Config(mbr.PATH_VECTOR, 1, 1, 2, 0, 16), mbr.Config(mbr.PATH_VECTOR, 1, 1, 64, 0, 16),
                mbr.Config(mbr.PATH_VECTOR, 1, 1, 8, 0, 12), mbr.Config(mbr.PATH_ELEMENT, 1, 1, 4, 0, 16),
                mbr.Config(mbr.PATH_VECTOR, 1, 1, 8, 0, 8), mbr.Config(mbr.PATH_TWO_PASS, 1, 0, 1, 0, 32)]:
        n = mbr.rmsnorm_bwd_workspace_size(rows, 128, torch.bfloat16, cfg)
        st = L.rmsnorm_bwd_ex(X, W, G, D, DW, rows, 128, 1e-5, 1, WS, n, ctypes.byref(cfg), None)
        assert st == INV, cfg.as_dict()
    # slots combine dweight in LDS (hidden * 4 bytes, at most 159 KiB): every
    # built multi-slot configuration fits (512 lanes of at most 8 vectors: 64 KiB)
    # vector path on an unaligned buffer
    cfg = mbr.Config(mbr.PATH_VECTOR, 8, 1, 1, 0)
    st = L.rmsnorm_bwd_ex(X + 2, W, G, D, None, rows, hidden, 1e-5, 1, None, 0, ctypes.byref(cfg), None)
    assert st == INV


def test_noalloc_argument_errors_before_any_hip_call():
    """rmsnorm_bwd_noalloc rejects bad sizes, null or overlapping pointers and a
    hidden size whose one partial dweight row would not fit its 16 MiB scratch
    array, all before its first HIP call (here there is no GPU: a HIP call
    would give RUNTIME, not INVALID_ARG)."""
    L = mbr.lib()
    INV = mbr.RMSNORM_ERR_INVALID_ARG
    base = 1 << 44
    assert L.rmsnorm_bwd_noalloc(None, None, None, None, None, 4, 64, 1e-5, 1, None) == INV
    assert L.rmsnorm_bwd_noalloc(base, base + (1 << 30), base + (2 << 30), base + (3 << 30), None, -1, 64, 1e-5, 1,
                                 None) == INV
    assert L.rmsnorm_bwd_noalloc(base, base + (1 << 30), base + (2 << 30), base + (3 << 30), None, 4, 64, 1e-5, 7,
                                 None) == mbr.RMSNORM_ERR_UNSUPPORTED_DTYPE
    # dx partially overlapping x
    assert L.rmsnorm_bwd_noalloc(base, base + (1 << 30), base + (2 << 30), base + 16, None, 4, 64, 1e-5, 1,
                                 None) == INV
    # one partial row of hidden 4194305 (round_up 4194368 floats) exceeds 16 MiB
    h = 4194305
    assert L.rmsnorm_bwd_noalloc(base, base + (1 << 36), base + (2 << 36), base + (3 << 36), base + (4 << 36), 2, h,
                                 1e-5, 0, None) == INV

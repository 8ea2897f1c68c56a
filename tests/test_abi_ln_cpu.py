"""C-ABI checks of the LayerNorm entry points that need no GPU."""
import pytest
import torch

import memory_bound_rmsnorm_amd as mbr
from tests.test_abi_cpu import HEADERS, _declared, fake_only
from tests import built

INV = mbr.RMSNORM_ERR_INVALID_ARG


def test_layernorm_declared():
    names = {n for h in HEADERS for n in _declared(h)}
    for n in ("layernorm_fwd", "layernorm_fwd_ex", "layernorm_select_config"):
        assert n in names


def test_rows_zero_needs_no_pointers():
    assert mbr.lib().layernorm_fwd(None, None, None, None, 0, 64, 1e-5, 1, None) == mbr.RMSNORM_OK


@pytest.mark.parametrize("rows,hidden,eps,dtype,want", [
    (-1, 16, 1e-5, 1, INV), (4, 0, 1e-5, 1, INV), (4, 2 ** 31, 1e-5, 1, INV), (4, 16, -1.0, 1, INV),
    (4, 16, float("nan"), 0, INV), (4, 16, 1e-5, 5, mbr.RMSNORM_ERR_UNSUPPORTED_DTYPE), (2 ** 62, 16, 1e-5, 1, INV),
])
def test_bad_sizes_rejected(rows, hidden, eps, dtype, want):
    assert mbr.lib().layernorm_fwd(None, None, None, None, rows, hidden, eps, dtype, None) == want


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("aligned", [True, False])
@pytest.mark.parametrize("rows", [1, 100, 2048, 4096, 100000])
def test_choice_is_built_and_covering(dtype, aligned, rows):
    v = 8 if dtype == torch.bfloat16 else 4
    for hidden in [1, 7, 8, 64, 100, 768, 1000, 2048, 4095, 4096, 5120, 8192, 16384, 32768, 32776, 65536, 131080]:
        c = mbr.layernorm_select_config(rows, hidden, dtype, aligned)
        lanes = c.lanes_per_row or 64 * c.waves_per_row
        assert c.waves_per_row in (1, 2, 4, 8, 16)
        assert c.max_blocks == (1024 if c.lanes_per_row and c.items_per_lane == 1 else 0)
        if c.lanes_per_row:  # rows narrower than a wave, several per wave, whole waves per workgroup
            assert c.path == mbr.PATH_VECTOR and c.lanes_per_row in (8, 16, 32) and c.waves_per_row == 1
            assert c.items_per_lane in (1, 2) and lanes * c.rows_per_block % 64 == 0
            assert lanes * c.rows_per_block <= 512 and not c.weight_lds
            assert rows >= 1024 and hidden // v <= 64
        elif c.weight_lds:  # gamma and beta (sized for both) in LDS, shared by the row slots
            assert c.path == mbr.PATH_VECTOR and (hidden // v) * 32 <= 60 * 1024
            assert c.rows_per_block >= 1 and lanes * c.rows_per_block <= 512
        else:
            assert c.rows_per_block == 1
        if c.path == mbr.PATH_VECTOR:
            assert aligned and hidden % v == 0 and lanes * c.items_per_lane >= hidden // v
            assert c.lanes_per_row or built.ln_vec(c.waves_per_row, c.items_per_lane)
        elif c.path == mbr.PATH_VECTOR_ANY:
            # any width of at least one vector, any element alignment
            assert not (aligned and hidden % v == 0) and hidden >= v
            assert lanes * c.items_per_lane >= hidden // v and c.rows_per_block == 1 and not c.weight_lds
            assert built.ln_any(c.waves_per_row, c.items_per_lane)
        elif c.path == mbr.PATH_ELEMENT:
            assert built.elem(c.waves_per_row, c.items_per_lane) and lanes * c.items_per_lane >= hidden
            assert hidden < v  # a row of at least one vector takes a vector path
        else:
            assert c.path == mbr.PATH_TWO_PASS and hidden > 8 * 1024


def test_stated_choices():
    # many rows of 512 vectors: 2 waves x 4 vectors, four row slots sharing gamma/beta in LDS
    c = mbr.layernorm_select_config(8192, 4096, torch.bfloat16, True)
    assert (c.path, c.waves_per_row, c.items_per_lane, c.rows_per_block, c.weight_lds) == (mbr.PATH_VECTOR, 2, 4, 4, 1)
    c = mbr.layernorm_select_config(4096, 8192, torch.bfloat16, True)
    assert (c.waves_per_row, c.items_per_lane, c.rows_per_block, c.weight_lds) == (4, 4, 2, 1)
    # one round of workgroups at 2048 rows of 1024 vectors
    c = mbr.layernorm_select_config(2048, 8192, torch.bfloat16, True)
    assert (c.waves_per_row, c.items_per_lane, c.rows_per_block, c.weight_lds) == (2, 8, 4, 1)
    # narrower rows keep one row per workgroup and per-row gamma/beta loads
    c = mbr.layernorm_select_config(8192, 2048, torch.bfloat16, True)
    assert (c.waves_per_row, c.items_per_lane, c.rows_per_block, c.weight_lds) == (1, 4, 1, 0)
    c = mbr.layernorm_select_config(64, 768, torch.float32, True)
    assert (c.path, c.waves_per_row, c.items_per_lane) == (mbr.PATH_VECTOR, 2, 2)  # few rows: spread
    # narrow rows: lane groups of 8, 16 or 32 with at most two vectors per lane
    for rows, hidden, dt, want in [(262144, 128, torch.bfloat16, (8, 2, 32, 0)),
                                   (262144, 64, torch.bfloat16, (8, 1, 64, 1024)),
                                   (131072, 256, torch.bfloat16, (16, 2, 16, 0)),
                                   (65536, 512, torch.bfloat16, (32, 2, 8, 0)),
                                   (131072, 128, torch.float32, (16, 2, 16, 0)),
                                   (4096, 128, torch.bfloat16, (8, 2, 16, 0)), (1024, 128, torch.bfloat16, (8, 2, 8, 0))]:
        c = mbr.layernorm_select_config(rows, hidden, dt, True)
        assert (c.path, c.waves_per_row, c.weight_lds) == (mbr.PATH_VECTOR, 1, 0), (rows, hidden)
        assert (c.lanes_per_row, c.items_per_lane, c.rows_per_block, c.max_blocks) == want, (rows, hidden)
    assert mbr.layernorm_select_config(1023, 128, torch.bfloat16, True).lanes_per_row == 0


@fake_only
def test_pointer_validation_and_forced_configs():
    L = mbr.lib()
    X, G, B, O = (0x7F0000000000 + i * 0x10000000 for i in range(4))
    for args in [(None, G, B, O), (X, None, B, O), (X, G, B, None), (X + 1, G, B, O), (X, G, B + 1, O),
                 (X, G, B, X + 2), (X, G, B, G), (X, G, B, B - 16)]:
        assert L.layernorm_fwd(*args, 4, 256, 1e-5, 1, None) == INV, args
    for cfg in [mbr.Config(mbr.PATH_VECTOR, 3, 2, 1, 0), mbr.Config(mbr.PATH_VECTOR, 4, 2, 4, 0),
                mbr.Config(mbr.PATH_VECTOR, 16, 5, 1, 0), mbr.Config(mbr.PATH_VECTOR, 1, 2, 1, 0),
                mbr.Config(mbr.PATH_ELEMENT, 4, 3, 1, 0), mbr.Config(mbr.PATH_VECTOR, 4, 2, 1, -1),
                mbr.Config(9, 4, 2, 1, 0), mbr.Config(mbr.PATH_VECTOR, 1, 1, 1, 0, 32),
                mbr.Config(mbr.PATH_VECTOR, 4, 2, 0, 0),            # no row slots
                mbr.Config(mbr.PATH_VECTOR, 4, 2, 2, 0),            # row slots need the LDS copy
                mbr.Config(mbr.PATH_VECTOR, 4, 2, 2, 0, 0, 2),      # weight_lds is 0 or 1
                mbr.Config(mbr.PATH_ELEMENT, 4, 16, 2, 0),          # row slots: vector path only
                mbr.Config(mbr.PATH_ELEMENT, 4, 16, 1, 0, 0, 1),    # so is the LDS copy
                mbr.Config(mbr.PATH_TWO_PASS, 16, 0, 1, 0, 0, 1)]:
        import ctypes
        assert L.layernorm_fwd_ex(X, G, B, O, 4, 4096, 1e-5, 1, ctypes.byref(cfg), None) == INV, cfg
    # rows narrower than a wave (hidden 128 bf16: 16 vectors)
    for cfg in [mbr.Config(mbr.PATH_VECTOR, 2, 1, 8, 0, 16), mbr.Config(mbr.PATH_VECTOR, 1, 3, 4, 0, 16),
                mbr.Config(mbr.PATH_VECTOR, 1, 1, 2, 0, 16), mbr.Config(mbr.PATH_VECTOR, 1, 1, 64, 0, 16),
                mbr.Config(mbr.PATH_VECTOR, 1, 1, 8, 0, 12), mbr.Config(mbr.PATH_ELEMENT, 1, 1, 4, 0, 16),
                mbr.Config(mbr.PATH_VECTOR, 1, 1, 8, 0, 8), mbr.Config(mbr.PATH_VECTOR, 1, 1, 4, 0, 16, 1),
                mbr.Config(mbr.PATH_TWO_PASS, 1, 0, 1, 0, 32)]:
        assert L.layernorm_fwd_ex(X, G, B, O, 4, 128, 1e-5, 1, ctypes.byref(cfg), None) == INV, cfg.as_dict()
    # gamma and beta in LDS (at most 159 KiB together): every built vector
    # configuration fits (1024 lanes x 4 vectors x 2 = 128 KiB)

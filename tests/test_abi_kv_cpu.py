"""C-ABI checks of kv_rmsnorm_rope_cache that need no GPU."""
import pytest
import torch

import memory_bound_rmsnorm_amd as mbr
from tests.test_abi_cpu import HEADERS, _declared, fake_only

INV = mbr.RMSNORM_ERR_INVALID_ARG


def _call(kv=1 << 40, g=2 << 40, c=3 << 40, s=4 << 40, p=5 << 40, sl=6 << 40, nc=7 << 40, rc=8 << 40, tokens=4,
          heads=1, dn=512, dr=64, max_pos=16, num_slots=32, eps=1e-6, style=1, dtype=1):
    return mbr.lib().kv_rmsnorm_rope_cache(kv, g, c, s, p, sl, nc, rc, tokens, heads, dn, dr, max_pos, num_slots,
                                           eps, style, dtype, None)


def test_declared():
    assert "kv_rmsnorm_rope_cache" in {n for h in HEADERS for n in _declared(h)}


def test_zero_tokens_needs_no_pointers():
    assert _call(kv=None, g=None, c=None, s=None, p=None, sl=None, nc=None, rc=None, tokens=0) == mbr.RMSNORM_OK


@pytest.mark.parametrize("kw,want", [
    (dict(tokens=-1), INV), (dict(heads=0), INV), (dict(dn=0), INV), (dict(dr=-2), INV), (dict(dr=3), INV),
    (dict(max_pos=-1), INV), (dict(num_slots=-1), INV), (dict(eps=-1.0), INV), (dict(eps=float("nan")), INV),
    (dict(style=2), INV), (dict(dtype=7), mbr.RMSNORM_ERR_UNSUPPORTED_DTYPE), (dict(tokens=1 << 60), INV),
    (dict(num_slots=1 << 60), INV),
])
def test_bad_sizes_rejected(kw, want):
    args = dict(kv=None, g=None, c=None, s=None, p=None, sl=None, nc=None, rc=None)
    args.update(kw)
    assert _call(**args) == want


@fake_only
def test_pointer_validation():
    for kw in [dict(kv=None), dict(g=None), dict(p=None), dict(sl=None), dict(nc=None), dict(rc=None),
               dict(c=None), dict(s=None), dict(kv=(1 << 40) + 1), dict(p=(5 << 40) + 2), dict(sl=(6 << 40) + 4),
               dict(c=(3 << 40) + 2), dict(nc=1 << 40), dict(rc=(1 << 40) + 64), dict(nc=8 << 40),
               dict(rc=(7 << 40) + 1024), dict(nc=(6 << 40) - 64)]:
        assert _call(**kw) == INV, kw


def _call_ex(cfg, dn=512, dr=64, style=1, dtype=1, kv=1 << 40):
    import ctypes
    return mbr.lib().kv_rmsnorm_rope_cache_ex(kv, 2 << 40, 3 << 40, 4 << 40, 5 << 40, 6 << 40, 7 << 40, 8 << 40,
                                              4, 1, dn, dr, 16, 32, 1e-6, style, dtype,
                                              ctypes.byref(cfg) if cfg is not None else None, None)


def test_ex_and_select_declared():
    names = {n for h in HEADERS for n in _declared(h)}
    assert {"kv_rmsnorm_rope_cache_ex", "kv_select_config"} <= names


def test_select_config():
    # the stated shape: two rows per wave, 32 lanes x 2 norm vectors each
    c = mbr.kv_select_config(16384, 1, 512, 64, mbr.ROPE_PAIRS, torch.bfloat16, True)
    assert (c.path, c.items_per_lane, c.waves_per_row, c.rows_per_block, c.max_blocks) == (mbr.PATH_VECTOR, 2, 1, 1, 0)
    assert c.lanes_per_row == 32
    # narrower heads take smaller lane groups; the rotated part must fit them
    for dn, dr, style, want in [(128, 64, 1, (8, 2)), (256, 64, 1, (16, 2)), (64, 64, 1, (8, 1)),
                                (128, 256, 1, (32, 1)), (128, 256, 0, (16, 1)), (1024, 64, 1, (0, 2)),
                                (4096, 64, 1, (0, 8))]:
        c = mbr.kv_select_config(64, 4, dn, dr, style, torch.bfloat16, True)
        assert (c.lanes_per_row, c.items_per_lane) == want, (dn, dr, style, c.as_dict())
    # unaligned buffers, a split that breaks a vector, or a wide rotated part: the element kernel
    assert mbr.kv_select_config(16, 1, 512, 64, 1, torch.bfloat16, False).path == mbr.PATH_ELEMENT
    assert mbr.kv_select_config(16, 1, 100, 30, 1, torch.bfloat16, True).path == mbr.PATH_ELEMENT
    assert mbr.kv_select_config(16, 1, 512, 1040, 1, torch.bfloat16, True).path == mbr.PATH_ELEMENT
    for dn in (8, 64, 512, 1024, 2048):  # fp32: up to 8 norm vectors per lane
        c = mbr.kv_select_config(4096, 2, dn, 64, 0, torch.float32, True)
        lanes = c.lanes_per_row or 64
        assert c.path == mbr.PATH_VECTOR and lanes * c.items_per_lane >= dn // 4
    with pytest.raises(mbr.RmsnormError):
        mbr.kv_select_config(16, 0, 512, 64, 1, torch.bfloat16, True)
    import ctypes
    assert mbr.lib().kv_select_config(16, 1, 512, 64, 1, 1, 1, None) == INV


@fake_only
def test_ex_bad_configs():
    V = mbr.PATH_VECTOR
    for cfg in [mbr.Config(V, 2, 1, 1, 0), mbr.Config(V, 1, 1, 2, 0), mbr.Config(V, 1, 1, 1, 3),
                mbr.Config(V, 1, 1, 1, 0, 0, 1), mbr.Config(V, 1, 3, 1, 0), mbr.Config(V, 1, 16, 1, 0),
                mbr.Config(V, 1, 2, 1, 0, 8), mbr.Config(V, 1, 4, 1, 0, 16), mbr.Config(V, 1, 1, 1, 0, 32),
                mbr.Config(V, 1, 2, 1, 0, 16),            # 16 lanes x 2 vectors cannot hold 64
                mbr.Config(mbr.PATH_ELEMENT, 1, 0, 1, 0, 32), mbr.Config(mbr.PATH_TWO_PASS, 1, 0, 1, 0),
                mbr.Config(9, 1, 1, 1, 0)]:
        assert _call_ex(cfg) == INV, cfg.as_dict()
    # the rotated part must fit the row's lanes: 40 rope lanes against 32
    assert _call_ex(mbr.Config(V, 1, 2, 1, 0, 32), dn=256, dr=320) == INV
    # vectors on unaligned buffers, or a shape that breaks them
    assert _call_ex(mbr.Config(V, 1, 1, 1, 0), kv=(1 << 40) + 2) == INV
    assert _call_ex(mbr.Config(V, 1, 8, 1, 0), dn=100, dr=30) == INV

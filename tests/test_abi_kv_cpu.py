"""C-ABI checks of kv_rmsnorm_rope_cache that need no GPU."""
import pytest

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

"""The launch configurations the library builds, per kernel family, as the
dispatch tables in rmsnorm_dispatch.hpp define them.  tests/test_built_cpu.py
checks this mirror against the library itself (forced configurations are
rejected exactly when they are not built)."""

WPR = (1, 2, 4, 8, 16)
VEC_VPL = (1, 2, 3, 4, 5, 6, 7, 8, 10)   # forward vector path
ANY_VPL = tuple(range(1, 9))             # any-alignment path (every family)
EPL = (1, 2, 4, 8, 16)                   # forward element path
BWD_VPL = tuple(range(1, 9))
BWD_EPL = (1, 2, 4, 8)
LN_VPL = tuple(range(1, 9))
LN_EPL = (1, 2, 4, 8)


def vec(wpr, vpl, fused):
    """Forward vector path, plain or fused."""
    if vpl not in VEC_VPL:
        return False
    return vpl <= ((5 if wpr < 16 else 6) if fused else (8 if wpr < 16 else 10))


def qvec(wpr, vpl):
    """Quantised forward, vector path (plain or fused)."""
    return vpl in VEC_VPL and vpl <= (5 if wpr < 16 else 4)


def any_(wpr, vpl, fused):
    return vpl in ANY_VPL and vpl <= (5 if wpr < 16 else 4 if fused else 6)


def qany(wpr, vpl):
    return vpl in ANY_VPL and vpl <= (5 if wpr < 16 else 4)


def elem(wpr, epl):
    """Every element-path family: rows narrower than one vector only."""
    return wpr == 1 and epl == 1


def bwd_vec(wpr, vpl):
    return vpl in BWD_VPL and vpl <= (8 if wpr == 1 else 6 if wpr < 16 else 4)


def bwd_any(wpr, vpl):
    return vpl in BWD_VPL and vpl <= (6 if wpr < 16 else 3)


def ln_vec(wpr, vpl):
    return vpl in LN_VPL and (wpr < 16 or vpl <= 4)


def ln_any(wpr, vpl):
    return vpl in ANY_VPL and (wpr < 16 or vpl <= 3)

"""Seeded random shapes through every entry point's automatic choice: rows,
widths (whole 16-byte vectors or not), dtypes and forms drawn from one fixed
generator, each compared with the oracle under the same bounds as the
dedicated suites.  A wide net over the launch-configuration rules."""
import os

import numpy as np
import pytest
import torch

import memory_bound_rmsnorm_amd as mbr
from memory_bound_rmsnorm_amd import inputs
from tests import parity
from tests.test_bwd_gpu import check as check_bwd
from tests.test_ln_gpu import check as check_ln
from tests.test_parity_gpu import check_workload
from tests.test_quant_gpu import QT, check as check_quant

pytestmark = pytest.mark.gpu

# A wider net on demand: RMSNORM_RANDOM_CASES=N (shape cases; a third as many
# offset cases) and RMSNORM_RANDOM_SEED=S replace the defaults below.
_N = int(os.environ.get("RMSNORM_RANDOM_CASES", "0"))
_SEED = int(os.environ.get("RMSNORM_RANDOM_SEED", "0"))


def _cases(n=240, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = "bf16" if rng.random() < 0.7 else "f32"
        v = 8 if dtype == "bf16" else 4
        r = rng.random()
        if r < 0.35:
            hidden = int(rng.integers(1, 65)) * v          # narrow, whole vectors
        elif r < 0.75:
            hidden = int(rng.integers(9, 1200)) * v        # wide, whole vectors
        else:
            hidden = int(rng.integers(1, 9000))            # any width
        rows = int(rng.integers(1, max(2, min(6000, 2_000_000 // hidden))))
        kind = ["fwd", "fused", "int8", "fp8", "bwd", "ln"][i % 6]
        out.append((i, kind, dtype, rows, hidden))
    return out


@pytest.mark.parametrize("i,kind,dtype,rows,hidden", _cases(_N or 240, _SEED or 20261202))
def test_random_shape(i, kind, dtype, rows, hidden):
    print("random case", i, kind, dtype, rows, hidden, flush=True)
    if kind in ("fwd", "fused"):
        w = inputs.custom(rows, hidden, dtype, kind == "fused")
        check_workload(w, inputs.make(w, seed=i))
    elif kind in ("int8", "fp8"):
        w = inputs.custom(rows, hidden, dtype, i % 4 == 0)
        check_quant(w, inputs.make(w, seed=i), QT[kind])
    elif kind == "bwd":
        w = inputs.custom(rows, hidden, dtype, backward=True)
        check_bwd(w, inputs.make(w, seed=i), want_dw=i % 5 != 0)
    else:
        w = inputs.custom(rows, hidden, dtype, layernorm=True)
        check_ln(w, inputs.make(w, seed=i), bias=i % 3 != 0)


def _offset_cases(n=72, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        hidden = int(rng.integers(8, 9000))
        rows = int(rng.integers(1, max(2, min(3000, 1_000_000 // hidden))))
        offs = tuple(int(o) for o in rng.integers(0, 8, 4))
        if rng.random() < 0.5:  # x, residual, h and out at one offset modulo 4 bytes: the shifted frame applies
            offs = tuple((offs[0] % 2) + 2 * (o // 2) for o in offs)
        kind = ["fwd", "fused", "int8", "fp8"][i % 4]
        out.append((i, kind, rows, hidden, offs, rng.random() < 0.2))
    return out


@pytest.mark.parametrize("i,kind,rows,hidden,offs,inplace",
                         _offset_cases(_N // 3 or 72, _SEED + 1 if _SEED else 20261203))
def test_random_offsets(i, kind, rows, hidden, offs, inplace):
    """bf16 rows of random widths with x, residual, h and out (or the codes)
    at random element offsets past a 16-byte boundary, through the automatic
    choice: half of the cases put every row tensor at one offset modulo 4
    bytes, where rows 2 bytes past a 4-byte boundary take the shifted frame."""
    from tests.test_parity_gpu import _run_any_offsets
    from tests.test_quant_gpu import _run_any_quant
    print("random offsets case", i, kind, rows, hidden, offs, inplace, flush=True)
    if kind in ("fwd", "fused"):
        _run_any_offsets(rows, hidden, kind == "fused", offs, inplace=inplace, seed=9000 + i)
    else:
        cfg = mbr.rmsnorm_select_quant_config(rows, hidden, torch.bfloat16, False, i % 8 == 2)
        _run_any_quant("bf16", rows, hidden, i % 8 == 2, QT[kind], cfg, offs[0], offs[3], 9000 + i)

"""C-ABI checks that need no GPU: the libraries load, export what the headers
declare, reject bad arguments before touching HIP, and choose only built,
spill-free configurations."""
import ctypes
import glob
import os
import re

import pytest
import torch

import memory_bound_rmsnorm_amd as mbr
from memory_bound_rmsnorm_amd import _build, inputs
from tests import built

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))
NO_GPU = not torch.cuda.is_available()
# Fake addresses are only ever passed where validation must reject the call;
# they are used only where no GPU is visible, so a validation bug cannot turn
# into a kernel launch on bogus memory.
fake_only = pytest.mark.skipif(not NO_GPU, reason="fake device addresses are only used without a GPU")


def _built():
    if not (os.path.exists(_build.LIB_RMSNORM) and os.path.exists(_build.LIB_COPY)
            and os.path.exists(_build.RESOURCE_USAGE)):
        _build.build()


def _declared(header):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"(?:RMSNORM_API|HBM_COPY_API)\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def test_headers_declare_the_boundary():
    names = {n for h in HEADERS for n in _declared(h)}
    for n in ("rmsnorm_fwd", "rmsnorm_residual_fwd", "rmsnorm_status_string", "rmsnorm_select_config",
              "rmsnorm_fwd_ex", "rmsnorm_residual_fwd_ex", "hbm_copy"):
        assert n in names


def test_libraries_export_every_declared_symbol():
    _built()
    libs = {"rmsnorm.h": ctypes.CDLL(_build.LIB_RMSNORM), "hbm_copy.h": ctypes.CDLL(_build.LIB_COPY)}
    for h in HEADERS:
        L = libs[os.path.basename(h)]
        for name in _declared(h):
            assert hasattr(L, name), "%s does not export %s" % (os.path.basename(h), name)


def test_no_internal_symbols_exported():
    _built()
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", _build.LIB_RMSNORM], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    declared = {n for h in HEADERS for n in _declared(h)}
    assert exported <= declared | {"_init", "_fini"}, exported - declared


def test_every_built_kernel_is_spill_free():
    _built()
    lines = open(_build.RESOURCE_USAGE).read().strip().splitlines()
    assert len(lines) > 400
    for l in lines:
        assert "| scratch 0 |" in l and "VGPR spill 0" in l and "SGPR spill 0" in l, l


def test_status_strings():
    for s in range(4):
        assert mbr.rmsnorm_status_string(s).startswith(
            ["RMSNORM_OK", "RMSNORM_ERR_INVALID_ARG", "RMSNORM_ERR_UNSUPPORTED_DTYPE", "RMSNORM_ERR_RUNTIME"][s])
    assert mbr.rmsnorm_status_string(99) == "unknown rmsnorm status"


def test_rows_zero_is_ok_without_pointers():
    L = mbr.lib()
    assert L.rmsnorm_fwd(None, None, None, 0, 16, 1e-5, 1, None) == mbr.RMSNORM_OK
    assert L.rmsnorm_residual_fwd(None, None, None, None, None, 0, 16, 1e-5, 0, None) == mbr.RMSNORM_OK


@pytest.mark.parametrize("rows,hidden,eps,dtype,want", [
    (-1, 16, 1e-5, 1, mbr.RMSNORM_ERR_INVALID_ARG),
    (4, 0, 1e-5, 1, mbr.RMSNORM_ERR_INVALID_ARG),
    (4, -8, 1e-5, 1, mbr.RMSNORM_ERR_INVALID_ARG),
    (4, 2 ** 31, 1e-5, 1, mbr.RMSNORM_ERR_INVALID_ARG),
    (4, 16, -1e-5, 1, mbr.RMSNORM_ERR_INVALID_ARG),
    (4, 16, float("nan"), 1, mbr.RMSNORM_ERR_INVALID_ARG),
    (4, 16, float("inf"), 1, mbr.RMSNORM_ERR_INVALID_ARG),
    (4, 16, 1e-5, 2, mbr.RMSNORM_ERR_UNSUPPORTED_DTYPE),
    (4, 16, 1e-5, -1, mbr.RMSNORM_ERR_UNSUPPORTED_DTYPE),
    (2 ** 62, 16, 1e-5, 1, mbr.RMSNORM_ERR_INVALID_ARG),
])
def test_bad_sizes_rejected_before_any_pointer_use(rows, hidden, eps, dtype, want):
    L = mbr.lib()
    assert L.rmsnorm_fwd(None, None, None, rows, hidden, eps, dtype, None) == want
    assert L.rmsnorm_residual_fwd(None, None, None, None, None, rows, hidden, eps, dtype, None) == want


@fake_only
def test_null_and_misaligned_pointers_rejected():
    L = mbr.lib()
    A, W, O = 0x7F0000000000, 0x7F0010000000, 0x7F0020000000
    INV = mbr.RMSNORM_ERR_INVALID_ARG
    assert L.rmsnorm_fwd(None, W, O, 4, 16, 1e-5, 1, None) == INV
    assert L.rmsnorm_fwd(A, None, O, 4, 16, 1e-5, 1, None) == INV
    assert L.rmsnorm_fwd(A, W, None, 4, 16, 1e-5, 1, None) == INV
    assert L.rmsnorm_fwd(A + 1, W, O, 4, 16, 1e-5, 1, None) == INV  # bf16 needs 2-byte alignment
    assert L.rmsnorm_fwd(A + 2, W, O, 4, 16, 1e-5, 0, None) == INV  # f32 needs 4-byte alignment
    R, H = 0x7F0030000000, 0x7F0040000000
    assert L.rmsnorm_residual_fwd(A, None, W, H, O, 4, 16, 1e-5, 1, None) == INV
    assert L.rmsnorm_residual_fwd(A, R, W, None, O, 4, 16, 1e-5, 1, None) == INV


@fake_only
def test_overlaps_rejected():
    L = mbr.lib()
    INV = mbr.RMSNORM_ERR_INVALID_ARG
    A = 0x7F0000000000
    nb = 4 * 16 * 2
    W = 0x7F0010000000
    assert L.rmsnorm_fwd(A, W, A + 32, 4, 16, 1e-5, 1, None) == INV       # out partially over x
    assert L.rmsnorm_fwd(A, W, W - 64, 4, 16, 1e-5, 1, None) == INV       # out over weight
    X, R, H, O = A, A + 0x100000, A + 0x200000, A + 0x300000
    assert L.rmsnorm_residual_fwd(X, R, W, H, H, 4, 16, 1e-5, 1, None) == INV     # out == residual_out
    assert L.rmsnorm_residual_fwd(X, R, W, H, H + 2, 4, 16, 1e-5, 1, None) == INV
    assert L.rmsnorm_residual_fwd(X, R, W, R + 2, O, 4, 16, 1e-5, 1, None) == INV  # h partially over residual
    assert L.rmsnorm_residual_fwd(X, R, W, H, X + nb - 2, 4, 16, 1e-5, 1, None) == INV
    assert L.rmsnorm_residual_fwd(X, R, W, W, O, 4, 16, 1e-5, 1, None) == INV       # h over weight


@fake_only
def test_bad_forced_configs_rejected():
    L = mbr.lib()
    INV = mbr.RMSNORM_ERR_INVALID_ARG
    A, W, O = 0x7F0000000000, 0x7F0010000000, 0x7F0020000000

    def call(path, wpr, per, rpb, hidden=2048, x=A, mb=0):
        cfg = mbr.Config(path, wpr, per, rpb, mb)
        return L.rmsnorm_fwd_ex(x, W, O, 8, hidden, 1e-5, 1, ctypes.byref(cfg), None)

    assert call(1, 3, 4, 1) == INV            # waves per row not built
    assert call(1, 1, 9, 1) == INV            # vectors per lane not built
    assert call(1, 1, 2, 1) == INV            # 64 lanes x 2 vectors do not cover 256 vectors
    assert call(1, 1, 4, 16) == INV           # 1024 lanes with a 512-lane bound
    assert call(1, 16, 16, 1, hidden=2048 * 64) == INV  # not built (would spill)
    assert call(1, 1, 4, 1, x=A + 2) == INV   # vector path needs 16-byte alignment
    assert call(1, 1, 4, 1, hidden=2044) == INV  # hidden * 2 not a multiple of 16
    assert call(2, 1, 16, 1, hidden=2048) == INV  # 64 x 16 elements do not cover 2048
    assert call(3, 16, 0, 2) == INV           # two-pass takes one row per workgroup
    assert call(7, 1, 4, 1) == INV            # unknown path
    assert call(1, 1, 4, 0) == INV            # zero rows per block
    assert call(1, 1, 4, 1, mb=-1) == INV
    # any-alignment vectors: whole-wave rows, one row per workgroup, vectors covering the full ones
    assert call(4, 1, 2, 1, hidden=2049) == INV   # 64 x 2 vectors do not cover 256
    assert call(4, 1, 9, 1, hidden=2049) == INV   # vectors per lane not built
    assert call(4, 1, 4, 2, hidden=2049) == INV   # one row per workgroup
    assert call(4, 16, 8, 1, hidden=65537) == INV  # not built (would spill)
    assert call(4, 1, 1, 1, hidden=7) == INV      # no full vector: the element path
    cfg = mbr.Config(4, 1, 4, 1, 0, 0, 1)           # no LDS weight on this path
    assert L.rmsnorm_fwd_ex(A + 2, W, O, 8, 2049, 1e-5, 1, ctypes.byref(cfg), None) == INV
    cfg = mbr.Config(4, 1, 4, 1, 0, 16)             # nor rows sharing a wave
    assert L.rmsnorm_fwd_ex(A + 2, W, O, 8, 2049, 1e-5, 1, ctypes.byref(cfg), None) == INV
    cfg = mbr.Config(4, 16, 5, 1, 0)                # quantised forms: at most 4 vectors at 16 waves
    assert L.rmsnorm_dynamic_quant_fwd_ex(A, None, W, None, O, 0x7F0030000000, 8, 16 * 64 * 5 * 8 - 3, 1e-5, 1, 0,
                                          ctypes.byref(cfg), None) == INV
    cfg = mbr.Config(4, 1, 4, 2, 0)                 # and one row per workgroup
    assert L.rmsnorm_dynamic_quant_fwd_ex(A, None, W, None, O, 0x7F0030000000, 8, 2049, 1e-5, 1, 0,
                                          ctypes.byref(cfg), None) == INV

    def sub(lpr, wpr, per, rpb, hidden=128, path=1):
        cfg = mbr.Config(path, wpr, per, rpb, 0, lpr)
        return L.rmsnorm_fwd_ex(A, W, O, 8, hidden, 1e-5, 1, ctypes.byref(cfg), None)

    assert sub(12, 1, 1, 16) == INV           # lanes per row not built
    assert sub(16, 2, 1, 8) == INV            # several rows per wave need waves_per_row 1
    assert sub(16, 1, 3, 16) == INV           # 1 or 2 vectors per lane only
    assert sub(8, 1, 1, 8) == INV             # 8 lanes x 1 vector do not cover 16 vectors
    assert sub(16, 1, 1, 3) == INV            # 48 lanes: not whole waves
    assert sub(16, 1, 1, 64) == INV           # 1024 lanes over the 512-lane bound
    assert sub(16, 1, 1, 4, path=2) == INV    # element path has whole-wave rows only
    assert sub(16, 1, 1, 4, path=3) == INV    # so has the two-pass path

    def lds(path, wpr, per, rpb, flag=1, hidden=2048, lpr=0):
        cfg = mbr.Config(path, wpr, per, rpb, 0, lpr, flag)
        return L.rmsnorm_fwd_ex(A, W, O, 8, hidden, 1e-5, 1, ctypes.byref(cfg), None)

    assert lds(1, 2, 1, 2, flag=2) == INV                # weight_lds is 0 or 1
    assert lds(2, 4, 8, 1) == INV                        # element path: no staged weight
    assert lds(3, 16, 0, 1) == INV                       # nor the two-pass path
    assert lds(1, 1, 1, 8, hidden=128, lpr=16) == INV    # nor rows sharing a wave
    assert lds(1, 16, 10, 1, hidden=81920) == INV        # 160 KiB of weight: over the 159 KiB bound
    # the quantised forms take a staged weight on the vector path only; the
    # backward entry point takes none
    cfg = mbr.Config(2, 4, 8, 1, 0, 0, 1)
    Q, S = 0x7F0030000000, 0x7F0040000000
    assert L.rmsnorm_dynamic_quant_fwd_ex(A, None, W, None, Q, S, 8, 2048, 1e-5, 1, 0, ctypes.byref(cfg),
                                          None) == INV
    G, D = 0x7F0050000000, 0x7F0060000000
    assert L.rmsnorm_bwd_ex(A, W, G, D, None, 8, 2048, 1e-5, 1, None, 0, ctypes.byref(mbr.Config(1, 4, 1, 1, 0, 0, 1)),
                            None) == INV


@pytest.mark.parametrize("name", list(inputs.WORKLOADS))
def test_selection_for_the_workloads(name):
    w = inputs.WORKLOADS[name]
    cfg = mbr.rmsnorm_select_config(w.rows, w.hidden, torch.float32 if w.dtype == "f32" else torch.bfloat16,
                                    True, w.fused)
    assert cfg.path == mbr.PATH_VECTOR
    vec = 4 if w.dtype == "f32" else 8
    assert 64 * cfg.waves_per_row * cfg.items_per_lane >= w.hidden // vec
    assert 64 * cfg.waves_per_row * cfg.rows_per_block <= (1024 if cfg.waves_per_row == 16 else 512)
    # one GPU's share of the token-split headline fits one residency round:
    # four rows per workgroup share an LDS copy of the weight
    assert cfg.weight_lds == (1 if name == "bf16_shard_2048x8192" else 0)


@pytest.mark.parametrize("hidden", [1, 3, 7, 8, 9, 64, 96, 127, 128, 256, 264, 769, 2048, 4095, 5120, 5121, 8192,
                                    8193, 16384, 65536, 81920, 131072, 1 << 20])
@pytest.mark.parametrize("rows", [1, 5, 4096, 12289])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("aligned", [True, False])
@pytest.mark.parametrize("fused", [False, True])
def test_selection_is_always_a_built_covering_config(hidden, rows, dtype, aligned, fused):
    cfg = mbr.rmsnorm_select_config(rows, hidden, dtype, aligned, fused)
    vec = 4 if dtype == torch.float32 else 8
    assert cfg.waves_per_row in (1, 2, 4, 8, 16) and cfg.rows_per_block >= 1
    if cfg.lanes_per_row:  # several rows per wave
        lpr = cfg.lanes_per_row
        assert cfg.path == mbr.PATH_VECTOR and aligned and hidden % vec == 0 and hidden // vec <= 64
        assert lpr in (8, 16, 32) and cfg.waves_per_row == 1 and cfg.items_per_lane in (1, 2)
        assert lpr * cfg.items_per_lane >= hidden // vec > lpr * (cfg.items_per_lane - 1)
        assert (lpr * cfg.rows_per_block) % 64 == 0 and lpr * cfg.rows_per_block <= 128
        per_wave = 64 // lpr
        assert cfg.rows_per_block == per_wave or rows >= 256 * cfg.rows_per_block
        if not fused:  # plain rows of 64 vectors fill a whole wave exactly
            assert hidden // vec != 64
        return
    if cfg.path == mbr.PATH_VECTOR:
        assert aligned and hidden % vec == 0
        assert 64 * cfg.waves_per_row * cfg.items_per_lane >= hidden // vec
        assert built.vec(cfg.waves_per_row, cfg.items_per_lane, fused)
    elif cfg.path == mbr.PATH_VECTOR_ANY:
        # any width of at least one vector, any element alignment: full
        # vectors per lane, the rest as a tail of single elements
        assert not (aligned and hidden % vec == 0) and hidden >= vec
        assert 64 * cfg.waves_per_row * cfg.items_per_lane >= hidden // vec
        assert built.any_(cfg.waves_per_row, cfg.items_per_lane, fused)
        assert cfg.rows_per_block == 1 and cfg.max_blocks == 0
    elif cfg.path == mbr.PATH_ELEMENT:
        assert 64 * cfg.waves_per_row * cfg.items_per_lane >= hidden
        assert built.elem(cfg.waves_per_row, cfg.items_per_lane)
        assert hidden < vec  # a row of at least one vector takes a vector path
    elif cfg.path == mbr.PATH_VECTOR_LDS:
        # past the register path: 1024 lanes, a register part plus at least
        # one staged vector, the staged part within LDS
        assert aligned and hidden % vec == 0 and cfg.waves_per_row == 16 and cfg.rows_per_block == 1
        assert cfg.items_per_lane == (10 if not fused else cfg.items_per_lane) and cfg.items_per_lane in (6, 7, 10)
        staged = hidden // vec - 1024 * cfg.items_per_lane
        assert 1 <= staged and staged * 16 <= 160 * 1024 - 1024
        assert hidden // vec > 1024 * (6 if fused else 10)  # the register path cannot hold it
    else:
        assert cfg.path == mbr.PATH_TWO_PASS and cfg.rows_per_block == 1
        assert hidden > 8192  # everything narrower fits a register-resident path
        if aligned and hidden % vec == 0:  # aligned rows take two passes only past registers + LDS
            assert hidden // vec > 1024 * (7 if fused else 10) + (160 * 1024 - 1024) // 16
    assert 64 * cfg.waves_per_row * cfg.rows_per_block <= (1024 if cfg.waves_per_row == 16 else 512)
    assert cfg.rows_per_block <= max(rows, 1)
    if cfg.weight_lds:
        assert cfg.weight_lds == 1 and cfg.path == mbr.PATH_VECTOR and not fused and not cfg.lanes_per_row
        assert (hidden // vec) * 16 <= 159 * 1024


def test_narrow_row_choices():
    """Rows narrower than a wave: plain rows of up to 32 vectors take one
    vector per lane in the smallest lane group that holds them; fused and
    quantised rows of up to 64 vectors, and plain ones of 33..63, take at
    most two vectors per lane in the smallest lane group, two waves per
    workgroup from 256 workgroups on."""
    B = torch.bfloat16
    for rows, hidden, fused, want in [(262144, 128, False, (16, 1, 4)), (262144, 64, False, (8, 1, 8)),
                                      (131072, 256, False, (32, 1, 2)), (65536, 384, False, (32, 2, 4)),
                                      (262144, 128, True, (8, 2, 16)), (65536, 512, True, (32, 2, 4)),
                                      (65536, 256, True, (16, 2, 8)), (100, 128, True, (8, 2, 8))]:
        c = mbr.rmsnorm_select_config(rows, hidden, B, True, fused)
        assert (c.path, c.waves_per_row) == (mbr.PATH_VECTOR, 1)
        assert (c.lanes_per_row, c.items_per_lane, c.rows_per_block) == want, (rows, hidden, fused, c.as_dict())
    c = mbr.rmsnorm_select_config(65536, 512, B, True, False)
    assert (c.lanes_per_row, c.waves_per_row, c.items_per_lane) == (0, 1, 1)  # 64 vectors: a whole wave
    for fused in (False, True):  # the quantised forms (int8 and fp8 share the choice)
        c = mbr.rmsnorm_select_quant_config(262144, 128, B, True, fused)
        assert (c.lanes_per_row, c.items_per_lane, c.rows_per_block) == (8, 2, 16)
        c = mbr.rmsnorm_select_quant_config(65536, 512, B, True, fused)
        assert (c.lanes_per_row, c.items_per_lane, c.rows_per_block) == (32, 2, 4)


def test_hbm_copy_rejects_bad_arguments():
    L = mbr.copy_lib()
    assert L.hbm_copy(None, None, 0, 0, None) == 0
    assert L.hbm_copy(None, None, 64, 0, None) == 1
    assert L.hbm_copy(None, None, -1, 0, None) == 1
    if NO_GPU:
        A = 0x7F0000000000
        assert L.hbm_copy(A + 8, A + 0x1000000, 64, 0, None) == 1   # misaligned
        assert L.hbm_copy(A, A + 32, 64, 0, None) == 1              # overlap
        assert L.hbm_copy(A, A + 0x1000000, 64, -1, None) == 1


def test_binding_refuses_cpu_tensors():
    x = torch.zeros(4, 8)
    with pytest.raises(ValueError, match="GPU tensor"):
        mbr.rmsnorm_fwd(x, torch.ones(8), torch.empty_like(x))
    with pytest.raises(TypeError):
        mbr.dtype_code(torch.float16)


def test_quant_rows_zero_and_bad_qtype():
    L = mbr.lib()
    assert L.rmsnorm_dynamic_quant_fwd(None, None, None, None, None, None, 0, 16, 1e-5, 1, 0, None) == mbr.RMSNORM_OK
    assert L.rmsnorm_dynamic_quant_fwd(None, None, None, None, None, None, 4, 16, 1e-5, 1, 2, None) == \
        mbr.RMSNORM_ERR_UNSUPPORTED_DTYPE
    assert L.rmsnorm_dynamic_quant_fwd(None, None, None, None, None, None, -1, 16, 1e-5, 1, 7, None) == \
        mbr.RMSNORM_ERR_INVALID_ARG


@fake_only
def test_quant_argument_validation():
    L = mbr.lib()
    INV = mbr.RMSNORM_ERR_INVALID_ARG
    X, W, Q, S, R, H = (0x7F0000000000, 0x7F0010000000, 0x7F0020000000, 0x7F0030000000, 0x7F0040000000,
                        0x7F0050000000)

    def call(x=X, r=None, w=W, h=None, q=Q, s=S, rows=4, hidden=64, dt=1, qt=0):
        return L.rmsnorm_dynamic_quant_fwd(x, r, w, h, q, s, rows, hidden, 1e-5, dt, qt, None)

    assert call(r=R) == INV                 # residual without residual_out
    assert call(h=H) == INV                 # residual_out without residual
    assert call(q=None) == INV
    assert call(s=None) == INV
    assert call(s=S + 2) == INV             # scale needs 4-byte alignment
    assert call(q=X + 16) == INV            # codes over x
    assert call(q=W) == INV                 # codes over weight
    assert call(s=X + 8) == INV             # scales over x
    assert call(s=Q + 100) == INV           # scales over codes
    assert call(r=R, h=W) == INV            # h over weight
    assert call(r=R, h=R + 2) == INV        # h partially over residual
    assert call(r=R, h=Q) == INV            # h over codes


@pytest.mark.parametrize("hidden", [1, 7, 8, 2048, 4095, 5120, 8192, 8193, 16384, 32768, 65536])
@pytest.mark.parametrize("rows", [1, 5, 4096])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("fused", [False, True])
def test_quant_selection_is_always_built(hidden, rows, dtype, fused):
    cfg = mbr.rmsnorm_select_quant_config(rows, hidden, dtype, True, fused)
    if cfg.path == mbr.PATH_VECTOR:
        assert cfg.lanes_per_row or built.qvec(cfg.waves_per_row, cfg.items_per_lane)
        assert 64 * cfg.waves_per_row * cfg.items_per_lane * (4 if dtype == torch.float32 else 8) >= hidden
    elif cfg.path == mbr.PATH_VECTOR_ANY:
        v = 4 if dtype == torch.float32 else 8
        assert hidden % v != 0 and hidden >= v and cfg.rows_per_block == 1 and cfg.lanes_per_row == 0
        assert built.qany(cfg.waves_per_row, cfg.items_per_lane)
        assert 64 * cfg.waves_per_row * cfg.items_per_lane >= hidden // v
    elif cfg.path == mbr.PATH_ELEMENT:
        assert built.elem(cfg.waves_per_row, cfg.items_per_lane)
        assert 64 * cfg.waves_per_row * cfg.items_per_lane >= hidden
    else:
        assert cfg.path == mbr.PATH_TWO_PASS

"""Parity of the dynamic-quant HIP path (through the C ABI) with the oracle.

Codes must equal the oracle's except where Q*v*w/max|v*w| lies within float32
error of a tie between two codes (tests/parity.py::compare_quant); scales
within 1e-5 relative; the residual sum h bitwise."""
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
QT = {"int8": mbr.QUANT_INT8, "fp8": mbr.QUANT_FP8_E4M3}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_quant(t, qtype, eps, cfg=None, residual=True, h=None):
    x, w = t["x"].cuda(), t["weight"].cuda()
    q = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
    s = torch.empty(x.shape[0], dtype=torch.float32, device="cuda")
    r = t["residual"].cuda() if residual and "residual" in t else None
    hh = (torch.empty_like(x) if h is None else h) if r is not None else None
    mbr.rmsnorm_dynamic_quant_fwd_ex(x, w, q, s, eps, qtype, r, hh, cfg)
    torch.cuda.synchronize()
    return (hh.cpu() if hh is not None else None), q.cpu().numpy(), s.cpu().numpy()


def check(w, t, qtype, cfg=None, eps=None):
    eps = w.eps if eps is None else eps
    xb, wb = inputs.bits(t["x"]), inputs.bits(t["weight"])
    rb = inputs.bits(t["residual"]) if w.fused else None
    h_g, q_g, s_g = run_quant(t, qtype, eps, cfg)
    h_o, q_o, s_o = parity.oracle_quant(xb, wb, eps, qtype, residual=rb)
    if w.fused:
        assert np.array_equal(inputs.bits(h_g), h_o), "residual sum differs"
    v = h_o if w.fused else xb
    q_o_view = q_o.view(np.uint8) if qtype == 0 else q_o
    q_g_view = q_g.view(np.int8) if qtype == 0 else q_g
    return parity.compare_quant(q_g_view, q_o if qtype == 0 else q_o_view, s_g, s_o,
                                parity.quant_t(v, wb, qtype), qtype)


@pytest.mark.parametrize("q", ["int8", "fp8"])
@pytest.mark.parametrize("name", ["bf16_residual_12289x5120", inputs.HEADLINE, "bf16_prefill_4096x2048",
                                  "fp32_64x2048", "bf16_decode_256x4096"])
def test_stated_shapes_full_size(name, q):
    w = inputs.WORKLOADS[name]
    cfg = mbr.rmsnorm_select_quant_config(w.rows, w.hidden, BF16 if w.dtype == "bf16" else F32, True, w.fused)
    say("quant", q, name, cfg)
    say(check(w, inputs.make(w, seed=0), QT[q]))


RAGGED = [(1, 1), (3, 7), (5, 9), (67, 127), (12, 769), (5, 2048), (3, 4095), (7, 5120), (5, 5121), (3, 8193),
          (2, 20000), (2, 65536), (2, 131080)]


@pytest.mark.parametrize("q", ["int8", "fp8"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("rows,hidden", RAGGED)
def test_ragged_shapes(rows, hidden, dtype, fused, q):
    w = inputs.custom(rows, hidden, dtype, fused)
    say("quant", q, rows, hidden, dtype, fused)
    check(w, inputs.make(w, seed=rows + hidden), QT[q])


def _qconfigs(path):
    vec = path == mbr.PATH_VECTOR
    for wpr in built.WPR:
        for per in (built.VEC_VPL if vec else built.EPL):
            if built.qvec(wpr, per) if vec else built.elem(wpr, per):
                yield wpr, per


@pytest.mark.parametrize("q", ["int8", "fp8"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("fused", [False, True])
def test_every_quant_config(dtype, fused, q):
    vecw = 8 if dtype == "bf16" else 4
    n = 0
    for wpr, vpl in _qconfigs(mbr.PATH_VECTOR):
        lanes = 64 * wpr
        max_rpb = (1024 if wpr == 16 else 512) // lanes
        for nvec in sorted({lanes * vpl, max(1, lanes * vpl - 37)}):
            for rpb, mb in ((1, 0), (max_rpb, 0), (1, 2)):
                rows = 2 * rpb + 1
                cfg = mbr.Config(mbr.PATH_VECTOR, wpr, vpl, rpb, mb)
                w = inputs.custom(rows, nvec * vecw, dtype, fused)
                say("quant vector", q, dtype, fused, cfg, "hidden", nvec * vecw)
                check(w, inputs.make(w, seed=n), QT[q], cfg)
                n += 1
    for wpr, epl in _qconfigs(mbr.PATH_ELEMENT):
        for hidden in (3, 7, 59):
            cfg = mbr.Config(mbr.PATH_ELEMENT, wpr, epl, 1, 0)
            w = inputs.custom(3, hidden, dtype, fused)
            say("quant element", q, dtype, fused, cfg, "hidden", hidden)
            check(w, inputs.make(w, seed=n), QT[q], cfg)
            n += 1
    for wpr in (1, 4, 16):
        for hidden in (4096, 4099):
            cfg = mbr.Config(mbr.PATH_TWO_PASS, wpr, 0, 1, 0)
            w = inputs.custom(5, hidden, dtype, fused)
            say("quant two-pass", q, dtype, fused, cfg, "hidden", hidden)
            check(w, inputs.make(w, seed=n), QT[q], cfg)
            n += 1
    assert n > 100


@pytest.mark.parametrize("q", ["int8", "fp8"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("fused", [False, True])
def test_weight_in_lds_matches_bitwise(dtype, fused, q):
    """weight_lds = 1 on every built quantised vector configuration (the lanes
    fill their weight registers from the workgroup's LDS copy): one and the
    most row slots, full and masked rows, a capped grid.  Codes, scales and h
    bitwise equal to the global-weight kernel, and within the oracle's rule."""
    vecw = 8 if dtype == "bf16" else 4
    n = 0
    for wpr, vpl in _qconfigs(mbr.PATH_VECTOR):
        lanes = 64 * wpr
        max_rpb = (1024 if wpr == 16 else 512) // lanes
        for nvec in sorted({lanes * vpl, max(1, lanes * vpl - 37)}):
            if nvec * 16 > 159 * 1024:
                continue
            for rpb, mb in sorted({(1, 0), (max_rpb, 0), (max_rpb, 2)}):
                rows = 2 * rpb + 1
                w = inputs.custom(rows, nvec * vecw, dtype, fused)
                t = inputs.make(w, seed=900 + n)
                on = mbr.Config(mbr.PATH_VECTOR, wpr, vpl, rpb, mb, 0, 1)
                off = mbr.Config(mbr.PATH_VECTOR, wpr, vpl, rpb, mb, 0, 0)
                say("quant weight in LDS", q, dtype, fused, on, "hidden", nvec * vecw)
                a, b = run_quant(t, QT[q], w.eps, on), run_quant(t, QT[q], w.eps, off)
                assert np.array_equal(a[1], b[1]) and np.array_equal(a[2].view(np.uint32), b[2].view(np.uint32))
                if fused:
                    assert torch.equal(a[0], b[0])
                if n % 5 == 0:
                    check(w, t, QT[q], on)
                n += 1
    assert n > 40


@pytest.mark.parametrize("q", ["int8", "fp8"])
def test_zero_rows_and_degenerate(q):
    """A zero row gets scale 0 and zero codes; a row with one non-zero element
    maps it to full scale."""
    H = 2048
    x = torch.randn(4, H, generator=torch.Generator().manual_seed(3)).to(BF16)
    x[1] = 0
    x[2] = 0
    x[2, 77] = -2.5
    wt = (1 + 0.1 * torch.randn(H, generator=torch.Generator().manual_seed(4))).to(BF16)
    t = {"x": x, "weight": wt}
    w = inputs.custom(4, H, "bf16", False)
    check(w, t, QT[q])
    _, qq, ss = run_quant(t, QT[q], w.eps)
    assert ss[1] == 0 and np.all(qq[1] == 0)
    assert qq[2, 77] == (0x81 if q == "int8" else 0xFE) and np.sum(qq[2] != 0) == 1


@pytest.mark.parametrize("alias", ["x", "residual"])
def test_residual_out_aliases_an_input(alias):
    w = inputs.custom(129, 5120, "bf16", True)
    t = inputs.make(w, seed=9)
    want = parity.oracle_quant(inputs.bits(t["x"]), inputs.bits(t["weight"]), w.eps, 0,
                               residual=inputs.bits(t["residual"]))
    x, r, wt = t["x"].cuda(), t["residual"].cuda(), t["weight"].cuda()
    h = x if alias == "x" else r
    q = torch.empty(x.shape, dtype=torch.int8, device="cuda")
    s = torch.empty(129, dtype=torch.float32, device="cuda")
    mbr.rmsnorm_dynamic_quant_fwd(x, wt, q, s, w.eps, mbr.QUANT_INT8, r, h)
    torch.cuda.synchronize()
    assert np.array_equal(inputs.bits(h), want[0])
    parity.compare_quant(q.cpu().numpy(), want[1], s.cpu().numpy(), want[2],
                         parity.quant_t(want[0], inputs.bits(t["weight"]), 0), 0)


def test_quant_matches_plain_path_codes_are_deterministic():
    w = inputs.WORKLOADS["bf16_residual_12289x5120"]
    t = inputs.make(w, seed=0, rows=2000)
    a = run_quant(t, mbr.QUANT_FP8_E4M3, w.eps)
    b = run_quant(t, mbr.QUANT_FP8_E4M3, w.eps)
    assert np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2])
    # h of the quantised form equals h of the plain fused form bitwise
    x, r, wt = t["x"].cuda(), t["residual"].cuda(), t["weight"].cuda()
    h2, y2 = torch.empty_like(x), torch.empty_like(x)
    mbr.rmsnorm_residual_fwd(x, r, wt, h2, y2, w.eps)
    torch.cuda.synchronize()
    assert torch.equal(a[0], h2.cpu())


def test_quant_rejects_overlaps_on_device_buffers():
    x = torch.zeros(4, 256, dtype=BF16, device="cuda")
    wt = torch.ones(256, dtype=BF16, device="cuda")
    s = torch.zeros(4, dtype=torch.float32, device="cuda")
    L = mbr.lib()
    st = L.rmsnorm_dynamic_quant_fwd(x.data_ptr(), None, wt.data_ptr(), None, x.data_ptr() + 64, s.data_ptr(),
                                     4, 256, 1e-5, 1, 0, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == mbr.RMSNORM_ERR_INVALID_ARG and torch.count_nonzero(x) == 0


@pytest.mark.parametrize("q", ["int8", "fp8"])
@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("dtype,hidden", [("bf16", 64), ("bf16", 128), ("bf16", 200), ("bf16", 384), ("bf16", 512),
                                          ("f32", 96), ("f32", 256)])
def test_narrow_rows_automatic_quant(dtype, hidden, fused, q):
    """Per-head widths through the automatic choice: lane groups with up to
    two vectors per lane wherever the row is whole vectors."""
    rows = 20001
    cfg = mbr.rmsnorm_select_quant_config(rows, hidden, torch.bfloat16 if dtype == "bf16" else torch.float32,
                                          True, fused)
    vecw = 8 if dtype == "bf16" else 4
    if hidden % vecw == 0:
        assert cfg.lanes_per_row in (8, 16, 32) and cfg.items_per_lane in (1, 2)
    say("quant narrow", q, dtype, hidden, fused, cfg.as_dict())
    w = inputs.custom(rows, hidden, dtype, fused)
    check(w, inputs.make(w, seed=hidden + 7), QT[q])


@pytest.mark.parametrize("q", ["int8", "fp8"])
@pytest.mark.parametrize("fused", [False, True])
def test_every_subwave_quant_config(fused, q):
    """Quantised output with several rows per wave (lanes_per_row 8, 16, 32)."""
    n = 0
    for dtype, vecw in (("bf16", 8), ("f32", 4)):
        for lpr in (8, 16, 32):
            for vpl in (1, 2):
                for nvec, rpb in ((lpr * vpl, 64 // lpr), (max(1, lpr * vpl - 3), 512 // lpr)):
                    cfg = mbr.Config(mbr.PATH_VECTOR, 1, vpl, rpb, 0, lpr)
                    w = inputs.custom(2 * rpb + 3, nvec * vecw, dtype, fused)
                    say("quant subwave", q, dtype, fused, cfg, "hidden", nvec * vecw)
                    check(w, inputs.make(w, seed=n), QT[q], cfg)
                    n += 1
    assert n == 24


@pytest.mark.parametrize("q", ["int8", "fp8"])
def test_non_finite_rows_stay_in_their_row(q):
    """A NaN or an infinity in one row leaves that row's scale non-finite and
    every other row exactly as the oracle has it."""
    w = inputs.custom(9, 512, "bf16", False)
    t = inputs.make(w, seed=31)
    t["x"][2, 5] = float("nan")
    t["x"][6, 7] = float("inf")
    _, q_g, s_g = run_quant(t, QT[q], w.eps, residual=False)
    assert not np.isfinite(s_g[2]) and not np.isfinite(s_g[6])
    keep = np.array([r for r in range(9) if r not in (2, 6)])
    xb, wb = inputs.bits(t["x"])[keep], inputs.bits(t["weight"])
    _, q_o, s_o = parity.oracle_quant(xb, wb, w.eps, QT[q])
    q_gk = q_g[keep].view(np.int8) if QT[q] == 0 else q_g[keep]
    say(parity.compare_quant(q_gk, q_o, s_g[keep], s_o, parity.quant_t(xb, wb, QT[q]), QT[q]))


def _run_any_quant(dtype, rows, hidden, fused, qtype, cfg, off, qoff, seed):
    """Forced configuration with x (residual, h) starting `off` elements and
    the codes `qoff` bytes past a 16-byte boundary, inside guard space: parity
    with the oracle, and no byte outside the outputs written."""
    w = inputs.custom(rows, hidden, dtype, fused)
    t = inputs.make(w, seed=seed)
    td = BF16 if dtype == "bf16" else F32
    es = 2 if dtype == "bf16" else 4
    n = rows * hidden
    g = 64
    bases = [g + off + i * (n + 2 * g) for i in range(3)]  # x, residual, h
    # guard space holds non-zero patterns, so that a stray write of a zero
    # (code or value) shows
    buf = torch.full((3 * (n + 2 * g) + 2 * g,), 1.0, dtype=td, device="cuda")
    buf[bases[0]:bases[0] + n] = t["x"].reshape(-1).cuda()
    if fused:
        buf[bases[1]:bases[1] + n] = t["residual"].reshape(-1).cuda()
    qbuf = torch.full((n + 2 * g,), 0xA5, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((rows + 2,), -1.0, dtype=torch.float32, device="cuda")
    wt = t["weight"].cuda()
    p = buf.data_ptr()
    ptr = [p + es * b for b in bases]
    st = mbr.lib().rmsnorm_dynamic_quant_fwd_ex(
        ptr[0], ptr[1] if fused else None, wt.data_ptr(), ptr[2] if fused else None, qbuf.data_ptr() + g + qoff,
        sbuf.data_ptr() + 4, rows, hidden, w.eps, mbr.dtype_code(td), qtype, ctypes.byref(cfg),
        torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == mbr.RMSNORM_OK, mbr.rmsnorm_status_string(st)
    cpu, q_all, s_all = inputs.bits(buf.cpu()), qbuf.cpu().numpy(), sbuf.cpu().numpy()
    xb, wb = inputs.bits(t["x"]), inputs.bits(t["weight"])
    rb = inputs.bits(t["residual"]) if fused else None
    h_o, q_o, s_o = parity.oracle_quant(xb, wb, w.eps, qtype, residual=rb)
    if fused:
        assert np.array_equal(cpu[bases[2]:bases[2] + n].reshape(rows, hidden), h_o), "residual sum differs"
    q_g = q_all[g + qoff:g + qoff + n].reshape(rows, hidden)
    v = h_o if fused else xb
    say(parity.compare_quant(q_g.view(np.int8) if qtype == 0 else q_g, q_o, s_all[1:1 + rows], s_o,
                             parity.quant_t(v, wb, qtype), qtype))
    written = np.zeros(cpu.shape, bool)
    for i in (0, 1, 2) if fused else (0,):
        written[bases[i]:bases[i] + n] = True
    assert np.all(cpu[~written] == inputs.bits(torch.ones(1, dtype=td))[0]), "a byte outside x, residual and h changed"
    assert np.all(q_all[:g + qoff] == 0xA5) and np.all(q_all[g + qoff + n:] == 0xA5), "a code outside q changed"
    assert s_all[0] == -1.0 and s_all[-1] == -1.0, "a scale outside the row range changed"


@pytest.mark.parametrize("q", ["int8", "fp8"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("fused", [False, True])
def test_every_any_alignment_quant_config(dtype, fused, q):
    """Every built quantised any-alignment configuration, forced: full and
    masked vector sets, tails of 0, 1 and V - 1 elements, inputs and codes
    at several offsets from a 16-byte boundary."""
    v = 8 if dtype == "bf16" else 4
    n = 0
    for wpr in built.WPR:
        for vpl in built.ANY_VPL:
            if not built.qany(wpr, vpl):
                continue
            lanes = 64 * wpr
            for nvec in sorted({lanes * vpl, max(1, lanes * (vpl - 1) + 3)}):
                tail = (0, 1, v - 1)[n % 3]
                off = (1, v - 1, 0)[n % 3]
                qoff = (3, 0, 1, 7)[n % 4]
                cfg = mbr.Config(mbr.PATH_VECTOR_ANY, wpr, vpl, 1, 2 if n % 4 == 3 else 0)
                say("quant any", q, dtype, fused, cfg, "hidden", nvec * v + tail, "offsets", off, qoff)
                _run_any_quant(dtype, 5, nvec * v + tail, fused, QT[q], cfg, off, qoff, 5000 + n)
                n += 1
    assert n == 48


@pytest.mark.parametrize("q", ["int8", "fp8"])
@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("hidden", [8191, 5121, 4097, 1031])
def test_odd_widths_automatic_quant(hidden, fused, q):
    """Widths that are not whole vectors take the any-alignment path by
    themselves, at the sizes of the workloads."""
    cfg = mbr.rmsnorm_select_quant_config(4096, hidden, BF16, True, fused)
    assert cfg.path == mbr.PATH_VECTOR_ANY
    say("quant odd width", q, hidden, fused, cfg.as_dict())
    _run_any_quant("bf16", 2048 if hidden > 5000 else 4096, hidden, fused, QT[q], cfg, 1, 5, hidden)


@pytest.mark.parametrize("qname", ["int8", "fp8"])
def test_quant_graph_capture_replays_match_eager(qname):
    """The fused quantised form (and a plain odd-width call on the
    any-alignment path) captured in one HIP graph: every replay, with eager
    work and synchronisations in between, equals the eager results bitwise."""
    qt = QT[qname]
    w = inputs.custom(3000, 5120, "bf16", True)
    t = {k: v.cuda() for k, v in inputs.make(w, seed=31).items()}
    w2 = inputs.custom(777, 4097, "bf16", False)
    t2 = {k: v.cuda() for k, v in inputs.make(w2, seed=32).items()}

    def outputs():
        return (torch.empty_like(t["x"]), torch.empty(t["x"].shape, dtype=torch.uint8, device="cuda"),
                torch.empty(t["x"].shape[0], dtype=torch.float32, device="cuda"),
                torch.empty(t2["x"].shape, dtype=torch.uint8, device="cuda"),
                torch.empty(t2["x"].shape[0], dtype=torch.float32, device="cuda"))

    def call(o):
        mbr.rmsnorm_dynamic_quant_fwd(t["x"], t["weight"], o[1], o[2], 1e-5, qt, t["residual"], o[0])
        mbr.rmsnorm_dynamic_quant_fwd(t2["x"], t2["weight"], o[3], o[4], 1e-5, qt)

    eager = outputs()
    call(eager)
    graphed = outputs()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(graphed)
    for rep in range(3):
        for o in graphed:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(eager, graphed):
            assert torch.equal(a, b), "replay %d differs" % rep
        call(outputs())  # eager work between replays

"""Several host threads, each on its own HIP stream, calling different entry
points at the same time: every result must equal, bit for bit, the same call
made alone on the default stream.  The library keeps no per-call state; the
backward's partial rows live in each caller's own workspace (the
allocation-free backward shares one scratch array per GPU and is left out,
since its overlapping calls race by contract)."""
import concurrent.futures

import pytest
import torch

import memory_bound_rmsnorm_amd as mbr

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16


def _inputs():
    g = torch.Generator().manual_seed(20261203)

    def t(*shape, dtype=BF16, scale=1.0, shift=0.0):
        return (torch.randn(*shape, generator=g) * scale + shift).to(dtype).cuda()

    return {
        "x1": t(2048, 4096), "w1": t(4096, shift=1.0, scale=0.1),
        "x2": t(1536, 5120), "r2": t(1536, 5120), "w2": t(5120, shift=1.0, scale=0.1),
        "x3": t(1024, 8192), "r3": t(1024, 8192), "w3": t(8192, shift=1.0, scale=0.1),
        "x4": t(2048, 2048), "dy4": t(2048, 2048), "w4": t(2048, shift=1.0, scale=0.1),
        "x5": t(1024, 4096, shift=3.0), "g5": t(4096, shift=1.0, scale=0.1), "b5": t(4096, scale=0.1),
        "x6": t(512, 1000, dtype=torch.float32), "w6": t(1000, dtype=torch.float32, shift=1.0, scale=0.1),
    }


def _jobs(d):
    def fwd():
        out = torch.empty_like(d["x1"])
        return (mbr.rmsnorm_fwd(d["x1"], d["w1"], out, 1e-5),)

    def fused():
        h, y = torch.empty_like(d["x2"]), torch.empty_like(d["x2"])
        return mbr.rmsnorm_residual_fwd(d["x2"], d["r2"], d["w2"], h, y, 1e-5)

    def quant():
        h = torch.empty_like(d["x3"])
        q = torch.empty(d["x3"].shape, dtype=torch.uint8, device="cuda")
        sc = torch.empty(d["x3"].shape[0], dtype=torch.float32, device="cuda")
        mbr.rmsnorm_dynamic_quant_fwd(d["x3"], d["w3"], q, sc, 1e-5, mbr.QUANT_INT8, d["r3"], h)
        return h, q, sc

    def bwd():
        dx, dw = torch.empty_like(d["x4"]), torch.empty_like(d["w4"])
        return mbr.rmsnorm_bwd(d["x4"], d["w4"], d["dy4"], dx, dw, 1e-5)

    def ln():
        out = torch.empty_like(d["x5"])
        return (mbr.layernorm_fwd(d["x5"], d["g5"], d["b5"], out, 1e-5),)

    def fwd_any_f32():
        out = torch.empty_like(d["x6"])
        return (mbr.rmsnorm_fwd(d["x6"], d["w6"], out, 1e-6),)

    return [fwd, fused, quant, bwd, ln, fwd_any_f32]


def test_threads_on_separate_streams_match_serial_calls_bitwise():
    d = _inputs()
    jobs = _jobs(d)
    want = [tuple(o.clone() for o in job()) for job in jobs]
    torch.cuda.synchronize()
    reps = 6

    def worker(job):
        s = torch.cuda.Stream()
        outs = []
        with torch.cuda.stream(s):
            for _ in range(reps):
                outs.append(job())
        s.synchronize()
        return outs

    with concurrent.futures.ThreadPoolExecutor(len(jobs)) as ex:
        got = list(ex.map(worker, jobs))
    torch.cuda.synchronize()
    for j, (w, outs) in enumerate(zip(want, got)):
        for rep, o in enumerate(outs):
            for a, b in zip(w, o):
                assert torch.equal(a, b), "job %d (%s), repetition %d differs" % (j, jobs[j].__name__, rep)


def test_calls_go_to_the_callers_current_stream():
    """The binding passes the caller's current stream: the default stream, or
    the one a `torch.cuda.stream` context selects, in this thread."""
    x = torch.zeros(1, device="cuda")
    assert mbr._stream(None, x.device) == torch.cuda.current_stream().cuda_stream
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        assert mbr._stream(None, x.device) == s.cuda_stream
    assert mbr._stream(s, x.device) == s.cuda_stream

#!/usr/bin/env python3
"""Throughput of the RMSNorm hot path on one MI355X.

A step is one rmsnorm_fwd call (or rmsnorm_residual_fwd for the fused
workload) over a whole [rows, hidden] batch: load rows, sum squares, inverse
root, scale and store.  Default workload: bf16 [16384, 8192], the
large-hidden configuration the headline bandwidth figure is quoted on.  The
quantised workloads time rmsnorm_dynamic_quant_fwd, the backward ones
rmsnorm_bwd (dx and dweight: the row kernel plus the dweight reduction), the
LayerNorm ones layernorm_fwd, the KV ones kv_rmsnorm_rope_cache (one call
writes every token's two cache rows; whole input-and-cache sets rotate).

Byte accounting follows the TileLang tutorial ch. 02, section 2.1: every input
read once, every output written once, the weight once; the figure reported is
algorithmic bytes / time, and its roofline is HBM bandwidth (MI355X: 8 TB/s).

Timing protocol: inputs are resident in HBM before the timed region; several
copies of the input/output set are rotated so that the footprint of a pass
(>= 2 GiB) exceeds the 256 MB last-level cache and every step reads from HBM;
W untimed warm-up steps; then exactly K steps between a device synchronise and
HIP events on the launch stream.  A step of at least 128 MiB (the headline;
the fused, quantised and backward forms at [16384, 8192] or [12289, 5120];
LayerNorm [8192, 4096]; the wide rows) takes >= 20 us, more than twice as
long as one call takes to issue (8-12 us), so the K steps are K
eager calls of the C-ABI entry point through the Python binding, the way a
caller issues them; before the copy ceiling the same K steps are also captured
in a HIP graph and timed as one replay, for the record (graph_us_per_call).
Smaller steps would time the host, so they are captured in a HIP graph
(before the warm-up, with an untimed upload replay) and replayed once inside
the timed region, with K eager calls timed before the capture, for the
record (eager_us_per_call).  --graph and --eager force either.  After the timed
region, S more batches of K steps are timed one by one (eager batches queued
back to back, or graph replays), for the spread of the per-call time (median,
minimum, 90th percentile).

Default run (the headline workload): before the headline's own warm-up the
other four stated configurations are measured -- fp32 [64, 2048], bf16
[4096, 2048], bf16 [256, 4096] and the fused bf16 [12289, 5120] -- each with
its launches captured in a HIP graph that cycles through enough rotating sets
to stay HBM-cold, 20 replays timed one by one (median, minimum, p90 per call),
plus, for those whose bytes fit the cache easily (C1-C3), a cache-resident
figure with one set reused by every launch (labelled as such, never an HBM
figure), each after 50 ms of back-to-back replays of its graph; then the
runtime's own device-to-device copy (hipMemcpyAsync) of the headline's bytes
as one ceiling; then the headline's graph record; then the copy ceiling (the
hand-written 16-byte copy kernel on the same bytes, after 100 ms of copies,
timed the same way as the headline), right before the headline's warm-up.
The configurations go into the line as per_config; the device (name, arch,
compute units, torch and HIP versions) as device.  Measured on MI355X, the
first ~20 ms of a burst of launches after an idle spell (a graph capture, a
buffer release) run slower than the steady state (bf16 [16384, 8192]: 87.2 us
per call after 20 launches, 84.7 after 300); the ceilings are steady-state
figures, and with nothing but the W warm-up steps and a synchronise between
the copies and the timed steps, the headline's steps run at steady state too.
Parity of every launch configuration timed here, at these sizes, with the CPU
oracle is the job of the GPU test suite, not of this script.

CPU baseline: the oracle (as it stands) over a bounded sample of the
headline's rows, with the rows split over every CPU this process may use
(its affinity mask capped by its cgroup CPU quota) and again on one thread;
one warm-up pass, then timed runs of at least a second each, the median
reported.  One more, untimed, pass of the oracle over the sample is set
beside the GPU's output for the same rows in the timed launch configuration
(cpu_baseline.oracle_vs_gpu: ulp histogram, bitwise-equal fraction, largest
errors); a report only, since the GPU test suite is the parity gate.

Prints ONE JSON line on stdout.  With --all, one JSON record per other
workload is written to stderr (lines starting with '#'); those also carry the
per-launch time with the launches replayed from a HIP graph, since the small
workloads finish faster than Python can issue them.
"""
import argparse
import concurrent.futures
import json
import os
import platform
import statistics
import sys
import time

import torch

import memory_bound_rmsnorm_amd as mbr
from memory_bound_rmsnorm_amd import _build, inputs
from memory_bound_rmsnorm_amd.profile_summary import kernel_instances, launch_dict

HBM_PEAK_GBPS = 8000.0  # MI355X published HBM3E bandwidth
MIN_FOOTPRINT = 2 << 30
PROFILE_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=300,
                    help="untimed warm-up steps (default 300: on MI355X the first ~20 ms of a burst of "
                         "launches run up to 3%% slower, 12%% for the quantised forms, than the steady state)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other stated configurations (per_config) in the default run")
    ap.add_argument("--spread", type=int, default=20,
                    help="extra timed replays of the headline graph for the per-call spread (0: none)")
    ap.add_argument("--workload", default=inputs.HEADLINE, choices=sorted(inputs.EVERY_WORKLOAD))
    ap.add_argument("--all", action="store_true", help="also time every other workload (stderr)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU-baseline budget; 0 disables it")
    ap.add_argument("--no-copy", action="store_true", help="skip the copy-ceiling measurement")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--graph", action="store_true",
                    help="time the K steps as one HIP-graph replay, whatever the step's size")
    ap.add_argument("--eager", action="store_true",
                    help="time the K steps as K eager calls, whatever the step's size")
    return ap.parse_args()


def cgroup_cpu_quota():
    """CPUs this process's cgroup may use (cgroup v2 cpu.max or v1 cfs quota),
    or None when unlimited or unknown."""
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            q, per = f.read().split()[:2]
            return None if q == "max" else int(q) / int(per)
    except (OSError, ValueError):
        pass
    try:
        with open("/sys/fs/cgroup/cpu/cpu.cfs_quota_us") as f:
            q = int(f.read())
        with open("/sys/fs/cgroup/cpu/cpu.cfs_period_us") as f:
            per = int(f.read())
        return None if q <= 0 else q / per
    except (OSError, ValueError):
        return None


def host_cpus():
    """(threads, detail): every CPU this process may use -- its affinity mask,
    capped by its cgroup CPU quota when there is one."""
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:
        aff = os.cpu_count() or 1
    quota = cgroup_cpu_quota()
    n = aff if quota is None else max(1, min(aff, int(quota)))
    return n, {"affinity_cpus": aff, "cgroup_cpu_quota": quota}


def host_threads() -> int:
    return host_cpus()[0]


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


QUANT_CODE = {"int8": mbr.QUANT_INT8, "fp8": mbr.QUANT_FP8_E4M3}


class Sets:
    """Rotating device copies of one workload's inputs and outputs."""

    def __init__(self, w, t, n_sets):
        dev = {k: v.cuda() for k, v in t.items()}
        self.weight = dev["weight"]
        self.sets = []
        self.backward = w.backward
        self.layernorm = w.layernorm
        self.beta = dev.get("beta")
        if w.backward:
            nbytes = mbr.rmsnorm_bwd_workspace_size(w.rows, w.hidden, self.weight.dtype)
            self.workspace = torch.empty(max(1, nbytes), dtype=torch.uint8, device="cuda")
        for i in range(n_sets):
            s = {"x": dev["x"] if i == 0 else dev["x"].clone()}
            if w.backward:
                s["dy"] = dev["dy"] if i == 0 else dev["dy"].clone()
                s["dx"] = torch.empty_like(s["x"])
                s["dw"] = torch.empty_like(self.weight)
                self.sets.append(s)
                continue
            if w.fused:
                s["residual"] = dev["residual"] if i == 0 else dev["residual"].clone()
                s["h"] = torch.empty_like(s["x"])
            if w.quant:
                s["q"] = torch.empty(s["x"].shape, dtype=torch.uint8, device="cuda")
                s["scale"] = torch.empty(w.rows, dtype=torch.float32, device="cuda")
            else:
                s["out"] = torch.empty_like(s["x"])
            self.sets.append(s)
        self.fused = w.fused
        self.quant = QUANT_CODE[w.quant] if w.quant else None
        self.eps = w.eps

    def launch(self, i):
        s = self.sets[i % len(self.sets)]
        if self.backward:
            mbr.rmsnorm_bwd(s["x"], self.weight, s["dy"], s["dx"], s["dw"], self.eps, self.workspace)
        elif self.layernorm:
            mbr.layernorm_fwd(s["x"], self.weight, self.beta, s["out"], self.eps)
        elif self.quant is not None:
            mbr.rmsnorm_dynamic_quant_fwd(s["x"], self.weight, s["q"], s["scale"], self.eps, self.quant,
                                          s.get("residual"), s.get("h"))
        elif self.fused:
            mbr.rmsnorm_residual_fwd(s["x"], s["residual"], self.weight, s["h"], s["out"], self.eps)
        else:
            mbr.rmsnorm_fwd(s["x"], self.weight, s["out"], self.eps)


class KvSets:
    """Rotating device copies of a KV workload's kv input and both caches."""

    def __init__(self, w, t, n_sets):
        dev = {k: v.cuda() for k, v in t.items()}
        self.w = w
        self.gamma, self.cos, self.sin = dev["gamma"], dev["cos"], dev["sin"]
        self.positions, self.slots = dev["positions"], dev["slots"]
        self.sets = []
        for i in range(n_sets):
            nc, rc = inputs.kv_caches(w, "cuda")
            self.sets.append({"kv": dev["kv"] if i == 0 else dev["kv"].clone(), "nc": nc, "rc": rc})

    def launch(self, i):
        s = self.sets[i % len(self.sets)]
        mbr.kv_rmsnorm_rope_cache(s["kv"], self.gamma, self.cos, self.sin, self.positions, self.slots, s["nc"],
                                  s["rc"], self.w.eps, self.w.rope_style)


def is_kv(w) -> bool:
    return isinstance(w, inputs.KvWorkload)


def n_sets_for(w) -> int:
    if is_kv(w):
        per_set = w.tokens * w.heads * (w.norm_dim + w.rope_dim) * w.elem_size + w.cache_bytes
    else:
        per_set = w.algorithmic_bytes - w.hidden * w.elem_size
    return max(2, -(-MIN_FOOTPRINT // per_set))


def percentile(vals, q):
    """Nearest-rank percentile q (0-100) of a non-empty list."""
    v = sorted(vals)
    k = max(0, min(len(v) - 1, -(-len(v) * q // 100) - 1))
    return v[int(k)]


def spread_us(per_call_s, launches):
    """Median, minimum and 90th percentile of per-call times (seconds), in us."""
    return {"us_median": round(statistics.median(per_call_s) * 1e6, 3), "us_min": round(min(per_call_s) * 1e6, 3),
            "us_p90": round(percentile(per_call_s, 90) * 1e6, 3), "samples": len(per_call_s),
            "launches_per_sample": launches}


def replay_samples(g, launches, samples):
    """Replay a captured graph `samples` times, each replay between its own HIP
    events on the current stream; per-call seconds of each replay."""
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(samples)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record(stream)
        g.replay()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) / 1e3 / launches for a, b in ev]


COPY_WARM_SECONDS = 0.1
GRAPH_WARM_SECONDS = 0.05


def capture(fn, steps, first):
    """fn(first), ..., fn(first + steps - 1) captured once in a HIP graph, then
    one untimed replay, which uploads it."""
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            fn(first + i)
    g.replay()
    torch.cuda.synchronize()
    return g


def time_steps_graph(fn, steps, warmup, spread=0, before=None):
    """Exactly `steps` calls, captured once in a HIP graph and replayed once
    between a device synchronise and HIP events on the launch stream.  Before
    that, in this order: one untimed call outside the capture (module load),
    the capture and its untimed upload replay, `before()` if given, and W eager
    warm-up calls.  The capture is host work that leaves the GPU idle, so it
    comes first: between the warm-up and the timed replay there is only a
    synchronise.  Consecutive calls stay ordered (a captured stream is a chain
    of dependent nodes); what a replay leaves out is the per-launch host work.
    After the timed replay, `spread` more replays are timed one by one.
    Returns (wall seconds, event seconds, per-call seconds of the extra replays)."""
    fn(0)
    g = capture(fn, steps, warmup)
    if before is not None:
        before()
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    g.replay()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    extra = replay_samples(g, steps, spread) if spread > 0 else []
    del g
    return wall, start.elapsed_time(end) / 1e3, extra


def time_steps(fn, steps, warmup, spread=0, before=None):
    """Exactly `steps` eager calls between a device synchronise and HIP events
    on the launch stream, after `before()` if given and W warm-up calls.  After
    the timed region, `spread` more batches of `steps` calls, queued back to
    back, are timed one by one, each between its own events.
    Returns (wall seconds, event seconds, per-call seconds of the extra batches)."""
    if before is not None:
        before()
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        fn(warmup + i)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    extra = []
    if spread > 0:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(spread)]
        for j, (a, b) in enumerate(ev):
            a.record(stream)
            for i in range(steps):
                fn(warmup + (j + 1) * steps + i)
            b.record(stream)
        torch.cuda.synchronize()
        extra = [a.elapsed_time(b) / 1e3 / steps for a, b in ev]
    return wall, start.elapsed_time(end) / 1e3, extra


def graph_samples(fn, n_sets, samples=20, warm_s=GRAPH_WARM_SECONDS):
    """Per-launch times with the launches captured once in a HIP graph that
    cycles through every rotation set (at least 64 launches), replayed
    `samples` times, each replay timed on its own.  Before the timed replays
    the graph is replayed back to back for `warm_s` seconds (steady state:
    the capture leaves the GPU idle, and the first ~20 ms of a burst of
    launches after an idle spell run slower).  The graph removes Python and
    launch-call overhead from the GPU timeline (the kernels allocate and
    memset nothing, so they capture cleanly).  Returns (per-call seconds of
    each replay, launches per replay)."""
    launches = min(4096, max(64, n_sets))
    g = capture(fn, launches, 0)
    warm_for(lambda i: g.replay(), warm_s, batch=4)
    per = replay_samples(g, launches, samples)
    del g
    return per, launches


def graph_time(fn, n_sets, replays=10):
    """Median per-launch time over `replays` timed graph replays."""
    per, _ = graph_samples(fn, n_sets, replays)
    return statistics.median(per)


def warm_for(fn, seconds, batch=16):
    """Launch fn in batches of `batch` until `seconds` of wall time have
    passed, synchronising after each batch; returns the number of launches."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    i = 0
    while True:
        for _ in range(batch):
            fn(i)
            i += 1
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return i


class CopyCeiling:
    """hbm_copy of the same read/write byte count as one step, rotated the same
    way and timed the same way (eager launches or one graph replay), after
    100 ms of copies: the ceiling is a steady-state figure.  The buffers live
    until free(), so that no deallocation idles the GPU between this and the
    headline steps that follow it."""

    def __init__(self, w):
        self.nbytes = w.copy_bytes
        self.n = max(2, -(-MIN_FOOTPRINT // (2 * self.nbytes)))
        self.src = [torch.empty(self.nbytes, dtype=torch.uint8, device="cuda").fill_(i % 251) for i in range(self.n)]
        self.dst = [torch.empty(self.nbytes, dtype=torch.uint8, device="cuda") for _ in range(self.n)]

    def launch(self, i):
        mbr.hbm_copy(self.src[i % self.n], self.dst[i % self.n])

    def measure(self, steps, warmup, graph=False):
        def warm():
            warm_for(self.launch, COPY_WARM_SECONDS)
        if graph:
            _, ev, _ = time_steps_graph(self.launch, steps, warmup, before=warm)
        else:
            warm()
            _, ev, _ = time_steps(self.launch, steps, warmup)
        return 2 * self.nbytes / (ev / steps) / 1e9

    def free(self):
        self.src, self.dst = [], []
        torch.cuda.empty_cache()


def memcpy_ceiling(w, steps, warmup):
    """The runtime's own device-to-device copy (hipMemcpyAsync, through torch's
    copy_ of contiguous same-type tensors) of the same byte count, rotated the
    same way, timed as eager calls between HIP events: a second ceiling beside
    the hand-written copy kernel."""
    nbytes = w.copy_bytes
    n = max(2, -(-MIN_FOOTPRINT // (2 * nbytes)))
    src = [torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(i % 251) for i in range(n)]
    dst = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(n)]
    copy = lambda i: dst[i % n].copy_(src[i % n])  # noqa: E731
    warm_for(copy, COPY_WARM_SECONDS)
    _, ev, _ = time_steps(copy, steps, warmup)
    del src, dst
    torch.cuda.empty_cache()
    return 2 * nbytes / (ev / steps) / 1e9


def device_info():
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", ""), "compute_units": p.multi_processor_count,
            "memory_gib": round(p.total_memory / 2 ** 30, 1), "torch": torch.__version__,
            "hip": getattr(torch.version, "hip", None)}


def load_traffic(w, launch):
    """HBM bytes per step from the committed counter summary, if it was taken
    on the current kernel sources in the current launch configuration; else None."""
    fam = kernel_instances(w)[0][0].split("<")[0].split("::")[1]
    path = os.path.join(PROFILE_DIR, "pmc_traffic_%s_%s.txt" % (fam, w.name))
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if ":" in line:
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    try:
        family = "kv" if is_kv(w) else "bwd" if w.backward else "ln" if w.layernorm else "fwd"
        if vals.get("source_sha256") != _build.source_digest(family):
            return None
        if vals.get("launch_config") != " ".join("%s=%s" % kv for kv in launch.items()):
            return None
        fetch = float(vals["rmsnorm_fetch_kib_per_dispatch"]) * 1024 * float(vals["copy_fetch_scale"])
        write = float(vals["rmsnorm_write_kib_per_dispatch"]) * 1024 * float(vals["copy_write_scale"])
        return fetch + write
    except (KeyError, ValueError):
        return None


def _cpu_rates(one_pass, sample_bytes, threads, runs, min_s):
    """One warm-up pass, then `runs` timed runs of at least min_s seconds each
    (whole passes); GB/s of each run."""
    one_pass(threads)
    rates = []
    for _ in range(runs):
        reps = 0
        t0 = time.perf_counter()
        while True:
            one_pass(threads)
            reps += 1
            el = time.perf_counter() - t0
            if el >= min_s:
                break
        rates.append(sample_bytes * reps / el / 1e9)
    return rates


def _cpu_record(one_pass, sample_bytes, seconds, sample_desc):
    """The oracle on every usable CPU and on one thread: median of 5 and of 3
    timed runs; `seconds` is the whole budget."""
    T, detail = host_cpus()
    min_s = max(0.2, seconds / 8)
    rates = _cpu_rates(one_pass, sample_bytes, T, 5, min_s)
    one = _cpu_rates(one_pass, sample_bytes, 1, 3, min_s) if T > 1 else rates
    med = statistics.median(rates)
    return {"value": round(med, 4), "unit": "GB/s", "cores": T, "kind": "oracle",
            "sample": "%s; rows split over %d threads (every CPU this process may use), median of %d timed runs "
                      "of >= %.1f s after a warm-up pass" % (sample_desc, T, len(rates), min_s),
            "runs_gbps": [round(r, 4) for r in rates],
            "one_thread": {"value": round(statistics.median(one), 4), "unit": "GB/s", "threads": 1,
                           "runs_gbps": [round(r, 4) for r in one]},
            "host": dict({"cpu_model": cpu_model(), "os_cpu_count": os.cpu_count()}, **detail)}


def _split(n, T):
    return [(i * n // T, (i + 1) * n // T) for i in range(T)]


def cpu_baseline_kv(w, t, seconds):
    """The oracle over the first tokens of a KV workload, tokens split across
    the host's threads, each thread writing compact caches of its own."""
    import numpy as np
    import oracle  # the CPU checker; timed here as a reported baseline only
    tokens = min(w.tokens, 2048)
    kvb = inputs.bits(t["kv"])[:tokens]
    gb = inputs.bits(t["gamma"])
    cos_t, sin_t = t["cos"].numpy(), t["sin"].numpy()
    pos = t["positions"].numpy()[:tokens]
    np_dtype = np.uint16 if w.dtype == "bf16" else np.float32

    def one_pass(T):
        with concurrent.futures.ThreadPoolExecutor(T) as ex:
            def job(r):
                n = r[1] - r[0]
                if n == 0:
                    return
                nc = np.empty((n, w.heads, w.norm_dim), np_dtype)
                rc = np.empty((n, w.heads, w.rope_dim), np_dtype)
                oracle.kv_rmsnorm_rope_cache(kvb[r[0]:r[1]], gb, cos_t, sin_t, pos[r[0]:r[1]],
                                             np.arange(n, dtype=np.int64), nc, rc, w.eps, w.rope_style)
            list(ex.map(job, _split(tokens, T)))

    sample_bytes = w.algorithmic_bytes * tokens // w.tokens
    return _cpu_record(one_pass, sample_bytes, seconds, "first %d of %d tokens" % (tokens, w.tokens))


def sample_rows(w) -> int:
    """Rows of the CPU baseline's bounded sample: about 64 MiB of algorithmic bytes."""
    return max(1, min(w.rows, (64 << 20) * w.rows // w.algorithmic_bytes))


def gpu_sample(w, sets):
    """The timed launch configuration's outputs for the sample rows of
    rotation set 0 (whose inputs are the host tensors), as host arrays."""
    if is_kv(w):
        return None
    rows = sample_rows(w)
    s = sets.sets[0]
    torch.cuda.synchronize()
    if w.backward:
        return {"dx": inputs.bits(s["dx"][:rows])}
    if w.quant:
        d = {"q": s["q"][:rows].cpu().numpy(), "scale": s["scale"][:rows].cpu().numpy()}
        if w.fused:
            d["h"] = inputs.bits(s["h"][:rows])
        return d
    d = {"y": inputs.bits(s["out"][:rows])}
    if w.fused:
        d["h"] = inputs.bits(s["h"][:rows])
    return d


def _agreement(gpu, ref, kind):
    """How the GPU's sample outputs compare with the oracle's: bf16 distance
    on the monotone line of bit patterns (+0 = -0), fp32 relative error,
    codes by count of differing codes."""
    import numpy as np
    n = int(ref.size)
    if kind == "codes":
        diff = np.ascontiguousarray(gpu).view(np.uint8).reshape(-1) != np.ascontiguousarray(ref).view(np.uint8).reshape(-1)
        return {"n": n, "n_differing": int(diff.sum())}
    if kind == "scale":
        rel = np.abs(gpu.astype(np.float64) - ref) / np.maximum(np.abs(ref.astype(np.float64)), 1e-300)
        return {"n": n, "max_rel_err": float(rel.max()) if n else 0.0}
    if kind == "bf16":
        def mono(p):
            p = p.astype(np.int32)
            return np.where(p & 0x8000, -(p & 0x7FFF), p)
        d = np.abs(mono(gpu) - mono(ref)).reshape(-1)
        gf = (gpu.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        rf = (ref.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        return {"n": n, "max_ulp": int(d.max()) if n else 0, "frac_bitwise_equal": float((d == 0).mean()) if n else 1.0,
                "ulp_histogram": {"0": int((d == 0).sum()), "1": int((d == 1).sum()), ">1": int((d > 1).sum())},
                "max_abs_err": float(np.abs(gf - rf).max()) if n else 0.0}
    g, r = gpu.astype(np.float64).reshape(-1), ref.astype(np.float64).reshape(-1)
    rel = np.abs(g - r) / np.maximum(np.abs(r), 1e-300)
    return {"n": n, "max_rel_err": float(rel.max()) if n else 0.0,
            "frac_bitwise_equal": float((gpu.reshape(-1) == ref.reshape(-1)).mean()) if n else 1.0,
            "max_abs_err": float(np.abs(g - r).max()) if n else 0.0}


def cpu_baseline(w, t, seconds):
    """The oracle, as it stands, over a bounded sample of the workload's rows
    (about 64 MiB of algorithmic bytes), rows split across the host's threads;
    GB/s with the same byte ledger."""
    if is_kv(w):
        return cpu_baseline_kv(w, t, seconds)
    import oracle  # the CPU checker; timed here as a reported baseline only
    rows = sample_rows(w)
    xb = inputs.bits(t["x"])[:rows]
    wb = inputs.bits(t["weight"])
    rb = inputs.bits(t["residual"])[:rows] if w.fused else None
    gb = inputs.bits(t["dy"])[:rows] if w.backward else None
    bb = inputs.bits(t["beta"]) if w.layernorm else None
    qt = {"int8": oracle.QUANT_INT8, "fp8": oracle.QUANT_FP8_E4M3}.get(w.quant)

    def one_pass(T):
        with concurrent.futures.ThreadPoolExecutor(T) as ex:
            def job(r):
                if r[0] == r[1]:
                    return
                if w.backward:  # each thread: dx and its rows' dweight
                    oracle.rmsnorm_bwd(xb[r[0]:r[1]], wb, gb[r[0]:r[1]], w.eps)
                elif w.layernorm:
                    oracle.layernorm_fwd(xb[r[0]:r[1]], wb, bb, w.eps)
                elif qt is not None:
                    oracle.rmsnorm_dynamic_quant_fwd(xb[r[0]:r[1]], wb, w.eps, qt,
                                                     residual=rb[r[0]:r[1]] if w.fused else None)
                elif w.fused:
                    oracle.rmsnorm_residual_fwd(xb[r[0]:r[1]], rb[r[0]:r[1]], wb, w.eps)
                else:
                    oracle.rmsnorm_fwd(xb[r[0]:r[1]], wb, w.eps)
            list(ex.map(job, _split(rows, T)))

    sample_bytes = inputs.Workload(w.name, w.dtype, rows, w.hidden, w.eps, w.fused, w.x, w.weight, w.residual,
                                   quant=w.quant, grad=w.grad, beta=w.beta).algorithmic_bytes
    rec = _cpu_record(one_pass, sample_bytes, seconds, "first %d of %d rows" % (rows, w.rows))
    gpu = t.get("gpu_sample")
    if gpu is not None:
        # one more (untimed) pass of the oracle over the sample, set beside
        # the GPU's output of the same rows in the timed launch configuration
        kind = w.dtype
        if w.backward:
            dx, _ = oracle.rmsnorm_bwd(xb, wb, gb, w.eps, want_dw=False)
            outs = {"dx": _agreement(gpu["dx"], dx, kind)}
        elif w.layernorm:
            outs = {"y": _agreement(gpu["y"], oracle.layernorm_fwd(xb, wb, bb, w.eps), kind)}
        elif qt is not None:
            h, q, sc = oracle.rmsnorm_dynamic_quant_fwd(xb, wb, w.eps, qt, residual=rb if w.fused else None)
            outs = {"codes": _agreement(gpu["q"], q, "codes"), "scale": _agreement(gpu["scale"], sc, "scale")}
            if w.fused:
                outs["h"] = _agreement(gpu["h"], h, kind)
        elif w.fused:
            h, y = oracle.rmsnorm_residual_fwd(xb, rb, wb, w.eps)
            outs = {"h": _agreement(gpu["h"], h, kind), "y": _agreement(gpu["y"], y, kind)}
        else:
            outs = {"y": _agreement(gpu["y"], oracle.rmsnorm_fwd(xb, wb, w.eps), kind)}
        note = ("the oracle's output for the sample rows against the GPU's output for the same rows of rotation "
                "set 0 in the timed launch configuration; a report: the GPU test suite is the parity gate")
        if qt is not None:
            note += " (it checks that every differing code sits at a rounding tie)"
        elif w.backward or w.layernorm:
            note += (" (these outputs cancel: their bound is on magnitude, so an output near zero may lie several "
                     "ulps from the oracle's and still be within it)")
        rec["oracle_vs_gpu"] = dict(outs, rows=rows, note=note)
    return rec


def setup_workload(w, seed):
    """(host tensors, rotating device sets, number of sets, shape fields)."""
    if is_kv(w):
        t = inputs.make_kv(w, seed=seed)
        n_sets = n_sets_for(w)
        return t, KvSets(w, t, n_sets), n_sets, {"tokens": w.tokens, "heads": w.heads, "norm_dim": w.norm_dim,
                                                 "rope_dim": w.rope_dim, "num_slots": w.num_slots}
    t = inputs.make(w, seed=seed)
    n_sets = n_sets_for(w)
    return t, Sets(w, t, n_sets), n_sets, {"rows": w.rows, "hidden": w.hidden, "fused": w.fused, "quant": w.quant,
                                           "backward": w.backward}


# Steps of at least this many algorithmic bytes take >= 20 us even at 6.4 TB/s,
# more than twice what the Python binding and the C ABI need to issue one call
# (8-12 us measured on the GPU machine), so K eager calls keep the GPU busy from the
# first to the last and are timed as such; smaller steps would time the host,
# so they are captured in a HIP graph and replayed.
EAGER_MIN_BYTES = 128 << 20


def timed_as_graph(w, args) -> bool:
    if args.graph or args.eager:
        return bool(args.graph)
    return w.algorithmic_bytes < EAGER_MIN_BYTES


def bench_workload(w, steps, warmup, seed, with_copy=True, graph=False, timed_graph=False, spread=0):
    t, sets, n_sets, shape = setup_workload(w, seed)
    nbytes = w.algorithmic_bytes
    rec = dict({"workload": w.name, "dtype": w.dtype}, **shape)
    copy = None
    if with_copy:
        rec["memcpy_ceiling_gbps"] = memcpy_ceiling(w, max(20, steps // 2), max(2, warmup // 2))
        copy = CopyCeiling(w)

    def ceiling():
        rec["copy_ceiling_gbps"] = copy.measure(max(20, steps // 2), max(2, warmup // 2), graph=timed_graph)
    before = ceiling if copy is not None else None
    sets.launch(0)  # first launch: module load
    if timed_graph:
        # the eager record first; the graph is captured before the copy
        # ceiling, which runs right before the headline's warm-up
        _, ev2, _ = time_steps(sets.launch, steps, warmup)
        rec["eager_us_per_call"] = ev2 / steps * 1e6
        rec["eager_gbps"] = nbytes / (ev2 / steps) / 1e9
        wall, ev, extra = time_steps_graph(sets.launch, steps, warmup, spread, before=before)
    else:
        # the same K steps as one graph replay first, for the record (after
        # 50 ms of replays: the capture idles the GPU); then the copy ceiling,
        # then the headline's warm-up and timed steps with nothing between
        # them but a synchronise
        _, ev2, _ = time_steps_graph(sets.launch, steps, warmup,
                                     before=lambda: warm_for(sets.launch, GRAPH_WARM_SECONDS))
        rec["graph_us_per_call"] = ev2 / steps * 1e6
        rec["graph_gbps"] = nbytes / (ev2 / steps) / 1e9
        wall, ev, extra = time_steps(sets.launch, steps, warmup, spread, before=before)
    if copy is not None:
        copy.free()
    kern_s = ev / steps
    rec.update({
        "timing": "graph" if timed_graph else "eager",
        "eps": w.eps, "algorithmic_bytes": nbytes, "rotation_sets": n_sets,
        "wall_s": wall, "event_s": ev, "us_per_call": kern_s * 1e6,
        "gbps_wall": nbytes * steps / wall / 1e9, "gbps_kernel": nbytes / kern_s / 1e9,
        "kernel_config": launch_dict(w),
    })
    if extra:
        rec["spread"] = spread_us(extra, steps)
    if graph:
        gs = graph_time(sets.launch, n_sets)
        rec["us_per_call_graph"] = gs * 1e6
        rec["gbps_graph"] = nbytes / gs / 1e9
    if with_copy:
        rec["frac_of_copy_ceiling"] = rec["gbps_kernel"] / rec["copy_ceiling_gbps"]
        rec["frac_of_memcpy_ceiling"] = rec["gbps_kernel"] / rec["memcpy_ceiling_gbps"]
    t["gpu_sample"] = gpu_sample(w, sets)
    del sets
    torch.cuda.empty_cache()
    return t, rec


# Workloads whose bytes fit comfortably in the 256 MB last-level cache also
# get a cache-resident figure in per_config.
CACHE_RESIDENT_MAX = 64 << 20

# The other stated configurations, measured in the default run (per_config).
STATED = {"C1": "fp32_64x2048", "C2": "bf16_prefill_4096x2048", "C3": "bf16_decode_256x4096",
          "C4": inputs.HEADLINE, "C5": "bf16_residual_12289x5120"}


def measure_config(w, seed, samples=20):
    """One stated configuration, HBM-cold: its launches captured in a HIP graph
    that cycles through the rotating sets, `samples` replays timed one by one;
    per-call median, minimum and p90, and GB/s and roofline fraction at the
    median.  A cache-resident figure, where there is one, is taken first, so
    that the HBM-cold replays are the configuration's last dispatches."""
    t, sets, n_sets, shape = setup_workload(w, seed)
    for i in range(2 * n_sets):  # first launches: module load, clocks
        sets.launch(i)
    warm = None
    if w.algorithmic_bytes <= CACHE_RESIDENT_MAX:
        # the same buffers every launch: cache-resident, not an HBM figure
        wper, wl = graph_samples(lambda i: sets.launch(0), 1, samples)
        warm = {"us_median": round(statistics.median(wper) * 1e6, 3), "launches_per_sample": wl,
                "note": "one input/output set reused by every launch: cache-resident, not HBM bandwidth"}
    per, launches = graph_samples(sets.launch, n_sets, samples)
    del sets, t
    torch.cuda.empty_cache()
    med = statistics.median(per)
    gbps = w.algorithmic_bytes / med / 1e9
    rec = dict({"workload": w.name, "dtype": w.dtype}, **shape, algorithmic_bytes=w.algorithmic_bytes,
               rotation_sets=n_sets, gbps=round(gbps, 2), frac=round(gbps / HBM_PEAK_GBPS, 4),
               launch=launch_dict(w), **spread_us(per, launches))
    if warm:
        rec["cache_resident"] = warm
    return rec


def describe(w):
    """(metric, workload description, config fields, parity test) of a workload."""
    if is_kv(w):
        desc = "KV RMSNorm + RoPE (%s) + paged cache scatter %s, %d tokens (%s) x %d heads x (%d norm + %d rope), " \
               "%d cache slots, eps %g" % ("adjacent pairs" if w.rope_style == 1 else "halves", w.dtype, w.tokens,
                                           "decode" if w.decode else "prefill", w.heads, w.norm_dim, w.rope_dim,
                                           w.num_slots, w.eps)
        fields = {"tokens": w.tokens, "heads": w.heads, "norm_dim": w.norm_dim, "rope_dim": w.rope_dim,
                  "num_slots": w.num_slots, "rope_style": w.rope_style}
        return ("KV RMSNorm+RoPE+cache achieved HBM GB/s (%s)" % w.name, desc, fields,
                "tests/test_kv_gpu.py::test_kv_workloads_full_size")
    if w.name == inputs.HEADLINE:
        metric = "bf16 RMSNorm achieved HBM GB/s and % of peak at 16384×8192"
    else:
        metric = "%s achieved HBM GB/s (%s)" % ("LayerNorm" if w.layernorm else
                                               "RMSNorm backward" if w.backward else "RMSNorm", w.name)
    desc = "%s %s%s [%d, %d]%s%s, eps %g" % (
        "LayerNorm" if w.layernorm else "RMSNorm", "backward (dx, dweight) " if w.backward else "", w.dtype,
        w.rows, w.hidden, " fused residual" if w.fused else "",
        " with %s dynamic quantisation" % w.quant if w.quant else "", w.eps)
    fields = {"rows": w.rows, "hidden": w.hidden, "fused": w.fused, "quant": w.quant, "backward": w.backward,
              "layernorm": w.layernorm}
    parity = ("tests/test_bwd_gpu.py::test_bwd_workloads_full_size" if w.backward else
              "tests/test_ln_gpu.py::test_ln_workloads_full_size" if w.layernorm else
              "tests/test_quant_gpu.py" if w.quant else
              "tests/test_parity_gpu.py::test_shape_workloads_full_size" if w.name in inputs.SHAPE_WORKLOADS else
              "tests/test_parity_gpu.py::test_stated_workloads_full_size")
    return metric, desc, fields, parity


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this RMSNorm path shards by rows with no communication, and "
              "runs on more than one GPU are not part of this build (asked for --gpus %d, WORLD_SIZE %d)"
              % (args.gpus, world), file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (HIP device); none is visible", file=sys.stderr)
        sys.exit(1)
    mbr.lib()  # fail loudly if the HIP library is not built
    w = inputs.EVERY_WORKLOAD[args.workload]
    log("# device:", torch.cuda.get_device_name(0), "| workload:", w.name, "| steps", args.steps, "warmup", args.warmup)
    per_config = {}
    if w.name == inputs.HEADLINE and not args.no_configs:
        for label, name in STATED.items():
            if name == w.name:
                continue
            per_config[label] = measure_config(inputs.WORKLOADS[name], args.seed)
            log("# %s:" % label, json.dumps(per_config[label]))
    t, rec = bench_workload(w, args.steps, args.warmup, args.seed, not args.no_copy,
                            timed_graph=timed_as_graph(w, args), spread=args.spread)
    log("# timed:", json.dumps(rec))

    achieved = rec["gbps_kernel"]
    metric, desc, fields, parity = describe(w)
    line = {
        "metric": metric,
        "value": round(rec["gbps_wall"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec["wall_s"] / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded; x ~ N(0,1) with 8 outlier channels x100, weight ~ N(1, 0.1))"
                if w.name == inputs.HEADLINE else "synthetic (seeded)",
        "config": dict({"workload": desc}, **fields, algorithmic_bytes_per_step=w.algorithmic_bytes,
                       rotation_sets=rec["rotation_sets"], launch=rec["kernel_config"]),
        "pct_of_peak": round(100 * rec["gbps_wall"] / HBM_PEAK_GBPS, 2),
        "us_per_call": round(rec["us_per_call"], 3),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": load_traffic(w, rec["kernel_config"])},
        "parity": "checked against the CPU oracle at this size and launch configuration by " + parity,
        "timing": ("the K steps captured in one HIP graph and replayed once between synchronisations"
                   if rec["timing"] == "graph" else
                   "K eager calls of the C-ABI entry point (through the Python binding) between synchronisations"),
    }
    if "spread" in rec:
        line["spread"] = dict(rec["spread"], note=(
            "the same K-step graph replayed again, each replay timed on its own with HIP events"
            if rec["timing"] == "graph" else
            "more batches of K eager calls, queued back to back, each batch timed on its own with HIP events"))
    if "eager_us_per_call" in rec:
        line["eager_us_per_call"] = round(rec["eager_us_per_call"], 3)
        line["eager_gbps"] = round(rec["eager_gbps"], 2)
    if "graph_us_per_call" in rec:
        line["graph_us_per_call"] = round(rec["graph_us_per_call"], 3)
        line["graph_gbps"] = round(rec["graph_gbps"], 2)
    if "copy_ceiling_gbps" in rec:
        line["copy_ceiling_gbps"] = round(rec["copy_ceiling_gbps"], 2)
        line["frac_of_copy_ceiling"] = round(rec["frac_of_copy_ceiling"], 4)
        line["memcpy_ceiling_gbps"] = round(rec["memcpy_ceiling_gbps"], 2)
        line["frac_of_memcpy_ceiling"] = round(rec["frac_of_memcpy_ceiling"], 4)
    line["device"] = device_info()
    if per_config:
        line["per_config"] = dict(per_config, note="measured before the headline: graph replays over rotating "
                                                   "sets (HBM-cold), per call; parity by tests/test_parity_gpu.py::"
                                                   "test_stated_workloads_full_size")
    if args.all:
        for name, other in inputs.EVERY_WORKLOAD.items():
            if name == w.name:
                continue
            _, r = bench_workload(other, args.steps, args.warmup, args.seed, graph=True,
                                  timed_graph=timed_as_graph(other, args))
            log("# workload:", json.dumps(r))
    if args.cpu_seconds > 0:
        line["cpu_baseline"] = cpu_baseline(w, t, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

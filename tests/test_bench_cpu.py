"""Host-side logic of bench.py that needs no GPU."""
import os
import subprocess
import sys

import bench
from memory_bound_rmsnorm_amd import _build, inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr and p.stdout == ""


def test_rotation_covers_two_gib():
    for w in inputs.ALL_WORKLOADS.values():
        n = bench.n_sets_for(w)
        per = w.algorithmic_bytes - w.hidden * w.elem_size
        assert n >= 2 and n * per >= 2 << 30


def test_digests_are_per_kernel_family():
    assert _build.source_digest("fwd") != _build.source_digest("bwd")
    assert "rmsnorm_bwd_kernels.hpp" in _build.KERNEL_SOURCES["bwd"]
    assert not any("bwd" in n for n in _build.KERNEL_SOURCES["fwd"])


def test_traffic_is_read_only_while_sources_match(monkeypatch):
    w = inputs.WORKLOADS[inputs.HEADLINE]
    path = os.path.join(bench.PROFILE_DIR, "pmc_traffic_rms_vec_kernel_%s.txt" % w.name)
    assert os.path.exists(path)
    vals = dict(l.split(":", 1) for l in open(path) if ":" in l and not l.startswith("#"))
    monkeypatch.setattr(_build, "source_digest", lambda family="fwd": vals["source_sha256"].strip())
    launch = dict(kv.split("=") for kv in vals["launch_config"].split())
    launch = {k: (v if k == "path" else int(v)) for k, v in launch.items()}
    t = bench.load_traffic(w, launch)
    assert t is not None and abs(t / w.algorithmic_bytes - 1) < 0.05
    assert bench.load_traffic(w, dict(launch, waves_per_row=4)) is None
    monkeypatch.setattr(_build, "source_digest", lambda family="fwd": "0" * 64)
    assert bench.load_traffic(w, launch) is None
    assert bench.load_traffic(w, dict(launch, path="two_pass")) is None


def test_cpu_baseline_uses_every_usable_cpu_and_one_thread():
    """The oracle timed on all CPUs this process may use and on one thread,
    medians of several timed runs, with the host recorded."""
    w = inputs.custom(256, 1024, "bf16", False)
    t = inputs.make(w, seed=0)
    rec = bench.cpu_baseline(w, t, 0.8)
    n, detail = bench.host_cpus()
    assert rec["cores"] == n and rec["kind"] == "oracle" and rec["unit"] == "GB/s"
    assert len(rec["runs_gbps"]) == 5 and rec["value"] > 0
    assert rec["one_thread"]["threads"] == 1 and len(rec["one_thread"]["runs_gbps"]) == (3 if n > 1 else 5)
    assert rec["host"]["affinity_cpus"] >= n


def test_spread_statistics():
    s = bench.spread_us([3e-6, 1e-6, 2e-6, 4e-6, 10e-6], 7)
    assert s["us_median"] == 3.0 and s["us_min"] == 1.0 and s["us_p90"] == 10.0
    assert s["samples"] == 5 and s["launches_per_sample"] == 7
    assert bench.percentile(list(range(1, 101)), 90) == 90


def test_stated_configurations_are_the_five_workloads():
    assert set(bench.STATED.values()) == set(inputs.WORKLOADS) - {"bf16_shard_2048x8192"}
    assert bench.STATED["C4"] == inputs.HEADLINE


def test_timing_method_follows_the_step_size():
    """K eager calls for steps of >= 128 MiB (the headline among them), one
    graph replay for smaller ones; --graph and --eager force either."""
    from types import SimpleNamespace as NS
    plain = NS(graph=False, eager=False)
    w = inputs.EVERY_WORKLOAD
    assert not bench.timed_as_graph(w[inputs.HEADLINE], plain)
    assert not bench.timed_as_graph(w["bf16_residual_12289x5120"], plain)
    assert not bench.timed_as_graph(w["bf16_ln_8192x4096"], plain)
    assert bench.timed_as_graph(w["bf16_prefill_4096x2048"], plain)
    assert bench.timed_as_graph(w["bf16_kv_prefill_4x4096_576"], plain)
    assert bench.timed_as_graph(w[inputs.HEADLINE], NS(graph=True, eager=False))
    assert not bench.timed_as_graph(w["fp32_64x2048"], NS(graph=False, eager=True))


def test_agreement_report():
    import numpy as np
    a = np.array([0x3F80, 0x3F81, 0xBF80, 0x8000, 0x0000], np.uint16)
    b = np.array([0x3F80, 0x3F80, 0xBF81, 0x0000, 0x0001], np.uint16)
    r = bench._agreement(a, b, "bf16")
    assert r["max_ulp"] == 1 and r["ulp_histogram"] == {"0": 2, "1": 3, ">1": 0}
    assert bench._agreement(np.array([1, 255], np.uint8), np.array([1, -1], np.int8), "codes")["n_differing"] == 0
    assert bench._agreement(np.array([1, 254], np.uint8), np.array([1, -1], np.int8), "codes")["n_differing"] == 1


def test_cpu_baseline_sets_the_oracle_beside_the_gpu_sample():
    """The CPU-baseline leg compares its oracle output with the sample the
    bench took from the GPU; here the 'GPU' sample is the oracle's own output
    with one element moved by one ulp."""
    import oracle
    w = inputs.custom(64, 512, "bf16", True)
    t = inputs.make(w, seed=0)
    rows = bench.sample_rows(w)
    xb, rb, wb = (inputs.bits(t[k]) for k in ("x", "residual", "weight"))
    h, y = oracle.rmsnorm_residual_fwd(xb[:rows], rb[:rows], wb, w.eps)
    y = y.copy()
    y[3, 7] += 1
    t["gpu_sample"] = {"h": h, "y": y}
    rec = bench.cpu_baseline(w, t, 0.4)
    agree = rec["oracle_vs_gpu"]
    assert agree["rows"] == rows and agree["h"]["max_ulp"] == 0
    assert agree["y"]["max_ulp"] == 1 and agree["y"]["ulp_histogram"]["1"] == 1

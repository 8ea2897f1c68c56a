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

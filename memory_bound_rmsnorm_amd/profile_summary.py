"""Condense rocprofv3 CSV output into the short text summaries kept in profiles/.

    python -m memory_bound_rmsnorm_amd.profile_summary stats --csv K_kernel_stats.csv \\
        --workload bf16_16384x8192 --command "<the rocprofv3 command>"
    python -m memory_bound_rmsnorm_amd.profile_summary pmc --fetch F_counter_collection.csv \\
        --write W_counter_collection.csv --workload bf16_16384x8192 --command "<...>"

`stats` lists per-kernel call counts and durations from --kernel-trace --stats
and the bandwidth implied by the RMSNorm kernel's average duration.
`pmc` averages FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the RMSNorm
kernel and of the plain copy kernel run in the same process, scales the
RMSNorm counters by the copy's known-bytes / counted-bytes ratio, and records
the kernel-source digest so that bench.py quotes the traffic only while the
kernels are unchanged.
"""
import argparse
import csv
import os
import sys
from collections import defaultdict

from memory_bound_rmsnorm_amd import _build, inputs

COPY_KERNEL_TAG = "hbm_copy_kernel"


def _is_kv(w):
    return isinstance(w, inputs.KvWorkload)


def _targ(kind, v):
    """One template argument: (demangled text, Itanium-mangled text)."""
    if kind == "class":
        return "mbr::" + v, "NS_%d%sE" % (len(v), v)
    if kind == "bool":
        return ("true" if v else "false"), "Lb%dE" % int(bool(v))
    return str(v), ("Li%dE" % v if v >= 0 else "Lin%dE" % -v)


def _instance(name, args):
    """(demangled 'mbr::name<...>' prefix, mangled fragment) of one kernel instance."""
    parts = [_targ(k, v) for k, v in args]
    return ("mbr::%s<%s>" % (name, ", ".join(d for d, _ in parts)),
            "%sI%sEEv" % (name, "".join(m for _, m in parts)))


def kernel_instances(w):
    """The kernel instances one step of workload w launches with the library's
    automatic configuration on 16-byte-aligned buffers, in launch order."""
    e = ("class", "F32" if w.dtype == "f32" else "Bf16")
    if _is_kv(w):
        k = kv_launch(w)
        if k["path"] == "vector":
            nv = w.norm_dim // (4 if w.dtype == "f32" else 8)
            masked = k["lanes_per_row"] * k["norm_vectors_per_lane"] != nv
            return [_instance("kv_vec_kernel", [e, ("int", k["norm_vectors_per_lane"]), ("bool", masked),
                                                ("int", w.rope_style), ("int", k["lanes_per_row"])])]
        return [_instance("kv_elem_kernel", [e, ("int", w.rope_style)])]
    cfg = launch_config(w)
    v = 4 if w.dtype == "f32" else 8
    units = w.hidden // v
    lpr = cfg.lanes_per_row or 64
    lanes = lpr if lpr < 64 else 64 * cfg.waves_per_row
    per = cfg.items_per_lane
    masked = lanes * per != units
    wpr, path = cfg.waves_per_row, cfg.path
    if w.backward:
        if path == 1:
            row = _instance("rms_bwd_vec_kernel", [e, ("int", wpr), ("int", per), ("bool", masked), ("bool", True),
                                                   ("int", lpr)])
        elif path == 2:
            row = _instance("rms_bwd_elem_kernel", [e, ("int", wpr), ("int", per), ("bool", True)])
        else:
            row = _instance("rms_bwd_twopass_kernel", [e, ("bool", True), ("bool", True)])
        return [row, _instance("rms_bwd_dw_kernel", [e])]
    if w.layernorm:
        if path == 1:
            return [_instance("ln_vec_kernel", [e, ("int", wpr), ("int", per), ("bool", masked),
                                                ("bool", bool(cfg.weight_lds)), ("int", lpr)])]
        if path == 2:
            return [_instance("ln_elem_kernel", [e, ("int", wpr), ("int", per)])]
        return [_instance("ln_multipass_kernel", [e, ("bool", True)])]
    qt = {None: 0, "int8": 1, "fp8": 2}[w.quant]
    if path == 1:
        return [_instance("rms_vec_kernel", [e, ("int", wpr), ("int", per), ("bool", masked), ("bool", w.fused),
                                             ("int", qt), ("int", lpr)])]
    if path == 2:
        return [_instance("rms_elem_kernel", [e, ("int", wpr), ("int", per), ("bool", w.fused), ("int", qt)])]
    if path == 4:
        # any alignment; bf16 rows of an odd width on aligned buffers take the
        # shifted frame when the launch covers one more element, which always
        # launches the masked kernel
        frame = w.dtype == "bf16" and w.hidden % 2 != 0 and lanes * per >= (w.hidden + 1) // v
        return [_instance("rms_any_kernel", [e, ("int", wpr), ("int", per), ("bool", frame or lanes * per != units),
                                             ("bool", w.fused), ("int", qt)])]
    if path == 5:  # rms_stage_kernel<E, RV, CH, FUSED>, CH as rmsnorm_misc.hip instantiates it
        ch = {(False, 10): 10, (True, 6): 5, (True, 7): 4}[(w.fused, per)]
        return [_instance("rms_stage_kernel", [e, ("int", per), ("int", ch), ("bool", w.fused)])]
    return [_instance("rms_twopass_kernel", [e, ("bool", True), ("bool", w.fused), ("int", qt)])]


def _step_kernels(w):
    """Predicates for the kernels one step of workload w launches, once each
    (the exact template instances of its automatic configuration): the
    forward kernel, or the backward row kernel plus the dweight reduction."""
    return [(lambda k, d=d: d in k) for d, _ in kernel_instances(w)]


def _family(w):
    if _is_kv(w):
        return "kv"
    return "bwd" if w.backward else "ln" if w.layernorm else "fwd"


def _title(w):
    if _is_kv(w):
        return "KV RMSNorm + RoPE + cache %s, %d tokens x %d heads x (%d + %d)" % (
            w.dtype, w.tokens, w.heads, w.norm_dim, w.rope_dim)
    return "%s %s [%d, %d]%s" % ("LayerNorm" if w.layernorm else "RMSNorm", w.dtype, w.rows, w.hidden,
                                 " fused residual" if w.fused else " backward" if w.backward else "")


def stats(args):
    w = inputs.EVERY_WORKLOAD[args.workload]
    with open(args.csv) as f:
        rows = list(csv.DictReader(f))
    out = ["# rocprofv3 --kernel-trace --stats summary: %s" % _title(w),
           "# command: %s" % args.command,
           "# algorithmic bytes per call: %d" % w.algorithmic_bytes,
           "%-90s %6s %12s %12s %12s" % ("kernel", "calls", "avg_us", "min_us", "max_us")]
    step_avg = []
    preds = _step_kernels(w)
    for r in rows:
        name = r["Name"]
        short = name if len(name) <= 90 else name[:87] + "..."
        avg = float(r["AverageNs"]) / 1e3
        out.append("%-90s %6s %12.3f %12.3f %12.3f" % (short, r["Calls"], avg, float(r["MinNs"]) / 1e3,
                                                        float(r["MaxNs"]) / 1e3))
    for pred in preds:
        hit = [r for r in rows if pred(r["Name"])]
        if hit:
            step_avg.append(float(hit[0]["AverageNs"]) / 1e3)
    if len(step_avg) == len(preds):
        t = sum(step_avg)
        if getattr(w, "backward", False):
            out.append("bwd_row_kernel_avg_us: %.3f" % step_avg[0])
            out.append("bwd_dw_kernel_avg_us: %.3f" % step_avg[1])
            out.append("step_avg_us: %.3f" % t)
            out.append("row_kernel_gbps_from_avg: %.1f" % (w.algorithmic_bytes / step_avg[0] / 1e3))
        else:
            out.append("rmsnorm_kernel_avg_us: %.3f" % t)
        out.append("rmsnorm_gbps_from_avg: %.1f" % (w.algorithmic_bytes / t / 1e3))
        out.append("rmsnorm_frac_of_8TBps: %.4f" % (w.algorithmic_bytes / t / 1e3 / 8000.0))
    # The average above covers every dispatch of the run: warm-up, the eager
    # pass and the graph replays.  The window below picks the dispatches that
    # a bench line's own HIP events timed (counted from the end of the run,
    # in launch order), from the per-dispatch trace next to the stats file.
    trace = os.path.join(os.path.dirname(args.csv), os.path.basename(args.csv).replace("kernel_stats", "kernel_trace"))
    if os.path.exists(trace) and trace != args.csv and len(step_avg) == len(preds) and args.window_count > 0:
        with open(trace) as f:
            disp = sorted(csv.DictReader(f), key=lambda r: int(r["Start_Timestamp"]))
        timed = []
        for pred in preds:
            d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in disp if pred(r["Kernel_Name"])]
            a = len(d) - args.window_from_end
            if a >= 0 and a + args.window_count <= len(d):
                win = d[a:a + args.window_count]
                timed.append((sum(win) / len(win), sorted(win)[len(win) // 2]))
        if len(timed) == len(preds):
            t = sum(x[0] for x in timed)
            out.append("timed_window: %s" % args.window_note)
            out.append("timed_window_dispatches: %d (from %d before the end)" % (args.window_count,
                                                                                 args.window_from_end))
            out.append("timed_window_avg_us: %.3f" % t)
            out.append("timed_window_median_us: %.3f" % sum(x[1] for x in timed))
            out.append("timed_window_gbps: %.1f" % (w.algorithmic_bytes / t / 1e3))
            out.append("timed_window_frac_of_8TBps: %.4f" % (w.algorithmic_bytes / t / 1e3 / 8000.0))
    print("\n".join(out))


def _counter_means(path, counter):
    per_kernel = defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") != counter:
                continue
            per_kernel[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in per_kernel.items()}, {k: len(v) for k, v in per_kernel.items()}


def _pick(means, pred):
    names = [k for k in means if pred(k)]
    if not names:
        raise SystemExit("no matching kernel in counter file")
    return names[0], means[names[0]]


def pmc(args):
    w = inputs.EVERY_WORKLOAD[args.workload]
    fm, fn = _counter_means(args.fetch, "FETCH_SIZE")
    wm, wn = _counter_means(args.write, "WRITE_SIZE")
    rname, rfetch, rwrite, ndisp = [], 0.0, 0.0, []
    for pred in _step_kernels(w):
        n, f = _pick(fm, pred)
        _, wr = _pick(wm, pred)
        rname.append(n)
        ndisp.append(fn[n])
        rfetch += f
        rwrite += wr
    rname = " + ".join(rname)
    cname, cfetch = _pick(fm, lambda k: COPY_KERNEL_TAG in k)
    _, cwrite = _pick(wm, lambda k: COPY_KERNEL_TAG in k)
    # read == written per dispatch: the copy ceiling of the workload the run was for
    copy_bytes = inputs.EVERY_WORKLOAD[args.copy_workload or args.workload].copy_bytes
    fscale = copy_bytes / (cfetch * 1024.0)
    wscale = copy_bytes / (cwrite * 1024.0)
    read_alg = w.read_bytes
    write_alg = w.write_bytes
    traffic = rfetch * 1024 * fscale + rwrite * 1024 * wscale
    out = ["# rocprofv3 --pmc summary: HBM traffic of %s" % _title(w),
           "# fetch command: %s" % args.command_fetch,
           "# write command: %s" % args.command_write,
           "# FETCH_SIZE / WRITE_SIZE are KiB per dispatch, averaged over dispatches; the copy kernel",
           "# moves a known byte count in the same process and calibrates both counters.",
           "rmsnorm_kernel: %s" % rname.replace(":", ";"),
           "rmsnorm_dispatches_counted: %d" % min(ndisp),
           "rmsnorm_fetch_kib_per_dispatch: %.1f" % rfetch,
           "rmsnorm_write_kib_per_dispatch: %.1f" % rwrite,
           "copy_kernel: %s (the copy ceiling of %s)" % (COPY_KERNEL_TAG, args.copy_workload or args.workload),
           "copy_bytes_read_and_written_per_dispatch: %d" % copy_bytes,
           "copy_fetch_kib_per_dispatch: %.1f" % cfetch,
           "copy_write_kib_per_dispatch: %.1f" % cwrite,
           "copy_fetch_scale: %.5f" % fscale,
           "copy_write_scale: %.5f" % wscale,
           "algorithmic_read_bytes: %d" % read_alg,
           "algorithmic_write_bytes: %d" % write_alg,
           "scaled_read_bytes: %.0f" % (rfetch * 1024 * fscale),
           "scaled_write_bytes: %.0f" % (rwrite * 1024 * wscale),
           "traffic_bytes_per_launch: %.0f" % traffic,
           "traffic_over_algorithmic: %.4f" % (traffic / w.algorithmic_bytes),
           "launch_config: %s" % _launch_config(w),
           "source_sha256: %s" % _build.source_digest(_family(w))]
    print("\n".join(out))


def kv_launch(w):
    """The kernel kv_rmsnorm_rope_cache runs for workload w on 16-byte-aligned
    buffers (the library's own choice, kv_select_config)."""
    import torch
    import memory_bound_rmsnorm_amd as mbr
    c = mbr.kv_select_config(w.tokens, w.heads, w.norm_dim, w.rope_dim, w.rope_style,
                             torch.float32 if w.dtype == "f32" else torch.bfloat16, True)
    vec = c.path == mbr.PATH_VECTOR
    lanes = c.lanes_per_row or 64
    return {"path": "vector" if vec else "element", "norm_vectors_per_lane": c.items_per_lane if vec else 0,
            "lanes_per_row": lanes if vec else 64, "rope_style": "pairs" if w.rope_style == 1 else "halves",
            "rows_per_workgroup": 4 * (64 // lanes) if vec else 4}


def launch_config(w):
    """The automatic configuration for workload w on 16-byte-aligned buffers."""
    import torch
    import memory_bound_rmsnorm_amd as mbr
    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    if w.backward:
        return mbr.rmsnorm_select_bwd_config(w.rows, w.hidden, dt, True)
    if w.layernorm:
        return mbr.layernorm_select_config(w.rows, w.hidden, dt, True)
    select = mbr.rmsnorm_select_quant_config if w.quant else mbr.rmsnorm_select_config
    return select(w.rows, w.hidden, dt, True, w.fused)


def launch_dict(w):
    return kv_launch(w) if _is_kv(w) else launch_config(w).as_dict()


def _launch_config(w):
    return " ".join("%s=%s" % kv for kv in launch_dict(w).items())


def resources(args):
    """Compile-time register/scratch/occupancy report of the built kernels,
    condensed: totals plus the kernels the stated workloads launch."""
    with open(_build.RESOURCE_USAGE) as f:
        lines = [l.strip() for l in f if l.strip()]
    spill = [l for l in lines if "| scratch 0 |" not in l or "VGPR spill 0" not in l or "SGPR spill 0" not in l]
    out = ["# compile-time resource usage of librmsnorm.so (gfx950), from hipcc -Rpass-analysis=kernel-resource-usage",
           "# command: %s" % args.command,
           "kernels_built: %d" % len(lines),
           "kernels_with_scratch_or_spills: %d" % len(spill)]
    for name, w in list(inputs.ALL_WORKLOADS.items()) + list(inputs.KV_WORKLOADS.items()):
        for _, mangled in kernel_instances(w):
            hit = [l for l in lines if mangled in l]
            out.append("%s -> %s | %s | %s" % (name, launch_dict(w), mangled.split("I", 1)[0],
                                               hit[0].split("|", 1)[1].strip() if hit else "?"))
    print("\n".join(out))


def occupancy(args):
    """Runtime occupancy of a workload's kernels from two rocprofv3 --pmc runs
    (the derived counters OccupancyPercent and MeanOccupancyPerCU), next to the
    copy kernel measured in the same process."""
    w = inputs.EVERY_WORKLOAD[args.workload]
    pm, pn = _counter_means(args.percent, "OccupancyPercent")
    mm, _ = _counter_means(args.mean, "MeanOccupancyPerCU")
    out = ["# rocprofv3 --pmc summary: runtime occupancy of %s" % _title(w),
           "# OccupancyPercent command: %s" % args.command_percent,
           "# MeanOccupancyPerCU command: %s" % args.command_mean,
           "# OccupancyPercent: resident wave-cycles as a share of the maximum (32 waves per CU on gfx950);",
           "# MeanOccupancyPerCU: mean resident waves per CU; both averaged over the dispatches counted."]
    for i, pred in enumerate(_step_kernels(w)):
        n, pv = _pick(pm, pred)
        _, mv = _pick(mm, pred)
        out += ["kernel_%d: %s" % (i, n.replace(":", ";")),
                "kernel_%d_dispatches_counted: %d" % (i, pn[n]),
                "kernel_%d_occupancy_percent: %.1f" % (i, pv),
                "kernel_%d_mean_waves_per_cu: %.2f" % (i, mv)]
    cn, cp = _pick(pm, lambda k: COPY_KERNEL_TAG in k)
    _, cm = _pick(mm, lambda k: COPY_KERNEL_TAG in k)
    out += ["copy_kernel: %s" % COPY_KERNEL_TAG,
            "copy_occupancy_percent: %.1f" % cp,
            "copy_mean_waves_per_cu: %.2f" % cm,
            "launch_config: %s" % _launch_config(w),
            "source_sha256: %s" % _build.source_digest(_family(w))]
    print("\n".join(out))


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--window-from-end", type=int, default=0,
                   help="first dispatch of the timed window, counted from the end of each kernel's dispatches")
    s.add_argument("--window-count", type=int, default=0, help="dispatches in the timed window (0: none)")
    s.add_argument("--window-note", default="", help="what the timed window is")
    s.add_argument("--csv", required=True)
    s.add_argument("--workload", default=inputs.HEADLINE, choices=sorted(inputs.EVERY_WORKLOAD))
    s.add_argument("--command", required=True)
    p = sub.add_parser("pmc")
    p.add_argument("--fetch", required=True)
    p.add_argument("--write", required=True)
    p.add_argument("--workload", default=inputs.HEADLINE)
    p.add_argument("--copy-workload", default=None,
                   help="workload whose copy ceiling the run's copy kernel moved (default: --workload)")
    p.add_argument("--command-fetch", required=True)
    p.add_argument("--command-write", required=True)
    o = sub.add_parser("occupancy")
    o.add_argument("--percent", required=True)
    o.add_argument("--mean", required=True)
    o.add_argument("--workload", default=inputs.HEADLINE)
    o.add_argument("--command-percent", required=True)
    o.add_argument("--command-mean", required=True)
    r = sub.add_parser("resources")
    r.add_argument("--command", default="python -m memory_bound_rmsnorm_amd._build && "
                                        "python -m memory_bound_rmsnorm_amd.profile_summary resources")
    a = ap.parse_args(argv)
    {"stats": stats, "pmc": pmc, "occupancy": occupancy, "resources": resources}[a.cmd](a)


if __name__ == "__main__":
    sys.exit(main())

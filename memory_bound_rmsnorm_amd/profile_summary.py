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

RMS_KERNEL_TAGS = ("rms_vec_kernel", "rms_elem_kernel", "rms_twopass_kernel")
BWD_KERNEL_TAGS = ("rms_bwd_vec_kernel", "rms_bwd_elem_kernel", "rms_bwd_twopass_kernel")
BWD_DW_TAG = "rms_bwd_dw_kernel"
LN_KERNEL_TAGS = ("ln_vec_kernel", "ln_elem_kernel", "ln_multipass_kernel")
KV_KERNEL_TAGS = ("kv_vec_kernel", "kv_elem_kernel")


def _is_kv(w):
    return isinstance(w, inputs.KvWorkload)
COPY_KERNEL_TAG = "hbm_copy_kernel"


def _is_rms(name):
    return any(t in name for t in RMS_KERNEL_TAGS)


def _step_kernels(w):
    """Predicates for the kernels one step of workload w launches, once each:
    the forward kernel, or the backward row kernel plus the dweight reduction."""
    if _is_kv(w):
        return [lambda k: any(t in k for t in KV_KERNEL_TAGS)]
    if w.backward:
        return [lambda k: any(t in k for t in BWD_KERNEL_TAGS), lambda k: BWD_DW_TAG in k]
    if w.layernorm:
        return [lambda k: any(t in k for t in LN_KERNEL_TAGS)]
    return [_is_rms]


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
    # pass and the graph replays.  bench.py's timed steps are the last
    # args.steps dispatches of each kernel (the timed graph replay); their
    # average, from the per-dispatch trace next to the stats file, is the
    # figure to set beside the bench line's own HIP-event reading.
    trace = os.path.join(os.path.dirname(args.csv), os.path.basename(args.csv).replace("kernel_stats", "kernel_trace"))
    if os.path.exists(trace) and trace != args.csv and len(step_avg) == len(preds):
        with open(trace) as f:
            disp = list(csv.DictReader(f))
        timed = []
        for pred in preds:
            d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in disp if pred(r["Kernel_Name"])]
            if len(d) >= args.steps:
                timed.append(sum(d[-args.steps:]) / args.steps)
        if len(timed) == len(preds):
            t = sum(timed)
            out.append("timed_steps: the last %d dispatches of each kernel (the timed graph replay)" % args.steps)
            out.append("timed_steps_avg_us: %.3f" % t)
            out.append("timed_steps_gbps: %.1f" % (w.algorithmic_bytes / t / 1e3))
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
    copy_bytes = w.copy_bytes  # read == written per dispatch, as bench.py's copy ceiling
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
           "copy_kernel: %s" % COPY_KERNEL_TAG,
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
    for name, w in inputs.ALL_WORKLOADS.items():
        cfg = launch_config(w)
        e = "F32" if w.dtype == "f32" else "Bf16"
        per = cfg.items_per_lane
        units = w.hidden // (4 if w.dtype == "f32" else 8)
        masked = 64 * cfg.waves_per_row * per != units
        if w.backward:
            if cfg.path == 1:  # rms_bwd_vec_kernel<E, WPR, VPL, MASKED, DW, LPR>
                lpr = cfg.lanes_per_row or 64
                masked = (lpr if lpr < 64 else 64 * cfg.waves_per_row) * per != units
                mangled = "rms_bwd_vec_kernelINS_%d%sELi%dELi%dELb%dELb1ELi%dEEEv" % (
                    len(e), e, cfg.waves_per_row, per, int(masked), lpr)
            else:  # rms_bwd_elem_kernel<E, WPR, EPL, DW>, rms_bwd_twopass_kernel<E, VEC, DW>
                fam = {2: "rms_bwd_elem_kernel", 3: "rms_bwd_twopass_kernel"}[cfg.path]
                mangled = "%sINS_%d%sELi%dELi%dELb%dELb1EEEv" % (fam, len(e), e, cfg.waves_per_row, per, int(masked))
        elif w.layernorm:
            mangled = "ln_vec_kernelINS_%d%sELi%dELi%dELb%dELb%dEEEv" % (len(e), e, cfg.waves_per_row, per, int(masked),
                                                                   int(bool(cfg.weight_lds)))
        else:
            qt = {None: 0, "int8": 1, "fp8": 2}[w.quant]
            if cfg.path == 1:  # rms_vec_kernel<E, WPR, VPL, MASKED, FUSED, QT, LPR>
                lpr = cfg.lanes_per_row or 64
                masked = (lpr if lpr < 64 else 64 * cfg.waves_per_row) * per != units
                mangled = "rms_vec_kernelINS_%d%sELi%dELi%dELb%dELb%dELi%dELi%dEEEv" % (
                    len(e), e, cfg.waves_per_row, per, int(masked), int(w.fused), qt, lpr)
            elif cfg.path == 2:  # rms_elem_kernel<E, WPR, EPL, FUSED, QT>
                mangled = "rms_elem_kernelINS_%d%sELi%dELi%dELb%dELi%dEEEv" % (len(e), e, cfg.waves_per_row, per,
                                                                              int(w.fused), qt)
            else:  # rms_twopass_kernel<E, VEC, FUSED, QT>
                mangled = "rms_twopass_kernelINS_%d%sELb1ELb%dELi%dEEEv" % (len(e), e, int(w.fused), qt)
        hit = [l for l in lines if mangled in l]
        out.append("%s -> %s | %s" % (name, cfg.as_dict(), hit[0].split("|", 1)[1].strip() if hit else "?"))
    for name, w in inputs.KV_WORKLOADS.items():
        k = kv_launch(w)
        e = "F32" if w.dtype == "f32" else "Bf16"
        if k["path"] == "vector":
            masked = k["lanes_per_row"] * k["norm_vectors_per_lane"] != w.norm_dim // (4 if w.dtype == "f32" else 8)
            mangled = "kv_vec_kernelINS_%d%sELi%dELb%dELi%dELi%dEEEv" % (len(e), e, k["norm_vectors_per_lane"],
                                                                        int(masked), w.rope_style, k["lanes_per_row"])
        else:
            mangled = "kv_elem_kernelINS_%d%sELi%dEEEv" % (len(e), e, w.rope_style)
        hit = [l for l in lines if mangled in l]
        out.append("%s -> %s | %s" % (name, k, hit[0].split("|", 1)[1].strip() if hit else "?"))
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
    s.add_argument("--steps", type=int, default=200, help="timed steps of the traced bench run")
    s.add_argument("--csv", required=True)
    s.add_argument("--workload", default=inputs.HEADLINE, choices=sorted(inputs.EVERY_WORKLOAD))
    s.add_argument("--command", required=True)
    p = sub.add_parser("pmc")
    p.add_argument("--fetch", required=True)
    p.add_argument("--write", required=True)
    p.add_argument("--workload", default=inputs.HEADLINE)
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

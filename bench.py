#!/usr/bin/env python3
"""Benchmark of one rank's sharded mixed-precision optimizer step on one GPU.

A step is one pass of the whole hot path over one batch of resident
synthetic gradients: shard reduce of the P bf16 replicas with the average,
non-finite count and exact norm (bucketed where the workload says so), the
gated fused AdamW on fp32 master/m/v with the bf16 param write, and, for the
30B workload, the MXFP8 pack of the param shard (the all-gather payload).

Prints ONE JSON line: params/s of the shard (whole job = one GPU), HBM GB/s
against the fused-minimum bytes, the roofline of the dominant kernel measured
with HIP events inside the timed region, each kernel against the measured
ceiling of its bare access pattern on the same buffers, and the CPU oracle's
rate on a bounded sample of the same workload.  With the default 30B shard
the 7B shard (35 buckets) is timed in the same process as "secondary".
"""
import argparse
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, 8 TB/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "include", "zero_step.h")] + [
    os.path.join(ROOT, "zero_sharded_mixed_step_amd", "csrc", f)
    for f in ("zs_abi.hip", "zs_device.h", "zs_internal.h", "zs_kernels.hip")]
# kernel-name fragments of the launch kinds, as rocprofv3 reports them
KERNEL_NAMES = {"reduce": "zs::shard_reduce_kernel", "adamw": "zs::adamw_kernel",
                "mxfp8_pack": "zs::mxfp8_kernel"}   # the pattern kernels are not in zs::


def source_digest() -> str:
    """sha256 of the kernel sources: measured traffic is only reported for
    the exact kernels it was measured on."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="30b-shard-p8",
                    choices=["flat-1m-p4", "gpt2-small-p8", "1.3b-unsharded", "7b-shard-p8",
                             "30b-shard-p8", "30b-shard-p8-mxgrads"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="with the default 30B shard, skip the 7B shard's secondary timing")
    ap.add_argument("--cpu-sample", type=int, default=1 << 26,
                    help="elements of the CPU-oracle sample")
    ap.add_argument("--cpu-steps", type=int, default=3)
    ap.add_argument("--no-offload", action="store_true",
                    help="skip the offload bill (PCIe copies + all-cores CPU AdamW)")
    ap.add_argument("--cpu-threads", type=int, default=16,
                    help="threads of the all-cores oracle legs (capped by the host)")
    ap.add_argument("--no-recycle", action="store_true",
                    help="allocate the workload without first writing and releasing a "
                         "scratch allocation of its size (same as --memory-prep none)")
    ap.add_argument("--memory-prep", choices=("recycle", "spacer", "none"), default="recycle",
                    help="untimed set-up before the workload allocates: write and release "
                         "a scratch allocation (recycle), write and hold a 60 GB spacer "
                         "for the whole run (spacer), or nothing")
    ap.add_argument("--no-unfused", action="store_true",
                    help="skip timing the unfused single-operation chain")
    ap.add_argument("--trace-report", nargs=2, metavar=("PROF_DIR", "BENCH_LOG"),
                    help="no GPU: print the text summary of a rocprofv3 --kernel-trace --stats "
                         "run of this workload (PROF_DIR) and the bench line it printed "
                         "(BENCH_LOG)")
    ap.add_argument("--traffic-report", nargs="+", metavar="WORKLOAD",
                    help="no GPU: print the HBM-traffic table of these workloads from "
                         "profiles/hbm_traffic.json")
    ap.add_argument("--placement-report", nargs="+", metavar="PROF_DIR_AND_LOG",
                    help="no GPU: print the per-launch counters of --placement-probe runs, "
                         "given as pairs: rocprofv3 --pmc output dir, log of that run")
    ap.add_argument("--placement-probe", type=float, default=None, metavar="GB",
                    help="only time the step's reduce and AdamW launches in two placements: "
                         "the workload allocated first, then again after a held, written "
                         "spacer allocation of GB gigabytes")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for the HBM "
                         "byte counters)")
    ap.add_argument("--summarize-pmc", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH",
                                                          "COPY_WRITE"),
                    help="no GPU: turn four rocprofv3 --pmc output directories (FETCH_SIZE "
                         "and WRITE_SIZE of this workload, then of --copy-calibration) "
                         "into profiles/hbm_traffic.json and a text summary")
    return ap.parse_args()


MX_BYTES = 1 + 1.0 / 32        # MXFP8 codes + one scale byte per 32 elements


def per_elem_bytes(w, st):
    """Fused-minimum HBM bytes per shard element, per launch kind.  With the
    MXFP8 pack fused into AdamW its output bytes belong to the AdamW pass."""
    g_b = MX_BYTES if w.mx_grads else w.g_bytes
    P = w.P
    if st.path == "fused":
        kinds = {"adamw": P * g_b + 26}
    elif st.path == "materialize":
        kinds = {"reduce": P * g_b + 4, "adamw": 4 + 26}
    else:
        kinds = {"reduce": P * g_b, "adamw": P * g_b + 26}
    if w.pack:
        if st.fuse_pack:
            kinds["adamw"] += MX_BYTES
        else:
            kinds["mxfp8_pack"] = 2 + MX_BYTES
    return kinds


def unfused_bytes(w):
    """HBM bytes per element of the single-operation chain: every operation
    reads its operands from HBM and writes its result back."""
    b = w.P * w.g_bytes + 4      # s = sum of replicas
    b += 4 + 4                   # g = s * inv_scale
    b += 4                       # norm state of g
    b += 4 + 4                   # g' = g * coef
    b += 8 + 4                   # m
    b += 8 + 4                   # v
    b += 8 + 4                   # u = m / (sqrt(v)/sqrt_bc2 + eps)
    b += 8 + 4                   # master
    b += 4 + 2                   # bf16 param
    if w.pack:
        b += 2 + MX_BYTES        # MXFP8 pack of the param
    return b


def _read_counters(d):
    """{kernel name: [value per dispatch, ...]} from a rocprofv3 csv directory."""
    import csv
    import glob
    out = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def summarize_pmc(w, dirs, cmdline):
    """Scale FETCH_SIZE/WRITE_SIZE (KiB per dispatch) by what the same counters
    read for a plain 1 GiB copy, and store HBM bytes per launch per kind."""
    fetch, write, cfetch, cwrite = (_read_counters(d) for d in dirs)
    copy = [k for k in cfetch if "copyBuffer" in k or "copy" in k.lower()]
    if not copy:
        raise SystemExit("no copy kernel in the calibration counters")
    gib = float(1 << 30)
    f_factor = gib / (1024 * statistics.mean(cfetch[copy[0]]))
    w_factor = gib / (1024 * statistics.mean(cwrite[copy[0]]))
    kinds = {}
    for kind, frag in KERNEL_NAMES.items():
        fk = [k for k in fetch if frag in k]
        wk = [k for k in write if frag in k]
        if not fk or not wk:
            continue
        fv = [v for k in fk for v in fetch[k]]
        wv = [v for k in wk for v in write[k]]
        kinds[kind] = {"dispatches": len(fv),
                       "fetch_kib": round(statistics.mean(fv), 1),
                       "write_kib": round(statistics.mean(wv), 1),
                       "hbm_bytes": round(1024 * (statistics.mean(fv) * f_factor +
                                                  statistics.mean(wv) * w_factor))}
    data = {}
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as fh:
            data = json.load(fh)
    data[w.name] = {"source_digest": source_digest(), "fetch_factor": round(f_factor, 4),
                    "write_factor": round(w_factor, 4), "kinds": kinds, "command": cmdline}
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(data, fh, indent=1, sort_keys=True)
    print(json.dumps(data[w.name]))


def _path_of(w):
    """The pass structure ShardStep picks for the workload (pure function)."""
    sys.path.insert(0, ROOT)
    from zero_sharded_mixed_step_amd.step import choose_path
    return choose_path(w.P, MX_BYTES if w.mx_grads else w.g_bytes, w.gated, w.mx_grads)


def algorithmic_bytes_per_launch(w, kind):
    """Fused-minimum bytes of one launch of `kind`: bytes per element times
    the elements one launch covers (a bucket for the bucketed reduce)."""
    from types import SimpleNamespace
    per = per_elem_bytes(w, SimpleNamespace(path=_path_of(w), fuse_pack=w.pack))
    if kind == "mxfp8_pack":
        return (2 + MX_BYTES) * w.S
    elems = w.bucket if (kind == "reduce" and w.bucket) else w.S
    return per[kind] * elems


def step_kernels(w):
    """(rocprofv3 kernel name, role, launches per step) of the kernels one
    step of the workload launches, from the pass structure and the library's
    dispatch: reduce template <replica dtype, P, writes g, norm, pipelined,
    one-shot> (one-shot with P >= 4 above 2^27 elements a launch, where
    ShardStep passes the workspace, then a fold launch; else pipelined for
    P in {4, 8}), AdamW template <gradient source (-1: materialised g), P,
    bf16 param, fused MXFP8, tiles per workgroup, first tiles loaded before
    the gate>."""
    from zero_sharded_mixed_step_amd.step import ONESHOT_MIN
    path = _path_of(w)
    dt = 2 if w.mx_grads else (1 if w.grad_bf16 else 0)
    pt = w.P if w.P in (1, 2, 4, 8) else 0
    per_launch = w.bucket or w.S
    oneshot = w.P >= 4 and per_launch > ONESHOT_MIN
    pipe = "true" if (not oneshot and pt >= 4 and per_launch <= (1 << 27)) else "false"
    form = f"{pipe}, {'true' if oneshot else 'false'}"
    launches = -(-w.S // w.bucket) if w.bucket else 1
    mx = "true" if w.pack else "false"
    # AdamW tiles per workgroup: 2, or 1 where two would give fewer than two
    # workgroups per compute unit (256 on MI355X); the first tiles are loaded
    # before the gate on grids of up to 128 workgroups per compute unit
    ntiles = -(-(-(-w.S // 8)) // 256)
    g2 = -(-ntiles // 2)
    u = 1 if g2 < 2 * 256 else 2
    early = "true" if u == 1 or g2 <= 128 * 256 else "false"
    mx = f"{mx}, {u}, {early}"
    out = []
    fold = ("zs::slot_fold_kernel(zero_norm_acc*, zero_norm_acc*)",
            "adds the one-shot reduce's slots to the accumulator", launches)
    if path == "materialize":
        out.append((f"void zs::shard_reduce_kernel<{dt}, {pt}, true, true, {form}>"
                    "(zs::ReduceParams)", "reduce + norm, writes fp32 g", launches))
        if oneshot:
            out.append(fold)
        out.append((f"void zs::adamw_kernel<-1, 1, true, {mx}>(zs::AdamParams)",
                    "gated AdamW reading g" + (", fused MXFP8" if w.pack else ""), 1))
    elif path == "recompute":
        out.append((f"void zs::shard_reduce_kernel<{dt}, {pt}, false, true, {form}>"
                    "(zs::ReduceParams)", "norm-only pass over the replicas", launches))
        if oneshot:
            out.append(fold)
        out.append((f"void zs::adamw_kernel<{dt}, {pt}, true, {mx}>(zs::AdamParams)",
                    "gated AdamW reducing the replicas again"
                    + (", fused MXFP8" if w.pack else ""), 1))
    else:
        out.append((f"void zs::adamw_kernel<{dt}, {pt}, true, {mx}>(zs::AdamParams)",
                    "one pass: reduce + AdamW" + (", fused MXFP8" if w.pack else ""), 1))
    out.append(("zs::step_advance_kernel(long*, zero_norm_acc const*, int, double, int)",
                "device step counter", 1))
    return out


PROFILE_CMD = ("rocprofv3 --kernel-trace --stats --output-format csv -d $R/<PROF_DIR> "
               "-o run -- python3 $R/bench.py --config {cfg} --steps 5 --warmup 1 "
               "--no-cpu-baseline")


def trace_report(w, prof_dir, bench_log):
    """Text summary of a kernel-trace run: rocprofv3's per-kernel statistics
    and the bench line the same run printed."""
    import csv
    cols = ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs",
            "StdDev"]
    with open(os.path.join(prof_dir, "run_kernel_stats.csv")) as fh:
        rows = list(csv.DictReader(fh))
    line = next((ln.strip() for ln in open(bench_log) if ln.startswith("{")), None)
    cmd = PROFILE_CMD.format(cfg=w.name)
    if line and "command" in json.loads(line):
        args = json.loads(line)["command"].split()[2:]
        cmd = cmd.split(" -- ")[0] + " -- python3 $R/bench.py" + "".join(" " + a for a in args)
    prof_rel, log_rel = os.path.normpath(prof_dir), os.path.normpath(bench_log)
    cmd = cmd.replace("<PROF_DIR>", prof_rel) + f" > $R/{log_rel} 2>&1"
    print(f"# rocprofv3 kernel-trace summary: optimizer step, {w.name} ({w.title})")
    print("# MI355X (gfx950), one GPU.  Data (run from /tmp with TMPDIR=/tmp, repo at $R):")
    print("#   " + cmd)
    print(f"# This summary: python bench.py --trace-report {prof_rel} {log_rel} "
          f"--config {w.name}")
    print(f"# Pass structure: {_path_of(w)}; bucket: {w.bucket}.  Durations in ns.  The run "
          "also times the unfused chain (unfused_kernel<..>, gate_kernel, and")
    print("# shard_reduce_kernel / mxfp8_kernel launches of the chain); fill_kernel is the "
          "input generator and FillFunctor torch fills (set-up, untimed).")
    print(f"# Kernel sources digest (bench.py source_digest): {source_digest()}")
    if w.bucket:
        print("# Bucket reduces alternate over two streams and overlap: a launch lasts about "
              "twice its share of the step (the bench line's kernels.reduce is the whole "
              "bucketed pass, timed by events).")
    print("# Kernels of one step (role, launches per step, average ns from the table):")
    avg = {r["Name"]: float(r["AverageNs"]) for r in rows}
    for name, role, launches in step_kernels(w):
        key = name if name in avg else None
        got = f"{avg[key]:.0f} ns" if key else "NOT IN THE TABLE"
        print(f"#   {name.split('(')[0]}: {role}; {launches}/step; {got}")
    print("#")
    print(",".join(f'"{c}"' for c in cols))
    for r in rows:
        print(",".join([f'"{r["Name"]}"'] + [r[c] for c in cols[1:]]))
    print("#")
    print("# bench.py line printed by the same run (roofline.traffic is null there when the "
          "counters of these kernels were summarised after it):")
    print(line)


def traffic_report(names):
    """Text table of the HBM traffic per launch stored in hbm_traffic.json,
    against the algorithmic bytes of the same launch."""
    from synth import configs
    with open(TRAFFIC_FILE) as fh:
        data = json.load(fh)
    digests = sorted({data[n]["source_digest"] for n in names})
    print("# HBM traffic per launch from rocprofv3 counters: " + ", ".join(names))
    print(f"# MI355X (gfx950), one GPU.  Kernel sources digest: {', '.join(digests)}")
    print("# Counter runs (each its own process, from /tmp with TMPDIR=/tmp, repo at $R), "
          "for CTR in FETCH_SIZE WRITE_SIZE:")
    def counter_dir(cmd, i):
        # the i-th directory argument of a recorded --summarize-pmc command,
        # without its _FETCH_SIZE / _WRITE_SIZE suffix
        args = cmd.split()
        d = args[args.index("--summarize-pmc") + 1 + i]
        return d.rsplit("_", 2)[0] if d.endswith("_SIZE") else d
    first = data[names[0]]["command"]
    print(f"#   rocprofv3 --pmc $CTR --output-format csv -d $R/{counter_dir(first, 2)}_$CTR -o run "
          "-- python3 $R/bench.py --copy-calibration")
    for n in names:
        print(f"#   rocprofv3 --pmc $CTR --output-format csv -d "
              f"$R/{counter_dir(data[n]['command'], 0)}_$CTR -o run "
              f"-- python3 $R/bench.py --config {n} --steps 2 --warmup 1 --no-cpu-baseline "
              "--no-unfused --no-secondary")
    print("# Scaled (no GPU), the commands recorded in profiles/hbm_traffic.json:")
    for n in names:
        print("#   python " + data[n]["command"])
    print("#   -> profiles/hbm_traffic.json; this table: python bench.py --traffic-report "
          + " ".join(names))
    print("# HBM bytes = 1024 * (FETCH_SIZE * f + WRITE_SIZE * w); a plain 1 GiB copy reads "
          "FETCH_SIZE = 1 GiB / f and WRITE_SIZE = 1 GiB / w (in KiB), so:")
    for n in names:
        print(f"#   {n}: f = {data[n]['fetch_factor']:.4f}, w = {data[n]['write_factor']:.4f}")
    print("#")
    print(f"# {'workload':22s} {'kind':11s} {'dispatches':>10s} {'FETCH_SIZE KiB':>15s} "
          f"{'WRITE_SIZE KiB':>15s} {'HBM bytes/launch':>17s} {'algorithmic':>15s}  ratio")
    for n in names:
        w = configs.ALL[n]
        for kind, k in sorted(data[n]["kinds"].items()):
            alg = algorithmic_bytes_per_launch(w, kind)
            print(f"  {n:22s} {kind:11s} {k['dispatches']:10d} {k['fetch_kib']:15.1f} "
                  f"{k['write_kib']:15.1f} {k['hbm_bytes']:17d} {alg:15.0f}  "
                  f"{k['hbm_bytes'] / alg:.4f}")
    print("#")
    print("# reduce = shard_reduce_kernel (replicas -> fp32 g and norm state, or the norm "
          "state alone), adamw = adamw_kernel (master/m/v update, bf16 param, fused MXFP8 "
          "output where set), mxfp8_pack = mxfp8_kernel (standalone pack, and the set-up "
          "packing of MXFP8-stored replicas).")
    print("# Algorithmic bytes per element: reduce P*g_b + 4 (materialised g) or P*g_b (norm "
          "only); AdamW 30 with g read, P*g_b + 26 when it re-reduces the replicas, +1.03125 "
          "with the fused MXFP8 output; pack 3.03125.  The bucketed reduce launch covers one "
          "bucket.")


def placement_report(pairs):
    """Per-launch counters of the reduce and AdamW launches of placement-probe
    runs (one rocprofv3 --pmc pass each): the first half of the launches
    uses the buffers allocated first, the second half the same buffers after
    the spacer.  Also echoes each run's bench line."""
    import csv
    if len(pairs) % 2:
        raise SystemExit("--placement-report takes (dir, log) pairs")
    runs = [(pairs[i], pairs[i + 1]) for i in range(0, len(pairs), 2)]
    print("# Per-launch counters of the 30B-shard step's reduce and AdamW launches in two "
          "placements of the same buffers:")
    print("# allocated first in the process, then again after a held, written spacer "
          "(bench.py --placement-probe GB).")
    print("# MI355X (gfx950), one GPU.  One counter pass per run (its own process, from /tmp "
          "with TMPDIR=/tmp, repo at $R); each pass below gives its command.")
    print("# This summary: python bench.py --placement-report " + " ".join(
        f"{os.path.normpath(d)} {os.path.normpath(lg)}" for d, lg in runs))
    print(f"# Kernel sources digest (bench.py source_digest): {source_digest()}")
    print("# Launch durations (ms) are rocprofv3's per-dispatch timestamps under counter "
          "collection.  TCC_EA0 DRAM read requests are 128 B, write requests 64 B; GMI = "
          "inter-die.")
    logs = []
    for k, (d, log) in enumerate(runs, 1):
        with open(os.path.join(d, "run_counter_collection.csv")) as fh:
            rows = list(csv.DictReader(fh))
        launches, names = {}, []
        for r in rows:
            kn = r["Kernel_Name"]
            if "adamw_kernel" not in kn and "shard_reduce_kernel" not in kn:
                continue
            e = launches.setdefault(int(r["Dispatch_Id"]), {
                "kind": "adamw" if "adamw_kernel" in kn else "reduce",
                "ms": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6})
            c = r["Counter_Name"]
            if c not in names:
                names.append(c)
            e[c] = float(r["Counter_Value"])
        order = [launches[i] for i in sorted(launches)]
        spacer = next((json.loads(ln).get("spacer_gb") for ln in open(log)
                       if ln.startswith("{") and json.loads(ln).get("spacer_gb")), None)
        spacer = "GB" if spacer is None else f"{spacer:g}"
        print("#")
        print(f"# pass {k}: " + " ".join(names))
        print(f"#   rocprofv3 --pmc {' '.join(names)} --output-format csv -d "
              f"$R/{os.path.normpath(d)} -o run -- python3 "
              f"$R/bench.py --placement-probe {spacer} > $R/{os.path.normpath(log)}"
              " 2>&1")
        print("# placement  kind       ms  " + "  ".join(f"{c:>{max(14, len(c))}s}"
                                                      for c in names))
        for i, e in enumerate(order):
            pl = "first" if i < len(order) // 2 else "spacer"
            print(f"  {pl:9s}  {e['kind']:6s} {e['ms']:7.2f}  " + "  ".join(
                f"{e.get(c, float('nan')):>{max(14, len(c))}.0f}" for c in names))
        logs += [ln.strip() for ln in open(log) if ln.startswith("{")]
    print("#")
    print("# bench.py lines of the runs (in-process HIP events per launch):")
    for ln in logs:
        print("# " + ln)


def copy_calibration():
    """A plain device copy of 1 GiB, the reference kernel whose FETCH_SIZE /
    WRITE_SIZE counters convert counter readings into HBM bytes."""
    import torch
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(5):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / 5
    print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n,
                      "avg_ms": round(ms, 4), "gbps": round(8 * n / (ms * 1e-3) / 1e9, 1)}),
          flush=True)


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo where there is one)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(w, sample, steps, threads=1):
    """The CPU oracle on the first `sample` elements of the workload's shard
    (inputs generated beforehand): single-threaded as it stands, or with
    threads > 1 its threaded driver (32-aligned slices, bitwise the same
    result)."""
    import numpy as np

    import oracle as O
    import synth
    sample = min(sample, w.S)
    start = w.shard_start()
    master = synth.fill(w.master_spec(), start, sample, False, threads=8)
    m = np.zeros(sample, np.float32)
    v = np.zeros(sample, np.float32)
    param = np.zeros(sample, np.uint16)
    g_tmp = np.empty(sample, np.float32)
    reps = [synth.fill(w.grad_spec(1, k), start, sample, w.grad_bf16, threads=8)
            for k in range(w.P)]
    if w.mx_grads:
        sample = sample // 32 * 32
        reps = [O.mxfp8_pack(r[:sample]) for r in reps]
        master, m, v, param, g_tmp = (a[:sample] for a in (master, m, v, param, g_tmp))
    inv = O.inv_scale(w.P, w.loss_scale)
    from concurrent.futures import ThreadPoolExecutor
    ex = ThreadPoolExecutor(threads) if threads > 1 else None
    psample = sample // 32 * 32
    cuts = O._cuts(psample, threads)

    def decode_all():
        if ex is None:
            return [O.mxfp8_decode(e, sc) for e, sc in reps]
        out = [np.empty(sample, np.float32) for _ in reps]

        def part(c):
            for o, (e, sc) in zip(out, reps):
                o[c[0]:c[1]] = O.mxfp8_decode(e[c[0]:c[1]], sc[c[0] // 32:c[1] // 32])
        list(ex.map(part, cuts))
        return out

    def pack_param():
        if ex is None:
            return O.mxfp8_pack(param[:psample])
        list(ex.map(lambda c: O.mxfp8_pack(param[c[0]:c[1]]), cuts))

    t0 = time.perf_counter()
    for t in range(1, steps + 1):
        # MXFP8-stored replicas: the decode is part of the timed step
        g_in = decode_all() if w.mx_grads else reps
        if ex is not None:
            O.step_parallel(g_in, inv, w.max_norm, w.check_overflow, w.lr, w.beta1, w.beta2,
                            w.eps, w.wd, t, master, m, v, param, g_tmp=g_tmp, threads=threads)
        else:
            O.step(g_in, inv, w.max_norm, w.check_overflow, w.lr, w.beta1, w.beta2, w.eps,
                   w.wd, t, master, m, v, param, g_tmp=g_tmp)
        if w.pack:
            pack_param()
    dt = time.perf_counter() - t0
    if ex is not None:
        ex.shutdown()
    rate = sample * steps / dt
    return {"value": rate, "unit": "params/s", "cores": threads, "kind": "oracle",
            "sample": f"first {sample} elements of the {w.name} shard, {steps} steps, "
                      f"inputs pre-generated, "
                      + ("single thread" if threads == 1 else f"{threads} threads"),
            "seconds": round(dt, 3), "cpu": cpu_model(),
            "host_cpus": os.cpu_count()}


def offloaded_step_measured(w, threads, sample, gpu_step_ms, chunks=8, steps=3):
    """The offloaded step run end to end on the first `sample` elements of
    the shard: the GPU reduces bf16 replicas (the library's reduce, with the
    norm state); the fp32 gradient and the 128-byte norm state cross PCIe to
    pinned host memory; the host evaluates the gate and runs AdamW on all
    its cores over the host-resident master/m/v (the oracle's gate and
    AdamW, threaded over slices); the bf16 param crosses back.  Serial: one
    phase after the other.  Pipelined: the gradient crosses in `chunks`
    pieces on one stream while the host updates the pieces that have
    landed, and each updated piece's param crosses back on another stream.
    Each figure is the median of `steps` steps after one untimed step,
    scaled to the shard by S / sample."""
    import numpy as np
    import torch

    import oracle as O
    import synth
    import zero_sharded_mixed_step_amd as zs
    from concurrent.futures import ThreadPoolExecutor
    dev = torch.device("cuda:0")
    n = min(sample, w.S) // 32 * 32
    start = w.shard_start()
    reps = []
    for k in range(w.P):
        r = torch.empty(n, dtype=torch.int16, device=dev)
        synth.fill_device(w.grad_spec(1, k), start, r)
        reps.append(r)
    g_dev = torch.empty(n, dtype=torch.float32, device=dev)
    p_dev = torch.empty(n, dtype=torch.int16, device=dev)
    acc = zs.new_norm_acc(1, dev)
    g_host = torch.empty(n, dtype=torch.float32, pin_memory=True)
    p_host = torch.zeros(n, dtype=torch.int16, pin_memory=True)
    acc_host = torch.empty((1, zs.ACC_WORDS), dtype=torch.int64, pin_memory=True)
    g_np, p_np = g_host.numpy(), p_host.numpy().view(np.uint16)
    master = synth.fill(w.master_spec(), start, n, False, threads=8)
    m, v = np.zeros(n, np.float32), np.zeros(n, np.float32)
    inv = zs.zero_inv_scale(w.P, w.loss_scale)
    d2h_s, h2d_s = torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)
    pieces = O._cuts(n, chunks)
    torch.cuda.synchronize()

    def host_gate():
        X, nonfinite = zs.read_norm_acc(acc_host)[0]
        a = O.acc_zero()
        for k in range(O.ACC_WORDS):
            a.w[k] = (X >> (32 * k)) & 0xFFFFFFFF
        a.nonfinite = nonfinite
        return O.gate(a, w.max_norm, w.check_overflow)

    def host_adamw(ex, lo, hi, coef, sc):
        cuts = [(lo + a, lo + b) for a, b in O._cuts(hi - lo, threads)]
        list(ex.map(lambda c: O.adamw(g_np[c[0]:c[1]], coef, sc, master[c[0]:c[1]],
                                      m[c[0]:c[1]], v[c[0]:c[1]], p_np[c[0]:c[1]]), cuts))

    def gpu_reduce():
        zs.zero_norm_acc_clear(acc)
        zs.zero_shard_reduce(reps, inv, g_out=g_dev, acc=acc)

    def serial_step(ex, t):
        gpu_reduce()
        g_host.copy_(g_dev, non_blocking=True)
        acc_host.copy_(acc, non_blocking=True)
        torch.cuda.synchronize()
        skip, coef = host_gate()
        if not skip:
            host_adamw(ex, 0, n, coef, O.make_scalars(w.lr, w.beta1, w.beta2, w.eps, w.wd, t))
        p_dev.copy_(p_host, non_blocking=True)
        torch.cuda.synchronize()

    def pipelined_step(ex, t):
        gpu_reduce()
        acc_host.copy_(acc, non_blocking=True)
        reduced = torch.cuda.Event()
        reduced.record()
        d2h_s.wait_event(reduced)
        landed = []
        with torch.cuda.stream(d2h_s):
            for a, b in pieces:
                g_host[a:b].copy_(g_dev[a:b], non_blocking=True)
                e = torch.cuda.Event()
                e.record(d2h_s)
                landed.append(e)
        reduced.synchronize()
        skip, coef = host_gate()
        sc = O.make_scalars(w.lr, w.beta1, w.beta2, w.eps, w.wd, t)
        for (a, b), e in zip(pieces, landed):
            e.synchronize()
            if not skip:
                host_adamw(ex, a, b, coef, sc)
            with torch.cuda.stream(h2d_s):
                p_dev[a:b].copy_(p_host[a:b], non_blocking=True)
        h2d_s.synchronize()

    times = {"serial": [], "pipelined": []}
    t = 0
    with ThreadPoolExecutor(threads) as ex:
        for name, fn in (("serial", serial_step), ("pipelined", pipelined_step)):
            for i in range(steps + 1):
                t += 1
                t0 = time.perf_counter()
                fn(ex, t)
                if i:                                   # the first is untimed
                    times[name].append(1e3 * (time.perf_counter() - t0))
    scale = w.S / n
    serial = statistics.median(times["serial"]) * scale
    pipelined = statistics.median(times["pipelined"]) * scale
    return {"sample_elems": n, "chunks": chunks, "cpu_threads": threads,
            "sample_ms_per_step": {k: round(statistics.median(v_), 3)
                                   for k, v_ in times.items()},
            "offloaded_ms_per_step_serial": round(serial, 2),
            "offloaded_ms_per_step_pipelined": round(pipelined, 2),
            "slowdown_serial": round(serial / gpu_step_ms, 1),
            "slowdown_pipelined": round(pipelined / gpu_step_ms, 1)}


def offload_bill(w, threads, sample, gpu_step_ms, reduce_ms):
    """What the step costs with the optimizer moved to the host (the
    offloading the ZeRO pages describe): the GPU still reduces (its measured
    reduce time), the fp32 averaged gradient shard crosses PCIe to pinned
    host memory, the CPU runs the gate + AdamW on all its cores (the
    oracle's AdamW, threaded over slices: the same arithmetic, so the same
    bits), and the bf16 param shard crosses back.  Transfer rates and the
    CPU rate are measured on bounded samples and scaled to the shard."""
    import numpy as np
    import torch

    import oracle as O
    import synth
    dev = torch.device("cuda:0")
    nt = 1 << 28                                    # 1 GiB of fp32, 512 MiB of bf16
    g_dev = torch.empty(nt, dtype=torch.float32, device=dev)
    p_dev = torch.empty(nt, dtype=torch.int16, device=dev)
    g_host = torch.empty(nt, dtype=torch.float32, pin_memory=True)
    p_host = torch.zeros(nt, dtype=torch.int16, pin_memory=True)
    g_dev.fill_(1.0)

    def copy_rate(dst, src, nbytes, reps=3):
        dst.copy_(src, non_blocking=True)           # warm
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            dst.copy_(src, non_blocking=True)
        b.record()
        torch.cuda.synchronize()
        return nbytes * reps / (a.elapsed_time(b) * 1e-3) / 1e9

    d2h = copy_rate(g_host, g_dev, 4 * nt)
    h2d = copy_rate(p_dev, p_host, 2 * nt)
    del g_dev, p_dev, g_host, p_host

    sample = min(sample, w.S) // 32 * 32
    start = w.shard_start()
    master = synth.fill(w.master_spec(), start, sample, False, threads=8)
    m, v = np.zeros(sample, np.float32), np.zeros(sample, np.float32)
    param = np.zeros(sample, np.uint16)
    reps = [synth.fill(w.grad_spec(1, k), start, sample, w.grad_bf16, threads=8)
            for k in range(w.P)]
    g = O.reduce(reps, O.inv_scale(w.P, w.loss_scale))
    del reps
    cuts = O._cuts(sample, threads)
    from concurrent.futures import ThreadPoolExecutor
    reps_t = 3
    with ThreadPoolExecutor(threads) as ex:
        t0 = time.perf_counter()
        for t in range(1, reps_t + 1):
            s = O.make_scalars(w.lr, w.beta1, w.beta2, w.eps, w.wd, t)
            list(ex.map(lambda c: O.adamw(g[c[0]:c[1]], 0.5, s, master[c[0]:c[1]],
                                          m[c[0]:c[1]], v[c[0]:c[1]], param[c[0]:c[1]]),
                        cuts))
        dt = time.perf_counter() - t0
    cpu_rate = sample * reps_t / dt
    S = w.S
    d2h_ms = 4 * S / (d2h * 1e9) * 1e3
    cpu_ms = S / cpu_rate * 1e3
    h2d_ms = 2 * S / (h2d * 1e9) * 1e3
    serial = reduce_ms + d2h_ms + cpu_ms + h2d_ms
    pipelined = reduce_ms + max(d2h_ms, cpu_ms, h2d_ms)
    measured = offloaded_step_measured(w, threads, sample, gpu_step_ms)
    return {"kind": "measured: the offloaded step run end to end (GPU reduce, PCIe both ways, "
                    "host gate and AdamW on all cores) on the first elements of the shard, "
                    "serial and pipelined, scaled to the shard; beside it, the same bill "
                    "composed from separately measured PCIe and host AdamW rates",
            "gpu_ms_per_step": round(gpu_step_ms, 3),
            "measured_end_to_end": measured,
            "modelled": {
                "d2h_gbps": round(d2h, 1), "h2d_gbps": round(h2d, 1),
                "cpu_adamw_params_per_s": round(cpu_rate, 1), "cpu_threads": threads,
                "per_step_ms": {"gpu_reduce": round(reduce_ms, 3),
                                "d2h_g_f32": round(d2h_ms, 2), "cpu_adamw": round(cpu_ms, 2),
                                "h2d_param_bf16": round(h2d_ms, 2)},
                "offloaded_ms_per_step_serial": round(serial, 2),
                "offloaded_ms_per_step_pipelined": round(pipelined, 2),
                "slowdown_serial": round(serial / gpu_step_ms, 1),
                "slowdown_pipelined": round(pipelined / gpu_step_ms, 1)},
            "sample": f"end to end: the first {measured['sample_elems']} elements of the "
                      f"{w.name} shard, {measured['chunks']} pieces when pipelined; modelled: "
                      f"1 GiB D2H fp32 and 512 MiB H2D bf16, pinned, x3, and the oracle's "
                      f"AdamW on the first {sample} elements x{reps_t}; scaled to S={S}"}


def cpu_baseline_leg(w, args, threads, gpu_step_ms, reduce_ms):
    """The host side of the report, all of it the CPU oracle: single-threaded
    on a bounded sample (the baseline proper), the same on all cores, and the
    offload bill (the GPU reduce's measured time + PCIe + the oracle's AdamW
    on all cores) that moving the optimizer to the host would cost."""
    res = cpu_baseline(w, args.cpu_sample, args.cpu_steps)
    res["all_cores"] = cpu_baseline(w, args.cpu_sample, args.cpu_steps, threads=threads)
    if not args.no_offload and reduce_ms is not None:
        res["offload_bill"] = offload_bill(w, threads, args.cpu_sample, gpu_step_ms, reduce_ms)
    return res


def pattern_ceilings(w, st, reps, kinds, per_kernel):
    """The bare access patterns of the step's two passes (libzs_patterns.so:
    the same grids, access shapes and bytes, no arithmetic), on the step's
    own buffers in this process, so the placement is the same: the ceiling
    each kernel is measured against, next to the 8 TB/s peak.  Also the
    bound of reading and writing serially at the read-only and write-only
    rates.  Workloads whose step materialises fp32 g from 4 or 8 bf16
    replicas (the 7B and 30B shards, the GPT-2-sized one); None otherwise.
    The AdamW pattern writes master/m/v back unchanged; it overwrites only
    outputs (g, param, MXFP8) that every step rewrites."""
    import ctypes as C

    import torch

    from zero_sharded_mixed_step_amd import build as zb
    if (w.mx_grads or not w.grad_bf16 or w.P not in (4, 8) or st.path != "materialize"
            or not os.path.exists(zb.PATTERNS_LIB)):
        return None
    L = C.CDLL(zb.PATTERNS_LIB)
    vp, sz = C.c_void_p, C.c_size_t
    L.zs_pattern_read.argtypes = [vp, C.c_int, sz, vp, vp]
    L.zs_pattern_write.argtypes = [vp, sz, vp]
    L.zs_pattern_fill.argtypes = [vp, sz, vp]
    L.zs_pattern_reduce.argtypes = [vp, C.c_int, sz, vp, vp]
    L.zs_pattern_adamw.argtypes = [vp] * 7 + [sz, vp]
    n = w.S // 2048 * 2048                       # whole tiles
    ptrs = (vp * w.P)(*[r.data_ptr() for r in reps])
    sink = torch.zeros(1 << 24, dtype=torch.int32, device=st.master.device)
    stream = vp(torch.cuda.current_stream().cuda_stream)
    mx = st.fuse_pack
    elem = vp(st.mx_elem.data_ptr()) if mx else None
    scale = vp(st.mx_scale.data_ptr()) if mx else None
    g, ma, m, v, prm = (vp(t.data_ptr()) for t in (st.g, st.master, st.m, st.v, st.param))
    runs = {
        "read_only": (2 * w.P, lambda: L.zs_pattern_read(ptrs, w.P, n, vp(sink.data_ptr()),
                                                         stream)),
        "write_only": (4, lambda: L.zs_pattern_fill(g, n, stream)),
        "write_g_store_shape": (4, lambda: L.zs_pattern_write(g, n, stream)),
        "reduce_like": (2 * w.P + 4, lambda: L.zs_pattern_reduce(ptrs, w.P, n, g, stream)),
        "adamw_like": (30 + (MX_BYTES if mx else 0),
                       lambda: L.zs_pattern_adamw(g, ma, m, v, prm, elem, scale, n, stream)),
    }
    # PyTorch's own elementwise kernels on the same buffers, as reference
    # points for mixed reads and writes that this library did not write
    # (they overwrite only g, which every step rewrites)
    gv, mv, vv = st.g[:n], st.m[:n], st.v[:n]
    vendor_runs = {
        "torch_copy": (8, lambda: (gv.copy_(mv), 0)[1]),
        "torch_add": (12, lambda: (torch.add(mv, vv, out=gv), 0)[1]),
    }

    def time_runs(table):
        res_ = {}
        for name, (bpe, fn) in table.items():
            if fn() != 0:
                raise RuntimeError(f"pattern {name} did not launch")
            evs = []
            for _ in range(5):
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record()
                fn()
                b.record()
                evs.append((a, b))
            torch.cuda.synchronize()
            ms = statistics.median(a.elapsed_time(b) for a, b in evs)
            res_[name] = {"avg_ms": round(ms, 4), "bytes_per_elem": bpe,
                          "gbps": round(bpe * n / (ms * 1e-3) / 1e9, 1)}
        return res_
    out = time_runs(runs)
    vendor = time_runs(vendor_runs)
    rd, wr = out["read_only"]["gbps"], out["write_only"]["gbps"]

    def serial(r_bytes, w_bytes):
        return round((r_bytes + w_bytes) / (r_bytes / rd + w_bytes / wr), 1)
    res = {"note": "bare access patterns of the two passes on the step's own buffers, same "
                   "grids, no arithmetic; median of 5 launches by HIP events.  read_only: the "
                   "reduce's P nontemporal streams; write_only: the fastest write shape "
                   "measured (plain 16-byte stores, 4 KB per workgroup); the serialised bound "
                   "reads at read_only's and writes at write_only's rate.  vendor_kernels: "
                   "PyTorch's copy (g <- m) and add (g <- m + v) on the same buffers",
           "patterns": out,
           "vendor_kernels": vendor,
           "serialised_bound_gbps": {"reduce": serial(2 * w.P, 4),
                                     "adamw": serial(16, 14 + (MX_BYTES if mx else 0))},
           "kernel_frac_of_pattern": {}}
    for k, pat in (("reduce", "reduce_like"), ("adamw", "adamw_like")):
        if k in per_kernel:
            res["kernel_frac_of_pattern"][k] = round(per_kernel[k]["gbps"] / out[pat]["gbps"], 4)
    return res


def context_fields(w):
    """Closed forms the pages' figures rest on, beside the measured line:
    state bytes per weight against weights alone, the 30B example's state per
    data-parallel copy, and what MXFP8 saves on stored state and on the
    wire."""
    state = 2 + 2 + 4 + 4 + 4                     # bf16 param, bf16 grad, fp32 master, m, v
    return {"state_bytes_per_weight": state, "weights_only_bytes_per_weight": 2,
            "state_per_copy_gib_30b_model": round(30e9 * state / 2 ** 30, 2),
            "copies_at_8_way_data_parallel": 8,
            "mxfp8_bytes_per_elem": MX_BYTES,
            "mxfp8_stored_state_saving": round(2 * (2 - MX_BYTES) / state, 4),
            "mxfp8_wire_saving_vs_bf16": round(1 - MX_BYTES / 2, 4),
            "this_shard_state_gb": round(w.S * state / 1e9, 2)}


def workload_bytes(w):
    """Device bytes the workload allocates: the P replicas, fp32 master/m/v
    and g, bf16 param and the MXFP8 outputs."""
    g_b = MX_BYTES if w.mx_grads else w.g_bytes
    per = 4 * 4 + 2 + (MX_BYTES if w.pack else 0)
    return int(w.S * (w.P * g_b + per))


def recycle_device_memory(dev, nbytes):
    """Untimed set-up: write and release a scratch allocation of
    max(150 GiB, 1.1 x the workload) before the workload allocates.  Where
    the workload's buffers land in HBM changed the write-heavy AdamW pass by
    up to 20 % on MI355X (the reduce by about 2 %).  Allocated first in a
    fresh process, the 30B and 1.3B workloads ran at their slowest; after
    such a scratch they ran at their fastest in every run measured (the 7B
    working set varied either way).  Recycling all free memory instead was
    slow again.  Returns the scratch size in bytes."""
    import torch
    free, _ = torch.cuda.mem_get_info(dev)
    size = min(max(150 << 30, int(nbytes * 1.1)), free - (8 << 30))
    if size <= 0:
        return 0
    x = torch.empty(size, dtype=torch.uint8, device=dev)
    x.fill_(0)
    torch.cuda.synchronize(dev)
    del x
    torch.cuda.empty_cache()
    return size


_HELD = []


def hold_spacer(dev, nbytes):
    """Untimed set-up: allocate, write and hold (until the process ends) a
    spacer of nbytes in 5 GB pieces before the workload allocates.  Returns
    the bytes held."""
    import torch
    while sum(x.numel() for x in _HELD) < nbytes:
        x = torch.empty(min(5 * 10**9, nbytes - sum(y.numel() for y in _HELD)),
                        dtype=torch.uint8, device=dev)
        x.fill_(1)
        _HELD.append(x)
    torch.cuda.synchronize(dev)
    return sum(x.numel() for x in _HELD)


def placement_probe(w, spacer_gb):
    """Time the step's reduce and AdamW launches with the workload's buffers
    allocated first in the process, then again after a held, written spacer
    allocation: the same kernels and inputs in two placements in HBM."""
    import torch

    import synth
    import zero_sharded_mixed_step_amd as zs
    dev = torch.device("cuda:0")
    spacers = []
    for phase, spacer in (("first", 0.0), ("after spacer", spacer_gb)):
        while sum(x.numel() for x in spacers) < spacer * 1e9:
            x = torch.empty(min(5 * 10**9, int(spacer * 1e9) - sum(y.numel() for y in spacers)),
                            dtype=torch.uint8, device=dev)
            x.fill_(1)
            spacers.append(x)
        st = zs.ShardStep(w.S, w.P, torch.bfloat16 if w.grad_bf16 else torch.float32, lr=w.lr,
                          beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.wd,
                          max_norm=w.max_norm, check_overflow=w.check_overflow,
                          loss_scale=w.loss_scale, bucket=w.bucket, pack=w.pack,
                          device_counter=True, device=dev)
        synth.fill_device(w.master_spec(), w.shard_start(), st.master)
        synth.fill_device(w.master_spec(), w.shard_start(), st.param)
        reps = []
        for k in range(w.P):
            r = torch.empty(w.S, dtype=torch.int16 if w.grad_bf16 else torch.float32, device=dev)
            synth.fill_device(w.grad_spec(1, k), w.shard_start(), r)
            reps.append(r)
        times = []
        for _ in range(3):
            a, b, c = (torch.cuda.Event(enable_timing=True) for _ in range(3))
            a.record()
            st.reduce(reps)
            b.record()
            st.update(reps)
            c.record()
            torch.cuda.synchronize()
            times.append({"reduce_ms": round(a.elapsed_time(b), 3),
                          "adamw_ms": round(b.elapsed_time(c), 3)})
        print(json.dumps({"workload": w.name, "placement": phase, "spacer_gb": spacer,
                          "steps": times}), flush=True)
        del st, reps
        torch.cuda.synchronize()
        torch.cuda.empty_cache()


_T0 = time.perf_counter()


def progress(msg):
    """One line per finished phase on stderr (stdout carries only the JSON line)."""
    print(f"bench [{time.perf_counter() - _T0:7.1f} s] {msg}", file=sys.stderr, flush=True)


def measure(w, args, dev, legs=True, recycle=True):
    """One workload's timed steps and the figures around them; returns the
    JSON object (without the CPU baseline) and what the CPU leg needs.
    legs=False leaves out the unfused chain, the standalone pack, and the
    cold and graph steps."""
    import torch

    import synth
    import zero_sharded_mixed_step_amd as zs

    prep = "none" if args.no_recycle or not recycle else args.memory_prep
    if prep == "recycle":
        recycled = recycle_device_memory(dev, workload_bytes(w))
        prep_note = f"{recycled} B scratch written and released before allocating"
    elif prep == "spacer":
        recycled = hold_spacer(dev, 60 * 10**9)
        prep_note = f"{recycled} B spacer written and held for the whole run"
    else:
        recycled, prep_note = None, "none"
    grad_dtype = "mxfp8" if w.mx_grads else (torch.bfloat16 if w.grad_bf16 else torch.float32)
    st = zs.ShardStep(w.S, w.P, grad_dtype, lr=w.lr,
                      beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.wd,
                      max_norm=w.max_norm, check_overflow=w.check_overflow,
                      loss_scale=w.loss_scale, bucket=w.bucket, pack=w.pack,
                      device_counter=True, device=dev)
    start = w.shard_start()
    synth.fill_device(w.master_spec(), start, st.master)
    synth.fill_device(w.master_spec(), start, st.param)
    gdt = torch.int16 if w.grad_bf16 else torch.float32
    reps = []
    if w.mx_grads:
        # MXFP8-stored replicas: the bf16 replicas, packed on the device
        tmp = torch.empty(w.S, dtype=gdt, device=dev)
        for k in range(w.P):
            synth.fill_device(w.grad_spec(1, k), start, tmp)
            codes = torch.empty(w.S, dtype=torch.uint8, device=dev)
            scales = torch.empty(w.S // 32, dtype=torch.uint8, device=dev)
            zs.zero_mxfp8_pack(tmp, codes, scales)
            reps.append((codes, scales))
        torch.cuda.synchronize()
        del tmp
    else:
        for k in range(w.P):
            r = torch.empty(w.S, dtype=gdt, device=dev)
            synth.fill_device(w.grad_spec(1, k), start, r)
            reps.append(r)
    torch.cuda.synchronize()
    progress(f"{w.name}: inputs resident ({w.P} replicas of {w.S} elements)")

    kinds = per_elem_bytes(w, st)
    events = {k: [] for k in kinds}

    def timed(kind, fn):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        events[kind].append((a, b))

    step_events = []

    def one_step(record):
        if not record:
            st.step(reps)
            return
        sa = torch.cuda.Event(enable_timing=True)
        sb = torch.cuda.Event(enable_timing=True)
        sa.record()
        _launch_step()
        sb.record()
        step_events.append((sa, sb))

    def _launch_step():
        if st.path != "fused":
            timed("reduce", lambda: st.reduce(reps))
        timed("adamw", lambda: st.update(reps))
        if w.pack and not st.fuse_pack:
            timed("mxfp8_pack", st.pack_param)

    for _ in range(args.warmup):
        one_step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        one_step(True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    applied = st.applied_steps()
    progress(f"{args.warmup} warmup + {args.steps} timed steps done: "
             f"{1e3 * elapsed / args.steps:.3f} ms/step")

    # The standalone MXFP8 pack entry point (outside the timed step: the step
    # packs inside AdamW), timed on its own for its roofline.
    standalone = {}
    if w.pack and legs:
        evs = []
        for _ in range(3):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            st.pack_param()
            b.record()
            evs.append((a, b))
        torch.cuda.synchronize()
        ms = sum(a.elapsed_time(b) for a, b in evs) / len(evs)
        standalone["mxfp8_pack"] = {"avg_ms": round(ms, 4), "bytes_per_elem": 2 + MX_BYTES,
                                    "gbps": round((2 + MX_BYTES) * w.S / (ms * 1e-3) / 1e9, 1)}

    unfused = None
    if legs and not args.no_unfused and not w.mx_grads:
        # The same step as a chain of single-operation kernels, same process
        # and buffers: what fusion saves (bit-identical results).  The chain
        # takes the host step counter.
        st.set_counter(device=False)
        for _ in range(max(1, args.warmup)):
            st.step_unfused(reps)
        torch.cuda.synchronize()
        u0 = time.perf_counter()
        for _ in range(args.steps):
            st.step_unfused(reps)
        torch.cuda.synchronize()
        u_ms = 1e3 * (time.perf_counter() - u0) / args.steps
        ub = unfused_bytes(w)
        unfused = {"ms_per_step": round(u_ms, 4), "bytes_per_param": ub,
                   "hbm_gbps": round(ub * w.S / (u_ms * 1e-3) / 1e9, 1),
                   "launches_per_step": 11 + (1 if w.pack else 0),
                   "fused_speedup": round(u_ms / (1e3 * elapsed / args.steps), 3)}
        st.set_counter(device=True)
        progress(f"unfused chain timed: {u_ms:.3f} ms/step")

    # Cold steps for workloads whose step fits in the caches (L2 4 MB per XCD,
    # 256 MB MALL): a 1 GiB scratch write before each step evicts the state,
    # so the step reads it from HBM.  Timed by two events around the step's
    # launches alone (no per-kernel events inside, whose markers would add
    # to a step of a few microseconds); the scratch write keeps the GPU busy
    # while the host queues them.
    cold = None
    if legs and sum(kinds.values()) * w.S < (2 << 30):
        scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        cold_ev = []
        for _ in range(args.steps):
            scratch.fill_(1)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            st.step(reps)
            b.record()
            cold_ev.append((a, b))
        torch.cuda.synchronize()
        del scratch
        cold_ms = statistics.median(a.elapsed_time(b) for a, b in cold_ev)
        cold = {"step_ms_median": round(cold_ms, 4),
                "params_per_s": round(w.S / (cold_ms * 1e-3), 1),
                "hbm_gbps": round(sum(kinds.values()) * w.S / (cold_ms * 1e-3) / 1e9, 1),
                "note": "1 GiB scratch write before each step (evicts L2 and MALL)"}
        st.applied_steps()

    # The same small steps recorded once as a graph and replayed back to back:
    # the steady-state rate of a loop that replays it (whichever of the
    # GPU's work and the host's graph launches is slower sets it).
    graph_steps = None
    if legs and sum(kinds.values()) * w.S < (2 << 30):
        graph = st.capture(reps)
        graph.replay()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        g0 = time.perf_counter()
        a.record()
        for _ in range(args.steps):
            graph.replay()
        b.record()
        torch.cuda.synchronize()
        g_wall = 1e3 * (time.perf_counter() - g0) / args.steps
        g_ms = a.elapsed_time(b) / args.steps
        graph_steps = {"ms_per_step": round(g_ms, 4), "wall_ms_per_step": round(g_wall, 4),
                       "params_per_s": round(w.S / (g_wall * 1e-3), 1),
                       "note": f"one recorded step (all its launches) replayed {args.steps} "
                               "times back to back; ms_per_step by events around them all"}
        del graph

    ms_per_step = 1e3 * elapsed / args.steps
    step_bytes = sum(kinds.values()) * w.S
    params_per_s = w.S / (elapsed / args.steps)
    gbps = step_bytes / (elapsed / args.steps) / 1e9
    kernel_ms = {k: sum(a.elapsed_time(b) for a, b in ev) / len(ev) for k, ev in events.items()}
    step_ms = sorted(a.elapsed_time(b) for a, b in step_events)
    p90 = step_ms[min(len(step_ms) - 1, int(round(0.9 * (len(step_ms) - 1))))]
    per_kernel = {k: {"avg_ms": round(kernel_ms[k], 4),
                      "bytes_per_elem": kinds[k],
                      "gbps": round(kinds[k] * w.S / (kernel_ms[k] * 1e-3) / 1e9, 1)}
                  for k in kinds}
    dom = max(kernel_ms, key=kernel_ms.get)
    dom_gbps = per_kernel[dom]["gbps"]
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh).get(w.name)
        if rec and rec["source_digest"] == source_digest() and dom in rec["kinds"]:
            per_launch = kinds[dom] * w.S if dom != "reduce" or not w.bucket else kinds[dom] * w.bucket
            traffic = (rec["kinds"][dom]["hbm_bytes"],
                       round(rec["kinds"][dom]["hbm_bytes"] / per_launch, 4))
    patterns = pattern_ceilings(w, st, reps, kinds, per_kernel)
    roof = {"bound": "hbm", "kernel": dom, "achieved": dom_gbps,
            "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(dom_gbps / HBM_PEAK_GBPS, 4),
            "traffic": traffic[0] if traffic else None,
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                            "scaled by a plain-copy calibration)",
            "traffic_vs_algorithmic": traffic[1] if traffic else None}
    if patterns and dom in patterns["kernel_frac_of_pattern"]:
        pat = {"reduce": "reduce_like", "adamw": "adamw_like"}[dom]
        roof["pattern_ceiling_gbps"] = patterns["patterns"][pat]["gbps"]
        roof["frac_of_pattern"] = patterns["kernel_frac_of_pattern"][dom]
    out = {
        "metric": "optimizer-step params/sec per shard + achieved HBM GB/s (% of peak)",
        "value": round(params_per_s, 1),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "step_ms_median": round(statistics.median(step_ms), 4),
        "step_ms_p90": round(p90, 4),
        "cold_steps": cold,
        "graph_steps": graph_steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.title}", "shard_elems": w.S, "P": w.P,
                   "grad_dtype": "mxfp8" if w.mx_grads else ("bf16" if w.grad_bf16 else "f32"),
                   "bucket": w.bucket,
                   "max_norm": w.max_norm, "check_overflow": w.check_overflow,
                   "mxfp8_pack": ("fused into AdamW" if st.fuse_pack else "separate pass")
                   if w.pack else False, "path": st.path},
        "memory_prep": prep_note,
        "hbm_gbps": round(gbps, 1),
        "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "bytes_per_param": sum(kinds.values()),
        "applied_steps": applied,
        "kernels": per_kernel,
        **({"kernels_note": "a step this short is bound by the host's launches: the events "
                            "around each pass also hold the GPU's wait for that pass's launch; "
                            "the rocprofv3 kernel trace gives the kernels' own durations"}
           if ms_per_step < 1.0 else {}),
        "standalone_kernels": standalone,
        "unfused_chain": unfused,
        "roofline": roof,
        "pattern_ceilings": patterns,
        "cpu_baseline": None,
        "context": context_fields(w),
        "command": " ".join(["python", "bench.py", *sys.argv[1:]]),
        "kernel_sources_digest": source_digest(),
    }
    return out, {"ms_per_step": ms_per_step, "reduce_ms": kernel_ms.get("reduce"),
                 "recycled": recycled}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: it runs one rank's shard step on a "
              f"single MI355X, and the exchanges between ranks are not implemented "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    if args.summarize_pmc:
        from synth import configs
        summarize_pmc(configs.ALL[args.config], args.summarize_pmc, " ".join(sys.argv))
        return
    if args.trace_report:
        from synth import configs
        trace_report(configs.ALL[args.config], *args.trace_report)
        return
    if args.placement_report:
        placement_report(args.placement_report)
        return
    if args.traffic_report:
        traffic_report(args.traffic_report)
        return

    import torch

    if args.copy_calibration:
        copy_calibration()
        return

    if args.placement_probe is not None:
        from synth import configs
        placement_probe(configs.ALL[args.config], args.placement_probe)
        return

    from synth import configs

    w = configs.ALL[args.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    out, ctx = measure(w, args, dev)
    if args.config == "30b-shard-p8" and not args.no_secondary:
        # The other shard the step is specified on, in the same process: the
        # 7B rank share with its 35 buckets, its own timed steps.
        import gc
        gc.collect()
        torch.cuda.empty_cache()
        sw = configs.SHARD_7B
        sec, _ = measure(sw, args, dev, legs=False, recycle=False)
        out["secondary"] = {k: sec[k] for k in (
            "config", "value", "unit", "ms_per_step", "step_ms_median", "step_ms_p90",
            "hbm_gbps", "hbm_frac", "bytes_per_param", "kernels", "roofline",
            "pattern_ceilings")}
        out["secondary"]["steps"] = args.steps
        progress(f"secondary {sw.name}: {sec['ms_per_step']:.3f} ms/step")
    threads = max(1, min(args.cpu_threads, os.cpu_count() or 1))
    if not args.no_cpu_baseline:
        progress("CPU oracle baseline (bounded sample) starts")
        out["cpu_baseline"] = cpu_baseline_leg(w, args, threads, ctx["ms_per_step"],
                                               ctx["reduce_ms"])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

"""Host-side logic, no GPU: the fused-minimum byte accounting of every
workload and pass structure, the unfused chain's bytes, the scaling of
rocprofv3 FETCH_SIZE/WRITE_SIZE counters into HBM bytes, the refusal of a
multi-GPU run (bench.py), and ShardStep's choice of pass structure."""
import csv
import json
import os
import subprocess
import sys
from types import SimpleNamespace

import pytest

import bench
from synth import configs

MX = 1 + 1 / 32


@pytest.mark.parametrize("name,path,fuse,want", [
    # 8 bf16 replicas, materialised g: reduce 8*2 + 4, AdamW 4 + 24 + 2 (+ MXFP8)
    ("30b-shard-p8", "materialize", True, {"reduce": 20, "adamw": 30 + MX}),
    ("30b-shard-p8", "materialize", False, {"reduce": 20, "adamw": 30, "mxfp8_pack": 2 + MX}),
    ("7b-shard-p8", "materialize", False, {"reduce": 20, "adamw": 30}),
    ("gpt2-small-p8", "materialize", False, {"reduce": 20, "adamw": 30}),
    # one bf16 replica, recomputed: norm pass 2, AdamW 2 + 26
    ("1.3b-unsharded", "recompute", False, {"reduce": 2, "adamw": 28}),
    # ungated: one pass, 4 fp32 replicas + 26
    ("flat-1m-p4", "fused", False, {"adamw": 42}),
    # MXFP8-stored replicas: 8 * (1 + 1/32) + 4
    ("30b-shard-p8-mxgrads", "materialize", True, {"reduce": 8 * MX + 4, "adamw": 30 + MX}),
])
def test_fused_minimum_bytes(name, path, fuse, want):
    w = configs.ALL[name]
    got = bench.per_elem_bytes(w, SimpleNamespace(path=path, fuse_pack=fuse))
    assert got.keys() == want.keys()
    for k in want:
        assert got[k] == pytest.approx(want[k], abs=0), (k, got[k], want[k])


def test_step_minimum_matches_the_pass_structure():
    # gated at P = 8 bf16: min(P*2 + 34, 2*P*2 + 26) = 50; the 30B case adds
    # the fused MXFP8 output
    w = configs.SHARD_30B
    kinds = bench.per_elem_bytes(w, SimpleNamespace(path="materialize", fuse_pack=True))
    assert sum(kinds.values()) == 50 + MX
    P, g_b = w.P, w.g_bytes
    assert min(P * g_b + 34, 2 * P * g_b + 26) == 50


def test_unfused_chain_bytes():
    # sum (P*2 + 4), scale (8), norm (4), clip (8), m (12), v (12),
    # direction (12), weight (12), cast (6), pack (2 + 1.03125)
    assert bench.unfused_bytes(configs.SHARD_7B) == 94
    assert bench.unfused_bytes(configs.SHARD_30B) == 94 + 2 + MX


def test_workload_bytes():
    w = configs.SHARD_30B
    assert bench.workload_bytes(w) == int(w.S * (8 * 2 + 18 + MX))


def _write_counters(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as fh:
        wr = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for name, value in rows:
            wr.writerow({"Kernel_Name": name, "Counter_Name": "X", "Counter_Value": value})


def test_counter_scaling(tmp_path, monkeypatch):
    """HBM bytes = 1024 * (FETCH_SIZE * f + WRITE_SIZE * w), where the plain
    1 GiB copy fixes f and w, averaged over dispatches per launch kind."""
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    copy = "__amd_rocclr_copyBuffer"
    adamw = "void zs::adamw_kernel<-1, 1, true, true, 2, false>(zs::AdamParams)"
    red = "void zs::shard_reduce_kernel<1, 8, true, true, false>(zs::ReduceParams)"
    d = {k: str(tmp_path / k) for k in ("f", "w", "cf", "cw")}
    _write_counters(d["cf"], [(copy, 524288.0)])          # a copy reads half its bytes
    _write_counters(d["cw"], [(copy, 1048576.0)])
    _write_counters(d["f"], [(adamw, 1000.0), (adamw, 1002.0), (red, 10.0)])
    _write_counters(d["w"], [(adamw, 700.0), (adamw, 700.0), (red, 5.0)])
    w = configs.SHARD_30B
    bench.summarize_pmc(w, [d["f"], d["w"], d["cf"], d["cw"]], "test")
    rec = json.load(open(tmp_path / "traffic.json"))[w.name]
    assert rec["fetch_factor"] == 2.0 and rec["write_factor"] == 1.0
    assert rec["source_digest"] == bench.source_digest()
    assert rec["kinds"]["adamw"] == {"dispatches": 2, "fetch_kib": 1001.0, "write_kib": 700.0,
                                     "hbm_bytes": 1024 * (1001 * 2 + 700)}
    assert rec["kinds"]["reduce"]["hbm_bytes"] == 1024 * (10 * 2 + 5)
    assert "mxfp8_pack" not in rec["kinds"]


def test_source_digest_is_stable():
    a, b = bench.source_digest(), bench.source_digest()
    assert a == b and len(a) == 16 and int(a, 16) >= 0


def test_multi_gpu_run_is_refused():
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_pass_structure_choice():
    """Gated steps materialise g when that moves fewer bytes than re-reducing
    the replicas (P*g_b + 34 < 2*P*g_b + 26, i.e. P*g_b > 8)."""
    from zero_sharded_mixed_step_amd import choose_path
    assert choose_path(4, 4, gated=False) == "fused"
    assert choose_path(8, 2, gated=True) == "materialize"       # 50 < 58
    assert choose_path(1, 2, gated=True) == "recompute"         # 30 < 36
    assert choose_path(4, 2, gated=True) == "recompute"         # 8: tie -> recompute
    assert choose_path(3, 4, gated=True) == "materialize"       # 46 < 50
    assert choose_path(1, 2, gated=True, mx_grads=True) == "materialize"
    for P, g_b in ((1, 2), (2, 2), (4, 2), (8, 2), (1, 4), (3, 4), (8, 4)):
        mat, rec = P * g_b + 34, 2 * P * g_b + 26
        got = choose_path(P, g_b, gated=True)
        assert (got == "materialize") == (mat < rec), (P, g_b, got)
    with pytest.raises(ValueError):
        choose_path(8, 2, gated=True, path="fused")
    with pytest.raises(ValueError):
        choose_path(8, 2, gated=True, mx_grads=True, path="recompute")


@pytest.mark.parametrize("name,kernels", [
    ("30b-shard-p8", ["void zs::shard_reduce_kernel<1, 8, true, true, false, true>"
                      "(zs::ReduceParams)",
                      "zs::slot_fold_kernel(zero_norm_acc*, zero_norm_acc*)",
                      "void zs::adamw_kernel<-1, 1, true, true, 2, false>(zs::AdamParams)"]),
    ("7b-shard-p8", ["void zs::shard_reduce_kernel<1, 8, true, true, true, false>"
                     "(zs::ReduceParams)",
                     "void zs::adamw_kernel<-1, 1, true, false, 2, false>(zs::AdamParams)"]),
    ("gpt2-small-p8", ["void zs::shard_reduce_kernel<1, 8, true, true, true, false>"
                       "(zs::ReduceParams)",
                       "void zs::adamw_kernel<-1, 1, true, false, 2, true>(zs::AdamParams)"]),
    ("1.3b-unsharded", ["void zs::shard_reduce_kernel<1, 1, false, true, false, false>"
                        "(zs::ReduceParams)",
                        "void zs::adamw_kernel<1, 1, true, false, 2, false>(zs::AdamParams)"]),
    ("flat-1m-p4", ["void zs::adamw_kernel<0, 4, true, false, 1, true>(zs::AdamParams)"]),
])
def test_step_kernel_names(name, kernels):
    """The kernels a step launches, named as rocprofv3 prints them, follow the
    pass structure; the 35 buckets of the 7B shard take one reduce each, the
    whole 30B shard the one-shot reduce and its fold."""
    got = bench.step_kernels(configs.ALL[name])
    assert [k for k, _, _ in got[:-1]] == kernels
    assert got[-1][0].startswith("zs::step_advance_kernel(")
    if name == "7b-shard-p8":
        assert got[0][2] == 35


def test_traffic_report_ratios(capsys):
    """The committed counter table: every launch kind within 3% of its
    algorithmic bytes (re-reads would show as a larger ratio)."""
    bench.traffic_report(["30b-shard-p8", "7b-shard-p8"])
    rows = [ln.split() for ln in capsys.readouterr().out.splitlines()
            if ln and not ln.startswith("#")]
    assert len(rows) == 5
    for r in rows:
        assert 0.99 < float(r[-1]) < 1.03, r


def test_trace_report_reads_a_kernel_stats_file(tmp_path, capsys):
    """The kernel-trace summary: rocprofv3's stats rows, the step kernels with
    their averages, and the bench line (with its command) of the same run."""
    w = configs.SHARD_30B
    names = [k for k, _, _ in bench.step_kernels(w)]
    d = tmp_path / "prof"
    d.mkdir()
    with open(d / "run_kernel_stats.csv", "w", newline="") as fh:
        wr = csv.writer(fh)
        wr.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs",
                     "MaxNs", "StdDev"])
        for i, n in enumerate(names):
            wr.writerow([n, 12, 12 * (i + 1) * 1000, (i + 1) * 1000.0, 10.0, 1, 2, 0.5])
    log = tmp_path / "run.log"
    log.write_text("noise\n" + json.dumps({"metric": "m", "command": "python bench.py --steps 3"})
                   + "\n")
    bench.trace_report(w, str(d), str(log))
    out = capsys.readouterr().out
    assert "-- python3 $R/bench.py --steps 3" in out
    assert "NOT IN THE TABLE" not in out
    for i, n in enumerate(names):
        assert f"{n.split('(')[0]}:" in out and f"{(i + 1) * 1000} ns" in out
    assert out.rstrip().endswith('"command": "python bench.py --steps 3"}')


def test_placement_report_splits_the_two_placements(tmp_path, capsys):
    """Per-launch counters: the first half of the reduce/AdamW launches is the
    first placement, the second half the one after the spacer; other kernels
    (the fold, fills) are left out."""
    d = tmp_path / "pmc"
    d.mkdir()
    rows = []
    kinds = ["void zs::shard_reduce_kernel<1, 8, true, true, false, true>(zs::ReduceParams)",
             "zs::slot_fold_kernel(zero_norm_acc*, zero_norm_acc*)",
             "void zs::adamw_kernel<-1, 1, true, true, 2, false>(zs::AdamParams)"] * 2
    for i, k in enumerate(kinds):
        rows.append({"Dispatch_Id": i, "Kernel_Name": k, "Counter_Name": "X_sum",
                     "Counter_Value": 100 + i, "Start_Timestamp": 0,
                     "End_Timestamp": (i + 1) * 1_000_000})
    with open(d / "run_counter_collection.csv", "w", newline="") as fh:
        wr = csv.DictWriter(fh, fieldnames=list(rows[0]))
        wr.writeheader()
        wr.writerows(rows)
    log = tmp_path / "p.log"
    log.write_text('{"placement": "first"}\n{"placement": "after spacer"}\n')
    bench.placement_report([str(d), str(log)])
    lines = [ln.split() for ln in capsys.readouterr().out.splitlines() if ln.startswith("  ")]
    assert [(r[0], r[1], r[-1]) for r in lines] == [
        ("first", "reduce", "100"), ("first", "adamw", "102"),
        ("spacer", "reduce", "103"), ("spacer", "adamw", "105")]

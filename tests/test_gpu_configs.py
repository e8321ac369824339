"""Parity at the workloads' real sizes over their whole schedules, in the
launch configuration the benchmark times (ShardStep with the workload's
bucket, gate and pack settings, the device step counter).

Every element of the final state is compared with the oracle, bit for bit:
master, m, v and the bf16 param (and the MXFP8 pack where the workload packs),
with the count of non-identical elements and the max relative error reported.
The global norm state of every call (the accumulator the device gate reads)
is compared bit for bit too, call by call.  The oracle holds the whole state
in host memory and regenerates each call's gradient replicas chunk by chunk
from the counter-based generator (OracleRun).

  - 1M-element P=4 fp32 case: every rank, one step.
  - GPT-2-small-sized P=8 case: all 8 ranks over 10 steps against the oracle
    on the whole vector (each rank's norm state added into the global one,
    the norm all-reduce), and the 8 shard steps against one unsharded
    step of the full vector on the GPU.
  - 1.3B unsharded (10 calls, loss scale, an injected inf at call 5 that is
    skipped), 7B shard (10 steps, 35 buckets of 25M, clip), 30B shard (5
    steps, clip + overflow check, MXFP8 pack fused, then the standalone
    pack): whole schedules, every element.
  - 30B shard with MXFP8-stored gradient replicas, all five calls: the host
    packs and decodes all 8 replicas of every chunk at every call.
"""
import numpy as np
import pytest

import oracle as O
import synth
from gpu_util import OracleRun, compare_full, from_dev, gpu_or_skip, log, same_bits
from synth import configs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def zs():
    gpu_or_skip()
    import zero_sharded_mixed_step_amd as zs
    zs.lib()
    return zs


def _step_for(zs, w, **over):
    import torch
    kw = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.wd,
              max_norm=w.max_norm, check_overflow=w.check_overflow, loss_scale=w.loss_scale,
              bucket=w.bucket, pack=w.pack)
    kw.update(over)
    n = kw.pop("n", w.S)
    gdt = "mxfp8" if w.mx_grads else (torch.bfloat16 if w.grad_bf16 else torch.float32)
    return zs.ShardStep(n, w.P, gdt, **kw)


def _device_replicas(w, call, lo, n, out=None):
    import torch
    gdt = torch.int16 if w.grad_bf16 else torch.float32
    if w.mx_grads:
        # MXFP8-stored replicas: each bf16 replica packed on the device
        import zero_sharded_mixed_step_amd as zs
        if out is None:
            out = [(torch.empty(n, dtype=torch.uint8, device="cuda"),
                    torch.empty(n // 32, dtype=torch.uint8, device="cuda")) for _ in range(w.P)]
        tmp = torch.empty(n, dtype=gdt, device="cuda")
        for k, (codes, scales) in enumerate(out):
            synth.fill_device(w.grad_spec(call, k), lo, tmp)
            zs.zero_mxfp8_pack(tmp, codes, scales)
        torch.cuda.synchronize()
        return out
    if out is None:
        out = [torch.empty(n, dtype=gdt, device="cuda") for _ in range(w.P)]
    for k, r in enumerate(out):
        synth.fill_device(w.grad_spec(call, k), lo, r)
    if w.inject and w.inject[0] == call and lo <= w.inject[1] < lo + n:
        out[0][w.inject[1] - lo] = 0x7F80 if w.grad_bf16 else float("inf")
    return out


def _init_state(st, w, lo):
    synth.fill_device(w.master_spec(), lo, st.master)
    synth.fill_device(w.master_spec(), lo, st.param)


def _acc_sum(zs, accs):
    """(X, nonfinite) of the sum of device accumulators."""
    rows = zs.read_norm_acc(accs)
    return sum(r[0] for r in rows), sum(r[1] for r in rows)


def _assert_state(st, run, where):
    """Every element of master/m/v/param of the device step `st` against the
    oracle run."""
    host = {"master": run.master, "m": run.m, "v": run.v, "param": run.param}
    for name in ("master", "m", "v", "param"):
        nbad, rel, first = compare_full(f"{where} {name}", getattr(st, name), host[name],
                                        bf16=name == "param")
        assert nbad == 0, f"{where} {name}: {nbad} elements differ (first at {first}), " \
                          f"max rel err {rel:.3e}"


# -------------------------------------------------------------- small ones --

def test_flat_1m_p4_fp32_all_ranks(zs):
    import torch
    w = configs.FLAT_1M
    for rank in range(w.P):
        lo = rank * w.S
        st = _step_for(zs, w)
        assert st.path == "fused"
        _init_state(st, w, lo)
        reps = _device_replicas(w, 1, lo, w.S)
        st.step(reps)
        torch.cuda.synchronize()
        master = synth.fill(w.master_spec(), lo, w.S, False)
        m, v = np.zeros(w.S, np.float32), np.zeros(w.S, np.float32)
        param = O.f32_to_bf16(master)
        hreps = [synth.fill(w.grad_spec(1, k), lo, w.S, False) for k in range(w.P)]
        skipped, _ = O.step(hreps, O.inv_scale(w.P, 1.0), 0.0, False, w.lr, w.beta1, w.beta2,
                            w.eps, w.wd, 1, master, m, v, param)
        assert not skipped
        for name, want in (("master", master), ("m", m), ("v", v), ("param", param)):
            got = from_dev(getattr(st, name), name == "param")
            assert same_bits(got, want), f"rank {rank} {name}"


@pytest.mark.timeout(900)
def test_gpt2_small_p8_ten_steps_all_ranks(zs):
    """All 8 ranks over the 10 steps against the oracle on the whole vector,
    and the 8 shard steps against one unsharded GPU step."""
    import torch
    w = configs.GPT2_SMALL
    ranks = [_step_for(zs, w, device_counter=True) for _ in range(w.P)]
    for r, st in enumerate(ranks):
        _init_state(st, w, r * w.S)
    full = _step_for(zs, w, n=w.N, path="materialize", device_counter=True)
    _init_state(full, w, 0)
    accs = zs.new_norm_acc(w.P)
    reps = None
    per_call = []
    for call in range(1, w.steps + 1):
        reps = _device_replicas(w, call, 0, w.N, out=reps)
        for r, st in enumerate(ranks):
            st.reduce([x[r * w.S:(r + 1) * w.S] for x in reps])
            accs[r].copy_(st.acc[0])
        for r, st in enumerate(ranks):
            st.update([x[r * w.S:(r + 1) * w.S] for x in reps], accs=accs)
        full.step(reps)
        per_call.append(accs.clone())
    torch.cuda.synchronize()
    for name in ("master", "m", "v", "param"):
        cat = torch.cat([getattr(st, name) for st in ranks])
        assert torch.equal(cat, getattr(full, name)), f"sharded != unsharded: {name}"
    del reps
    log(f"{w.name}: GPU done, oracle over all {w.N} elements")
    run = OracleRun(w, 0, w.N)
    try:
        for call in range(1, w.steps + 1):
            skip, _, acc = run.call(call)
            assert not skip
            assert _acc_sum(zs, per_call[call - 1]) == (acc.X, int(acc.nonfinite)), call
        assert [st.applied_steps() for st in ranks] == [w.steps] * w.P
        for r, st in enumerate(ranks):
            sl = slice(r * w.S, (r + 1) * w.S)
            for name, host in (("master", run.master), ("m", run.m), ("v", run.v),
                               ("param", run.param)):
                nbad, rel, first = compare_full(f"rank {r} {name}", getattr(st, name),
                                                np.ascontiguousarray(host[sl]),
                                                bf16=name == "param")
                assert nbad == 0, f"rank {r} {name}: {nbad} differ (first {first}), rel {rel:.3e}"
    finally:
        run.close()


# ------------------------------------------------------- full-size ones --

def _run_full(zs, w, calls, pack_checks=False):
    """The workload's schedule on the GPU as the benchmark runs it (device
    counter), the global norm state read after every call; then the oracle
    over the whole shard and the comparison of every call's norm state and
    every element of the final state."""
    import torch
    st = _step_for(zs, w, device_counter=True)
    _init_state(st, w, w.shard_start())
    reps = None
    dev_accs = []
    for call in calls:
        reps = _device_replicas(w, call, w.shard_start(), w.S, out=reps)
        st.step(reps)
        dev_accs.append(st.acc.clone())
    applied = st.applied_steps()
    torch.cuda.synchronize()
    del reps
    log(f"{w.name}: GPU done ({len(calls)} calls), oracle over {w.S} elements")
    run = OracleRun(w, w.shard_start(), w.S)
    try:
        for call, dacc in zip(calls, dev_accs):
            skip, coef, acc = run.call(call)
            log(f"{w.name}: call {call}: skip {skip}, coef {coef!r}")
            assert _acc_sum(zs, dacc) == (acc.X, int(acc.nonfinite)), f"norm state, call {call}"
        assert applied == run.t, (applied, run.t)
        _assert_state(st, run, w.name)
        if pack_checks:
            want_e, want_s = run.mxfp8()
            assert st.fuse_pack
            assert compare_full(f"{w.name} fused mxfp8 codes", st.mx_elem, want_e)[0] == 0
            assert compare_full(f"{w.name} fused mxfp8 scales", st.mx_scale, want_s)[0] == 0
            st.mx_elem.zero_()
            st.mx_scale.zero_()
            st.pack_param()                       # the standalone pack kernel
            torch.cuda.synchronize()
            assert compare_full(f"{w.name} mxfp8 codes", st.mx_elem, want_e)[0] == 0
            assert compare_full(f"{w.name} mxfp8 scales", st.mx_scale, want_s)[0] == 0
        return st, run
    finally:
        run.close()


@pytest.mark.timeout(900)
def test_1p3b_unsharded_loss_scale_skip(zs):
    w = configs.UNSHARDED_1P3B
    st, run = _run_full(zs, w, calls=range(1, w.steps + 1))
    assert [s for _, s, _, _ in run.gates] == [c == 5 for c in range(1, 11)]
    assert st.path == "recompute" and run.t == 9
    del st


@pytest.mark.timeout(900)
def test_7b_shard_35_buckets_clip(zs):
    w = configs.SHARD_7B
    st, run = _run_full(zs, w, calls=range(1, w.steps + 1))
    assert st.path == "materialize" and st.bucket == 25_000_000 and run.t == w.steps
    assert all(0 < c < 1 for _, _, c, _ in run.gates)       # the clip acts at every step
    del st


@pytest.mark.timeout(1200)
def test_30b_shard_clip_overflow_then_mxfp8(zs):
    w = configs.SHARD_30B
    st, run = _run_full(zs, w, calls=range(1, w.steps + 1), pack_checks=True)
    assert run.t == w.steps
    del st


@pytest.mark.timeout(1200)
def test_30b_shard_mxfp8_stored_grads(zs):
    # all five calls; the host packs and decodes every replica chunk of every
    # call (8 x 3.75e9 elements per call, about 80 s on 16 threads)
    w = configs.SHARD_30B_MX
    st, run = _run_full(zs, w, calls=range(1, w.steps + 1), pack_checks=True)
    assert st.path == "materialize" and run.t == w.steps
    del st

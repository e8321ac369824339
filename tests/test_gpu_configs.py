"""Parity at the five workloads' real sizes, in the launch configuration the
benchmark times (ShardStep with the workload's bucket, gate and pack
settings).

  - 1M-element, P=4 fp32 case and the GPT-2-small-sized P=8 case: every
    element of every rank compared with the oracle; the P=8 case also checks
    that the 8 shard steps equal one unsharded step of the full vector on the
    GPU (reduce-scatter + all-gather = all-reduce).
  - 1.3B, 7B and 30B cases: the oracle computes each call's global norm and
    overflow count over the whole shard (inputs regenerated on the host from
    the counter-based generator, spread over threads), then follows sampled
    elements (random indices plus tile, bucket and tail boundaries) through
    every call; the GPU state at those indices must match bit for bit.  The
    30B case also checks the MXFP8 pack of sampled 32-element blocks.
Step counts of the three large cases are cut (noted per test) to keep the host
side of the oracle within a couple of minutes.
"""
import numpy as np
import pytest

import oracle as O
import synth
from gpu_util import (from_dev, gpu_or_skip, mismatch_report, oracle_norm_parallel,
                      same_bits)
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


def _host_replicas(w, call, lo, n):
    reps = [synth.fill(w.grad_spec(call, k), lo, n, w.grad_bf16, threads=8) for k in range(w.P)]
    if w.inject and w.inject[0] == call and lo <= w.inject[1] < lo + n:
        reps[0][w.inject[1] - lo] = 0x7F80 if w.grad_bf16 else np.float32(np.inf)
    return reps


def _compare_state(st, want, where=""):
    names = ("master", "m", "v", "param")
    got = (from_dev(st.master), from_dev(st.m), from_dev(st.v), from_dev(st.param, True))
    for name, g, h in zip(names, got, want):
        assert same_bits(g, h), mismatch_report(f"{where} {name}", g, h)


# -------------------------------------------------------------- full ones --

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
        hreps = _host_replicas(w, 1, lo, w.S)
        skipped, _ = O.step(hreps, O.inv_scale(w.P, 1.0), 0.0, False, w.lr, w.beta1, w.beta2,
                            w.eps, w.wd, 1, master, m, v, param)
        assert not skipped
        _compare_state(st, (master, m, v, param), f"rank {rank}")


@pytest.mark.timeout(900)
def test_gpt2_small_p8_ten_steps_all_ranks(zs):
    import torch
    w = configs.GPT2_SMALL
    ranks = [_step_for(zs, w) for _ in range(w.P)]
    for r, st in enumerate(ranks):
        _init_state(st, w, r * w.S)
    # unsharded reference on the GPU: one rank holding the whole vector
    full = _step_for(zs, w, n=w.N, path="materialize")
    _init_state(full, w, 0)
    accs = zs.new_norm_acc(w.P)
    reps = None
    # oracle: rank 0 in full, global norm from all ranks
    master = synth.fill(w.master_spec(), 0, w.S, False)
    m, v = np.zeros(w.S, np.float32), np.zeros(w.S, np.float32)
    param = O.f32_to_bf16(master)
    inv = O.inv_scale(w.P, 1.0)
    for call in range(1, w.steps + 1):
        reps = _device_replicas(w, call, 0, w.N, out=reps)
        for r, st in enumerate(ranks):
            st.reduce([x[r * w.S:(r + 1) * w.S] for x in reps])
            accs[r].copy_(st.acc[0])
        for r, st in enumerate(ranks):
            st.update([x[r * w.S:(r + 1) * w.S] for x in reps], accs=accs)
        full.reduce(reps)
        full.update(reps)
        rest = oracle_norm_parallel(w, call, w.S, w.N)
        skipped, _ = O.step(_host_replicas(w, call, 0, w.S), inv, w.max_norm, w.check_overflow,
                            w.lr, w.beta1, w.beta2, w.eps, w.wd, call, master, m, v, param,
                            extra_accs=[rest])
        assert not skipped
    torch.cuda.synchronize()
    _compare_state(ranks[0], (master, m, v, param), "rank 0 vs oracle")
    for name in ("master", "m", "v", "param"):
        cat = torch.cat([getattr(st, name) for st in ranks])
        assert torch.equal(cat, getattr(full, name)), f"sharded != unsharded: {name}"


# ----------------------------------------------------------- sampled ones --

def _sample_indices(w, rng, k=4096):
    S = w.S
    idx = set(int(i) for i in rng.integers(0, S, size=k))
    marks = [0, 1, 7, 8, 31, 32, 2047, 2048, S - 33, S - 32, S - 1]
    if w.bucket:
        for b in range(w.bucket, S, w.bucket):
            marks += [b - 1, b]
    if w.inject:
        marks += [w.inject[1] - 1, w.inject[1], w.inject[1] + 1]
    idx.update(i for i in marks if 0 <= i < S)
    idx = np.array(sorted(idx), dtype=np.uint64)
    if w.mx_grads:
        # whole 32-element blocks: a decoded element depends on its block
        blocks = np.unique(idx // np.uint64(32))
        idx = (blocks[:, None] * np.uint64(32) + np.arange(32, dtype=np.uint64)[None, :]).ravel()
    return idx


def _oracle_gates(w, calls):
    gates = []
    for call in calls:
        acc = oracle_norm_parallel(w, call, w.shard_start(), w.shard_start() + w.S)
        skip, coef = O.gate(acc, w.max_norm, w.check_overflow)
        gates.append((coef, skip))
    return gates


def _oracle_samples(w, idx, calls, gates):
    gidx = idx + np.uint64(w.shard_start())
    master = synth.gather(w.master_spec(), gidx, False)
    m, v = np.zeros(idx.size, np.float32), np.zeros(idx.size, np.float32)
    param = O.f32_to_bf16(master)
    inv = O.inv_scale(w.P, w.loss_scale)
    t = 0
    for call, (coef, skip) in zip(calls, gates):
        if skip:
            continue
        t += 1
        reps = [synth.gather(w.grad_spec(call, k), gidx, w.grad_bf16) for k in range(w.P)]
        if w.inject and w.inject[0] == call:
            hit = np.nonzero(gidx == np.uint64(w.inject[1]))[0]
            for h in hit:
                reps[0][h] = 0x7F80 if w.grad_bf16 else np.float32(np.inf)
        if w.mx_grads:      # idx holds whole blocks, in order
            reps = [O.mxfp8_decode(*O.mxfp8_pack(r)) for r in reps]
        g = O.reduce(reps, inv)
        O.adamw(g, coef, O.make_scalars(w.lr, w.beta1, w.beta2, w.eps, w.wd, t), master, m,
                v, param)
    return master, m, v, param, t


def _run_sampled(zs, w, calls, seed):
    import torch
    rng = np.random.default_rng(seed)
    idx = _sample_indices(w, rng)
    st = _step_for(zs, w, device_counter=True)     # as the benchmark runs the step
    _init_state(st, w, w.shard_start())
    reps = None
    for call in calls:
        reps = _device_replicas(w, call, w.shard_start(), w.S, out=reps)
        st.step(reps)
    applied = st.applied_steps()
    torch.cuda.synchronize()
    di = torch.from_numpy(idx.astype(np.int64)).cuda()
    got = (from_dev(st.master[di]), from_dev(st.m[di]), from_dev(st.v[di]),
           from_dev(st.param[di], True))
    del reps
    gates = _oracle_gates(w, calls)
    want = _oracle_samples(w, idx, calls, gates)
    assert applied == want[4], (applied, want[4])
    for name, g, h in zip(("master", "m", "v", "param"), got, want[:4]):
        assert same_bits(g, h), mismatch_report(f"{w.name} {name}", g, h)
    return st, idx, gates


@pytest.mark.timeout(900)
def test_1p3b_unsharded_loss_scale_skip(zs):
    # calls 1..6 of 10: covers the injected overflow at call 5 and the
    # applied step after it
    w = configs.UNSHARDED_1P3B
    st, _, gates = _run_sampled(zs, w, calls=range(1, 7), seed=3)
    assert [s for _, s in gates] == [False, False, False, False, True, False]
    assert st.path == "recompute"
    assert int(st.skipped.item()) == 0


@pytest.mark.timeout(900)
def test_7b_shard_35_buckets_clip(zs):
    # 2 of the 10 steps at the full 875M shard, 35 buckets of 25M
    w = configs.SHARD_7B
    st, _, _ = _run_sampled(zs, w, calls=range(1, 3), seed=4)
    assert st.path == "materialize" and st.bucket == 25_000_000


@pytest.mark.timeout(1200)
def test_30b_shard_clip_overflow_then_mxfp8(zs):
    # 2 of the 5 steps at the full 3.75B shard, then the MXFP8 pack
    import torch
    w = configs.SHARD_30B
    rng = np.random.default_rng(5)
    st, idx, gates = _run_sampled(zs, w, calls=range(1, 3), seed=5)
    blocks = np.unique(rng.integers(0, w.S // 32, size=256))
    blocks = np.unique(np.concatenate([blocks, [0, w.S // 32 - 1]]))
    eidx = (blocks[:, None] * 32 + np.arange(32)[None, :]).ravel().astype(np.uint64)
    de = torch.from_numpy(eidx.astype(np.int64)).cuda()
    ds = torch.from_numpy(blocks.astype(np.int64)).cuda()
    assert st.fuse_pack
    fused_e, fused_s = from_dev(st.mx_elem[de]), from_dev(st.mx_scale[ds])
    st.pack_param()                       # the standalone pack kernel
    torch.cuda.synchronize()
    got_e, got_s = from_dev(st.mx_elem[de]), from_dev(st.mx_scale[ds])
    _, _, _, param, _ = _oracle_samples(w, eidx, range(1, 3), gates)
    want_e, want_s = O.mxfp8_pack(param)
    for e, sc in ((fused_e, fused_s), (got_e, got_s)):
        assert np.array_equal(sc, want_s)
        assert np.array_equal(e, want_e)


@pytest.mark.timeout(1200)
def test_30b_shard_mxfp8_stored_grads(zs):
    # 1 of the 5 steps at the full 3.75B shard: the host oracle packs and
    # decodes all 8 replicas of the whole shard for the norm (~2 min on 16
    # threads), so one call is what fits
    w = configs.SHARD_30B_MX
    st, idx, gates = _run_sampled(zs, w, calls=range(1, 2), seed=6)
    assert st.path == "materialize" and idx.size % 32 == 0
    assert gates[0][1] is False

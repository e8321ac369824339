"""Seeded random configurations of the whole step, each run through ShardStep
(the sequencing the benchmark uses) and compared bit for bit with the
oracle's step after three calls: master, m, v, the bf16 param, the MXFP8
pack of the param, the count of applied updates and the last call's norm
state.

Each case draws: the replica count P (1 to 64), the replica type (fp32, bf16,
or bf16 stored as MXFP8), a length n (ragged, or a multiple of 32 where MXFP8
needs it), the gate (none, clip, overflow check, both) with a clip threshold
from very tight to never acting, a loss scale, buckets of any multiple of 32
or none, the one-shot or pipelined reduce, a forced pass structure, the
fused or standalone pack, the host or device step counter, one or two
bucket streams, and the AdamW hyperparameters.  With the overflow check on,
some cases put an infinity into one replica at one call, which the gate
must skip.  Forty more configurations run as a recorded graph, replayed for
each call on fresh gradients and compared after every replay.
"""
import numpy as np
import pytest

import oracle as O
import synth
from gpu_util import acc_from_oracle, from_dev, gpu_or_skip, mismatch_report, same_bits

pytestmark = pytest.mark.gpu

N_CASES = 200
STEPS = 3


@pytest.fixture(scope="module")
def zs():
    gpu_or_skip()
    import zero_sharded_mixed_step_amd as zs
    zs.lib()
    return zs


def _draw(case):
    rng = np.random.default_rng(7000 + case)
    kind = ("f32", "bf16", "mxfp8")[int(rng.integers(3))]
    P = int(rng.choice([1, 2, 3, 4, 5, 8, 16, 64]))
    pack = bool(rng.integers(2))
    n = int(rng.integers(1, 3000 if P == 64 else 70000))
    if pack or kind == "mxfp8":
        n = max(32, n // 32 * 32)
    gate = int(rng.integers(4))                    # none, clip, check, clip + check
    check = gate >= 2
    cfg = dict(
        kind=kind, P=P, n=n, pack=pack,
        max_norm=float(rng.choice([1e-3, 0.05, 1.0, 1e6])) if gate in (1, 3) else 0.0,
        check_overflow=check,
        loss_scale=float(rng.choice([1.0, 1024.0, 65536.0])),
        bucket=None if rng.integers(2) else int(rng.integers(1, n // 32 + 2)) * 32,
        oneshot_min=None if rng.integers(2) else 0,
        path=(("materialize", "recompute")[int(rng.integers(2))]
              if gate and kind != "mxfp8" and rng.integers(3) == 0 else None),
        fuse_pack=bool(rng.integers(2)),
        device_counter=bool(rng.integers(2)),
        bucket_streams=int(rng.choice([1, 2])),
        lr=float(10.0 ** rng.uniform(-4, -1)),
        beta1=float(rng.choice([0.9, 0.5, 0.0])),
        beta2=float(rng.choice([0.999, 0.95])),
        eps=float(rng.choice([1e-8, 1e-6])),
        weight_decay=float(rng.choice([0.0, 0.01, 0.1])),
        inject=(int(rng.integers(1, STEPS + 1)) if check and rng.integers(3) == 0 else 0),
        inject_at=(int(rng.integers(P)), int(rng.integers(n))),
    )
    return cfg


def _grad_spec(case, call, k, loss_scale):
    return synth.make_spec(seed=case, cfg=70, stream=1, step=call, replica=k, sigma=1e-3,
                           outlier_rate=0.01, outlier_mult=100.0, post_mul=loss_scale)


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_step_configuration(zs, case):
    import torch
    c = _draw(case)
    n, P, kind = c["n"], c["P"], c["kind"]
    gdt = {"f32": torch.float32, "bf16": torch.bfloat16, "mxfp8": "mxfp8"}[kind]
    st = zs.ShardStep(n, P, gdt, lr=c["lr"], beta1=c["beta1"], beta2=c["beta2"], eps=c["eps"],
                      weight_decay=c["weight_decay"], max_norm=c["max_norm"],
                      check_overflow=c["check_overflow"], loss_scale=c["loss_scale"],
                      bucket=c["bucket"], pack=c["pack"], fuse_pack=c["fuse_pack"],
                      path=c["path"], device_counter=c["device_counter"],
                      oneshot_min=c["oneshot_min"], bucket_streams=c["bucket_streams"])
    mspec = synth.make_spec(seed=case, cfg=70, stream=0, sigma=0.02)
    synth.fill_device(mspec, 0, st.master)
    synth.fill_device(mspec, 0, st.param)
    if c["pack"]:
        st.mx_elem.zero_()
        st.mx_scale.zero_()
    master = synth.fill(mspec, 0, n, False)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    param = O.f32_to_bf16(master)

    bf16_src = kind != "f32"
    dev_src = [torch.empty(n, dtype=torch.int16 if bf16_src else torch.float32, device="cuda")
               for _ in range(P)]
    if kind == "mxfp8":
        dev_reps = [(torch.empty(n, dtype=torch.uint8, device="cuda"),
                     torch.empty(n // 32, dtype=torch.uint8, device="cuda")) for _ in range(P)]
    else:
        dev_reps = dev_src
    inv = O.inv_scale(P, c["loss_scale"])
    applied, own = 0, None
    for call in range(1, STEPS + 1):
        host = [synth.fill(_grad_spec(case, call, k, c["loss_scale"]), 0, n, bf16_src)
                for k in range(P)]
        for k, r in enumerate(dev_src):
            synth.fill_device(_grad_spec(case, call, k, c["loss_scale"]), 0, r)
        if c["inject"] == call:
            k, i = c["inject_at"]
            host[k][i] = 0x7F80 if bf16_src else np.float32(np.inf)
            dev_src[k][i] = 0x7F80 if bf16_src else float("inf")
        if kind == "mxfp8":
            for r, (codes, scales) in zip(dev_src, dev_reps):
                zs.zero_mxfp8_pack(r, codes, scales)
            host = [O.mxfp8_decode(*O.mxfp8_pack(r)) for r in host]
        st.step(dev_reps)
        skipped, own = O.step(host, inv, c["max_norm"], c["check_overflow"], c["lr"],
                              c["beta1"], c["beta2"], c["eps"], c["weight_decay"], applied + 1,
                              master, m, v, param)
        applied += 0 if skipped else 1
    torch.cuda.synchronize()

    where = f"case {case} {c}"
    assert st.applied_steps() == applied, where
    for name, want in (("master", master), ("m", m), ("v", v), ("param", param)):
        got = from_dev(getattr(st, name), name == "param")
        assert same_bits(got, want), mismatch_report(f"{where} {name}", got, want)
    if st.path != "fused":
        assert zs.read_norm_acc(st.acc)[0] == acc_from_oracle(own), where
    if c["pack"] and applied:
        want_e, want_s = O.mxfp8_pack(param)
        assert same_bits(from_dev(st.mx_elem), want_e), f"{where} mxfp8 codes"
        assert same_bits(from_dev(st.mx_scale), want_s), f"{where} mxfp8 scales"


N_GRAPH_CASES = 40


@pytest.mark.parametrize("case", range(N_GRAPH_CASES))
def test_random_configuration_graph_replay(zs, case):
    """A random configuration (as above, with the device step counter that
    recording needs) recorded once as a graph and replayed for three calls,
    with fresh gradients written into the same replica buffers by eager
    work between the replays: after every replay the state is bit for bit
    the oracle's."""
    import torch
    c = _draw(10_000 + case)
    c["device_counter"] = True
    n, P, kind = c["n"], c["P"], c["kind"]
    gdt = {"f32": torch.float32, "bf16": torch.bfloat16, "mxfp8": "mxfp8"}[kind]
    st = zs.ShardStep(n, P, gdt, lr=c["lr"], beta1=c["beta1"], beta2=c["beta2"], eps=c["eps"],
                      weight_decay=c["weight_decay"], max_norm=c["max_norm"],
                      check_overflow=c["check_overflow"], loss_scale=c["loss_scale"],
                      bucket=c["bucket"], pack=c["pack"], fuse_pack=c["fuse_pack"],
                      path=c["path"], device_counter=True, oneshot_min=c["oneshot_min"],
                      bucket_streams=c["bucket_streams"])
    mspec = synth.make_spec(seed=case, cfg=71, stream=0, sigma=0.02)
    synth.fill_device(mspec, 0, st.master)
    synth.fill_device(mspec, 0, st.param)
    if c["pack"]:
        st.mx_elem.zero_()
        st.mx_scale.zero_()
    master = synth.fill(mspec, 0, n, False)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    param = O.f32_to_bf16(master)
    bf16_src = kind != "f32"
    dev_src = [torch.empty(n, dtype=torch.int16 if bf16_src else torch.float32, device="cuda")
               for _ in range(P)]
    if kind == "mxfp8":
        dev_reps = [(torch.empty(n, dtype=torch.uint8, device="cuda"),
                     torch.empty(n // 32, dtype=torch.uint8, device="cuda")) for _ in range(P)]
    else:
        dev_reps = dev_src
    inv = O.inv_scale(P, c["loss_scale"])

    def fill(call):
        host = [synth.fill(_grad_spec(10_000 + case, call, k, c["loss_scale"]), 0, n, bf16_src)
                for k in range(P)]
        for k, r in enumerate(dev_src):
            synth.fill_device(_grad_spec(10_000 + case, call, k, c["loss_scale"]), 0, r)
        if c["inject"] == call:
            k, i = c["inject_at"]
            host[k][i] = 0x7F80 if bf16_src else np.float32(np.inf)
            dev_src[k][i] = 0x7F80 if bf16_src else float("inf")
        if kind == "mxfp8":
            for r, (codes, scales) in zip(dev_src, dev_reps):
                zs.zero_mxfp8_pack(r, codes, scales)
            host = [O.mxfp8_decode(*O.mxfp8_pack(r)) for r in host]
        return host

    torch.cuda.synchronize()
    graph = st.capture(dev_reps)                 # records; runs nothing
    torch.cuda.synchronize()
    applied = 0
    where = f"graph case {case} {c}"
    for call in range(1, STEPS + 1):
        host = fill(call)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        skipped, own = O.step(host, inv, c["max_norm"], c["check_overflow"], c["lr"],
                              c["beta1"], c["beta2"], c["eps"], c["weight_decay"], applied + 1,
                              master, m, v, param)
        applied += 0 if skipped else 1
        assert st.applied_steps() == applied, f"{where} call {call}"
        for name, want in (("master", master), ("m", m), ("v", v), ("param", param)):
            got = from_dev(getattr(st, name), name == "param")
            assert same_bits(got, want), mismatch_report(f"{where} call {call} {name}", got, want)
        if st.path != "fused":
            assert zs.read_norm_acc(st.acc)[0] == acc_from_oracle(own), f"{where} call {call}"
        if c["pack"] and applied:
            want_e, want_s = O.mxfp8_pack(param)
            assert same_bits(from_dev(st.mx_elem), want_e), f"{where} call {call} codes"
            assert same_bits(from_dev(st.mx_scale), want_s), f"{where} call {call} scales"
    del graph

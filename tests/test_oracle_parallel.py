"""The threaded driver of the oracle step (used for the all-cores CPU
timing) gives bit for bit the serial oracle step: the norm state is an
integer sum, so slicing the vector across threads changes nothing."""
import numpy as np
import pytest

import oracle as O
import synth


@pytest.mark.parametrize("threads", [1, 3, 8])
@pytest.mark.parametrize("inject", [False, True])
def test_step_parallel_equals_step(threads, inject):
    n, P = 32 * 3001 + 17, 4
    reps = [synth.fill(synth.make_spec(seed=9, cfg=60, stream=1, step=1, replica=k, sigma=1e-3,
                                       outlier_rate=0.01, outlier_mult=100.0), 0, n, True)
            for k in range(P)]
    if inject:
        reps[2][n // 2] = 0x7F80
    master0 = synth.fill(synth.make_spec(seed=9, cfg=60, stream=0, sigma=0.02), 0, n, False)
    states = []
    for fn in (O.step, lambda *a: O.step_parallel(*a, threads=threads)):
        master, m, v = master0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
        param = O.f32_to_bf16(master)
        flags = []
        for t in (1, 2, 3):
            skipped, acc = fn(reps, O.inv_scale(P, 1.0), 0.05, True, 1e-3, 0.9, 0.999, 1e-8,
                              0.01, t, master, m, v, param)
            flags.append((skipped, acc.X, int(acc.nonfinite)))
        states.append((flags, master, m, v, param))
    (f1, *a1), (f2, *a2) = states
    assert f1 == f2
    assert f1[0][0] == inject
    for x, y in zip(a1, a2):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


@pytest.mark.parametrize("mx", [False, True])
def test_oracle_run_equals_plain_steps(mx):
    """The whole-workload driver the full-size GPU parity tests use
    (chunked, threaded, host state) gives bit for bit what plain oracle steps
    on whole arrays give, through a skipped call, with clipping and a ragged
    last chunk."""
    import dataclasses
    from gpu_util import OracleRun
    from synth import configs
    w = dataclasses.replace(configs.SHARD_30B_MX if mx else configs.SHARD_30B,
                            S=32 * 9001, N=32 * 9001 * 8, steps=3, inject=(2, 32 * 9001 + 77),
                            rank=1)
    lo = w.shard_start()
    run = OracleRun(w, lo, w.S, threads=3, chunk=32 * 1000)
    master = synth.fill(w.master_spec(), lo, w.S, False)
    m, v = np.zeros(w.S, np.float32), np.zeros(w.S, np.float32)
    param = O.f32_to_bf16(master)
    t = 0
    for call in range(1, 4):
        reps = [synth.fill(w.grad_spec(call, k), lo, w.S, True) for k in range(w.P)]
        if call == 2:
            reps[0][77] = 0x7F80
        if mx:
            reps = [O.mxfp8_decode(*O.mxfp8_pack(r)) for r in reps]
        skipped, acc = O.step(reps, O.inv_scale(w.P, 1.0), w.max_norm, w.check_overflow,
                              w.lr, w.beta1, w.beta2, w.eps, w.wd, t + 1, master, m, v, param)
        t += 0 if skipped else 1
        skip, _, racc = run.call(call)
        assert skip == skipped == (call == 2)
        assert (racc.X, racc.nonfinite) == (acc.X, acc.nonfinite)
    assert run.t == t == 2
    for a, b in ((run.master, master), (run.m, m), (run.v, v), (run.param, param)):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    e1, s1 = run.mxfp8()
    run.close()
    e2, s2 = O.mxfp8_pack(param)
    assert np.array_equal(e1, e2) and np.array_equal(s1, s2)

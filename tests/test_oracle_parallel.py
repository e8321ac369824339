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

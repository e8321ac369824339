"""Checkpoint and resume change nothing: 10 steps equal 5 steps, the state
saved to a file and loaded into fresh buffers, then the other 5 steps, bit
for bit.  The schedule skips one call (an injected inf with the overflow
check), so the count of applied updates must survive the round trip too.
On the oracle (CPU) and on the device path through ShardStep (GPU)."""
import numpy as np
import pytest

import oracle as O
import synth

N, P = 32 * 1003, 4          # several tiles and a ragged last one
HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.01)
MAX_NORM = 0.05


def _grads(call):
    reps = [synth.fill(synth.make_spec(seed=2, cfg=71, stream=1, step=call, replica=k,
                                       sigma=1e-3, outlier_rate=0.01, outlier_mult=100.0),
                       0, N, True) for k in range(P)]
    if call == 4:
        reps[1][N // 2] = 0x7F80              # this call is skipped
    return reps


def _master0():
    return synth.fill(synth.make_spec(seed=2, cfg=71, stream=0, sigma=0.02), 0, N, False)


def _oracle_run(state, calls):
    master, m, v, param, t = state
    for call in calls:
        skipped, _ = O.step(_grads(call), O.inv_scale(P, 1.0), MAX_NORM, True, HP["lr"],
                            HP["beta1"], HP["beta2"], HP["eps"], HP["wd"], t + 1,
                            master, m, v, param)
        t += 0 if skipped else 1
    return master, m, v, param, t


def test_oracle_resume_equals_uninterrupted(tmp_path):
    master = _master0()
    fresh = lambda: [master.copy(), np.zeros(N, np.float32), np.zeros(N, np.float32),
                     O.f32_to_bf16(master), 0]
    whole = _oracle_run(fresh(), range(1, 11))
    half = _oracle_run(fresh(), range(1, 6))
    path = tmp_path / "ckpt.npz"
    np.savez(path, master=half[0], m=half[1], v=half[2], param=half[3], t=half[4])
    with np.load(path) as z:
        state = [z["master"].copy(), z["m"].copy(), z["v"].copy(), z["param"].copy(), int(z["t"])]
    resumed = _oracle_run(state, range(6, 11))
    assert whole[4] == resumed[4] == 9
    for a, b in zip(whole[:4], resumed[:4]):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


@pytest.mark.gpu
@pytest.mark.parametrize("device_counter", [True, False])
def test_shard_step_resume_equals_uninterrupted(tmp_path, device_counter):
    from gpu_util import from_dev, gpu_or_skip, to_dev
    torch = gpu_or_skip()
    import zero_sharded_mixed_step_amd as zs

    def new():
        st = zs.ShardStep(N, P, torch.bfloat16, lr=HP["lr"], beta1=HP["beta1"],
                          beta2=HP["beta2"], eps=HP["eps"], weight_decay=HP["wd"],
                          max_norm=MAX_NORM, check_overflow=True, pack=True,
                          device_counter=device_counter)
        st.master.copy_(to_dev(_master0()))
        st.param.copy_(to_dev(O.f32_to_bf16(_master0())))
        return st

    def run(st, calls):
        for call in calls:
            st.step([to_dev(r) for r in _grads(call)])

    whole = new()
    run(whole, range(1, 11))
    first = new()
    run(first, range(1, 6))
    path = tmp_path / "ckpt.pt"
    torch.save(first.state(), path)
    del first
    resumed = new()
    resumed.load_state(torch.load(path, weights_only=True))
    run(resumed, range(6, 11))
    torch.cuda.synchronize()
    assert whole.applied_steps() == resumed.applied_steps() == 9
    for name in ("master", "m", "v", "param", "mx_elem", "mx_scale"):
        a, b = from_dev(getattr(whole, name)), from_dev(getattr(resumed, name))
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), name
    # and the device path equals the oracle's uninterrupted run
    master = _master0()
    want = _oracle_run([master.copy(), np.zeros(N, np.float32), np.zeros(N, np.float32),
                        O.f32_to_bf16(master), 0], range(1, 11))
    for name, w in zip(("master", "m", "v", "param"), want[:4]):
        got = from_dev(getattr(resumed, name), name == "param")
        assert np.array_equal(got.view(np.uint8), w.view(np.uint8)), name

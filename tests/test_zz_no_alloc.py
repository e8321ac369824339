"""zero_shard_reduce_noalloc (the reduce whose norm slots live in the
library's static device array) against zero_shard_reduce_ws (the same reduce
with a caller workspace) and the oracle, through the C ABI: two calls in a
row on the same GPU, the second on a smaller input, bitwise."""
import numpy as np
import pytest

import oracle as O
import synth
from gpu_util import acc_from_oracle, from_dev, gpu_or_skip, same_bits, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def zs():
    gpu_or_skip()
    import zero_sharded_mixed_step_amd as zs
    zs.lib()
    return zs


def _replicas(P, n, bf16, seed):
    reps = []
    for k in range(P):
        sp = synth.make_spec(seed=seed, cfg=70, stream=1, step=1, replica=k, sigma=1e-3,
                             outlier_rate=0.01, outlier_mult=100.0)
        reps.append(synth.fill(sp, 0, n, bf16))
    # non-finite values and a large finite one (its group's sum of squares
    # is past 2^64)
    reps[0][n // 3] = 0x7F80 if bf16 else np.float32(np.inf)
    reps[P - 1][7] = 0x7FC0 if bf16 else np.float32(np.nan)
    reps[P // 2][n - 40] = 0x5080 if bf16 else np.float32(2.0 ** 34)
    return reps


@pytest.mark.parametrize("P,bf16", [(8, True), (4, False), (16, True)])
def test_noalloc_reduce_equals_workspace_reduce(zs, P, bf16):
    import torch
    ws = zs.new_reduce_workspace()
    # the second call is smaller than the first; both span many workgroups
    # (several per slot) and end in a ragged tail
    for n in (2048 * 3001 + 8 * 77 + 5, 2048 * 517 + 3):
        reps = _replicas(P, n, bf16, seed=n)
        inv = O.inv_scale(P, 1.0)
        want_g = O.reduce(reps, inv)
        want_acc = acc_from_oracle(O.norm_accumulate(want_g))
        dreps = [to_dev(r) for r in reps]
        g_ws = torch.empty(n, dtype=torch.float32, device="cuda")
        acc_ws = zs.new_norm_acc(1)
        zs.zero_shard_reduce_ws(dreps, inv, ws, g_out=g_ws, acc=acc_ws)
        g_na = torch.full((n,), 7.0, dtype=torch.float32, device="cuda")
        acc_na = zs.new_norm_acc(1)
        zs.zero_shard_reduce_noalloc(dreps, inv, g_out=g_na, acc=acc_na)
        acc_only = zs.new_norm_acc(1)
        zs.zero_shard_reduce_noalloc(dreps, inv, acc=acc_only)
        torch.cuda.synchronize()
        assert same_bits(from_dev(g_na), from_dev(g_ws)), n
        assert same_bits(from_dev(g_na), want_g), n
        assert zs.read_norm_acc(acc_na)[0] == zs.read_norm_acc(acc_ws)[0] == want_acc, n
        assert zs.read_norm_acc(acc_only)[0] == want_acc, n
        assert int(ws.abs().sum().item()) == 0


def test_noalloc_reduce_argument_checks(zs):
    import torch
    g = torch.empty(64, dtype=torch.float32, device="cuda")
    r = torch.zeros(64, dtype=torch.int16, device="cuda")
    with pytest.raises(zs.ZeroStepError):
        zs.zero_shard_reduce_noalloc([r, r], 0.5)                 # neither g_out nor acc
    with pytest.raises(zs.ZeroStepError):
        zs.zero_shard_reduce_noalloc([r[1:33], r[:32]], 0.5, g_out=g[:32])   # misaligned
    zs.zero_shard_reduce_noalloc([r, r], 0.5, g_out=g, n=0)       # n == 0: a no-op

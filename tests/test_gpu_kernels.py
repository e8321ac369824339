"""Kernel-level parity of the HIP path against the CPU oracle, through the C
ABI, at sizes that span several tiles plus ragged tails.  Bitwise throughout:
reduction, norm accumulator, clip/skip gate, AdamW state, bf16 param and
MXFP8 codes."""
import numpy as np
import pytest

import oracle as O
import synth
from gpu_util import (acc_from_oracle, from_dev, gpu_or_skip, mismatch_report, same_bits,
                      to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def zs():
    gpu_or_skip()
    import zero_sharded_mixed_step_amd as zs
    zs.lib()
    return zs


def _replicas(P, n, bf16, seed, inject=()):
    reps = []
    for k in range(P):
        sp = synth.make_spec(seed=seed, cfg=50, stream=1, step=1, replica=k, sigma=1e-3,
                             outlier_rate=0.01, outlier_mult=100.0)
        reps.append(synth.fill(sp, 0, n, bf16))
    for (k, i, val) in inject:
        if bf16:
            reps[k][i] = O.f32_to_bf16(np.array([val], np.float32))[0]
        else:
            reps[k][i] = np.float32(val)
    return reps


# ------------------------------------------------------------- generator --

@pytest.mark.parametrize("bf16", [False, True])
def test_device_generator_matches_host(zs, bf16):
    import torch
    cases = [(0, 1), (0, 1000), (12345, 1 << 20), ((1 << 32) + 7, 4099)]
    for start, count in cases:
        sp = synth.make_spec(seed=3, cfg=9, stream=1, step=2, replica=5, sigma=1e-3,
                             outlier_rate=0.01, outlier_mult=100.0, post_mul=65536.0)
        t = torch.empty(count, dtype=torch.int16 if bf16 else torch.float32, device="cuda")
        synth.fill_device(sp, start, t)
        assert same_bits(from_dev(t, bf16), synth.fill(sp, start, count, bf16)), (start, count)


# ---------------------------------------------------------------- reduce --

SIZES = [1, 7, 8, 16, 17, 31, 32, 33, 1024, 4097, 65536 + 13]


@pytest.mark.parametrize("P", [1, 2, 3, 4, 8, 16, 64])   # 64 = ZERO_MAX_REPLICAS
@pytest.mark.parametrize("bf16", [False, True])
def test_shard_reduce_and_norm(zs, P, bf16):
    import torch
    for n in SIZES:
        inject = [(P - 1, n - 1, np.inf)] if n > 5 else []
        if n > 100:
            inject += [(0, 3, np.nan), (P // 2, n // 2, -np.inf)]
            # large finite values: group sums of squares past 2^64, and one
            # near the top of binary32 (about 2^256): every group counts
            inject += [(0, 40, 2.0 ** 36), (P // 2, 72, 3.0e38 / P), (P - 1, 75, -1.0e10)]
        reps = _replicas(P, n, bf16, seed=n, inject=inject)
        inv = O.inv_scale(P, 1.0)
        want_g = O.reduce(reps, inv)
        want_acc = acc_from_oracle(O.norm_accumulate(want_g))
        dreps = [to_dev(r) for r in reps]
        g = torch.empty(n, dtype=torch.float32, device="cuda")
        acc = zs.new_norm_acc(1)
        zs.zero_shard_reduce(dreps, inv, g_out=g, acc=acc)
        acc2 = zs.new_norm_acc(1)
        zs.zero_shard_reduce(dreps, inv, acc=acc2)           # norm only
        g2 = torch.empty(n, dtype=torch.float32, device="cuda")
        zs.zero_shard_reduce(dreps, inv, g_out=g2)           # write only
        torch.cuda.synchronize()
        assert same_bits(from_dev(g), want_g), mismatch_report(f"g n={n}", from_dev(g), want_g)
        assert same_bits(from_dev(g2), want_g), n
        assert zs.read_norm_acc(acc)[0] == want_acc, (n, zs.read_norm_acc(acc)[0], want_acc)
        assert zs.read_norm_acc(acc2)[0] == want_acc, n
        # with the workspace (the one-shot grid for P >= 4): the same bits,
        # and the workspace is zero again after every call
        ws = zs.new_reduce_workspace()
        g3 = torch.empty(n, dtype=torch.float32, device="cuda")
        acc3 = zs.new_norm_acc(1)
        zs.zero_shard_reduce_ws(dreps, inv, ws, g_out=g3, acc=acc3)
        acc4 = zs.new_norm_acc(1)
        zs.zero_shard_reduce_ws(dreps, inv, ws, acc=acc4)
        g4 = torch.empty(n, dtype=torch.float32, device="cuda")
        zs.zero_shard_reduce_ws(dreps, inv, ws, g_out=g4)
        torch.cuda.synchronize()
        assert same_bits(from_dev(g3), want_g), n
        assert same_bits(from_dev(g4), want_g), n
        assert zs.read_norm_acc(acc3)[0] == want_acc, n
        assert zs.read_norm_acc(acc4)[0] == want_acc, n
        assert int(ws.abs().sum().item()) == 0, n


def test_grad_norm_with_loss_scale(zs):
    import torch
    for bf16 in (False, True):
        for n in (31, 4096, 100003):
            sp = synth.make_spec(seed=1, cfg=51, stream=1, sigma=1e-3, post_mul=65536.0)
            x = synth.fill(sp, 0, n, bf16)
            if bf16:
                x[n // 3] = 0x7F80
            inv = O.inv_scale(1, 65536.0)
            want = acc_from_oracle(O.norm_accumulate(O.reduce([x], inv)))
            acc = zs.new_norm_acc(1)
            zs.zero_grad_norm(to_dev(x), inv, acc)
            torch.cuda.synchronize()
            assert zs.read_norm_acc(acc)[0] == want, (bf16, n)


def test_buckets_and_grid_shapes_do_not_change_the_norm(zs):
    import torch
    P, n = 8, 32 * 50_001
    reps = [to_dev(r) for r in _replicas(P, n, True, seed=7)]
    inv = O.inv_scale(P, 1.0)
    whole = zs.new_norm_acc(1)
    zs.zero_shard_reduce(reps, inv, acc=whole)
    ws = zs.new_reduce_workspace()
    for bucket in (32, 4096, 32 * 7919, 1 << 20):
        for workspace in (None, ws):
            acc = zs.new_norm_acc(1)
            for lo in range(0, n, bucket):
                hi = min(n, lo + bucket)
                views = [r[lo:hi] for r in reps]
                if workspace is None:
                    zs.zero_shard_reduce(views, inv, acc=acc)
                else:
                    zs.zero_shard_reduce_ws(views, inv, workspace, acc=acc)
            torch.cuda.synchronize()
            assert zs.read_norm_acc(acc) == zs.read_norm_acc(whole), (bucket, workspace)
    assert int(ws.abs().sum().item()) == 0


@pytest.mark.parametrize("P,bf16", [(8, True), (4, False), (16, True)])
def test_one_shot_reduce_folds_many_slots(zs, P, bf16):
    """The one-shot form with thousands of workgroups, each slot of the
    workspace taken by several of them, then a ragged tail; repeated calls
    reuse the workspace, which each call leaves zero."""
    import torch
    n = 2048 * 6007 + 8 * 333 + 3
    reps = _replicas(P, n, bf16, seed=13, inject=[(0, n - 2, np.nan), (P - 1, 5, -np.inf)])
    inv = O.inv_scale(P, 1.0)
    want_g = O.reduce(reps, inv)
    want_acc = acc_from_oracle(O.norm_accumulate(want_g))
    dreps = [to_dev(r) for r in reps]
    ws = zs.new_reduce_workspace()
    g = torch.empty(n, dtype=torch.float32, device="cuda")
    accs = zs.new_norm_acc(3)
    for k in range(3):
        zs.zero_shard_reduce_ws(dreps, inv, ws, g_out=g, acc=accs[k])
    torch.cuda.synchronize()
    assert same_bits(from_dev(g), want_g), mismatch_report("g", from_dev(g), want_g)
    assert zs.read_norm_acc(accs) == [want_acc] * 3
    assert int(ws.abs().sum().item()) == 0


@pytest.mark.parametrize("P,bf16", [(4, True), (8, True), (4, False), (8, False)])
def test_pipelined_reduce_many_iterations(zs, P, bf16):
    """With 4 or 8 replicas the reduce's fast path is software pipelined over
    a one-workgroup-per-CU grid: sizes of a few million elements run many
    pipeline stages per workgroup, then a ragged tail (not a multiple of 8)."""
    import torch
    n = 3 * (1 << 20) + 8 * 1000 + 5
    reps = _replicas(P, n, bf16, seed=11, inject=[(P - 1, n // 2, np.inf)])
    inv = O.inv_scale(P, 1.0)
    want_g = O.reduce(reps, inv)
    want_acc = acc_from_oracle(O.norm_accumulate(want_g))
    dreps = [to_dev(r) for r in reps]
    g = torch.empty(n, dtype=torch.float32, device="cuda")
    acc = zs.new_norm_acc(1)
    zs.zero_shard_reduce(dreps, inv, g_out=g, acc=acc)
    acc2 = zs.new_norm_acc(1)
    zs.zero_shard_reduce(dreps, inv, acc=acc2)
    torch.cuda.synchronize()
    assert same_bits(from_dev(g), want_g), mismatch_report("g", from_dev(g), want_g)
    assert zs.read_norm_acc(acc)[0] == want_acc
    assert zs.read_norm_acc(acc2)[0] == want_acc


# ------------------------------------------------- MXFP8-stored replicas --

def test_mx_reduce_decodes_every_code_under_every_scale(zs):
    """P = 1, inv_scale = 1: the reduce output is the decoded MXFP8 value of
    all 256 codes under each of the 256 scale bytes (65536 pairs)."""
    import torch
    codes = np.tile(np.arange(256, dtype=np.uint8), 256)
    scales = np.repeat(np.arange(256, dtype=np.uint8), 8)       # 8 blocks of 32 per byte
    want = O.mxfp8_decode(codes, scales)
    # NaN: every code under scale 0xFF, and codes 0x7F / 0xFF under the others
    assert int(np.isnan(want).sum()) == 256 + 255 * 2
    g = torch.empty(codes.size, dtype=torch.float32, device="cuda")
    acc = zs.new_norm_acc(1)
    zs.zero_shard_reduce_mx([to_dev(codes)], [to_dev(scales)], 1.0, g_out=g, acc=acc)
    torch.cuda.synchronize()
    got = from_dev(g)
    bad = np.nonzero(got.view(np.uint32) != want.view(np.uint32))[0]
    assert bad.size == 0, [(int(codes[i]), int(scales[i // 32]), hex(got.view(np.uint32)[i]),
                            hex(want.view(np.uint32)[i])) for i in bad[:6]]
    assert zs.read_norm_acc(acc)[0] == acc_from_oracle(O.norm_accumulate(want))


@pytest.mark.parametrize("P", [1, 3, 4, 8, 64])
def test_mx_reduce_and_norm(zs, P):
    """Replicas packed to MXFP8 by the oracle (with inf/NaN blocks, all-zero
    blocks and tiny blocks) against decode-then-reduce in the oracle."""
    import torch
    for n in (32, 64, 32 * 33, 32 * 4099, 32 * 65537):
        reps = _replicas(P, n, True, seed=n + P)
        if n >= 1024:
            reps[0][3] = 0x7FC0                  # NaN: its block's scale is NaN
            reps[P - 1][n - 1] = 0x7F80          # +inf
            reps[P // 2][64:96] = 0              # an all-zero block
            reps[0][96:128] = O.f32_to_bf16(np.full(32, 1e-30, np.float32))
        packed = [O.mxfp8_pack(r) for r in reps]
        inv = O.inv_scale(P, 1.0)
        want_g = O.reduce([O.mxfp8_decode(e, s) for e, s in packed], inv)
        want_acc = acc_from_oracle(O.norm_accumulate(want_g))
        codes = [to_dev(e) for e, _ in packed]
        scales = [to_dev(s) for _, s in packed]
        g = torch.empty(n, dtype=torch.float32, device="cuda")
        acc = zs.new_norm_acc(1)
        zs.zero_shard_reduce_mx(codes, scales, inv, g_out=g, acc=acc)
        acc2 = zs.new_norm_acc(1)
        zs.zero_shard_reduce_mx(codes, scales, inv, acc=acc2)
        ws = zs.new_reduce_workspace()
        g3 = torch.empty(n, dtype=torch.float32, device="cuda")
        acc3 = zs.new_norm_acc(1)
        zs.zero_shard_reduce_mx_ws(codes, scales, inv, ws, g_out=g3, acc=acc3)
        torch.cuda.synchronize()
        got = from_dev(g)
        assert same_bits(got, want_g), mismatch_report(f"g n={n}", got, want_g)
        assert same_bits(from_dev(g3), want_g), n
        assert zs.read_norm_acc(acc)[0] == want_acc, n
        assert zs.read_norm_acc(acc2)[0] == want_acc, n
        assert zs.read_norm_acc(acc3)[0] == want_acc, n
        assert int(ws.abs().sum().item()) == 0, n


def test_mx_reduce_rejects_bad_sizes(zs):
    import torch
    c = torch.zeros(64, dtype=torch.uint8, device="cuda")
    s = torch.zeros(2, dtype=torch.uint8, device="cuda")
    g = torch.empty(64, dtype=torch.float32, device="cuda")
    with pytest.raises(zs.ZeroStepError):
        zs.zero_shard_reduce_mx([c[:48]], [s], 1.0, g_out=g[:48])      # n % 32 != 0
    with pytest.raises((ValueError, zs.ZeroStepError)):
        zs.zero_shard_reduce_mx([c], [s[:1]], 1.0, g_out=g)            # too few scales
    with pytest.raises((ValueError, zs.ZeroStepError)):
        zs.zero_shard_reduce_mx([c], [s], 1.0, g_out=g[:32])           # short g_out


@pytest.mark.parametrize("oneshot_min", [None, 0])
def test_shard_step_with_mxfp8_gradients(zs, oneshot_min):
    """ShardStep over MXFP8-stored replicas, gated (clip + overflow check),
    with one overflowing call: the oracle step on the decoded replicas.
    oneshot_min=0 runs every bucket's reduce in the one-shot form."""
    import torch
    n, P = 32 * 40_009, 8
    lr, b1, b2, eps, wd, max_norm = 1e-3, 0.9, 0.999, 1e-8, 0.01, 0.05
    master = synth.fill(synth.make_spec(seed=5, cfg=56, stream=0, sigma=0.02), 0, n, False)
    m, v = np.zeros(n, np.float32), np.zeros(n, np.float32)
    param = O.f32_to_bf16(master)
    st = zs.ShardStep(n, P, "mxfp8", lr=lr, beta1=b1, beta2=b2, eps=eps, weight_decay=wd,
                      max_norm=max_norm, check_overflow=True, bucket=32 * 10_000,
                      oneshot_min=oneshot_min)
    assert st.path == "materialize"
    st.master.copy_(to_dev(master))
    st.param.copy_(to_dev(param))
    t = 0
    for call in range(1, 5):
        reps = _replicas(P, n, True, seed=31 * call)
        if call == 2:
            reps[5][n // 2] = 0xFF80             # -inf: this call is skipped
        packed = [O.mxfp8_pack(r) for r in reps]
        skipped, _ = O.step([O.mxfp8_decode(e, s) for e, s in packed], O.inv_scale(P, 1.0),
                            max_norm, True, lr, b1, b2, eps, wd, t + 1, master, m, v, param)
        t += 0 if skipped else 1
        st.step([(to_dev(e), to_dev(s)) for e, s in packed])
    assert st.applied_steps() == t == 3
    torch.cuda.synchronize()
    for name, got, want in (("master", st.master, master), ("m", st.m, m), ("v", st.v, v),
                            ("param", st.param, param)):
        hg = from_dev(got, name == "param")
        assert same_bits(hg, want), mismatch_report(name, hg, want)


# ------------------------------------------------------------------ gate --

ACC_DIGITS = 13


def _acc_words(X, nonfinite, rng):
    """Device layout of an accumulator holding X (13 digits with pending
    carries, the non-finite count, two reserved zero words)."""
    d = [(X >> (32 * k)) & 0xFFFFFFFF for k in range(ACC_DIGITS)]
    d[-1] += (X >> (32 * ACC_DIGITS)) << 32
    for k in range(ACC_DIGITS - 1, 0, -1):   # push some value down as pending carries
        c = int(rng.integers(0, min(d[k], 1 << 31) + 1)) if d[k] else 0
        d[k] -= c
        d[k - 1] += c << 32
    assert all(0 <= v < (1 << 64) for v in d)
    words = [v - (1 << 64) if v >= (1 << 63) else v for v in d]
    return words + [nonfinite, 0, 0]


def test_gate_matches_oracle(zs):
    """The device gate (the AdamW prologue's) against the oracle's over
    accumulator values up to the 13 digits' range (including RNE ties and
    pending carries), several thresholds, and the skip / clip-to-zero rules."""
    import torch
    rng = np.random.default_rng(21)
    top = 1 << (32 * ACC_DIGITS + 20)
    Xs = [0, 1, 3, (1 << 53) - 1, 1 << 53, (1 << 53) + 1, (1 << 54) + 2, (1 << 54) + 6,
          25 << 128, (1 << 224) - 1, 1 << 224, (1 << 389) - 1, 281474943156225 << 341]
    for bits in range(1, 32 * ACC_DIGITS + 18, 3):
        Xs.append(int(rng.integers(1, 1 << 62)) << max(0, bits - 62))
    for m in ((1 << 52) + 1, (1 << 53) - 1):
        for sh in (1, 60, 150, 300):
            Xs += [(2 * m + 1) << sh, ((2 * m + 1) << sh) + 1, ((2 * m + 1) << sh) - 1]
    coef = torch.empty(1, dtype=torch.float32, device="cuda")
    skip = torch.empty(1, dtype=torch.int32, device="cuda")
    rows, expect = [], []
    for X in Xs:
        X %= top
        for max_norm in (1.0, 0.37, 1e6, 1e200, 0.0):
            for nonfinite, check in ((0, 1), (2, 1), (3, 0), (0, 0)):
                parts = [X // 3, X // 3, X - 2 * (X // 3)]
                words = []
                oacc = O.acc_zero()
                for j, part in enumerate(parts):
                    nf = nonfinite if j == 0 else 0
                    words.append(_acc_words(part, nf, rng))
                    a = O.acc_zero()
                    for k in range(O.ACC_WORDS):
                        a.w[k] = (part >> (32 * k)) & 0xFFFFFFFF
                    a.nonfinite = nf
                    O.acc_add(oacc, a)
                want_skip, want_coef = O.gate(oacc, max_norm, check)
                rows.append((words, max_norm, check))
                expect.append((want_coef, int(want_skip), X))
    got = []
    for words, max_norm, check in rows:
        accs = torch.tensor(words, dtype=torch.int64, device="cuda")
        zs.zero_step_gate(accs, max_norm, check, coef, skip)
        got.append((coef.clone(), skip.clone()))
    torch.cuda.synchronize()
    for (c, s), (wc, ws, X) in zip(got, expect):
        assert int(s.item()) == ws, hex(X)
        if not ws:
            assert np.float32(c.item()).view(np.uint32) == np.float32(wc).view(np.uint32), \
                (hex(X), c.item(), wc)


# ----------------------------------------------------------------- AdamW --

HP = [(1e-3, 0.9, 0.999, 1e-8, 0.01), (0.1, 0.5, 0.75, 1e-3, 0.5)]


@pytest.mark.parametrize("source", ["grad_f32", "f32_P4", "bf16_P8", "bf16_P1", "bf16_P3",
                                    "bf16_P16", "f32_P64"])
@pytest.mark.parametrize("gated", [False, True])
def test_adamw_multi_step(zs, source, gated):
    import torch
    for n in (16, 17, 31, 32, 33, 1024, 4096 + 5, 70001):
        for hp in HP:
            lr, b1, b2, eps, wd = hp
            if source == "grad_f32":
                P, bf16 = 1, False
            else:
                P, bf16 = int(source.split("_P")[1]), source.startswith("bf16")
            ms = synth.make_spec(seed=n, cfg=52, stream=0, sigma=0.02)
            master = synth.fill(ms, 0, n, False)
            m = np.zeros(n, np.float32)
            v = np.zeros(n, np.float32)
            param = O.f32_to_bf16(master)
            d = [to_dev(a) for a in (master, m, v, param)]
            acc = zs.new_norm_acc(1)
            skipped = torch.zeros(1, dtype=torch.int32, device="cuda")
            max_norm = 0.05 if gated else 0.0
            for t in range(1, 5):
                reps = _replicas(P, n, bf16, seed=1000 * t + n)
                inv = O.inv_scale(P, 1.0)
                g = O.reduce(reps, inv)
                coef = 1.0
                if gated:
                    skip, coef = O.gate(O.norm_accumulate(g), max_norm, True)
                    assert not skip
                O.adamw(g, coef, O.make_scalars(lr, b1, b2, eps, wd, t), master, m, v, param)
                dreps = [to_dev(r) for r in reps]
                kw = dict(step=t, lr=lr, beta1=b1, beta2=b2, eps=eps, weight_decay=wd,
                          param_bf16=d[3])
                if gated:
                    zs.zero_norm_acc_clear(acc)
                    zs.zero_shard_reduce(dreps, inv, acc=acc)
                    kw.update(accs=acc, max_norm=max_norm, check_overflow=True,
                              skipped_out=skipped)
                if source == "grad_f32":
                    zs.zero_adamw_step(d[0], d[1], d[2], grad_f32=to_dev(g), **kw)
                else:
                    zs.zero_adamw_step(d[0], d[1], d[2], replicas=dreps, inv_scale=inv, **kw)
            torch.cuda.synchronize()
            for name, got, want in zip(("master", "m", "v", "param"), d, (master, m, v, param)):
                hg = from_dev(got, name == "param")
                assert same_bits(hg, want), mismatch_report(f"{name} n={n} hp={hp}", hg, want)
            if gated:
                assert int(skipped.item()) == 0


# IEEE corner values of the update: zeros of both signs, subnormals, the
# edges of the normal range, values whose squares underflow or overflow,
# infinities and NaN, in gradients and in the state.
_CORNER_G = [0.0, -0.0, 1e-45, -1e-45, 1e-40, -3e-39, 1.1754942e-38, 1.17549435e-38, 1e-30,
             -1e-20, 1e-3, -0.5, 1.0, 1e19, -3e19, 1e30, 3.4028235e38, -3.4028235e38,
             np.inf, -np.inf, np.nan]
_CORNER_MASTER = [0.0, -0.0, 1e-45, -1e-40, 1.17549435e-38, 0.02, -1.5, 1e30, 3.4028235e38,
                  -np.inf]
_CORNER_M = [0.0, -0.0, 1e-45, -1e-40, 1e-30, 1e-3, -0.2, 1e30, 3.4028235e38]
_CORNER_V = [0.0, 1e-45, 1e-40, 1.17549435e-38, 1e-20, 1e-6, 1.0, 1e30, 3.4028235e38]
# (lr, beta1, beta2, eps, weight_decay): the usual set, beta1 = 0 with eps = 0
# (0/0 where v is zero), beta2 = 0 with full decay (lr * wd = 1)
_CORNER_HP = [(1e-3, 0.9, 0.999, 1e-8, 0.01), (0.1, 0.0, 0.5, 0.0, 0.0),
              (1.0, 0.999, 0.0, 1e-30, 1.0)]


def _same_or_nan(got, want, bf16=False):
    """Bit for bit, except that where the oracle holds a NaN the device must
    hold a NaN of any sign and payload: IEEE 754 leaves both open for the
    result of an invalid operation (inf * 0, inf - inf, 0 / 0), and x86
    returns the negative default NaN where the GPU returns the positive one."""
    if bf16:
        gb, wb = got.view(np.uint16), want.view(np.uint16)
        gn, wn = (gb & 0x7FFF) > 0x7F80, (wb & 0x7FFF) > 0x7F80
    else:
        gb, wb = got.view(np.uint32), want.view(np.uint32)
        gn, wn = np.isnan(got), np.isnan(want)
    return got.shape == want.shape and np.array_equal(gn, wn) and np.array_equal(gb[~wn], wb[~wn])


@pytest.mark.parametrize("source", ["grad_f32", "bf16_P3"])
@pytest.mark.parametrize("gate", ["none", "clip_finite", "clip_nonfinite"])
def test_adamw_ieee_corner_values(zs, source, gate):
    """Three steps on corner-valued gradients and state, against the oracle:
    subnormal inputs and products (no flush to zero), g^2 overflowing into an
    infinite v, 0/0 with eps = 0, a clip coefficient that rounds to a
    subnormal (huge finite gradients), coef = 0 on non-finite gradients
    (inf * 0 = NaN).  The bf16 source also reduces corner-valued replicas,
    its fp32 g and norm state compared where the step materialises them."""
    import torch
    n = 4 * 2048 + 37
    rng = np.random.default_rng(7)
    gvals = np.array([x for x in _CORNER_G if gate != "clip_finite" or np.isfinite(x)],
                     np.float32)
    P, bf16 = (1, False) if source == "grad_f32" else (3, True)
    if bf16 and gate == "clip_finite":
        # the largest binary32 rounds to inf in bf16, and a sum of three
        # bf16 maxima overflows binary32
        gvals = gvals[np.abs(gvals) < 1e37]
    reached_subnormal = reached_nan = False
    for hp in _CORNER_HP:
        master = rng.choice(np.array(_CORNER_MASTER, np.float32), n)
        m = rng.choice(np.array(_CORNER_M, np.float32), n)
        v = rng.choice(np.array(_CORNER_V, np.float32), n)
        param = O.f32_to_bf16(master)
        d = [to_dev(a) for a in (master, m, v, param)]
        acc = zs.new_norm_acc(1)
        g_dev = torch.empty(n, dtype=torch.float32, device="cuda")
        max_norm = 0.0 if gate == "none" else 1.0
        for t in range(1, 4):
            reps = [rng.choice(gvals, n) for _ in range(P)]
            if gate == "clip_nonfinite":
                reps[0][rng.integers(0, n)] = np.inf
            if bf16:
                reps = [O.f32_to_bf16(r) for r in reps]
            inv = O.inv_scale(P, 1.0)
            g = O.reduce(reps, inv)
            want_acc = O.norm_accumulate(g)
            skip, coef = O.gate(want_acc, max_norm, False)
            assert not skip
            if gate == "clip_finite":
                assert 0.0 < coef < 1.0
            if gate == "clip_nonfinite":
                assert coef == 0.0
            O.adamw(g, coef, O.make_scalars(*hp, t), master, m, v, param)
            dreps = [to_dev(r) for r in reps]
            kw = dict(step=t, lr=hp[0], beta1=hp[1], beta2=hp[2], eps=hp[3], weight_decay=hp[4],
                      param_bf16=d[3])
            if gate != "none":
                zs.zero_norm_acc_clear(acc)
                zs.zero_shard_reduce(dreps, inv, g_out=g_dev, acc=acc)
                kw.update(accs=acc, max_norm=max_norm, check_overflow=False)
                zs.zero_adamw_step(d[0], d[1], d[2], grad_f32=g_dev, **kw)
                torch.cuda.synchronize()
                assert _same_or_nan(from_dev(g_dev), g), f"g, step {t}, hp {hp}"
                assert zs.read_norm_acc(acc)[0] == (want_acc.X, int(want_acc.nonfinite)), t
            elif source == "grad_f32":
                zs.zero_adamw_step(d[0], d[1], d[2], grad_f32=to_dev(g), **kw)
            else:
                zs.zero_adamw_step(d[0], d[1], d[2], replicas=dreps, inv_scale=inv, **kw)
            torch.cuda.synchronize()
            for name, got, want in zip(("master", "m", "v", "param"), d, (master, m, v, param)):
                hg = from_dev(got, name == "param")
                assert _same_or_nan(hg, want, name == "param"), \
                    mismatch_report(f"{name} step {t} hp {hp}", hg, want)
            sub = [a[(a != 0) & (np.abs(a) < 1.17549435e-38)] for a in (master, m, v)]
            reached_subnormal |= any(x.size for x in sub)
            reached_nan |= bool(np.isnan(master).any())
    # the corners were reached: subnormal state, and NaN where g holds a non-finite
    assert reached_subnormal
    assert reached_nan or gate == "clip_finite"


def test_adamw_fused_mxfp8_epilogue(zs):
    import torch
    for n, P, bf16 in ((32, 1, True), (4096 + 32, 8, True), (32 * 30011, 4, False)):
        ms = synth.make_spec(seed=n, cfg=54, stream=0, sigma=0.02)
        master = synth.fill(ms, 0, n, False)
        master[5] = np.float32(3.0e38)            # a huge value (block saturates/overflows)
        if n > 64:
            master[40:72] = 0.0                   # an all-zero block before the update
        m, v = np.zeros(n, np.float32), np.zeros(n, np.float32)
        param = O.f32_to_bf16(master)
        d = [to_dev(a) for a in (master, m, v, param)]
        elem = torch.empty(n, dtype=torch.uint8, device="cuda")
        scale = torch.empty(n // 32, dtype=torch.uint8, device="cuda")
        for t in (1, 2, 3):
            reps = _replicas(P, n, bf16, seed=77 * t + n)
            inv = O.inv_scale(P, 1.0)
            O.adamw(O.reduce(reps, inv), 1.0, O.make_scalars(1e-3, 0.9, 0.999, 1e-8, 0.01, t),
                    master, m, v, param)
            zs.zero_adamw_step(d[0], d[1], d[2], replicas=[to_dev(r) for r in reps],
                               inv_scale=inv, step=t, lr=1e-3, weight_decay=0.01,
                               param_bf16=d[3], mx_elem_out=elem, mx_scale_out=scale)
        torch.cuda.synchronize()
        want_e, want_s = O.mxfp8_pack(param)
        assert same_bits(from_dev(d[3], True), param)
        assert np.array_equal(from_dev(scale), want_s), n
        assert np.array_equal(from_dev(elem), want_e), n


def test_binding_rejects_short_buffers(zs):
    """The C ABI takes raw pointers; the binding refuses any buffer shorter
    than the elements a call would touch (no launch happens)."""
    import torch
    n = 4096
    f = lambda k: torch.zeros(k, dtype=torch.float32, device="cuda")
    h = lambda k: torch.zeros(k, dtype=torch.int16, device="cuda")
    u8 = lambda k: torch.zeros(k, dtype=torch.uint8, device="cuda")
    kw = dict(step=1, lr=1e-3)
    for bad in (dict(param_bf16=h(n - 1)), dict(mx_elem_out=u8(n - 1), mx_scale_out=u8(n // 32)),
                dict(mx_elem_out=u8(n), mx_scale_out=u8(n // 32 - 1))):
        with pytest.raises(ValueError):
            zs.zero_adamw_step(f(n), f(n), f(n), grad_f32=f(n), **kw, **bad)
    with pytest.raises(ValueError):
        zs.zero_adamw_step(f(n), f(n), f(n), grad_f32=f(n - 8), **kw)
    with pytest.raises(ValueError):
        zs.zero_adamw_step(f(n), f(n), f(n), replicas=[h(n), h(n - 1)], **kw)
    with pytest.raises(ValueError):
        zs.zero_adamw_step(f(n), f(n), f(n), grad_f32=f(n), n=n + 1, **kw)
    with pytest.raises(ValueError):
        zs.zero_shard_reduce([h(n), h(n)], 0.5, g_out=f(n - 1))
    with pytest.raises(ValueError):
        zs.zero_grad_norm(h(n), 1.0, zs.new_norm_acc(1), n=n + 32)
    with pytest.raises(ValueError):
        zs.zero_mxfp8_pack(h(n), u8(n), u8(n // 32 - 1))


def test_adamw_skip_leaves_state_untouched(zs):
    import torch
    n, P = 4096 + 3, 4
    reps = _replicas(P, n, True, seed=5, inject=[(2, n - 1, np.inf)])
    ms = synth.make_spec(seed=5, cfg=53, stream=0, sigma=0.02)
    master = synth.fill(ms, 0, n, False)
    m = (master * np.float32(0.01)).astype(np.float32)
    v = (master * master).astype(np.float32)
    param = O.f32_to_bf16(master)
    d = [to_dev(a) for a in (master, m, v, param)]
    acc = zs.new_norm_acc(1)
    skipped = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    dreps = [to_dev(r) for r in reps]
    inv = O.inv_scale(P, 1.0)
    zs.zero_shard_reduce(dreps, inv, acc=acc)
    zs.zero_adamw_step(d[0], d[1], d[2], replicas=dreps, inv_scale=inv, step=3, lr=1e-3,
                       weight_decay=0.01, param_bf16=d[3], accs=acc, max_norm=1.0,
                       check_overflow=True, skipped_out=skipped)
    torch.cuda.synchronize()
    assert int(skipped.item()) == 1
    assert zs.read_norm_acc(acc)[0][1] == 1
    for got, want in zip(d, (master, m, v, param)):
        assert same_bits(from_dev(got, want.dtype == np.uint16), want)


@pytest.mark.timeout(600)
def test_gated_step_past_2_32_elements(zs):
    """64-bit indexing and one norm call over more than 2^32 elements: a
    gated step (clip 1.0 and the overflow check) of one bf16 replica on
    n > 2^32 elements (about 73 GB of state), with the MXFP8 pack fused.  One
    gradient of 2^34 (a group norm of about 1.7e10, a group sum of squares
    past 2^64) dominates the norm, so the clip coefficient depends on it.  The
    oracle computes the global norm over all n elements on the host, then
    follows sampled blocks around the 2^31 and 2^32 element boundaries, the
    large gradient and the ragged end."""
    import torch
    from synth.configs import Workload
    from gpu_util import oracle_norm_parallel
    n = (1 << 32) + 4096 + 32 * 3
    big_at, big = (1 << 32) + 37, 0x5080                 # bf16 bits of 2^34
    w = Workload("past-2^32", "one bf16 replica past 2^32 elements", N=n, P=1, S=n,
                 grad_bf16=True, grad_sigma=1e-3, steps=1, max_norm=1.0, check_overflow=True,
                 pack=True, cfg_id=55, seed=1)
    st = zs.ShardStep(n, 1, torch.bfloat16, lr=w.lr, weight_decay=w.wd, max_norm=w.max_norm,
                      check_overflow=True, pack=True)
    assert st.path == "recompute"
    rep = torch.empty(n, dtype=torch.int16, device="cuda")
    synth.fill_device(w.grad_spec(1, 0), 0, rep)
    rep[big_at] = big
    synth.fill_device(w.master_spec(), 0, st.master)
    synth.fill_device(w.master_spec(), 0, st.param)
    st.step([rep])
    torch.cuda.synchronize()
    assert st.applied_steps() == 1
    print("gated step past 2^32: GPU done, oracle norm over", n, "elements", flush=True)
    # the oracle's global norm state: the group holding the large gradient
    # on its own, the rest split at that group's 32-aligned bounds
    g0 = big_at // 32 * 32
    acc = oracle_norm_parallel(w, 1, 0, g0)
    O.acc_add(acc, oracle_norm_parallel(w, 1, g0 + 32, n))
    grp = synth.fill(w.grad_spec(1, 0), g0, 32, True)
    grp[big_at - g0] = big
    O.acc_add(acc, O.norm_accumulate(O.reduce([grp], 1.0)))
    skip, coef = O.gate(acc, w.max_norm, True)
    assert not skip and 0 < coef < 1e-9
    assert zs.read_norm_acc(st.acc)[0] == (acc.X, int(acc.nonfinite))
    blocks = np.array([0, (1 << 26) - 1, 1 << 26, (1 << 27) - 1, 1 << 27, big_at // 32,
                       n // 32 - 1], dtype=np.int64)
    idx = (blocks[:, None] * 32 + np.arange(32)[None, :]).ravel()
    di = torch.from_numpy(idx).cuda()
    hg = synth.gather(w.grad_spec(1, 0), idx.astype(np.uint64), True)
    hg[idx == big_at] = big
    hmaster = synth.gather(w.master_spec(), idx.astype(np.uint64), False)
    hm, hv = np.zeros(idx.size, np.float32), np.zeros(idx.size, np.float32)
    hparam = np.zeros(idx.size, np.uint16)
    O.adamw(O.reduce([hg], 1.0), coef, O.make_scalars(w.lr, w.beta1, w.beta2, w.eps, w.wd, 1),
            hmaster, hm, hv, hparam)
    we, ws = O.mxfp8_pack(hparam)
    assert same_bits(from_dev(st.master[di]), hmaster)
    assert same_bits(from_dev(st.m[di]), hm) and same_bits(from_dev(st.v[di]), hv)
    assert same_bits(from_dev(st.param[di], True), hparam)
    assert np.array_equal(from_dev(st.mx_elem[di]), we)
    assert np.array_equal(from_dev(st.mx_scale[torch.from_numpy(blocks).cuda()]), ws)
    del st, rep
    torch.cuda.empty_cache()


def test_clip_only_counts_large_groups_and_zeroes_on_nonfinite(zs):
    """Clipping without the overflow check, four calls: ordinary gradients;
    one averaged gradient of about 1.25e10 (its group's sum of squares past 2^64 counts
    in full and sets the coefficient); one infinite gradient (the norm is
    infinite, the coefficient 0: every finite element steps with a zero
    gradient and the infinite one's state becomes NaN); ordinary again.
    Against the oracle bit for bit, except that a NaN result is compared as
    NaN: IEEE 754 leaves the sign and payload of a NaN made by inf * 0
    unspecified, and the two processors make different ones."""
    import torch
    n, P = 32 * 4099 + 5, 8
    lr, b1, b2, eps, wd, max_norm = 1e-3, 0.9, 0.999, 1e-8, 0.01, 1.0
    master = synth.fill(synth.make_spec(seed=8, cfg=57, stream=0, sigma=0.02), 0, n, False)
    m, v = np.zeros(n, np.float32), np.zeros(n, np.float32)
    param = O.f32_to_bf16(master)
    st = zs.ShardStep(n, P, torch.bfloat16, lr=lr, beta1=b1, beta2=b2, eps=eps,
                      weight_decay=wd, max_norm=max_norm, check_overflow=False)
    st.master.copy_(to_dev(master))
    st.param.copy_(to_dev(param))
    coefs = []
    for call in range(1, 5):
        inject = {2: [(3, 1000, 1.0e11)], 3: [(5, 77, -np.inf)]}.get(call, [])
        reps = _replicas(P, n, True, seed=41 * call, inject=inject)
        _, acc = O.step(reps, O.inv_scale(P, 1.0), max_norm, False, lr, b1, b2, eps, wd, call,
                        master, m, v, param)
        coefs.append(O.gate(acc, max_norm, False)[1])
        st.step([to_dev(r) for r in reps])
    assert coefs[2] == 0.0 and 0 < coefs[1] < 1e-9
    torch.cuda.synchronize()
    for name, want in (("master", master), ("m", m), ("v", v), ("param", param)):
        got = from_dev(getattr(st, name), name == "param")
        wf = O.bf16_to_f32(want) if name == "param" else want
        gf = O.bf16_to_f32(got) if name == "param" else got
        nan = np.isnan(wf)
        assert nan.sum() == 1 and nan[77]
        assert np.array_equal(np.isnan(gf), nan), name
        assert same_bits(got[~nan], want[~nan]), mismatch_report(name, got[~nan], want[~nan])


@pytest.mark.parametrize("P,bf16", [(1, True), (3, True), (4, False), (8, True)])
def test_unfused_chain_equals_fused_and_oracle(zs, P, bf16):
    """The single-operation chain gives bit for bit the fused result (and the
    oracle's), including the clip, a skipped call and the MXFP8 pack."""
    import torch
    for n, pack in ((4096 + 32 * 5, True), (33331, False)):
        kw = dict(lr=1e-3, weight_decay=0.01, max_norm=0.05, check_overflow=True, pack=pack)
        gdt = torch.bfloat16 if bf16 else torch.float32
        fused = zs.ShardStep(n, P, gdt, **kw)
        chain = zs.ShardStep(n, P, gdt, **kw)
        ms = synth.make_spec(seed=n, cfg=56, stream=0, sigma=0.02)
        master = synth.fill(ms, 0, n, False)
        m, v = np.zeros(n, np.float32), np.zeros(n, np.float32)
        param = O.f32_to_bf16(master)
        for st in (fused, chain):
            st.master.copy_(to_dev(master))
            st.param.copy_(to_dev(param))
        t = 0
        for call in (1, 2, 3):
            inject = [(P - 1, n // 2, np.inf)] if call == 2 else []
            reps = _replicas(P, n, bf16, seed=500 * call + n, inject=inject)
            dreps = [to_dev(r) for r in reps]
            fused.step(dreps)
            chain.step_unfused(dreps)
            skipped, _ = O.step(reps, O.inv_scale(P, 1.0), 0.05, True, 1e-3, 0.9, 0.999, 1e-8,
                                0.01, t + 1, master, m, v, param)
            t += 0 if skipped else 1
        torch.cuda.synchronize()
        assert fused.applied_steps() == chain.applied_steps() == t == 2
        for name, want in (("master", master), ("m", m), ("v", v), ("param", param)):
            gf = from_dev(getattr(fused, name), name == "param")
            gc = from_dev(getattr(chain, name), name == "param")
            assert same_bits(gc, want), mismatch_report(f"unfused {name} n={n}", gc, want)
            assert same_bits(gf, gc), name
        if pack:
            want_e, want_s = O.mxfp8_pack(param)
            for st in (fused, chain):
                assert np.array_equal(from_dev(st.mx_elem), want_e)
                assert np.array_equal(from_dev(st.mx_scale), want_s)


# ----------------------------------------------------------------- MXFP8 --

def test_mxfp8_all_patterns_and_blocks(zs):
    import torch
    rng = np.random.default_rng(31)
    allpat = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    parts = [allpat, rng.permutation(allpat)]
    finite = allpat[(allpat & 0x7F80) != 0x7F80]
    parts.append(rng.permutation(finite)[: (finite.size // 32) * 32])
    scaled = (rng.standard_normal(32 * 4096) * np.repeat(
        np.exp2(rng.integers(-140, 128, size=4096)), 32)).astype(np.float32)
    parts.append(O.f32_to_bf16(scaled))
    blk = np.zeros(32 * 6, np.uint16)
    blk[32 * 1 + 7] = 0x8000
    blk[32 * 2] = 0x0001
    blk[32 * 3:32 * 4] = 0x7F7F
    blk[32 * 4 + 31] = 0xFF80
    blk[32 * 5:32 * 6] = rng.integers(0, 1 << 16, 32)
    parts.append(blk)
    x = np.concatenate(parts)
    for n in (x.size, 32, 32 * 5, 32 * 67):
        xs = np.ascontiguousarray(x[:n])
        want_e, want_s = O.mxfp8_pack(xs)
        elem = torch.empty(n, dtype=torch.uint8, device="cuda")
        scale = torch.empty(n // 32, dtype=torch.uint8, device="cuda")
        zs.zero_mxfp8_pack(to_dev(xs), elem, scale)
        torch.cuda.synchronize()
        ge, gs = from_dev(elem), from_dev(scale)
        assert np.array_equal(gs, want_s), (n, np.nonzero(gs != want_s)[0][:5])
        assert np.array_equal(ge, want_e), (n, np.nonzero(ge != want_e)[0][:5])


def _reachable_blocks():
    """For every scale exponent e_s in [-127, 119]: blocks of one anchor
    element 2^(e_s + 8) (which sets e_s) and 31 of the bf16 values that can
    share a block with it (|x| < 2^(e_s + 9)), both signs, all of them."""
    mags = np.arange(0x7F80, dtype=np.int64)          # finite bf16 magnitudes
    out = []
    for e_s in range(-127, 120):
        E = e_s + 8
        anchor = (E + 127) << 7 if E >= -126 else 1 << (E + 133)
        if e_s == -127:
            anchor = (-119 + 127) << 7                   # any amax with E <= -119
        limit = (E + 128) << 7 if E + 128 <= 0xFF else 0x7F80
        cand = mags[mags < limit]
        xs = np.concatenate([cand, cand | 0x8000]).astype(np.uint16)
        pad = (-xs.size) % 31
        xs = np.concatenate([xs, np.zeros(pad, np.uint16)]).reshape(-1, 31)
        blk = np.empty((xs.shape[0], 32), np.uint16)
        blk[:, 0] = anchor
        blk[:, 1:] = xs
        out.append(blk.ravel())
    return np.concatenate(out)


def test_mxfp8_every_reachable_element_and_scale(zs):
    import torch
    x = _reachable_blocks()
    want_e, want_s = O.mxfp8_pack(x)
    n = x.size
    elem = torch.empty(n, dtype=torch.uint8, device="cuda")
    scale = torch.empty(n // 32, dtype=torch.uint8, device="cuda")
    zs.zero_mxfp8_pack(to_dev(x), elem, scale)
    torch.cuda.synchronize()
    ge, gs = from_dev(elem), from_dev(scale)
    assert np.array_equal(gs, want_s), np.nonzero(gs != want_s)[0][:5]
    bad = np.nonzero(ge != want_e)[0]
    assert bad.size == 0, [(hex(int(x[i])), int(want_s[i // 32]) - 127, hex(ge[i]), hex(want_e[i]))
                           for i in bad[:6]]


# ---------------------------------------------------------- determinism --

def test_runs_are_bitwise_reproducible(zs):
    import torch
    n, P = 32 * 100_003, 8
    dreps = [to_dev(r) for r in _replicas(P, n, True, seed=9)]
    outs = []
    for _ in range(2):
        st = zs.ShardStep(n, P, torch.bfloat16, lr=1e-3, weight_decay=0.01, max_norm=1.0,
                          check_overflow=True, bucket=32 * 10_000)
        st.master.fill_(0.01)
        st.step(dreps)
        st.step(dreps)
        torch.cuda.synchronize()
        outs.append([t.cpu().numpy().copy() for t in (st.master, st.m, st.v, st.param, st.acc)])
    for a, b in zip(*outs):
        assert same_bits(a, b)


# ------------------------------------------------------ zero-length calls --

def test_zero_length_calls_touch_nothing(zs):
    """n = 0 is a valid no-op for every entry point: status ok, no element of
    any output written.  AdamW still reports its gate decision through
    skipped_out (a rank whose shard slice is empty takes part in the step)."""
    import torch
    n = 64
    reps = [to_dev(r) for r in _replicas(2, n, True, seed=5, inject=[(1, 9, np.inf)])]
    g = torch.full((n,), 7.0, dtype=torch.float32, device="cuda")
    acc = zs.new_norm_acc(1)
    zs.zero_shard_reduce(reps, 0.5, g_out=g, acc=acc, n=0)
    zs.zero_grad_norm(reps[0], 0.5, acc, n=0)
    codes = [torch.zeros(n, dtype=torch.uint8, device="cuda") for _ in range(2)]
    scales = [torch.zeros(n // 32, dtype=torch.uint8, device="cuda") for _ in range(2)]
    zs.zero_shard_reduce_mx(codes, scales, 0.5, g_out=g, acc=acc, n=0)
    elem = torch.full((n,), 0xAB, dtype=torch.uint8, device="cuda")
    scale = torch.full((n // 32,), 0xCD, dtype=torch.uint8, device="cuda")
    zs.zero_mxfp8_pack(reps[0], elem, scale, n=0)
    torch.cuda.synchronize()
    assert torch.all(g == 7.0).item()
    assert zs.read_norm_acc(acc)[0] == (0, 0)
    assert torch.all(elem == 0xAB).item() and torch.all(scale == 0xCD).item()

    bad = zs.new_norm_acc(1)
    zs.zero_shard_reduce(reps, 0.5, acc=bad)            # one inf -> nonfinite 1
    master = torch.full((n,), 0.25, dtype=torch.float32, device="cuda")
    m = torch.full((n,), 0.5, dtype=torch.float32, device="cuda")
    v = torch.full((n,), 0.75, dtype=torch.float32, device="cuda")
    param = torch.full((n,), 0x1234, dtype=torch.int16, device="cuda")
    skipped = torch.full((1,), -5, dtype=torch.int32, device="cuda")
    for accs, check, want_skip in ((bad, True, 1), (acc, True, 0), (bad, False, 0)):
        skipped.fill_(-5)
        zs.zero_adamw_step(master, m, v, step=1, lr=1e-3, weight_decay=0.01, grad_f32=g,
                           param_bf16=param, accs=accs, max_norm=1.0, check_overflow=check,
                           skipped_out=skipped, mx_elem_out=elem, mx_scale_out=scale, n=0)
        zs.zero_adamw_step(master, m, v, step=1, lr=1e-3, replicas=reps, inv_scale=0.5,
                           param_bf16=param, n=0)
        torch.cuda.synchronize()
        assert int(skipped.item()) == want_skip, (check, want_skip)
    # the device step counter advances on a zero-length call unless skipped
    t_dev = torch.full((1,), 41, dtype=torch.int64, device="cuda")
    for accs, check, want_t in ((bad, True, 41), (acc, True, 42), (bad, False, 43), (None, False, 44)):
        zs.zero_adamw_step(master, m, v, lr=1e-3, weight_decay=0.01, grad_f32=g,
                           param_bf16=param, accs=accs, max_norm=1.0, check_overflow=check,
                           step_dev=t_dev, n=0)
        torch.cuda.synchronize()
        assert int(t_dev.item()) == want_t, (check, want_t)
    assert torch.all(master == 0.25).item() and torch.all(m == 0.5).item()
    assert torch.all(v == 0.75).item() and torch.all(param == 0x1234).item()
    assert torch.all(elem == 0xAB).item() and torch.all(scale == 0xCD).item()
    assert torch.all(g == 7.0).item()


# ------------------------------------------- device step counter, graphs --

_HP = dict(lr=3e-4, beta1=0.85, beta2=0.95, eps=1e-8, weight_decay=0.1, max_norm=1.0,
           check_overflow=True, pack=True)
_STATE = ("master", "m", "v", "param", "mx_elem", "mx_scale")


def _same_state(a, b):
    import torch
    return all(torch.equal(getattr(a, k).view(torch.uint8), getattr(b, k).view(torch.uint8))
               for k in _STATE)


def _fill_grads(reps, call, inject_call):
    for k, r in enumerate(reps):
        synth.fill_device(synth.make_spec(seed=4, cfg=60, stream=1, step=call, replica=k,
                                          sigma=1e-3, outlier_rate=0.01, outlier_mult=100.0),
                          0, r)
    if call == inject_call:
        reps[2][77] = 0x7F80                   # +inf in one replica: the step is skipped


def _init(*steps):
    mspec = synth.make_spec(seed=4, cfg=60, stream=0, sigma=0.02)
    for st in steps:
        synth.fill_device(mspec, 0, st.master)
        synth.fill_device(mspec, 0, st.param)
        st.mx_elem.zero_()
        st.mx_scale.zero_()


def test_device_counter_matches_host_counter(zs):
    """The device counter (scalars derived on the device from the counter,
    advanced on the device unless the gate skips) gives the bits of the
    host-counter step, through a skipped call and at a large step index."""
    import torch
    n, P = 65536 + 96, 8
    host = zs.ShardStep(n, P, torch.bfloat16, **_HP)
    dev = zs.ShardStep(n, P, torch.bfloat16, device_counter=True, **_HP)
    _init(host, dev)
    reps = [torch.empty(n, dtype=torch.int16, device="cuda") for _ in range(P)]
    for call in range(1, 13):
        _fill_grads(reps, call, inject_call=5)
        host.step(reps)
        dev.step(reps)
        torch.cuda.synchronize()
        assert _same_state(host, dev), call
    assert host.applied_steps() == dev.applied_steps() == 11
    host.t = 99_999
    dev.t_dev.fill_(99_999)
    _fill_grads(reps, 13, inject_call=0)
    host.step(reps)
    dev.step(reps)
    torch.cuda.synchronize()
    assert _same_state(host, dev)
    assert host.applied_steps() == dev.applied_steps() == 100_000


@pytest.mark.parametrize("case", ["buckets", "recompute", "fused", "oneshot", "oneshot_buckets"])
def test_graph_replay_matches_eager(zs, case):
    """One step recorded once and replayed: after every replay, with eager
    work and synchronisation between replays, the state is bitwise that of
    the same step run eagerly.  Cases: 8 bf16 replicas in 34 buckets with the
    gate and fused MXFP8 (materialised g, a skipped replay); one bf16 replica
    with a loss scale and the overflow check (recompute path, a skipped
    replay); 4 fp32 replicas, no gate (one fused pass); 8 bf16 replicas on
    the one-shot reduce, whose workspace each replay leaves zero; the same in
    34 one-shot buckets alternating over the two streams, each stream with
    its own workspace."""
    import torch
    n = 65536 + 96
    if case == "oneshot":
        # the one-shot reduce (workspace) at this size too
        P, dt, kw, skip_call = 8, torch.bfloat16, dict(_HP, oneshot_min=0), 5
    elif case == "oneshot_buckets":
        P, dt, kw, skip_call = 8, torch.bfloat16, dict(_HP, bucket=32 * 61, oneshot_min=0), 3
    elif case == "buckets":
        P, dt, kw, skip_call = 8, torch.bfloat16, dict(_HP, bucket=32 * 61), 4
    elif case == "recompute":
        P, dt, skip_call = 1, torch.bfloat16, 4
        kw = dict(lr=1e-3, weight_decay=0.01, check_overflow=True, loss_scale=65536.0, pack=True)
    else:
        P, dt, skip_call = 4, torch.float32, 0
        kw = dict(lr=1e-3, weight_decay=0.01, pack=True)
    eager = zs.ShardStep(n, P, dt, device_counter=True, **kw)
    graphed = zs.ShardStep(n, P, dt, device_counter=True, **kw)
    assert eager.path == {"buckets": "materialize", "recompute": "recompute",
                          "fused": "fused", "oneshot": "materialize",
                          "oneshot_buckets": "materialize"}[case]
    if case in ("buckets", "oneshot_buckets"):
        assert graphed._side is not None
    _init(eager, graphed)
    reps = [torch.empty(n, dtype=torch.int16 if dt == torch.bfloat16 else torch.float32,
                        device="cuda") for _ in range(P)]

    def fill(call):
        for k, r in enumerate(reps):
            synth.fill_device(synth.make_spec(seed=4, cfg=61, stream=1, step=call, replica=k,
                                              sigma=1e-3, post_mul=kw.get("loss_scale", 1.0)),
                              0, r)
        if call == skip_call:
            reps[P - 1][77] = 0x7F80 if dt == torch.bfloat16 else float("inf")

    fill(1)
    torch.cuda.synchronize()
    g = graphed.capture(reps)                  # records; runs nothing
    torch.cuda.synchronize()
    assert graphed.applied_steps() == 0 and _same_state(eager, graphed)
    for call in range(1, 8):
        fill(call)
        eager.step(reps)
        g.replay()
        torch.cuda.synchronize()
        assert _same_state(eager, graphed), call
        assert eager.applied_steps() == graphed.applied_steps()
        assert int(graphed.reduce_ws.abs().sum().item()) == 0, call
        if graphed._side_ws is not None:
            assert int(graphed._side_ws.abs().sum().item()) == 0, call
    assert graphed.applied_steps() == (6 if skip_call else 7)


def test_counter_moves_between_host_and_device(zs):
    """Steps with the count moved device -> host -> device in between (as the
    benchmark does around the unfused chain) equal host-counted steps, the
    unfused steps included."""
    import torch
    n, P = 4096 + 96, 8
    ref = zs.ShardStep(n, P, torch.bfloat16, **_HP)
    mix = zs.ShardStep(n, P, torch.bfloat16, device_counter=True, **_HP)
    _init(ref, mix)
    reps = [torch.empty(n, dtype=torch.int16, device="cuda") for _ in range(P)]
    for call in range(1, 9):
        _fill_grads(reps, call, inject_call=3)
        if call == 4:
            mix.set_counter(device=False)
        if call == 6:
            mix.set_counter(device=True)
        if 4 <= call < 6:
            ref.step_unfused(reps)
            mix.step_unfused(reps)
        else:
            ref.step(reps)
            mix.step(reps)
        torch.cuda.synchronize()
        assert _same_state(ref, mix), call
    assert ref.applied_steps() == mix.applied_steps() == 7

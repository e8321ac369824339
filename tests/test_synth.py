"""The synthetic input generator on the host: determinism, counter
addressing, distribution shape, and bf16 storage."""
import numpy as np

import oracle as O
import synth
from synth import configs


def test_deterministic_and_counter_addressed():
    sp = synth.make_spec(seed=0, cfg=2, stream=1, step=3, replica=5, sigma=1e-3,
                         outlier_rate=0.01, outlier_mult=100.0)
    a = synth.fill(sp, 1000, 5000, bf16=False)
    b = synth.fill(sp, 1000, 5000, bf16=False)
    assert np.array_equal(a, b)
    c = synth.fill(sp, 1500, 100, bf16=False)
    assert np.array_equal(a[500:600], c)
    idx = np.array([1000, 1001, 5999, 3333], dtype=np.uint64)
    assert np.array_equal(synth.gather(sp, idx, bf16=False), a[(idx - 1000).astype(np.int64)])
    big = synth.fill(sp, 0, 3 << 20, bf16=True, threads=4)
    assert np.array_equal(big[1000:6000], synth.fill(sp, 1000, 5000, bf16=True))


def test_distribution():
    n = 1 << 21
    plain = synth.fill(synth.make_spec(sigma=0.02, cfg=9), 0, n, bf16=False).astype(np.float64)
    assert abs(plain.mean()) < 5 * 0.02 / np.sqrt(n)
    assert abs(plain.std() / 0.02 - 1) < 0.005
    assert np.abs(plain).max() <= 131070 / 37837.2272 * 0.02 * (1 + 1e-6)
    out = synth.fill(synth.make_spec(sigma=1e-3, cfg=9, stream=1, outlier_rate=0.01,
                                     outlier_mult=100.0), 0, n, bf16=False).astype(np.float64)
    frac = np.mean(np.abs(out) > 0.0035)          # beyond the plain support
    assert 0.0085 < frac < 0.0105
    scaled = synth.fill(synth.make_spec(sigma=1e-3, cfg=9, stream=1, post_mul=65536.0),
                        0, 4096, bf16=False)
    base = synth.fill(synth.make_spec(sigma=1e-3, cfg=9, stream=1), 0, 4096, bf16=False)
    assert np.array_equal(scaled, base * np.float32(65536.0))


def test_streams_independent():
    n = 1 << 16
    w = configs.GPT2_SMALL
    a = synth.fill(w.grad_spec(1, 0), 0, n, bf16=False).astype(np.float64)
    b = synth.fill(w.grad_spec(1, 1), 0, n, bf16=False).astype(np.float64)
    c = synth.fill(w.grad_spec(2, 0), 0, n, bf16=False).astype(np.float64)
    for x, y in ((a, b), (a, c), (b, c)):
        assert abs(np.corrcoef(x, y)[0, 1]) < 0.02


def test_bf16_storage_is_round_to_nearest_even():
    sp = synth.make_spec(sigma=1e-3, cfg=9, stream=1, outlier_rate=0.01, outlier_mult=100.0)
    f = synth.fill(sp, 0, 1 << 18, bf16=False)
    h = synth.fill(sp, 0, 1 << 18, bf16=True)
    assert np.array_equal(h, O.f32_to_bf16(f))


def test_workload_table():
    for w in configs.ALL.values():
        assert w.S % 32 == 0 and w.N % w.S == 0 and w.N // w.S in (1, w.P)
        if w.bucket:
            assert w.S % w.bucket == 0 and w.bucket % 32 == 0
    assert configs.GPT2_SMALL.N == 8 * configs.GPT2_SMALL.S
    assert configs.SHARD_7B.S // configs.SHARD_7B.bucket == 35

"""Helpers of the GPU parity tests: device transfer of numpy arrays, the
oracle over whole workloads (inputs regenerated on the host from the
counter-based generator, chunk by chunk, across threads; the oracle does all
arithmetic), and full comparisons of device state with it."""
import os
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle as O
import synth

THREADS = max(1, min(16, os.cpu_count() or 1))


def gpu_or_skip():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def to_dev(a: np.ndarray):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).cuda()
    return torch.from_numpy(np.ascontiguousarray(a).copy()).cuda()


def from_dev(t, bf16=False) -> np.ndarray:
    a = t.detach().cpu().numpy()
    if bf16 or a.dtype == np.int16:
        return a.view(np.uint16)
    return a


def same_bits(a: np.ndarray, b: np.ndarray) -> bool:
    return a.shape == b.shape and np.array_equal(a.view(np.uint8), b.view(np.uint8))


def mismatch_report(name, got, want):
    """Max relative error and count of non-identical elements (for messages)."""
    g = got.astype(np.float64)
    w = want.astype(np.float64)
    diff = got.view(np.uint8).reshape(got.size, -1) != want.view(np.uint8).reshape(want.size, -1)
    nbad = int(np.count_nonzero(diff.any(axis=1)))
    with np.errstate(invalid="ignore", divide="ignore"):
        rel = np.where(w != 0, np.abs(g - w) / np.abs(w), np.where(g == 0, 0.0, np.inf))
    return f"{name}: {nbad} elements differ, max rel err {np.nanmax(rel):.3e}"


def acc_from_oracle(a) -> tuple:
    return (a.X, int(a.nonfinite))


def oracle_norm_range(workload, call, lo, hi, chunk=1 << 21):
    """Oracle norm state of elements [lo, hi) (global indices, 32-aligned lo)
    of the averaged gradient of one call of a workload."""
    acc = O.acc_zero()
    P = workload.P
    inv = O.inv_scale(P, workload.loss_scale)
    for s in range(lo, hi, chunk):
        e = min(hi, s + chunk)
        reps = [synth.fill(workload.grad_spec(call, k), s, e - s, workload.grad_bf16)
                for k in range(P)]
        if workload.inject and workload.inject[0] == call and s <= workload.inject[1] < e:
            reps[0][workload.inject[1] - s] = 0x7F80 if workload.grad_bf16 else np.float32(np.inf)
        if getattr(workload, "mx_grads", False):     # MXFP8-stored: pack, then decode
            reps = [O.mxfp8_decode(*O.mxfp8_pack(r)) for r in reps]
        O.norm_accumulate(O.reduce(reps, inv), acc)
    return acc


def oracle_norm_parallel(workload, call, lo, hi, threads=THREADS):
    """Same as oracle_norm_range, split over threads at 32-aligned cuts; the
    integer sums make the split invisible."""
    n = hi - lo
    per = max(32, ((n // threads) + 31) // 32 * 32)
    cuts = [(lo + i, min(hi, lo + i + per)) for i in range(0, n, per)]
    with ThreadPoolExecutor(threads) as ex:
        parts = list(ex.map(lambda c: oracle_norm_range(workload, call, *c), cuts))
    total = O.acc_zero()
    for p in parts:
        O.acc_add(total, p)
    return total


CAPTURE = None     # pytest's capture manager, set by conftest


def log(msg):
    """Progress line of a long parity test, written to the terminal at once
    even while pytest captures the test's output."""
    line = f"[parity {time.strftime('%H:%M:%S')}] {msg}"
    if CAPTURE is None:
        print(line, flush=True)
        return
    with CAPTURE.global_and_fixture_disabled():
        print(line, flush=True)


def _chunks(n, chunk):
    return [(a, min(n, a + chunk)) for a in range(0, n, chunk)]


class OracleRun:
    """The oracle following a workload's whole step schedule on elements
    [lo, lo + n) of the flat vector (one rank's shard, or the whole vector of
    all ranks), with the whole state in host memory: master, m, v, param and
    one call's averaged gradient.  Each call regenerates that call's gradient
    replicas chunk by chunk (never all of them at once), reduces them into
    the gradient and adds the chunk's norm state (32-aligned chunks, integer
    sums: the split changes nothing); then the gate of the global state, then
    AdamW chunk by chunk.  Every arithmetic step is an oracle call; threads
    only spread the chunks."""

    def __init__(self, w, lo, n, threads=THREADS, chunk=1 << 22):
        assert lo % 32 == 0 and chunk % 32 == 0
        self.w, self.lo, self.n, self.threads = w, lo, n, threads
        self.cuts = _chunks(n, chunk)
        self.ex = ThreadPoolExecutor(threads)
        self.master = synth.fill(w.master_spec(), lo, n, False, threads=threads)
        self.m = np.zeros(n, np.float32)
        self.v = np.zeros(n, np.float32)
        self.param = np.empty(n, np.uint16)
        self.g = np.empty(n, np.float32)
        self.inv = O.inv_scale(w.P, w.loss_scale)
        self.t = 0
        self.gates = []                      # (call, skip, coef, acc) per call

        def init(c):
            a, b = c
            self.param[a:b] = O.f32_to_bf16(self.master[a:b])
        list(self.ex.map(init, self.cuts))

    def _grad_chunk(self, call, c):
        w = self.w
        a, b = c
        s = self.lo + a
        reps = [synth.fill(w.grad_spec(call, k), s, b - a, w.grad_bf16) for k in range(w.P)]
        if w.inject and w.inject[0] == call and s <= w.inject[1] < s + (b - a):
            reps[0][w.inject[1] - s] = 0x7F80 if w.grad_bf16 else np.float32(np.inf)
        if w.mx_grads:                       # MXFP8-stored replicas: pack, then decode
            reps = [O.mxfp8_decode(*O.mxfp8_pack(r)) for r in reps]
        O.reduce(reps, self.inv, out=self.g[a:b])
        return O.norm_accumulate(self.g[a:b])

    def call(self, call, extra_accs=()):
        """One call of the schedule; `extra_accs`: norm states of elements
        outside [lo, lo + n) that belong to the same global norm."""
        w = self.w
        acc = O.acc_zero()
        for part in self.ex.map(lambda c: self._grad_chunk(call, c), self.cuts):
            O.acc_add(acc, part)
        glob = acc.copy()
        for e in extra_accs:
            O.acc_add(glob, e)
        skip, coef = O.gate(glob, w.max_norm, w.check_overflow)
        self.gates.append((call, skip, coef, acc))
        if skip:
            return skip, coef, acc
        self.t += 1
        s = O.make_scalars(w.lr, w.beta1, w.beta2, w.eps, w.wd, self.t)

        def upd(c):
            a, b = c
            O.adamw(self.g[a:b], coef, s, self.master[a:b], self.m[a:b], self.v[a:b],
                    self.param[a:b])
        list(self.ex.map(upd, self.cuts))
        return skip, coef, acc

    def mxfp8(self):
        """The oracle's MXFP8 pack of the current param, chunk by chunk."""
        elem = np.empty(self.n, np.uint8)
        scale = np.empty(self.n // 32, np.uint8)

        def pack(c):
            a, b = c
            elem[a:b], scale[a // 32:b // 32] = O.mxfp8_pack(self.param[a:b])
        list(self.ex.map(pack, self.cuts))
        return elem, scale

    def close(self):
        self.ex.shutdown()


def compare_full(name, dev, host, lo=0, chunk=1 << 26, bf16=False, threads=THREADS):
    """Every element of a device tensor against a host array, copied back in
    chunks: returns (count of non-identical elements, max relative error,
    first differing index or None).  A reference of 0 needs an exact 0."""
    n = host.size
    cuts = _chunks(n, chunk)

    def part(c):
        a, b = c
        got = from_dev(dev[lo + a:lo + b], bf16)
        want = host[a:b]
        diff = got.view(np.uint8).reshape(b - a, -1) != want.view(np.uint8).reshape(b - a, -1)
        bad = np.nonzero(diff.any(axis=1))[0]
        if bad.size == 0:
            return 0, 0.0, None
        gv = got[bad].astype(np.float64) if not bf16 else O.bf16_to_f32(got[bad]).astype(np.float64)
        wv = want[bad].astype(np.float64) if not bf16 else O.bf16_to_f32(want[bad]).astype(np.float64)
        with np.errstate(invalid="ignore", divide="ignore"):
            rel = np.where(wv != 0, np.abs(gv - wv) / np.abs(wv), np.inf)
        return int(bad.size), float(np.nanmax(rel)), a + int(bad[0])

    with ThreadPoolExecutor(min(threads, 8)) as ex:
        res = list(ex.map(part, cuts))
    nbad = sum(r[0] for r in res)
    worst = max(r[1] for r in res)
    first = next((r[2] for r in res if r[2] is not None), None)
    log(f"{name}: {n} elements, {nbad} non-identical, max rel err {worst:.3e}")
    return nbad, worst, first

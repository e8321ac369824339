"""Helpers of the GPU parity tests: device transfer of numpy arrays and the
streaming oracle (inputs regenerated on the host from the counter-based
generator, chunk by chunk, across threads; the oracle does all arithmetic)."""
import os
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

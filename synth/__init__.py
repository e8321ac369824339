"""Seeded, counter-based synthetic inputs (recipe in synth_core.h).

Holds none of the optimizer's arithmetic: it only produces gradient replicas
and initial master weights, on the host (numpy) or in device memory (torch
tensors), bit-identically on both.
"""
import ctypes as C
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import build as _build

_cpu = None
_dev = None


class Spec(C.Structure):
    _fields_ = [("seed", C.c_uint64), ("cfg", C.c_uint32), ("stream", C.c_uint32),
                ("step", C.c_uint32), ("replica", C.c_uint32), ("sigma", C.c_double),
                ("outlier_mult", C.c_float), ("outlier_threshold", C.c_uint32),
                ("post_mul", C.c_float), ("pad_", C.c_uint32)]


def make_spec(seed=0, cfg=0, stream=0, step=0, replica=0, sigma=1.0,
              outlier_rate=0.0, outlier_mult=1.0, post_mul=1.0) -> Spec:
    thr = int(outlier_rate * 4294967296.0) if outlier_rate > 0 else 0
    return Spec(seed, cfg, stream, step, replica, sigma, outlier_mult, thr, post_mul, 0)


def cpu():
    global _cpu
    if _cpu is None:
        if not os.path.exists(_build.LIB_CPU):
            _build.build_cpu()
        L = C.CDLL(_build.LIB_CPU)
        for name, t in (("synth_fill_f32", C.c_void_p), ("synth_fill_bf16", C.c_void_p)):
            getattr(L, name).argtypes = [C.POINTER(Spec), C.c_uint64, C.c_size_t, t]
        for name in ("synth_gather_f32", "synth_gather_bf16"):
            getattr(L, name).argtypes = [C.POINTER(Spec), C.c_void_p, C.c_size_t, C.c_void_p]
        _cpu = L
    return _cpu


def dev():
    global _dev
    if _dev is None:
        if not os.path.exists(_build.LIB_DEV):
            raise RuntimeError("libsynth_dev.so is not built (run __graft_entry__.build())")
        L = C.CDLL(_build.LIB_DEV)
        for name in ("synth_dev_fill_f32", "synth_dev_fill_bf16"):
            f = getattr(L, name)
            f.argtypes = [C.POINTER(Spec), C.c_uint64, C.c_uint64, C.c_void_p, C.c_void_p]
            f.restype = C.c_int
        _dev = L
    return _dev


def fill(spec: Spec, start: int, count: int, bf16: bool, threads: int = 1) -> np.ndarray:
    """Host copy of elements [start, start+count) of a stream."""
    out = np.empty(count, dtype=np.uint16 if bf16 else np.float32)
    f = cpu().synth_fill_bf16 if bf16 else cpu().synth_fill_f32
    if threads <= 1 or count < (1 << 20):
        f(C.byref(spec), start, count, C.c_void_p(out.ctypes.data))
        return out
    step = -(-count // threads)
    item = out.itemsize

    def work(j):
        lo = j * step
        hi = min(count, lo + step)
        if hi > lo:
            f(C.byref(spec), start + lo, hi - lo, C.c_void_p(out.ctypes.data + lo * item))

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(work, range(threads)))
    return out


def gather(spec: Spec, idx: np.ndarray, bf16: bool) -> np.ndarray:
    idx = np.ascontiguousarray(idx, dtype=np.uint64)
    out = np.empty(idx.size, dtype=np.uint16 if bf16 else np.float32)
    f = cpu().synth_gather_bf16 if bf16 else cpu().synth_gather_f32
    f(C.byref(spec), C.c_void_p(idx.ctypes.data), idx.size, C.c_void_p(out.ctypes.data))
    return out


def fill_device(spec: Spec, start: int, tensor) -> None:
    """Fill a contiguous torch CUDA tensor (float32 or bfloat16/int16 bits)
    with elements [start, start + numel) of a stream, on the current stream."""
    import torch
    assert tensor.is_cuda and tensor.is_contiguous()
    stream = torch.cuda.current_stream(tensor.device).cuda_stream
    if tensor.dtype == torch.float32:
        rc = dev().synth_dev_fill_f32(C.byref(spec), start, tensor.numel(),
                                      C.c_void_p(tensor.data_ptr()), C.c_void_p(stream))
    elif tensor.element_size() == 2:
        rc = dev().synth_dev_fill_bf16(C.byref(spec), start, tensor.numel(),
                                       C.c_void_p(tensor.data_ptr()), C.c_void_p(stream))
    else:
        raise TypeError("float32 or 16-bit tensor expected")
    if rc != 0:
        raise RuntimeError(f"synth device fill failed ({rc})")

"""CPU oracle of one rank's sharded mixed-precision optimizer step.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product package never imports
this module, and the two share no code.

This module is argument marshalling over liboracle.so (oracle.c), which holds
every piece of arithmetic; the numpy arrays passed in must be C-contiguous.
The definitions each function follows are stated in oracle.h.
"""
import ctypes as C
import os

import numpy as np

from . import build as _build

F32, BF16 = 0, 1

_lib = None


class Scalars(C.Structure):
    _fields_ = [(n, C.c_float) for n in
                ("b1", "b2", "omb1", "omb2", "step_size", "sqrt_bc2", "decay", "eps")]


ACC_WORDS = 16


class Acc(C.Structure):
    """Exact sum of squares: X * 2^-128, X held in 16 little-endian u32 digits."""
    _fields_ = [("w", C.c_uint32 * ACC_WORDS), ("nonfinite", C.c_uint64)]

    @property
    def X(self) -> int:
        return sum(int(self.w[k]) << (32 * k) for k in range(ACC_WORDS))

    def copy(self) -> "Acc":
        out = Acc()
        C.memmove(C.byref(out), C.byref(self), C.sizeof(Acc))
        return out


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _lib = _load(_build.LIB)
    return _lib


def use_library(path):
    """Swap the loaded oracle for another build of oracle.c (the mutation
    tests load deliberately broken copies); returns the previous handle."""
    global _lib
    old = _lib
    _lib = _load(path) if isinstance(path, str) else path
    return old


def _load(path):
    L = C.CDLL(path)
    vp, sz = C.c_void_p, C.c_size_t
    L.oracle_f32_to_bf16.argtypes = [C.c_float]
    L.oracle_f32_to_bf16.restype = C.c_uint16
    L.oracle_f32_to_bf16_array.argtypes = [vp, sz, vp]
    L.oracle_bf16_to_f32.argtypes = [C.c_uint16]
    L.oracle_bf16_to_f32.restype = C.c_float
    L.oracle_make_scalars.argtypes = [C.c_double] * 5 + [C.c_int64, C.POINTER(Scalars)]
    L.oracle_pow_u.argtypes = [C.c_double, C.c_int64]
    L.oracle_pow_u.restype = C.c_double
    L.oracle_inv_scale.argtypes = [C.c_int, C.c_double]
    L.oracle_inv_scale.restype = C.c_float
    L.oracle_reduce.argtypes = [C.POINTER(vp), C.c_int, C.c_int, sz, C.c_float, vp]
    L.oracle_acc_zero.argtypes = [C.POINTER(Acc)]
    L.oracle_acc_add.argtypes = [C.POINTER(Acc), C.POINTER(Acc)]
    L.oracle_acc_add_fixed.argtypes = [C.POINTER(Acc), C.c_double]
    L.oracle_norm_accumulate.argtypes = [vp, sz, C.POINTER(Acc)]
    L.oracle_acc_sumsq.argtypes = [C.POINTER(Acc)]
    L.oracle_acc_sumsq.restype = C.c_double
    L.oracle_clip_coef.argtypes = [C.c_double, C.c_double]
    L.oracle_clip_coef.restype = C.c_float
    L.oracle_gate.argtypes = [C.POINTER(Acc), C.c_double, C.c_int, C.POINTER(C.c_float)]
    L.oracle_gate.restype = C.c_int
    L.oracle_adamw.argtypes = [sz, vp, C.c_float, C.POINTER(Scalars), vp, vp, vp, vp]
    L.oracle_step.argtypes = [C.POINTER(vp), C.c_int, C.c_int, sz, C.c_float,
                              C.c_double, C.c_int] + [C.c_double] * 5 + [
                              C.c_int64, C.POINTER(Acc), C.c_int,
                              vp, vp, vp, vp, vp, C.POINTER(Acc)]
    L.oracle_step.restype = C.c_int
    L.oracle_e4m3_encode.argtypes = [C.c_double]
    L.oracle_e4m3_encode.restype = C.c_uint8
    L.oracle_mx_encode.argtypes = [C.c_uint16, C.c_int]
    L.oracle_mx_encode.restype = C.c_uint8
    L.oracle_mx_encode_array.argtypes = [vp, sz, C.c_int, vp]
    L.oracle_mxfp8_pack.argtypes = [vp, sz, vp, vp]
    L.oracle_mxfp8_pack.restype = C.c_int
    L.oracle_e4m3_value.argtypes = [C.c_uint8]
    L.oracle_e4m3_value.restype = C.c_double
    L.oracle_mxfp8_decode.argtypes = [vp, vp, sz, vp]
    L.oracle_mxfp8_decode.restype = C.c_int
    return L


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return C.c_void_p(a.ctypes.data)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError("replicas must be float32 or uint16 (bf16 bits)")


# ------------------------------------------------------------------ bf16 ---

def f32_to_bf16(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32).ravel()
    out = np.empty(x.size, dtype=np.uint16)
    lib().oracle_f32_to_bf16_array(_ptr(x), x.size, _ptr(out))
    return out


def bf16_to_f32(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16).ravel()
    f = lib().oracle_bf16_to_f32
    return np.fromiter((f(int(v)) for v in h), dtype=np.float32, count=h.size)


# --------------------------------------------------------------- scalars ---

def make_scalars(lr, beta1, beta2, eps, wd, t) -> Scalars:
    s = Scalars()
    rc = lib().oracle_make_scalars(lr, beta1, beta2, eps, wd, int(t), C.byref(s))
    if rc != 0:
        raise ValueError("t must be >= 1")
    return s


def pow_u(base: float, t: int) -> float:
    return lib().oracle_pow_u(base, int(t))


def inv_scale(P: int, loss_scale: float) -> float:
    return lib().oracle_inv_scale(int(P), float(loss_scale))


# ---------------------------------------------------------------- reduce ---

def _ptr_array(arrs):
    return (C.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])


def reduce(replicas, inv_scale_f: float, out: np.ndarray = None) -> np.ndarray:
    reps = [np.ascontiguousarray(r) for r in replicas]
    n = reps[0].size
    code = _dtype_code(reps[0])
    assert all(r.size == n and r.dtype == reps[0].dtype for r in reps)
    g = np.empty(n, dtype=np.float32) if out is None else out
    assert g.dtype == np.float32 and g.size == n and g.flags["C_CONTIGUOUS"]
    lib().oracle_reduce(_ptr_array(reps), len(reps), code, n, inv_scale_f, _ptr(g))
    return g


# ------------------------------------------------------------------ norm ---

def acc_zero() -> Acc:
    a = Acc()
    lib().oracle_acc_zero(C.byref(a))
    return a


def acc_add(dst: Acc, src: Acc) -> Acc:
    lib().oracle_acc_add(C.byref(dst), C.byref(src))
    return dst


def acc_add_fixed(acc: Acc, S: float) -> Acc:
    lib().oracle_acc_add_fixed(C.byref(acc), float(S))
    return acc


def norm_accumulate(g: np.ndarray, acc: Acc = None) -> Acc:
    g = np.ascontiguousarray(g, dtype=np.float32)
    acc = acc_zero() if acc is None else acc
    lib().oracle_norm_accumulate(_ptr(g), g.size, C.byref(acc))
    return acc


def acc_sumsq(acc: Acc) -> float:
    return lib().oracle_acc_sumsq(C.byref(acc))


def clip_coef(sumsq: float, max_norm: float) -> float:
    return lib().oracle_clip_coef(float(sumsq), float(max_norm))


def gate(acc: Acc, max_norm: float, check_overflow: bool):
    """(skip, coef) of a step from its global accumulator (oracle_gate)."""
    coef = C.c_float()
    skip = lib().oracle_gate(C.byref(acc), float(max_norm), int(bool(check_overflow)),
                             C.byref(coef))
    return bool(skip), coef.value


# ----------------------------------------------------------------- AdamW ---

def adamw(g, coef, s: Scalars, master, m, v, param=None):
    """In place on master/m/v (float32) and param (uint16 bf16 bits)."""
    g = np.ascontiguousarray(g, dtype=np.float32)
    n = g.size
    for a in (master, m, v):
        assert a.dtype == np.float32 and a.size == n and a.flags["C_CONTIGUOUS"]
    pp = None
    if param is not None:
        assert param.dtype == np.uint16 and param.size == n and param.flags["C_CONTIGUOUS"]
        pp = _ptr(param)
    lib().oracle_adamw(n, _ptr(g), float(coef), C.byref(s), _ptr(master), _ptr(m),
                       _ptr(v), pp)


def step(replicas, inv_scale_f, max_norm, check_overflow, lr, beta1, beta2, eps,
         wd, t, master, m, v, param=None, extra_accs=(), g_tmp=None):
    """One rank's whole step in place.  Returns (skipped, own_acc)."""
    reps = [np.ascontiguousarray(r) for r in replicas]
    n = reps[0].size
    code = _dtype_code(reps[0])
    if g_tmp is None:
        g_tmp = np.empty(n, dtype=np.float32)
    extra = (Acc * max(1, len(extra_accs)))(*extra_accs) if extra_accs else None
    own = Acc()
    pp = _ptr(param) if param is not None else None
    rc = lib().oracle_step(_ptr_array(reps), len(reps), code, n, float(inv_scale_f),
                           float(max_norm), int(bool(check_overflow)), lr, beta1,
                           beta2, eps, wd, int(t), extra, len(extra_accs),
                           _ptr(g_tmp), _ptr(master), _ptr(m), _ptr(v), pp,
                           C.byref(own))
    return bool(rc), own


def _cuts(n: int, parts: int):
    per = max(32, ((n + parts - 1) // parts + 31) // 32 * 32)
    return [(a, min(n, a + per)) for a in range(0, n, per)]


def step_parallel(replicas, inv_scale_f, max_norm, check_overflow, lr, beta1, beta2, eps,
                  wd, t, master, m, v, param=None, g_tmp=None, threads=None):
    """The same step as `step`, spread over threads (the ctypes calls release
    the GIL): reduce + norm state per 32-aligned slice, the integer norm
    states added, then AdamW per slice.  Integer addition is associative, so
    the result is bit for bit that of `step`.  Returns (skipped, own_acc)."""
    from concurrent.futures import ThreadPoolExecutor
    reps = [np.ascontiguousarray(r) for r in replicas]
    n = reps[0].size
    threads = threads or os.cpu_count() or 1
    if g_tmp is None:
        g_tmp = np.empty(n, dtype=np.float32)
    cuts = _cuts(n, threads)

    def first(c):
        a, b = c
        g_tmp[a:b] = reduce([r[a:b] for r in reps], inv_scale_f)
        return norm_accumulate(g_tmp[a:b])

    with ThreadPoolExecutor(threads) as ex:
        parts = list(ex.map(first, cuts))
        own = acc_zero()
        for part in parts:
            acc_add(own, part)
        skip, coef = gate(own, max_norm, check_overflow)
        if skip:
            return True, own
        s = make_scalars(lr, beta1, beta2, eps, wd, t)

        def second(c):
            a, b = c
            adamw(g_tmp[a:b], coef, s, master[a:b], m[a:b], v[a:b],
                  None if param is None else param[a:b])

        list(ex.map(second, cuts))
    return False, own


# ----------------------------------------------------------------- MXFP8 ---

def e4m3_encode(q: float) -> int:
    return lib().oracle_e4m3_encode(float(q))


def e4m3_value(code: int) -> float:
    return lib().oracle_e4m3_value(int(code))


def mx_encode_array(x: np.ndarray, e_s: int) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.uint16)
    out = np.empty(x.size, dtype=np.uint8)
    lib().oracle_mx_encode_array(_ptr(x), x.size, int(e_s), _ptr(out))
    return out


def mxfp8_pack(x: np.ndarray):
    x = np.ascontiguousarray(x, dtype=np.uint16)
    n = x.size
    if n % 32:
        raise ValueError("MXFP8 packing needs a multiple of 32 elements")
    elem = np.empty(n, dtype=np.uint8)
    scale = np.empty(n // 32, dtype=np.uint8)
    rc = lib().oracle_mxfp8_pack(_ptr(x), n, _ptr(elem), _ptr(scale))
    assert rc == 0
    return elem, scale


def mxfp8_decode(elem: np.ndarray, scale: np.ndarray) -> np.ndarray:
    elem = np.ascontiguousarray(elem, dtype=np.uint8)
    scale = np.ascontiguousarray(scale, dtype=np.uint8)
    n = elem.size
    if n % 32 or scale.size < n // 32:
        raise ValueError("MXFP8 decode needs n % 32 == 0 and n/32 scales")
    out = np.empty(n, dtype=np.float32)
    rc = lib().oracle_mxfp8_decode(_ptr(elem), _ptr(scale), n, _ptr(out))
    assert rc == 0
    return out

"""The C-ABI library without a GPU: it loads, exports every function the
header declares, and rejects bad arguments before touching the device.
No call here launches a kernel."""
import ctypes as C
import os
import re

import pytest

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zero_step.h")
LIB = os.path.join(ROOT, "zero_sharded_mixed_step_amd", "libzero_step.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(zero_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libzero_step.so is not built (run __graft_entry__.build())")
    return C.CDLL(LIB)


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"zero_shard_reduce", "zero_grad_norm", "zero_adamw_step",
            "zero_mxfp8_pack"} <= set(names)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_constants_match_the_header():
    """The binding's copies of the header's constants."""
    from zero_sharded_mixed_step_amd import _binding as B
    text = open(HEADER).read()
    consts = {m.group(1): m.group(2) for m in
              re.finditer(r"#define (ZERO_[A-Z_]+) (.+)", text)}
    assert int(consts["ZERO_ABI_VERSION"]) == B.ABI_VERSION
    assert int(consts["ZERO_MAX_REPLICAS"]) == B.ZERO_MAX_REPLICAS
    a, b = re.fullmatch(r"\((\d+) \* (\d+)\)", consts["ZERO_REDUCE_WORKSPACE_BYTES"]).groups()
    assert int(a) * int(b) == B.REDUCE_WORKSPACE_BYTES


def test_version_and_status_strings(lib):
    lib.zero_abi_version.restype = C.c_int
    assert lib.zero_abi_version() == 4
    lib.zero_strerror.restype = C.c_char_p
    lib.zero_strerror.argtypes = [C.c_int]
    texts = {lib.zero_strerror(s).decode() for s in (0, -1, -2, -3, -4, 7)}
    assert len(texts) == 6 and all(texts)


def test_inv_scale_matches_definition(lib):
    lib.zero_inv_scale.restype = C.c_float
    lib.zero_inv_scale.argtypes = [C.c_int, C.c_double]
    for P in (1, 2, 3, 4, 7, 8, 64):
        for ls in (1.0, 65536.0, 1024.0, 3.0):
            assert lib.zero_inv_scale(P, ls) == O.inv_scale(P, ls)


def test_argument_checks(lib):
    vp = C.c_void_p
    lib.zero_shard_reduce.argtypes = [vp, C.c_int, C.c_int, C.c_size_t, C.c_float, vp, vp, vp,
                                      C.c_size_t, vp]
    lib.zero_shard_reduce_mx.argtypes = [vp, vp, C.c_int, C.c_size_t, C.c_float, vp, vp, vp,
                                         C.c_size_t, vp]
    lib.zero_mxfp8_pack.argtypes = [vp, C.c_size_t, vp, vp, vp]
    lib.zero_grad_norm.argtypes = [vp, C.c_int, C.c_size_t, C.c_float, vp, vp]
    lib.zero_adamw_step.argtypes = [vp, vp]
    lib.zero_norm_acc_clear.argtypes = [vp, C.c_int, vp]
    fake = 0x10000                     # aligned, never dereferenced
    reps = (vp * 2)(fake, fake + 0x1000)
    assert lib.zero_shard_reduce(None, 2, 1, 64, 1.0, fake, None, None, 0, None) == -1
    assert lib.zero_shard_reduce(reps, 0, 1, 64, 1.0, fake, None, None, 0, None) == -1
    assert lib.zero_shard_reduce(reps, 65, 1, 64, 1.0, fake, None, None, 0, None) == -1
    assert lib.zero_shard_reduce(reps, 2, 5, 64, 1.0, fake, None, None, 0, None) == -1
    assert lib.zero_shard_reduce(reps, 2, 1, 64, 1.0, None, None, None, 0, None) == -1
    assert lib.zero_shard_reduce(reps, 2, 1, 64, 1.0, fake + 4, None, None, 0, None) == -2
    bad = (vp * 2)(fake, fake + 2)
    assert lib.zero_shard_reduce(bad, 2, 1, 64, 1.0, fake, None, None, 0, None) == -2
    assert lib.zero_shard_reduce(reps, 2, 1, 1 << 32, 1.0, None, fake, None, 0, None) == -3
    assert lib.zero_shard_reduce(reps, 2, 1, 0, 1.0, fake, None, None, 0, None) == 0
    # the optional reduce workspace: 16-byte aligned, at least
    # ZERO_REDUCE_WORKSPACE_BYTES (64 * 512)
    ws = 64 * 512
    assert lib.zero_shard_reduce(reps, 2, 1, 64, 1.0, fake, None, fake + 8, ws, None) == -2
    assert lib.zero_shard_reduce(reps, 2, 1, 64, 1.0, fake, None, fake, ws - 1, None) == -3
    assert lib.zero_shard_reduce(reps, 2, 1, 0, 1.0, fake, fake, fake, ws, None) == 0
    scales = (vp * 2)(fake + 1, fake + 3)
    assert lib.zero_shard_reduce_mx(reps, scales, 2, 64, 1.0, fake, None, fake + 8, ws,
                                    None) == -2
    assert lib.zero_shard_reduce_mx(reps, scales, 2, 64, 1.0, fake, None, fake, 64,
                                    None) == -3
    assert lib.zero_shard_reduce_mx(reps, scales, 2, 0, 1.0, fake, None, fake, ws, None) == 0
    assert lib.zero_grad_norm(None, 1, 64, 1.0, fake, None) == -1
    assert lib.zero_mxfp8_pack(fake, 33, fake, fake, None) == -3
    assert lib.zero_mxfp8_pack(fake, 64, fake, fake + 1, None) == -2
    assert lib.zero_mxfp8_pack(None, 64, fake, fake, None) == -1
    assert lib.zero_mxfp8_pack(fake, 0, fake, fake, None) == 0
    assert lib.zero_adamw_step(None, None) == -1
    assert lib.zero_norm_acc_clear(None, 1, None) == -1
    assert lib.zero_norm_acc_clear(fake + 8, 1, None) == -2
    assert lib.zero_norm_acc_clear(None, 0, None) == 0
    lib.zero_unfused_workspace_bytes.restype = C.c_size_t
    lib.zero_unfused_workspace_bytes.argtypes = [C.c_size_t, C.c_int]
    assert lib.zero_unfused_workspace_bytes(1000, 2) >= 2 * 4000 + 3 * 64
    lib.zero_adamw_step_unfused.argtypes = [vp, vp, C.c_size_t, vp]
    assert lib.zero_adamw_step_unfused(None, fake, 1 << 20, None) == -1


def test_adamw_step_counter_checks(lib):
    """The step index: a host `step` >= 1, or a device counter (8-byte
    aligned); the unfused chain takes the host form only.  Every case here
    fails its checks, so nothing is launched."""
    from zero_sharded_mixed_step_amd._binding import _AdamArgs
    vp = C.c_void_p
    lib.zero_adamw_step.argtypes = [vp, vp]
    lib.zero_adamw_step_unfused.argtypes = [vp, vp, C.c_size_t, vp]
    fake = 0x10000
    a = _AdamArgs()
    a.n, a.grad_f32, a.P, a.dtype = 64, fake, 1, 0
    a.master, a.m, a.v = fake + 0x1000, fake + 0x2000, fake + 0x3000
    a.lr, a.beta1, a.beta2, a.eps = 1e-3, 0.9, 0.999, 1e-8
    a.step, a.step_dev = 0, None
    assert lib.zero_adamw_step(C.byref(a), None) == -1          # no step at all
    a.step_dev = fake + 4
    assert lib.zero_adamw_step(C.byref(a), None) == -2          # counter misaligned
    a.step_dev = fake + 8
    assert lib.zero_adamw_step_unfused(C.byref(a), fake, 1 << 30, None) == -1

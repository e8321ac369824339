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
    assert int(a) == 8 * B.ACC_WORDS                      # one slot = one zero_norm_acc
    body = re.search(r"typedef struct zero_norm_acc \{(.*?)\} zero_norm_acc;", text, re.S).group(1)
    fields = re.findall(r"uint64_t (\w+)(?:\[(\d+)\])?;", body)
    assert fields == [("digit", str(B.ACC_DIGITS)), ("nonfinite", ""), ("reserved", "2")]
    assert sum(int(k or 1) for _, k in fields) == B.ACC_WORDS


def _prototype(text, name):
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    m = re.search(r"\bint\s+" + name + r"\s*\(([^)]*)\)\s*;", text)
    assert m, name
    params = [" ".join(p.split()) for p in m.group(1).split(",")]
    return [re.sub(r"\s*\*\s*", "* ", p).replace("* ", "*").strip() for p in params]


def test_path_calls_have_the_specified_signatures():
    """The four calls of the path, parameter by parameter: plain pointers and
    sizes, the stream last (void* stands for hipStream_t in this C header)."""
    text = open(HEADER).read()
    want = {
        "zero_shard_reduce": ["const void *const *replicas", "int P", "int dtype", "size_t n",
                              "float inv_scale", "float *g_out", "zero_norm_acc *acc",
                              "void *stream"],
        "zero_grad_norm": ["const void *grad", "int dtype", "size_t n", "float inv_scale",
                           "zero_norm_acc *acc", "void *stream"],
        "zero_adamw_step": ["const zero_adamw_args *args", "void *stream"],
        "zero_mxfp8_pack": ["const uint16_t *bf16_in", "size_t n", "uint8_t *elem_out",
                            "uint8_t *scale_out", "void *stream"],
    }
    norm = lambda ps: [re.sub(r"\s*\*\s*", "*", p) for p in ps]
    for name, params in want.items():
        assert norm(_prototype(text, name)) == norm(params), name


def test_version_and_status_strings(lib):
    lib.zero_abi_version.restype = C.c_int
    assert lib.zero_abi_version() == 5
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
    """Every case fails its checks or is a zero-length no-op, so nothing is
    launched.  Alignment: 16 bytes for device arrays and accumulators, any for
    MXFP8 scale bytes, 4 for int32/float outputs, 8 for the step counter."""
    vp, sz, i, f = C.c_void_p, C.c_size_t, C.c_int, C.c_float
    lib.zero_shard_reduce.argtypes = [vp, i, i, sz, f, vp, vp, vp]
    lib.zero_shard_reduce_ws.argtypes = [vp, i, i, sz, f, vp, vp, vp, sz, vp]
    lib.zero_shard_reduce_mx.argtypes = [vp, vp, i, sz, f, vp, vp, vp]
    lib.zero_shard_reduce_mx_ws.argtypes = [vp, vp, i, sz, f, vp, vp, vp, sz, vp]
    lib.zero_mxfp8_pack.argtypes = [vp, sz, vp, vp, vp]
    lib.zero_grad_norm.argtypes = [vp, i, sz, f, vp, vp]
    lib.zero_adamw_step.argtypes = [vp, vp]
    lib.zero_norm_acc_clear.argtypes = [vp, i, vp]
    lib.zero_step_gate.argtypes = [vp, i, C.c_double, i, vp, vp, vp]
    fake = 0x10000                     # aligned, never dereferenced
    reps = (vp * 2)(fake, fake + 0x1000)
    red = lib.zero_shard_reduce
    assert red(None, 2, 1, 64, 1.0, fake, None, None) == -1
    assert red(reps, 0, 1, 64, 1.0, fake, None, None) == -1
    assert red(reps, 65, 1, 64, 1.0, fake, None, None) == -1
    assert red(reps, 2, 5, 64, 1.0, fake, None, None) == -1
    assert red(reps, 2, 1, 64, 1.0, None, None, None) == -1
    assert red(reps, 2, 1, 64, 1.0, fake + 4, None, None) == -2
    assert red(reps, 2, 1, 64, 1.0, None, fake + 8, None) == -2     # accumulator: 16 bytes
    bad = (vp * 2)(fake, fake + 2)
    assert red(bad, 2, 1, 64, 1.0, fake, None, None) == -2
    # a norm call takes up to 2^37 elements (the accumulator's capacity)
    assert red(reps, 2, 1, (1 << 37) + 32, 1.0, None, fake, None) == -3
    assert red(reps, 2, 1, 0, 1.0, fake, None, None) == 0
    assert red(reps, 2, 1, 0, 1.0, fake, fake, None) == 0
    # the workspace form: 16-byte aligned, at least ZERO_REDUCE_WORKSPACE_BYTES
    ws = 128 * 512
    rws = lib.zero_shard_reduce_ws
    assert rws(reps, 2, 1, 64, 1.0, fake, None, fake + 8, ws, None) == -2
    assert rws(reps, 2, 1, 64, 1.0, fake, None, fake, ws - 1, None) == -3
    assert rws(reps, 2, 1, 64, 1.0, fake, None, None, ws, None) == -1   # no workspace
    assert rws(reps, 2, 1, 0, 1.0, fake, fake, fake, ws, None) == 0
    scales = (vp * 2)(fake + 1, fake + 3)                            # scale bytes: any
    mx, mxws = lib.zero_shard_reduce_mx, lib.zero_shard_reduce_mx_ws
    assert mx(reps, scales, 2, 48, 1.0, fake, None, None) == -3     # n % 32
    assert mx(reps, scales, 2, (1 << 37) + 32, 1.0, None, fake, None) == -3
    assert mx(bad, scales, 2, 64, 1.0, fake, None, None) == -2
    assert mx(reps, scales, 2, 0, 1.0, fake, None, None) == 0
    assert mxws(reps, scales, 2, 64, 1.0, fake, None, fake + 8, ws, None) == -2
    assert mxws(reps, scales, 2, 64, 1.0, fake, None, fake, 64, None) == -3
    assert mxws(reps, scales, 2, 0, 1.0, fake, None, fake, ws, None) == 0
    assert mxws(reps, scales, 2, 64, 1.0, fake, None, None, ws, None) == -1
    assert lib.zero_grad_norm(None, 1, 64, 1.0, fake, None) == -1
    assert lib.zero_grad_norm(fake, 1, 64, 1.0, fake + 8, None) == -2
    assert lib.zero_grad_norm(fake, 1, (1 << 37) + 1, 1.0, fake, None) == -3
    assert lib.zero_mxfp8_pack(fake, 33, fake, fake, None) == -3
    assert lib.zero_mxfp8_pack(fake, 64, fake, fake + 1, None) == -2
    assert lib.zero_mxfp8_pack(None, 64, fake, fake, None) == -1
    assert lib.zero_mxfp8_pack(fake, 0, fake, fake, None) == 0
    assert lib.zero_adamw_step(None, None) == -1
    assert lib.zero_norm_acc_clear(None, 1, None) == -1
    assert lib.zero_norm_acc_clear(fake + 8, 1, None) == -2
    assert lib.zero_norm_acc_clear(None, 0, None) == 0
    assert lib.zero_step_gate(fake + 8, 1, 1.0, 1, fake, fake, None) == -2
    assert lib.zero_step_gate(fake, 1, 1.0, 1, fake + 2, fake, None) == -2
    assert lib.zero_step_gate(fake, 1, 1.0, 1, None, fake, None) == -1
    lib.zero_unfused_workspace_bytes.restype = C.c_size_t
    lib.zero_unfused_workspace_bytes.argtypes = [C.c_size_t, C.c_int]
    assert lib.zero_unfused_workspace_bytes(1000, 2) >= 2 * 4000 + 3 * 128
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



def test_header_compiles_as_c11():
    """zero_step.h is plain C: the C program that drives the ABI in the GPU
    tests (tests/c_abi/abi_roundtrip.c) compiles as pedantic C11 with every
    warning an error (HIP's own headers as system headers)."""
    import subprocess
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = ["gcc", "-std=c11", "-pedantic", "-Werror", "-Wall", "-Wextra", "-fsyntax-only",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "oracle"), "-I", os.path.join(ROOT, "synth"),
           "-isystem", os.path.join(rocm, "include"),
           os.path.join(ROOT, "tests", "c_abi", "abi_roundtrip.c")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr

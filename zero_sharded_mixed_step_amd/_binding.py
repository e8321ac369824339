"""ctypes binding of libzero_step.so, with the C entry points' names.

Argument marshalling only: tensors become device pointers, the current torch
stream becomes the hipStream_t, and a nonzero status raises ZeroStepError.
Every step of the computation runs in the library's HIP kernels; there is no
host or fallback path.  PyTorch supplies device memory and streams.
"""
import ctypes as C
import os

import torch

from . import build as _build

ZERO_F32, ZERO_BF16, ZERO_MXFP8 = 0, 1, 2
ABI_VERSION = 5        # the zero_step.h this binding's structs follow
ZERO_MAX_REPLICAS = 64
ACC_WORDS = 16         # one zero_norm_acc = 128 bytes = 16 int64 words
ACC_DIGITS = 13        # digit[13]; then nonfinite, reserved[2]
REDUCE_WORKSPACE_BYTES = 128 * 512   # ZERO_REDUCE_WORKSPACE_BYTES

_lib = None


class ZeroStepError(RuntimeError):
    def __init__(self, status, fn):
        super().__init__(f"{fn}: {zero_strerror(status)} (status {status})")
        self.status = status


class _AdamArgs(C.Structure):
    _fields_ = [("n", C.c_size_t), ("grad_f32", C.c_void_p), ("replicas", C.c_void_p),
                ("P", C.c_int), ("dtype", C.c_int), ("inv_scale", C.c_float),
                ("master", C.c_void_p), ("m", C.c_void_p), ("v", C.c_void_p),
                ("param_bf16", C.c_void_p), ("accs", C.c_void_p), ("n_accs", C.c_int),
                ("max_norm", C.c_double), ("check_overflow", C.c_int),
                ("lr", C.c_double), ("beta1", C.c_double), ("beta2", C.c_double),
                ("eps", C.c_double), ("weight_decay", C.c_double), ("step", C.c_int64),
                ("skipped_out", C.c_void_p), ("mx_elem_out", C.c_void_p),
                ("mx_scale_out", C.c_void_p), ("step_dev", C.c_void_p)]


def lib():
    """Load libzero_step.so; fails loudly when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            raise RuntimeError(f"{_build.LIB} is not built: run __graft_entry__.build() "
                               "(there is no non-HIP implementation)")
        L = C.CDLL(_build.LIB)
        vp, sz, i = C.c_void_p, C.c_size_t, C.c_int
        L.zero_abi_version.restype = i
        L.zero_strerror.argtypes = [i]
        L.zero_strerror.restype = C.c_char_p
        L.zero_inv_scale.argtypes = [i, C.c_double]
        L.zero_inv_scale.restype = C.c_float
        L.zero_norm_acc_clear.argtypes = [vp, i, vp]
        L.zero_shard_reduce.argtypes = [vp, i, i, sz, C.c_float, vp, vp, vp]
        L.zero_shard_reduce_ws.argtypes = [vp, i, i, sz, C.c_float, vp, vp, vp, sz, vp]
        L.zero_shard_reduce_noalloc.argtypes = [vp, i, i, sz, C.c_float, vp, vp, vp]
        L.zero_grad_norm.argtypes = [vp, i, sz, C.c_float, vp, vp]
        L.zero_adamw_step.argtypes = [C.POINTER(_AdamArgs), vp]
        L.zero_step_gate.argtypes = [vp, i, C.c_double, i, vp, vp, vp]
        L.zero_mxfp8_pack.argtypes = [vp, sz, vp, vp, vp]
        L.zero_shard_reduce_mx.argtypes = [vp, vp, i, sz, C.c_float, vp, vp, vp]
        L.zero_shard_reduce_mx_ws.argtypes = [vp, vp, i, sz, C.c_float, vp, vp, vp, sz, vp]
        L.zero_unfused_workspace_bytes.argtypes = [sz, i]
        L.zero_unfused_workspace_bytes.restype = sz
        L.zero_adamw_step_unfused.argtypes = [C.POINTER(_AdamArgs), vp, sz, vp]
        for f in (L.zero_norm_acc_clear, L.zero_shard_reduce, L.zero_shard_reduce_ws,
                  L.zero_shard_reduce_noalloc,
                  L.zero_shard_reduce_mx, L.zero_shard_reduce_mx_ws, L.zero_grad_norm,
                  L.zero_adamw_step, L.zero_step_gate, L.zero_mxfp8_pack,
                  L.zero_adamw_step_unfused):
            f.restype = i
        if L.zero_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{_build.LIB} has ABI version {L.zero_abi_version()}, the "
                               f"binding expects {ABI_VERSION}: rebuild it")
        _lib = L
    return _lib


def _check(status, fn):
    if status != 0:
        raise ZeroStepError(status, fn)


def _stream(stream):
    if stream is None:
        return C.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return C.c_void_p(stream.cuda_stream)
    return C.c_void_p(int(stream))


def _dev_ptr(t, name):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name} is on {t.device}; the library launches on the current "
                         f"device, cuda:{torch.cuda.current_device()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return C.c_void_p(t.data_ptr())


def _need(t, n, name, dtypes):
    """Every buffer a kernel touches must hold the elements it will touch:
    the C ABI takes raw pointers, so lengths are checked here, before launch."""
    if t is None:
        return
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if t.numel() < n:
        raise ValueError(f"{name} holds {t.numel()} elements, the call touches {n}")


F32 = (torch.float32,)
BITS16 = (torch.bfloat16, torch.int16, torch.uint16)
U8 = (torch.uint8,)
I32 = (torch.int32,)


def _dtype_code(t):
    if t.dtype == torch.float32:
        return ZERO_F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return ZERO_BF16
    raise TypeError("replicas must be float32 or bf16 (bfloat16 / 16-bit bits)")


def _ptr_array(tensors, name):
    ptrs = [_dev_ptr(t, name).value for t in tensors]
    return (C.c_void_p * len(ptrs))(*ptrs)


def _acc_ptr(acc):
    if acc is None:
        return None, 0
    if acc.dtype != torch.int64 or acc.numel() % ACC_WORDS:
        raise TypeError(f"norm accumulators are int64 tensors of shape (k, {ACC_WORDS})")
    return _dev_ptr(acc, "acc"), acc.numel() // ACC_WORDS


# ------------------------------------------------------------ helpers ---

def zero_abi_version() -> int:
    return lib().zero_abi_version()


def zero_strerror(status: int) -> str:
    return lib().zero_strerror(int(status)).decode()


def zero_inv_scale(P: int, loss_scale: float = 1.0) -> float:
    return lib().zero_inv_scale(int(P), float(loss_scale))


def new_reduce_workspace(device="cuda") -> torch.Tensor:
    """A zeroed reduce workspace (ZERO_REDUCE_WORKSPACE_BYTES, as int64 words
    so that zero_norm_acc_clear can zero it)."""
    ws = torch.empty((REDUCE_WORKSPACE_BYTES // (8 * ACC_WORDS), ACC_WORDS), dtype=torch.int64,
                     device=device)
    zero_norm_acc_clear(ws)
    return ws


def _ws_ptr(workspace):
    if workspace is None:
        raise ValueError("the _ws entry points need a workspace (new_reduce_workspace())")
    nbytes = workspace.numel() * workspace.element_size()
    if nbytes < REDUCE_WORKSPACE_BYTES:
        raise ValueError(f"reduce workspace holds {nbytes} bytes, needs {REDUCE_WORKSPACE_BYTES}")
    return _dev_ptr(workspace, "workspace"), nbytes


def new_norm_acc(k: int = 1, device="cuda") -> torch.Tensor:
    """k zeroed accumulators (128 bytes each) as an int64 (k, 16) tensor."""
    acc = torch.empty((k, ACC_WORDS), dtype=torch.int64, device=device)
    zero_norm_acc_clear(acc)
    return acc


def read_norm_acc(acc: torch.Tensor):
    """Host view of accumulators: list of (X, nonfinite) with X the integer
    whose value times 2^-128 is the sum of squares."""
    words = acc.detach().reshape(-1, ACC_WORDS).cpu().tolist()
    out = []
    for w in words:
        digits = [d & 0xFFFFFFFFFFFFFFFF for d in w[:ACC_DIGITS]]
        X = sum(d << (32 * k) for k, d in enumerate(digits))
        out.append((X, w[ACC_DIGITS] & 0xFFFFFFFFFFFFFFFF))
    return out


# -------------------------------------------------------- entry points ---

def zero_norm_acc_clear(accs: torch.Tensor, stream=None) -> None:
    p, k = _acc_ptr(accs)
    _check(lib().zero_norm_acc_clear(p, k, _stream(stream)), "zero_norm_acc_clear")


def _reduce_args(replicas, n, g_out, acc, name):
    reps = list(replicas)
    if not reps:
        raise ValueError("at least one replica")
    n = reps[0].numel() if n is None else int(n)
    for r in reps:
        if r.dtype != reps[0].dtype:
            raise ValueError("replicas must share one dtype")
        _need(r, n, "replica", F32 + BITS16)
    _need(g_out, n, "g_out", F32)
    ap, k = _acc_ptr(acc)
    if k > 1:
        raise ValueError(f"{name} adds to one accumulator")
    return reps, n, ap


def zero_shard_reduce(replicas, inv_scale: float, g_out=None, acc=None, n=None,
                      stream=None) -> None:
    reps, n, ap = _reduce_args(replicas, n, g_out, acc, "zero_shard_reduce")
    _check(lib().zero_shard_reduce(_ptr_array(reps, "replica"), len(reps), _dtype_code(reps[0]),
                                   n, float(inv_scale), _dev_ptr(g_out, "g_out"), ap,
                                   _stream(stream)), "zero_shard_reduce")


def zero_shard_reduce_ws(replicas, inv_scale: float, workspace, g_out=None, acc=None, n=None,
                         stream=None) -> None:
    """zero_shard_reduce with the one-shot form's workspace
    (new_reduce_workspace())."""
    reps, n, ap = _reduce_args(replicas, n, g_out, acc, "zero_shard_reduce_ws")
    wp, wb = _ws_ptr(workspace)
    _check(lib().zero_shard_reduce_ws(_ptr_array(reps, "replica"), len(reps),
                                      _dtype_code(reps[0]), n, float(inv_scale),
                                      _dev_ptr(g_out, "g_out"), ap, wp, wb, _stream(stream)),
           "zero_shard_reduce_ws")


def zero_shard_reduce_noalloc(replicas, inv_scale: float, g_out=None, acc=None, n=None,
                              stream=None) -> None:
    """zero_shard_reduce_ws with the library's own static slots (no
    workspace, nothing allocated); calls on one GPU must not overlap."""
    reps, n, ap = _reduce_args(replicas, n, g_out, acc, "zero_shard_reduce_noalloc")
    _check(lib().zero_shard_reduce_noalloc(_ptr_array(reps, "replica"), len(reps),
                                           _dtype_code(reps[0]), n, float(inv_scale),
                                           _dev_ptr(g_out, "g_out"), ap, _stream(stream)),
           "zero_shard_reduce_noalloc")


def _mx_args(codes, scales, n, g_out, acc, name):
    codes, scales = list(codes), list(scales)
    if not codes or len(codes) != len(scales):
        raise ValueError("one code array and one scale array per replica")
    n = codes[0].numel() if n is None else int(n)
    for c, sc in zip(codes, scales):
        _need(c, n, "codes", U8)
        _need(sc, n // 32, "scales", U8)
    _need(g_out, n, "g_out", F32)
    ap, k = _acc_ptr(acc)
    if k > 1:
        raise ValueError(f"{name} adds to one accumulator")
    return codes, scales, n, ap


def zero_shard_reduce_mx(codes, scales, inv_scale: float, g_out=None, acc=None, n=None,
                         stream=None) -> None:
    """Shard reduce of MXFP8-stored replicas: codes[k] uint8[n] and scales[k]
    uint8[n/32] per rank (n % 32 == 0)."""
    codes, scales, n, ap = _mx_args(codes, scales, n, g_out, acc, "zero_shard_reduce_mx")
    _check(lib().zero_shard_reduce_mx(_ptr_array(codes, "codes"), _ptr_array(scales, "scales"),
                                      len(codes), n, float(inv_scale), _dev_ptr(g_out, "g_out"),
                                      ap, _stream(stream)), "zero_shard_reduce_mx")


def zero_shard_reduce_mx_ws(codes, scales, inv_scale: float, workspace, g_out=None, acc=None,
                            n=None, stream=None) -> None:
    codes, scales, n, ap = _mx_args(codes, scales, n, g_out, acc, "zero_shard_reduce_mx_ws")
    wp, wb = _ws_ptr(workspace)
    _check(lib().zero_shard_reduce_mx_ws(_ptr_array(codes, "codes"),
                                         _ptr_array(scales, "scales"), len(codes), n,
                                         float(inv_scale), _dev_ptr(g_out, "g_out"), ap, wp,
                                         wb, _stream(stream)), "zero_shard_reduce_mx_ws")


def zero_grad_norm(grad, inv_scale: float, acc, n=None, stream=None) -> None:
    n = grad.numel() if n is None else int(n)
    _need(grad, n, "grad", F32 + BITS16)
    ap, k = _acc_ptr(acc)
    if k != 1:
        raise ValueError("zero_grad_norm adds to one accumulator")
    _check(lib().zero_grad_norm(_dev_ptr(grad, "grad"), _dtype_code(grad), n,
                                float(inv_scale), ap, _stream(stream)), "zero_grad_norm")


def _adam_args(master, m, v, step, lr, beta1, beta2, eps, weight_decay, grad_f32, replicas,
               inv_scale, param_bf16, accs, max_norm, check_overflow, skipped_out, mx_elem_out,
               mx_scale_out, n, step_dev=None):
    n = master.numel() if n is None else int(n)
    for name, t in (("master", master), ("m", m), ("v", v), ("grad_f32", grad_f32)):
        _need(t, n, name, F32)
    if replicas is not None:
        for r in replicas:
            if r.dtype != replicas[0].dtype:
                raise ValueError("replicas must share one dtype")
            _need(r, n, "replica", F32 + BITS16)
    _need(param_bf16, n, "param_bf16", BITS16)
    _need(skipped_out, 1, "skipped_out", I32)
    _need(mx_elem_out, n, "mx_elem_out", U8)
    _need(mx_scale_out, n // 32, "mx_scale_out", U8)
    _need(step_dev, 1, "step_dev", (torch.int64,))
    a = _AdamArgs()
    a.n = n
    keep = None
    if replicas is not None:
        reps = list(replicas)
        keep = _ptr_array(reps, "replica")
        a.replicas = C.cast(keep, C.c_void_p)
        a.P = len(reps)
        a.dtype = _dtype_code(reps[0])
    else:
        a.P = 1
        a.dtype = ZERO_F32
    a.grad_f32 = _dev_ptr(grad_f32, "grad_f32")
    a.inv_scale = float(inv_scale)
    a.master, a.m, a.v = (_dev_ptr(master, "master"), _dev_ptr(m, "m"), _dev_ptr(v, "v"))
    a.param_bf16 = _dev_ptr(param_bf16, "param_bf16")
    a.accs, a.n_accs = _acc_ptr(accs)
    a.max_norm = float(max_norm)
    a.check_overflow = int(bool(check_overflow))
    a.lr, a.beta1, a.beta2, a.eps, a.weight_decay = (float(lr), float(beta1), float(beta2),
                                                      float(eps), float(weight_decay))
    a.step = int(step)
    a.skipped_out = _dev_ptr(skipped_out, "skipped_out")
    a.mx_elem_out = _dev_ptr(mx_elem_out, "mx_elem_out")
    a.mx_scale_out = _dev_ptr(mx_scale_out, "mx_scale_out")
    a.step_dev = _dev_ptr(step_dev, "step_dev")
    return a, keep


def zero_adamw_step(master, m, v, *, step=0, lr, beta1=0.9, beta2=0.999, eps=1e-8,
                    weight_decay=0.0, grad_f32=None, replicas=None, inv_scale=1.0,
                    param_bf16=None, accs=None, max_norm=0.0, check_overflow=False,
                    skipped_out=None, mx_elem_out=None, mx_scale_out=None, n=None,
                    step_dev=None, stream=None) -> None:
    """`step`: 1-based index of this applied update; or `step_dev`: an int64
    device tensor holding the count of updates applied so far, read and
    advanced on the device (then `step` is ignored)."""
    a, keep = _adam_args(master, m, v, step, lr, beta1, beta2, eps, weight_decay, grad_f32,
                         replicas, inv_scale, param_bf16, accs, max_norm, check_overflow,
                         skipped_out, mx_elem_out, mx_scale_out, n, step_dev)
    rc = lib().zero_adamw_step(C.byref(a), _stream(stream))
    del keep
    _check(rc, "zero_adamw_step")


def zero_unfused_workspace_bytes(n: int, n_accs: int = 0) -> int:
    return lib().zero_unfused_workspace_bytes(int(n), int(n_accs))


def zero_adamw_step_unfused(master, m, v, workspace, *, step, lr, beta1=0.9, beta2=0.999,
                            eps=1e-8, weight_decay=0.0, grad_f32=None, replicas=None,
                            inv_scale=1.0, param_bf16=None, accs=None, max_norm=0.0,
                            check_overflow=False, skipped_out=None, mx_elem_out=None,
                            mx_scale_out=None, n=None, stream=None) -> None:
    """The step as a chain of single-operation kernels (`accs`: the OTHER
    ranks' accumulators; `workspace`: a uint8 device tensor of at least
    zero_unfused_workspace_bytes(n, k) bytes)."""
    if workspace is None:
        raise ValueError("the unfused chain needs a workspace of "
                         "zero_unfused_workspace_bytes(n, k) bytes")
    a, keep = _adam_args(master, m, v, step, lr, beta1, beta2, eps, weight_decay, grad_f32,
                         replicas, inv_scale, param_bf16, accs, max_norm, check_overflow,
                         skipped_out, mx_elem_out, mx_scale_out, n)
    rc = lib().zero_adamw_step_unfused(C.byref(a), _dev_ptr(workspace, "workspace"),
                                       workspace.numel() * workspace.element_size(),
                                       _stream(stream))
    del keep
    _check(rc, "zero_adamw_step_unfused")


def zero_step_gate(accs, max_norm, check_overflow, coef_out, skip_out, stream=None) -> None:
    _need(coef_out, 1, "coef_out", F32)
    _need(skip_out, 1, "skip_out", I32)
    ap, k = _acc_ptr(accs)
    _check(lib().zero_step_gate(ap, k, float(max_norm), int(bool(check_overflow)),
                                _dev_ptr(coef_out, "coef_out"), _dev_ptr(skip_out, "skip_out"),
                                _stream(stream)), "zero_step_gate")


def zero_mxfp8_pack(x_bf16, elem_out, scale_out, n=None, stream=None) -> None:
    n = x_bf16.numel() if n is None else int(n)
    _need(x_bf16, n, "x_bf16", BITS16)
    _need(elem_out, n, "elem_out", U8)
    _need(scale_out, n // 32, "scale_out", U8)
    _check(lib().zero_mxfp8_pack(_dev_ptr(x_bf16, "x"), n, _dev_ptr(elem_out, "elem_out"),
                                 _dev_ptr(scale_out, "scale_out"), _stream(stream)),
           "zero_mxfp8_pack")

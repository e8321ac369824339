"""One data-parallel rank's sharded mixed-precision optimizer step on MI355X.

The kernels live in libzero_step.so (HIP, gfx950) behind the C ABI declared in
include/zero_step.h; this package is its ctypes binding (`_binding`, same
names as the C entry points) plus `ShardStep`, which sequences the calls of
one step.  There is no host fallback: loading fails if the library is not
built.
"""
from ._binding import (ACC_DIGITS, ACC_WORDS, REDUCE_WORKSPACE_BYTES, ZERO_BF16,  # noqa: F401
                       ZERO_F32,
                       ZERO_MAX_REPLICAS, ZERO_MXFP8, ZeroStepError, lib, new_norm_acc,
                       new_reduce_workspace, read_norm_acc, zero_abi_version, zero_adamw_step,
                       zero_adamw_step_unfused, zero_grad_norm, zero_inv_scale, zero_mxfp8_pack,
                       zero_norm_acc_clear, zero_shard_reduce, zero_shard_reduce_mx,
                       zero_shard_reduce_mx_ws, zero_shard_reduce_noalloc, zero_shard_reduce_ws,
                       zero_step_gate,
                       zero_strerror,
                       zero_unfused_workspace_bytes)
from .step import ShardStep, choose_path  # noqa: F401

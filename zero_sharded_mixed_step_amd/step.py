"""Sequencing of one rank's optimizer step over the C-ABI calls.

`ShardStep` owns the rank's state buffers (fp32 master/m/v, bf16 param,
optional fp32 gradient, the norm accumulator, the skip flag, MXFP8 output)
and issues, on the current stream, the kernel launches of one step.  It
computes nothing itself.

Pass structure (bytes per shard element; g_b = bytes per replica element):
  - no gate (no clip, no overflow check): one fused pass, AdamW reads the P
    replicas directly: P*g_b + 26 bytes;
  - gated: the update waits for the global norm / non-finite count, so either
    materialise:  reduce writes fp32 g (+4) and AdamW re-reads it (+4), or
    recompute:    a norm-only pass over the replicas, then AdamW reduces the
                  replicas again (+P*g_b);
    whichever moves fewer bytes (materialise when P*g_b > 8).
The reduce runs bucket by bucket when `bucket` is set; the norm state of all
buckets accumulates in one accumulator (integer sums, so bucketing changes no
bit of the result).

MXFP8: with `pack`, the AdamW pass also writes the MXFP8 pack of the new
bf16 params (codes + block scales), saving the re-read of the bf16 param
shard and a launch; `pack_param()` runs the standalone pack kernel.

Step counter: `t` counts applied updates.  With the overflow check on, the
device decides the skip; the flag travels to pinned host memory behind an
event and is read just before the next step's AdamW launch, after that
step's reduce work is already queued, so the GPU never waits on the host.
With `device_counter=True` the counter lives in device memory instead: the
AdamW kernel derives its scalars from it and a one-lane kernel advances it
when the step applies, so a step needs nothing from the host and `capture()`
can record it once as a graph that is replayed every step.
"""
from typing import List, Optional

import torch

from . import _binding as B


def choose_path(P: int, g_b: float, gated: bool, mx_grads: bool = False,
                path: Optional[str] = None) -> str:
    """The pass structure of a step: "fused" (one pass, ungated),
    "materialize" (reduce writes fp32 g, AdamW re-reads it: P*g_b + 34 B per
    element) or "recompute" (norm-only pass, then AdamW reduces the replicas
    again: 2*P*g_b + 26 B), whichever moves fewer bytes when gated.
    MXFP8-stored replicas are read by the reduce pass only, so they always
    materialise.  `path` forces a choice (checked)."""
    if mx_grads:
        if path not in (None, "materialize"):
            raise ValueError("MXFP8 gradient replicas need the materialise path")
        return "materialize"
    if path is None:
        if not gated:
            return "fused"
        return "materialize" if P * g_b > 8 else "recompute"
    if path not in ("fused", "materialize", "recompute"):
        raise ValueError(path)
    if path == "fused" and gated:
        raise ValueError("a gated step needs the norm before the update")
    return path


# Reduce launches above this many elements take the one-shot form (the
# library's workspace); bucket-sized ones (the 7B shard's 25e6) ran faster
# on the persistent pipelined form, without the extra fold launch.
ONESHOT_MIN = 1 << 27


class ShardStep:
    def __init__(self, n: int, P: int, grad_dtype: torch.dtype, *, lr: float,
                 beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8,
                 weight_decay: float = 0.0, max_norm: float = 0.0,
                 check_overflow: bool = False, loss_scale: float = 1.0,
                 bucket: Optional[int] = None, pack: bool = False,
                 fuse_pack: bool = True, path: Optional[str] = None,
                 device_counter: bool = False, oneshot_min: Optional[int] = None,
                 bucket_streams: int = 2, device="cuda"):
        self.n, self.P = int(n), int(P)
        self.lr, self.beta1, self.beta2, self.eps, self.wd = lr, beta1, beta2, eps, weight_decay
        self.max_norm, self.check_overflow = float(max_norm), bool(check_overflow)
        self.inv_scale = B.zero_inv_scale(P, loss_scale)
        self.bucket = int(bucket) if bucket else None
        if self.bucket is not None and self.bucket % 32:
            raise ValueError("buckets must be multiples of 32 elements")
        # grad_dtype: torch.float32, torch.bfloat16, or "mxfp8" (replicas given
        # as (codes, scales) pairs; only the reduce pass reads them, so the
        # gradient is always materialised)
        self.mx_grads = grad_dtype == "mxfp8"
        g_b = 4 if grad_dtype == torch.float32 else 2
        if self.mx_grads and self.n % 32:
            raise ValueError("MXFP8 gradients need n % 32 == 0")
        self.path = path = choose_path(self.P, g_b, self.gated, self.mx_grads, path)
        dev = torch.device(device)
        self.master = torch.empty(self.n, dtype=torch.float32, device=dev)
        self.m = torch.zeros(self.n, dtype=torch.float32, device=dev)
        self.v = torch.zeros(self.n, dtype=torch.float32, device=dev)
        self.param = torch.empty(self.n, dtype=torch.int16, device=dev)   # bf16 bits
        self.g = (torch.empty(self.n, dtype=torch.float32, device=dev)
                  if path == "materialize" else None)
        self.acc = B.new_norm_acc(1, dev)
        # The reduce's one-shot workspace, for launches above oneshot_min
        # elements (default ONESHOT_MIN): zeroed here, left zeroed by every
        # reduce call (so a recorded graph replays without clearing it).
        self.reduce_ws = B.new_reduce_workspace(dev)
        self.oneshot_min = ONESHOT_MIN if oneshot_min is None else int(oneshot_min)
        # Bucket reduces alternate over this many streams (same priority),
        # joined before the update: a bucket's launch ramps up while the
        # previous one drains (the 7B shard's 35 buckets of 25e6: 3.10 ms
        # against 3.21 on one stream, measured in one process on MI355X).
        # The integer norm sums make the order of the buckets' atomic adds
        # irrelevant.
        if bucket_streams not in (1, 2):
            raise ValueError("bucket_streams is 1 or 2")
        self.bucket_streams = bucket_streams if self.bucket is not None else 1
        self._side = torch.cuda.Stream(device=dev) if self.bucket_streams == 2 else None
        # the side stream's buckets get their own one-shot workspace: calls
        # that share one must not run concurrently
        self._side_ws = B.new_reduce_workspace(dev) if self._side is not None else None
        self.skipped = torch.zeros(1, dtype=torch.int32, device=dev)
        self._skip_host = torch.zeros(1, dtype=torch.int32, pin_memory=True)
        self._skip_event = None
        self.t = 0
        self.device_counter = bool(device_counter)
        self.t_dev = (torch.zeros(1, dtype=torch.int64, device=dev)
                      if self.device_counter else None)
        self.pack = pack
        self.fuse_pack = bool(pack and fuse_pack)
        if pack:
            if self.n % 32:
                raise ValueError("MXFP8 packing needs n % 32 == 0")
            self.mx_elem = torch.empty(self.n, dtype=torch.uint8, device=dev)
            self.mx_scale = torch.empty(self.n // 32, dtype=torch.uint8, device=dev)

    @property
    def gated(self) -> bool:
        return self.max_norm > 0 or self.check_overflow

    def _ranges(self):
        if self.bucket is None:
            yield 0, self.n
        else:
            for lo in range(0, self.n, self.bucket):
                yield lo, min(self.n, lo + self.bucket)

    def reduce(self, replicas: List[torch.Tensor]) -> None:
        """Clear the accumulator and run the reduce/norm pass(es).  The fused
        path (no gate) has none: its single pass reduces inside AdamW and
        reads no accumulator."""
        if self.path == "fused":
            return
        B.zero_norm_acc_clear(self.acc)
        if self._side is None:
            for lo, hi in self._ranges():
                self._reduce_range(replicas, lo, hi)
            return
        main = torch.cuda.current_stream(self.master.device)
        self._side.wait_stream(main)
        for i, (lo, hi) in enumerate(self._ranges()):
            with torch.cuda.stream(self._side if i % 2 else main):
                self._reduce_range(replicas, lo, hi, self._side_ws if i % 2 else self.reduce_ws)
        main.wait_stream(self._side)

    def _reduce_range(self, replicas, lo: int, hi: int, ws=None) -> None:
        """One reduce launch over [lo, hi) on the current stream; ranges above
        oneshot_min take the one-shot form with workspace `ws`."""
        ws = self.reduce_ws if ws is None else ws
        g = self.g[lo:hi] if self.path == "materialize" else None
        oneshot = hi - lo > self.oneshot_min
        if self.mx_grads:
            codes = [c[lo:hi] for c, _ in replicas]
            scales = [sc[lo // 32:hi // 32] for _, sc in replicas]
            if oneshot:
                B.zero_shard_reduce_mx_ws(codes, scales, self.inv_scale, ws, g_out=g,
                                          acc=self.acc)
            else:
                B.zero_shard_reduce_mx(codes, scales, self.inv_scale, g_out=g, acc=self.acc)
            return
        views = [r[lo:hi] for r in replicas]
        if oneshot:
            B.zero_shard_reduce_ws(views, self.inv_scale, ws, g_out=g, acc=self.acc)
        else:
            B.zero_shard_reduce(views, self.inv_scale, g_out=g, acc=self.acc)

    def _resolve_pending_skip(self) -> None:
        if self._skip_event is not None:
            self._skip_event.synchronize()
            self._skip_event = None
            if int(self._skip_host[0]) == 0:
                self.t += 1

    def update(self, replicas: Optional[List[torch.Tensor]] = None,
               accs: Optional[torch.Tensor] = None) -> None:
        """AdamW on the shard; `accs` (k, 16) replaces the own accumulator when
        the global norm state includes other ranks."""
        self._resolve_pending_skip()
        kw = dict(step=self.t + 1, lr=self.lr, beta1=self.beta1, beta2=self.beta2,
                  eps=self.eps, weight_decay=self.wd, param_bf16=self.param,
                  max_norm=self.max_norm, check_overflow=self.check_overflow)
        if self.gated:
            kw["accs"] = self.acc if accs is None else accs
        if self.check_overflow:
            kw["skipped_out"] = self.skipped
        if self.fuse_pack:
            kw["mx_elem_out"], kw["mx_scale_out"] = self.mx_elem, self.mx_scale
        if self.device_counter:
            kw["step_dev"] = self.t_dev
        if self.path == "materialize":
            B.zero_adamw_step(self.master, self.m, self.v, grad_f32=self.g, **kw)
        else:
            B.zero_adamw_step(self.master, self.m, self.v, replicas=replicas,
                              inv_scale=self.inv_scale, **kw)
        if self.device_counter:
            return
        if self.check_overflow:
            self._skip_host.copy_(self.skipped, non_blocking=True)
            self._skip_event = torch.cuda.Event()
            self._skip_event.record()
        else:
            self.t += 1

    def pack_param(self) -> None:
        B.zero_mxfp8_pack(self.param, self.mx_elem, self.mx_scale)

    def step(self, replicas: List[torch.Tensor], accs: Optional[torch.Tensor] = None) -> None:
        """One whole step: reduce (+ norm), gated AdamW, bf16 param, and the
        MXFP8 pack of the param shard when enabled (by default inside the
        AdamW pass; with fuse_pack=False as a separate pass over the param)."""
        self.reduce(replicas)
        self.update(replicas, accs)
        if self.pack and not self.fuse_pack:
            self.pack_param()

    def set_counter(self, device: bool) -> None:
        """Move the count of applied updates between host and device memory
        (waits for the work queued so far)."""
        if device == self.device_counter:
            return
        if device:
            self._resolve_pending_skip()
            if self.t_dev is None:
                self.t_dev = torch.zeros(1, dtype=torch.int64, device=self.master.device)
            self.t_dev.fill_(self.t)
        else:
            self.t = int(self.t_dev.item())
        self.device_counter = device

    def capture(self, replicas: List[torch.Tensor],
                accs: Optional[torch.Tensor] = None) -> "torch.cuda.CUDAGraph":
        """Record one whole step (accumulator clear, reduce, gated AdamW with
        the device counter, MXFP8 pack) as a graph; each `replay()` is one
        step on the current contents of the same replica buffers.  Recording
        runs nothing.  Needs device_counter=True (no host state per step)."""
        if not self.device_counter:
            raise ValueError("capture() needs device_counter=True")
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.step(replicas, accs)
        return graph

    def step_unfused(self, replicas: List[torch.Tensor],
                     other_accs: Optional[torch.Tensor] = None) -> None:
        """The same step as `step`, as the chain of single-operation kernels
        (one HBM round trip per operation): the unfused baseline.  Results are
        bit for bit those of `step`."""
        need = B.zero_unfused_workspace_bytes(
            self.n, 0 if other_accs is None else other_accs.numel() // B.ACC_WORDS)
        ws = getattr(self, "_unfused_ws", None)
        if ws is None or ws.numel() < need:
            ws = self._unfused_ws = torch.empty(need, dtype=torch.uint8, device=self.master.device)
        self._resolve_pending_skip()
        kw = dict(step=self.t + 1, lr=self.lr, beta1=self.beta1, beta2=self.beta2,
                  eps=self.eps, weight_decay=self.wd, param_bf16=self.param,
                  max_norm=self.max_norm, check_overflow=self.check_overflow,
                  replicas=replicas, inv_scale=self.inv_scale, accs=other_accs)
        if self.check_overflow:
            kw["skipped_out"] = self.skipped
        if self.pack:
            kw["mx_elem_out"], kw["mx_scale_out"] = self.mx_elem, self.mx_scale
        if self.device_counter:
            raise ValueError("the unfused chain takes the host step counter")
        B.zero_adamw_step_unfused(self.master, self.m, self.v, ws, **kw)
        if self.check_overflow:
            self._skip_host.copy_(self.skipped, non_blocking=True)
            self._skip_event = torch.cuda.Event()
            self._skip_event.record()
        else:
            self.t += 1

    def state(self) -> dict:
        """A checkpoint of the optimizer state: host copies of master, m, v and
        the bf16 param, and the count of applied updates (waits for the work
        queued so far).  The MXFP8 outputs are not state: every step rewrites
        them from the param."""
        t = self.applied_steps()
        torch.cuda.synchronize(self.master.device)
        return {"master": self.master.cpu(), "m": self.m.cpu(), "v": self.v.cpu(),
                "param": self.param.cpu(), "t": t}

    def load_state(self, state: dict) -> None:
        """Restore a checkpoint taken by state() (same shard length): the
        next step continues exactly where the saved run stood."""
        for name in ("master", "m", "v", "param"):
            src = state[name]
            dst = getattr(self, name)
            if src.numel() != dst.numel():
                raise ValueError(f"{name}: checkpoint holds {src.numel()} elements, "
                                 f"the shard {dst.numel()}")
            dst.copy_(src.view(dst.dtype) if src.dtype != dst.dtype else src)
        self._skip_event = None
        self.t = int(state["t"])
        if self.device_counter:
            self.t_dev.fill_(self.t)

    def applied_steps(self) -> int:
        """Applied updates so far (waits for the last skip flag, or reads the
        device counter)."""
        if self.device_counter:
            return int(self.t_dev.item())
        self._resolve_pending_skip()
        return self.t

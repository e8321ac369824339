"""The five synthetic workloads of the optimizer step, with their sizes, value
distributions and step schedules.  Each is stand-in data of the shape the
ZeRO material's running examples imply; no dataset is involved.

Stream 0 of a workload is the initial fp32 master vector (sigma 0.02); stream 1
holds the gradient replicas, keyed by (1-based call index, replica k) and
indexed by the global element index of the flat vector, so rank r's shard is
elements [r*S, (r+1)*S).  Readings of unstated details:
  - "~N(0, s)" gives the standard deviation s;
  - hyperparameters the later workloads leave open reuse the first one's
    (lr 1e-3, betas (0.9, 0.999), eps 1e-8, weight decay 0.01);
  - every multi-step workload draws fresh gradients at every call;
  - "1.3B" is exactly 1 300 000 000;
  - the injected overflow of the 1.3B case is +inf (bf16 0x7F80) at element
    floor(N/3) of call 5, so 9 of its 10 calls apply an update;
  - the 7B and 30B cases simulate rank 0 only, so their global norm and
    overflow flag are rank 0's own.
"""
from dataclasses import dataclass
from typing import Optional, Tuple

from . import make_spec


@dataclass(frozen=True)
class Workload:
    name: str
    title: str
    N: int                      # full flat vector length
    P: int                      # data-parallel replicas
    S: int                      # this rank's shard length
    grad_bf16: bool
    grad_sigma: float
    steps: int
    max_norm: float = 0.0       # <= 0: no clipping
    check_overflow: bool = False
    outlier_rate: float = 0.0
    outlier_mult: float = 100.0
    loss_scale: float = 1.0
    master_sigma: float = 0.02
    bucket: Optional[int] = None
    pack: bool = False
    mx_grads: bool = False      # replicas stored as MXFP8 (codes + E8M0 scales)
    inject: Optional[Tuple[int, int]] = None   # (1-based call, element)
    rank: int = 0
    cfg_id: int = 0
    seed: int = 0
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    wd: float = 0.01

    @property
    def gated(self) -> bool:
        return self.max_norm > 0 or self.check_overflow

    @property
    def g_bytes(self) -> int:
        return 2 if self.grad_bf16 else 4

    def master_spec(self):
        return make_spec(self.seed, self.cfg_id, 0, 0, 0, self.master_sigma)

    def grad_spec(self, call: int, replica: int):
        return make_spec(self.seed, self.cfg_id, 1, call, replica, self.grad_sigma,
                         self.outlier_rate, self.outlier_mult, self.loss_scale)

    def shard_start(self, rank: Optional[int] = None) -> int:
        r = self.rank if rank is None else rank
        return r * self.S


FLAT_1M = Workload(
    "flat-1m-p4", "flat N=1,048,576, P=4 fp32 replicas, rank-0 shard, 1 step",
    N=1_048_576, P=4, S=262_144, grad_bf16=False, grad_sigma=1e-2, steps=1, cfg_id=1)
GPT2_SMALL = Workload(
    "gpt2-small-p8", "GPT-2-small-sized N=124,439,808, P=8 bf16 replicas with 1% x100 "
    "outliers, shard N/8, 10 steps, clip 1.0",
    N=124_439_808, P=8, S=15_554_976, grad_bf16=True, grad_sigma=1e-3,
    steps=10, max_norm=1.0, outlier_rate=0.01, cfg_id=2)
UNSHARDED_1P3B = Workload(
    "1.3b-unsharded", "1.3B unsharded P=1, bf16 grads x65536 loss scale, 10 calls, "
    "overflow check with one injected inf",
    N=1_300_000_000, P=1, S=1_300_000_000, grad_bf16=True, grad_sigma=1e-3,
    steps=10, check_overflow=True, loss_scale=65536.0,
    inject=(5, 1_300_000_000 // 3), cfg_id=3)
SHARD_7B = Workload(
    "7b-shard-p8", "7B model, rank-0 shard of 875M at P=8, 8 bf16 replicas in 25M "
    "buckets, 10 steps, clip 1.0",
    N=7_000_000_000, P=8, S=875_000_000, grad_bf16=True, grad_sigma=1e-3,
    steps=10, max_norm=1.0, bucket=25_000_000, cfg_id=4)
SHARD_30B = Workload(
    "30b-shard-p8", "30B model ZeRO-3, rank-0 shard of 3.75B at P=8, 8 bf16 replicas, "
    "clip 1.0 + overflow check, 5 steps, then MXFP8 pack",
    N=30_000_000_000, P=8, S=3_750_000_000, grad_bf16=True, grad_sigma=1e-3,
    steps=5, max_norm=1.0, check_overflow=True, pack=True, cfg_id=5)

# The 30B shard with its gradient replicas stored as MXFP8 (the bf16 replicas
# of the 30B shard above, packed): the stored-state saving of the pages' MXFP8
# item.
SHARD_30B_MX = Workload(
    "30b-shard-p8-mxgrads", "30B model ZeRO-3, rank-0 shard of 3.75B at P=8, 8 MXFP8-stored "
    "grad replicas, clip 1.0 + overflow check, 5 steps, MXFP8 param pack",
    N=30_000_000_000, P=8, S=3_750_000_000, grad_bf16=True, grad_sigma=1e-3,
    steps=5, max_norm=1.0, check_overflow=True, pack=True, mx_grads=True, cfg_id=5)

ALL = {w.name: w for w in (FLAT_1M, GPT2_SMALL, UNSHARDED_1P3B, SHARD_7B, SHARD_30B,
                            SHARD_30B_MX)}

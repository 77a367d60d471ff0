"""Workload shapes for the multi-round dropless MoE layer forward.

Each workload fixes the layer shape (T tokens, d_model, d_ff, E experts,
top-k), the per-expert capacity C of one round, the element type of the
activations and weights, and how the router logits are skewed. Capacity and
the skew come from the workload definitions, not from the pages: the pages
(MAI-Base-2 pre-training write-up, section "Scaling MoE") only say that the
per-expert capacity is fixed and tunable and that overflow goes to extra
rounds.
"""
from __future__ import annotations

import dataclasses
import math


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d_model: int
    d_ff: int
    E: int
    k: int
    C: int
    dtype: str  # "f32" or "bf16"
    # logit skew: ("none",), ("zipf", s) -> b_e = s*log(1/(e+1)), ("hot", e0, b)
    skew: tuple = ("none",)
    seed: int = 0
    sweep_C: tuple = ()

    def with_C(self, C: int) -> "Workload":
        return dataclasses.replace(self, C=int(C))

    def with_T(self, T: int) -> "Workload":
        return dataclasses.replace(self, T=int(T))

    @property
    def flops(self) -> int:
        """Algorithmic FLOPs of the expert FFNs: 6*T*k*d*f (gate, up, down)."""
        return 6 * self.T * self.k * self.d_model * self.d_ff


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


TINY_F32 = Workload("tiny_f32", T=512, d_model=64, d_ff=128, E=8, k=2, C=64,
                    dtype="f32")
BALANCED_BF16 = Workload("balanced_bf16", T=8192, d_model=2048, d_ff=1024,
                         E=32, k=4, C=_ceil_div(8192 * 4, 32), dtype="bf16")
SKEWED_BF16 = dataclasses.replace(BALANCED_BF16, name="skewed_bf16",
                                  skew=("zipf", 1.2))
FRONTIER_SHARE_BF16 = Workload("frontier_share_bf16", T=16384, d_model=7168,
                               d_ff=2048, E=64, k=6,
                               C=_ceil_div(16384 * 6, 64), dtype="bf16",
                               skew=("zipf", 0.8))
HOT_EXPERT_BF16 = Workload("hot_expert_bf16", T=32768, d_model=4096,
                           d_ff=1536, E=64, k=8,
                           C=_ceil_div(32768 * 8, 2 * 64), dtype="bf16",
                           skew=("hot", 0, 10.0),
                           sweep_C=(256, 1024, 2048, 4096, 32768))

WORKLOADS = {w.name: w for w in (TINY_F32, BALANCED_BF16, SKEWED_BF16,
                                 FRONTIER_SHARE_BF16, HOT_EXPERT_BF16)}

# the workload the throughput line is quoted on: the largest that fits one
# GPU (the training-step benchmark keeps the balanced layer)
BENCH_WORKLOAD = HOT_EXPERT_BF16
BACKWARD_BENCH_WORKLOAD = BALANCED_BF16

assert math.isclose(BALANCED_BF16.C, 1024)
assert FRONTIER_SHARE_BF16.C == 1536 and HOT_EXPERT_BF16.C == 2048

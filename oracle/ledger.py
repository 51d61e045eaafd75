"""Training-state bytes per parameter under data parallelism and ZeRO stages.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The ledger of mixed-precision Adam training ("CS336 2026 Lecture 8:
Parallelism Basics", Slide 17; "并行策略总览：六个维度各切什么、怎么通信",
data-parallel section): a 16-bit parameter (2 B), a 16-bit gradient (2 B),
an fp32 master copy (4 B) and Adam's first and second moments (4 B each),
16 bytes per parameter in all.  ZeRO shards these over the N data-parallel
ranks stage by stage (Lecture 8, ZeRO stage table and Slides 19-25):
stage 1 shards the optimizer state (master, m, v), stage 2 also the
gradients, stage 3 also the parameters.
"""
from __future__ import annotations

import dataclasses


@dataclasses.dataclass(frozen=True)
class Ledger:
    param: float        # bytes per parameter of the working (16-bit) weights
    grad: float         # bytes per parameter of the gradient
    optimizer: float    # bytes per parameter of optimizer state (master + m + v)

    @property
    def total(self) -> float:
        return self.param + self.grad + self.optimizer

    def per_rank_bytes_per_param(self, stage: int, n_ranks: int) -> float:
        """Bytes each rank holds per model parameter.  stage 0 = plain DP."""
        p, g, o, n = self.param, self.grad, self.optimizer, float(n_ranks)
        if stage == 0:
            return p + g + o
        if stage == 1:
            return p + g + o / n
        if stage == 2:
            return p + (g + o) / n
        if stage == 3:
            return (p + g + o) / n
        raise ValueError(stage)

    def max_params(self, hbm_bytes: float, stage: int, n_ranks: int) -> float:
        """Largest model whose training state fits one rank's memory."""
        return hbm_bytes / self.per_rank_bytes_per_param(stage, n_ranks)


# bf16 parameter + bf16 gradient + fp32 master, m, v.
MIXED_PRECISION_ADAM = Ledger(param=2, grad=2, optimizer=4 + 4 + 4)

# Everything but the fp32 master in bf16: 2 + 2 + (4 master + 2 m + 2 v).
BF16_MOMENTS_ADAM = Ledger(param=2, grad=2, optimizer=4 + 2 + 2)

# Pure bf16 with a compensated update: bf16 parameter (the only weight copy),
# gradient, m, v and Kahan compensation; no fp32 master.
PURE_BF16_KAHAN = Ledger(param=2, grad=2, optimizer=2 + 2 + 2)

# Element sizes of the arrays the shard step reads and writes: bf16 param
# slot, bf16 gradient partial, fp32 master, fp32 m, fp32 v.
STATE_ELEMENT_BYTES = {"param": 2, "grad": 2, "master": 4, "m": 4, "v": 4}


def shard_step_bytes_per_param(n_ranks: int, grad_bytes: int = 2, moment_bytes: int = 4) -> int:
    """HBM bytes the fused step must move per shard element: read N gradient
    partials and the master, m, v; write master, m, v and the 16-bit
    parameter.  moment_bytes = 2 for the 12-byte ledger's bf16 moments."""
    s = STATE_ELEMENT_BYTES
    return n_ranks * grad_bytes + 2 * (s["master"] + 2 * moment_bytes) + s["param"]


def unfused_step_bytes_per_param(n_ranks: int, grad_bytes: int = 2) -> int:
    """HBM bytes per shard element when the three phases run as separate
    passes with an fp32 gradient shard between them ("并行训练优化、MoE扩展与系统瓶颈",
    2.2.4: reduce-scatter, then the optimizer step on the shard, then the
    all-gather): the reduce reads N partials and writes the gradient; the
    optimizer step reads the gradient and master, m, v and writes master, m,
    v; the parameter write reads the master again and writes the 16-bit
    parameter."""
    s = STATE_ELEMENT_BYTES
    g32 = 4
    reduce_pass = n_ranks * grad_bytes + g32
    adam_pass = g32 + 2 * (s["master"] + s["m"] + s["v"])
    write_pass = s["master"] + s["param"]
    return reduce_pass + adam_pass + write_pass


def kahan_step_bytes_per_param(n_ranks: int, grad_bytes: int = 2) -> int:
    """HBM bytes of the fused pure-bf16 step per shard element: N gradient
    partials read; parameter, compensation, m, v (bf16 each) read and
    written."""
    return n_ranks * grad_bytes + 2 * (2 + 2 + 2 + 2)


# ---- communication volumes ---------------------------------------------------
# Ring collectives over a buffer of M elements on n ranks ("并行策略总览：六个维度
# 各切什么、怎么通信", collectives table): all-reduce sends 2(n-1)M/n elements per
# rank, reduce-scatter, all-gather and all-to-all (n-1)M/n; and all-reduce =
# reduce-scatter + all-gather.

RING_FACTOR = {"all-reduce": 2, "reduce-scatter": 1, "all-gather": 1, "all-to-all": 1}


def ring_volume(collective: str, n_ranks: int, m: float) -> float:
    """Elements each rank sends in a ring `collective` over m elements."""
    return RING_FACTOR[collective] * (n_ranks - 1) * m / n_ranks


def step_volume(stage: int, n_ranks: int, psi: float) -> float:
    """Elements each rank sends per optimizer step for a model of psi
    parameters (same page, data-parallel section): plain data parallelism
    all-reduces the gradient; ZeRO-1/2 reduce-scatter it and all-gather the
    updated parameters, the same volume (about 2 psi); ZeRO-3 also
    all-gathers the parameters a second time, for the backward pass (about
    3 psi)."""
    rs = ring_volume("reduce-scatter", n_ranks, psi)
    ag = ring_volume("all-gather", n_ranks, psi)
    if stage == 0:
        return ring_volume("all-reduce", n_ranks, psi)
    if stage in (1, 2):
        return rs + ag
    if stage == 3:
        return rs + 2 * ag
    raise ValueError(stage)

"""Tensor-list shapes and input recipes of the shard-step workloads.

Each workload is a list of parameter-tensor sizes (flattened, in model order),
a number of data-parallel ranks N, the gradient-partial dtype, and the
distribution parameters of the synthetic inputs.  The flat concatenation of
the tensor list is cut into N equal contiguous shards (the last one shorter
when N does not divide the total); a shard cuts across tensor boundaries.

Shapes follow the model families named for the workloads (GPT-2 small,
Llama-7B, Llama-70B with grouped-query attention) and a seeded ragged list.
No weights or data are involved: everything is synthetic and seeded.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Tuple

import numpy as np

from . import KIND_RAGGED_SIZE, KIND_ZERO_TENSOR, stream_id, uniform

SEED_BASE = 0x5EED0000


@dataclasses.dataclass
class Workload:
    name: str
    config_id: int
    numels: List[int]
    n_ranks: int
    gdt: str                       # "bf16" or "f32" gradient partials
    sigma_grad: float
    sigma_master: float = 0.02
    outlier_frac: float = 0.0
    outlier_mult: float = 1.0
    zero_tensors: Tuple[int, ...] = ()   # tensors whose gradient partials are all zero
    steps: int = 10
    warm_prefix: int = 0           # >0: m, v warm-started on this many leading shard elements
    warm_steps: int = 0
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.1

    @property
    def seed(self) -> int:
        return SEED_BASE + self.config_id

    @property
    def total(self) -> int:
        return int(sum(self.numels))

    @property
    def shard_len(self) -> int:
        return -(-self.total // self.n_ranks)

    def shard_range(self, rank: int) -> Tuple[int, int]:
        s = self.shard_len
        lo = min(rank * s, self.total)
        return lo, min(lo + s, self.total)

    def bytes_per_param(self) -> int:
        """Algorithmic HBM bytes per shard element of the fused step."""
        g = 2 if self.gdt == "bf16" else 4
        return g * self.n_ranks + 26

    def hparams(self) -> dict:
        return dict(lr=self.lr, beta1=self.beta1, beta2=self.beta2, eps=self.eps,
                    weight_decay=self.weight_decay)


def gpt2_small_numels() -> List[int]:
    d, ff, vocab, ctx, layers = 768, 3072, 50257, 1024, 12
    out = [vocab * d, ctx * d]                      # wte, wpe
    for _ in range(layers):
        out += [d, d,                               # ln_1 weight, bias
                d * 3 * d, 3 * d,                   # attn qkv weight, bias
                d * d, d,                           # attn proj weight, bias
                d, d,                               # ln_2 weight, bias
                d * ff, ff,                         # mlp fc weight, bias
                ff * d, d]                          # mlp proj weight, bias
    out += [d, d]                                   # ln_f weight, bias
    return out


def llama_numels(d: int, layers: int, ff: int, vocab: int, kv_dim: Optional[int] = None) -> List[int]:
    kv = d if kv_dim is None else kv_dim
    out = [vocab * d]                               # token embedding
    for _ in range(layers):
        out += [d,                                  # attention norm
                d * d, d * kv, d * kv, d * d,       # q, k, v, o
                d,                                  # ffn norm
                d * ff, d * ff, ff * d]             # gate, up, down
    out += [d, vocab * d]                           # final norm, lm_head
    return out


def ragged_numels(seed: int, n: int = 1200, lo: int = 64, hi: int = 64 << 20,
                  total: int = 2_000_000_000) -> List[int]:
    """Log-uniform sizes in [lo, hi], rescaled so the sum is exactly `total`.

    Raw log-uniform draws over [64, 64M] average ~4.8M, so 1,200 of them sum
    to ~5.8B; they are scaled by total/sum, rounded, clamped at lo, and the
    rounding residual goes to the largest tensor.  Odd sizes are kept.
    """
    u = uniform(seed, stream_id(KIND_RAGGED_SIZE), np.arange(n)).astype(np.float64)
    raw = lo * (hi / lo) ** u
    sizes = np.maximum(np.rint(raw * (total / raw.sum())).astype(np.int64), lo)
    sizes[int(np.argmax(sizes))] += total - int(sizes.sum())
    assert int(sizes.sum()) == total and int(sizes.min()) >= lo
    return [int(x) for x in sizes]


def ragged_zero_tensors(seed: int, numels: List[int], n_ranks: int, frac: float = 0.05) -> Tuple[int, ...]:
    """About `frac` of the tensors get all-zero gradients (by tensor hash); the
    tensor that straddles the rank-0/rank-1 shard boundary is always one."""
    u = uniform(seed, stream_id(KIND_ZERO_TENSOR), np.arange(len(numels)))
    zs = set(int(t) for t in np.nonzero(u < frac)[0])
    s = -(-sum(numels) // n_ranks)
    starts = np.cumsum([0] + numels[:-1])
    for t, (a, n) in enumerate(zip(starts, numels)):
        if a < s < a + n:
            zs.add(t)
            break
    return tuple(sorted(zs))


def tiny() -> Workload:
    return Workload("tiny", 0, [1 << 20], 4, "bf16", 1e-3, steps=10)


def gpt2() -> Workload:
    return Workload("gpt2-small", 1, gpt2_small_numels(), 8, "bf16", 1e-3,
                    outlier_frac=0.01, outlier_mult=100.0, steps=20)


def llama7b() -> Workload:
    return Workload("llama-7b", 2, llama_numels(4096, 32, 11008, 32000), 8, "bf16", 1e-4,
                    steps=20, warm_prefix=1 << 20, warm_steps=100)


def llama70b() -> Workload:
    return Workload("llama-70b", 3, llama_numels(8192, 80, 28672, 128256, kv_dim=1024), 16,
                    "bf16", 1e-4, steps=1)


def ragged() -> Workload:
    seed = SEED_BASE + 4
    numels = ragged_numels(seed)
    return Workload("ragged-fp32", 4, numels, 32, "f32", 1e-4,
                    zero_tensors=ragged_zero_tensors(seed, numels, 32), steps=3)


ALL = {"tiny": tiny, "gpt2": gpt2, "llama7b": llama7b, "llama70b": llama70b, "ragged": ragged}


def get(name: str) -> Workload:
    return ALL[name]()


def zero_ranges(w: Workload, lo: int, hi: int) -> List[Tuple[int, int]]:
    """Shard-relative [a, b) ranges of [lo, hi) whose gradients are all zero."""
    out = []
    start = 0
    zs = set(w.zero_tensors)
    for t, n in enumerate(w.numels):
        a, b = start, start + n
        start = b
        if t in zs and b > lo and a < hi:
            out.append((max(a, lo) - lo, min(b, hi) - lo))
    return out


def zero_mask(w: Workload, flat_idx: np.ndarray) -> np.ndarray:
    """True where a global flat index lies in a tensor with all-zero gradients."""
    if not w.zero_tensors:
        return np.zeros(np.shape(flat_idx), dtype=bool)
    starts = np.cumsum([0] + w.numels[:-1])
    t = np.searchsorted(starts, flat_idx, side="right") - 1
    return np.isin(t, np.asarray(w.zero_tensors))

"""The named workloads (shapes, masks, dtypes, seeds).

Layout everywhere is contiguous BHSD: q, k, v, o are [B, H, N, d] with d fastest; lse is [B, H, Nq].
A "ring share" workload is one device's part of Ring Attention: a local query shard attended against a list of
key/value blocks, each with its own global position offset. "Striped" assigns token t to stripe t mod W, so local
row i of stripe r sits at global position W*i + r.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Tuple


@dataclass(frozen=True)
class Config:
    key: str
    seed: int
    description: str
    B: int
    H: int
    Nq: int
    d: int
    dtype: str                      # "f32" or "bf16" (inputs; accumulation is always fp32)
    causal: bool
    stride: int = 1                 # global position step between adjacent local rows
    q_off: int = 0                  # global position of local query row 0
    blocks: Tuple[Tuple[int, int], ...] = field(default_factory=tuple)  # (Nk, k_off) per key/value block
    global_N: int = 0               # length of the global sequence the shard was cut from (ring shares)

    @property
    def scale(self) -> float:
        return 1.0 / float(self.d) ** 0.5

    @property
    def Nk_total(self) -> int:
        return sum(n for n, _ in self.blocks)


def _tiny_f32() -> Config:
    return Config("tiny_f32", 1, "non-causal fp32, N=256, d=64; K/V also split into 4 blocks of 64 and merged",
                  B=1, H=1, Nq=256, d=64, dtype="f32", causal=False,
                  blocks=tuple((64, 64 * i) for i in range(4)), global_N=256)


def _causal_8k() -> Config:
    return Config("causal_8k", 2, "causal self-attention bf16, B=4 H=32 N=8192 d=128",
                  B=4, H=32, Nq=8192, d=128, dtype="bf16", causal=True,
                  blocks=((8192, 0),), global_N=8192)


def _causal_long(n: int, key: str) -> Config:
    return Config(key, 6, f"causal self-attention bf16 on one GPU, B=1 H=32 N={n} d=128",
                  B=1, H=32, Nq=n, d=128, dtype="bf16", causal=True, blocks=((n, 0),), global_N=n)


def _ring_rank2of4() -> Config:
    n = 32768
    return Config("ring_rank2of4_128k", 3,
                  "ring share: Q shard = global rows 65536..98303 of N=131072, 4 K/V blocks of 32768, causal",
                  B=1, H=32, Nq=n, d=128, dtype="bf16", causal=True, q_off=2 * n,
                  blocks=tuple((n, i * n) for i in range(4)), global_N=4 * n)


def striped(rank: int) -> Config:
    n = 16384
    return Config(f"striped_r{rank}_64k", 4,
                  f"striped causal: Q stripe {rank} of 4 (16384 tokens) vs 4 K/V stripes, N=65536, H=16",
                  B=1, H=16, Nq=n, d=128, dtype="bf16", causal=True, stride=4, q_off=rank,
                  blocks=tuple((n, s) for s in range(4)), global_N=4 * n)


def _tabular_rows() -> Config:
    # (batch=1, rows=150000, features=8, heads=4, head_dim=24) -> row axis: B = 8 features, H = 4 heads
    return Config("tabular_rows_150k", 5, "row-axis attention over 150000 tokens, d=24, non-causal",
                  B=8, H=4, Nq=150000, d=24, dtype="bf16", causal=False,
                  blocks=((150000, 0),), global_N=150000)


def _tabular_features() -> Config:
    # feature axis: B = 150000 rows, H = 4 heads, N = 8 features
    return Config("tabular_features_8", 5, "feature-axis attention over 8 tokens per (row, head), d=24",
                  B=150000, H=4, Nq=8, d=24, dtype="bf16", causal=False,
                  blocks=((8, 0),), global_N=8)


CONFIGS = {
    "tiny_f32": _tiny_f32(),
    "causal_8k": _causal_8k(),
    "causal_32k": _causal_long(32768, "causal_32k"),
    "causal_128k": _causal_long(131072, "causal_128k"),
    "ring_rank2of4_128k": _ring_rank2of4(),
    "striped_r0_64k": striped(0),
    "striped_r1_64k": striped(1),
    "striped_r2_64k": striped(2),
    "striped_r3_64k": striped(3),
    "tabular_rows_150k": _tabular_rows(),
    "tabular_features_8": _tabular_features(),
}


def tabular_shape() -> List[int]:
    """Input of the multi-axis workload: (batch, rows, features, heads, head_dim)."""
    return [1, 150000, 8, 4, 24]

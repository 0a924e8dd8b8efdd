"""Seeded synthetic inputs for the BitLinear workloads.

This module only draws random numbers; it holds none of the method's arithmetic
(no scales, no rounding to codes, no packing).  Both the HIP path and the CPU oracle
consume the exact bytes it produces: GPU tensors are copied to the host for the oracle.

Recipe (the workloads' shapes and distributions):
  * latent weights W[N][K] (out x in), fp32, i.i.d. N(0, sigma^2) with sigma = 0.02;
  * activations x[M][K], i.i.d. N(0, 1); an optional outlier mask draws each entry
    independently with probability p and multiplies it by a factor (x20 at p = 1 %,
    x30 at p = 0.5 %), before the cast to bf16 where the workload is bf16;
  * sub-layer normalisation gains g[K], fp32, i.i.d. uniform on [0.5, 1.5);
  * seeds: 1000 * workload + 10 * layer + matrix index for weights, +500 for activations,
    +700 for gains.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

SIGMA_W = 0.02


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def latent_weights(n: int, k: int, seed: int, device="cpu", sigma: float = SIGMA_W) -> torch.Tensor:
    """fp32 [n][k] ~ N(0, sigma^2)."""
    g = _gen(seed, device)
    w = torch.randn((n, k), generator=g, device=device, dtype=torch.float32)
    return w.mul_(sigma)


def activations(m: int, k: int, seed: int, dtype=torch.bfloat16, device="cpu",
                outlier_p: float = 0.0, outlier_mult: float = 1.0) -> torch.Tensor:
    """[m][k] ~ N(0, 1) with an i.i.d. Bernoulli(outlier_p) mask scaled by outlier_mult,
    then cast (round-to-nearest-even) to ``dtype``."""
    g = _gen(seed, device)
    x = torch.randn((m, k), generator=g, device=device, dtype=torch.float32)
    if outlier_p > 0.0:
        mask = torch.rand((m, k), generator=g, device=device) < outlier_p
        x = torch.where(mask, x * outlier_mult, x)
    return x.to(dtype)


def subln_gain(k: int, seed: int, device="cpu") -> torch.Tensor:
    """fp32 [k] ~ uniform[0.5, 1.5): a per-feature gain of the sub-layer normalisation."""
    g = _gen(seed, device)
    return torch.rand(k, generator=g, device=device, dtype=torch.float32).add_(0.5)


def weight_seed(workload: int, layer: int, matrix: int) -> int:
    return 1000 * workload + 10 * layer + matrix


def act_seed(workload: int, layer: int, matrix: int) -> int:
    return weight_seed(workload, layer, matrix) + 500


def gain_seed(workload: int, layer: int, matrix: int) -> int:
    return weight_seed(workload, layer, matrix) + 700


@dataclass
class Workload:
    """One benchmark/parity workload: a list of (name, K, N) matrices applied at M tokens."""
    index: int
    name: str
    m_list: tuple
    matrices: tuple  # ((name, K, N), ...)
    act_dtype: torch.dtype
    outlier_p: float = 0.0
    outlier_mult: float = 1.0
    layers: int = 1
    rotate_sets: int = 1  # distinct weight sets cycled through to defeat cache reuse
    notes: str = ""
    extra: dict = field(default_factory=dict)

    def packed_bytes_per_layer(self, packed_bytes) -> int:
        return sum(packed_bytes(n, k) for _, k, n in self.matrices)


WORKLOADS = {
    0: Workload(0, "single BitLinear M=1, K=256 -> N=512 (fp32 acts, 1% x20 outliers)",
                (1,), (("w", 256, 512),), torch.float32, 0.01, 20.0),
    1: Workload(1, "2B-class decode GEMV M=1: gate/up 2560->6912, down 6912->2560 (bf16 acts)",
                (1,), (("gate", 2560, 6912), ("up", 2560, 6912), ("down", 6912, 2560)),
                torch.bfloat16, rotate_sets=48),
    2: Workload(2, "2B-class full layer at M=16 decode (Q, K, V, O, gate, up, down; bf16 acts)",
                (16,), (("q", 2560, 2560), ("k", 2560, 640), ("v", 2560, 640), ("o", 2560, 2560),
                        ("gate", 2560, 6912), ("up", 2560, 6912), ("down", 6912, 2560)),
                torch.bfloat16, rotate_sets=32),
    3: Workload(3, "prefill GEMM M=2048: 2560->6912 and 6912->2560 (bf16 acts, 0.5% x30 outliers)",
                (2048,), (("up", 2560, 6912), ("down", 6912, 2560)), torch.bfloat16, 0.005, 30.0),
    4: Workload(4, "100B-class decode M=1 and M=8: 8192->28672 and 28672->8192 over 80 layers",
                (1, 8), (("up", 8192, 28672), ("down", 28672, 8192)), torch.bfloat16, layers=80),
    # one GPU's share of workload 4 split over 8 GPUs: the up projection sharded by output
    # rows (28672 / 8), the down projection by input columns (28672 / 8, partial sums)
    5: Workload(5, "100B-class one-of-8 shard, M=1 and M=8: 8192->3584 and 3584->8192 over 80 layers",
                (1, 8), (("up_shard", 8192, 3584), ("down_shard", 3584, 8192)), torch.bfloat16, layers=80),
}

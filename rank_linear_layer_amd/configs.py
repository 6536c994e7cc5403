"""Named workloads of the factorized linear layer (shapes and seeds only).

Shapes follow the Llama-3-8B projections that the low-rank pages compress
("Why Smaller Is Slower? ...", section 1 and Table 5; "LowRankArena ...",
evaluation on Llama-3.1-8B), with irregular ranks such as r = 107
(the rank that section 1 of the misalignment page reduces 128 to), 817,
1637 and 2867, and a pruned width N = 3999.

Seeds: seed_base = 1000 * workload_index + 10 * projection_index; X, A and B
take seed_base + 0, + 1, + 2 (see datagen.factorized_inputs).
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class Proj:
    name: str
    K: int
    r: int
    N: int


# Workload 0: tiny factorized linear (parity).
TINY = dict(index=0, M=16, K=512, r=107, N=512)

# Workload 0b: 64 x 48 Gaussian matrix, truncated SVD at k = 5.
EY = dict(index=0, K=64, N=48, k=5, w_seed=1, x_seed=7)

# Workload 1: Llama-3-8B-shaped q_proj at decode, misaligned rank.
QPROJ_DECODE = dict(index=1, M=8, K=4096, r=1637, N=4096)

# Workload 2: MLP up-projection at prefill.
MLP_UP_PREFILL = dict(index=2, M=4096, K=4096, r=2867, N=14336)

# Workload 3: one decoder layer of factorized projections.
LAYER_INDEX = 3
LAYER_PROJS = (
    Proj("q", 4096, 1637, 4096),
    Proj("k", 4096, 817, 1024),
    Proj("v", 4096, 817, 1024),
    Proj("o", 4096, 1637, 4096),
    Proj("gate", 4096, 2867, 14336),
    Proj("up", 4096, 2867, 14336),
    Proj("down", 14336, 2867, 4096),
)
LAYER_M = (1, 2048)

# Workload 4: alignment sweep.
SWEEP_INDEX = 4
SWEEP_K = 4096
SWEEP_N = (4096, 3999)
SWEEP_R = tuple(range(1000, 1101))
SWEEP_M = (1, 512)
# the strided subset a default benchmark run measures: stride 3, so every
# residue of r mod 8 appears twice
SWEEP_R_DEFAULT = tuple(range(1024, 1072, 3))


def seed_base(workload_index: int, projection_index: int = 0) -> int:
    return 1000 * workload_index + 10 * projection_index


def sweep_seed(N: int, r: int) -> int:
    """Distinct seed per sweep point (the M values share weights)."""
    return 1000 * SWEEP_INDEX + 100000 * (0 if N == 4096 else 1) + 10 * r

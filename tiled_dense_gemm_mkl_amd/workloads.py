"""Seeded synthetic inputs for the GEMM and RMSNorm workloads.

This module holds no GEMM or RMSNorm arithmetic.  It only draws random operands and
stores them in the operand dtype, so that the GPU path and the CPU oracle can
be fed the very same stored bits.

Recipe (one ``numpy.random.Generator(PCG64(seed))`` per workload):
  for l in 0..L-1:  draw A[l] (M*K values), then B[l] (N*K values), in binary64;
  scale as the distribution says; convert to the operand dtype with torch's
  CPU conversion (round to nearest even).  Integer-valued variants draw
  ``integers(-2, 3)`` instead, which every dtype holds exactly.

The returned arrays are the stored bits: float32 for fp32, uint16 for fp16 and
bf16, shaped A [L, M, K] and B [L, N, K].
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

DTYPE_NAMES = ("f32", "f16", "bf16")


@dataclass(frozen=True)
class Workload:
    key: str          # short handle used by tests and the benchmark
    name: str         # what it is, with its sizes
    dtype: str        # "f32" | "f16" | "bf16" (A, B and C)
    M: int
    N: int
    K: int
    L: int
    epilogue: str     # "identity" | "relu" | "silu"
    dist_a: tuple     # ("uniform", lo, hi) | ("normal", std)
    dist_b: tuple
    seed: int

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K * self.L

    @property
    def algorithmic_bytes(self) -> int:
        es = 4 if self.dtype == "f32" else 2
        return es * self.L * (self.M * self.K + self.N * self.K + self.M * self.N)


_INV_SQRT_8192 = 1.0 / np.sqrt(8192.0)

WORKLOADS = {
    w.key: w
    for w in [
        Workload("f32_128x128x128_identity",
                 "fp32 GEMM M=N=K=128 L=1, identity epilogue",
                 "f32", 128, 128, 128, 1, "identity",
                 ("uniform", -1.0, 1.0), ("uniform", -1.0, 1.0), 1),
        Workload("f32_128x2048x2048_relu",
                 "fp32 GEMM M=128 N=2048 K=2048 L=1 (128-token block x 2048x2048 projection), ReLU",
                 "f32", 128, 2048, 2048, 1, "relu",
                 ("uniform", -1.0, 1.0), ("uniform", -1.0, 1.0), 2),
        Workload("bf16_512x5632x2048_relu",
                 "bf16 GEMM M=512 N=5632 K=2048 L=1 (512 tokens x 2048->5632 MLP up-projection), ReLU",
                 "bf16", 512, 5632, 2048, 1, "relu",
                 ("normal", 1.0), ("normal", 0.02), 3),
        Workload("f16_8192x8192x8192_identity",
                 "fp16 GEMM M=N=K=8192 L=1, operands N(0,1)/sqrt(K), identity",
                 "f16", 8192, 8192, 8192, 1, "identity",
                 ("normal", _INV_SQRT_8192), ("normal", _INV_SQRT_8192), 4),
        Workload("bf16_L8_512x3584x18944_silu",
                 "bf16 batched GEMM L=8 M=512 N=3584 K=18944 (K-heavy down-projection), SiLU",
                 "bf16", 512, 3584, 18944, 8, "silu",
                 ("normal", 1.0), ("normal", 0.02), 5),
    ]
}

# The workload the headline throughput is quoted on.
HEADLINE = "bf16_512x5632x2048_relu"


def _draw(rng: np.random.Generator, n: int, dist: tuple, integer: bool) -> np.ndarray:
    if integer:
        return rng.integers(-2, 3, size=n).astype(np.float64)
    if dist[0] == "uniform":
        return rng.uniform(dist[1], dist[2], size=n)
    if dist[0] == "normal":
        return rng.standard_normal(size=n) * dist[1]
    raise ValueError(f"unknown distribution {dist!r}")


def to_storage(x64: np.ndarray, dtype: str) -> np.ndarray:
    """binary64 values -> stored bits of dtype (float32 or uint16 array)."""
    import torch

    if dtype == "f32":
        return np.ascontiguousarray(x64, dtype=np.float32)
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    t = torch.from_numpy(np.ascontiguousarray(x64)).to(tdt)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def random_operands(dtype: str, M: int, N: int, K: int, L: int, seed: int,
                    dist_a=("uniform", -1.0, 1.0), dist_b=("uniform", -1.0, 1.0),
                    integer: bool = False):
    """Seeded A [L,M,K] and B [L,N,K] as stored bits of dtype."""
    if dtype not in DTYPE_NAMES:
        raise ValueError(f"unknown dtype {dtype!r}")
    rng = np.random.Generator(np.random.PCG64(seed))
    store = np.float32 if dtype == "f32" else np.uint16
    A = np.empty((L, M, K), dtype=store)
    B = np.empty((L, N, K), dtype=store)
    for l in range(L):
        A[l] = to_storage(_draw(rng, M * K, dist_a, integer), dtype).reshape(M, K)
        B[l] = to_storage(_draw(rng, N * K, dist_b, integer), dtype).reshape(N, K)
    return A, B


def make_inputs(w: Workload | str, integer: bool = False):
    """Operands of a named workload (integer variants use seed + 100)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    seed = w.seed + 100 if integer else w.seed
    return random_operands(w.dtype, w.M, w.N, w.K, w.L, seed, w.dist_a, w.dist_b, integer)


@dataclass(frozen=True)
class GroupedWorkload:
    key: str
    name: str
    dtype: str
    G: int            # groups (experts), each with its own B[g] [N][K]
    total_m: int      # rows of A and C, routed to the groups
    N: int
    K: int
    epilogue: str
    dist_a: tuple
    dist_b: tuple
    seed: int

    @property
    def flops(self) -> int:
        return 2 * self.total_m * self.N * self.K

    @property
    def algorithmic_bytes(self) -> int:
        es = 4 if self.dtype == "f32" else 2
        return es * (self.total_m * self.K + self.G * self.N * self.K + self.total_m * self.N)


GROUPED_WORKLOADS = {
    w.key: w
    for w in [
        GroupedWorkload(
            "grouped_bf16_G8_4096x5632x2048_relu",
            "bf16 grouped GEMM, 4096 rows routed to 8 groups (own 5632x2048 B each), ReLU",
            "bf16", 8, 4096, 5632, 2048, "relu", ("normal", 1.0), ("normal", 0.02), 6),
    ]
}


def group_sizes(G: int, total_m: int, seed: int) -> np.ndarray:
    """Seeded uneven split of total_m rows over G groups: every row picks a
    group with probabilities drawn from a Dirichlet(1) (so some groups are far
    larger than others, and a group can be empty)."""
    rng = np.random.Generator(np.random.PCG64(seed + 1000))
    p = rng.dirichlet(np.ones(G))
    return rng.multinomial(total_m, p).astype(np.int64)


def make_grouped_inputs(w: GroupedWorkload | str, integer: bool = False):
    """A [total_m, K], B [G, N, K] (stored bits) and int32 cumulative row ends."""
    if isinstance(w, str):
        w = GROUPED_WORKLOADS[w]
    seed = w.seed + 100 if integer else w.seed
    A, _ = random_operands(w.dtype, w.total_m, 1, w.K, 1, seed, w.dist_a, w.dist_b, integer)
    _, B = random_operands(w.dtype, 1, w.N, w.K, w.G, seed + 1, w.dist_a, w.dist_b, integer)
    offs = np.cumsum(group_sizes(w.G, w.total_m, w.seed)).astype(np.int32)
    return A[0], B, offs


@dataclass(frozen=True)
class RmsNormWorkload:
    key: str
    name: str
    dtype: str        # x, weight and y
    rows: int
    hidden: int
    eps: float
    weight: tuple     # ("ones",) | ("normal", mean, std)
    seed: int

    @property
    def algorithmic_bytes(self) -> int:
        """x read once, y written once, the weight read once."""
        es = 4 if self.dtype == "f32" else 2
        return es * (2 * self.rows * self.hidden + self.hidden)


RMSNORM_WORKLOADS = {
    w.key: w
    for w in [
        RmsNormWorkload(
            "rmsnorm_f32_32x2048",
            "fp32 RMSNorm(2048) over 32 rows of N(0,1), unit weight, eps 1e-6 (the compiler page's example)",
            "f32", 32, 2048, 1e-6, ("ones",), 7),
        RmsNormWorkload(
            "rmsnorm_f32_65536x2048",
            "fp32 RMSNorm(2048) over 65536 rows of N(0,1), weight 1 + N(0,0.1^2), eps 1e-6",
            "f32", 65536, 2048, 1e-6, ("normal", 1.0, 0.1), 8),
        RmsNormWorkload(
            "rmsnorm_bf16_65536x3584",
            "bf16 RMSNorm(3584) over 65536 rows of N(0,1), weight 1 + N(0,0.1^2), eps 1e-6",
            "bf16", 65536, 3584, 1e-6, ("normal", 1.0, 0.1), 9),
    ]
}


def make_rms_inputs(w: RmsNormWorkload | str, rows: int | None = None):
    """x [rows, hidden] ~ N(0, 1) and the weight [hidden], as stored bits.
    The weight is drawn first, then the rows in order, so a prefix of the rows
    (rows < w.rows) is the same prefix of the full input."""
    if isinstance(w, str):
        w = RMSNORM_WORKLOADS[w]
    rows = w.rows if rows is None else rows
    rng = np.random.Generator(np.random.PCG64(w.seed))
    if w.weight[0] == "ones":
        wt = np.ones(w.hidden)
    else:
        wt = w.weight[1] + w.weight[2] * rng.standard_normal(w.hidden)
    x = rng.standard_normal((rows, w.hidden))
    return to_storage(x, w.dtype), to_storage(wt, w.dtype)


def storage_to_torch(x: np.ndarray, dtype: str):
    """View stored bits as a torch CPU tensor of the operand dtype (no copy)."""
    import torch

    t = torch.from_numpy(x)
    if dtype == "f32":
        return t
    return t.view(torch.int16).view(torch.float16 if dtype == "f16" else torch.bfloat16)


def torch_to_storage(t) -> np.ndarray:
    """torch tensor (any device) of fp32/fp16/bf16 -> stored bits on the host."""
    import torch

    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.float32:
        return t.numpy()
    return t.view(torch.int16).numpy().view(np.uint16)

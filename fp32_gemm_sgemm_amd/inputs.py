"""Seeded synthetic inputs for single-precision GEMM.

This module draws random numbers and builds structured matrices; it holds no
part of the product's arithmetic.  Both the CPU reference (through the tests)
and the HIP path (through the tests and the benchmark) take their inputs from
here, so the two sides always see bit-identical operands.

Recipe (the pages name shapes but no value distribution; their workloads use
"random data"):
  * numpy.random.default_rng(seed) (PCG64);
  * A is drawn first, then B, in float64, and each is rounded to float32;
  * "uniform" draws i.i.d. U[-1, 1], "normal" draws i.i.d. N(0, 1).
A workload's "identity" variant draws A and B exactly as the random one and
then overwrites A with the identity, so B is bit-identical between the two.

The shapes follow the pages: 3072^3 from the cuda-kernels README (tiled matmul
table), the four H100 shapes and the 512/1024/2048 squares from the
cuda-sgemm-optimization README (results tables), and the odd sizes of the
DD2360 workbook, section 14.3 (lab: 64x64, 100x50x70, 1024^3, 513x8192x1023).
"""
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    seed: int
    dist: str = "uniform"      # "uniform" U[-1,1] or "normal" N(0,1)
    variant: str = "random"    # "random" or "identity" (A := I, needs M == K)
    check: str = "sampled"     # "full" or "sampled"

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


# The five measured configurations and their variants, named by what they are.
WORKLOADS = {
    w.name: w for w in [
        Workload("sgemm_512x512x512_uniform_seed0", 512, 512, 512, 0, check="full"),
        Workload("sgemm_2048x2048x2048_uniform_seed1", 2048, 2048, 2048, 1),
        Workload("sgemm_2048x2048x2048_identityA_seed1", 2048, 2048, 2048, 1,
                 variant="identity", check="full"),
        Workload("sgemm_3072x3072x3072_normal_seed2", 3072, 3072, 3072, 2, dist="normal"),
        Workload("sgemm_8192x8192x4096_uniform_seed3", 8192, 8192, 4096, 3),
        Workload("sgemm_4096x4096x8192_uniform_seed3", 4096, 4096, 8192, 3),
        Workload("sgemm_4099x4099x4099_uniform_seed3", 4099, 4099, 4099, 3),
        Workload("sgemm_8192x8192x8192_uniform_seed4", 8192, 8192, 8192, 4),
        # not graded; the workbook's lab sizes and one more full-check square
        Workload("sgemm_1024x1024x1024_uniform_seed5", 1024, 1024, 1024, 5, check="full"),
        Workload("sgemm_513x8192x1023_uniform_seed6", 513, 8192, 1023, 6),
        Workload("sgemm_100x70x50_uniform_seed7", 100, 70, 50, 7, check="full"),
    ]
}


def draw(rng: np.random.Generator, shape, dist: str = "uniform") -> np.ndarray:
    """One float32 matrix of i.i.d. values, drawn in float64 then rounded."""
    if dist == "uniform":
        x = rng.uniform(-1.0, 1.0, size=shape)
    elif dist == "normal":
        x = rng.standard_normal(size=shape)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return x.astype(np.float32)


def make_operands(M: int, N: int, K: int, seed: int, dist: str = "uniform",
                  variant: str = "random"):
    """(A, B): A is M x K, B is K x N, both C-contiguous float32."""
    rng = np.random.default_rng(seed)
    A = draw(rng, (M, K), dist)
    B = draw(rng, (K, N), dist)
    if variant == "identity":
        if M != K:
            raise ValueError("the identity variant needs M == K")
        A = identity(K)
    elif variant != "random":
        raise ValueError(f"unknown variant {variant!r}")
    return A, B


def workload_operands(w: Workload):
    return make_operands(w.M, w.N, w.K, w.seed, w.dist, w.variant)


def sample_indices(M: int, N: int, seed: int, n_uniform: int = 3584,
                   n_edge: int = 512, band: int = 256, last: int = 0):
    """Seeded output positions to check above full-check sizes.

    n_uniform positions uniform over [0, M) x [0, N), then n_edge positions
    uniform over the edge band (row >= M - band or col >= N - band), then, if
    last > 0, every element of the last `last` rows and columns.  Returns
    (rows, cols) as int64 arrays; duplicates are kept (they are harmless).
    """
    rng = np.random.default_rng(100_000 + seed)
    rows = [rng.integers(0, M, size=n_uniform)]
    cols = [rng.integers(0, N, size=n_uniform)]
    if n_edge > 0 and M > 0 and N > 0:
        bm, bn = min(band, M), min(band, N)
        # the band is the union of a bottom strip and a right strip; pick the
        # strip with probability proportional to its area, then a point in it
        area_bottom = bm * N
        area_right = (M - bm) * bn
        pick_bottom = rng.random(n_edge) * (area_bottom + area_right) < area_bottom
        r_b = rng.integers(M - bm, M, size=n_edge)
        c_b = rng.integers(0, N, size=n_edge)
        r_r = rng.integers(0, max(M - bm, 1), size=n_edge)
        c_r = rng.integers(N - bn, N, size=n_edge)
        rows.append(np.where(pick_bottom, r_b, r_r))
        cols.append(np.where(pick_bottom, c_b, c_r))
    if last > 0:
        lr = np.arange(max(M - last, 0), M)
        lc = np.arange(max(N - last, 0), N)
        rr, cc = np.meshgrid(lr, np.arange(N), indexing="ij")
        rows.append(rr.reshape(-1)); cols.append(cc.reshape(-1))
        rr, cc = np.meshgrid(np.arange(M), lc, indexing="ij")
        rows.append(rr.reshape(-1)); cols.append(cc.reshape(-1))
    return (np.concatenate(rows).astype(np.int64),
            np.concatenate(cols).astype(np.int64))


# ---- structured operands (closed-form cases) ---------------------------------

def identity(n: int) -> np.ndarray:
    return np.eye(n, dtype=np.float32)


def permutation(n: int, seed: int) -> np.ndarray:
    """A permutation matrix P with P[i, perm[i]] = 1; returns (P, perm)."""
    perm = np.random.default_rng(seed).permutation(n)
    P = np.zeros((n, n), dtype=np.float32)
    P[np.arange(n), perm] = 1.0
    return P, perm


def small_integers(rng: np.random.Generator, shape, lo: int = -2, hi: int = 2) -> np.ndarray:
    """i.i.d. integers in [lo, hi] as float32 (exact in float32)."""
    return rng.integers(lo, hi + 1, size=shape).astype(np.float32)


def ones(shape) -> np.ndarray:
    return np.ones(shape, dtype=np.float32)


def small_integers_device(shape, seed: int, lo: int = -3, hi: int = 3, device="cuda"):
    """i.i.d. integers in [lo, hi] as a float32 device tensor, drawn on the
    device by torch's seeded generator (for operands too large to draw and
    upload from the host; the checks copy back only the rows and columns they
    need)."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return torch.randint(lo, hi + 1, tuple(shape), generator=gen, device=device,
                         dtype=torch.float32)


def grid_sample(n: int, seed: int, k: int = 40) -> np.ndarray:
    """Sorted distinct indices in [0, n): the first, middle and last, and k
    seeded uniform picks."""
    if n <= 0:
        return np.zeros(0, dtype=np.int64)
    rng = np.random.default_rng(200_000 + seed)
    picks = {0, n // 2, n - 1} | set(rng.integers(0, n, size=k).tolist())
    return np.array(sorted(picks), dtype=np.int64)

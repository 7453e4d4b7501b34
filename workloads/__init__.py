"""Seeded synthetic inputs for the fp16 TN GEMM (shared by tests and bench).

This module only draws and lays out numbers; it holds none of the GEMM's
arithmetic.  Recipe (the pages fix no data, so this is a stated choice):
  * generator: numpy.random.default_rng(seed) (PCG64); draws in the order
    A, then B, then C, each as a logical (rows, cols) array in C order;
  * "unif":   float64 uniform on [-1, 1), rounded to the storage dtype;
  * "normal": float64 normal with the given sigma, rounded to storage dtype;
  * "int":    integers drawn uniformly from {-2, -1, 0, 1, 2};
  * "dyadic": integers drawn uniformly from {-64..64}, divided by 64 (values
              in [-1, 1] on a 2^-6 grid, exact in fp16);
  * rounding to fp16/fp32 is numpy's cast (round to nearest even);
  * A is stored K-contiguous, A(m,k) = A[m*lda + k], or M-contiguous,
    A(m,k) = A[m + k*lda]; B(n,k) = B[n*ldb + k]; C(m,n) = C[m*ldc + n];
    padding elements between rows are filled with fp16 NaN ("poison") so a
    kernel that reads them produces NaN.

The named workloads are the five shapes the TN GEMM is measured and checked
on; ``integer twin`` = same shapes, strides and dtypes, integer values.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

F16_NAN = np.array([0x7E00], dtype=np.uint16).view(np.float16)[0]


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    a_order: str = "k"          # "k": K-contiguous A, "m": M-contiguous A
    lda: Optional[int] = None
    ldb: Optional[int] = None
    c: Optional[str] = None     # None, "f16", "f32"
    ldc: Optional[int] = None
    d: str = "f32"              # "f16" or "f32"
    ldd: Optional[int] = None
    dist: str = "unif"          # "unif", "normal", "int"
    sigma: float = 1.0          # for "normal" A/B
    c_dist: str = "unif"        # for C: "unif", "normal" (sigma 1), "int"
    seed: int = 0
    twin_seed: Optional[int] = None
    algo: str = "auto"          # "direct", "lds" or "auto"
    note: str = ""

    # resolved leading dimensions
    @property
    def lda_(self):
        return self.lda if self.lda is not None else (self.K if self.a_order == "k" else self.M)

    @property
    def ldb_(self):
        return self.ldb if self.ldb is not None else self.K

    @property
    def ldc_(self):
        return self.ldc if self.ldc is not None else self.N

    @property
    def ldd_(self):
        return self.ldd if self.ldd is not None else self.N

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    def algorithmic_bytes(self) -> int:
        """2(MK+NK) + sizeof(C)MN (if read) + sizeof(D)MN; padding excluded."""
        b = 2 * (self.M * self.K + self.N * self.K)
        if self.c is not None:
            b += (2 if self.c == "f16" else 4) * self.M * self.N
        b += (2 if self.d == "f16" else 4) * self.M * self.N
        return b

    def twin(self) -> "Workload":
        """Integer-valued twin: same shapes, strides and dtypes."""
        return replace(self, name=self.name + "_int", dist="int", c_dist="int",
                       seed=self.twin_seed if self.twin_seed is not None else self.seed + 100)


WORKLOADS = {
    "tiny_32x16x16": Workload("tiny_32x16x16", 32, 16, 16, d="f32", dist="int",
                              c_dist="int", seed=1,
                              note="integer inputs in [-2,2], C absent, fp32 out"),
    "direct_256": Workload("direct_256", 256, 256, 256, d="f16", dist="unif",
                           seed=2, twin_seed=102, algo="direct",
                           note="direct-from-global kernel (no LDS), fp16 out"),
    "lds_4096": Workload("lds_4096", 4096, 4096, 4096, d="f32", dist="unif",
                         seed=3, twin_seed=103, algo="lds",
                         note="LDS-staged tiled GEMM, fp32 out"),
    "accum_mmajor_8192x8192x2048": Workload(
        "accum_mmajor_8192x8192x2048", 8192, 8192, 2048, a_order="m", lda=8192 + 8,
        c="f32", d="f32", dist="normal", sigma=0.5, c_dist="normal", seed=4,
        twin_seed=104, note="M-contiguous A with lda=M+8, C fp32 N(0,1)"),
    "ragged_8191x6143x4097": Workload(
        "ragged_8191x6143x4097", 8191, 6143, 4097, c="f16", d="f16", dist="unif",
        c_dist="unif", seed=5, twin_seed=105,
        note="partial tiles in M, N and K; odd leading dimensions; fp16 C and D"),
    "shard_512x4096x4096": Workload(
        "shard_512x4096x4096", 512, 4096, 4096, d="f32", dist="unif", seed=6, twin_seed=106,
        note="one GPU's share of an 8-way M split of the 4096^3 GEMM: 256 tiles of "
             "128x64, long K"),
}


@dataclass
class Inputs:
    w: Workload
    A: np.ndarray          # fp16 storage buffer (2-D: rows x ld)
    B: np.ndarray          # fp16 (N, ldb)
    C: Optional[np.ndarray]  # (M, ldc) fp16/fp32 or None
    integer: bool


def _draw(rng, dist: str, shape, sigma: float = 1.0) -> np.ndarray:
    if dist == "unif":
        return rng.uniform(-1.0, 1.0, size=shape)
    if dist == "normal":
        return rng.normal(0.0, sigma, size=shape)
    if dist == "int":
        return rng.integers(-2, 3, size=shape).astype(np.float64)
    if dist == "dyadic":
        return rng.integers(-64, 65, size=shape) / 64.0
    raise ValueError(dist)


def make_inputs(w: Workload) -> Inputs:
    rng = np.random.default_rng(w.seed)
    M, N, K = w.M, w.N, w.K
    a_vals = _draw(rng, w.dist, (M, K), w.sigma).astype(np.float16)
    if w.a_order == "k":
        lda = w.lda_
        A = np.full((M, lda), F16_NAN, dtype=np.float16)
        A[:, :K] = a_vals
    else:
        lda = w.lda_
        A = np.full((K, lda), F16_NAN, dtype=np.float16)
        A[:, :M] = a_vals.T
    del a_vals
    b_vals = _draw(rng, w.dist, (N, K), w.sigma).astype(np.float16)
    ldb = w.ldb_
    if ldb == K:
        B = b_vals
    else:
        B = np.full((N, ldb), F16_NAN, dtype=np.float16)
        B[:, :K] = b_vals
    C = None
    if w.c is not None:
        cdt = np.float16 if w.c == "f16" else np.float32
        c_vals = _draw(rng, w.c_dist, (M, N), 1.0).astype(cdt)
        ldc = w.ldc_
        if ldc == N:
            C = c_vals
        else:
            C = np.full((M, ldc), np.nan, dtype=cdt)
            C[:, :N] = c_vals
    return Inputs(w, A, B, C, integer=(w.dist == "int"))


def custom(M, N, K, *, a_order="k", lda=None, ldb=None, c=None, ldc=None, d="f32",
           ldd=None, dist="unif", sigma=1.0, c_dist=None, seed=0, algo="auto",
           name=None) -> Workload:
    return Workload(name or f"custom_{M}x{N}x{K}", M, N, K, a_order=a_order, lda=lda,
                    ldb=ldb, c=c, ldc=ldc, d=d, ldd=ldd, dist=dist, sigma=sigma,
                    c_dist=c_dist or ("int" if dist == "int" else "unif"), seed=seed,
                    algo=algo)


def sample_indices(M: int, N: int, n_random: int, seed: int, tile: int = 128,
                   edge: int = 8) -> tuple:
    """Output positions to check at full size: the corner blocks, rows and
    columns on both sides of every tile boundary near the edges, plus uniform
    random positions.  Returns (ms, ns) int64 arrays without duplicates."""
    rng = np.random.default_rng(seed)
    ms_set = set()
    pts = []
    rows = sorted({r for r in list(range(min(edge, M))) + list(range(max(M - edge, 0), M))})
    cols = sorted({c for c in list(range(min(edge, N))) + list(range(max(N - edge, 0), N))})
    for r in rows:
        for c in cols:
            pts.append((r, c))
    # tile boundaries (last full tile / partial tile seams)
    for b in (tile - 1, tile, (M // tile) * tile - 1, (M // tile) * tile):
        if 0 <= b < M:
            for c in cols:
                pts.append((b, c))
    for b in (tile - 1, tile, (N // tile) * tile - 1, (N // tile) * tile):
        if 0 <= b < N:
            for r in rows:
                pts.append((r, b))
    pts.extend(zip(rng.integers(0, M, n_random).tolist(), rng.integers(0, N, n_random).tolist()))
    for p in pts:
        ms_set.add(p)
    arr = np.array(sorted(ms_set), dtype=np.int64).reshape(-1, 2)
    return arr[:, 0].copy(), arr[:, 1].copy()


# --------------------------------------------------------- back-to-back GEMM
@dataclass(frozen=True)
class ChainWorkload:
    """D_b = rne16(A_b B_b^T) W_b^T per batch b: A (M,K), B (N1,K), W (N2,N1),
    stored as 3-D arrays (batch, rows, ld) with contiguous rows and padding
    (fp16 NaN) past the logical columns when ld exceeds them."""
    name: str
    batch: int
    M: int
    N1: int
    N2: int
    K: int
    d: str = "f16"
    dist: str = "unif"
    seed: int = 0
    twin_seed: Optional[int] = None
    lda: Optional[int] = None
    ldb: Optional[int] = None
    ldw: Optional[int] = None
    note: str = ""

    @property
    def flops(self) -> int:
        return 2 * self.batch * self.M * self.N1 * (self.K + self.N2)

    def algorithmic_bytes(self) -> int:
        """A, B and W read once, D written once."""
        e = 2 if self.d == "f16" else 4
        return self.batch * (2 * (self.M * self.K + self.N1 * self.K + self.N2 * self.N1)
                             + e * self.M * self.N2)

    def twin(self) -> "ChainWorkload":
        return replace(self, name=self.name + "_int", dist="int",
                       seed=self.twin_seed if self.twin_seed is not None else self.seed + 100)


@dataclass
class ChainInputs:
    w: ChainWorkload
    A: np.ndarray   # (batch, M, lda) fp16
    B: np.ndarray   # (batch, N1, ldb)
    W: np.ndarray   # (batch, N2, ldw)
    integer: bool


def make_chain_inputs(w: ChainWorkload) -> ChainInputs:
    """Draw order A, B, W (each (batch, rows, cols) in C order); "int" draws
    from {-2..2} for A and B and {-1, 0, 1} for W so that S stays exact in
    fp16 and D in fp32 (and in fp16 where |D| <= 2048); "dyadic" draws A and
    B on the 2^-6 grid (S exact in fp32, its rounding to fp16 not) and W
    uniform."""
    rng = np.random.default_rng(w.seed)

    def draw(shape, ld, lo_hi=(-2, 2), is_w=False):
        if w.dist == "int":
            v = rng.integers(lo_hi[0], lo_hi[1] + 1, size=shape).astype(np.float16)
        else:
            dist = "unif" if (is_w and w.dist == "dyadic") else w.dist
            v = _draw(rng, dist, shape).astype(np.float16)
        if ld == shape[2]:
            return v
        out = np.full(shape[:2] + (ld,), F16_NAN, dtype=np.float16)
        out[:, :, :shape[2]] = v
        return out

    A = draw((w.batch, w.M, w.K), w.lda or w.K)
    B = draw((w.batch, w.N1, w.K), w.ldb or w.K)
    W = draw((w.batch, w.N2, w.N1), w.ldw or max(w.N1, 1), (-1, 1), is_w=True)
    return ChainInputs(w, A, B, W, integer=(w.dist == "int"))


CHAIN_WORKLOADS = {
    "chain_b32_2048x2048_k128_n128": ChainWorkload(
        "chain_b32_2048x2048_k128_n128", 32, 2048, 2048, 128, 128, d="f16", seed=7,
        twin_seed=107,
        note="attention-shaped: 32 batch x heads, sequence 2048 for queries and keys, "
             "head dimension 128 for both products, fp16 out"),
    "chain_b8_2048x2048_k128_n128": ChainWorkload(
        "chain_b8_2048x2048_k128_n128", 8, 2048, 2048, 128, 128, d="f16", seed=8,
        twin_seed=108,
        note="the same shape with 8 batches: 64 workgroups, a quarter of the compute units"),
}

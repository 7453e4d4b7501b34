"""Back-to-back GEMM reference (test infrastructure only).

The attention-style chain of "CuTe Layout 到 Tensor Core" (§17, "为什么这套抽
象对 FlashAttention 特别重要"): the accumulator of a first MMA, after an
element-wise step, is an operand of a second MMA.  The element-wise step here
is the conversion that feeds the second MMA its fp16 operand (no softmax),
per batch b:

    S_b = A_b B_b^T      (M x N1, the sum over K)
    P_b = rne16(S_b)     (rounded once to binary16, ties to even)
    D_b = P_b W_b^T      (M x N2, the sum over N1)

with A_b (M, K), B_b (N1, K), W_b (N2, N1), each row contiguous along the
summed index (the "TN" form of the TiledMMA page's D = C + A B^T).

Both products are the pinned float64 GEMM of ``gemm.py`` (exact fp16
products, float64 sums) and the rounding is ``fp16.rne16_array``; a float64
sum flips an fp16 rounding decision only when S lies within ~1e-13 relative
of a rounding midpoint (integer-valued inputs are exact).  ``chain_py`` is the
same definition in pure Python with exact rational sums, for tiny shapes.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

from . import fp16
from .gemm import gemm_f64


def _batch_view(X: np.ndarray, b: int, stride: int) -> np.ndarray:
    flat = np.asarray(X).reshape(-1)
    return flat[b * stride:]


def chain_f64(batch: int, M: int, N1: int, N2: int, K: int,
              A: np.ndarray, lda: int, sa: int, B: np.ndarray, ldb: int, sb: int,
              W: np.ndarray, ldw: int, sw: int, with_s: bool = False):
    """D (batch, M, N2) float64; with ``with_s`` also S (batch, M, N1) and
    P (batch, M, N1) for tolerance computations."""
    D = np.zeros((batch, M, N2), dtype=np.float64)
    Ss, Ps = [], []
    for b in range(batch):
        S = gemm_f64(M, N1, K, _batch_view(A, b, sa), lda, False, _batch_view(B, b, sb), ldb) \
            if N1 > 0 else np.zeros((M, 0))
        P = fp16.rne16_array(S)
        P16 = P.astype(np.float16)
        D[b] = gemm_f64(M, N2, N1, P16, N1, False, _batch_view(W, b, sw), ldw) \
            if N2 > 0 else np.zeros((M, 0))
        if with_s:
            Ss.append(S)
            Ps.append(P)
    if with_s:
        return D, np.array(Ss), np.array(Ps)
    return D


def chain_py(M, N1, N2, K, A_at, B_at, W_at):
    """Pure-Python definition with exact rational sums; ``A_at(m,k)``,
    ``B_at(n1,k)``, ``W_at(n2,n1)`` return the (exactly decoded) values."""
    P = [[0.0] * N1 for _ in range(M)]
    for m in range(M):
        for n1 in range(N1):
            s = sum((Fraction(A_at(m, k)) * Fraction(B_at(n1, k)) for k in range(K)), Fraction(0))
            P[m][n1] = fp16.decode_bits(fp16.encode_rne(float(s)))
    D = [[Fraction(0)] * N2 for _ in range(M)]
    for m in range(M):
        for n2 in range(N2):
            D[m][n2] = sum((Fraction(P[m][n1]) * Fraction(W_at(n2, n1)) for n1 in range(N1)),
                           Fraction(0))
    return D


def _gamma(n: int, u: float) -> float:
    """n u / (1 - n u): the bound on the relative error of n rounded
    operations, each with unit roundoff u (standard rounding error analysis)."""
    return n * u / (1.0 - n * u)


def _grain(X: np.ndarray) -> float:
    """Largest power of two g with every element of X an integer multiple of
    g (X holds binary16 values, so X 2^24 is an exact integer); 1 for an
    all-zero X."""
    n = np.abs(np.asarray(X, dtype=np.float64) * 2.0 ** 24).astype(np.int64).reshape(-1)
    n = n[n != 0]
    if n.size == 0:
        return 1.0
    return float((n & -n).min()) * 2.0 ** -24


def chain_tolerance(A32: np.ndarray, B32: np.ndarray, W32: np.ndarray,
                    S: np.ndarray, P: np.ndarray) -> np.ndarray:
    """Per-element bound on |D_gpu - D| for one batch when both sums run in
    fp32 (in any order) and P is rounded from the fp32 S (operands as float
    arrays A (M,K), B (N1,K), W (N2,N1); S and P from ``chain_f64``).

    From the arithmetic, with u32 = 2^-24, u64 = 2^-53 and
    g(n) = n u / (1 - n u):

      dS  = (g32(K) + g64(K)) sum_k |A B|      fp32 sum on the GPU, plus the
                                               float64 sum that produced S;
      dS  = 0 where every product is a multiple of gA gB (the power-of-two
            grains of A and B) and sum_k |A B| <= 2^24 gA gB: every partial
            sum, in any order, is then an integer multiple of gA gB below
            2^24 of them, which fp32 (and float64) hold exactly;
      the GPU's S lies in [S - dS, S + dS]; rounding to nearest is monotone,
      so its P lies in [rne16(S - dS), rne16(S + dS)] and
      dP  = max(rne16(S + dS) - P, P - rne16(S - dS)),
      which is 0 wherever no binary16 rounding boundary lies within dS of S
      (P is then the GPU's P exactly);
      |D_gpu - D| <= sum_n1 dP |W| + g32(N1) sum_n1 (|P| + dP) |W|
                     + g64(N1) sum_n1 |P| |W|   (the float64 sum of D).

    Matrix products of absolute values are library steps."""
    u32, u64 = 2.0 ** -24, 2.0 ** -53
    K = A32.shape[1]
    N1 = B32.shape[0]
    sab = np.abs(A32) @ np.abs(B32).T
    dS = (_gamma(K, u32) + _gamma(K, u64)) * sab
    dS = np.where(sab <= 2.0 ** 24 * _grain(A32) * _grain(B32), 0.0, dS)
    lo = fp16.rne16_array(S - dS)
    hi = fp16.rne16_array(S + dS)
    dP = np.maximum(hi - P, P - lo)
    aW = np.abs(W32).T
    return (dP @ aW + _gamma(N1, u32) * ((np.abs(P) + dP) @ aW)
            + _gamma(N1, u64) * (np.abs(P) @ aW))

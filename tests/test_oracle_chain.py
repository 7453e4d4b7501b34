"""Pins for the back-to-back GEMM reference (oracle/chain.py).

The chain is two GEMMs with one rounding to binary16 between them.  Pinned
by: the exact rational definition on small shapes (transposed operands,
swapped roles or a wrong batch stride fail it), W = identity (D is exactly
the rounded S), the rounding of S at the binary16 midpoints 2049, 2050 and
2051 (ties to even: 2048, 2050, 2052 -- no rounding, rounding toward zero or
half-up each fail), and the tolerance bound against the fp32 arithmetic it
describes.  Planted mistakes fail these pins.
"""
import numpy as np
import pytest

from oracle import chain as CH
from oracle import fp16


def _ints(rng, shape, lo=-2, hi=2):
    return rng.integers(lo, hi + 1, size=shape).astype(np.float16)


def _accessors(A, B, W):
    return (lambda m, k: float(A[m, k]), lambda n1, k: float(B[n1, k]),
            lambda n2, n1: float(W[n2, n1]))


@pytest.mark.parametrize("M,N1,N2,K", [(3, 5, 2, 4), (5, 3, 4, 7), (1, 6, 1, 2), (4, 4, 4, 4)])
def test_matches_exact_definition(M, N1, N2, K):
    rng = np.random.default_rng(M * 100 + N1 * 10 + K)
    A = rng.uniform(-1, 1, (M, K)).astype(np.float16)
    B = rng.uniform(-1, 1, (N1, K)).astype(np.float16)
    W = rng.uniform(-1, 1, (N2, N1)).astype(np.float16)
    D = CH.chain_f64(1, M, N1, N2, K, A, K, 0, B, K, 0, W, N1, 0)[0]
    ref = CH.chain_py(M, N1, N2, K, *_accessors(A, B, W))
    for m in range(M):
        for n2 in range(N2):
            assert D[m, n2] == pytest.approx(float(ref[m][n2]), rel=1e-12, abs=1e-12)


def test_identity_w_gives_the_rounded_s():
    rng = np.random.default_rng(3)
    M, N1, K = 7, 9, 33
    A = rng.uniform(-1, 1, (M, K)).astype(np.float16)
    B = rng.uniform(-1, 1, (N1, K)).astype(np.float16)
    W = np.eye(N1, dtype=np.float16)
    D, S, P = CH.chain_f64(1, M, N1, N1, K, A, K, 0, B, K, 0, W, N1, 0, with_s=True)
    S_direct = A.astype(np.float64) @ B.astype(np.float64).T
    assert np.allclose(S[0], S_direct, rtol=0, atol=1e-12)
    assert np.array_equal(D[0], fp16.rne16_array(S_direct))


@pytest.mark.parametrize("s,want", [(2049, 2048), (2050, 2050), (2051, 2052), (2047, 2047),
                                    (4097, 4096), (4099, 4100)])
def test_rounds_s_once_to_nearest_even(s, want):
    """S = s from K = s ones; W = [[1]] -> D = rne16(s)."""
    A = np.ones((1, s), dtype=np.float16)
    B = np.ones((1, s), dtype=np.float16)
    W = np.ones((1, 1), dtype=np.float16)
    D = CH.chain_f64(1, 1, 1, 1, s, A, s, 0, B, s, 0, W, 1, 0)[0]
    assert D[0, 0] == want


def test_batches_use_their_own_slices():
    rng = np.random.default_rng(7)
    bt, M, N1, N2, K = 3, 4, 5, 3, 6
    sa, sb, sw = M * K + 5, N1 * K + 3, N2 * N1 + 1
    A = rng.uniform(-1, 1, bt * sa).astype(np.float16)
    B = rng.uniform(-1, 1, bt * sb).astype(np.float16)
    W = rng.uniform(-1, 1, bt * sw).astype(np.float16)
    D = CH.chain_f64(bt, M, N1, N2, K, A, K, sa, B, K, sb, W, N1, sw)
    for b in range(bt):
        Ab = A[b * sa:b * sa + M * K].reshape(M, K)
        Bb = B[b * sb:b * sb + N1 * K].reshape(N1, K)
        Wb = W[b * sw:b * sw + N2 * N1].reshape(N2, N1)
        ref = CH.chain_py(M, N1, N2, K, *_accessors(Ab, Bb, Wb))
        assert np.allclose(D[b], np.array(ref, dtype=np.float64), rtol=1e-12, atol=1e-12)


def test_integer_inputs_are_exact():
    rng = np.random.default_rng(11)
    M, N1, N2, K = 6, 40, 5, 64
    A, B, W = _ints(rng, (M, K)), _ints(rng, (N1, K)), _ints(rng, (N2, N1))
    D = CH.chain_f64(1, M, N1, N2, K, A, K, 0, B, K, 0, W, N1, 0)[0]
    S = A.astype(np.int64) @ B.astype(np.int64).T          # |S| <= 256: exact in fp16
    assert np.array_equal(D, (S @ W.astype(np.int64).T).astype(np.float64))


def test_tolerance_covers_fp32_arithmetic():
    """Simulate both sums in fp32 (sequential order) and the fp16 rounding of
    the fp32 S: the difference stays inside the bound, which is far below
    the size of D."""
    rng = np.random.default_rng(5)
    M, N1, N2, K = 8, 64, 8, 128
    A = rng.uniform(-1, 1, (M, K)).astype(np.float16)
    B = rng.uniform(-1, 1, (N1, K)).astype(np.float16)
    W = rng.uniform(-1, 1, (N2, N1)).astype(np.float16)
    D, S, P = CH.chain_f64(1, M, N1, N2, K, A, K, 0, B, K, 0, W, N1, 0, with_s=True)
    S32 = np.zeros((M, N1), dtype=np.float32)
    for k in range(K):
        S32 += A[:, k:k + 1].astype(np.float32) * B[:, k].astype(np.float32)[None, :]
    P16 = S32.astype(np.float16).astype(np.float32)
    D32 = np.zeros((M, N2), dtype=np.float32)
    for n1 in range(N1):
        D32 += P16[:, n1:n1 + 1] * W[:, n1].astype(np.float32)[None, :]
    tol = CH.chain_tolerance(A.astype(np.float64), B.astype(np.float64), W.astype(np.float64),
                             S[0], P[0])
    err = np.abs(D32.astype(np.float64) - D[0])
    assert (err <= tol).all()
    assert tol.max() < 0.05 * np.abs(D[0]).max()


# ---------------------------------------------------------- planted mistakes
def _pins_pass():
    try:
        for shape in [(3, 5, 2, 4), (5, 3, 4, 7)]:
            test_matches_exact_definition(*shape)
        test_identity_w_gives_the_rounded_s()
        for s, want in [(2049, 2048), (2051, 2052)]:
            test_rounds_s_once_to_nearest_even(s, want)
        test_batches_use_their_own_slices()
        test_integer_inputs_are_exact()
    except (AssertionError, ValueError, IndexError):
        return False
    return True


def test_pins_pass_on_the_oracle():
    assert _pins_pass()


def _mut_no_rounding(x):
    return np.asarray(x, dtype=np.float64)


_REAL_RNE = fp16.rne16_array


def _mut_truncate(x):
    """Mistake: round toward zero (one binary16 step back where RNE went up)."""
    a = np.asarray(x, dtype=np.float64)
    r = _REAL_RNE(a)
    down = np.nextafter(r.astype(np.float16), np.float16(0)).astype(np.float64)
    return np.where(np.abs(r) > np.abs(a), down, r)


@pytest.mark.parametrize("mut", [_mut_no_rounding, _mut_truncate])
def test_planted_rounding_mistakes_are_caught(monkeypatch, mut):
    monkeypatch.setattr(CH.fp16, "rne16_array", mut)
    assert not _pins_pass()


def _mut_roles_swapped(batch, M, N1, N2, K, A, lda, sa, B, ldb, sb, W, ldw, sw, with_s=False):
    """Mistake: S = B A^T read back as (M, N1)."""
    D = np.zeros((batch, M, N2))
    for b in range(batch):
        S = CH.gemm_f64(N1, M, K, CH._batch_view(B, b, sb), ldb, False, CH._batch_view(A, b, sa), lda)
        P16 = fp16.rne16_array(S.reshape(M, N1)).astype(np.float16)
        D[b] = CH.gemm_f64(M, N2, N1, P16, N1, False, CH._batch_view(W, b, sw), ldw)
    return D


def _mut_w_not_transposed(batch, M, N1, N2, K, A, lda, sa, B, ldb, sb, W, ldw, sw, with_s=False):
    """Mistake: D = P W with W read as (N1, N2)."""
    D = np.zeros((batch, M, N2))
    for b in range(batch):
        S = CH.gemm_f64(M, N1, K, CH._batch_view(A, b, sa), lda, False, CH._batch_view(B, b, sb), ldb)
        P = fp16.rne16_array(S)
        Wb = CH._batch_view(W, b, sw)[:N1 * N2].astype(np.float64).reshape(N1, N2)
        D[b] = P @ Wb
    return D


def _mut_stride_ignored(batch, M, N1, N2, K, A, lda, sa, B, ldb, sb, W, ldw, sw, with_s=False):
    """Mistake: every batch reads batch 0."""
    return CH.__dict__["_real_chain"](batch, M, N1, N2, K, A, lda, 0, B, ldb, 0, W, ldw, 0,
                                      with_s=with_s)


@pytest.mark.parametrize("mut", [_mut_roles_swapped, _mut_w_not_transposed, _mut_stride_ignored])
def test_planted_composition_mistakes_are_caught(monkeypatch, mut):
    monkeypatch.setattr(CH, "_real_chain", CH.chain_f64, raising=False)
    monkeypatch.setattr(CH, "chain_f64", mut)
    assert not _pins_pass()

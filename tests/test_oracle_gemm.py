"""Pins for the float64 GEMM oracle (oracle/gemm_ref.c, oracle/gemm.py).

Pinned against: a hand-worked example (tests/golden/gemm_hand.txt), exact
rational arithmetic on tiny inputs, closed forms (A=0, all-ones, identity B),
numpy's float64 matmul, and the sampled entry point against the full one.
The mutant checks at the bottom show that plausible mistakes (B transposed,
C dropped, last k skipped, M-major A read K-major) fail these pins.
"""
import math

import numpy as np
import pytest

from oracle import gemm as G
from oracle import fp16
from helpers import keyed
import workloads as W


def _hand():
    tok = dict((t[0], t[1:]) for t in [l.split() for l in open(
        __import__("helpers").GOLDEN + "/gemm_hand.txt") if l.strip() and not l.startswith("#")])
    M, N, K = (int(x) for x in tok["shape"])
    A = np.array([float(x) for x in tok["A"]]).reshape(M, K).astype(np.float16)
    B = np.array([float(x) for x in tok["B"]]).reshape(N, K).astype(np.float16)
    C = np.array([float(x) for x in tok["C"]]).reshape(M, N).astype(np.float32)
    D = np.array([float(x) for x in tok["D"]]).reshape(M, N)
    return M, N, K, A, B, C, D


def test_hand_example_c_and_python():
    M, N, K, A, B, C, D = _hand()
    got = G.gemm_f64(M, N, K, A, K, False, B, K, C)
    assert np.array_equal(got, D)
    a_at, b_at, c_at = G.operand_accessors(A, K, False, B, K, C)
    py = np.array(G.gemm_f64_py(M, N, K, a_at, b_at, c_at), dtype=np.float64)
    assert np.array_equal(py, D)


def _random_case(rng, M, N, K, a_mmajor, c_kind, integer, pad=3):
    def vals(shape):
        if integer:
            return rng.integers(-2, 3, size=shape).astype(np.float16)
        return rng.uniform(-1, 1, size=shape).astype(np.float16)
    a = vals((M, K))
    if a_mmajor:
        lda = M + pad
        A = np.full((K, lda), W.F16_NAN, dtype=np.float16)
        A[:, :M] = a.T
    else:
        lda = K + pad
        A = np.full((M, lda), W.F16_NAN, dtype=np.float16)
        A[:, :K] = a
    ldb = K + 1
    B = np.full((N, ldb), W.F16_NAN, dtype=np.float16)
    B[:, :K] = vals((N, K))
    C = None
    if c_kind == "f16":
        C = vals((M, N)).astype(np.float16)
    elif c_kind == "f32":
        C = vals((M, N)).astype(np.float32)
    return A, lda, B, ldb, C, a


@pytest.mark.parametrize("a_mmajor", [False, True])
@pytest.mark.parametrize("c_kind", [None, "f16", "f32"])
@pytest.mark.parametrize("integer", [True, False])
def test_c_loop_equals_exact_rational(a_mmajor, c_kind, integer):
    rng = np.random.default_rng(11)
    M, N, K = 5, 7, 9
    A, lda, B, ldb, C, _ = _random_case(rng, M, N, K, a_mmajor, c_kind, integer)
    got = G.gemm_f64(M, N, K, A, lda, a_mmajor, B, ldb, C)
    a_at, b_at, c_at = G.operand_accessors(A, lda, a_mmajor, B, ldb, C)
    exact = G.gemm_f64_py(M, N, K, a_at, b_at, c_at, exact=True)
    for m in range(M):
        for n in range(N):
            # sums of <= 10 exact products of 11-bit significands: exact in double
            assert got[m, n] == float(exact[m][n])


def test_integer_results_are_python_ints():
    rng = np.random.default_rng(12)
    M, N, K = 6, 4, 33
    A, lda, B, ldb, C, a = _random_case(rng, M, N, K, False, "f32", True, pad=0)
    got = G.gemm_f64(M, N, K, A, lda, False, B, ldb, C)
    ai = a.astype(np.int64)
    bi = B[:, :K].astype(np.int64)
    want = C.astype(np.int64) + ai @ bi.T
    assert np.array_equal(got, want.astype(np.float64))


def test_closed_forms():
    rng = np.random.default_rng(13)
    M, N, K = 7, 12, 10
    C = rng.normal(size=(M, N)).astype(np.float32)
    zeros = np.zeros((M, K), np.float16)
    B = rng.uniform(-1, 1, (N, K)).astype(np.float16)
    assert np.array_equal(G.gemm_f64(M, N, K, zeros, K, False, B, K, C), C.astype(np.float64))
    ones_a = np.ones((M, K), np.float16)
    ones_b = np.ones((N, K), np.float16)
    assert np.array_equal(G.gemm_f64(M, N, K, ones_a, K, False, ones_b, K, C),
                          C.astype(np.float64) + K)
    A = rng.uniform(-1, 1, (M, K)).astype(np.float16)
    eye = np.zeros((N, K), np.float16)
    for i in range(K):
        eye[i, i] = 1
    D = G.gemm_f64(M, N, K, A, K, False, eye, K, C)
    want = C.astype(np.float64).copy()
    want[:, :K] += A.astype(np.float64)
    assert np.array_equal(D, want)


def test_matches_numpy_matmul():
    rng = np.random.default_rng(14)
    M, N, K = 37, 29, 301
    A = rng.uniform(-1, 1, (M, K)).astype(np.float16)
    B = rng.uniform(-1, 1, (N, K)).astype(np.float16)
    C = rng.uniform(-1, 1, (M, N)).astype(np.float16)
    D = G.gemm_f64(M, N, K, A, K, False, B, K, C)
    ref = C.astype(np.float64) + A.astype(np.float64) @ B.astype(np.float64).T
    assert np.max(np.abs(D - ref)) <= 1e-12 * K


def test_sampled_equals_full_and_rows_window():
    w = W.custom(67, 45, 130, a_order="m", lda=70, c="f16", dist="unif", seed=3)
    x = W.make_inputs(w)
    full = G.gemm_f64(w.M, w.N, w.K, x.A, w.lda_, True, x.B, w.ldb_, x.C)
    ms, ns = W.sample_indices(w.M, w.N, 200, seed=1, tile=16)
    s = G.gemm_f64_sampled(w.M, w.N, w.K, x.A, w.lda_, True, x.B, w.ldb_, x.C, ms, ns)
    assert np.array_equal(s, full[ms, ns])
    part = G.gemm_f64(w.M, w.N, w.K, x.A, w.lda_, True, x.B, w.ldb_, x.C, rows=(10, 20))
    assert np.array_equal(part[10:20], full[10:20])
    assert np.isnan(part[:10]).all() and np.isnan(part[20:]).all()
    with pytest.raises(IndexError):
        G.gemm_f64_sampled(w.M, w.N, w.K, x.A, w.lda_, True, x.B, w.ldb_, x.C,
                           np.array([w.M]), np.array([0]))


def test_poisoned_padding_is_never_read():
    w = W.custom(33, 17, 21, lda=40, ldb=30, dist="unif", seed=4)
    x = W.make_inputs(w)
    assert np.isnan(x.A[:, 21:].astype(np.float32)).all()
    D = G.gemm_f64(w.M, w.N, w.K, x.A, w.lda_, False, x.B, w.ldb_, None)
    assert np.isfinite(D).all()


def test_degenerate_sizes():
    A = np.zeros((4, 1), np.float16)
    B = np.zeros((3, 1), np.float16)
    C = np.arange(12, dtype=np.float32).reshape(4, 3)
    D = G.gemm_f64(4, 3, 0, A, 1, False, B, 1, C)
    assert np.array_equal(D, C.astype(np.float64))
    D = G.gemm_f64(0, 3, 5, A, 5, False, B, 5, None)
    assert D.shape == (0, 3)


# --------------------------------------------------------- mutant detection
def _pins_pass(fn):
    """Run the hand example and two closed forms through a candidate
    reference ``fn(M,N,K,A64,B64,C64) -> D``."""
    M, N, K, A, B, C, D = _hand()
    ok = np.array_equal(fn(M, N, K, A.astype(np.float64), B.astype(np.float64),
                           C.astype(np.float64)), D)
    rng = np.random.default_rng(5)
    A2 = rng.integers(-2, 3, (5, 3)).astype(np.float64)
    eye = np.eye(4, 3)
    C2 = rng.integers(-2, 3, (5, 4)).astype(np.float64)
    want = C2.copy()
    want[:, :3] += A2
    try:
        ok = ok and np.array_equal(fn(5, 4, 3, A2, eye, C2), want)
    except (IndexError, ValueError):
        ok = False
    return ok


def _ref(M, N, K, A, B, C):
    return C + A @ B.T


@pytest.mark.parametrize("mutant", [
    lambda M, N, K, A, B, C: C + A @ B.reshape(K, N),       # B read as (K,N)
    lambda M, N, K, A, B, C: C + (A @ B.T)[:, ::-1],        # n index reversed
    lambda M, N, K, A, B, C: A @ B.T,                       # C dropped
    lambda M, N, K, A, B, C: C + A[:, :K - 1] @ B[:, :K - 1].T,  # last k skipped
    lambda M, N, K, A, B, C: C - A @ B.T,                   # sign
    lambda M, N, K, A, B, C: C + A.reshape(K, M).T @ B.T,   # A read in the wrong order
])
def test_pins_reject_mutants(mutant):
    assert _pins_pass(_ref)
    assert not _pins_pass(mutant)

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


def _fp32_chain(A, B, W, order="seq", drop=None):
    """The chain as a GPU computes it: both sums in fp32 (products of two
    binary16 values are exact in fp32), S rounded once to binary16.  order:
    "seq" k ascending, "rev" k descending, "blk16" sums of 16 consecutive
    terms added in turn (the grouping a 16-deep matrix instruction gives).
    drop=(m, n1, k): leave that product out of S (a planted mistake)."""
    def fsum(terms):                      # terms (T, ...) float32, summed over axis 0
        idx = list(range(terms.shape[0]))
        if order == "rev":
            idx = idx[::-1]
        acc = np.zeros(terms.shape[1:], dtype=np.float32)
        if order == "blk16":
            for b0 in range(0, len(idx), 16):
                part = np.zeros(terms.shape[1:], dtype=np.float32)
                for k in idx[b0:b0 + 16]:
                    part = part + terms[k]
                acc = acc + part
            return acc
        for k in idx:
            acc = acc + terms[k]
        return acc

    A32, B32, W32 = A.astype(np.float32), B.astype(np.float32), W.astype(np.float32)
    prod = A32.T[:, :, None] * B32.T[:, None, :]          # (K, M, N1), exact
    if drop is not None:
        m, n1, k = drop
        prod[k, m, n1] = 0.0
    S32 = fsum(prod)
    P16 = S32.astype(np.float16).astype(np.float32)
    return fsum(P16.T[:, :, None] * W32.T[:, None, :]), P16   # (M, N2), P


def _pin_data(dist="unif"):
    """Pin shapes M, N1, N2, K = 8, 64, 8, 128.  "unif": binary16 values of
    uniform [-1, 1); "dyadic": multiples of 2^-6 in [-1, 1] for A and B (so
    S is exact in fp32 in any order and P's rounding does all the work), W
    uniform."""
    rng = np.random.default_rng(5)
    M, N1, N2, K = 8, 64, 8, 128
    if dist == "dyadic":
        A = (rng.integers(-64, 65, (M, K)) / 64.0).astype(np.float16)
        B = (rng.integers(-64, 65, (N1, K)) / 64.0).astype(np.float16)
    else:
        A = rng.uniform(-1, 1, (M, K)).astype(np.float16)
        B = rng.uniform(-1, 1, (N1, K)).astype(np.float16)
    W = rng.uniform(-1, 1, (N2, N1)).astype(np.float16)
    D, S, P = CH.chain_f64(1, M, N1, N2, K, A, K, 0, B, K, 0, W, N1, 0, with_s=True)
    tol = CH.chain_tolerance(A.astype(np.float64), B.astype(np.float64), W.astype(np.float64),
                             S[0], P[0])
    return A, B, W, D[0], S[0], P[0], tol


@pytest.mark.parametrize("dist", ["unif", "dyadic"])
@pytest.mark.parametrize("order", ["seq", "rev", "blk16"])
def test_tolerance_covers_fp32_arithmetic(order, dist):
    """Simulate both sums in fp32 in three orders and the fp16 rounding of
    the fp32 S: every element of the difference stays inside the bound."""
    A, B, W, D, S, P, tol = _pin_data(dist)
    D32, _ = _fp32_chain(A, B, W, order)
    err = np.abs(D32.astype(np.float64) - D)
    assert (err <= tol).all()


def test_dyadic_inputs_make_s_exact():
    """The exactness the bound uses: with A, B multiples of 2^-6 and K = 128,
    the fp32 S equals the float64 S in every order, so P_gpu = P and the
    bound charges no flip; one element of finer grain (2^-20) removes the
    exemption."""
    A, B, W, D, S, P, tol = _pin_data("dyadic")
    for order in ("seq", "rev", "blk16"):
        _, P16 = _fp32_chain(A, B, W, order)
        assert np.array_equal(P16, P)
    assert CH._grain(A.astype(np.float64)) == 2.0 ** -6
    assert (tol <= 64 * 2.0 ** -23 * (np.abs(P) @ np.abs(W.astype(np.float64)).T)).all()
    A2 = A.copy()
    A2[3, 7] = np.float16(2.0 ** -20)                # a subnormal: grain 2^-20
    assert CH._grain(A2.astype(np.float64)) == 2.0 ** -20
    D2, S2, P2 = CH.chain_f64(1, 8, 64, 8, 128, A2, 128, 0, B, 128, 0, W, 64, 0, with_s=True)
    tol2 = CH.chain_tolerance(A2.astype(np.float64), B.astype(np.float64), W.astype(np.float64),
                              S2[0], P2[0])
    assert (tol2 > 64 * 2.0 ** -23 * (np.abs(P2[0]) @ np.abs(W.astype(np.float64)).T)).any()


def _flip_case():
    """S = 1024 + (1 + 2^-9) 2^-11 - 1024 + 1 = 1 + 2^-11 + 2^-20 exactly, just
    above the binary16 midpoint 1 + 2^-11 (so P = 1 + 2^-10), while the fp32
    sum in k order loses the 2^-20 against 1024 and lands on the midpoint,
    which rounds to even: P_gpu = 1.  W = [[1]], so D = P."""
    A = np.array([[1024.0, 1.0 + 2.0 ** -9, -1024.0, 1.0]], dtype=np.float16)
    B = np.array([[1.0, 2.0 ** -11, 1.0, 1.0]], dtype=np.float16)
    W = np.ones((1, 1), dtype=np.float16)
    D, S, P = CH.chain_f64(1, 1, 1, 1, 4, A, 4, 0, B, 4, 0, W, 1, 0, with_s=True)
    tol = CH.chain_tolerance(A.astype(np.float64), B.astype(np.float64), W.astype(np.float64),
                             S[0], P[0])
    return A, B, W, D[0], tol


def test_flip_case_is_what_it_claims():
    A, B, W, D, tol = _flip_case()
    assert D[0, 0] == 1.0 + 2.0 ** -10
    D32, P16 = _fp32_chain(A, B, W, "seq")
    assert P16[0, 0] == 1.0 and D32[0, 0] == 1.0


def test_bound_is_attained_where_rounding_can_flip():
    """Tightness: on the flip case the fp32 chain's error is more than half
    the bound (a bound twice as loose fails this), and on the random pin data
    the bound charges a flip only to elements whose S lies near a binary16
    rounding boundary (elsewhere P_gpu must equal P, and does)."""
    A, B, W, D, tol = _flip_case()
    D32, _ = _fp32_chain(A, B, W, "seq")
    err = abs(float(D32[0, 0]) - D[0, 0])
    assert err <= tol[0, 0] and err > 0.5 * tol[0, 0], (err, tol[0, 0])
    A, B, W, D, S, P, tol = _pin_data()
    u = 2.0 ** -24
    dS = 1.01 * 128 * u * (np.abs(A.astype(np.float64)) @ np.abs(B.astype(np.float64)).T)
    near = (fp16.rne16_array(S - dS) != P) | (fp16.rne16_array(S + dS) != P)
    assert 0 < near.sum() < near.size
    for order in ("seq", "rev", "blk16"):
        _, P16 = _fp32_chain(A, B, W, order)
        assert np.array_equal(P16[~near], P[~near])


def _old_tolerance(A32, B32, W32, S, P):
    """The earlier, looser bound: every element charged dS + ulp16(|S| + dS),
    as if every rounding of S could flip."""
    u = 2.0 ** -24
    K, N1 = A32.shape[1], B32.shape[0]
    dS = K * u * (np.abs(A32) @ np.abs(B32).T)
    dP = dS + fp16.ulp16_array(np.abs(S) + dS)
    return dP @ np.abs(W32).T + N1 * u * (np.abs(P) @ np.abs(W32).T)


@pytest.mark.parametrize("dist,min_caught", [("dyadic", 0.0), ("unif", 0.05)])
def test_dropped_product_term_is_caught(dist, min_caught):
    """A planted mistake in the simulated chain: one product of S left out.
    Products across the whole range are tried.  Every omission that moves D
    at all (the rounding of S to binary16 hides the small ones) and that the
    earlier bound still accepted is rejected by the derived bound: on dyadic
    inputs whatever its size, on uniform ones from 0.05 up (below that the
    possible flips of S near binary16 boundaries leave the room a correct
    fp32 chain needs)."""
    A, B, W, D, S, P, tol = _pin_data(dist)
    old = _old_tolerance(A.astype(np.float64), B.astype(np.float64), W.astype(np.float64), S, P)
    D0, _ = _fp32_chain(A, B, W, "seq")
    prods = np.abs(A.astype(np.float64)[:, None, :] * B.astype(np.float64)[None, :, :])
    caught = 0
    for flat in np.argsort(-prods, axis=None)[::97]:      # products across the range
        m, n1, k = np.unravel_index(flat, prods.shape)
        if prods[m, n1, k] < min_caught:
            continue
        D32, _ = _fp32_chain(A, B, W, "seq", drop=(m, n1, k))
        if np.array_equal(D32, D0):
            continue                                    # absorbed by the rounding of S
        err = np.abs(D32.astype(np.float64) - D)
        if (err <= old).all():                          # inside the old bound ...
            assert not (err <= tol).all(), (m, n1, k, prods[m, n1, k])   # ... not the new
            caught += 1
    assert caught >= 5, caught


@pytest.mark.parametrize("dist", ["unif", "dyadic"])
def test_perturbed_element_is_caught(dist):
    """Any element of D moved by 1e-3 max|D| falls outside the bound."""
    A, B, W, D, S, P, tol = _pin_data(dist)
    D32, _ = _fp32_chain(A, B, W, "seq")
    eps = 1e-3 * np.abs(D).max()
    for m in range(D.shape[0]):
        for n in range(D.shape[1]):
            bad = D32.astype(np.float64).copy()
            bad[m, n] += eps
            assert not (np.abs(bad - D) <= tol).all(), (m, n)


def test_bound_that_ignores_flips_fails_the_flip_case():
    """A planted mistake in the bound (no charge for a flipped rounding of S)
    does not cover the fp32 chain on the flip case."""
    A, B, W, D, tol = _flip_case()
    u = 2.0 ** -24
    no_flip = 1 * u * 1.0 + 0 * tol                    # only the second sum's rounding
    D32, _ = _fp32_chain(A, B, W, "seq")
    assert abs(float(D32[0, 0]) - D[0, 0]) > no_flip[0, 0]


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

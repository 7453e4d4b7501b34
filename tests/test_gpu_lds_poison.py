"""Debug checks of the LDS pipeline.

* Poisoned LDS: test-only instances of the LDS kernels fill their whole LDS
  array with fp16 NaN before the first fetch (mfl_probe_gemm_poisoned).  A
  fragment read or an epilogue read of any location the kernel did not write
  (a wrong swizzle, a missing zero fill of a K tail or edge row, a stage read
  before it is fetched) puts a NaN or a wrong value in D; integer inputs must
  still come out bit-exact.  Ragged M, N and K, every C/D kind, the fetch
  paths the instances cover.
* One K-tile against many: K = BK against K = 4 BK whose extra columns of A
  and B are zero.  The extra matrix instructions add exact zeros, so D agrees
  value for value even on random floats: the pipelined K loop (prologue,
  steady state, peeled last steps) computes the same sums as a single step.
"""
import numpy as np
import pytest

import workloads as W
from gpu_helpers import oracle_full, run_gemm, say, verdict

pytestmark = pytest.mark.gpu

# (algo, A M-contiguous, 16-byte rows for A, for B): the instances' fetch paths
POISONED = [("lds128", False, True, True), ("lds128", False, False, False),
            ("lds256", True, True, True), ("lds256", True, False, False),
            ("lds128w1", False, True, False), ("splitk", False, True, True),
            ("lds256w4_16", False, False, False), ("lds256_16", False, True, True),
            ("lds128_16", True, True, True), ("splitk_16", False, True, True)]
SHAPES = [(130, 70, 65), (257, 300, 129), (64, 64, 64), (33, 200, 300), (512, 256, 1000)]


@pytest.mark.parametrize("algo,mm,al_a,al_b", POISONED,
                         ids=[f"{p[0]}-{'m' if p[1] else 'k'}{int(p[2])}{int(p[3])}"
                              for p in POISONED])
def test_poisoned_lds_never_reaches_d(algo, mm, al_a, al_b):
    for idx, (M, N, K) in enumerate(SHAPES):
        for c, d in ((None, "f32"), ("f16", "f16"), ("f32", "f32")):
            if mm:
                M8 = (M + 7) // 8 * 8           # the transposing direct path needs M % 8 == 0
                lda = M8 + 8 if al_a else M8 + 3
                Mx = M8 if al_a else M
            else:
                Mx = M
                lda = (K + 7) // 8 * 8 + 8 if al_a else K + 1
            ldb = (K + 7) // 8 * 8 + 8 if al_b else K + 3
            w = W.custom(Mx, N, K, a_order="m" if mm else "k", lda=lda, ldb=ldb, c=c, d=d,
                         dist="int", seed=500 + idx)
            x = W.make_inputs(w)
            D, checks = run_gemm(w, x, algo, poisoned=True)
            assert all(checks.values()), (w.name, checks)
            assert np.isfinite(D).all(), (algo, w.name, c, d)
            v = verdict(D, oracle_full(w, x), w, True)
            assert v.ok, (algo, w.name, w.a_order, c, d, lda, ldb, str(v))
    say(f"[gpu] poisoned LDS {algo}: all shapes bit-exact")


@pytest.mark.parametrize("algo", ["lds128", "lds256", "lds256w4", "lds128w1", "splitk",
                                  "lds256w4_16", "lds256_16", "lds128_16", "splitk_16",
                                  "direct"])
def test_one_k_tile_equals_many(algo):
    bk = {"lds256": 64, "lds256w4": 64, "splitk": 128, "lds256w4_16": 64, "lds256_16": 64,
          "lds128_16": 64, "splitk_16": 128}.get(algo, 32)
    M, N = 300, 260
    w1 = W.custom(M, N, bk, c="f32", d="f32", dist="unif", seed=77, lda=bk, ldb=bk)
    x1 = W.make_inputs(w1)
    w4 = W.custom(M, N, 4 * bk, c="f32", d="f32", dist="unif", seed=77, lda=4 * bk, ldb=4 * bk)
    x4 = W.make_inputs(w4)
    x4.A[:] = 0
    x4.B[:] = 0
    x4.A[:, :bk] = x1.A
    x4.B[:, :bk] = x1.B
    x4.C[:] = x1.C
    D1, c1 = run_gemm(w1, x1, algo)
    D4, c4 = run_gemm(w4, x4, algo)
    assert all(c1.values()) and all(c4.values())
    assert np.array_equal(D1, D4), (algo, float(np.abs(D1 - D4).max()))
    assert verdict(D1, oracle_full(w1, x1), w1, False).ok

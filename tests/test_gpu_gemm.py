"""GEMM parity on the GPU: the HIP path (through the C ABI) against the
float64 oracle.

* small and ragged shapes: every element, integer inputs bit-exact and float
  inputs within tolerance, for every kernel and dtype combination;
* the five named workloads at full size, in the launch configuration the
  benchmark times: every element of D against the full float64 oracle (for
  float and integer inputs), plus, for integer inputs with fp32 output, a
  Freivalds check of the whole matrix in exact integer arithmetic;
* guard canaries after every buffer and untouched padding."""
import math

import numpy as np
import pytest

import mma_fragment_layouts_tn_amd as mfl
import workloads as W
from gpu_helpers import (freivalds_exact, oracle_full, oracle_full_cached, refused, run_gemm,
                         say, verdict)

pytestmark = pytest.mark.gpu

# the 16x16x32 configurations (same block tiles on the other f16 instruction)
X16 = ["lds256w4_16", "lds256_16", "lds128_16", "splitk_16"]
ALGOS = ["direct", "lds128", "lds256", "lds256w4", "lds128w1", "splitk"] + X16
LDS_ALGOS = ["lds128", "lds256", "lds256w4", "lds128w1", "splitk"] + X16


def _assert_checks(checks):
    assert all(checks.values()), checks


# ------------------------------------------------------------ small shapes
SMALL = [(1, 1, 1), (5, 7, 3), (32, 16, 16), (33, 17, 9), (64, 64, 64), (127, 129, 31),
         (130, 260, 65), (257, 255, 97), (300, 70, 200), (129, 383, 8), (16, 300, 47)]


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("shape", SMALL)
def test_small_integer_bit_exact(algo, shape):
    M, N, K = shape
    # odd leading dimensions: register fetch; 16-byte rows: direct-to-LDS fetch
    ld16 = (K + 7) // 8 * 8 + 8
    cases = (((None, "f32"), K + 3, K + 1), (("f16", "f16"), ld16, ld16),
             (("f32", "f32"), ld16, K + 1), ((None, "f16"), K + 3, ld16),
             (("f32", "f16"), ld16, ld16))
    for (c, d), lda, ldb in cases:
        w = W.custom(M, N, K, c=c, d=d, dist="int", seed=M * 7 + N * 3 + K, lda=lda, ldb=ldb)
        if refused(w, algo):
            continue
        x = W.make_inputs(w)
        D, checks = run_gemm(w, x, algo)
        _assert_checks(checks)
        v = verdict(D, oracle_full(w, x), w, True)
        assert v.ok, (w.name, c, d, str(v))


# K remainders of every size class for every stage depth (BK 32, 64, 128):
# the last, partial K-step is staged by 16-byte chunks with zero fill and
# runs only the sub-steps that hold some k < K
K_TAILS = [65, 79, 80, 81, 97, 113, 127, 143, 193]


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("K", K_TAILS)
def test_k_remainder_integer_bit_exact(algo, K):
    M, N = 130, 96
    ld16 = (K + 7) // 8 * 8 + 8
    for (c, d), lda, ldb in (((None, "f32"), K, K), (("f16", "f16"), ld16, K + 1),
                             (("f32", "f16"), K + 3, ld16)):
        w = W.custom(M, N, K, c=c, d=d, dist="int", seed=K * 11 + lda, lda=lda, ldb=ldb)
        if refused(w, algo):
            continue
        x = W.make_inputs(w)
        D, checks = run_gemm(w, x, algo)
        _assert_checks(checks)
        v = verdict(D, oracle_full(w, x), w, True)
        assert v.ok, (w.name, algo, c, d, lda, ldb, str(v))


# Split-K (K-groups of waves, partial tiles reduced through LDS): K from one
# 128-deep stage to several, with and without a K tail, ragged M and N, every
# C/D combination, both fetch paths
SPLITK_SHAPES = [(128, 64, 128), (128, 64, 256), (200, 100, 384), (257, 129, 1000),
                 (64, 200, 4097), (130, 70, 640), (1, 1, 300), (300, 260, 129)]


@pytest.mark.parametrize("shape", SPLITK_SHAPES)
def test_splitk_integer_bit_exact(shape):
    M, N, K = shape
    ld16 = (K + 7) // 8 * 8 + 8
    for (c, d), lda, ldb in (((None, "f32"), ld16, ld16), (("f16", "f16"), K + 1, ld16),
                             (("f32", "f32"), ld16, K + 3), ((None, "f16"), K + 1, K + 1)):
        w = W.custom(M, N, K, c=c, d=d, dist="int", seed=M + 3 * N + 7 * K, lda=lda, ldb=ldb)
        x = W.make_inputs(w)
        say(f"[gpu] splitk {w.name} c={c} d={d} lda={lda} ldb={ldb}")
        D, checks = run_gemm(w, x, "splitk")
        _assert_checks(checks)
        v = verdict(D, oracle_full(w, x), w, True)
        assert v.ok, (w.name, c, d, str(v))


# lda = M + 8: with M % 8 == 0 the rows are 16-byte aligned and A goes
# straight into LDS (transposing fragment reads); otherwise, or with the
# register flag, it is transposed in registers
MMAJOR_SHAPES = [(40, 24, 33), (130, 260, 65), (257, 129, 100), (8, 9, 10), (300, 264, 200),
                 (264, 130, 100), (512, 300, 129), (136, 520, 64)]


@pytest.mark.parametrize("algo", LDS_ALGOS + ["lds256+reg"])
@pytest.mark.parametrize("shape", MMAJOR_SHAPES)
def test_mmajor_a_bit_exact(algo, shape):
    M, N, K = shape
    for c, d, ldb in ((None, "f32", K), ("f32", "f32", (K + 7) // 8 * 8), ("f16", "f16", K + 1)):
        w = W.custom(M, N, K, a_order="m", lda=M + 8, ldb=ldb, c=c, d=d, dist="int",
                     seed=M + N + K)
        if refused(w, algo):
            continue
        x = W.make_inputs(w)
        D, checks = run_gemm(w, x, algo)
        _assert_checks(checks)
        v = verdict(D, oracle_full(w, x), w, True)
        assert v.ok, (w.name, c, d, str(v))


@pytest.mark.parametrize("algo", LDS_ALGOS)
def test_mmajor_a_float_within_tolerance(algo):
    M, N, K = 520, 264, 700
    w = W.custom(M, N, K, a_order="m", lda=M + 8, ldb=K + 8, c="f32", d="f32", dist="unif",
                 seed=11)
    if refused(w, algo):
        return
    x = W.make_inputs(w)
    D, checks = run_gemm(w, x, algo)
    _assert_checks(checks)
    v = verdict(D, oracle_full(w, x), w, False)
    assert v.ok, (w.name, str(v))


@pytest.mark.parametrize("algo", ALGOS + ["lds256+reg", "lds128+reg"])
def test_float_inputs_within_tolerance(algo):
    for (M, N, K, c, d) in ((513, 384, 300, None, "f32"), (300, 517, 1000, "f16", "f16"),
                            (256, 256, 256, "f32", "f32")):
        ld = (K + 7) // 8 * 8
        w = W.custom(M, N, K, c=c, d=d, dist="unif", seed=M + K, lda=ld, ldb=ld)
        if refused(w, algo):
            continue
        x = W.make_inputs(w)
        D, checks = run_gemm(w, x, algo)
        _assert_checks(checks)
        v = verdict(D, oracle_full(w, x), w, False)
        assert v.ok, (w.name, str(v))


@pytest.mark.parametrize("algo", LDS_ALGOS)
def test_float_fetch_paths_bit_identical(algo):
    """The fetch path carries data, not arithmetic: direct-to-LDS and
    register fetch fill the same swizzled LDS tiles, so the same fragments
    meet the same MFMAs in the same order and D agrees bit for bit on random
    inputs (K remainder and fp16 C included), where any change in the order
    of a sum would show.  Both also pass the oracle comparison."""
    for (M, N, K, c, d) in ((513, 384, 320, None, "f32"), (300, 517, 1000, "f16", "f16")):
        w = W.custom(M, N, K, c=c, d=d, dist="unif", seed=M + N + K, lda=K, ldb=K)
        x = W.make_inputs(w)
        D_dma, checks = run_gemm(w, x, algo)
        _assert_checks(checks)
        if refused(w, algo + "+reg"):
            continue
        D_reg, checks = run_gemm(w, x, algo + "+reg")
        _assert_checks(checks)
        assert np.array_equal(D_dma, D_reg), (algo, M, N, K)
        v = verdict(D_dma, oracle_full(w, x), w, False)
        assert v.ok, (w.name, str(v))


@pytest.mark.parametrize("algo", ALGOS)
def test_k_zero_gives_c(algo):
    w = W.custom(70, 50, 0, c="f32", d="f32", dist="int", seed=3, lda=8, ldb=8)
    x = W.make_inputs(w)
    D, checks = run_gemm(w, x, algo)
    _assert_checks(checks)
    assert np.array_equal(D, x.C.astype(np.float64))


def test_in_place_accumulate():
    w = W.custom(200, 136, 72, c="f32", d="f32", dist="int", seed=9)
    x = W.make_inputs(w)
    ref = oracle_full(w, x)
    D, checks = run_gemm(w, x, "lds128", in_place=True)
    _assert_checks(checks)
    assert verdict(D, ref, w, True).ok


def test_kernel_properties():
    info = mfl.kernel_info("direct")
    assert info["lds_bytes"] == 0          # the direct kernel uses no LDS
    assert mfl.kernel_info("lds128")["lds_bytes"] == 2 * (128 + 128) * 32 * 2
    assert mfl.kernel_info("lds256")["lds_bytes"] == 2 * (256 + 256) * 64 * 2
    assert mfl.kernel_info("lds256w4")["lds_bytes"] == 2 * (256 + 256) * 64 * 2
    assert mfl.kernel_info("lds128w1")["lds_bytes"] == 2 * (128 + 128) * 32 * 2
    assert mfl.kernel_info("lds256")["threads"] == 512
    assert mfl.kernel_info("lds128w1")["threads"] == 64
    assert mfl.kernel_info("splitk")["lds_bytes"] == 3 * (128 + 64) * 128 * 2   # three stages
    assert mfl.kernel_info("splitk")["threads"] == 256
    assert mfl.kernel_info("lds256w4_16")["lds_bytes"] == 2 * (256 + 256) * 64 * 2
    assert mfl.kernel_info("lds256_16")["threads"] == 512
    assert mfl.kernel_info("lds128_16")["lds_bytes"] == 2 * (128 + 128) * 64 * 2
    assert mfl.kernel_info("splitk_16")["lds_bytes"] == 3 * (128 + 64) * 128 * 2
    assert mfl.kernel_info("splitk_16")["threads"] == 512
    say("[gpu] kernel info", {a: mfl.kernel_info(a) for a in ALGOS})


# --------------------------------------------------------- named workloads
NAMED = [
    ("tiny_32x16x16", ["direct", "lds128", "lds256"], False),
    ("direct_256", ["direct"], True),
    ("lds_4096", ["lds128", "lds256", "lds256w4", "lds256+reg", "lds128w1"] + X16, True),
    ("accum_mmajor_8192x8192x2048", ["auto", "lds128", "lds256+reg", "lds256_16"], True),
    ("ragged_8191x6143x4097", ["auto", "lds128", "lds256w4", "lds128w1", "splitk",
                               "lds256w4_16"], True),
    ("shard_512x4096x4096", ["auto", "splitk", "lds128"], True),
]


def _named_cases():
    for name, algos, twin in NAMED:
        for algo in algos:
            yield pytest.param(name, algo, False, id=f"{name}-{algo}")
            if twin:
                yield pytest.param(name, algo, True, id=f"{name}-{algo}-int")


@pytest.mark.parametrize("name,algo,integer", list(_named_cases()))
def test_named_workload(name, algo, integer):
    w = W.WORKLOADS[name]
    if integer:
        w = w.twin()
    if refused(w, algo):
        return
    x = W.make_inputs(w)
    D, checks = run_gemm(w, x, algo)
    _assert_checks(checks)
    assert np.isfinite(D).all()
    ref = oracle_full_cached(w, x)
    v = verdict(D, ref, w, x.integer)
    say(f"[gpu] {w.name} {algo} every element ({D.size}): {v}")
    assert v.ok, str(v)
    if x.integer and w.d == "f32":
        assert freivalds_exact(D, w, x), "full-matrix integer check failed"

"""fp16 subnormal operands and results on the GPU, against the oracle, which
decodes every fp16 input exactly (subnormals included).

* Subnormal A (k * 2^-24, 1 <= |k| <= 1023) times small-integer B: every
  product and every partial sum is an integer multiple of 2^-24 far below
  2^24 ulps, so fp32 accumulation is exact in any order and D (fp32) must
  equal the oracle bit for bit.  A matrix core that flushed fp16 subnormal
  inputs would give 0.
* fp16 D whose exact values lie in the fp16 subnormal range (below 2^-14,
  multiples of 2^-24): representable, so the nearest-even conversion must
  return them exactly; a conversion that flushed subnormal results would
  give 0."""
import numpy as np
import pytest
import torch

import mma_fragment_layouts_tn_amd as mfl
from gpu_helpers import say
from oracle import gemm as G

pytestmark = pytest.mark.gpu

ALGOS = ["direct", "lds128", "lds256", "lds256w4", "lds128w1", "splitk", "lds256w4_16",
         "lds256_16", "lds128_16", "splitk_16"]
TINY = 2.0 ** -24   # the smallest fp16 subnormal


def _subnormal(rng, shape, kmax):
    k = rng.integers(1, kmax + 1, size=shape) * rng.choice([-1, 1], size=shape)
    return (k * TINY).astype(np.float16)


@pytest.mark.parametrize("algo", ALGOS)
def test_subnormal_inputs_exact_fp32(algo):
    M, N, K = 200, 136, 96
    rng = np.random.default_rng(71)
    A = _subnormal(rng, (M, K), 1023)
    B = rng.integers(-2, 3, size=(N, K)).astype(np.float16)
    assert np.all(np.abs(A.astype(np.float64)) < 2.0 ** -14)   # all subnormal
    D = mfl.gemm_tn(torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda(),
                    out_dtype=torch.float32, algo=algo).cpu().numpy().astype(np.float64)
    want = G.gemm_f64(M, N, K, A, K, False, B, K)
    assert np.count_nonzero(want) > 0.9 * want.size
    bad = np.argwhere(D != want)
    assert bad.size == 0, (algo, bad[:5], D[tuple(bad[0])], want[tuple(bad[0])])
    say(f"[gpu] subnormal fp16 inputs, {algo}: exact (no flush), max |D| {np.abs(want).max():.3g}")


@pytest.mark.parametrize("algo", ALGOS)
def test_subnormal_results_exact_fp16(algo):
    M, N, K = 130, 72, 64
    rng = np.random.default_rng(72)
    A = _subnormal(rng, (M, K), 3)                                # |a| <= 3 * 2^-24
    B = rng.integers(0, 2, size=(N, K)).astype(np.float16)       # 0 or 1
    D = mfl.gemm_tn(torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda(),
                    out_dtype=torch.float16, algo=algo).cpu().numpy().astype(np.float64)
    want = G.gemm_f64(M, N, K, A, K, False, B, K)
    assert np.abs(want).max() < 2.0 ** -14                      # results subnormal in fp16
    assert np.array_equal(want.astype(np.float16).astype(np.float64), want)   # representable
    assert np.count_nonzero(want) > 0.8 * want.size
    bad = np.argwhere(D != want)
    assert bad.size == 0, (algo, bad[:5], D[tuple(bad[0])], want[tuple(bad[0])])

"""Brute force over tiny ragged shapes on the GPU: M, N, K drawn from
{1..40} and the tile-edge values {63, 64, 65, 127, 128, 129}, integer inputs,
every kernel, bit-exact against the oracle (the TiledMMA page checks every
coordinate of its small configurations, section "打印布局，核对一次"; here the
check is every output element of every shape).  The draws are seeded; each
shape also varies the C and D types, the leading dimensions (16-byte rows,
so the direct-to-LDS fetch runs, or odd ones, so registers carry the tiles)
and, for every third shape, an M-contiguous A."""
import numpy as np
import pytest

import workloads as W
from gpu_helpers import oracle_full, refused, run_gemm, say, verdict

pytestmark = pytest.mark.gpu

ALGOS = ["direct", "lds128", "lds256", "lds256w4", "lds128w1", "splitk", "lds256w4_16",
         "lds256_16", "lds128_16", "splitk_16"]
SIZES = list(range(1, 41)) + [63, 64, 65, 127, 128, 129]
_rng = np.random.default_rng(20261202)
SHAPES = [(1, 1, 1), (129, 129, 129), (40, 1, 129), (1, 129, 40), (128, 64, 65), (65, 127, 63)]
SHAPES += [tuple(int(x) for x in _rng.choice(SIZES, 3)) for _ in range(42)]
CD = [(None, "f32"), ("f16", "f16"), ("f32", "f32"), (None, "f16"), ("f32", "f16"), ("f16", "f32")]


@pytest.mark.parametrize("algo", ALGOS)
def test_tiny_ragged_shapes_bit_exact(algo):
    ran = 0
    for idx, (M, N, K) in enumerate(SHAPES):
        c, d = CD[idx % len(CD)]
        aligned = idx % 2 == 0
        mmajor = idx % 3 == 2 and algo != "direct"
        ld = (K + 7) // 8 * 8 + 8 if aligned else K + 1
        if mmajor:
            lda = (M + 7) // 8 * 8 + 8 if aligned else M + 3
            w = W.custom(M, N, K, a_order="m", lda=lda, ldb=ld, c=c, d=d, dist="int",
                         seed=1000 + idx)
        else:
            w = W.custom(M, N, K, lda=ld, ldb=ld, c=c, d=d, dist="int", seed=1000 + idx)
        if refused(w, algo):
            continue
        x = W.make_inputs(w)
        D, checks = run_gemm(w, x, algo)
        assert all(checks.values()), (w.name, checks)
        v = verdict(D, oracle_full(w, x), w, True)
        assert v.ok, (algo, w.name, w.a_order, c, d, w.lda_, w.ldb_, str(v))
        ran += 1
    say(f"[gpu] tiny sweep {algo}: {ran} shapes bit-exact")
    assert ran >= len(SHAPES) // 3     # configurations without register fetch skip the rest

"""The seeded input generator: determinism, layouts, poison and ranges."""
import numpy as np

import workloads as W


def test_deterministic_and_ordered_draws():
    w = W.custom(20, 12, 9, c="f32", seed=7)
    a, b = W.make_inputs(w), W.make_inputs(w)
    assert np.array_equal(a.A, b.A) and np.array_equal(a.B, b.B) and np.array_equal(a.C, b.C)
    rng = np.random.default_rng(7)
    assert np.array_equal(a.A, rng.uniform(-1, 1, (20, 9)).astype(np.float16))
    assert np.array_equal(a.B, rng.uniform(-1, 1, (12, 9)).astype(np.float16))


def test_mmajor_layout_and_poison():
    w = W.custom(10, 4, 6, a_order="m", lda=13, seed=1)
    x = W.make_inputs(w)
    assert x.A.shape == (6, 13)
    vals = np.random.default_rng(1).uniform(-1, 1, (10, 6)).astype(np.float16)
    assert np.array_equal(x.A[:, :10], vals.T)
    assert np.isnan(x.A[:, 10:].astype(np.float32)).all()


def test_integer_twin_range():
    w = W.WORKLOADS["direct_256"].twin()
    x = W.make_inputs(w)
    assert w.seed == 102 and x.integer
    u = np.unique(x.A.astype(np.float32))
    assert set(u.tolist()) == {-2.0, -1.0, 0.0, 1.0, 2.0}


def test_named_workloads():
    c = W.WORKLOADS
    assert (c["lds_4096"].M, c["lds_4096"].N, c["lds_4096"].K) == (4096, 4096, 4096)
    assert c["accum_mmajor_8192x8192x2048"].lda_ == 8200
    r = c["ragged_8191x6143x4097"]
    assert (r.lda_, r.ldb_, r.ldc_, r.ldd_) == (4097, 4097, 6143, 6143)
    assert c["lds_4096"].flops == 2 * 4096 ** 3
    assert c["lds_4096"].algorithmic_bytes() == 2 * 2 * 4096 * 4096 + 4 * 4096 * 4096


def test_sample_indices_cover_edges():
    ms, ns = W.sample_indices(300, 200, 50, seed=0)
    pts = set(zip(ms.tolist(), ns.tolist()))
    assert (299, 199) in pts and (0, 0) in pts and (128, 0) in pts and (0, 127) in pts
    assert ms.max() < 300 and ns.max() < 200

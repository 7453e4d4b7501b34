"""Pins for the oracle's binary16 helpers and acceptance rules."""
import math

import numpy as np
import pytest

from oracle import compare, fp16


def test_decode_all_bit_patterns_vs_numpy():
    bits = np.arange(1 << 16, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    mine = fp16.decode_array(bits)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(mine))
    assert np.array_equal(ref[~nan], mine[~nan])
    # sign of zero survives
    assert math.copysign(1.0, fp16.decode_bits(0x8000)) < 0


def test_known_patterns():
    assert fp16.decode_bits(0x3C00) == 1.0
    assert fp16.decode_bits(0x7BFF) == 65504.0
    assert fp16.decode_bits(0x0001) == 2.0 ** -24
    assert fp16.decode_bits(0x0400) == 2.0 ** -14
    assert fp16.decode_bits(0xC000) == -2.0


def test_encode_rne_vs_numpy_including_ties():
    rng = np.random.default_rng(0)
    xs = list(rng.standard_normal(4000) * 10.0 ** rng.uniform(-9, 5, 4000))
    # exact ties between neighbours, in every binade and among subnormals
    for e in range(-24, 16):
        for f in (0, 1, 2, 3, 1021, 1022):
            lo = (1024 + f) * 2.0 ** (e - 10) if e >= -14 else f * 2.0 ** -24
            step = 2.0 ** (max(e, -14) - 10)
            xs += [lo + step / 2, -(lo + step / 2), lo + step / 2 * (1 + 2 ** -30)]
    xs += [65504.0, 65519.99, 65520.0, 1e6, 2.0 ** -25, 3 * 2.0 ** -25, 0.0, -0.0]
    for x in xs:
        with np.errstate(over="ignore"):
            want = int(np.array([x]).astype(np.float16).view(np.uint16)[0])
        assert fp16.encode_rne(float(x)) == want, x


def test_rne16_array_matches_encoder():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(2000) * 1000
    got = fp16.rne16_array(x)
    want = [fp16.decode_bits(fp16.encode_rne(float(v))) for v in x]
    assert np.array_equal(got, np.array(want))


def test_ulp16():
    assert fp16.ulp16(1.0) == 2.0 ** -10
    assert fp16.ulp16(0.999) == 2.0 ** -11
    assert fp16.ulp16(65504.0) == 32.0
    assert fp16.ulp16(2.0 ** -20) == 2.0 ** -24
    assert fp16.ulp16(0.0) == 2.0 ** -24
    assert fp16.ulp16(-3.0) == 2.0 ** -9
    x = np.array([1.0, 0.999, 65504.0, 2.0 ** -20, 0.0, -3.0, 2048.0, 2047.9])
    assert np.array_equal(fp16.ulp16_array(x), np.array([fp16.ulp16(v) for v in x]))
    # ulp is the gap between consecutive binary16 values
    for h in range(0x0400, 0x7BFF, 97):
        v = fp16.decode_bits(h)
        assert fp16.decode_bits(h + 1) - v == fp16.ulp16(v)


def test_compare_rules():
    ref = np.array([[1.0, 2.5], [-3.0, 4096.0 + 1]])
    ok = compare.check(ref.astype(np.float32), ref, "f32", 16, True)
    assert ok.ok
    bad = ref.astype(np.float32).copy()
    bad[0, 1] += 2 ** -20
    assert not compare.check(bad, ref, "f32", 16, True).ok
    # fp16 exact rule rounds 4097 to 4096 (ties to even)
    d16 = fp16.rne16_array(ref)
    assert d16[1, 1] == 4096.0
    assert compare.check(d16, ref, "f16", 16, True).ok
    # float tolerance
    K = 400
    tol = 1e-4 * math.sqrt(K)
    near = ref + tol * 0.9
    assert compare.check(near, ref, "f32", K, False).ok
    assert not compare.check(ref + tol * 1.1, ref, "f32", K, False).ok
    lim = fp16.ulp16_array(ref) + tol
    assert compare.check(ref + lim * 0.99, ref, "f16", K, False).ok
    assert not compare.check(ref + lim * 1.01, ref, "f16", K, False).ok
    nan = ref.copy()
    nan[0, 0] = np.nan
    assert not compare.check(nan, ref, "f32", K, False).ok
    # signed zeros compare equal
    assert compare.check(np.array([-0.0]), np.array([0.0]), "f32", 1, True).ok

"""Back-to-back GEMM on the GPU (gemm_tn_chain through the C ABI) against
the oracle chain (oracle/chain.py): D_b = rne16(A_b B_b^T) W_b^T.

* integer inputs: bit-exact (S stays exact in fp16, D in fp32; fp16 D is
  the nearest-even rounding of the exact D);
* random inputs: every element within the bound ``chain_tolerance`` derives
  from fp32 summation and the rounding of S (fp16 D: plus one rounding);
  uniform inputs, and dyadic ones (A and B on a 2^-6 grid) for which the
  first sum is exact in fp32 and the bound charges no rounding flip of S;
* the attention-shaped workload at full size, every element of every batch;
* ragged M, N1 and N2, N1 not a multiple of the 32-wide chunk, N1 = 0,
  padded rows, shared (stride 0) operands, guard canaries after every buffer.
"""
import numpy as np
import pytest
import torch

import mma_fragment_layouts_tn_amd as mfl
import workloads as W
from gpu_helpers import GUARD, Guarded, out_buffer, say
from oracle import chain as CH
from oracle import fp16

pytestmark = pytest.mark.gpu

STAGINGS_SEEN = set()   # (staging, K) of every launch in this module
LAST = {}               # staging and N2 tile of the latest launch


def run_chain(x: W.ChainInputs, d: str, share=(False, False, False)):
    """Upload, call gemm_tn_chain, download.  share[i]: operand i (A, B, W)
    is passed with batch stride 0 (its batch 0 serves every batch)."""
    w = x.w
    say(f"[gpu] chain {w.name} batch={w.batch} M={w.M} N1={w.N1} N2={w.N2} K={w.K} d={d} "
        f"share={share} int={x.integer}")
    bufs = []
    args = []
    for X, sh in zip((x.A, x.B, x.W), share):
        g = Guarded(X[:1] if sh else X)
        bufs.append(g)
        args += [g.ptr, X.shape[2], 0 if sh else X.shape[1] * X.shape[2]]
    ldd = max(w.N2, 1)
    Dt = out_buffer(w.batch * w.M, ldd, d)
    dk = mfl.F16 if d == "f16" else mfl.F32
    rc, staging, tile_n = mfl.gemm_chain_plan(w.batch, w.M, w.N1, w.N2, w.K, *args,
                                              Dt.data_ptr(), ldd, w.M * ldd, dk)
    assert rc == 0, mfl.strerror(rc)
    say(f"[gpu]   staging {staging}, N2 tile {tile_n}")
    STAGINGS_SEEN.add((staging, w.K, tile_n))
    LAST.update(staging=staging, tile_n=tile_n)
    rc = mfl.gemm_chain_raw(w.batch, w.M, w.N1, w.N2, w.K, *args, Dt.data_ptr(), ldd,
                            w.M * ldd, dk, torch.cuda.current_stream().cuda_stream)
    assert rc == 0, mfl.strerror(rc)
    torch.cuda.synchronize()
    n = w.batch * w.M * ldd
    raw = Dt.cpu()
    if d == "f16":
        D = raw[:n].numpy().view(np.float16).astype(np.float64)
    else:
        D = raw[:n].numpy().view(np.float32).astype(np.float64)
    guard_ok = torch.equal(raw[n:], out_buffer(0, 0, d, dev="cpu")[:GUARD]) if GUARD else True
    checks = {"D guard": guard_ok, "inputs unchanged": all(g.unchanged() for g in bufs)}
    return D.reshape(w.batch, w.M, ldd)[:, :, :w.N2], checks


def oracle_chain(x: W.ChainInputs, share=(False, False, False), with_s=False):
    w = x.w
    ops = []
    for X, sh in zip((x.A, x.B, x.W), share):
        ops += [X, X.shape[2], 0 if sh else X.shape[1] * X.shape[2]]
    return CH.chain_f64(w.batch, w.M, w.N1, w.N2, w.K, *ops, with_s=with_s)


def _logical(X, cols):
    return X[:, :, :cols].astype(np.float64)


SHAPES = [  # batch, M, N1, N2, K
    (1, 32, 32, 32, 32), (1, 256, 64, 128, 64), (2, 300, 100, 130, 128),
    (3, 257, 33, 129, 256), (1, 1, 1, 1, 32), (2, 512, 1000, 64, 128), (1, 70, 31, 200, 64),
    (2, 300, 96, 130, 256), (1, 130, 160, 70, 32), (2, 256, 288, 256, 128),
    (1, 130, 192, 70, 32), (2, 256, 128, 256, 128),
    # N2 tiles of 64: whole chunks (direct-to-LDS when aligned) at every K
    (2, 100, 128, 48, 32), (1, 90, 192, 64, 64), (2, 260, 256, 40, 128), (1, 200, 64, 64, 256),
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("d", ["f32", "f16"])
@pytest.mark.parametrize("rows", ["padded", "aligned"])
def test_integer_bit_exact(shape, d, rows):
    """padded: A and W rows off 16-byte alignment (register staging);
    aligned: 16-byte rows, direct-to-LDS staging wherever N1 fills whole
    chunks (64 columns, 32 at K = 256)."""
    bt, M, N1, N2, K = shape
    ld = dict(lda=K + 8, ldw=N1 + 3) if rows == "padded" else dict(ldw=-(-N1 // 8) * 8 or 8)
    w = W.ChainWorkload("int", bt, M, N1, N2, K, d=d, dist="int", seed=sum(shape), **ld)
    x = W.make_chain_inputs(w)
    D, checks = run_chain(x, d)
    assert all(checks.values()), checks
    ref = oracle_chain(x)
    want = fp16.rne16_array(ref) if d == "f16" else ref
    bad = np.argwhere(D != want)
    assert bad.size == 0, (shape, d, bad[:5], D[tuple(bad[0])], want[tuple(bad[0])])


@pytest.mark.parametrize("K", [32, 64, 128, 256])
def test_odd_leading_dims(K):
    """Rows of A, B and W only 2-byte aligned (odd leading dimensions): A's
    fragments and B's register staging use unaligned 16-byte loads."""
    w = W.ChainWorkload("odd", 2, 140, 100, 70, K, d="f32", dist="int", seed=K,
                        lda=K + 1, ldb=K + 3, ldw=101)
    x = W.make_chain_inputs(w)
    D, checks = run_chain(x, "f32")
    assert all(checks.values()), checks
    assert np.array_equal(D, oracle_chain(x))


def test_n1_zero_gives_zero():
    w = W.ChainWorkload("n1zero", 2, 40, 0, 70, 64, d="f32", dist="int", seed=3)
    x = W.make_chain_inputs(w)
    D, checks = run_chain(x, "f32")
    assert all(checks.values()), checks
    assert (D == 0).all()


@pytest.mark.parametrize("share", [(True, False, False), (False, True, True), (True, True, True)])
@pytest.mark.parametrize("N1", [96, 128])   # register / direct-to-LDS staging at K = 128
def test_shared_operands(share, N1):
    w = W.ChainWorkload("share", 3, 130, N1, 100, 128, d="f32", dist="int", seed=5)
    x = W.make_chain_inputs(w)
    D, checks = run_chain(x, "f32", share)
    assert all(checks.values()), checks
    assert np.array_equal(D, oracle_chain(x, share))


def _float_bound(x, S, P, d, D_ref):
    w = x.w
    tol = np.stack([CH.chain_tolerance(_logical(x.A[b:b + 1], w.K)[0],
                                       _logical(x.B[b:b + 1], w.K)[0],
                                       _logical(x.W[b:b + 1], w.N1)[0], S[b], P[b])
                    for b in range(w.batch)])
    if d == "f16":
        tol = tol + fp16.ulp16_array(np.abs(D_ref) + tol)
    return tol


@pytest.mark.parametrize("shape", [(2, 300, 200, 130, 128), (1, 256, 1024, 128, 64),
                                   (1, 100, 77, 60, 256), (2, 260, 128, 200, 256)])
@pytest.mark.parametrize("d", ["f32", "f16"])
@pytest.mark.parametrize("dist", ["unif", "dyadic"])
def test_float_within_derived_bound(shape, d, dist):
    bt, M, N1, N2, K = shape
    w = W.ChainWorkload("float", bt, M, N1, N2, K, d=d, dist=dist, seed=sum(shape) + 1)
    x = W.make_chain_inputs(w)
    D, checks = run_chain(x, d)
    assert all(checks.values()), checks
    ref, S, P = oracle_chain(x, with_s=True)
    want = fp16.rne16_array(ref) if d == "f16" else ref
    tol = _float_bound(x, S, P, d, ref)
    err = np.abs(D - want)
    assert np.isfinite(D).all()
    assert (err <= tol).all(), (shape, d, dist, float((err - tol).max()))
    say(f"[gpu] chain {dist} {shape} {d}: max err {err.max():.3g}, max bound {tol.max():.3g}, "
        f"max |D| {np.abs(ref).max():.3g}")


@pytest.mark.parametrize("name", sorted(W.CHAIN_WORKLOADS))
@pytest.mark.parametrize("integer", [False, True])
def test_named_workload(integer, name):
    """The attention-shaped workloads at full size, in the launch the bench
    times: every element of every batch against the oracle, batch by batch
    (integer inputs bit-exact, random ones within the derived bound)."""
    w = W.CHAIN_WORKLOADS[name]
    if integer:
        w = w.twin()
    x = W.make_chain_inputs(w)
    D, checks = run_chain(x, w.d)
    assert all(checks.values()), checks
    assert np.isfinite(D).all()
    worst = 0.0
    for b in range(w.batch):
        sub = W.ChainInputs(W.ChainWorkload("batch", 1, w.M, w.N1, w.N2, w.K, d=w.d),
                            x.A[b:b + 1], x.B[b:b + 1], x.W[b:b + 1], x.integer)
        ref, S, P = oracle_chain(sub, with_s=True)
        want = fp16.rne16_array(ref) if w.d == "f16" else ref
        got = D[b:b + 1]
        if integer:
            assert np.array_equal(got, want), b
        else:
            tol = _float_bound(sub, S, P, w.d, ref)
            err = np.abs(got - want)
            assert (err <= tol).all(), (b, float((err - tol).max()))
            worst = max(worst, float((err / tol).max()))
    say(f"[gpu] chain named workload int={integer}: all {w.batch}x{w.M}x{w.N2} elements "
        f"checked; largest error / bound {worst:.3g}")


@pytest.mark.parametrize("K", [32, 64, 128, 256])
def test_float_stagings_bit_identical(K):
    """The staging path carries data, not arithmetic: with N1 in whole
    chunks, direct-to-LDS (16-byte rows) and register staging (rows off
    alignment) put the same fragments in front of the same MFMAs in the same
    order, so D agrees bit for bit on random inputs, where any change in the
    order of a sum would show.  Both also sit within the oracle's bound."""
    bt, M, N1, N2 = 2, 300, 128, 130
    w = W.ChainWorkload("stg", bt, M, N1, N2, K, d="f32", dist="unif", seed=K + 7)
    x = W.make_chain_inputs(w)

    def padded(X, cols, extra):
        out = np.zeros(X.shape[:2] + (cols + extra,), X.dtype)
        out[:, :, :cols] = X[:, :, :cols]
        return out

    xp = W.ChainInputs(w, padded(x.A, K, 8), x.B, padded(x.W, N1, 3), x.integer)
    D_dma, checks = run_chain(x, "f32")
    assert all(checks.values()), checks
    assert LAST["staging"] == "dma", LAST
    D_reg, checks = run_chain(xp, "f32")
    assert all(checks.values()), checks
    assert LAST["staging"] == "regs", LAST
    assert np.array_equal(D_dma, D_reg)
    ref, S, P = oracle_chain(x, with_s=True)
    assert (np.abs(D_dma - ref) <= _float_bound(x, S, P, "f32", ref)).all()


def test_phase_probe_matches_and_stamps_are_ordered():
    """The timed instance behind the phase breakdown computes what the
    product computes: D bit-identical to gemm_tn_chain on the same inputs,
    and each wave's shader-clock stamps rise through every iteration's four
    phases, the loop and the epilogue."""
    w = W.ChainWorkload("phases", 4, 512, 1024, 128, 128, d="f16", dist="unif", seed=31)
    x = W.make_chain_inputs(w)
    D_ref, checks = run_chain(x, "f16")
    assert all(checks.values()), checks
    dev = torch.device("cuda", 0)
    A, B, Wt = (torch.from_numpy(np.ascontiguousarray(t)).to(dev) for t in (x.A, x.B, x.W))
    D = torch.full((w.batch, w.M, w.N2), float("nan"), dtype=torch.float16, device=dev)
    stamps = torch.zeros(int(np.prod(mfl.CHAIN_STAMP_SHAPE)), dtype=torch.int32, device=dev)
    say(f"[gpu] chain phase probe batch={w.batch} M={w.M} N1={w.N1} N2={w.N2} K={w.K}")
    rc = mfl.probe_chain_phases_raw(w.batch, w.M, w.N1, w.N2, w.K,
                                    A.data_ptr(), w.K, w.M * w.K, B.data_ptr(), w.K, w.N1 * w.K,
                                    Wt.data_ptr(), w.N1, w.N2 * w.N1, D.data_ptr(), w.N2,
                                    w.M * w.N2, mfl.F16, stamps.data_ptr(),
                                    torch.cuda.current_stream().cuda_stream)
    assert rc == 0, mfl.strerror(rc)
    torch.cuda.synchronize()
    assert np.array_equal(D.cpu().numpy().astype(np.float64), D_ref)
    t = stamps.view(*mfl.CHAIN_STAMP_SHAPE).cpu().numpy().astype(np.int64) & 0xFFFFFFFF
    nch = w.N1 // 64
    for blk in range(mfl.CHAIN_STAMP_SHAPE[0]):
        for wave in range(mfl.CHAIN_STAMP_SHAPE[1]):
            s = t[blk, wave]
            seq = [s[256]]
            for c in range(nch - 1):
                seq += list(s[4 * c:4 * c + 4])
            seq += [s[4 * (nch - 1)], s[257], s[258]]
            steps = np.diff(np.array(seq)) % (1 << 32)
            assert (steps < (1 << 24)).all(), (blk, wave, steps.max())   # no step backwards
            assert steps.sum() > 0, (blk, wave)

def test_every_kernel_variant_ran():
    """Collected after the cases above: each K ran through both stagings
    with both N2 tile widths."""
    for K in (32, 64, 128, 256):
        for staging in ("dma", "regs"):
            for tile_n in (64, 128):
                assert (staging, K, tile_n) in STAGINGS_SEEN, (staging, K, tile_n,
                                                               sorted(STAGINGS_SEEN))

"""Per-lane fragment coordinates read back from the GPU (mfl_probe_fragments).

The kernels' index maps are asserted at compile time and checked on the host
(test_layout_module.py) as the constexpr functions the kernels compile.  This
test checks what the compiled kernels actually do: one K-step of each LDS
configuration runs on inputs whose values encode their coordinates, and every
thread dumps its operand fragment registers and accumulators instead of the
epilogue.  Four input pairs, all exact in fp16 and in the fp32 sums:

  A(m,k) = m+1, B(n,k) = n+1        fragment values give the row of each slot
  A(m,k) = k+1, B(n,k) = k+1        ... and its k
  A(m,k) = (m+1)[k=0], B = [k=0]    accumulator (i, j, v) gives its m
  A = [k=0], B(n,k) = (n+1)[k=0]    ... and its n

Every lane's every slot is compared with the oracle's closed-form gfx950 MFMA
maps (oracle/layout.py) placed in the workgroup tile the way the kernel
design states it: wave (wm, wn, wk), repeat (i, j), K sub-step, and the N
permutation the B fetch applies.  This is the per-thread coordinate dump the
simple-GEMM page prints for thread 0 ("cute(7) simple_gemm" §4), for every
lane of every configuration and fetch path."""
import numpy as np
import pytest
import torch

import mma_fragment_layouts_tn_amd as mfl
from gpu_helpers import say
from oracle import layout as L

pytestmark = pytest.mark.gpu

DMA, REG, REGT, DMAT = 0, 1, 2, 3
A32, A16 = "f32_32x32x16_f16", "f32_16x16x32_f16"
# BM, BN, BK, waves M, N, K, fragment distance, instruction
CFG = {"lds128": (128, 128, 32, 2, 2, 1, 1, A32), "lds256": (256, 256, 64, 2, 4, 1, 1, A32),
       "lds256w4": (256, 256, 64, 2, 2, 1, 2, A32), "lds128w1": (128, 128, 32, 1, 1, 1, 1, A32),
       "splitk": (128, 64, 128, 1, 1, 4, 1, A32), "lds256w4_16": (256, 256, 64, 2, 2, 1, 1, A16),
       "lds256_16": (256, 256, 64, 2, 4, 1, 1, A16), "lds128_16": (128, 128, 64, 2, 2, 1, 1, A16),
       "splitk_16": (128, 64, 128, 4, 1, 2, 1, A16)}
ATOM = {A32: (32, 16, 16), A16: (16, 32, 4)}      # atom M = N, atom K, accumulator values
CASES = [(a, DMA, DMA) for a in CFG] + [("lds256", REG, REG), ("lds256", REGT, DMA),
                                        ("lds256", DMAT, DMA), ("lds256w4_16", REG, REG),
                                        ("lds256w4_16", DMAT, DMA)]


def _perm_n(n, WTN, RN, AN):
    V = min(RN, 4)
    w, r = divmod(n, WTN)
    j, c = divmod(r, AN)
    return w * WTN + AN * V * (j // V) + V * c + j % V


def _dump(algo, fa, fb, a_val, b_val, M, N, K):
    """a_val(m, k), b_val(n, k): values on the index grids."""
    m, k = np.meshgrid(np.arange(M), np.arange(K), indexing="ij")
    a = a_val(m, k).astype(np.float16)
    n, kb = np.meshgrid(np.arange(N), np.arange(K), indexing="ij")
    b = b_val(n, kb).astype(np.float16)
    if fa in (DMAT, REGT):            # M-contiguous A: (K, lda), lda = M + 8
        lda = M + 8
        buf = np.zeros((K, lda), np.float16)
        buf[:, :M] = a.T
    else:
        lda = K + 8
        buf = np.zeros((M, lda), np.float16)
        buf[:, :K] = a
    ldb = K + 8                       # rows padded to 16-byte multiples
    bbuf = np.zeros((N, ldb), np.float16)
    bbuf[:, :K] = b
    A = torch.from_numpy(buf).cuda()
    B = torch.from_numpy(bbuf).cuda()
    return mfl.probe_fragments(algo, fa, fb, A, lda, B, ldb, M, N, K)


@pytest.mark.parametrize("algo,fa,fb", CASES, ids=[f"{a}-{f}{g}" for a, f, g in CASES])
def test_registers_hold_the_atom_layout_coordinates(algo, fa, fb):
    BM, BN, BK, WM, WN, WK, dist, op = CFG[algo]
    AM, AK, NV = ATOM[op]
    M, N, K = BM, BN, BK
    RM, RN = BM // WM // AM, BN // WN // AM
    KW = BK // AK // WK
    nbuf = 2 if dist == 1 else KW
    # sub-step each register buffer holds after the kernel's one K-step
    sub = [KW - 2 + b for b in range(2)] if dist == 1 else list(range(KW))
    say(f"[gpu] fragment dump {algo} fetch {fa}/{fb}: {BM}x{BN}x{BK}, {RM}x{RN} atoms {op}")
    rows = _dump(algo, fa, fb, lambda m, k: m + 1, lambda n, k: n + 1, M, N, K)[0]
    ks = _dump(algo, fa, fb, lambda m, k: k + 1, lambda n, k: k + 1, M, N, K)[0]
    accm = _dump(algo, fa, fb, lambda m, k: (m + 1) * (k == 0), lambda n, k: 1.0 * (k == 0),
                 M, N, K)[0]
    accn = _dump(algo, fa, fb, lambda m, k: 1.0 * (k == 0), lambda n, k: (n + 1) * (k == 0),
                 M, N, K)[0]
    T = rows.shape[0]
    fw = nbuf * (RM + RN) * 4

    def frags(d):      # (T, nbuf, RM+RN, 8) fragment values
        return d[:, :fw].copy().view(np.uint16).view(np.float16).reshape(T, nbuf, RM + RN, 8) \
            .astype(np.int64)

    def accs(d):       # (T, RM, RN, NV)
        return d[:, fw:].copy().view(np.float32).reshape(T, RM, RN, NV).astype(np.int64)

    fr, fk, am, an = frags(rows), frags(ks), accs(accm), accs(accn)
    want_r = np.zeros_like(fr)
    want_k = np.zeros_like(fk)
    want_am = np.zeros_like(am)
    want_an = np.zeros_like(an)
    for t in range(T):
        w, lane = divmod(t, 64)
        wm, wn, wk = w % WM, (w // WM) % WN, w // (WM * WN)
        for b in range(nbuf):
            kk = wk * KW + sub[b]
            for v in range(8):
                r, ka = L.mfma_ab_coord(op, lane, v)
                for i in range(RM):
                    want_r[t, b, i, v] = wm * (BM // WM) + AM * i + r + 1
                    want_k[t, b, i, v] = AK * kk + ka + 1
                for j in range(RN):
                    n_log = wn * (BN // WN) + AM * j + r
                    want_r[t, b, RM + j, v] = _perm_n(n_log, BN // WN, RN, AM) + 1
                    want_k[t, b, RM + j, v] = AK * kk + ka + 1
        sees_k0 = wk == 0           # only the first K-group's sub-steps hold k = 0
        for v in range(NV):
            mc, nc = L.mfma_c_coord(op, lane, v)
            for i in range(RM):
                for j in range(RN):
                    mm = wm * (BM // WM) + AM * i + mc
                    nn = _perm_n(wn * (BN // WN) + AM * j + nc, BN // WN, RN, AM)
                    want_am[t, i, j, v] = (mm + 1) if sees_k0 else 0
                    want_an[t, i, j, v] = (nn + 1) if sees_k0 else 0
    for what, got, want in (("fragment rows", fr, want_r), ("fragment k", fk, want_k),
                            ("accumulator m", am, want_am), ("accumulator n", an, want_an)):
        bad = np.argwhere(got != want)
        assert bad.size == 0, (algo, fa, fb, what, bad[:4].tolist(),
                               [(int(got[tuple(x)]), int(want[tuple(x)])) for x in bad[:4]])

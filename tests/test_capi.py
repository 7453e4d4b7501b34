"""The C ABI without a GPU: every declared symbol is exported, and the
argument checks return the documented codes (gemm_tn_validate runs the same
checks gemm_tn runs before launching)."""
import glob
import os
import re
import subprocess

import pytest

import mma_fragment_layouts_tn_amd as mfl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
P = 0x10000          # a fake, aligned device address (never dereferenced)


def _declared():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:int|const char\*|void)\s+(\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return names


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert {"gemm_tn", "gemm_tn_validate", "gemm_strerror", "mfl_layout_compose",
            "mfl_probe_mfma"} <= names
    out = subprocess.run(["nm", "-D", "--defined-only", mfl.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.strip()}
    missing = names - exported
    assert not missing, missing
    for n in names:
        assert hasattr(mfl.lib, n)


def _v(M=64, N=64, K=64, A=P, lda=None, B=P, ldb=None, C=None, ldc=0, D=P, ldd=None, **kw):
    dt = mfl.dtypes(**kw)
    lda = lda if lda is not None else (K if dt.a_order == mfl.A_KMAJOR else M)
    ldb = ldb if ldb is not None else K
    ldd = ldd if ldd is not None else N
    return mfl.validate(M, N, K, A, lda, B, ldb, C, ldc, D, ldd, dt)


def test_valid_cases():
    assert _v()[0] == 0
    assert _v(c=mfl.F32, C=P + 0x100000, ldc=64)[0] == 0
    assert _v(a_order=mfl.A_MMAJOR, lda=72)[0] == 0
    assert _v(M=8191, N=6143, K=4097, c=mfl.F16, d=mfl.F16, C=P, ldc=6143)[0] == 0


@pytest.mark.parametrize("kw,code", [
    (dict(M=-1), -1), (dict(K=-5), -1),
    (dict(lda=63), -2), (dict(ldb=10), -2), (dict(ldd=63), -2),
    (dict(c=mfl.F16, C=P, ldc=63), -2),
    (dict(a_order=mfl.A_MMAJOR, lda=63), -2),
    (dict(A=0), -3), (dict(B=0), -3), (dict(D=0), -3),
    (dict(c=mfl.F32, ldc=64), -3), (dict(C=P + 4096, ldc=64), -3),
    (dict(d=mfl.NONE), -4), (dict(c=7, C=P, ldc=64), -4), (dict(a_order=2), -4),
    (dict(algo=11), -4),
    (dict(a_order=mfl.A_MMAJOR, algo=1), -6),
    # the 16x16x32 configurations have no register-transposing fetch for an
    # M-contiguous A: rows off 16-byte alignment need a 32x32x16 one
    (dict(a_order=mfl.A_MMAJOR, lda=65, algo=7), -6),
    (dict(a_order=mfl.A_MMAJOR, lda=64, algo=7 | 0x100), -6),
    (dict(algo=0x200), -4), (dict(algo=12), -4),
    (dict(A=P + 1), -7), (dict(d=mfl.F32, D=P + 2), -7),
    (dict(c=mfl.F16, C=P, ldc=64, d=mfl.F32, D=P), -8),
    (dict(c=mfl.F32, C=P, ldc=128, d=mfl.F32, D=P, ldd=64), -8),
    (dict(M=1 << 20, K=1 << 11, lda=1 << 11), -9),
])
def test_error_codes(kw, code):
    assert _v(**kw)[0] == code
    assert mfl.strerror(code) not in ("", "unknown error code")


def test_in_place_accumulate_allowed():
    assert _v(c=mfl.F32, C=P, ldc=64, d=mfl.F32, D=P)[0] == 0


def test_degenerate_sizes_are_ok():
    assert _v(M=0)[0] == 0
    assert _v(N=0, D=0, ldd=1)[0] == 0
    assert _v(K=0, A=0, B=0, lda=1, ldb=1)[0] == 0


def _plan(M=64, N=64, K=64, A=P, lda=None, B=P, ldb=None, **kw):
    dt = mfl.dtypes(**kw)
    lda = lda if lda is not None else (K if dt.a_order == mfl.A_KMAJOR else M)
    ldb = ldb if ldb is not None else K
    return mfl.plan(M, N, K, A, lda, B, ldb, None, 0, P, N, dt)


def test_fetch_policy_choice():
    DMA, REG, REGT, DMAT = 0, 1, 2, 3
    assert _plan(M=4096, N=4096, K=4096)[1:] == (mfl.ALGOS["lds256_16"], DMA, DMA)
    assert _plan(M=4096, N=4096, K=4097, lda=4097, ldb=4097)[1:] == (mfl.ALGOS["lds256"], REG, REG)
    assert _plan(lda=72, ldb=68)[2:] == (DMA, REG)
    assert _plan(A=P + 2, lda=64)[2:] == (REG, DMA)
    assert _plan(a_order=mfl.A_MMAJOR, lda=72)[2:] == (DMAT, DMA)
    assert _plan(a_order=mfl.A_MMAJOR, lda=68)[2:] == (REGT, DMA)           # rows not 16-byte
    assert _plan(M=60, a_order=mfl.A_MMAJOR, lda=72)[2:] == (REGT, DMA)     # M % 8 != 0
    assert _plan(a_order=mfl.A_MMAJOR, lda=72, A=P + 8)[2:] == (REGT, DMA)
    assert _plan(a_order=mfl.A_MMAJOR, lda=72, algo=mfl.algo_code("lds256+reg"))[2:] == (REGT, REG)
    assert _plan(M=8192, N=8192, K=2048, a_order=mfl.A_MMAJOR, lda=8200)[1:] == (
        mfl.ALGOS["lds256"], DMAT, DMA)
    assert _plan(algo=mfl.ALGOS["lds256"] | mfl.REG_FETCH)[1:] == (mfl.ALGOS["lds256"], REG, REG)
    assert _plan(algo=mfl.algo_code("lds128+reg"))[2:] == (REG, REG)


def test_auto_choice():
    assert _v(M=4096, N=4096, K=4096)[1] == mfl.ALGOS["lds256_16"]
    assert _v(M=4096, N=4096, K=4096, c=mfl.F32, C=P, ldc=4096)[1] == mfl.ALGOS["lds256"]
    assert _v(M=4096, N=4096, K=4096, lda=4100)[1] == mfl.ALGOS["lds256"]
    assert _v(M=256, N=256, K=256)[1] == mfl.ALGOS["lds128"]
    assert _v(M=32, N=16, K=16, algo=1)[1] == mfl.ALGOS["direct"]
    # fewer 128x128 tiles than CUs and a long K: split K inside the workgroup,
    # on the 16x16x32 tile when both operands go straight into LDS and C is
    # absent, else on the 32x32x16 one
    assert _v(M=512, N=4096, K=4096)[1] == mfl.ALGOS["splitk_16"]
    assert _v(M=256, N=4096, K=8192)[1] == mfl.ALGOS["splitk_16"]
    assert _v(M=512, N=4096, K=4096, lda=4100)[1] == mfl.ALGOS["splitk"]
    assert _v(M=512, N=4096, K=4096, c=mfl.F32, C=P, ldc=4096)[1] == mfl.ALGOS["splitk"]
    assert _v(M=512, N=4096, K=512)[1] == mfl.ALGOS["lds128"]       # K too short
    assert _v(M=1024, N=4096, K=4096)[1] == mfl.ALGOS["lds128"]     # 256 tiles fill the CUs


def test_binding_rejects_cpu_tensors():
    import torch
    a = torch.zeros(4, 4, dtype=torch.float16)
    with pytest.raises(ValueError):
        mfl.gemm_tn(a, a)


# ------------------------------------------------------- back-to-back GEMM
def _cv(batch=2, M=100, N1=300, N2=128, K=128, A=P, lda=None, sa=None, B=P, ldb=None, sb=None,
        W=P, ldw=None, sw=None, D=P, ldd=None, sd=None, d=mfl.F16):
    lda = K if lda is None else lda
    ldb = K if ldb is None else ldb
    ldw = max(N1, 1) if ldw is None else ldw
    ldd = max(N2, 1) if ldd is None else ldd
    sa = M * lda if sa is None else sa
    sb = N1 * ldb if sb is None else sb
    sw = N2 * ldw if sw is None else sw
    sd = M * ldd if sd is None else sd
    return mfl.gemm_chain_validate(batch, M, N1, N2, K, A, lda, sa, B, ldb, sb, W, ldw, sw,
                                   D, ldd, sd, d)


def test_chain_validation():
    assert _cv() == 0
    assert _cv(d=mfl.F32) == 0
    for K in (32, 64, 128, 256):
        assert _cv(K=K) == 0
    assert _cv(N1=0) == 0                          # D = 0
    assert _cv(batch=0, D=None) == 0
    assert _cv(sa=0, sb=0, sw=0) == 0              # shared operands
    assert _cv(M=-1) == mfl.ERR["NEGATIVE_DIM"]
    for K in (0, 16, 96, 512):
        assert _cv(K=K) == mfl.ERR["UNSUPPORTED"], K
    assert _cv(d=0) == mfl.ERR["UNSUPPORTED"]
    assert _cv(lda=100) == mfl.ERR["LEADING_DIM"]
    assert _cv(ldw=299) == mfl.ERR["LEADING_DIM"]
    assert _cv(ldd=127) == mfl.ERR["LEADING_DIM"]
    assert _cv(sb=-1) == mfl.ERR["LEADING_DIM"]
    assert _cv(sd=100 * 128 - 1) == mfl.ERR["ALIAS"]   # D batches overlap
    assert _cv(D=None) == mfl.ERR["NULL_POINTER"]
    assert _cv(W=None) == mfl.ERR["NULL_POINTER"]
    assert _cv(A=P + 1) == mfl.ERR["MISALIGNED"]
    assert _cv(D=P + 2, d=mfl.F32) == mfl.ERR["MISALIGNED"]
    for kw in (dict(M=1 << 40), dict(N2=1 << 31), dict(ldd=1 << 40), dict(batch=1 << 31),
               dict(batch=1 << 20, sa=1 << 30), dict(batch=2, sw=(1 << 62) + 1)):
        assert _cv(**kw) == mfl.ERR["TOO_LARGE"], kw


def _cplan(**kw):
    args = dict(batch=2, M=100, N1=256, N2=128, K=128, A=P, lda=128, sa=100 * 128, B=P, ldb=128,
                sb=256 * 128, W=P, ldw=256, sw=128 * 256, D=P, ldd=128, sd=100 * 128, d=mfl.F16)
    args.update(kw)
    a = args
    return mfl.gemm_chain_plan(a["batch"], a["M"], a["N1"], a["N2"], a["K"], a["A"], a["lda"],
                               a["sa"], a["B"], a["ldb"], a["sb"], a["W"], a["ldw"], a["sw"],
                               a["D"], a["ldd"], a["sd"], a["d"])[:2]


def test_chain_staging_rule():
    """Direct-to-LDS staging only for whole N1 chunks and 16-byte rows."""
    assert _cplan() == (0, "dma")
    assert _cplan(K=32) == (0, "dma")
    assert _cplan(sa=0, sb=0, sw=0) == (0, "dma")
    assert _cplan(N1=250, ldw=256) == (0, "regs")        # ragged last chunk
    assert _cplan(N1=96, ldw=96) == (0, "regs")          # chunks of 64 at K = 128
    assert _cplan(N1=96, ldw=96, K=256, lda=256, ldb=256) == (0, "dma")   # 32 at K = 256
    assert _cplan(ldw=260) == (0, "regs")                # W rows 8-byte aligned
    assert _cplan(ldb=136) == (0, "dma")
    assert _cplan(ldb=130) == (0, "regs")
    assert _cplan(B=P + 8) == (0, "regs")
    assert _cplan(W=P + 2) == (0, "regs")
    assert _cplan(sw=128 * 256 + 4) == (0, "regs")
    assert _cplan(sb=256 * 128 + 2) == (0, "regs")
    assert _cplan(A=P + 2, lda=130) == (0, "dma")        # A is read through registers
    assert _cplan(K=96)[0] == mfl.ERR["UNSUPPORTED"]


def test_chain_n2_tile_rule():
    """N2 tiles of 64 columns when N2 fits, else 128."""
    def tile(N2):
        return mfl.gemm_chain_plan(1, 100, 256, N2, 128, P, 128, 0, P, 128, 0, P, 256, 0,
                                   P, max(N2, 1), 0, mfl.F16)[2]
    assert [tile(n) for n in (1, 63, 64, 65, 128, 129, 1000)] == [64, 64, 64, 128, 128, 128, 128]


def test_microbenchmark_arguments():
    """The rate kernels refuse bad sizes, depths and NULL pointers before any
    launch."""
    assert mfl.lib.mfl_bench_dma_rate(256, 10, 256, 5, P, P, P, None) == -4      # depth
    assert mfl.lib.mfl_bench_dma_rate(100, 10, 256, 12, P, P, P, None) == -4     # threads
    assert mfl.lib.mfl_bench_dma_rate(256, 10, 256, 12, 0, P, P, None) == -4     # buf
    assert mfl.lib.mfl_bench_lds_read(256, 10, 256, 3, P, P, None) == -4         # depth
    assert mfl.lib.mfl_bench_lds_read(256, 0, 256, 8, P, P, None) == -4          # iters

def test_chain_phase_probe_arguments():
    """The timed instance exists only for K = 128, fp16 D, direct-to-LDS
    staging and 128-column N2 tiles; anything else, or no stamp buffer, is
    refused before a launch."""
    def probe(stamps=P, **kw):
        a = dict(batch=2, M=100, N1=256, N2=128, K=128, A=P, lda=128, sa=100 * 128, B=P,
                 ldb=128, sb=256 * 128, W=P, ldw=256, sw=128 * 256, D=P, ldd=128, sd=100 * 128,
                 d=mfl.F16)
        a.update(kw)
        return mfl.probe_chain_phases_raw(*a.values(), stamps, 0)
    assert probe(stamps=0) == mfl.ERR["NULL_POINTER"]
    assert probe(K=64, lda=64, ldb=64) == mfl.ERR["UNSUPPORTED"]
    assert probe(d=mfl.F32) == mfl.ERR["UNSUPPORTED"]
    assert probe(N1=250) == mfl.ERR["UNSUPPORTED"]                 # register staging
    assert probe(N2=64, ldd=64, sd=100 * 64, sw=64 * 256) == mfl.ERR["UNSUPPORTED"]
    assert probe(M=-1) == mfl.ERR["NEGATIVE_DIM"]
    assert mfl.CHAIN_STAMP_SHAPE == (8, 8, 4 * 64 + 4)

def test_chain_perm_is_derived_from_the_atoms():
    """The map behind the kernel's B row order: position p = 16 kc + 8 h + v
    of the second product's K is accumulator row 8 (2 kc + v / 4) + 4 h +
    v % 4 of the first (closed form from the 32x32x16 maps of the oracle); the
    kernel puts N1 row pi^-1(r) of a chunk in LDS row r, so P arrives in
    natural N1 order."""
    from oracle import layout as OL
    op = "f32_32x32x16_f16"
    pi = {}
    for lane in range(64):
        row, k0 = OL.mfma_ab_coord(op, lane, 0)
        for kc in range(2):
            for v in range(8):
                m_c, n_c = OL.mfma_c_coord(op, lane, 8 * kc + v)
                # transposed first product: accumulator row = n1, column = m
                assert n_c == row
                pi.setdefault(16 * kc + k0 + v, set()).add(m_c)
    assert all(len(s) == 1 for s in pi.values()) and len(pi) == 32
    got = [next(iter(pi[p])) for p in range(32)]
    assert got == [8 * (2 * (p // 16) + (p % 8) // 4) + 4 * ((p % 16) // 8) + p % 4
                   for p in range(32)]
    assert sorted(got) == list(range(32))
    assert mfl.chain_k_perm().tolist() == got          # the kernel's compile-time map

"""Shared helpers for the GPU tests: guarded device buffers, one GEMM call
through the C ABI, and the oracle comparison."""
import sys

import numpy as np
import torch

import mma_fragment_layouts_tn_amd as mfl
import workloads as W
from oracle import compare
from oracle import gemm as G

GUARD = 64
CANARY16 = int(np.array([0x7E5A], np.uint16).view(np.int16)[0])        # an fp16 NaN
CANARY32 = int(np.array([0x7FC0DEAD], np.uint32).view(np.int32)[0])    # an fp32 NaN


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


class Guarded:
    """Device copy of a host buffer followed by GUARD canary elements."""

    def __init__(self, host: np.ndarray, dev="cuda"):
        flat = np.ascontiguousarray(host).reshape(-1)
        self.n = flat.size
        if flat.dtype.itemsize == 2:
            bits = flat.view(np.int16)
            t = torch.full((self.n + GUARD,), CANARY16, dtype=torch.int16)
        else:
            bits = flat.view(np.int32)
            t = torch.full((self.n + GUARD,), CANARY32, dtype=torch.int32)
        t[: self.n] = torch.from_numpy(bits.copy())
        self.host_bits = t.clone()
        self.t = t.to(dev)

    @property
    def ptr(self):
        return self.t.data_ptr()

    def guard_intact(self):
        return torch.equal(self.t[self.n:].cpu(), self.host_bits[self.n:])

    def unchanged(self):
        return torch.equal(self.t.cpu(), self.host_bits)


def out_buffer(M, ldd, d, dev="cuda"):
    n = M * ldd
    if d == "f16":
        t = torch.full((n + GUARD,), CANARY16, dtype=torch.int16, device=dev)
    else:
        t = torch.full((n + GUARD,), CANARY32, dtype=torch.int32, device=dev)
    return t


# configurations that offer only some fetch paths (the 16x16x32 ones, and
# the four-wave 256x256 one without M-contiguous A straight to LDS with B
# through registers)
PARTIAL_FETCH_ALGOS = {"lds256w4_16", "lds256_16", "lds128_16", "splitk_16", "lds256w4"}


def refused(w: W.Workload, algo: str) -> bool:
    """True when `algo` does not offer the fetch path this case needs (it is
    one of PARTIAL_FETCH_ALGOS and the C ABI answers MFL_E_ALGO_CASE); any
    other refusal fails the calling test."""
    ckind = {None: mfl.NONE, "f16": mfl.F16, "f32": mfl.F32}[w.c]
    dkind = {"f16": mfl.F16, "f32": mfl.F32}[w.d]
    a_order = mfl.A_KMAJOR if w.a_order == "k" else mfl.A_MMAJOR
    dt = mfl.dtypes(ckind, dkind, a_order, mfl.algo_code(algo))
    # distinct 256-byte aligned stand-in addresses, aligned as torch's device buffers
    PA, PB, PC, PD = (k << 20 for k in (1, 2, 3, 4))
    rc = mfl.validate(w.M, w.N, w.K, PA, w.lda_, PB, w.ldb_, None if w.c is None else PC,
                      w.ldc_ if w.c is not None else 0, PD, w.ldd_, dt)[0]
    if rc == -6 and algo.split("+")[0] in PARTIAL_FETCH_ALGOS:
        say(f"[gpu] {w.name} {algo}: fetch path not offered by this configuration")
        return True
    assert rc == 0, (w.name, algo, rc, mfl.strerror(rc))
    return False


def run_gemm(w: W.Workload, x: W.Inputs, algo: str, in_place: bool = False,
             poisoned: bool = False):
    """Upload, call gemm_tn through the C ABI (with `poisoned`, its
    LDS-poisoned test instances), download.  Returns (D as float64 (M,N)
    array, checks dict)."""
    say(f"[gpu] {w.name} algo={algo} M={w.M} N={w.N} K={w.K} a={w.a_order} "
        f"c={w.c} d={w.d} int={x.integer}")
    A = Guarded(x.A)
    B = Guarded(x.B)
    C = Guarded(x.C) if x.C is not None else None
    ldd = w.ldd_
    if in_place:
        assert C is not None and w.c == w.d and w.ldc_ == ldd
        Dt = C.t
    else:
        Dt = out_buffer(w.M, ldd, w.d)
    ckind = {None: mfl.NONE, "f16": mfl.F16, "f32": mfl.F32}[w.c]
    dkind = {"f16": mfl.F16, "f32": mfl.F32}[w.d]
    a_order = mfl.A_KMAJOR if w.a_order == "k" else mfl.A_MMAJOR
    dt = mfl.dtypes(ckind, dkind, a_order, mfl.algo_code(algo))
    stream = torch.cuda.current_stream().cuda_stream
    entry = mfl.gemm_tn_poisoned_raw if poisoned else mfl.gemm_tn_raw
    rc = entry(w.M, w.N, w.K, A.ptr, w.lda_, B.ptr, w.ldb_,
                         None if C is None else C.ptr, w.ldc_ if C is not None else 0,
                         Dt.data_ptr(), ldd, dt, stream)
    assert rc == 0, (rc, mfl.strerror(rc))
    torch.cuda.synchronize()
    raw = Dt.cpu().numpy()
    n = w.M * ldd
    if w.d == "f16":
        D = raw[:n].view(np.float16).reshape(w.M, ldd)[:, : w.N].astype(np.float64)
        guard_ok = (raw[n:] == np.int16(CANARY16)).all()
        pad_ok = (raw[:n].reshape(w.M, ldd)[:, w.N:] == np.int16(CANARY16)).all()
    else:
        D = raw[:n].view(np.float32).reshape(w.M, ldd)[:, : w.N].astype(np.float64)
        guard_ok = (raw[n:] == np.int32(CANARY32)).all()
        pad_ok = (raw[:n].reshape(w.M, ldd)[:, w.N:] == np.int32(CANARY32)).all()
    checks = {"A_unchanged": A.unchanged(), "B_unchanged": B.unchanged(),
              "C_unchanged": (C is None or in_place or C.unchanged()),
              "D_guard": bool(guard_ok), "D_padding": bool(pad_ok)}
    if in_place:
        checks["C_guard"] = C.guard_intact()
        checks["D_guard"] = checks["C_guard"]
    return D, checks


def oracle_full(w: W.Workload, x: W.Inputs):
    return G.gemm_f64(w.M, w.N, w.K, x.A, w.lda_, w.a_order == "m", x.B, w.ldb_, x.C)


_FULL_CACHE = {}


def oracle_full_cached(w: W.Workload, x: W.Inputs):
    """oracle_full, kept for the two most recent workloads (the named
    workloads' cases run one workload's algorithms and its integer twin in a
    row, so each full reference is computed once)."""
    key = w
    if key not in _FULL_CACHE:
        while len(_FULL_CACHE) >= 2:
            _FULL_CACHE.pop(next(iter(_FULL_CACHE)))
        _FULL_CACHE[key] = oracle_full(w, x)
    return _FULL_CACHE[key]


def oracle_sampled(w: W.Workload, x: W.Inputs, ms, ns):
    return G.gemm_f64_sampled(w.M, w.N, w.K, x.A, w.lda_, w.a_order == "m", x.B, w.ldb_,
                              x.C, ms, ns)


def verdict(D, ref, w: W.Workload, integer: bool):
    return compare.check(D, ref, w.d, w.K, integer)


def freivalds_exact(D, w: W.Workload, x: W.Inputs, trials=2, seed=0):
    """Full-matrix check for integer-valued inputs with exact fp32 output:
    D x == C x + A (B^T x) in int64 for random x (any wrong element of D
    changes D x)."""
    rng = np.random.default_rng(seed)
    M, N, K = w.M, w.N, w.K
    Di = D.astype(np.int64)
    if not np.array_equal(Di.astype(np.float64), D):
        return False
    if w.a_order == "k":
        Ai = x.A[:, :K].astype(np.int64)
    else:
        Ai = x.A[:, :M].astype(np.int64).T
    Bi = x.B[:, :K].astype(np.int64)
    Ci = x.C[:, :N].astype(np.int64) if x.C is not None else None
    for _ in range(trials):
        v = rng.integers(1, 1 << 20, size=N, dtype=np.int64)
        lhs = Di @ v
        rhs = Ai @ (Bi.T @ v)
        if Ci is not None:
            rhs = rhs + Ci @ v
        if not np.array_equal(lhs, rhs):
            return False
    return True

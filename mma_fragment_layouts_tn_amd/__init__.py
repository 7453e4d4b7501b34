"""Python binding of the MI355X fp16 TN GEMM library (libmfl_gemm.so).

Argument marshalling only: every step of the GEMM runs in the HIP kernels
behind the C ABI declared in include/mfl_gemm.h, include/mfl_layout.h and
include/mfl_probe.h.  PyTorch provides device memory and the current stream.
There is no fallback: if the library is missing, importing this package
raises.

D(m,n) = C(m,n) + sum_k A(m,k) * B(n,k); A (M,K), B (N,K) fp16, both
K-contiguous (or A M-contiguous), C absent/fp16/fp32, D fp16/fp32.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

# torch first: its HIP runtime (soname libamdhip64.so.7) must be the one the
# library binds to, so device pointers and streams are shared.
import torch  # noqa: E402
import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmfl_gemm.so")

NONE, F16, F32 = 0, 1, 2
A_KMAJOR, A_MMAJOR = 0, 1
ALGOS = {"auto": 0, "direct": 1, "lds128": 2, "lds256": 3, "lds256w4": 4, "lds128w1": 5,
         "splitk": 6, "lds256w4_16": 7, "lds256_16": 8, "lds128_16": 9, "splitk_16": 10}
REG_FETCH = 0x100          # or-ed into the algo: fetch through registers
FETCH_NAMES = {0: "dma", 1: "reg", 2: "regT", 3: "dmaT"}
ALGO_NAMES = {v: k for k, v in ALGOS.items()}


def algo_code(name: str) -> int:
    """'lds256' -> 3; 'lds256+reg' -> 3 | REG_FETCH."""
    base, _, flag = name.partition("+")
    code = ALGOS[base]
    if flag == "reg":
        code |= REG_FETCH
    elif flag:
        raise ValueError(name)
    return code
MFMA_OPS = {"f32_32x32x16_f16": 0, "f32_16x16x32_f16": 1, "f32_32x32x8_f16": 2,
            "f32_16x16x16_f16": 3}

ERRORS = {
    0: "MFL_OK", -1: "MFL_E_NEGATIVE_DIM", -2: "MFL_E_LEADING_DIM", -3: "MFL_E_NULL_POINTER",
    -4: "MFL_E_UNSUPPORTED", -5: "MFL_E_LAUNCH", -6: "MFL_E_ALGO_CASE",
    -7: "MFL_E_MISALIGNED", -8: "MFL_E_ALIAS", -9: "MFL_E_TOO_LARGE",
}
ERR = {v.replace("MFL_E_", "").replace("MFL_", ""): k for k, v in ERRORS.items()}


class GemmDtypes(ctypes.Structure):
    _fields_ = [("a", ctypes.c_int32), ("b", ctypes.c_int32), ("c", ctypes.c_int32),
                ("d", ctypes.c_int32), ("a_order", ctypes.c_int32), ("algo", ctypes.c_int32)]


class MflError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{ERRORS.get(code, code)}: {msg}")
        self.code = code


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python mma_fragment_layouts_tn_amd/_build.py` "
            "(hipcc, gfx950).  There is no CPU fallback.")
    lib = ctypes.CDLL(LIB_PATH)
    i64, i32, vp, cp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_char_p
    P = ctypes.POINTER
    lib.gemm_tn.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, vp, i64, GemmDtypes, vp]
    lib.gemm_tn.restype = ctypes.c_int
    lib.gemm_tn_validate.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, vp, i64,
                                     GemmDtypes, P(i32)]
    lib.gemm_tn_validate.restype = ctypes.c_int
    lib.gemm_tn_plan.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, vp, i64,
                                 GemmDtypes, P(i32), P(i32), P(i32)]
    lib.gemm_tn_plan.restype = ctypes.c_int
    lib.gemm_strerror.argtypes = [ctypes.c_int]
    lib.gemm_strerror.restype = cp
    lib.gemm_tn_chain.argtypes = [i64] * 5 + [vp, i64, i64] * 4 + [i32, vp]
    lib.gemm_tn_chain.restype = ctypes.c_int
    lib.gemm_tn_chain_validate.argtypes = [i64] * 5 + [vp, i64, i64] * 4 + [i32]
    lib.gemm_tn_chain_validate.restype = ctypes.c_int
    lib.gemm_tn_chain_plan.argtypes = [i64] * 5 + [vp, i64, i64] * 4 + [i32, vp, vp]
    lib.gemm_tn_chain_plan.restype = ctypes.c_int
    lib.mfl_kernel_info.argtypes = [i32, GemmDtypes] + [P(i32)] * 6
    lib.mfl_kernel_info.restype = ctypes.c_int
    for name in ("mfl_layout_size", "mfl_layout_cosize"):
        getattr(lib, name).argtypes = [cp, P(i64)]
        getattr(lib, name).restype = ctypes.c_int
    lib.mfl_layout_eval.argtypes = [cp, i64, P(i64)]
    lib.mfl_layout_eval.restype = ctypes.c_int
    lib.mfl_layout_table.argtypes = [cp, vp, i64]
    lib.mfl_layout_table.restype = ctypes.c_int
    for name in ("mfl_layout_coalesce", "mfl_layout_right_inverse"):
        getattr(lib, name).argtypes = [cp, ctypes.c_char_p, i64]
        getattr(lib, name).restype = ctypes.c_int
    lib.mfl_layout_compose.argtypes = [cp, cp, ctypes.c_char_p, i64]
    lib.mfl_layout_complement.argtypes = [cp, i64, ctypes.c_char_p, i64]
    lib.mfl_layout_logical_divide.argtypes = [cp, cp, ctypes.c_char_p, i64]
    lib.mfl_layout_zipped_divide.argtypes = [cp, cp, ctypes.c_char_p, i64]
    lib.mfl_layout_logical_product.argtypes = [cp, cp, ctypes.c_char_p, i64]
    lib.mfl_layout_upcast.argtypes = [cp, i64, ctypes.c_char_p, i64]
    lib.mfl_layout_with_shape.argtypes = [cp, cp, ctypes.c_char_p, i64]
    lib.mfl_layout_tiled_product.argtypes = [cp, cp, ctypes.c_char_p, i64]
    lib.mfl_layout_partition_c.argtypes = [cp, cp, cp, i64, i64, i64, i64, ctypes.c_char_p,
                                           ctypes.c_char_p, i64]
    lib.mfl_layout_retile.argtypes = [cp, cp, cp, i64, i64, ctypes.c_char_p, i64]
    lib.mfl_layout_compose.restype = ctypes.c_int
    lib.mfl_layout_mfma_tv.argtypes = [i32, i32, ctypes.c_char_p, i64]
    lib.mfl_layout_mfma_tv.restype = ctypes.c_int
    lib.mfl_fragment_coords.argtypes = [i32, i32, vp, i64, P(i32), P(i32)]
    lib.mfl_fragment_coords.restype = ctypes.c_int
    lib.mfl_lds_tile_offsets.argtypes = [i32, i32, vp, i64, P(i32), P(i32)]
    lib.mfl_lds_tile_offsets.restype = ctypes.c_int
    lib.mfl_chain_k_perm.argtypes = [vp]
    lib.mfl_chain_k_perm.restype = ctypes.c_int
    lib.mfl_tile_order.argtypes = [i32, i32, i32, vp, vp]
    lib.mfl_tile_order.restype = ctypes.c_int
    lib.mfl_probe_mfma.argtypes = [i32, vp, vp, vp, vp, vp]
    lib.mfl_probe_mfma.restype = ctypes.c_int
    lib.mfl_probe_lds_tr16.argtypes = [vp, vp, vp, vp]
    lib.mfl_probe_lds_tr16.restype = ctypes.c_int
    lib.mfl_probe_xcc.argtypes = [i32, vp, vp]
    lib.mfl_probe_xcc.restype = ctypes.c_int
    lib.mfl_probe_gemm_poisoned.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, vp, i64,
                                            GemmDtypes, vp]
    lib.mfl_probe_gemm_poisoned.restype = ctypes.c_int
    lib.mfl_probe_fragments.argtypes = [i32, i32, i32, i32, i32, i32, vp, i32, vp, i32, vp, i64,
                                        P(i32), P(i32), vp]
    lib.mfl_probe_fragments.restype = ctypes.c_int
    lib.mfl_probe_chain_phases.argtypes = [i64] * 5 + [vp, i64, i64] * 4 + [i32, vp, vp]
    lib.mfl_probe_chain_phases.restype = ctypes.c_int
    lib.mfl_bench_mfma.argtypes = [i32, vp, i32, i32, i32, vp, vp, vp]
    lib.mfl_bench_mfma.restype = ctypes.c_int
    lib.mfl_bench_lds_read.argtypes = [i32, i32, i32, i32, vp, vp, vp]
    lib.mfl_bench_dma_rate.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp]
    lib.mfl_bench_dma_rate.restype = ctypes.c_int
    lib.mfl_bench_lds_read.restype = ctypes.c_int
    lib.mfl_wall_clock_khz.argtypes = [P(i32)]
    lib.mfl_wall_clock_khz.restype = ctypes.c_int
    return lib


_lib = _load()
lib = _lib


def strerror(code: int) -> str:
    return _lib.gemm_strerror(code).decode()


def _check(code: int):
    if code != 0:
        raise MflError(code, strerror(code))


def dtypes(c: int = NONE, d: int = F32, a_order: int = A_KMAJOR, algo: int = 0) -> GemmDtypes:
    return GemmDtypes(F16, F16, c, d, a_order, algo)


# ----------------------------------------------------------------- GEMM
def gemm_tn_raw(M: int, N: int, K: int, A: int, lda: int, B: int, ldb: int, C: Optional[int],
                ldc: int, D: int, ldd: int, dt: GemmDtypes, stream: int) -> int:
    """Direct call of the C ABI with integer pointers; returns the code."""
    return _lib.gemm_tn(M, N, K, A, lda, B, ldb, C, ldc, D, ldd, dt, stream)


def gemm_tn_poisoned_raw(M: int, N: int, K: int, A: int, lda: int, B: int, ldb: int,
                         C: Optional[int], ldc: int, D: int, ldd: int, dt: GemmDtypes,
                         stream: int) -> int:
    """gemm_tn on the LDS-poisoned test instances (mfl_probe_gemm_poisoned)."""
    return _lib.mfl_probe_gemm_poisoned(M, N, K, A, lda, B, ldb, C, ldc, D, ldd, dt, stream)


def validate(M, N, K, A, lda, B, ldb, C, ldc, D, ldd, dt: GemmDtypes) -> Tuple[int, int]:
    """(code, algo AUTO would pick) without touching the GPU."""
    algo = ctypes.c_int32(-1)
    rc = _lib.gemm_tn_validate(M, N, K, A, lda, B, ldb, C, ldc, D, ldd, dt, ctypes.byref(algo))
    return rc, algo.value


def plan(M, N, K, A, lda, B, ldb, C, ldc, D, ldd, dt: GemmDtypes):
    """(code, algo, fetch_a, fetch_b) the call would use, without the GPU."""
    a, fa, fb = ctypes.c_int32(-1), ctypes.c_int32(-1), ctypes.c_int32(-1)
    rc = _lib.gemm_tn_plan(M, N, K, A, lda, B, ldb, C, ldc, D, ldd, dt, ctypes.byref(a),
                           ctypes.byref(fa), ctypes.byref(fb))
    return rc, a.value, fa.value, fb.value


def _kind(t: Optional[torch.Tensor]) -> int:
    if t is None:
        return NONE
    if t.dtype == torch.float16:
        return F16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def a_view_args(A: torch.Tensor):
    """(a_order, lda) of a 2-D (M,K) fp16 tensor view."""
    if A.dim() != 2:
        raise ValueError("A must be 2-D (M,K)")
    M, K = A.shape
    if A.stride(1) == 1 and (M <= 1 or A.stride(0) >= max(K, 1)):
        return A_KMAJOR, max(A.stride(0), max(K, 1))
    if A.stride(0) == 1 and (K <= 1 or A.stride(1) >= max(M, 1)):
        return A_MMAJOR, max(A.stride(1), max(M, 1))
    raise ValueError("A must be K-contiguous or M-contiguous")


def gemm_tn(A: torch.Tensor, B: torch.Tensor, C: Optional[torch.Tensor] = None,
            out_dtype: torch.dtype = torch.float32, algo: str = "auto",
            D: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """D = C + A @ B.T on the GPU.  A (M,K) fp16 K- or M-contiguous view,
    B (N,K) fp16 K-contiguous, C (M,N) fp16/fp32 row-contiguous or None.
    D is allocated (M,N) when not given."""
    if A.dtype != torch.float16 or B.dtype != torch.float16:
        raise TypeError("A and B must be float16")
    if not (A.is_cuda and B.is_cuda):
        raise ValueError("A and B must be device tensors (no CPU path)")
    M, K = A.shape
    N, K2 = B.shape
    if K2 != K:
        raise ValueError("A and B disagree on K")
    a_order, lda = a_view_args(A)
    if B.stride(1) != 1 and K > 1:
        raise ValueError("B must be K-contiguous")
    ldb = max(B.stride(0), max(K, 1)) if N > 1 else max(K, 1)
    if C is not None:
        if tuple(C.shape) != (M, N) or (C.stride(1) != 1 and N > 1):
            raise ValueError("C must be (M,N) with contiguous rows")
        ldc = max(C.stride(0), max(N, 1)) if M > 1 else max(N, 1)
    else:
        ldc = 0
    if D is None:
        D = torch.empty((M, N), dtype=out_dtype, device=A.device)
    if tuple(D.shape) != (M, N) or (D.stride(1) != 1 and N > 1):
        raise ValueError("D must be (M,N) with contiguous rows")
    ldd = max(D.stride(0), max(N, 1)) if M > 1 else max(N, 1)
    dt = dtypes(_kind(C), _kind(D), a_order, algo_code(algo))
    if stream is None:
        stream = torch.cuda.current_stream(A.device).cuda_stream
    rc = gemm_tn_raw(M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb,
                     None if C is None else C.data_ptr(), ldc, D.data_ptr(), ldd, dt, stream)
    _check(rc)
    return D


# ------------------------------------------------------- back-to-back GEMM
def gemm_chain_raw(batch, M, N1, N2, K, A, lda, sa, B, ldb, sb, W, ldw, sw, D, ldd, sd,
                   d_dtype: int, stream: int) -> int:
    """Direct call of gemm_tn_chain with integer pointers; returns the code."""
    return _lib.gemm_tn_chain(batch, M, N1, N2, K, A, lda, sa, B, ldb, sb, W, ldw, sw, D, ldd,
                              sd, d_dtype, stream)


# phase stamps of the timed chain instance: workgroups x waves x slots
CHAIN_STAMP_SHAPE = (8, 8, 260)


def probe_chain_phases_raw(batch, M, N1, N2, K, A, lda, sa, B, ldb, sb, W, ldw, sw, D, ldd, sd,
                           d_dtype: int, stamps: int, stream: int) -> int:
    """mfl_probe_chain_phases with integer pointers; `stamps` points to
    8 * 8 * 260 uint32 of device memory (CHAIN_STAMP_SHAPE)."""
    return _lib.mfl_probe_chain_phases(batch, M, N1, N2, K, A, lda, sa, B, ldb, sb, W, ldw, sw,
                                       D, ldd, sd, d_dtype, stamps, stream)


def gemm_chain_validate(batch, M, N1, N2, K, A, lda, sa, B, ldb, sb, W, ldw, sw, D, ldd, sd,
                        d_dtype: int) -> int:
    return _lib.gemm_tn_chain_validate(batch, M, N1, N2, K, A, lda, sa, B, ldb, sb, W, ldw, sw,
                                       D, ldd, sd, d_dtype)


CHAIN_STAGING = {0: "regs", 1: "dma"}


def gemm_chain_plan(batch, M, N1, N2, K, A, lda, sa, B, ldb, sb, W, ldw, sw, D, ldd, sd,
                    d_dtype: int):
    """(code, staging name, N2 tile width) gemm_tn_chain would take for these
    arguments."""
    st, tn = ctypes.c_int32(-1), ctypes.c_int32(-1)
    rc = _lib.gemm_tn_chain_plan(batch, M, N1, N2, K, A, lda, sa, B, ldb, sb, W, ldw, sw,
                                 D, ldd, sd, d_dtype, ctypes.byref(st), ctypes.byref(tn))
    return rc, CHAIN_STAGING.get(st.value), (tn.value if rc == 0 else None)


def _rows_view(X: torch.Tensor, name: str):
    """(batch, rows, cols, ld, batch stride) of a 2-D or 3-D view whose rows
    are contiguous."""
    if X.dim() == 2:
        X = X.unsqueeze(0)
    if X.dim() != 3:
        raise ValueError(f"{name} must be 2-D or 3-D")
    bt, r, c = X.shape
    if c > 1 and X.stride(2) != 1:
        raise ValueError(f"{name} rows must be contiguous")
    ld = max(X.stride(1), max(c, 1)) if r > 1 else max(c, 1)
    sb = X.stride(0) if bt > 1 else 0
    return bt, r, c, ld, sb


def gemm_chain(A: torch.Tensor, B: torch.Tensor, W: torch.Tensor,
               out_dtype: torch.dtype = torch.float16, stream=None) -> torch.Tensor:
    """D = rne16(A @ B.T) @ W.T per batch on the GPU.  A (batch,M,K),
    B (batch,N1,K), W (batch,N2,N1), fp16 with contiguous rows (2-D views are
    one batch; a batch of 1 broadcasts).  Returns D (batch,M,N2)."""
    for X in (A, B, W):
        if X.dtype != torch.float16:
            raise TypeError("A, B and W must be float16")
        if not X.is_cuda:
            raise ValueError("A, B and W must be device tensors (no CPU path)")
    ba, M, K, lda, sa = _rows_view(A, "A")
    bb, N1, K2, ldb, sb = _rows_view(B, "B")
    bw, N2, N1w, ldw, sw = _rows_view(W, "W")
    if K2 != K or N1w != N1:
        raise ValueError("A, B and W disagree on K or N1")
    batch = max(ba, bb, bw)
    if any(x not in (1, batch) for x in (ba, bb, bw)):
        raise ValueError("batch sizes disagree")
    D = torch.empty((batch, M, N2), dtype=out_dtype, device=A.device)
    dk = _kind(D)
    if stream is None:
        stream = torch.cuda.current_stream(A.device).cuda_stream
    rc = gemm_chain_raw(batch, M, N1, N2, K, A.data_ptr(), lda, sa, B.data_ptr(), ldb, sb,
                        W.data_ptr(), ldw, sw, D.data_ptr(), max(N2, 1), M * max(N2, 1), dk,
                        stream)
    _check(rc)
    return D


def kernel_info(algo: str, c: int = NONE, d: int = F32, a_order: int = A_KMAJOR) -> dict:
    vals = [ctypes.c_int32(-1) for _ in range(6)]
    rc = _lib.mfl_kernel_info(algo_code(algo), dtypes(c, d, a_order, algo_code(algo)),
                              *[ctypes.byref(v) for v in vals])
    _check(rc)
    keys = ("bm", "bn", "bk", "threads", "lds_bytes", "scratch_bytes")
    return dict(zip(keys, (v.value for v in vals)))


# --------------------------------------------------------------- layouts
class LayoutError(ValueError):
    pass


def _lay_check(rc: int, what: str):
    if rc != 0:
        raise LayoutError(f"{what}: code {rc}")


def layout_size(text: str) -> int:
    out = ctypes.c_int64()
    _lay_check(_lib.mfl_layout_size(text.encode(), ctypes.byref(out)), text)
    return out.value


def layout_cosize(text: str) -> int:
    out = ctypes.c_int64()
    _lay_check(_lib.mfl_layout_cosize(text.encode(), ctypes.byref(out)), text)
    return out.value


def layout_eval(text: str, idx: int) -> int:
    out = ctypes.c_int64()
    _lay_check(_lib.mfl_layout_eval(text.encode(), idx, ctypes.byref(out)), text)
    return out.value


def layout_table(text: str) -> np.ndarray:
    n = layout_size(text)
    out = np.empty(n, dtype=np.int64)
    _lay_check(_lib.mfl_layout_table(text.encode(), out.ctypes.data, n), text)
    return out


def _text_op(fn, *args) -> str:
    buf = ctypes.create_string_buffer(1024)
    _lay_check(fn(*[a.encode() if isinstance(a, str) else a for a in args], buf, 1024),
               str(args))
    return buf.value.decode()


def layout_coalesce(text: str) -> str:
    return _text_op(_lib.mfl_layout_coalesce, text)


def layout_compose(a: str, b: str) -> str:
    return _text_op(_lib.mfl_layout_compose, a, b)


def layout_right_inverse(text: str) -> str:
    return _text_op(_lib.mfl_layout_right_inverse, text)


def _tiler_text(tiler) -> str:
    """One layout text, or a sequence with one entry per mode (None = keep)."""
    if isinstance(tiler, str):
        return tiler
    text = ";".join("_" if t is None else t for t in tiler)
    return text + ";" if len(tiler) == 1 else text     # one entry: still per mode


def layout_complement(text: str, cotarget: int) -> str:
    return _text_op(_lib.mfl_layout_complement, text, cotarget)


def layout_logical_divide(a: str, tiler) -> str:
    return _text_op(_lib.mfl_layout_logical_divide, a, _tiler_text(tiler))


def layout_zipped_divide(a: str, tiler) -> str:
    return _text_op(_lib.mfl_layout_zipped_divide, a, _tiler_text(tiler))


def layout_logical_product(a: str, b: str) -> str:
    return _text_op(_lib.mfl_layout_logical_product, a, b)


def layout_upcast(text: str, n: int) -> str:
    return _text_op(_lib.mfl_layout_upcast, text, n)


def layout_with_shape(text: str, shape: str) -> str:
    return _text_op(_lib.mfl_layout_with_shape, text, shape)


def layout_tiled_product(a: str, b: str) -> str:
    return _text_op(_lib.mfl_layout_tiled_product, a, b)


def layout_partition_c(c: str, atom_tv: str, atom_mn, warps_mn, tile=None) -> Tuple[str, str]:
    """(thread layout, value layout) of partition_C; ``tile`` = None or the
    (M, N) permutation layouts (None entries unpermuted)."""
    thr, val = ctypes.create_string_buffer(1024), ctypes.create_string_buffer(1024)
    tile_txt = "" if tile is None else ";".join("_" if t is None else t for t in tile)
    _lay_check(_lib.mfl_layout_partition_c(c.encode(), tile_txt.encode(), atom_tv.encode(),
                                           atom_mn[0], atom_mn[1], warps_mn[0], warps_mn[1],
                                           thr, val, 1024), c)
    return thr.value.decode(), val.value.decode()


def layout_retile(frag: str, tv: str, tile_shape: str, nthr: int, atom_nval: int) -> str:
    return _text_op(_lib.mfl_layout_retile, frag, tv, tile_shape, nthr, atom_nval)


def mfma_tv(op: str, operand: str) -> str:
    return _text_op(_lib.mfl_layout_mfma_tv, MFMA_OPS[op], {"A": 0, "B": 1, "C": 2}[operand])


def fragment_coords(algo: str, operand: str) -> np.ndarray:
    """(threads, slots, 2) int32 array of the kernel's per-lane coordinates."""
    opnd = {"A": 0, "B": 1, "C": 2, "A_tr": 3}[operand]
    t, s = ctypes.c_int32(), ctypes.c_int32()
    _lay_check(_lib.mfl_fragment_coords(algo_code(algo), opnd, None, 0, ctypes.byref(t),
                                        ctypes.byref(s)), algo)
    out = np.empty((t.value, s.value, 2), dtype=np.int32)
    _lay_check(_lib.mfl_fragment_coords(algo_code(algo), opnd, out.ctypes.data, out.size,
                                        ctypes.byref(t), ctypes.byref(s)), algo)
    return out


def lds_tile_offsets(algo: str, operand: str) -> np.ndarray:
    """LDS element offsets of one operand stage: "A"/"B" (rows, BK) indexed
    [row, k]; "A_mmajor" (BK, BM) indexed [k, m]."""
    opnd = {"A": 0, "B": 1, "A_mmajor": 2}[operand]
    r, k = ctypes.c_int32(), ctypes.c_int32()
    _lay_check(_lib.mfl_lds_tile_offsets(algo_code(algo), opnd, None, 0, ctypes.byref(r),
                                         ctypes.byref(k)), algo)
    out = np.empty((r.value, k.value), dtype=np.int32)
    _lay_check(_lib.mfl_lds_tile_offsets(algo_code(algo), opnd, out.ctypes.data, out.size,
                                         ctypes.byref(r), ctypes.byref(k)), algo)
    return out


def chain_k_perm() -> np.ndarray:
    """pi of the back-to-back GEMM: K position p of the second product's
    operand over a 32-row block -> row of the first (transposed) accumulator."""
    out = np.empty(32, dtype=np.int32)
    _lay_check(_lib.mfl_chain_k_perm(out.ctypes.data), "chain_k_perm")
    return out


def tile_order(tiles_m: int, tiles_n: int, group_m: int):
    """(tm, tn) int32 arrays indexed by workgroup id."""
    tm = np.empty(tiles_m * tiles_n, dtype=np.int32)
    tn = np.empty_like(tm)
    _lay_check(_lib.mfl_tile_order(tiles_m, tiles_n, group_m, tm.ctypes.data, tn.ctypes.data),
               "tile_order")
    return tm, tn


# ----------------------------------------------------------------- probes
def probe_mfma(op: str, a_slots: torch.Tensor, b_slots: torch.Tensor,
               c_slots: torch.Tensor) -> torch.Tensor:
    """Run one matrix instruction; slot tensors are device tensors (64, VA)
    fp16 / (64, VC) fp32.  Returns the (64, VC) fp32 outputs."""
    d = torch.empty_like(c_slots)
    stream = torch.cuda.current_stream(c_slots.device).cuda_stream
    rc = _lib.mfl_probe_mfma(MFMA_OPS[op], a_slots.data_ptr(), b_slots.data_ptr(),
                             c_slots.data_ptr(), d.data_ptr(), stream)
    _check(rc)
    return d


def probe_lds_tr16(lane_offsets, lds_in: torch.Tensor) -> torch.Tensor:
    """One transposing LDS read: lds_in is a device int16 tensor of 4096
    values, lane_offsets 64 ints (multiples of 4 in [0, 4092]).  Returns the
    (64, 4) int16 values each lane receives."""
    offs = (ctypes.c_int32 * 64)(*[int(v) for v in lane_offsets])
    out = torch.empty((64, 4), dtype=torch.int16, device=lds_in.device)
    stream = torch.cuda.current_stream(lds_in.device).cuda_stream
    rc = _lib.mfl_probe_lds_tr16(offs, lds_in.data_ptr(), out.data_ptr(), stream)
    _check(rc)
    return out


def probe_xcc(nblocks: int) -> torch.Tensor:
    """XCD index (0..7) of each of nblocks workgroups (int32, on the GPU)."""
    out = torch.full((nblocks,), -1, dtype=torch.int32, device="cuda")
    rc = _lib.mfl_probe_xcc(nblocks, out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    _check(rc)
    return out


# ------------------------------------------------------- microbenchmarks
def bench_mfma_raw(op: int, operands: int, n_operands: int, iters: int, nwg: int, sink: int,
                   clocks: int, stream: int) -> int:
    """Enqueue the MFMA issue-rate kernel (mfl_bench_mfma); raw pointers."""
    return _lib.mfl_bench_mfma(op, operands, n_operands, iters, nwg, sink, clocks, stream)


def bench_dma_rate_raw(threads: int, iters: int, nwg: int, depth: int, buf: int, sink: int,
                       clocks: int, stream: int) -> int:
    """Enqueue the direct-to-LDS fetch-rate kernel (mfl_bench_dma_rate); raw pointers."""
    return _lib.mfl_bench_dma_rate(threads, iters, nwg, depth, buf, sink, clocks, stream)


def bench_lds_read_raw(threads: int, iters: int, nwg: int, depth: int, sink: int, clocks: int,
                       stream: int) -> int:
    """Enqueue the LDS read-rate kernel (mfl_bench_lds_read); raw pointers."""
    return _lib.mfl_bench_lds_read(threads, iters, nwg, depth, sink, clocks, stream)


def wall_clock_khz() -> int:
    """Rate of the real-time counter the microbenchmarks record (kHz)."""
    out = ctypes.c_int32(0)
    _check(_lib.mfl_wall_clock_khz(ctypes.byref(out)))
    return int(out.value)


def probe_fragments(algo: str, fetch_a: int, fetch_b: int, A: torch.Tensor, lda: int,
                    B: torch.Tensor, ldb: int, M: int, N: int, K: int) -> np.ndarray:
    """Register dump of one K-step of an LDS kernel (mfl_probe_fragments):
    A and B are device fp16 tensors laid out as the fetch policies expect.
    Returns uint32 words, shape (tiles, threads, words per thread)."""
    words, threads = ctypes.c_int32(0), ctypes.c_int32(0)
    code = algo_code(algo)
    _check(_lib.mfl_probe_fragments(code, fetch_a, fetch_b, M, N, K, None, lda, None, ldb, None,
                                    0, ctypes.byref(words), ctypes.byref(threads), None))
    info = kernel_info(algo)
    tiles = (M // info["bm"]) * (N // info["bn"])
    out = torch.zeros(tiles * threads.value * words.value, dtype=torch.int32, device=A.device)
    stream = torch.cuda.current_stream(A.device).cuda_stream
    _check(_lib.mfl_probe_fragments(code, fetch_a, fetch_b, M, N, K, A.data_ptr(), lda,
                                    B.data_ptr(), ldb, out.data_ptr(), out.numel(),
                                    ctypes.byref(words), ctypes.byref(threads), stream))
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint32).reshape(tiles, threads.value, words.value)

"""Plain shape:stride layout evaluator and thread/value maps (oracle side).

Test infrastructure only (see ``oracle/__init__.py``).

Pages cited below, by title:
  [TiledMMA]  "读懂 CuTe 的 make_tiled_mma：一条 MMA 怎样铺成一块矩阵"
  [retile]    "读懂 CuTe 的 retile_D：给 MMA 寄存器换一种分组方式"
  [L2TC]      "CuTe Layout 到 Tensor Core：从 Shape/Stride 到 Core Matrix"
  [simple]    "cute(7) simple_gemm" (7 简单 GEMM（不用 Shared Memory）)
  [route]     "ldmatrix 怎样对上 MMA 的寄存器：从目的槽位反推源地址"

A layout is a pair (shape, stride) of congruent nested tuples of ints
([L2TC] §1 "最外围：矩阵首先就是一个 Shape + Stride Layout").  An integer
index is split into leaf coordinates with the first leaf varying fastest
([TiledMMA] "从 C 的四个值开始读"); the offset is the sum of
leaf-coordinate times leaf-stride ([TiledMMA] "先固定矩阵和方向": size-1
modes only take coordinate 0).  Composition and right inverse are built
here as brute-force tables (functions), never in shape:stride form, so the
shape:stride algebra of the HIP-side module is checked against plain
function values.
"""
from __future__ import annotations

from typing import Iterable, List, Sequence, Tuple, Union

Nested = Union[int, tuple]


# --------------------------------------------------------------------------
# parsing / printing
# --------------------------------------------------------------------------
def _parse_tuple(s: str, pos: int) -> Tuple[Nested, int]:
    while s[pos] == " ":
        pos += 1
    if s[pos] == "(":
        items = []
        pos += 1
        while True:
            item, pos = _parse_tuple(s, pos)
            items.append(item)
            while s[pos] == " ":
                pos += 1
            if s[pos] == ",":
                pos += 1
                continue
            if s[pos] == ")":
                return tuple(items), pos + 1
            raise ValueError(f"bad layout text at {pos}: {s!r}")
    start = pos
    if s[pos] == "_":          # CuTe prints static ints as _N
        pos += 1
        start = pos
    if s[pos] == "-":
        pos += 1
    while pos < len(s) and s[pos].isdigit():
        pos += 1
    if start == pos:
        raise ValueError(f"bad layout text at {pos}: {s!r}")
    return int(s[start:pos]), pos


def parse(text: str) -> Tuple[Nested, Nested]:
    """Parse "shape:stride", e.g. "((4,8),(2,2)):((32,1),(16,8))"."""
    text = text.strip()
    shape_txt, stride_txt = text.split(":")
    shape, p = _parse_tuple(shape_txt, 0)
    if shape_txt[p:].strip():
        raise ValueError(text)
    stride, p = _parse_tuple(stride_txt, 0)
    if stride_txt[p:].strip():
        raise ValueError(text)
    if not congruent(shape, stride):
        raise ValueError(f"shape and stride are not congruent: {text}")
    return shape, stride


def format_layout(layout) -> str:
    """shape:stride text of a layout, in the form ``parse`` reads."""
    def f(t):
        if isinstance(t, int):
            return str(t)
        return "(" + ",".join(f(x) for x in t) + ")"
    shape, stride = layout
    return f(shape) + ":" + f(stride)


def congruent(a: Nested, b: Nested) -> bool:
    if isinstance(a, int):
        return isinstance(b, int)
    return (isinstance(b, tuple) and len(a) == len(b)
            and all(congruent(x, y) for x, y in zip(a, b)))


def leaves(t: Nested) -> List[int]:
    if isinstance(t, int):
        return [t]
    out: List[int] = []
    for x in t:
        out.extend(leaves(x))
    return out


def size(shape: Nested) -> int:
    n = 1
    for s in leaves(shape):
        n *= s
    return n


# --------------------------------------------------------------------------
# decode / evaluate
# --------------------------------------------------------------------------
def decode(i: int, shape: Nested, unbounded_last: bool = False) -> Nested:
    """Integer -> nested coordinate, first leaf fastest.

    With ``unbounded_last`` the last leaf takes whatever remains (used when
    a composed layout's output runs past the outer layout's size)."""
    ls = leaves(shape)
    coords = []
    rem = i
    for j, s in enumerate(ls):
        if unbounded_last and j == len(ls) - 1:
            coords.append(rem)
            rem = 0
        else:
            coords.append(rem % s)
            rem //= s
    if rem != 0:
        raise IndexError(f"index {i} outside shape {shape}")
    it = iter(coords)

    def rebuild(t):
        if isinstance(t, int):
            return next(it)
        return tuple(rebuild(x) for x in t)

    return rebuild(shape)


def _eval_nested(coord: Nested, shape: Nested, stride: Nested) -> int:
    if isinstance(shape, int):
        assert isinstance(coord, int)
        return coord * stride
    if isinstance(coord, int):          # an integer for a nested mode
        coord = decode(coord, shape)
    return sum(_eval_nested(c, s, d) for c, s, d in zip(coord, shape, stride))


def evaluate(layout: Tuple[Nested, Nested], coord: Nested) -> int:
    """L(coord): ``coord`` is an int (decoded over the whole shape) or a
    tuple with one entry per top-level mode (each an int or a tuple)."""
    shape, stride = layout
    if isinstance(coord, int):
        if coord < 0 or coord >= size(shape):
            raise IndexError(coord)
        coord = decode(coord, shape)
    return _eval_nested(coord, shape, stride)


def table(layout) -> List[int]:
    shape, _ = layout
    return [evaluate(layout, i) for i in range(size(shape))]


def cosize(layout) -> int:
    """Storage needed = largest offset + 1 ([L2TC] §3 size vs cosize)."""
    return max(table(layout)) + 1


# --------------------------------------------------------------------------
# composition / inverse as functions
# --------------------------------------------------------------------------
def compose_table(outer, inner) -> List[int]:
    """(outer o inner)(i) = outer(inner(i)); inner's output integer is decoded
    in outer's shape ([retile] "把编号接到原来的存储上")."""
    shape_o, stride_o = outer
    out = []
    for i in range(size(inner[0])):
        j = evaluate(inner, i)
        c = decode(j, shape_o, unbounded_last=True)
        out.append(_eval_nested(c, shape_o, stride_o))
    return out


def right_inverse_table(values: Sequence[int]) -> List[int]:
    """R with L(R(j)) = j for j < n, where n is the first integer missing
    from the image of L; R(j) is the smallest preimage."""
    first = {}
    for i, v in enumerate(values):
        if v not in first:
            first[v] = i
    out = []
    j = 0
    while j in first:
        out.append(first[j])
        j += 1
    return out


def tv_table(layout, nthr: int) -> List[int]:
    """A TV layout as a table over one index, thread fastest: entry t +
    nthr*v is thread t's value v ([retile] "先确定要从哪些 fragment 位置取
    值")."""
    shape, _ = layout
    nval = size(shape) // nthr
    return [evaluate(layout, (t, v)) for v in range(nval) for t in range(nthr)]


# --------------------------------------------------------------------------
# SM80 atom closed forms printed on the pages (m16n8k16, 32 lanes)
# --------------------------------------------------------------------------
SM80_C_TV = "((4,8),(2,2)):((32,1),(16,8))"        # [TiledMMA] 从 C 的四个值开始读
SM80_A_TV = "((4,8),(2,2,2)):((32,1),(16,8,128))"  # [TiledMMA] A 的八个值和 B 的四个值
SM80_B_TV = "((4,8),(2,2)):((16,1),(8,64))"        # same section


def sm80_c_coord(lane: int, v: int) -> Tuple[int, int]:
    """[TiledMMA] 从 C 的四个值开始读: m = l/4 + 8(v/2), n = 2(l%4) + v%2."""
    return lane // 4 + 8 * (v // 2), 2 * (lane % 4) + v % 2


def sm80_a_coord(lane: int, v: int) -> Tuple[int, int]:
    """[TiledMMA] A 的八个值: m = l/4 + 8((v/2)%2), k = 2(l%4) + v%2 + 8(v/4)."""
    return lane // 4 + 8 * ((v // 2) % 2), 2 * (lane % 4) + v % 2 + 8 * (v // 4)


def sm80_b_coord(lane: int, v: int) -> Tuple[int, int]:
    """[TiledMMA] B 的四个值: n = l/4, k = 2(l%4) + v%2 + 8(v/2)."""
    return lane // 4, 2 * (lane % 4) + v % 2 + 8 * (v // 2)


# --------------------------------------------------------------------------
# TiledMMA partition model ([TiledMMA] sections 第二个参数 … K 方向的线程组)
# --------------------------------------------------------------------------
ATOM_M, ATOM_N, ATOM_K = 16, 8, 16


def perm_m(i: int) -> int:
    """PermM = (8,4):(4,1), p(i) = 4(i%8) + i/8 ([TiledMMA] 用 Layout 改变 M
    方向的坐标顺序)."""
    return 4 * (i % 8) + i // 8


class TiledConfig:
    """One TiledMMA configuration of the [TiledMMA] page.

    thr = (WM, WN, WK) warp counts, thr_stride = strides of the warp-group
    layout (default compact, M fastest); tile = (TM, TN, TK) covered by one
    "tile"; problem = (M, N, K); perm = optional callable on the M index."""

    def __init__(self, thr, problem, thr_stride=None, tile=None, perm=None):
        self.WM, self.WN, self.WK = thr
        if thr_stride is None:
            thr_stride = (1, self.WM, self.WM * self.WN)
        self.thr_stride = thr_stride
        if tile is None:
            tile = (ATOM_M * self.WM, ATOM_N * self.WN, ATOM_K * self.WK)
        self.tile = tile
        self.M, self.N, self.K = problem
        self.perm = perm

    @property
    def nthreads(self):
        return 32 * self.WM * self.WN * self.WK

    def thr_layout_vmnk(self):
        sm, sn, sk = self.thr_stride
        shape = (32, self.WM, self.WN, self.WK)
        stride = (1, 32 * sm if self.WM > 1 else 0, 32 * sn if self.WN > 1 else 0,
                  32 * sk if self.WK > 1 else 0)
        return shape, stride

    def flat_coord(self, t: int):
        """Inverse of ThrLayoutVMNK by search (get_slice / get_flat_coord)."""
        lay = self.thr_layout_vmnk()
        for lane in range(32):
            for wm in range(self.WM):
                for wn in range(self.WN):
                    for wk in range(self.WK):
                        if evaluate(lay, (lane, wm, wn, wk)) == t:
                            return lane, wm, wn, wk
        raise ValueError(t)

    def _reps(self):
        TM, TN, TK = self.tile
        # inside one declared tile, the per-warp atom repeats
        am = TM // (ATOM_M * self.WM)
        an = TN // (ATOM_N * self.WN)
        ak = TK // (ATOM_K * self.WK)
        return am, an, ak, self.M // TM, self.N // TN, self.K // TK

    def _m(self, base_m, wm, im):
        i = base_m + ATOM_M * wm + ATOM_M * self.WM * im
        return self.perm(i) if self.perm else i

    def coords_A(self, t):
        lane, wm, wn, wk = self.flat_coord(t)
        am, an, ak, gm, gn, gk = self._reps()
        out = []
        for rk in range(ak * gk):
            for rm in range(am * gm):
                for v in range(8):
                    m0, k0 = sm80_a_coord(lane, v)
                    out.append((self._m(m0, wm, rm),
                                k0 + ATOM_K * wk + ATOM_K * self.WK * rk))
        return out

    def coords_B(self, t):
        lane, wm, wn, wk = self.flat_coord(t)
        am, an, ak, gm, gn, gk = self._reps()
        out = []
        for rk in range(ak * gk):
            for rn in range(an * gn):
                for v in range(4):
                    n0, k0 = sm80_b_coord(lane, v)
                    out.append((n0 + ATOM_N * wn + ATOM_N * self.WN * rn,
                                k0 + ATOM_K * wk + ATOM_K * self.WK * rk))
        return out

    def coords_C(self, t):
        lane, wm, wn, wk = self.flat_coord(t)
        am, an, ak, gm, gn, gk = self._reps()
        out = []
        for rn in range(an * gn):
            for rm in range(am * gm):
                for v in range(4):
                    m0, n0 = sm80_c_coord(lane, v)
                    out.append((self._m(m0, wm, rm),
                                n0 + ATOM_N * wn + ATOM_N * self.WN * rn))
        return out


def page_trace_configs():
    """The seven configurations the [TiledMMA] page's trace program checks
    (打印布局，核对一次): one warp, four warps, larger input, swapped warp
    order, explicit Tile<64,32,16>, PermM, K-direction warp groups."""
    return {
        "one_warp": TiledConfig((1, 1, 1), (16, 8, 16)),
        "four_warp": TiledConfig((2, 2, 1), (32, 16, 16)),
        "larger_input": TiledConfig((2, 2, 1), (64, 32, 32)),
        "swapped": TiledConfig((2, 2, 1), (32, 16, 16), thr_stride=(2, 1, 0)),
        "tile_64_32_16": TiledConfig((2, 2, 1), (64, 32, 16), tile=(64, 32, 16)),
        "perm_m": TiledConfig((2, 2, 1), (32, 16, 16), perm=perm_m),
        "split_k": TiledConfig((1, 1, 2), (16, 8, 32)),
    }


# --------------------------------------------------------------------------
# ldmatrix.x4 route rule and the Copy-atom layouts ([route] 第二步, 第六步)
# --------------------------------------------------------------------------
LDSM_X4_SRC = "(32,8):(8,1)"            # S: source thread, element in row
LDSM_X4_DST = "(32,(2,4)):(2,(1,64))"   # D = R: destination thread, value


def ldsm_x4_route(b: int, row: int, col: int):
    """Non-transposed m8n8.x4: matrix b, row, col (0..7) ->
    (address lane, receiving lane, output register, half within it)."""
    return 8 * b + row, 4 * row + col // 2, b, col % 2


# --------------------------------------------------------------------------
# gfx950 MFMA operand maps (closed forms, NOT shape:stride on purpose)
# --------------------------------------------------------------------------
# These describe which lane/slot of a wave64 holds which matrix element for
# the CDNA matrix instructions.  The pages say nothing about AMD hardware:
# these maps are pinned only by the GPU probe test against the hardware.
# K order inside a lane is observable only up to a permutation common to A
# and B, so the maps fix "8 (or 4) contiguous K per lane".
MFMA_OPS = {
    # name: (M, N, K, values per lane for A/B, accumulators per lane)
    "f32_32x32x16_f16": (32, 32, 16, 8, 16),
    "f32_16x16x32_f16": (16, 16, 32, 8, 4),
    "f32_32x32x8_f16": (32, 32, 8, 4, 16),
    "f32_16x16x16_f16": (16, 16, 16, 4, 4),
}


def mfma_ab_coord(op: str, lane: int, v: int) -> Tuple[int, int]:
    """(row, k) of A slot v (row = m) or B slot v (row = n) in lane ``lane``."""
    M, N, K, nv, _ = MFMA_OPS[op]
    return lane % M, nv * (lane // M) + v


def mfma_c_coord(op: str, lane: int, v: int) -> Tuple[int, int]:
    """(m, n) of accumulator v in lane ``lane``."""
    M, N, K, nv, nacc = MFMA_OPS[op]
    if M == 32:
        return 8 * (v // 4) + 4 * (lane // 32) + v % 4, lane % 32
    return 4 * (lane // 16) + v, lane % 16

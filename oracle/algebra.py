"""Tiling algebra of the pages, as plain functions (oracle side).

Test infrastructure only (see ``oracle/__init__.py``).  Pages cited by the
titles listed in ``oracle/layout.py``.

The pages build their partitions from a few layout operations: the
``logical_divide`` / ``zipped_divide`` steps of partition_C ([TiledMMA]
"partition_C 怎样把分工应用到一个 Tensor"), and ``upcast``, ``with_shape``,
``logical_product`` and the divides inside retile ([retile] "带着 8 和 2，读一
遍 retile 的源码" and "两个 K fragment 怎样连成一组").  The pages name the
operations and print their results; they do not define them.  Here each one
is written as a function of integer indices (a table), from the property
that pins it, never by manipulating shape:stride text:

  complement(B, M)     the increasing offsets r_0 < r_1 < ... where r_j is the
                       smallest offset in [0, M) not yet reached by B + r_k
                       (k < j); B and its complement together tile [0, M)
  logical_divide(A, B) index i + |B| j  ->  A(B(i) + R(j)),  R = complement(B, |A|)
  zipped_divide(A, T)  per-mode divides of A by T = (T_0, T_1, ...), the
                       tile parts of all modes first, then the rest parts
  logical_product(A,B) index i + |A| j  ->  A(i) + C(B(j)),
                       C = complement(A, |A| cosize(B))
  with_shape(L, S)     the same function on a domain reshaped to S
  upcast(L, N)         a layout of elements viewed in units of N (defined
                       leaf by leaf: it depends on the representation)

A result is returned as (mode sizes, table): the sizes of its top-level
modes and the offset of every flattened index (first mode fastest).  Tests
compare them with the pages' printed layouts evaluated by ``layout.table``.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

from .layout import Nested, decode, evaluate, leaves, size, table, _eval_nested

Result = Tuple[Tuple[int, ...], List[int]]


def _at_unbounded(layout, k: int) -> int:
    """L(k) with L's last leaf taken as unbounded (composition convention of
    [retile] "把编号接到原来的存储上")."""
    shape, stride = layout
    return _eval_nested(decode(k, shape, unbounded_last=True), shape, stride)


def complement_offsets(values: Sequence[int], cotarget: int) -> List[int]:
    """Representatives r_0 < r_1 < ...: each the smallest offset below
    ``cotarget`` not covered by {v + r_k : v in values, k < j}."""
    image = sorted(set(values))
    covered = set()
    reps: List[int] = []
    x = 0
    while True:
        while x in covered:
            x += 1
        if x >= cotarget:
            return reps
        reps.append(x)
        covered.update(x + v for v in image)
        x += 1


def complement(layout, cotarget: int) -> Result:
    reps = complement_offsets(table(layout), cotarget)
    return (len(reps),), reps


def logical_divide(a, b) -> Result:
    """A divided by the single layout B: (tile, rest) over A's whole domain."""
    tb = table(b)
    rest = complement_offsets(tb, size(a[0]))
    out = [_at_unbounded(a, tb[i] + rest[j]) for j in range(len(rest)) for i in range(len(tb))]
    return (len(tb), len(rest)), out


def _mode(a, m):
    shape, stride = a
    if isinstance(shape, int):
        assert m == 0
        return shape, stride
    return shape[m], stride[m]


def _rank(a) -> int:
    return 1 if isinstance(a[0], int) else len(a[0])


def _mode_parts(a, tilers):
    """Per mode m: (tile size, rest size, f(t, r) -> offset within mode m).
    A tiler entry None keeps the whole mode as the tile."""
    parts = []
    for m in range(_rank(a)):
        am = _mode(a, m)
        t = tilers[m] if m < len(tilers) else None
        if t is None:
            n = size(am[0])
            parts.append((n, 1, lambda i, j, am=am: evaluate(am, i)))
            continue
        tb = table(t)
        rest = complement_offsets(tb, size(am[0]))
        parts.append((len(tb), len(rest),
                      lambda i, j, am=am, tb=tb, rest=rest: _at_unbounded(am, tb[i] + rest[j])))
    return parts


def _digits(i: int, radices: Sequence[int]) -> List[int]:
    out = []
    for r in radices:
        out.append(i % r)
        i //= r
    assert i == 0
    return out


def logical_divide_modes(a, tilers) -> Result:
    """Each top-level mode m of A divided by tilers[m] (None: unchanged);
    mode m of the result is (tile_m, rest_m), flattened index t + |T| r."""
    parts = _mode_parts(a, tilers)
    sizes = tuple(p[0] * p[1] for p in parts)
    out = []
    for i in range(size(sizes)):
        dig = _digits(i, sizes)
        out.append(sum(p[2](d % p[0], d // p[0]) for p, d in zip(parts, dig)))
    return sizes, out


def zipped_divide(a, tilers) -> Result:
    """((tile_0, tile_1, ...), (rest_0, rest_1, ...)): mode 0 gathers the tile
    parts of all modes, mode 1 the rest parts ([TiledMMA] "再切出单条指令的
    输出块")."""
    parts = _mode_parts(a, tilers)
    ts = [p[0] for p in parts]
    rs = [p[1] for p in parts]
    nt, nr = size(tuple(ts)), size(tuple(rs))
    out = []
    for r in range(nr):
        rd = _digits(r, rs)
        for t in range(nt):
            td = _digits(t, ts)
            out.append(sum(p[2](ti, ri) for p, ti, ri in zip(parts, td, rd)))
    return (nt, nr), out


def logical_product(a, b) -> Result:
    ta, tb = table(a), table(b)
    cob = max(tb) + 1
    c = complement_offsets(ta, len(ta) * cob)
    out = [ta[i] + c[tb[j]] for j in range(len(tb)) for i in range(len(ta))]
    return (len(ta), len(tb)), out


def compact(shape: Nested):
    """make_layout(shape): column-major strides (first leaf fastest)."""
    acc = [1]

    def build(s):
        if isinstance(s, int):
            d = acc[0]
            acc[0] *= s
            return d
        return tuple(build(x) for x in s)

    return shape, build(shape)


def _shape_div(a: int, b: int) -> int:
    """a / b when b divides a; 1 when a divides b (units of b exceed a)."""
    if a % b == 0:
        return a // b
    if b % a == 0:
        return 1
    raise ValueError(f"{a} and {b} do not divide")


def upcast(layout, n: int):
    """Leaf (s, d): s becomes s / (n / d) and d becomes d / n, each rounded
    up to 1 when the unit is larger ([retile] "upcast<32*8> 按 256 个元素为一
    个单位压缩布局"); stride-0 leaves are unchanged."""
    shape, stride = layout

    def leaf(s, d):
        if d == 0:
            return s, 0
        return _shape_div(s, _shape_div(n, abs(d))), _shape_div(d, n)

    def walk(s, d):
        if isinstance(s, int):
            return leaf(s, d)
        pairs = [walk(x, y) for x, y in zip(s, d)]
        return tuple(p[0] for p in pairs), tuple(p[1] for p in pairs)

    return walk(shape, stride)


def product_each(shape: Nested) -> Tuple[int, ...]:
    if isinstance(shape, int):
        return (shape,)
    return tuple(size(s) for s in shape)


# --------------------------------------------------------------------------
# the pages' two derivations, step by step on function tables
# --------------------------------------------------------------------------
def divide_table(tab: Sequence[int], tiler) -> Result:
    """A function given by its table, divided by the single layout ``tiler``
    over its whole domain: index i + |T| j -> tab[T(i) + R(j)]."""
    tt = table(tiler)
    rest = complement_offsets(tt, len(tab))
    return (len(tt), len(rest)), [tab[tt[i] + rest[j]] for j in range(len(rest)) for i in range(len(tt))]


def product_tables(ta: Sequence[int], tb: Sequence[int]) -> Result:
    """logical_product of two functions given by their tables."""
    c = complement_offsets(ta, len(ta) * (max(tb) + 1))
    return (len(ta), len(tb)), [ta[i] + c[tb[j]] for j in range(len(tb)) for i in range(len(ta))]


def _factor_mode(f, n: int):
    """Leaves (size, step) of one mode whose values are f(0..n-1), f(0) = 0:
    each leaf is the longest run of constant step, in units of the leaves
    before it, whose length divides what is left of the mode."""
    if n == 1:
        return [1], [0]
    ls, ld = [], []
    blk = 1
    while blk < n:
        left = n // blk
        d = f(blk)
        run = 2
        while run < left and f(blk * run) == run * d:
            run += 1
        while left % run:
            run -= 1
        ls.append(run), ld.append(d)
        blk *= run
    return ls, ld


def factor_table(tab: Sequence[int], shape: Tuple[int, ...]):
    """A layout with top-level modes ``shape`` (first fastest) that has the
    table ``tab``, each mode split into the fewest leaves of constant step: the
    form the pages print for a with_shape result ([retile] "带着 8 和 2，读一遍
    retile 的源码"), which upcast then reads leaf by leaf.  Raises ValueError
    when no such layout has this table."""
    assert len(tab) == size(shape) and tab[0] == 0
    ms, md = [], []
    step = 1
    for n in shape:
        ls, ld = _factor_mode(lambda k, st=step: tab[k * st], n)
        ms.append(ls[0] if len(ls) == 1 else tuple(ls))
        md.append(ld[0] if len(ld) == 1 else tuple(ld))
        step *= n
    out = (tuple(ms), tuple(md))
    if table(out) != list(tab):
        raise ValueError("table is not a shape:stride layout over this shape")
    return out


def right_inverse_shaped(tv, shape: Tuple[int, ...]):
    """right_inverse(TV).with_shape(shape): position (first coordinate fastest)
    -> TV index lane + nlanes*value, as a layout over ``shape``."""
    from .layout import right_inverse_table
    inv = right_inverse_table(table(tv))
    assert len(inv) == size(shape), "TV layout must cover the tile exactly"
    return factor_table(inv, shape)


def _divided(mode_fn, n: int, tiler) -> List[int]:
    """One mode (a function of its index, domain n) divided by ``tiler``:
    index i + |T| j -> mode(T(i) + R(j)), R = complement(T, n)."""
    tt = table(tiler)
    rest = complement_offsets(tt, n)
    return [mode_fn(tt[i] + rest[j]) for j in range(len(rest)) for i in range(len(tt))]


def partition_c(c_layout, atom_tv, atom_mn, nlanes: int, warps_mn, tile=None):
    """partition_C ([TiledMMA] "partition_C 怎样把分工应用到一个 Tensor") of
    the rank-2 tensor ``c_layout`` (M, N), on functions of indices:

      1. each mode divided by the tile entry: ``tile`` = (layout M, layout N),
         the tiled MMA's permutations ("用 Layout 改变 M 方向的坐标顺序"),
         default compact (AtomM*WM):1, (AtomN*WN):1;
      2. each mode divided again by the atom extent (AtomM:1, AtomN:1):
         index = a + Atom*b, the atom parts (aM, aN) zipped into one mode
         q = aM + AtomM*aN and the block indices (bM, bN) into the other;
      3. q replaced by the atom's C TV layout: (lane, value) -> q;
      4. each block index divided by the warp count: b = w + W*r.

    Returns ({thread: [offset of (value, rM, rN), value fastest]}, step 1
    result, step 2 result), thread = lane + nlanes*(wM + WM*wN)."""
    am, an = atom_mn
    wm_n, wn_n = warps_mn
    shape, stride = c_layout
    nM, nN = size(shape[0]), size(shape[1])
    cm = lambda k: _at_unbounded((shape[0], stride[0]), k)
    cn = lambda k: _at_unbounded((shape[1], stride[1]), k)
    tiles = tile or ((am * wm_n, 1), (an * wn_n, 1))
    # step 1
    fM = _divided(cm, nM, tiles[0])
    fN = _divided(cn, nN, tiles[1])
    step1 = (len(fM), len(fN)), [fM[i] + fN[j] for j in range(len(fN)) for i in range(len(fM))]
    # step 2
    gM = _divided(lambda k: fM[k], len(fM), (am, 1))
    gN = _divided(lambda k: fN[k], len(fN), (an, 1))
    bM, bN = len(gM) // am, len(gN) // an
    assert bM * am == len(gM) and bN * an == len(gN), "the atom must divide the tile"

    def c_tensor(q, b):
        return gM[q % am + am * (b % bM)] + gN[q // am + an * (b // bM)]

    step2 = (am * an, bM * bN), [c_tensor(q, b) for b in range(bM * bN) for q in range(am * an)]
    # steps 3 and 4
    tv = table(atom_tv)
    nvals = len(tv) // nlanes
    rM, rN = bM // wm_n, bN // wn_n
    assert rM * wm_n == bM and rN * wn_n == bN, "the warps must divide the blocks"
    out = {}
    for wn in range(wn_n):
        for wm in range(wm_n):
            for lane in range(nlanes):
                vals = []
                for jn in range(rN):
                    for im in range(rM):
                        b = (wm + wm_n * im) + bM * (wn + wn_n * jn)
                        vals.extend(c_tensor(tv[lane + nlanes * v], b) for v in range(nvals))
                out[lane + nlanes * (wm + wm_n * wn)] = vals
    return out, step1, step2


def tiled_product(a, b) -> Result:
    """logical_product(A, B) with B's top-level modes kept apart: sizes
    (|A|, |B_0|, |B_1|, ...) ([TiledMMA] "第二个参数怎样把一个 warp 扩展成四个")."""
    bs = b[0] if isinstance(b[0], tuple) else (b[0],)
    sizes, tab = product_tables(table(a), table(b))
    return (sizes[0],) + tuple(size(x) for x in bs), tab


def retile(frag, tiled_tv, tile_shape: Tuple[int, ...], nthr: int, atom_nval: int):
    """retile_D's chain ([retile] "带着 8 和 2，读一遍 retile 的源码" and "两个 K
    fragment 怎样连成一组") for a register fragment ``frag`` (tCrX: mode 0 the
    V values of one MMA, then one mode per repeat direction), the tiled TV
    layout of the copy's reference tile ``tiled_tv`` over ``tile_shape``:

      frg_layout_mn = upcast<nthr*V>(right_inverse(TV).with_shape(tile))
      G             = right_inverse(frg_layout_mn)
      frg_layout_v  = divide(logical_product(V:1, G), atom_nval:1)
      t_tensor      = zipped_divide(frag, (V, product_each(frg_layout_mn)...))
      result        = t_tensor with mode 0 composed with frg_layout_v, the
                      rest coordinate of the value mode fixed to 0

    Returns a dict of the intermediate results and ``slots``: {(copy index
    c, rest index r): register slot}, c over the copy atom's values (and its
    groups), r over the remaining repeats (first fastest)."""
    from .layout import right_inverse_table
    V = size(frag[0][0])
    shaped = right_inverse_shaped(tiled_tv, tile_shape)
    mn = upcast(shaped, nthr * V)
    each = product_each(mn[0])
    g = right_inverse_table(table(mn))
    prod = product_tables(list(range(V)), g)
    fv = divide_table(prod[1], (atom_nval, 1))
    tiler = [(V, 1)] + [(e, 1) for e in each]
    tt = zipped_divide(frag, tiler)
    (n_t, n_r), t_tab = tt
    assert _mode_parts(frag, tiler)[0][1] == 1, "the value mode is taken whole"
    slots = {(c, r): t_tab[fv[1][c] + n_t * r] for r in range(n_r) for c in range(len(fv[1]))}
    return {"with_shape": shaped, "frg_layout_mn": mn, "product_each": each,
            "G": g, "product": prod, "frg_layout_v": fv, "t_tensor": tt, "slots": slots}

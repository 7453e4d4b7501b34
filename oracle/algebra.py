"""Tiling algebra of the pages, as plain functions (oracle side).

Test infrastructure only (see ``oracle/__init__.py``).  Pages cited by the
titles listed in ``oracle/layout.py``.

The pages build their partitions from a few layout operations: divides
([TiledMMA] "partition_C 怎样把分工应用到一个 Tensor"), and ``upcast``,
``with_shape``, ``logical_product`` and the divides inside retile ([retile]
"带着 8 和 2，读一遍 retile 的源码" and "两个 K fragment 怎样连成一组").  The
pages name the operations and print their results; they do not define them.
Here each one is written as a function of integer indices (a table), from
the property that pins it, never by manipulating shape:stride text:

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

partition_C is computed from the element each (thread, value, repeat)
holds, in plain loops; retile, which the pages define only by its
algorithm, by that algorithm's steps on tables.
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
    """The layout read in units of n elements, leaf by leaf ([retile] "带着 8
    和 2，读一遍 retile 的源码"): leaf (s, d) keeps s / (n / d) coordinates at
    stride d / n, and a leaf whose whole extent lies inside one unit shrinks
    to one coordinate; stride-0 leaves are unchanged."""
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


def _warp_block(w: int, nwarps: int, reps: int, rep: int) -> int:
    """Atom block held by warp w in its rep-th repeat along one direction: the
    warps take turns, block w + nwarps * rep."""
    return w + nwarps * rep


def _atom_mn(q: int, am: int):
    """Element q of the atom's C block (first coordinate fastest) -> (m, n)."""
    return q % am, q // am


def _c_row(perm: Sequence[int], am: int, a: int, b: int) -> int:
    """Row of C for atom coordinate a of atom block b, blocks numbered down a
    tile first and then across tiles; inside a tile the logical row i is the
    physical row perm[i]."""
    per_tile = len(perm) // am
    return perm[a + am * (b % per_tile)] + len(perm) * (b // per_tile)


def partition_c(c_layout, atom_tv, atom_mn, nlanes: int, warps_mn, tile=None):
    """partition_C of a tiled MMA ([TiledMMA] "partition_C 怎样把分工应用到一个
    Tensor"), as the element every thread holds, by brute force over threads,
    values and repeats.

    The atom (AtomM x AtomN, C layout ``atom_tv``: lane + nlanes*value -> q, q
    = m + AtomM*n) is repeated over WM x WN warps; C (modes M, N of the storage
    layout ``c_layout``) is covered by tiles whose rows are permuted by the
    tile entries ("用 Layout 改变 M 方向的坐标顺序"; default compact
    AtomM*WM:1, AtomN*WN:1).  Along M the atom-sized row blocks are numbered
    down a tile and then across tiles, and warp row wm holds blocks wm, wm +
    WM, wm + 2 WM, ... (the interleaving of "把剩余块分给 M、N 方向的线程组");
    likewise along N.  Lane l's value v is atom element q = atom_tv(l, v).

    Returns {thread: [C offset of (value, rM, rN), value fastest]}, thread =
    lane + nlanes*(wM + WM*wN).  The tile entries must permute their rows."""
    am, an = atom_mn
    wm_n, wn_n = warps_mn
    shape, _ = c_layout
    n_m, n_n = size(shape[0]), size(shape[1])
    tiles = tile or ((am * wm_n, 1), (an * wn_n, 1))
    perm_m, perm_n = table(tiles[0]), table(tiles[1])
    assert sorted(perm_m) == list(range(len(perm_m))), "the M entry must permute the tile's rows"
    assert sorted(perm_n) == list(range(len(perm_n))), "the N entry must permute the tile's columns"
    assert n_m % len(perm_m) == 0 and n_n % len(perm_n) == 0, "the tile must divide C"
    assert len(perm_m) % am == 0 and len(perm_n) % an == 0, "the atom must divide the tile"
    blocks_m = len(perm_m) // am * (n_m // len(perm_m))
    blocks_n = len(perm_n) // an * (n_n // len(perm_n))
    assert blocks_m % wm_n == 0 and blocks_n % wn_n == 0, "the warps must divide the blocks"
    r_m, r_n = blocks_m // wm_n, blocks_n // wn_n
    tv = table(atom_tv)
    nvals = len(tv) // nlanes
    out = {}
    for wn in range(wn_n):
        for wm in range(wm_n):
            for lane in range(nlanes):
                vals = []
                for jn in range(r_n):
                    for im in range(r_m):
                        for v in range(nvals):
                            ma, na = _atom_mn(tv[lane + nlanes * v], am)
                            m = _c_row(perm_m, am, ma, _warp_block(wm, wm_n, r_m, im))
                            n = _c_row(perm_n, an, na, _warp_block(wn, wn_n, r_n, jn))
                            vals.append(evaluate(c_layout, (m, n)))
                out[lane + nlanes * (wm + wm_n * wn)] = vals
    return out


def tiled_product(a, b) -> Result:
    """logical_product(A, B) with B's top-level modes kept apart: sizes
    (|A|, |B_0|, |B_1|, ...) ([TiledMMA] "第二个参数怎样把一个 warp 扩展成四个")."""
    bs = b[0] if isinstance(b[0], tuple) else (b[0],)
    sizes, tab = product_tables(table(a), table(b))
    return (sizes[0],) + tuple(size(x) for x in bs), tab


def retile(frag, tiled_tv, tile_shape: Tuple[int, ...], nthr: int, atom_nval: int):
    """retile_D ([retile] "带着 8 和 2，读一遍 retile 的源码" and "两个 K
    fragment 怎样连成一组"): the pages define it only by its algorithm, so this
    follows the algorithm's steps in the pages' order, each on a function
    table.  ``frag`` is one thread's register fragment (mode 0 the V values
    of one MMA, then a mode per repeat direction); ``tiled_tv`` the copy's TV
    layout over the reference tile of ``tile_shape``.

    First the tile positions are numbered by the copy index that reaches
    them (the right inverse, reshaped to the tile) and read in units of
    nthr*V, which gives each position the MMA block it belongs to; the right
    inverse of that gives each block number its coarse position.  Pairing
    the V values of a block with that position (a logical product) and
    cutting the result into groups of ``atom_nval`` gives the copy's value
    order; the fragment, split into the V values and the blocks the copy
    covers along each repeat mode, is then read in that order.

    Returns the intermediate results and ``slots``: {(copy index c, rest
    index r): register slot}, c over the copy atom's values and groups, r over
    the repeats the copy leaves (first fastest)."""
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

"""Pins for the oracle's tiling algebra (oracle/algebra.py).

Expected values are the pages' printed intermediate results (tests/golden/
algebra.txt, retile.txt and tiledmma_tiling.txt, each line cited there),
closed forms of the operations on compact layouts, and brute-force
properties (a complement tiles its cotarget; a divide is a bijective
re-indexing).  The two derivations (partition_C, retile) are also checked
against the closed-form index model in oracle/layout.py, which the page
tables pin separately.  The last tests plant plausible mistakes in the
oracle and check that these pins catch them.
"""
import itertools
import random

import pytest

from oracle import algebra as G
from oracle import layout as L
from helpers import keyed, lines, pairs

P = L.parse


def _golden(key):
    return keyed("algebra.txt", key)


def _split_eq(tokens):
    i = tokens.index("=")
    return tokens[:i], tokens[i + 1]


def _tup(text):
    return tuple(int(x) for x in text.strip("()").split(","))


def _shape(text):
    """A printed shape alone (nested tuple text)."""
    shape, _ = P(text + ":" + text)
    return shape


# ------------------------------------------------------------ page values
@pytest.mark.parametrize("case", ["A", "Bx1", "Bx2", "Bx4"])
def test_retile_steps_match_page(case):
    args = {t[0]: t[1:] for t in _golden("retile_case")}[case]
    frag, tv, shape, nthr, nval = P(args[0]), P(args[1]), _tup(args[2]), int(args[3]), int(args[4])
    r = G.retile(frag, tv, shape, nthr, nval)
    V = L.size(frag[0][0]) if isinstance(frag[0][0], tuple) else frag[0][0]
    steps = [t[1:] for t in _golden("retile_step") if t[0] == case]
    assert steps
    for name, val in steps:
        if name == "upcast_n":
            assert nthr * V == int(val)
        elif name == "with_shape":
            assert r["with_shape"] == P(val)          # the representation upcast reads
        elif name == "frg_mn":
            assert r["frg_layout_mn"] == P(val)
        elif name == "product_each":
            assert r["product_each"] == _tup(val)
        elif name == "G":
            assert r["G"] == L.table(P(val))
        elif name in ("product", "frg_v"):
            sizes, tab = r["product" if name == "product" else "frg_layout_v"]
            want = P(val)
            assert tab == L.table(want)
            assert sizes == tuple(L.size(s) for s in want[0])
        elif name == "t_tensor":
            want = P(val)
            assert r["t_tensor"][1] == L.table(want)
            assert r["t_tensor"][0] == tuple(L.size(s) for s in want[0])
        elif name == "t_tensor_shape":
            assert r["t_tensor"][0] == tuple(L.size(s) for s in _shape(val))
        elif name == "v_tensor_shape":
            assert (len(r["frg_layout_v"][1]), r["t_tensor"][0][1]) == \
                tuple(L.size(s) for s in _shape(val))
        elif name in ("v_tensor", "result"):
            want = L.table(P(val))
            n_c = len(r["frg_layout_v"][1])
            got = [r["slots"][(i % n_c, i // n_c)] for i in range(len(want))]
            assert got == want and len(r["slots"]) == len(want)
        else:
            raise AssertionError(name)


def test_retile_result_matches_printed_tXr_layouts():
    printed = {t[0]: t[1] for t in keyed("retile.txt", "print")}
    cases = {"A": "tXrA", "Bx1": "tXrB", "Bx2": "tXrB_x2"}
    args = {t[0]: t[1:] for t in _golden("retile_case")}
    for case, name in cases.items():
        a = args[case]
        r = G.retile(P(a[0]), P(a[1]), _tup(a[2]), int(a[3]), int(a[4]))
        want = L.table(P(printed[name]))
        n_c = len(r["frg_layout_v"][1])
        assert [r["slots"][(i % n_c, i // n_c)] for i in range(len(want))] == want


def test_with_shape_matches_printed_inverses():
    got = {t[0]: t[1] for t in keyed("retile.txt", "rinv_with_shape")}
    assert G.right_inverse_shaped(P(L.SM80_B_TV), (8, 16)) == P(got["B"])
    k32 = P("((4,8),(2,2,2)):((16,1),(8,64,128))")
    assert G.right_inverse_shaped(k32, (8, 32)) == \
        P({t[0]: t[1] for t in keyed("retile.txt", "rinv_with_shape_k32")}["B"])


def test_k_gather_lane0_elements():
    """Slots 0..7 of lane 0's n = 0 group hold the printed B elements."""
    a = {t[0]: t[1:] for t in _golden("retile_case")}["Bx4"]
    r = G.retile(P(a[0]), P(a[1]), (8, 32), 32, 8)
    want = pairs(next(s for s in lines("algebra.txt") if s.startswith("gather_lane0")))
    tv = P(a[1])
    # fragment slot s of lane 0 is copy value s (the gather result is 0..7)
    slots = [r["slots"][(c, 0)] for c in range(8)]
    assert slots == list(range(8))
    # copy value c of lane 0 is TV value c: position n + 8k
    got = [(q % 8, q // 8) for q in (L.evaluate(tv, (0, c)) for c in range(8))]
    assert got == want


def test_k_gather_vs_direct_divide():
    """The gather tile (4,1,2) reads slots 0..7; zipped_divide(tCrB, 8:1)
    reads 0..3 and 8..11; index 7 decodes differently in the two shapes."""
    frag = P("(4,4,2):(1,8,4)")
    slots = {t[0]: [int(x) for x in t[1:]] for t in
             ([s.split()[0]] + s.split()[1:] for s in lines("retile.txt")
              if s.startswith("gather_slots"))}
    r = G.retile(frag, P("((4,8),(2,2,2)):((16,1),(8,64,128))"), (8, 32), 32, 8)
    assert [r["slots"][(c, 0)] for c in range(8)] == slots["gather_slots_retile"]
    sizes, tab = G.divide_table(L.table(frag), (8, 1))
    assert tab[:8] == slots["gather_slots_direct"]
    for shp, idx, coord, slot in _golden("decode"):
        shape = _tup(shp)
        c = tuple(L.decode(int(idx), shape))
        assert c == _tup(coord)
        assert L.evaluate((shape, frag[1]), c) == int(slot)


@pytest.mark.parametrize("key", ["zdiv", "ldiv_modes"])
def test_direct_divides_match_page(key):
    for toks in _golden(key):
        (a, t), want = _split_eq(toks)
        if key == "zdiv":
            sizes, tab = G.logical_divide(P(a), P(t))
        else:
            sizes, tab = G.logical_divide_modes(P(a), [P(t.rstrip(";"))])
        w = P(want)
        assert tab == L.table(w)
        assert sizes == tuple(L.size(s) for s in w[0])


def test_tiled_product_matches_page():
    seen = 0
    for toks in _golden("tiled_product"):
        (a, b), want = _split_eq(toks)
        sizes, tab = G.tiled_product(P(a), P(b))
        w = P(want)
        assert tab == L.table(w) and sizes == w[0]
        seen += 1
    # the same thread layouts as the tiling fixture prints
    thr = {t[0]: t[1] for t in keyed("tiledmma_tiling.txt", "thr_layout")}
    assert G.tiled_product(P("32:1"), P("(2,2,1):(1,2,0)"))[1] == L.table(P(thr["four_warp"]))
    assert G.tiled_product(P("32:1"), P("(2,2,1):(2,1,0)"))[1] == L.table(P(thr["swapped"]))
    assert G.tiled_product(P("32:1"), P("(1,1,2):(0,0,1)"))[1] == L.table(P(thr["split_k"]))
    assert seen == 3


def test_partition_c_page_steps():
    """The printed intermediate tensors pin the divides the page applies (by
    the tile, then by the atom); the partition itself is pinned by thread 0's
    printed view and the printed start coordinates."""
    c = P(_golden("pc_c")[0][0])
    out = G.partition_c(c, P(L.SM80_C_TV), (16, 8), 32, (2, 2))
    want_sizes = [_tup(x) for x in _golden("pc_t_tensor_sizes")[0]]
    assert _tup(_golden("pc_t_tile")[0][0]) == (16 * 2, 8 * 2)
    s1 = G.logical_divide_modes(c, [(32, 1), (16, 1)])
    assert s1[0] == tuple(a * b for a, b in want_sizes)
    # the printed c_tensor is the tiling fixture's only such line
    (only,) = [s for s in lines("tiledmma_tiling.txt") if s.startswith("c_tensor")]
    s2 = G.zipped_divide(c, [(16, 1), (8, 1)])
    assert s2[1] == L.table(P(only.split()[1]))
    # lane 0 value 2 -> block (8,0) -> offset 128
    toks = _golden("pc_tv")[0]
    lane, v, blk, off = int(toks[1]), int(toks[3]), _tup(toks[5]), int(toks[7])
    q = L.evaluate(P(L.SM80_C_TV), (lane, v))
    assert (q % 16, q // 16) == blk
    assert out[0][v] == off
    # thread 0's view and offsets
    assert out[0] == [int(x) for x in next(iter(keyed("tiledmma_tiling.txt",
                                                        "partition_C_thread0_offsets")))]
    assert out[0] == L.table(P(next(iter(keyed("tiledmma_tiling.txt",
                                               "partition_C_thread0")))[0]))
    for t, coord in _golden("pc_start"):
        m, n = _tup(coord)
        assert out[int(t)][0] == L.evaluate(c, (m, n))


def test_partition_c_larger_input_view():
    view = next(iter(keyed("tiledmma_tiling.txt", "partition_C_view")))
    c = P("(64,32):(32,1)")
    out = G.partition_c(c, P(L.SM80_C_TV), (16, 8), 32, (2, 2))
    assert out[0] == L.table(P(view[1]))


def test_partition_c_with_perm_m_matches_printed_coords():
    c = P("(32,16):(16,1)")
    out = G.partition_c(c, P(L.SM80_C_TV), (16, 8), 32, (2, 2),
                              tile=(P("(8,4):(4,1)"), (16, 1)))
    from helpers import table as gtable
    rows = gtable("tiledmma_tiling.txt", "C perm_m")
    assert rows
    for t, want in rows.items():
        assert [(o // 16, o % 16) for o in out[int(t)]] == want


@pytest.mark.parametrize("name", list(L.page_trace_configs()))
def test_partition_c_equals_closed_form_model(name):
    """The algebraic chain and the closed-form thread model agree on every
    thread and value of the seven page configurations."""
    cfg = L.page_trace_configs()[name]
    M, N = cfg.M, cfg.N
    c = (M, N), (N, 1)
    tile = None
    if name == "tile_64_32_16":
        tile = ((64, 1), (32, 1))
    if name == "perm_m":
        tile = (P("(8,4):(4,1)"), (16, 1))
    out = G.partition_c(c, P(L.SM80_C_TV), (16, 8), 32, (cfg.WM, cfg.WN), tile=tile)
    for t in range(cfg.nthreads):
        lane, wm, wn, wk = cfg.flat_coord(t)
        got = out[lane + 32 * (wm + cfg.WM * wn)]
        assert got == [m * N + n for m, n in cfg.coords_C(t)], (name, t)


# ------------------------------------------------------------ closed forms
@pytest.mark.parametrize("s,d,M", [(4, 2, 16), (4, 1, 32), (2, 4, 32), (8, 2, 64), (3, 1, 12),
                                   (2, 3, 18), (1, 5, 10)])
def test_complement_of_one_leaf(s, d, M):
    """complement(s:d, M) = (d, M/(s d)):(1, s d) when s d divides M (size-1
    parts dropped): the offsets below d, then whole blocks of s d."""
    reps = G.complement(((s,), (d,)), M)[1]
    want = [a + s * d * b for b in range(M // (s * d)) for a in range(d)]
    assert reps == want


def _random_tiling(rng):
    """A layout B whose strides nest (each stride a multiple of the extent
    below it), and a cotarget M its cosize divides."""
    n = rng.randint(1, 3)
    shape, stride, ext = [], [], 1
    for _ in range(n):
        gap = rng.choice([1, 1, 2, 3])
        s = rng.choice([2, 3, 4])
        stride.append(ext * gap)
        shape.append(s)
        ext = ext * gap * s
    order = list(range(n))
    rng.shuffle(order)
    b = (tuple(shape[i] for i in order), tuple(stride[i] for i in order))
    return b, ext * rng.choice([1, 2, 3])


def test_complement_tiles_its_cotarget():
    rng = random.Random(5)
    for _ in range(200):
        b, M = _random_tiling(rng)
        reps = G.complement(b, M)[1]
        sums = sorted(x + r for r in reps for x in L.table(b))
        assert sums == list(range(M)), (b, M)
        assert reps == sorted(reps)


def test_divides_are_bijective_reindexings():
    """(tile, rest) of a divide of an injective layout hits every offset of
    the layout once, and the tile mode is the tiler composed in."""
    rng = random.Random(6)
    for _ in range(100):
        b, M = _random_tiling(rng)
        a = ((M,), (rng.choice([1, 2]),))
        sizes, tab = G.logical_divide(a, b)
        assert sorted(tab) == sorted(L.table(a))
        assert tab[:sizes[0]] == [a[1][0] * x for x in L.table(b)]


def test_zipped_divide_is_block_indexing():
    """A row-major R x C matrix zipped by (tm:1, tn:1): ((i, j), (bi, bj)) ->
    (bi tm + i) C + (bj tn + j)."""
    for R, Cc, tm, tn in [(8, 6, 2, 3), (16, 16, 4, 8), (12, 4, 3, 4), (6, 10, 6, 5)]:
        sizes, tab = G.zipped_divide(((R, Cc), (Cc, 1)), [(tm, 1), (tn, 1)])
        assert sizes == (tm * tn, (R // tm) * (Cc // tn))
        for bj in range(Cc // tn):
            for bi in range(R // tm):
                for j in range(tn):
                    for i in range(tm):
                        idx = (i + tm * j) + tm * tn * (bi + (R // tm) * bj)
                        assert tab[idx] == (bi * tm + i) * Cc + bj * tn + j


def test_logical_product_of_compact_layouts_is_compact():
    for s, t in [(4, 2), (8, 1), (2, 8), (3, 5)]:
        sizes, tab = G.logical_product(((s,), (1,)), ((t,), (1,)))
        assert sizes == (s, t) and tab == list(range(s * t))
    # a strided A leaves gaps that the product fills from the complement
    sizes, tab = G.logical_product(((2,), (2,)), ((3,), (1,)))
    assert tab == [0, 2, 1, 3, 4, 6]


def test_upcast_of_row_major_rows():
    """A row-major (R, C) layout of halves in units of u | C: (R, C/u):(C/u, 1)."""
    for R, Cc, u in [(8, 16, 8), (4, 32, 4), (16, 8, 8), (2, 64, 16)]:
        assert G.upcast(((R, Cc), (Cc, 1)), u) == ((R, Cc // u), (Cc // u, 1))


def test_factor_table_recovers_canonical_layouts():
    """A layout whose adjacent leaves never continue each other is the unique
    fewest-leaf factorisation of its own table."""
    rng = random.Random(7)
    for _ in range(200):
        modes_s, modes_d = [], []
        for _m in range(rng.randint(1, 3)):
            n = rng.randint(1, 3)
            ls = [rng.choice([2, 3, 4]) for _ in range(n)]
            ld = [rng.choice([1, 2, 5, 7, 16, 33]) for _ in range(n)]
            if any(ld[i + 1] == ls[i] * ld[i] for i in range(n - 1)):
                continue
            modes_s.append(ls[0] if n == 1 else tuple(ls))
            modes_d.append(ld[0] if n == 1 else tuple(ld))
        if not modes_s:
            continue
        lay = (tuple(modes_s), tuple(modes_d))
        tab = L.table(lay)
        if len(set(tab)) != len(tab):
            continue                                  # skip non-injective draws
        shape = tuple(L.size(s) for s in lay[0])
        assert G.factor_table(tab, shape) == lay


# ---------------------------------------------------- planted mistakes
def _pins_pass():
    """Every pin above, page values and closed forms alike."""
    try:
        for case in ("A", "Bx1", "Bx2", "Bx4"):
            test_retile_steps_match_page(case)
        test_retile_result_matches_printed_tXr_layouts()
        test_with_shape_matches_printed_inverses()
        test_k_gather_lane0_elements()
        test_k_gather_vs_direct_divide()
        test_direct_divides_match_page("zdiv")
        test_direct_divides_match_page("ldiv_modes")
        test_tiled_product_matches_page()
        test_partition_c_page_steps()
        test_partition_c_larger_input_view()
        test_partition_c_with_perm_m_matches_printed_coords()
        for name in L.page_trace_configs():
            test_partition_c_equals_closed_form_model(name)
        for s_, d, M in [(4, 2, 16), (2, 4, 32), (2, 3, 18)]:
            test_complement_of_one_leaf(s_, d, M)
        test_complement_tiles_its_cotarget()
        test_divides_are_bijective_reindexings()
        test_zipped_divide_is_block_indexing()
        test_logical_product_of_compact_layouts_is_compact()
        test_upcast_of_row_major_rows()
        test_factor_table_recovers_canonical_layouts()
    except (AssertionError, ValueError, IndexError, KeyError, ZeroDivisionError, TypeError):
        return False
    return True


def test_pins_pass_on_the_oracle():
    assert _pins_pass()


def _mut_complement_by_cosize(values, cotarget):
    """Mistake: the complement steps by the cosize, as if B were compact."""
    step = max(values) + 1
    return list(range(0, cotarget, step))


def _mut_zipped_rest_first(a, tilers):
    """Mistake: the rest parts in mode 0 and the tile parts in mode 1."""
    sizes, tab = _ORIG["zipped_divide"](a, tilers)
    nt, nr = sizes
    return (nr, nt), [tab[r * nt + t] for t in range(nt) for r in range(nr)]


def _mut_upcast_floor(layout, n):
    shape, stride = layout

    def leaf(s, d):
        return (max(1, s * d // n), max(1, d // n)) if d else (s, 0)

    def walk(s, d):
        if isinstance(s, int):
            return leaf(s, d)
        pr = [walk(x, y) for x, y in zip(s, d)]
        return tuple(p[0] for p in pr), tuple(p[1] for p in pr)
    return walk(shape, stride)


def _mut_product_no_complement(ta, tb):
    return (len(ta), len(tb)), [ta[i] + tb[j] for j in range(len(tb)) for i in range(len(ta))]


def _mut_factor_swapped(tab, shape):
    lay = _ORIG["factor_table"](tab, shape)
    return (lay[0][::-1], lay[1][::-1])


def _mut_warp_block_consecutive(w, nwarps, reps, rep):
    """Mistake: each warp takes a run of consecutive blocks."""
    return w * reps + rep


def _mut_atom_mn_swapped(q, am):
    """Mistake: the atom element read n fastest."""
    return q // am, q % am


def _mut_c_row_unpermuted(perm, am, a, b):
    """Mistake: the tile entry's row permutation ignored."""
    return a + am * b


_ORIG = {"zipped_divide": G.zipped_divide, "factor_table": G.factor_table}


@pytest.mark.parametrize("name,fn", [
    ("complement_offsets", _mut_complement_by_cosize),
    ("zipped_divide", _mut_zipped_rest_first),
    ("upcast", _mut_upcast_floor),
    ("product_tables", _mut_product_no_complement),
    ("factor_table", _mut_factor_swapped),
    ("_warp_block", _mut_warp_block_consecutive),
    ("_atom_mn", _mut_atom_mn_swapped),
    ("_c_row", _mut_c_row_unpermuted),
])
def test_planted_mistakes_are_caught(monkeypatch, name, fn):
    monkeypatch.setattr(G, name, fn)
    assert not _pins_pass(), name

"""The layout module's tiling algebra (C++ behind include/mfl_layout.h)
against the pages' printed results and against the oracle (oracle/algebra.py)
on random inputs; then the same derivations for the gfx950 MFMA atoms, checked
against the fragment coordinates the GEMM kernels use.  No GPU needed: the
layout entry points are host code."""
import random

import numpy as np
import pytest

import mma_fragment_layouts_tn_amd as mfl
from oracle import algebra as G
from oracle import layout as L
from helpers import keyed

P = L.parse
F = L.format_layout

A32, A16 = "f32_32x32x16_f16", "f32_16x16x32_f16"
# BM, BN, BK, waves along M, N, K, and the matrix instruction
KERNEL_TILES = {"lds128": (128, 128, 32, 2, 2, 1, A32), "lds256": (256, 256, 64, 2, 4, 1, A32),
                "lds256w4": (256, 256, 64, 2, 2, 1, A32), "lds128w1": (128, 128, 32, 1, 1, 1, A32),
                "splitk": (128, 64, 128, 1, 1, 4, A32),
                "lds256w4_16": (256, 256, 64, 2, 2, 1, A16),
                "lds256_16": (256, 256, 64, 2, 4, 1, A16),
                "lds128_16": (128, 128, 64, 2, 2, 1, A16),
                "splitk_16": (128, 64, 128, 4, 1, 2, A16)}
ATOM = {A32: (32, 16, 16), A16: (16, 32, 4)}      # atom M = N, atom K, values per lane


def _tab(text):
    return list(mfl.layout_table(text))


def _mode_sizes(text):
    return tuple(L.size(s) for s in P(text)[0]) if isinstance(P(text)[0], tuple) \
        else (P(text)[0],)


def _split_eq(tokens):
    i = tokens.index("=")
    return tokens[:i], tokens[i + 1]


# ------------------------------------------------------------ page strings
def test_tiled_product_prints_page_layouts():
    rows = keyed("algebra.txt", "tiled_product")
    assert len(rows) == 3
    for toks in rows:
        (a, b), want = _split_eq(toks)
        assert mfl.layout_tiled_product(a, b) == want


def test_divides_print_page_layouts():
    for toks in keyed("algebra.txt", "zdiv"):
        (a, t), want = _split_eq(toks)
        assert mfl.layout_zipped_divide(a, t) == want
    for toks in keyed("algebra.txt", "ldiv_modes"):
        (a, t), want = _split_eq(toks)
        assert mfl.layout_logical_divide(a, [t.rstrip(";")]) == want
    c = keyed("algebra.txt", "pc_c")[0][0]
    (ct,) = [t[0] for t in keyed("tiledmma_tiling.txt", "c_tensor")]
    assert mfl.layout_zipped_divide(c, ["16:1", "8:1"]) == ct


def test_partition_c_prints_page_layouts():
    c = keyed("algebra.txt", "pc_c")[0][0]
    thr, val = mfl.layout_partition_c(c, L.SM80_C_TV, (16, 8), (2, 2))
    assert val == keyed("tiledmma_tiling.txt", "partition_C_thread0")[0][0]
    for t, coord in keyed("algebra.txt", "pc_start"):
        m, n = (int(x) for x in coord.strip("()").split(","))
        assert mfl.layout_eval(thr, int(t)) == L.evaluate(P(c), (m, n))
    view = keyed("tiledmma_tiling.txt", "partition_C_view")[0]
    assert mfl.layout_partition_c("(64,32):(32,1)", L.SM80_C_TV, (16, 8), (2, 2))[1] == view[1]


@pytest.mark.parametrize("case", ["A", "Bx1", "Bx2", "Bx4"])
def test_retile_prints_page_layouts(case):
    a = {t[0]: t[1:] for t in keyed("algebra.txt", "retile_case")}[case]
    steps = {t[1]: t[2] for t in keyed("algebra.txt", "retile_step") if t[0] == case}
    assert mfl.layout_retile(a[0], a[1], a[2], int(a[3]), int(a[4])) == steps["result"]
    if "with_shape" in steps:
        ws = mfl.layout_with_shape(mfl.layout_right_inverse(a[1]), a[2])
        assert ws == steps["with_shape"]
        if "frg_mn" in steps:
            mn = mfl.layout_upcast(ws, int(steps["upcast_n"]))
            assert mn == steps["frg_mn"]
            assert mfl.layout_right_inverse(mn) == steps["G"]
    for key in ("product", "frg_v"):
        if key not in steps:
            continue
        V = L.size(P(a[0])[0][0]) if isinstance(P(a[0])[0][0], tuple) else P(a[0])[0][0]
        prod = mfl.layout_logical_product(f"{V}:1", steps["G"])
        if key == "product":
            assert prod == steps["product"]
        else:
            assert mfl.layout_zipped_divide(prod, f"{a[4]}:1") == steps["frg_v"]
    if "t_tensor" in steps:
        each = steps.get("product_each", "(1,1)").strip("()").split(",")
        V = _mode_sizes(a[0])[0]
        tiler = [f"{V}:1"] + [f"{e}:1" for e in each]
        assert mfl.layout_zipped_divide(a[0], tiler) == steps["t_tensor"]


# ------------------------------------------------------ module vs oracle
def _random_tiling(rng):
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
    lay = (tuple(shape[i] for i in order), tuple(stride[i] for i in order))
    return lay, ext


def test_complement_matches_oracle():
    rng = random.Random(11)
    for _ in range(300):
        b, ext = _random_tiling(rng)
        M = ext * rng.choice([1, 2, 3])
        got = mfl.layout_complement(F(b), M)
        assert _tab(got) == G.complement(b, M)[1], (b, M)


def _same_or_rejected(call, sizes, tab):
    """The module's result equals the oracle's function, or the module
    rejected the composition complement o B as inadmissible (-11: a stride of
    B that does not divide the complement's leaf shapes, where the leaf form
    would not be the function)."""
    try:
        got = call()
    except mfl.LayoutError as e:
        assert "code -11" in str(e)
        return False
    assert _tab(got) == tab and _mode_sizes(got) == sizes
    return True


def test_whole_divide_and_product_match_oracle():
    rng = random.Random(12)
    accepted = 0
    for _ in range(300):
        b, ext = _random_tiling(rng)
        n = ext * rng.choice([1, 2, 4])
        d = rng.choice([1, 2])
        a = ((n,), (d,))
        got = mfl.layout_logical_divide(F(a), F(b))
        sizes, tab = G.logical_divide(a, b)
        assert _tab(got) == tab and _mode_sizes(got) == sizes, (a, b)
        c = ((rng.choice([2, 4]),), (rng.choice([1, 2, 3]),))
        sizes, tab = G.logical_product(b, c)
        accepted += _same_or_rejected(lambda: mfl.layout_logical_product(F(b), F(c)),
                                          sizes, tab)
        e = rng.choice([((2, 2), (1, 2)), ((2, 3), (1, 2)), ((2, 1, 2), (1, 0, 2))])
        sizes, tab = G.tiled_product(b, e)
        accepted += _same_or_rejected(lambda: mfl.layout_tiled_product(F(b), F(e)),
                                          sizes, tab)
    assert accepted >= 400       # of 600 draws (fixed seed)


def test_mode_divides_match_oracle():
    """Padded row- or column-major matrices divided by compact or strided
    per-mode tilers."""
    rng = random.Random(13)
    for _ in range(300):
        R, C = rng.choice([4, 6, 8, 12, 16]), rng.choice([4, 8, 10, 16])
        pad = rng.choice([0, 1, 8])
        a = ((R, C), (C + pad, 1)) if rng.random() < 0.5 else ((R, C), (1, R + pad))
        tilers = []
        for n in (R, C):
            t = rng.choice([x for x in (1, 2, 3, 4, 8) if n % x == 0])
            if t > 1 and n % (2 * t) == 0 and rng.random() < 0.3:
                tilers.append(((t,), (2,)))          # strided tiler
            else:
                tilers.append(((t,), (1,)))
        txt = [F(t) for t in tilers]
        got = mfl.layout_logical_divide(F(a), txt)
        sizes, tab = G.logical_divide_modes(a, tilers)
        assert _tab(got) == tab and _mode_sizes(got) == sizes, (a, tilers)
        got = mfl.layout_zipped_divide(F(a), txt)
        sizes, tab = G.zipped_divide(a, tilers)
        assert _tab(got) == tab and _mode_sizes(got) == sizes, (a, tilers)


def test_upcast_matches_oracle_leaf_by_leaf():
    rng = random.Random(14)
    for _ in range(300):
        nm = rng.randint(1, 3)
        shape, stride = [], []
        for _m in range(nm):
            ls = tuple(rng.choice([1, 2, 4, 8, 16]) for _ in range(rng.randint(1, 3)))
            ld = tuple(rng.choice([0, 1, 2, 4, 8, 16, 32, 64, 128]) for _ in ls)
            shape.append(ls if len(ls) > 1 else ls[0])
            stride.append(ld if len(ld) > 1 else ld[0])
        lay = (tuple(shape), tuple(stride)) if nm > 1 else (shape[0], stride[0])
        n = rng.choice([1, 2, 4, 8, 16])
        try:
            want = G.upcast(lay, n)
        except ValueError:
            with pytest.raises(mfl.LayoutError):
                mfl.layout_upcast(F(lay), n)
            continue
        assert P(mfl.layout_upcast(F(lay), n)) == want, (lay, n)


def _mfma_tv(op, operand):
    """The oracle's MFMA map as a layout text (factored from its table)."""
    M, N, K, nv, nacc = L.MFMA_OPS[op]
    if operand == "C":
        tab = [m + M * n for v in range(nacc) for lane in range(64)
               for m, n in [L.mfma_c_coord(op, lane, v)]]
        return F(G.factor_table(tab, (64, nacc)))
    rows = M if operand == "A" else N
    tab = [r + rows * k for v in range(nv) for lane in range(64)
           for r, k in [L.mfma_ab_coord(op, lane, v)]]
    return F(G.factor_table(tab, (64, nv)))


TV_CASES = [(L.SM80_A_TV, (16, 16)), (L.SM80_B_TV, (8, 16)), (L.SM80_C_TV, (16, 8))] + [
    (op, None) for op in L.MFMA_OPS]


@pytest.mark.parametrize("tv,shape", TV_CASES)
def test_with_shape_of_inverse_matches_oracle(tv, shape):
    """right_inverse(TV).with_shape(tile): the representation upcast reads."""
    cases = []
    if shape is None:
        M, N, K, nv, _ = L.MFMA_OPS[tv]
        cases = [(_mfma_tv(tv, "A"), (M, K)), (_mfma_tv(tv, "B"), (N, K)),
                 (_mfma_tv(tv, "C"), (M, N))]
    else:
        cases = [(tv, shape)]
    for text, shp in cases:
        got = mfl.layout_with_shape(mfl.layout_right_inverse(text), str(shp).replace(" ", ""))
        assert P(got) == G.right_inverse_shaped(P(text), shp), text


def _partition_oracle(c, tv_text, atom, nl, warps, tile):
    tl = None if tile is None else tuple(P(t) if t else (atom[i] * warps[i], 1)
                                         for i, t in enumerate(tile))
    out = G.partition_c(P(c), P(tv_text), atom, nl, warps, tile=tl)
    return out


def _check_partition(c, tv_text, atom, nl, warps, tile=None):
    thr, val = mfl.layout_partition_c(c, tv_text, atom, warps,
                                      tile=None if tile is None else
                                      tuple(t or None for t in tile))
    T, V = _tab(thr), _tab(val)
    want = _partition_oracle(c, tv_text, atom, nl, warps, tile)
    assert len(T) == len(want)
    for t in range(len(T)):
        assert [T[t] + v for v in V] == want[t], (c, atom, warps, tile, t)


def test_partition_c_matches_oracle_random():
    rng = random.Random(15)
    atoms = [(L.SM80_C_TV, (16, 8), 32)] + [
        (_mfma_tv(op, "C"), L.MFMA_OPS[op][:2], 64) for op in ("f32_32x32x16_f16",
                                                               "f32_16x16x32_f16")]
    for _ in range(40):
        tv, (am, an), nl = rng.choice(atoms)
        wm, wn = rng.choice([1, 2]), rng.choice([1, 2, 4])
        rm, rn = rng.choice([1, 2]), rng.choice([1, 2])
        Mt, Nt = am * wm * rm, an * wn * rn
        gm, gn = rng.choice([1, 2]), rng.choice([1, 2])
        M, N = Mt * gm, Nt * gn
        pad = rng.choice([0, 4])
        c = F(((M, N), (N + pad, 1))) if rng.random() < 0.5 else F(((M, N), (1, M + pad)))
        tile = None
        if rng.random() < 0.5:
            # a tile of Mt x Nt; wave-contiguous repeats along M where possible
            pm = F(((am, wm, rm), (1, am * rm, am))) if rm > 1 and wm > 1 else F(((Mt,), (1,)))
            tile = (pm, F(((Nt,), (1,))))
        _check_partition(c, tv, (am, an), nl, (wm, wn), tile)


def test_retile_matches_oracle_on_page_and_mfma_cases():
    cases = [tuple(t[1:]) for t in keyed("algebra.txt", "retile_case")]
    for op in ("f32_32x32x16_f16", "f32_16x16x32_f16"):
        M, N, K, nv, _ = L.MFMA_OPS[op]
        for R, KS in [(1, 1), (2, 2), (4, 2)]:
            frag = F(((nv, R, KS), (1, nv, nv * R)))
            for nval in (8, 4, 2):
                cases.append((frag, _mfma_tv(op, "A"), f"({M},{K})", "64", str(nval)))
    for frag, tv, shp, nthr, nval in cases:
        got = mfl.layout_retile(frag, tv, shp, int(nthr), int(nval))
        r = G.retile(P(frag), P(tv), tuple(int(x) for x in shp.strip("()").split(",")),
                     int(nthr), int(nval))
        n_c = len(r["frg_layout_v"][1])
        want = [r["slots"][(i % n_c, i // n_c)] for i in range(len(r["slots"]))]
        assert _tab(got) == want, (frag, tv, nval)


def test_error_codes():
    with pytest.raises(mfl.LayoutError):       # rank-3 C
        mfl.layout_partition_c("(4,4,4):(1,4,16)", L.SM80_C_TV, (16, 8), (1, 1))
    with pytest.raises(mfl.LayoutError):       # atom larger than C
        mfl.layout_partition_c("(8,8):(8,1)", L.SM80_C_TV, (16, 8), (1, 1))
    with pytest.raises(mfl.LayoutError):       # fragment rank does not match the tile
        mfl.layout_retile("(4,4):(1,4)", L.SM80_B_TV, "(8,16)", 32, 2)
    with pytest.raises(mfl.LayoutError):       # TV does not cover the tile
        mfl.layout_retile("((2,2),1,1):((1,2),0,0)", "((4,8),(2,2)):((16,1),(8,128))",
                          "(8,16)", 32, 2)
    with pytest.raises(mfl.LayoutError):       # leaves interacting through a carry
        mfl.layout_compose("(4,3):(1,10)", "3:2")


# ------------------------------------------------- gfx950 MFMA analogues
@pytest.mark.parametrize("algo", sorted(KERNEL_TILES))
def test_kernel_accumulators_are_partition_c(algo):
    """The kernels' accumulator coordinates are partition_C of the block tile
    for their atom (AM x AM, 32x32x16 or 16x16x32) with tile permutations:
    M (AM, WM, RM):(1, AM RM, AM) (wave-contiguous repeats), N (AM, WN, V,
    RN/V):(V, AM RN, 1, AM V) (the same, with a lane's repeats on runs of V =
    min(RN, 4) adjacent columns for vector stores).  partition_C selects
    (lane, wm, wn) only, so every K-group of a split-K tile holds the same
    view."""
    BM, BN, BK, WM, WN, WK, op = KERNEL_TILES[algo]
    AM, _, NV = ATOM[op]
    RM, RN = BM // WM // AM, BN // WN // AM
    V = min(RN, 4)
    if RN // V > 1:
        tn = F(((AM, WN, V, RN // V), (V, AM * RN, 1, AM * V)))
    else:
        tn = F(((AM, WN, RN), (RN, AM * RN, 1)))
    tile = (F(((AM, WM, RM), (1, AM * RM, AM))), tn)
    c = F(((BM, BN), (1, BM)))
    thr, val = mfl.layout_partition_c(c, _mfma_tv(op, "C"), (AM, AM), (WM, WN), tile=tile)
    T, Vt = np.array(_tab(thr)), np.array(_tab(val))
    fc = mfl.fragment_coords(algo, "C")                 # slot = (i RN + j) NV + v
    want = fc[..., 0] + BM * fc[..., 1]
    i, j, v = np.meshgrid(np.arange(RM), np.arange(RN), np.arange(NV), indexing="ij")
    order = (v + NV * (i + RM * j)).reshape(-1)        # value layout index of each slot
    thr = np.arange(want.shape[0]) % (64 * WM * WN)      # the thread's (lane, wm, wn)
    assert want.shape[0] == 64 * WM * WN * WK
    assert np.array_equal(T[thr][:, None] + Vt[None, order], want)
    # the oracle's chain gives the same
    _check_partition(c, _mfma_tv(op, "C"), (AM, AM), 64, (WM, WN), tile)


@pytest.mark.parametrize("op", ["f32_32x32x16_f16", "f32_16x16x32_f16"])
def test_ds_read_b128_retile_is_identity(op):
    """One 16-byte LDS read per lane delivers a whole 8-value operand, so the
    copy view is the MMA view: ((8,1), R, KSUB) over the same slots."""
    M, N, K, nv, _ = L.MFMA_OPS[op]
    for R, KS in [(4, 2), (4, 4), (2, 1)]:
        frag = F(((nv, R, KS), (1, nv, nv * R)))
        for operand, rows in (("A", M), ("B", N)):
            got = mfl.layout_retile(frag, _mfma_tv(op, operand), f"({rows},{K})", 64, 8)
            assert got == f"((8,1),{R},{KS}):((1,0),{8 if R > 1 else 0},{8 * R if KS > 1 else 0})"
            assert _tab(got) == _tab(frag)


def test_transposed_reads_retile_in_pairs_of_four():
    """The two ds_read_b64_tr_b16 reads that fill one 32x32x16 A operand
    write 4 values each: retile groups values 0..3 and 4..7, and the second
    group's positions are the first's 4 k further (the kernel's second read
    address)."""
    op = "f32_32x32x16_f16"
    tv = _mfma_tv(op, "A")
    got = mfl.layout_retile("(8,4,2):(1,8,32)", tv, "(32,16)", 64, 4)
    assert got == "((4,2),4,2):((1,4),8,32)"
    tvl = P(tv)
    for lane in range(64):
        for e in range(4):
            q0, q1 = L.evaluate(tvl, (lane, e)), L.evaluate(tvl, (lane, 4 + e))
            assert (q1 % 32, q1 // 32) == (q0 % 32, q0 // 32 + 4)


def test_k_gather_with_the_32x32x8_atom():
    """The page's K gather, on gfx950: the 32x32x8 atom holds 4 values per
    lane, a 16-byte read writes 8.  Over a 32x16 reference tile (two K
    fragments) retile gathers both K fragments of one repeat (slots 0..7);
    a plain zipped_divide by 8 would take slots 0..3 and 8..11, two M
    repeats."""
    op = "f32_32x32x8_f16"
    one = _mfma_tv(op, "A")                     # ((32,2),4):((1,128),32)
    assert P(one) == P("((32,2),4):((1,128),32)")
    # the atom repeated once along K: value leaf 2:(32*8)
    tiled = "((32,2),(4,2)):((1,128),(32,256))"
    frag = "(4,4,2):(1,8,4)"                     # r[v + 8 i + 4 k]
    got = mfl.layout_retile(frag, tiled, "(32,16)", 64, 8)
    assert got == "((8,1),4,1):((1,0),8,0)"
    assert _tab(got)[:8] == list(range(8))
    assert _tab(mfl.layout_zipped_divide(frag, "8:1"))[:8] == [0, 1, 2, 3, 8, 9, 10, 11]
    r = G.retile(P(frag), P(tiled), (32, 16), 64, 8)
    assert [r["slots"][(c, 0)] for c in range(8)] == list(range(8))
    # every (lane, copy value) of the 64 x 8 destination lands on a distinct
    # position of the 32x16 tile: 512 destination matches
    t = P(tiled)
    pos = {L.evaluate(t, (lane, c)) for lane in range(64) for c in range(8)}
    assert pos == set(range(512))


def _code(fn, *args):
    try:
        fn(*args)
    except mfl.LayoutError as e:
        return int(str(e).rsplit("code", 1)[1])
    return 0


def test_out_of_range_inputs_are_refused():
    """Inputs the algebra cannot represent come back as error codes, never as
    wrapped int64 values or a division by zero: a negative stride on the
    right of a composition (-14), sizes and offsets beyond int64 at parsing
    (-10), and intermediate values beyond int64 inside an operation (-10)."""
    big = 1 << 40
    assert _code(mfl.layout_compose, "(4,8):(1,4)", "4:-1") == -14
    assert _code(mfl.layout_compose, "(4,8):(1,4)", "(2,2):(1,-4)") == -14
    assert _code(mfl.layout_size, f"({big},{big}):(1,0)") == -10
    assert _code(mfl.layout_eval, f"({big},{1 << 24}):({big},1)", 0) == -10
    assert _code(mfl.layout_logical_product, f"({1 << 20},{1 << 20}):(1,{1 << 20})",
                 f"{1 << 20}:{big}") == -10
    assert _code(mfl.layout_tiled_product, f"({1 << 20},{1 << 20}):(1,{1 << 20})",
                 f"({1 << 20},2):({big},1)") == -10
    # the same operations on representable inputs still succeed
    assert mfl.layout_compose("(4,8):(1,4)", "4:2") == "4:2"
    assert mfl.layout_size(f"({1 << 20},{1 << 20}):(1,0)") == 1 << 40

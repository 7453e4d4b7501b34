"""The HIP-side layout module (C++ behind include/mfl_layout.h) against the
independent oracle evaluator, on full domains.  No GPU needed."""
import itertools
import random

import numpy as np
import pytest

import mma_fragment_layouts_tn_amd as mfl
from oracle import layout as L
from helpers import keyed

PAGE_LAYOUTS = [
    L.SM80_C_TV, L.SM80_A_TV, L.SM80_B_TV,
    "(2,2,1):(1,2,4)", "(32,2,2,1):(1,32,64,0)", "(32,2,2,1):(1,64,32,0)",
    "(32,1,1,2):(1,0,0,32)", "((16,8),(2,2)):((16,1),(256,8))",
    "((2,2),1,1):((1,128),0,0)", "((2,2),2,2):((1,256),1024,16)",
    "((2,2,2),2,2):((1,2,4),8,16)", "((2,2),2,2):((1,2),4,8)", "(8,4):(4,1)",
    "(8,(2,4,2)):(4,(32,1,64))", "(8,(2,4,4)):(4,(32,1,64))",
    "((2,2,2),1,1):((1,2,4),0,0)", "((2,4),1,1):((1,2),0,0)", "(2,4):(1,2)",
    "((4,1),1,1):((1,0),0,0)", "(4,4,2):(1,8,4)",
    "(32,8):(8,1)", "(32,(2,4)):(2,(1,64))", "(16,16):(16,1)",
    "(128,16,4):(64,1,16)", "((2,2,2),4,1,4):((1,512,8),2048,0,16)",
    "((2,2),(2,4),1,4):((1,8),(1024,2048),0,16)", "((2,2),4,8):((1,2048),8192,16)",
    "_8:_1", "(_2,_4):(_1,_2)",
]


@pytest.mark.parametrize("text", PAGE_LAYOUTS)
def test_eval_size_cosize_match_oracle(text):
    lay = L.parse(text)
    assert mfl.layout_size(text) == L.size(lay[0])
    assert list(mfl.layout_table(text)) == L.table(lay)
    assert mfl.layout_cosize(text) == L.cosize(lay)
    assert mfl.layout_eval(text, L.size(lay[0]) - 1) == L.table(lay)[-1]


@pytest.mark.parametrize("text", PAGE_LAYOUTS)
def test_coalesce_is_same_function(text):
    c = mfl.layout_coalesce(text)
    assert L.table(L.parse(c)) == L.table(L.parse(text))


def test_partition_c_composition_from_pages():
    # atom block of a row-major 32x16 C composed with the C TV layout gives
    # lane 0 offsets 0, 1, 128, 129 (TiledMMA page, partition_C section)
    out = mfl.layout_compose("(16,8):(16,1)", L.SM80_C_TV)
    tab = L.table(L.parse(out))
    assert [tab[32 * v] for v in range(4)] == [0, 1, 128, 129]
    assert tab == L.compose_table(L.parse("(16,8):(16,1)"), L.parse(L.SM80_C_TV))


def test_route_through_module():
    # route page: right_inverse(S) o D at (0,5) -> flat 48 == source (16,1);
    # F o right_inverse(R) o D at (0,5) -> q = 144 == A(0,9)
    S, D = "(32,8):(8,1)", "(32,(2,4)):(2,(1,64))"
    s_inv = mfl.layout_right_inverse(S)
    route = mfl.layout_compose(s_inv, D)
    flat = L.evaluate(L.parse(route), (0, 5))
    assert flat == 48 and L.decode(flat, (32, 8)) == (16, 1)
    r_inv = mfl.layout_right_inverse(D)
    f_r = mfl.layout_compose(L.SM80_A_TV, r_inv)
    f_r_d = mfl.layout_compose(f_r, D)
    assert L.evaluate(L.parse(f_r_d), (0, 5)) == 144
    # and the same map equals the MMA layout F everywhere (R = D)
    assert L.table(L.parse(f_r_d)) == L.table(L.parse(L.SM80_A_TV))


def test_right_inverse_of_page_tv_layouts():
    for text in (L.SM80_A_TV, L.SM80_B_TV, L.SM80_C_TV, "(32,(2,4)):(2,(1,64))"):
        r = mfl.layout_right_inverse(text)
        assert list(L.table(L.parse(r))) == L.right_inverse_table(L.table(L.parse(text)))
    r = mfl.layout_right_inverse(L.SM80_B_TV)
    assert L.table(L.parse(r)) == L.table(L.parse("(8,(2,4,2)):(4,(32,1,64))"))


def _rand_compact(rng, nleaf):
    shapes = [rng.choice([1, 2, 3, 4, 8]) for _ in range(nleaf)]
    order = list(range(nleaf))
    rng.shuffle(order)
    strides = [0] * nleaf
    acc = 1
    for i in order:
        strides[i] = acc
        acc *= shapes[i]
    return shapes, strides


def _fmt(shapes, strides):
    if len(shapes) == 1:
        return f"{shapes[0]}:{strides[0]}"
    return "(" + ",".join(map(str, shapes)) + "):(" + ",".join(map(str, strides)) + ")"


def test_right_inverse_random_permutation_layouts():
    rng = random.Random(5)
    for _ in range(300):
        shapes, strides = _rand_compact(rng, rng.randint(1, 5))
        if rng.random() < 0.3:          # a broadcast mode
            shapes.append(rng.choice([2, 3]))
            strides.append(0)
        text = _fmt(shapes, strides)
        r = mfl.layout_right_inverse(text)
        want = L.right_inverse_table(L.table(L.parse(text)))
        assert L.table(L.parse(r)) == want, (text, r)


def test_compose_random_against_tables():
    rng = random.Random(7)
    checked = 0
    for _ in range(600):
        a_sh, a_st = _rand_compact(rng, rng.randint(1, 4))
        if rng.random() < 0.3:
            a_st = [d * rng.choice([1, 2, 3]) for d in a_st]   # gaps
        A = _fmt(a_sh, a_st)
        # B: arbitrary small shapes and strides; the module must either
        # return exactly A o B or refuse
        n = rng.randint(1, 3)
        b_sh = [rng.choice([1, 2, 4]) for _ in range(n)]
        b_st = [rng.choice([0, 1, 2, 4, 8, 16]) for _ in range(n)]
        B = _fmt(b_sh, b_st)
        try:
            out = mfl.layout_compose(A, B)
        except mfl.LayoutError:
            continue
        want = L.compose_table(L.parse(A), L.parse(B))
        assert L.table(L.parse(out)) == want, (A, B, out)
        checked += 1
    assert checked > 250


def test_compose_rejects_non_divisible():
    with pytest.raises(mfl.LayoutError):
        mfl.layout_compose("(3,4):(1,5)", "2:2")


def test_bad_text_rejected():
    for bad in ("(2,2):(1)", "((2,2):(1,2)", "2,2:1,2", "(2,a):(1,2)", ""):
        with pytest.raises(mfl.LayoutError):
            mfl.layout_size(bad)


# --------------------------------------------------- gfx950 atom TV layouts
@pytest.mark.parametrize("op", sorted(L.MFMA_OPS))
def test_mfma_tv_layouts_equal_oracle_closed_forms(op):
    M, N, K, nv, nacc = L.MFMA_OPS[op]
    for operand in ("A", "B"):
        lay = L.parse(mfl.mfma_tv(op, operand))
        for lane, v in itertools.product(range(64), range(nv)):
            q = L.evaluate(lay, (lane, v))
            assert (q % M, q // M) == L.mfma_ab_coord(op, lane, v)
    lay = L.parse(mfl.mfma_tv(op, "C"))
    for lane, v in itertools.product(range(64), range(nacc)):
        q = L.evaluate(lay, (lane, v))
        assert (q % M, q // M) == L.mfma_c_coord(op, lane, v)


# --------------------------------------------- kernel fragment addressing
# BM, BN, BK, waves along M, N and K (K-groups split each stage's sub-steps),
# and the matrix instruction
A32, A16 = "f32_32x32x16_f16", "f32_16x16x32_f16"
KERNEL_TILES = {"direct": (128, 128, 32, 2, 2, 1, A32), "lds128": (128, 128, 32, 2, 2, 1, A32),
                "lds256": (256, 256, 64, 2, 4, 1, A32), "lds256w4": (256, 256, 64, 2, 2, 1, A32),
                "lds128w1": (128, 128, 32, 1, 1, 1, A32), "splitk": (128, 64, 128, 1, 1, 4, A32),
                "lds256w4_16": (256, 256, 64, 2, 2, 1, A16),
                "lds256_16": (256, 256, 64, 2, 4, 1, A16),
                "lds128_16": (128, 128, 64, 2, 2, 1, A16),
                "splitk_16": (128, 64, 128, 4, 1, 2, A16)}
LDS_KERNELS = ["lds128", "lds256", "lds256w4", "lds128w1", "splitk", "lds256w4_16", "lds256_16",
               "lds128_16", "splitk_16"]
ATOM = {A32: (32, 16, 16), A16: (16, 32, 4)}      # atom M = N, atom K, values per lane


@pytest.mark.parametrize("algo", sorted(KERNEL_TILES))
def test_fragment_coords_follow_the_atom_layout(algo):
    BM, BN, BK, WM, WN, WK, op = KERNEL_TILES[algo]
    AM, AK, NV = ATOM[op]
    fa = mfl.fragment_coords(algo, "A")
    fb = mfl.fragment_coords(algo, "B")
    fc = mfl.fragment_coords(algo, "C")
    T = 64 * WM * WN * WK
    assert fa.shape[0] == fb.shape[0] == fc.shape[0] == T
    RM, RN, KW = BM // WM // AM, BN // WN // AM, BK // AK // WK
    V = min(RN, 4)
    for t in range(T):
        w, lane = divmod(t, 64)
        wm, wn, wk = w % WM, (w // WM) % WN, w // (WM * WN)
        s = 0
        for kk in range(KW):
            for i in range(RM):
                for v in range(8):
                    r, k = L.mfma_ab_coord(op, lane, v)
                    assert tuple(fa[t, s]) == (wm * (BM // WM) + AM * i + r,
                                               AK * (wk * KW + kk) + k)
                    s += 1
        s = 0
        for kk in range(KW):
            for j in range(RN):
                for v in range(8):
                    r, k = L.mfma_ab_coord(op, lane, v)
                    assert tuple(fb[t, s]) == (wn * (BN // WN) + AM * j + r,
                                               AK * (wk * KW + kk) + k)
                    s += 1
        s = 0
        for i in range(RM):
            for j in range(RN):
                for v in range(NV):
                    # the N permutation: repeat j of atom column n is column
                    # AM V (j // V) + V n + j % V (V = RN when RN <= 4)
                    m, n = L.mfma_c_coord(op, lane, v)
                    assert tuple(fc[t, s]) == (wm * (BM // WM) + AM * i + m,
                                               wn * (BN // WN) + AM * V * (j // V) + V * n
                                               + j % V)
                    s += 1


def _perm_n(n, WTN, RN, AN):
    """Logical column (wave, repeat, atom column) -> physical column."""
    V = min(RN, 4)
    w, r = divmod(n, WTN)
    j, c = divmod(r, AN)
    return w * WTN + AN * V * (j // V) + V * c + j % V


@pytest.mark.parametrize("algo", sorted(KERNEL_TILES))
def test_output_columns_are_the_permuted_b_rows(algo):
    """Each lane's accumulator column for repeat j is the B row it multiplies
    (the lane's row of the fragment for repeat j), through the N permutation
    that the B fetch applies: LDS row r holds global row perm(r).  A
    transposed or unpermuted pairing fails this for every lane but the
    first."""
    BM, BN, BK, WM, WN, WK, op = KERNEL_TILES[algo]
    AM, AK, NV = ATOM[op]
    RM, RN, KW = BM // WM // AM, BN // WN // AM, BK // AK // WK
    fb = mfl.fragment_coords(algo, "B")            # (T, KW*RN*8, 2): LDS rows
    fc = mfl.fragment_coords(algo, "C")            # (T, RM*RN*NV, 2): physical
    for t in range(fb.shape[0]):
        for j in range(RN):
            brow = fb[t, (0 * RN + j) * 8, 0]      # kk = 0, repeat j, value 0
            for i in range(RM):
                for v in range(NV):
                    col = fc[t, (i * RN + j) * NV + v, 1]
                    assert col == _perm_n(brow, BN // WN, RN, AM), (algo, t, j)
    assert sorted({_perm_n(n, BN // WN, RN, AM) for n in range(BN)}) == list(range(BN))


@pytest.mark.parametrize("algo", sorted(KERNEL_TILES))
def test_fragment_multiplicities(algo):
    """A held WAVES_N times, B WAVES_M times, C once per K-group (the pages'
    2/2/1, and C twice for two K-direction warp groups)."""
    BM, BN, BK, WM, WN, WK, _ = KERNEL_TILES[algo]
    for operand, rows, mult in (("A", BM, WN), ("B", BN, WM)):
        f = mfl.fragment_coords(algo, operand).reshape(-1, 2)
        idx = f[:, 0] * BK + f[:, 1]
        counts = np.bincount(idx, minlength=rows * BK)
        assert counts.shape[0] == rows * BK and (counts == mult).all()
    f = mfl.fragment_coords(algo, "C").reshape(-1, 2)
    counts = np.bincount(f[:, 0] * BN + f[:, 1], minlength=BM * BN)
    assert (counts == WK).all()


# ------------------------------------------------ LDS tile layout, tile order
@pytest.mark.parametrize("algo", LDS_KERNELS)
@pytest.mark.parametrize("operand", ["A", "B"])
def test_lds_tile_layout_bijective_and_conflict_free(algo, operand):
    """The swizzled tile is a permutation of rows*BK halves that keeps each
    8-half chunk contiguous, and the 16 rows read by 16 consecutive lanes at a
    fixed K chunk land in 16 different 16-byte bank groups (64 banks of 4 B)."""
    off = mfl.lds_tile_offsets(algo, operand)
    rows, bk = off.shape
    assert sorted(off.reshape(-1).tolist()) == list(range(rows * bk))
    assert (off[:, 1:8] - off[:, 0:1] == np.arange(1, 8)).all()
    for k0 in range(0, bk, 8):
        for r0 in range(0, rows, 16):
            groups = {(int(off[r, k0]) * 2 // 16) % 16 for r in range(r0, r0 + 16)}
            assert len(groups) == 16, (algo, operand, k0, r0)


@pytest.mark.parametrize("tiles", [(1, 1), (16, 16), (32, 24), (64, 48), (3, 7), (33, 5)])
@pytest.mark.parametrize("group_m", [4, 8])
def test_tile_order_is_a_bijection(tiles, group_m):
    tm, tn = mfl.tile_order(tiles[0], tiles[1], group_m)
    pairs = set(zip(tm.tolist(), tn.tolist()))
    assert len(pairs) == tiles[0] * tiles[1]
    assert tm.min() >= 0 and tm.max() < tiles[0] and tn.min() >= 0 and tn.max() < tiles[1]


def test_tile_order_keeps_xcd_blocks_compact():
    """With 256 tiles of 16x16 and 8 XCDs (workgroup id % 8), each XCD's 32
    tiles span 4 A-row blocks and 8 B-column blocks (the minimum, 12)."""
    tm, tn = mfl.tile_order(16, 16, 4)
    for x in range(8):
        ids = np.arange(x, 256, 8)
        assert len(set(tm[ids].tolist())) + len(set(tn[ids].tolist())) == 12


# ----------------------------------------- M-contiguous A: transposing reads
@pytest.mark.parametrize("algo", LDS_KERNELS)
def test_mmajor_tile_and_transposed_reads_conflict_free(algo):
    """The M-contiguous A tile is a permutation keeping 8-half chunks whole,
    and every transposing read (64 lanes x 8 bytes, served 32 lanes per pass)
    touches each of the 64 four-byte banks exactly once per pass."""
    lay = mfl.lds_tile_offsets(algo, "A_mmajor")                   # [k, m]
    bk, bm = lay.shape
    assert sorted(lay.reshape(-1).tolist()) == list(range(bk * bm))
    chunks = lay.reshape(bk, bm // 8, 8)
    assert (chunks - chunks[:, :, :1] == np.arange(8)).all()
    src = mfl.fragment_coords(algo, "A_tr")                         # (threads, KSUB*RM, 2)
    for t0 in range(0, src.shape[0], 64):
        for slot in range(src.shape[1]):
            for h in (0, 1):
                for half in (0, 32):
                    banks = []
                    for l in range(half, half + 32):
                        m, k = src[t0 + l, slot]
                        byte = 2 * int(lay[k + 4 * h, m])
                        assert byte % 8 == 0
                        banks += [(byte // 4) % 64, (byte // 4 + 1) % 64]
                    assert sorted(banks) == list(range(64)), (algo, t0, slot, h, half)


@pytest.mark.parametrize("algo", LDS_KERNELS)
def test_transposed_reads_give_the_operand_fragments(algo):
    """Applying the transposing read's lane regrouping (pinned on the GPU by
    test_gpu_probe) to the kernel's source coordinates yields exactly the A
    fragment coordinates of the K-contiguous path, value by value."""
    src = mfl.fragment_coords(algo, "A_tr")                         # (T, KSUB*RM, 2)
    frag = mfl.fragment_coords(algo, "A")                           # (T, KSUB*RM*8, 2)
    T, slots, _ = src.shape
    for t in range(T):
        w, l = divmod(t, 64)
        b, i = divmod(l, 16)
        for slot in range(slots):
            for v in range(8):
                h, e = divmod(v, 4)
                m, k = src[64 * w + 16 * b + 4 * e + i // 4, slot]
                assert (m + i % 4, k + 4 * h) == tuple(frag[t, slot * 8 + v]), (algo, t, slot, v)

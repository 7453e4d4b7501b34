"""Pins for the oracle's layout evaluator and thread/value models.

Every expected value here is printed on one of the pages (fixtures in
tests/golden/, each line cited there) or follows from a bijection/count the
pages state.  A wrong decode order, a swapped stride, a dropped mode or a
transposed coordinate in oracle/layout.py fails at least one of these.
"""
import itertools

import pytest

from oracle import layout as L
from helpers import keyed, lines, pairs, table

pytestmark = pytest.mark.filterwarnings("ignore")


def _golden_layouts(name):
    return {t[0]: L.parse(t[1]) for t in keyed(name, "layout")}


# ---------------------------------------------------------------- atom maps
def test_eval_warp_group_layout():
    for tok in keyed("tiledmma_atom.txt", "eval"):
        lay = L.parse(tok[0])
        coord = tuple(int(x) for x in tok[1].strip("()").split(","))
        assert L.evaluate(lay, coord) == int(tok[2])


def test_sm80_atom_layouts_match_printed_lane_tables():
    lays = _golden_layouts("tiledmma_atom.txt")
    enc = {"C": lambda q: (q % 16, q // 16),   # q = m + 16 n
           "A": lambda q: (q % 16, q // 16),   # q = m + 16 k
           "B": lambda q: (q % 8, q // 8)}     # q = n + 8 k
    for op, rows in (("C", table("tiledmma_atom.txt", "C")),
                     ("A", table("tiledmma_atom.txt", "A")),
                     ("B", table("tiledmma_atom.txt", "B"))):
        assert rows, op
        for lane, want in rows.items():
            got = [enc[op](L.evaluate(lays[op], (int(lane), v))) for v in range(len(want))]
            assert got == want, (op, lane)


def test_sm80_layouts_equal_page_closed_forms_everywhere():
    lays = _golden_layouts("tiledmma_atom.txt")
    for lane in range(32):
        for v in range(4):
            q = L.evaluate(lays["C"], (lane, v))
            assert (q % 16, q // 16) == L.sm80_c_coord(lane, v)
            q = L.evaluate(lays["B"], (lane, v))
            assert (q % 8, q // 8) == L.sm80_b_coord(lane, v)
        for v in range(8):
            q = L.evaluate(lays["A"], (lane, v))
            assert (q % 16, q // 16) == L.sm80_a_coord(lane, v)


@pytest.mark.parametrize("op,n", [("C", 128), ("A", 256), ("B", 128)])
def test_sm80_tv_layouts_are_bijections(op, n):
    lay = _golden_layouts("tiledmma_atom.txt")[op]
    assert sorted(L.table(lay)) == list(range(n))
    assert L.size(lay[0]) == n and L.cosize(lay) == n


def test_decode_is_first_mode_fastest():
    shape = ((4, 8), (2, 2))
    assert L.decode(1, shape) == ((1, 0), (0, 0))
    assert L.decode(4, shape) == ((0, 1), (0, 0))
    assert L.decode(32, shape) == ((0, 0), (1, 0))
    assert L.decode(127, shape) == ((3, 7), (1, 1))


def test_size_one_and_stride_zero_modes():
    lay = L.parse("(32,1,1,2):(1,0,0,32)")
    assert L.evaluate(lay, (5, 0, 0, 1)) == 37
    bcast = L.parse("(4,3):(1,0)")
    assert L.table(bcast) == [0, 1, 2, 3] * 3
    assert L.cosize(bcast) == 4


def test_size_vs_cosize_under_padding():
    # 128 x 32 tile, K contiguous, rows padded by 8 halves (stride 40)
    lay = L.parse("(128,32):(40,1)")
    assert L.size(lay[0]) == 4096
    assert L.cosize(lay) == 127 * 40 + 31 + 1


# ------------------------------------------------------------ TiledMMA model
def test_thr_layouts_printed():
    cfgs = L.page_trace_configs()
    for tok in keyed("tiledmma_tiling.txt", "thr_layout"):
        shape, stride = L.parse(tok[1])
        got_shape, got_stride = cfgs[tok[0]].thr_layout_vmnk()
        assert tuple(got_shape) == shape
        # size-1 modes: stride is irrelevant, compare where size > 1
        for s, a, b in zip(shape, got_stride, stride):
            if s > 1:
                assert a == b
    for tok in keyed("tiledmma_tiling.txt", "tile"):
        assert cfgs[tok[0]].tile == tuple(int(x) for x in tok[1].strip("()").split(","))


def test_four_warp_and_permuted_c_tables():
    cfgs = L.page_trace_configs()
    rows = table("tiledmma_tiling.txt", "C")
    assert len(rows) >= 9
    for key, want in rows.items():
        cfg_name, t = key.split()
        got = cfgs[cfg_name].coords_C(int(t))
        assert got == want, key


def test_swapped_stride_moves_warps():
    cfgs = L.page_trace_configs()
    sw = cfgs["swapped"]
    # warp 1 (t = 32) sits to the right (n offset 8), warp 2 below (m offset 16)
    assert sw.coords_C(32)[0] == (0, 8)
    assert sw.coords_C(64)[0] == (16, 0)
    assert sw.flat_coord(32) == (0, 0, 1, 0)


def test_partition_c_layouts():
    c_tensor = L.parse(dict((t[0], t[1]) for t in [s.split(" ", 1) for s in lines("tiledmma_tiling.txt")])["c_tensor"])
    # ((atom m, atom n), (rest m, rest n)) -> row-major offset of a 32x16 C
    for (am, an, rm, rn) in itertools.product(range(16), range(8), range(2), range(2)):
        assert L.evaluate(c_tensor, ((am, an), (rm, rn))) == (am + 16 * rm) * 16 + an + 8 * rn
    # compose the atom block with the C TV layout: lane 0 values 0..3
    atom_block = L.parse("(16,8):(16,1)")
    tv = L.compose_table(atom_block, L.parse(L.SM80_C_TV))
    want = [int(x) for x in keyed("tiledmma_tiling.txt", "partition_C_thread0_offsets")[0]]
    assert [tv[32 * v] for v in range(4)] == want
    thr0 = L.parse(keyed("tiledmma_tiling.txt", "partition_C_thread0")[0][0])
    assert L.table(thr0) == want


def test_multiplicities_four_warp():
    cfg = L.page_trace_configs()["four_warp"]
    for tok in keyed("tiledmma_tiling.txt", "multiplicity"):
        _, op, holdings, distinct = tok
        coords = []
        for t in range(cfg.nthreads):
            coords += getattr(cfg, f"coords_{op}")(t)
        assert len(coords) == int(holdings)
        assert len(set(coords)) == int(distinct)
    for op, mult in (("A", 2), ("B", 2), ("C", 1)):
        counts = {}
        for t in range(cfg.nthreads):
            for c in getattr(cfg, f"coords_{op}")(t):
                counts[c] = counts.get(c, 0) + 1
        assert set(counts.values()) == {mult}


def test_larger_input_views_and_fragments():
    cfg = L.page_trace_configs()["larger_input"]
    view = L.parse(keyed("tiledmma_tiling.txt", "partition_C_view")[0][1])
    got = [divmod(L.evaluate(view, i), 32) for i in range(16)]   # C is 64x32 row-major
    assert got == cfg.coords_C(0)
    for tok in keyed("tiledmma_tiling.txt", "fragment"):
        frag = L.parse(tok[2])
        n = L.size(frag[0])
        assert L.table(frag) == list(range(n))      # compact, colex order
    # every element of the 64x32 output covered once, A/B twice
    for op, mult, n in (("C", 1, 64 * 32), ("A", 2, 64 * 32), ("B", 2, 32 * 32)):
        counts = {}
        for t in range(cfg.nthreads):
            for c in getattr(cfg, f"coords_{op}")(t):
                counts[c] = counts.get(c, 0) + 1
        assert len(counts) == n and set(counts.values()) == {mult}


def test_perm_m_values():
    tok = keyed("tiledmma_tiling.txt", "perm")[0]
    lay = L.parse(tok[0])
    for kv in tok[1:]:
        i, p = (int(x) for x in kv.split(":"))
        assert L.perm_m(i) == p
        assert L.evaluate(lay, i) == p
    assert sorted(L.perm_m(i) for i in range(32)) == list(range(32))


def test_split_k_covers_c_twice():
    cfg = L.page_trace_configs()["split_k"]
    ks0 = {k for t in range(32) for (_, k) in cfg.coords_A(t)}
    ks1 = {k for t in range(32, 64) for (_, k) in cfg.coords_A(t)}
    assert ks0 == set(range(16)) and ks1 == set(range(16, 32))
    c = [x for t in range(cfg.nthreads) for x in cfg.coords_C(t)]
    assert len(set(c)) == 128 and len(c) == 256


def test_trace_counts():
    cfgs = L.page_trace_configs()
    per = {}
    for name, cfg in cfgs.items():
        per[name] = sum(len(cfg.coords_A(t)) + len(cfg.coords_B(t)) + len(cfg.coords_C(t))
                        for t in range(cfg.nthreads))
    for tok in keyed("tiledmma_tiling.txt", "trace_count"):
        assert per[tok[0]] == int(tok[1])
    assert sum(per.values()) == int(keyed("tiledmma_tiling.txt", "trace_total")[0][0])


# -------------------------------------------------------------------- retile
def test_right_inverse_of_tv_layouts():
    a_tv = L.tv_table(L.parse(L.SM80_A_TV), 32)
    b_tv = L.tv_table(L.parse(L.SM80_B_TV), 32)
    ra, rb = L.right_inverse_table(a_tv), L.right_inverse_table(b_tv)
    assert len(ra) == 256 and len(rb) == 128
    for tok in keyed("retile.txt", "rinv"):
        op, (x, y), want = tok[0], pairs(tok[1])[0], int(tok[2])
        q = x + 16 * y if op == "A" else x + 8 * y
        assert (ra if op == "A" else rb)[q] == want
    printed = L.parse(keyed("retile.txt", "rinv_with_shape")[0][1])
    assert L.table(printed) == rb


def test_right_inverse_k32_gather_reference():
    # one-warp Tile<16,8,32>: B values 0..3 from the first K=16 atom, 4..7 from the second
    tv = []
    for v in range(8):
        for lane in range(32):
            n, k = L.sm80_b_coord(lane, v % 4)
            tv.append(n + 8 * (k + 16 * (v // 4)))
    printed = L.parse(keyed("retile.txt", "rinv_with_shape_k32")[0][1])
    assert L.table(printed) == L.right_inverse_table(tv)


def test_gather_slots():
    frag = L.parse(keyed("retile.txt", "gather_tCrB")[0][0])
    retile = [L.evaluate(frag, L.decode(a, (4, 1, 2))) for a in range(8)]
    direct = [L.evaluate(frag, L.decode(a, (4, 4, 2))) for a in range(8)]
    assert retile == [int(x) for x in keyed("retile.txt", "gather_slots_retile")[0]]
    assert direct == [int(x) for x in keyed("retile.txt", "gather_slots_direct")[0]]


def test_printed_register_layouts():
    got = {t[0]: L.parse(t[1]) for t in keyed("retile.txt", "print")}
    for name in ("tCrA", "tXrA", "direct_zip", "direct_mode"):
        assert L.table(got[name]) == list(range(8)), name
    for name in ("tCrB", "tXrB", "tXrB_x2"):
        assert L.table(got[name]) == list(range(4)), name
    # (a,b) in the copy grouping addresses slot a + 2b of the MMA fragment
    for a, b in itertools.product(range(2), range(4)):
        assert L.evaluate(got["tXrA"], ((a, b), 0, 0)) == L.evaluate(got["tCrA"], (a + 2 * b, 0, 0))


def test_ldmatrix_x1_route_and_counts():
    lanes = {}
    for i, j in itertools.product(range(8), range(4)):
        lanes[4 * i + j] = ((i, 2 * j), (i, 2 * j + 1))
    cells = [c for v in lanes.values() for c in v]
    assert sorted(cells) == sorted(itertools.product(range(8), range(8)))
    # B with x1: 2 copies x 32 lanes, each source row of 8 halves referenced
    counts = keyed("retile.txt", "counts")[0]
    want = dict(zip(counts[::2], (int(x) for x in counts[1::2])))
    b_dst = sum(1 for lane in range(32) for v in range(4))
    assert b_dst == want["b_dst"]
    assert 2 * 32 * 8 == want["src_refs"]
    assert 32 * 4 == want["x2_dst"]


# -------------------------------------------------------------- ldmatrix x4
def _route_layouts():
    lays = _golden_layouts("ldmatrix_route.txt")
    return lays["S"], lays["D"]


def test_route_target_and_inverse():
    S, D = _route_layouts()
    A = L.parse(L.SM80_A_TV)
    tok = keyed("ldmatrix_route.txt", "target")[0]
    lane, v, q, m, k = (int(tok[i]) for i in (1, 3, 5, 7, 9))
    assert L.evaluate(A, (lane, v)) == q and (q % 16, q // 16) == (m, k)
    tok = keyed("ldmatrix_route.txt", "route")[0]
    dst = pairs(tok[1])[0]
    e = L.evaluate(D, dst)
    assert e == int(tok[3])
    s_inv = L.right_inverse_table(L.table(S))
    src_flat = s_inv[e]
    assert L.decode(src_flat, S[0]) == pairs(tok[5])[0]


def test_route_rows_and_blocks():
    S, D = _route_layouts()
    A = L.parse(L.SM80_A_TV)
    r_inv = L.right_inverse_table(L.table(D))          # R = D
    for tok in keyed("ldmatrix_route.txt", "row"):
        src = pairs(tok[0])[0]
        e = L.evaluate(S, src)
        tv = r_inv[e]
        ref = L.decode(tv, D[0])
        q = L.table(A)[tv]
        mk = (q % 16, q // 16)
        off = 16 * mk[0] + mk[1]                         # sA = (16,16):(16,1)
        assert [e, tv, q, off, 0x1000 + 2 * off] == [int(tok[1]), int(tok[3]), int(tok[4]), int(tok[6]), int(tok[7], 16)]
        assert (ref[0], ref[1][0] + 2 * ref[1][1]) == pairs(tok[2])[0]
        assert mk == pairs(tok[5])[0]
    for tok in keyed("ldmatrix_route.txt", "block"):
        b = int(tok[0])
        l0, l1 = (int(x) for x in tok[1].split("-"))
        m0, m1 = (int(x) for x in tok[2].split("-"))
        k0, k1 = (int(x) for x in tok[3].split("-"))
        for t in range(l0, l1 + 1):
            for p in range(8):
                q = L.table(A)[r_inv[L.evaluate(S, (t, p))]]
                m, k = q % 16, q // 16
                assert m0 <= m <= m1 and k0 <= k <= k1 and k == k0 + p and m == m0 + (t - l0)


def test_x4_routes_agree_with_copy_layouts():
    S, D = _route_layouts()
    A = L.parse(L.SM80_A_TV)
    r_inv = L.right_inverse_table(L.table(D))
    d_inv = r_inv
    a_tab = L.table(A)
    routes = slots = 0
    seen_slots = set()
    for b, row, col in itertools.product(range(4), range(8), range(8)):
        addr_lane, recv_lane, reg, half = L.ldsm_x4_route(b, row, col)
        e = L.evaluate(S, (addr_lane, col))
        dst = L.decode(d_inv[e], D[0])                  # (lane, (half, reg))
        assert dst == (recv_lane, (half, reg))
        v = half + 2 * reg
        assert a_tab[r_inv[e]] == L.evaluate(A, (recv_lane, v))
        routes += 1
        seen_slots.add((recv_lane, v))
    slots = len(seen_slots)
    c = keyed("ldmatrix_route.txt", "counts")[0]
    assert routes == int(c[1]) and slots == int(c[3]) and slots // 2 == int(c[5])


def test_lane0_packed_operands_with_labels():
    A = L.parse(L.SM80_A_TV)
    label = {}
    for m, k in itertools.product(range(16), range(16)):
        label[(m, k)] = 16 * m + k
    label[(0, 9)] = 37
    vals = []
    for v in range(8):
        q = L.evaluate(A, (0, v))
        vals.append(label[(q % 16, q // 16)])
    ops = keyed("ldmatrix_route.txt", "operand")
    assert [(int(o[1]), int(o[2])) for o in ops] == [(vals[2 * i], vals[2 * i + 1]) for i in range(4)]


# ---------------------------------------------------------------- simple GEMM
def test_simple_gemm_printed_partitions():
    pr = {t[0]: L.parse(t[1]) for t in keyed("simple_gemm.txt", "print")}
    K, N = 64, 256
    for (m, k, ik) in itertools.product(range(128), range(16), range(4)):
        assert L.evaluate(pr["gA"], (m, k, ik)) == m * K + k + 16 * ik
    cfg = L.TiledConfig((2, 2, 1), (128, 128, 64), tile=(32, 32, 16))
    rows = table("simple_gemm.txt", "A")
    assert len(rows) == 9
    for key, want in rows.items():
        ik = int(key.split()[0].split("=")[1])
        mm = int(key.split()[1].split("=")[1])
        got = [divmod(L.evaluate(pr["tAgA"], (v, mm, 0, ik)), K) for v in range(8)]
        assert got == want, key
    # the whole thread-0 view agrees with the TiledMMA model
    model_a = cfg.coords_A(0)
    view_a = [divmod(L.evaluate(pr["tAgA"], (v, mm, 0, ik)), K)
              for ik in range(4) for mm in range(4) for v in range(8)]
    assert view_a == model_a
    model_b = cfg.coords_B(0)
    view_b = [divmod(L.evaluate(pr["tBgB"], (v, rn, 0, ik)), K)
              for ik in range(4) for rn in range(8) for v in range(4)]
    assert view_b == model_b
    model_c = cfg.coords_C(0)
    view_c = [divmod(L.evaluate(pr["tDgD"], (v, mm, nn)), N)
              for nn in range(8) for mm in range(4) for v in range(4)]
    assert view_c == model_c


# ------------------------------------------------- gfx950 maps (CPU shape checks)
@pytest.mark.parametrize("op", sorted(L.MFMA_OPS))
def test_mfma_maps_are_bijections(op):
    """Shape checks only; the maps are pinned by the GPU probe test."""
    M, N, K, nv, nacc = L.MFMA_OPS[op]
    ab = [L.mfma_ab_coord(op, lane, v) for lane in range(64) for v in range(nv)]
    assert sorted(ab) == sorted(itertools.product(range(M), range(K)))
    c = [L.mfma_c_coord(op, lane, v) for lane in range(64) for v in range(nacc)]
    assert sorted(c) == sorted(itertools.product(range(M), range(N)))

// Tile configurations and per-lane index maps shared by the kernels and the
// host-side fragment-coordinate export (the same functions run in both).
//
// Structure (pages' prior art, redone for wave64 + MFMA):
//  * a workgroup owns a BM x BN block of D and walks K in BK steps, the CTA
//    tiling of "CuTe Layout 到 Tensor Core" §4 (local_tile with cta_tiler
//    (128,128,32)) and of the simple-GEMM page ("cute(7) simple_gemm" §3.1);
//  * the workgroup's waves are arranged WAVES_M x WAVES_N x WAVES_K, wave id
//    w = wm + WAVES_M*wn + WAVES_M*WAVES_N*wk (M fastest, the compact
//    arrangement of the TiledMMA page, section "第二个参数怎样把一个 warp 扩
//    展成四个").  The WAVES_K K-groups ("K 方向的线程组，与 K 方向的循环") hold
//    the same accumulator positions and split every stage's K sub-steps
//    between them; their partial sums are reduced through LDS at the end, C
//    added once;
//  * each wave repeats the MFMA atom RM x RN times over its WTM x WTN tile
//    and KSUB times along BK (the repeat modes of the TiledMMA page, section
//    "输入扩大以后，后两个 mode 怎样工作", and the register reuse of the
//    simple-GEMM page §2.4);
//  * the N direction carries a tile permutation (TiledMMA page, section "用
//    Layout 改变 M 方向的坐标顺序", applied to N): repeat j of atom column c
//    of a wave's tile is physical column RN*c + j of that tile (in runs of
//    four repeats when a wave has more), so each lane's accumulators of one
//    row come in adjacent columns and D is written in vectors of up to four
//    elements.  B's rows are permuted the same way when they are
//    fetched (global row P(r) goes to LDS row r), so LDS and the fragment
//    reads are unchanged;
//  * operand (row, k) of lane/value comes from the atom's TV layout
//    (mfma_atoms.hpp), composed with the LDS tile layout below, the role the
//    route page ("ldmatrix 怎样对上 MMA 的寄存器") gives F o right_inverse(R)
//    o S.  On gfx950 one 16-byte LDS read fills a whole operand, so the copy
//    needs no regrouping (retile is the identity).
//
// LDS tile layout: rows of BK halves, K contiguous, split into 16-byte chunks
// (8 halves); chunk c of row r is stored at chunk c ^ swz(r).  The XOR keeps
// the 16-byte reads of 16 consecutive rows on distinct banks.  The pages name
// swizzling as an option without giving a function ("CuTe Layout 到 Tensor
// Core" §5); this one is our own.
#pragma once

#include "layout.hpp"
#include "mfma_atoms.hpp"

namespace mfl {

// The matrix instruction a tile configuration issues: atom extent and the
// number of accumulator values per lane.
template <int OP>
struct AtomTraits;
template <>
struct AtomTraits<kMfma32x32x16> {
  static constexpr int M = 32, N = 32, K = 16, NV = 16;
};
template <>
struct AtomTraits<kMfma16x16x32> {
  static constexpr int M = 16, N = 16, K = 32, NV = 4;
};

// DIST: how many K sub-steps ahead the operand fragments are read from LDS
// (1: two register buffers; 2: one buffer per sub-step, the step's barrier
// one sub-step earlier).  WAVES_K: K-groups splitting each stage's sub-steps.
// STAGES: LDS stages; a tile is fetched STAGES-1 steps before it is used.
// OP: the matrix instruction (mfma_atoms.hpp numbering).
template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_, int DIST_ = 1, int WAVES_K_ = 1,
          int STAGES_ = 2, int OP_ = kMfma32x32x16>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_;
  static constexpr int kFragDist = DIST_;
  static constexpr int kStages = STAGES_;
  static constexpr int kOp = OP_;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, WAVES_K = WAVES_K_;
  static constexpr int kGroupWaves = WAVES_M * WAVES_N;   // waves of one K-group
  static constexpr int kWaves = kGroupWaves * WAVES_K;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  static constexpr int kAtomM = AtomTraits<OP_>::M, kAtomN = AtomTraits<OP_>::N,
                       kAtomK = AtomTraits<OP_>::K;
  static constexpr int kNV = AtomTraits<OP_>::NV;   // accumulator values per lane
  static constexpr int RM = WTM / kAtomM, RN = WTN / kAtomN;
  // a lane's repeats along N are stored in runs of kVec adjacent columns
  static constexpr int kVec = RN < 4 ? RN : 4;
  static constexpr int KSUB = BK / kAtomK;        // K sub-steps per stage
  static constexpr int KSUB_W = KSUB / WAVES_K;   // ... taken by each wave
  static constexpr int CH = BK / 8;               // 16-byte chunks per LDS row
  // split-K: one kNV x 64 fp32 block per (wave of a K-group, atom block,
  // other member), written into the operand stages once they are free
  static constexpr int kRedBytes = kGroupWaves * RM * RN * (WAVES_K - 1) * kNV * 64 * 4;
  static constexpr int kLdsA = BM * BK;           // halves per stage
  static constexpr int kLdsB = BN * BK;
  // epilogue: atom rows of accumulators staged through LDS per pass (fp32,
  // every wave at once), the most that fit in the two operand stages
  static constexpr int kEpiRows =
      (RM % 2 == 0 && kWaves * 2 * kAtomM * WTN * 4 <= 4 * (BM + BN) * BK) ? 2 : 1;

  static_assert(BM % (WAVES_M * kAtomM) == 0 && BN % (WAVES_N * kAtomN) == 0,
                "wave tile must be a multiple of the atom");
  static_assert(BK % kAtomK == 0, "BK must be a multiple of the atom K");
  static_assert((BM * CH) % kThreads == 0 && (BN * CH) % kThreads == 0,
                "operand tile chunks must divide evenly over the threads");
  static_assert(CH == 4 || CH == 8 || CH == 16, "swizzle defined for 4, 8 or 16 chunks per row");
  static_assert(DIST_ == 1 || (DIST_ == 2 && KSUB_W >= 4),
                "fragment distance 1, or 2 with 4+ sub-steps per wave");
  static_assert(KSUB % WAVES_K == 0 && KSUB_W % 2 == 0,
                "each K-group takes an even number of the stage's sub-steps");
  static_assert(WAVES_K == 1 || (RM % WAVES_K == 0 &&
                                 kRedBytes <= kStages * 2 * (BM + BN) * BK),
                "split-K: row blocks divide over the K-groups, partials fit in the stages");
  static_assert((kStages == 2 || kStages == 3) && kStages * 2 * (BM + BN) * BK <= 160 * 1024,
                "two or three stages within the 160 KB of LDS");
  static_assert(kWaves * kEpiRows * kAtomM * WTN * 4 <= 4 * (BM + BN) * BK,
                "epilogue staging must fit in the operand stages");
  static_assert(RN % kVec == 0, "runs of adjacent columns must divide the repeats");
};

// Epilogue staging tile of one wave: rows of WTN fp32, 16-byte groups
// XOR-swizzled by bit 2 of the row.  An accumulator store (32 lanes on row r,
// 32 on row r+4, 32 consecutive n each) and a 16-byte read (16 lanes along
// one row) both touch each 4-byte bank once.
template <int WTN>
MFL_HD constexpr int epi_offset(int r, int n) {
  static_assert(WTN % 64 == 0, "needs 16 groups of 4 per row");
  return r * WTN + (((n >> 2) ^ (((r >> 2) & 1) << 3)) << 2) + (n & 3);
}

// XOR swizzle of the 16-byte chunk index within an LDS row.  A 16-byte LDS
// read is served 16 lanes at a time across 64 four-byte banks (256 bytes), so
// the 16 rows that 16 consecutive lanes read (same logical chunk) must land
// on 16 different 16-byte bank groups: (row*CH + chunk') mod 16 distinct.
// For CH = 8 that is parity(row) and (row>>1)&7; for CH = 4, row&3 and
// (row>>2)&3; for CH = 16 a row spans all 64 banks and the chunk alone
// decides, so the XOR is row&15.
template <int CH>
MFL_HD constexpr int swz(int row) {
  return CH == 16 ? (row & 15) : CH == 8 ? ((row >> 1) & 7) : ((row >> 2) & 3);
}

struct RowK {
  int row, k;
};

// element offset (in halves) of (row, k) in one LDS operand tile
template <int BK>
MFL_HD constexpr int lds_offset(int row, int k) {
  constexpr int CH = BK / 8;
  return row * BK + (((k >> 3) ^ swz<CH>(row)) << 3) + (k & 7);
}

// M-contiguous A tile (BK rows of BM halves, one per k): 16-byte chunk c of
// row k is stored at chunk c ^ mn_swz(k), mn_swz(k) = 4(k & 3) + 2((k >> 3)
// & 1).  A 32-lane pass of the transposed LDS read below takes four k-rows x
// 32 m (32x32x16 operand: both 16-lane blocks at the same k) or two sets of
// four k-rows 8 apart x 16 m (16x16x32 operand); with this XOR the 16 chunks
// of a pass fall in 16 different 16-byte bank groups either way.
MFL_HD constexpr int mn_swz(int k) { return ((k & 3) << 2) | (((k >> 3) & 1) << 1); }

template <int BM>
MFL_HD constexpr int lds_offset_mn(int m, int k) {
  static_assert(BM % 128 == 0, "needs at least 16 chunks per row");
  return k * BM + (((m >> 3) ^ mn_swz(k)) << 3) + (m & 7);
}

// Transposed LDS read (ds_read_b64_tr_b16), as measured on gfx950: within
// each block of 16 lanes, output lane i receives element e from source lane
// 4e + i/4, element i%4 (each source lane supplies 4 consecutive halves at
// its own address).  So if source lane s of the block addresses k-row
// k0 + s/4 at m = m0 + 4(s%4), output lane i gets A(m0 + i, k0 + e) for
// e = 0..3: an (m, k) tile stored M-contiguous arrives K-contiguous per
// lane, the regrouping the route page gives ldmatrix ("ldmatrix 怎样对上
// MMA 的寄存器").  Two such reads (k0 and k0 + 4) fill one 32x32x16 operand.
// Source coordinates of lane `lane`'s first read for the atom operand
// (row = l%32, k = 8(l/32) + v): m within the atom, k within the atom.
MFL_HD constexpr RowK atom_a_tr_source(int lane);

// Operand value 0 of `lane` for instruction OP: (row within atom, k within
// atom); values 1..7 follow at k+1..k+7 (the value mode of the layout has
// stride ROWS, i.e. unit step in k).
template <int OP>
MFL_HD constexpr RowK atom_ab_coord_of(int lane) {
  const Layout tv = mfma_tv(OP, 0);
  const int64_t q = eval2(tv, lane, 0);
  return RowK{int(q % AtomTraits<OP>::M), int(q / AtomTraits<OP>::M)};
}

// Accumulator value v of `lane` for instruction OP: (m, n) within the atom
// block.
template <int OP>
MFL_HD constexpr RowK atom_c_coord_of(int lane, int v) {
  const Layout tv = mfma_tv(OP, 2);
  const int64_t q = eval2(tv, lane, v);
  return RowK{int(q % AtomTraits<OP>::M), int(q / AtomTraits<OP>::M)};
}

// Source (m, k) within the atom of lane `lane`'s first transposed read: the
// 16-lane block blk holds operand lanes 16 blk .. 16 blk + 15, i.e. rows
// (16 blk) % M .. +15 at k from 8 ((16 blk) / M); source lane s addresses
// k-row k0 + s/4 at m = m0 + 4 (s % 4).
template <int OP>
MFL_HD constexpr RowK atom_a_tr_source_of(int lane) {
  constexpr int M = AtomTraits<OP>::M;
  const int s = lane & 15, blk = lane >> 4;
  const int m0 = (16 * blk) % M, k0 = 8 * ((16 * blk) / M);
  return RowK{m0 + 4 * (s & 3), k0 + (s >> 2)};
}

// The instruction the back-to-back GEMM issues (and the 32x32 names the
// host exports use).
MFL_HD constexpr Layout atom_ab_tv() { return mfma_tv(kMfma32x32x16, 0); }
MFL_HD constexpr Layout atom_c_tv() { return mfma_tv(kMfma32x32x16, 2); }
MFL_HD constexpr RowK atom_ab_coord(int lane) { return atom_ab_coord_of<kMfma32x32x16>(lane); }
MFL_HD constexpr RowK atom_c_coord(int lane, int v) {
  return atom_c_coord_of<kMfma32x32x16>(lane, v);
}
MFL_HD constexpr RowK atom_a_tr_source(int lane) {
  return atom_a_tr_source_of<kMfma32x32x16>(lane);
}

// The transposed reads deliver exactly the atom's operand layout: output
// lane l, value v = 4h + e comes from source lane 16(l/16) + 4e + (l%16)/4 of
// read h, element (l%16)%4.
template <int OP>
MFL_HD constexpr bool tr_reads_match_atom() {
  for (int l = 0; l < 64; ++l)
    for (int v = 0; v < 8; ++v) {
      const int h = v / 4, e = v % 4, i = l % 16;
      const RowK src = atom_a_tr_source_of<OP>(16 * (l / 16) + 4 * e + i / 4);
      const RowK want = atom_ab_coord_of<OP>(l);
      if (src.row + i % 4 != want.row || src.k + 4 * h != want.k + v) return false;
    }
  return true;
}
static_assert(tr_reads_match_atom<kMfma32x32x16>() && tr_reads_match_atom<kMfma16x16x32>(),
              "transposed reads must produce the MFMA operand layout");

// The accumulator layout splits into a lane part and a value part:
// coord(l, v) = coord(l, 0) + coord(0, v).  The epilogue keeps the lane part
// in a per-lane offset and folds the value part into a uniform base address.
template <int OP>
MFL_HD constexpr bool c_layout_separable() {
  for (int l = 0; l < 64; ++l)
    for (int v = 0; v < AtomTraits<OP>::NV; ++v) {
      const RowK a = atom_c_coord_of<OP>(l, v), b = atom_c_coord_of<OP>(l, 0),
                 c = atom_c_coord_of<OP>(0, v);
      if (a.row != b.row + c.row || a.k != b.k + c.k) return false;
    }
  return true;
}
static_assert(c_layout_separable<kMfma32x32x16>() && c_layout_separable<kMfma16x16x32>(),
              "accumulator (m, n) must split into lane + value parts");

// The value mode must step k by one, so 8 values are one 16-byte run, and
// the layouts must cover their atoms.
template <int OP>
MFL_HD constexpr bool atom_layouts_ok() {
  constexpr int M = AtomTraits<OP>::M, N = AtomTraits<OP>::N, K = AtomTraits<OP>::K;
  const Layout ab = mfma_tv(OP, 0), c = mfma_tv(OP, 2);
  return eval2(ab, 0, 1) - eval2(ab, 0, 0) == M && size(ab) == M * K && size(c) == M * N &&
         size_mode(c, 1) == AtomTraits<OP>::NV;
}
static_assert(atom_layouts_ok<kMfma32x32x16>() && atom_layouts_ok<kMfma16x16x32>(),
              "operand values must be K-contiguous and the layouts cover the atom");

// Wave w of the workgroup: (wm, wn) within its K-group, and the K-group.
template <class Cfg>
MFL_HD constexpr int wave_m(int w) { return (w % Cfg::kGroupWaves) % Cfg::WAVES_M; }
template <class Cfg>
MFL_HD constexpr int wave_n(int w) { return (w % Cfg::kGroupWaves) / Cfg::WAVES_M; }
template <class Cfg>
MFL_HD constexpr int wave_k(int w) { return w / Cfg::kGroupWaves; }

// K offset within a stage of wave w's sub-step kk (0 <= kk < KSUB_W)
template <class Cfg>
MFL_HD constexpr int sub_k(int w, int kk) {
  return (wave_k<Cfg>(w) * Cfg::KSUB_W + kk) * Cfg::kAtomK;
}

// Operand fragment of wave `w`, repeat i (along M or N), the wave's K
// sub-step kk: (row, k) of value 0 within the workgroup tile.
template <class Cfg>
MFL_HD constexpr RowK frag_a_coord(int w, int lane, int i, int kk) {
  const RowK a = atom_ab_coord_of<Cfg::kOp>(lane);
  return RowK{wave_m<Cfg>(w) * Cfg::WTM + i * Cfg::kAtomM + a.row, sub_k<Cfg>(w, kk) + a.k};
}

// Source (m, k) within the workgroup tile of the first transposed read that
// fills A fragment i, K sub-step kk, when A sits M-contiguous in LDS; the
// second read is 4 k-rows further.
template <class Cfg>
MFL_HD constexpr RowK frag_a_tr_coord(int w, int lane, int i, int kk) {
  const RowK t = atom_a_tr_source_of<Cfg::kOp>(lane);
  return RowK{wave_m<Cfg>(w) * Cfg::WTM + i * Cfg::kAtomM + t.row, sub_k<Cfg>(w, kk) + t.k};
}

template <class Cfg>
MFL_HD constexpr RowK frag_b_coord(int w, int lane, int j, int kk) {
  const RowK b = atom_ab_coord_of<Cfg::kOp>(lane);
  return RowK{wave_n<Cfg>(w) * Cfg::WTN + j * Cfg::kAtomN + b.row, sub_k<Cfg>(w, kk) + b.k};
}

// N permutation of the block tile: logical column n = wn*WTN + AN j + c
// (wave, repeat, atom column; the LDS row of B; AN the atom's width) is
// physical column wn*WTN + AN V (j / V) + V c + j % V, V = kVec: a lane's
// repeats come in runs of V adjacent columns (all RN of them when RN <= 4,
// the 32x32 configurations: wn*WTN + RN*c + j).
template <class Cfg>
MFL_HD constexpr int perm_n(int n) {
  constexpr int V = Cfg::kVec, AN = Cfg::kAtomN;
  const int r = n % Cfg::WTN, j = r / AN, c = r % AN;
  return n - r + AN * V * (j / V) + V * c + j % V;
}

// Accumulator value v of repeat (i, j): physical (m, n) within the workgroup
// tile; the same for every K-group.  For a fixed (i, v) a lane's RN repeats
// are adjacent columns.
template <class Cfg>
MFL_HD constexpr RowK frag_c_coord(int w, int lane, int i, int j, int v) {
  const RowK c = atom_c_coord_of<Cfg::kOp>(lane, v);
  return RowK{wave_m<Cfg>(w) * Cfg::WTM + i * Cfg::kAtomM + c.row,
              perm_n<Cfg>(wave_n<Cfg>(w) * Cfg::WTN + j * Cfg::kAtomN + c.k)};
}

// frag_c_coord is the tiled MMA's partition_C written out in closed form.
// Derived with the layout algebra (TiledMMA page, "partition_C 怎样把分工应用
// 到一个 Tensor", with the tile permutations of "用 Layout 改变 M 方向的坐标
// 顺序"): a BM x BN tile stored M-contiguous, divided per direction by a
// permutation -- M: (AM, WAVES_M, RM):(1, AM RM, AM), wave wm takes RM
// adjacent atom blocks instead of every WAVES_M-th one; N: (AN, WAVES_N, V,
// RN/V):(V, AN RN, 1, AN V), the same wave-contiguous blocks with the
// repeats interleaved column by column in runs of V -- then by the AM x AN
// atom, composed with the atom's C TV layout and split over the wave grid.
// Thread lane + 64 w's view is thr(t) + val(v + NV (i + RM j)).  Every
// thread's base and thread 0's values are compared; with the atom layout
// separable (asserted above) that covers every (thread, value).
template <class Cfg>
constexpr bool frag_c_is_partition_c() {
  constexpr int AM = Cfg::kAtomM, AN = Cfg::kAtomN, V = Cfg::kVec, NV = Cfg::kNV;
  Layout C;
  C.open_mode();
  C.push_leaf(Cfg::BM, 1);
  C.open_mode();
  C.push_leaf(Cfg::BN, Cfg::BM);
  const int64_t pm_s[3] = {AM, Cfg::WAVES_M, Cfg::RM}, pm_d[3] = {1, AM * Cfg::RM, AM};
  const int64_t pn_s[4] = {AN, Cfg::WAVES_N, V, Cfg::RN / V},
                pn_d[4] = {V, AN * Cfg::RN, 1, AN * V};
  const Layout tile[2] = {make_flat(3, pm_s, pm_d), make_flat(Cfg::RN / V > 1 ? 4 : 3, pn_s, pn_d)};
  const CPartition p =
      partition_c(C, tile, mfma_tv(Cfg::kOp, 2), AM, AN, Cfg::WAVES_M, Cfg::WAVES_N);
  if (p.thr.status != kLayoutOk || p.val.status != kLayoutOk) return false;
  // partition_C selects (lane, wm, wn) only: every K-group sees the view of
  // the thread with the same (lane, wm, wn)
  for (int t = 0; t < Cfg::kThreads; ++t) {
    const RowK c = frag_c_coord<Cfg>(t / 64, t % 64, 0, 0, 0);
    if (eval(p.thr, t % (64 * Cfg::kGroupWaves)) != c.row + int64_t(Cfg::BM) * c.k) return false;
  }
  for (int j = 0; j < Cfg::RN; ++j)
    for (int i = 0; i < Cfg::RM; ++i)
      for (int v = 0; v < NV; ++v) {
        const RowK c = frag_c_coord<Cfg>(0, 0, i, j, v);
        if (eval(p.val, v + NV * (i + Cfg::RM * j)) != c.row + int64_t(Cfg::BM) * c.k) return false;
      }
  return true;
}

// Workgroup -> output tile.  Workgroups are handed to the 8 XCDs round-robin
// (XCD = id % 8); regrouping ids so each XCD gets a contiguous run, then
// walking that run in GROUP_M-tall column bands, keeps the A rows and B
// columns one XCD touches together in its L2.
struct TileIndex {
  int tm, tn;
};

MFL_HD constexpr TileIndex tile_of_block(int bid, int nb, int tiles_m, int tiles_n,
                                         int group_m) {
  constexpr int kXcds = 8;
  const int q = nb / kXcds, r = nb % kXcds;
  const int xcd = bid % kXcds, idx = bid / kXcds;
  const int lin = xcd * q + (xcd < r ? xcd : r) + idx;
  const int band = group_m * tiles_n;
  const int g = lin / band;
  const int first_m = g * group_m;
  const int gm = (tiles_m - first_m) < group_m ? (tiles_m - first_m) : group_m;
  const int in = lin - g * band;
  return TileIndex{first_m + in % gm, in / gm};
}

}  // namespace mfl

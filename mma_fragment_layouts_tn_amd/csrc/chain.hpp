// Back-to-back GEMM with the first accumulator reused as the second
// operand in registers: per batch,
//
//     P = rne16(A B^T)  (M x N1, fp32 sums),   D = P W^T  (M x N2, fp32 sums)
//
// the attention-style chain of "CuTe Layout 到 Tensor Core" (§17, "为什么这
// 套抽象对 FlashAttention 特别重要"): whether the register ownership of the
// first MMA's accumulator can be read as the operand ownership the second
// MMA needs, by layout algebra instead of moving the matrix.
//
// On gfx950, with v_mfma_f32_32x32x16_f16, it can.  The first product is
// issued transposed (S^T = B A^T: B's rows are the A operand), so lane l's
// accumulators hold row m = l % 32 of S.  The second MMA's A operand wants
// row m = l % 32 as well, 8 values per 16-wide K chunk.  The accumulators
// 8 kc .. 8 kc + 7 of a lane become chunk kc of that operand as they are
// (converted to fp16): K position p = 16 kc + 8 h + v of the second MMA is
// row pi(p) of the first (transposed) accumulator.  pi is derived below from
// the two atom TV layouts and checked at compile time.  The kernel absorbs it
// in the order it stages B: LDS row r of a 32-row block holds N1 row
// pi^-1(r), so P arrives in natural N1 order and W is staged as it lies in
// memory, every lane reading its 8 values with one 16-byte read.
#pragma once

#include <hip/hip_runtime.h>

#include "gemm_tile.hpp"

namespace mfl {

struct ChainParams {
  int batch, M, N1, N2;
  int64_t lda, ldb, ldw, ldd;
  int64_t sa, sb, sw, sd;           // batch strides (elements)
  int tiles_m, tiles_n, group_m;    // tiles_m counts batch x M tiles
  int d_vec;                        // D rows take aligned 4-element vectors
  const void* A;
  const void* B;
  const void* W;
  void* D;
  unsigned* stamps;                 // phase clock stamps (timed probe instance only)
};

// ---------------------------------------------------------------- the pi map
// K position p (0..31) of the second MMA over one 32-row block -> row of the
// first accumulator: lane l, chunk kc, value v of the operand (row
// atom_ab(l).row, k = 16 kc + atom_ab(l).k + v) takes accumulator value
// 8 kc + v of the same lane, which sits at (row r, column m) =
// atom_c(l, 8 kc + v) of the transposed first product (row r: the B row in
// LDS row r of the block).  Requires: the accumulator's column is the
// operand's row (so the values stay in their lane), every lane with the same
// k agrees on the row (pi is a function of p), and pi is a bijection.
struct ChainPerm {
  int n1[32];     // pi: accumulator row feeding K position p
  int pos[32];    // pi^-1
  bool ok;
};

MFL_HD constexpr ChainPerm chain_k_perm() {
  ChainPerm r{};
  for (int p = 0; p < 32; ++p) r.n1[p] = r.pos[p] = -1;
  r.ok = true;
  for (int lane = 0; lane < 64; ++lane)
    for (int kc = 0; kc < 2; ++kc)
      for (int v = 0; v < 8; ++v) {
        const RowK a = atom_ab_coord(lane);
        const RowK c = atom_c_coord(lane, 8 * kc + v);
        const int p = 16 * kc + a.k + v;
        if (c.k != a.row) r.ok = false;                    // same lane, same m
        if (r.n1[p] == -1) r.n1[p] = c.row;
        else if (r.n1[p] != c.row) r.ok = false;           // pi well defined
      }
  for (int p = 0; p < 32; ++p) {
    if (r.n1[p] < 0 || r.n1[p] > 31 || r.pos[r.n1[p]] != -1) {
      r.ok = false;
      return r;
    }
    r.pos[r.n1[p]] = p;
  }
  return r;
}

// runs of 4 consecutive N1 columns stay together under pi, so pi^-1 is
// known from its values at the run starts
MFL_HD constexpr bool chain_runs_of_4() {
  const ChainPerm r = chain_k_perm();
  for (int n = 0; n < 32; ++n)
    if (r.pos[n] != r.pos[n - n % 4] + n % 4 || r.pos[n - n % 4] % 4 != 0) return false;
  return true;
}

static_assert(chain_k_perm().ok, "the accumulator must read as the next operand");
static_assert(chain_runs_of_4(), "pi must keep runs of 4 N1 columns");

// ------------------------------------------------------------------ kernel
// Workgroup: 256 rows of M x BN columns of N2 (RN = BN / 32 atom columns,
// N-permuted: repeat j of atom column c is column RN c + j, so D leaves in
// RN-element vectors).  At K = 64 and 128, 8 waves of 32 rows (RM = 1 atom
// row), two per SIMD, so one wave's own issue work (fetch instructions,
// fragment reads, the S -> P conversion, waits) runs under the other's
// MFMAs; otherwise 4 waves of 64 rows (RM = 2), where the fetch does not
// divide over 8 waves (K = 32: a B chunk is 4 KiB) or the registers do not
// allow two waves (K = 256).  N1 is consumed in chunks of CW = 32 H columns,
// H blocks of 32.
//
// Where pi goes: LDS row 32 h + r of a B chunk holds N1 row 32 h + pi^-1(r)
// of it, so the first product's accumulator value at atom row r of block h
// is N1 column 32 h + pi^-1(r), and lane l's values 8 kc .. 8 kc + 7 of that
// block become K positions 32 h + 16 kc + 8 (l / 32) + v = N1 columns in
// natural order.  W is then staged as it is in memory.
//
// Software pipeline: iteration c issues the second product of chunk c (its
// P in registers) interleaved with the first product of chunk c+1, so the
// matrix core never waits for a first product before the second can start.
// Slot c of the LDS ring (stage c mod 4) holds B of chunk c+1 and W of chunk
// c, the operands of iteration c; slot -1 holds B of chunk 0 for the
// prologue.  One barrier per iteration, before the second product's last K
// chunk: after it every wave is done with slot c and can read slot c+1, and
// the last K chunk runs on registers while the next slot's first fragments
// are read.  Fetch: direct global-to-LDS loads when B and W are 16-byte
// aligned and N1 fills whole chunks, slot c+3 issued during iteration c into
// the stage slot c-1 left (it lands before the barrier of iteration c+2);
// otherwise through registers with zero fill, slot c+2 loaded after the
// barrier of iteration c and written to LDS before that of iteration c+1.
namespace chain {
constexpr int BM = 256, NST = 4;
// waves per workgroup (two per SIMD at K = 64 and 128) and threads
MFL_HD constexpr int waves(int kd) { return kd == 64 || kd == 128 ? 8 : 4; }
MFL_HD constexpr int threads(int kd) { return 64 * waves(kd); }
// N2 columns per workgroup: 128 (RN = 4 atom columns per wave), 64 when N2
// fits in it (RN = 2: no MFMAs on columns past N2)
MFL_HD constexpr int tile_n(int64_t n2) { return n2 <= 64 ? 64 : 128; }
// N1 columns per iteration (H = CW / 32 atom blocks): 64 halves the
// iterations' fixed costs (barrier, conversion); at K = 256 the register
// budget keeps it at 32
MFL_HD constexpr int chunk_width(int kd) { return kd >= 256 ? 32 : 64; }

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
using lds_t = __attribute__((address_space(3))) void*;

// B chunk tile: CW rows x KD halves, 16-byte chunks XOR-swizzled as the GEMM
// tiles (16 consecutive rows at one chunk land on distinct bank groups)
template <int KD>
MFL_HD constexpr int b_swz(int row) {
  return KD / 8 >= 16 ? (row & 15) : swz<KD / 8>(row);
}
template <int KD>
__device__ __forceinline__ int b_off(int row, int k) {
  return row * KD + (((k >> 3) ^ b_swz<KD>(row)) << 3) + (k & 7);
}

// W chunk tile: BN rows x CW halves (N1 in natural order), the CW / 8
// 16-byte chunks of a row XOR-swizzled so that 16 consecutive rows at one
// chunk fall on distinct bank groups
template <int CW>
MFL_HD constexpr int w_swz(int row) {
  return CW == 32 ? (row >> 2) & 3 : (row >> 1) & 7;
}
template <int CW>
__device__ __forceinline__ int w_off(int row, int n) {
  return row * CW + (((n >> 3) ^ w_swz<CW>(row)) << 3) + (n & 7);
}

// the N2 column held by W's LDS row r (the N permutation of the tile)
template <int RN>
__device__ __forceinline__ int w_col(int r) { return RN * (r % 32) + r / 32; }

template <bool V>
struct BoolC {
  static constexpr bool value = V;
};

__device__ __forceinline__ uint4 load16(const _Float16* p) {
  uint4 v;
  __builtin_memcpy(&v, p, 16);
  return v;
}

// n (1..7) leading halves of p, the rest zero
__device__ __forceinline__ uint4 load_partial(const _Float16* p, int n) {
  union {
    uint4 u;
    _Float16 h[8];
  } r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r.h[e] = e < n ? p[e] : (_Float16)0.0f;
  return r.u;
}

// LDS reads and writes of this wave done, then the workgroup barrier (no
// memory fence: direct-to-LDS loads still in flight are waited for by count)
__device__ __forceinline__ void barrier() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

// wait until at most VM vector-memory operations of this wave are in flight
template <int VM>
__device__ __forceinline__ void wait_vm() {
  static_assert(VM >= 0 && VM < 64, "vmcnt has 6 bits");
  __builtin_amdgcn_s_waitcnt((VM & 15) | (((VM >> 4) & 3) << 14) | (7 << 4) | (15 << 8));
}
}  // namespace chain

// Phase stamps of the timed probe instance: per wave, kStampIters x 4
// shader-clock readings (iteration c: 4c + 0 at its start, + 1 before the
// wait for the next slot's fetch, + 2 before the barrier, + 3 after it), then
// 3 more (kernel start, after the loop, after the epilogue); kStampWaves per
// workgroup.
namespace chain {
constexpr int kStampIters = 64, kStampsPerWave = 4 * kStampIters + 4, kStampBlocks = 8,
              kStampWaves = 8;
}

template <int KD, int DK, bool DMA, int BN, bool TIMED = false>
__global__ void __launch_bounds__(chain::threads(KD), 1) gemm_chain(const ChainParams p) {
  using namespace chain;
  constexpr int WAVES = waves(KD), THREADS = threads(KD), RM = BM / WAVES / 32;
  static_assert(!TIMED || WAVES <= kStampWaves, "stamp slots for every wave");
  static_assert(KD == 32 || KD == 64 || KD == 128 || KD == 256, "K is 32, 64, 128 or 256");
  static_assert(BN == 64 || BN == 128, "N2 tiles of 64 or 128 columns");
  constexpr int RN = BN / 32;
  constexpr int KSUB = KD / 16, CH = KD / 8;
  constexpr int CW = chunk_width(KD), H = CW / 32;
  static_assert(CW == 32 || CW == 64, "chunks of 32 or 64 N1 columns");
  constexpr int BSTAGE = CW * KD, WSTAGE = BN * CW, STAGE = BSTAGE + WSTAGE;   // halves
  __shared__ __attribute__((aligned(1024))) _Float16 smem[NST * STAGE];
  constexpr ChainPerm kPi = chain_k_perm();
  // pi^-1 of an LDS row: runs of 4 keep their order, the run start is a
  // select over the table's compile-time entries (no indexed memory)
  auto pi_inv = [&](int r) {
    const int r0 = r & 28;
    int q = kPi.pos[0];
#pragma unroll
    for (int e = 4; e < 32; e += 4)
      if (r0 == e) q = kPi.pos[e];
    return (r & ~31) + q + (r & 3);   // within each 32-row block
  };

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // timed instance: the shader clock at fixed points.  A reading stays in a
  // scalar register until a point where the wave waits for its LDS reads
  // anyway (the barrier, the end of the iteration), and goes to lane c of
  // tv[k] for iteration c: the readings add no LDS traffic and no waits.
  auto now = [&]() -> unsigned {
    unsigned t = 0;
    if constexpr (TIMED) {
      __builtin_amdgcn_sched_barrier(0);
      t = (unsigned)__builtin_amdgcn_s_memtime();
      __builtin_amdgcn_sched_barrier(0);
    }
    return t;
  };
  unsigned tv[4] = {0, 0, 0, 0};
  auto keep = [&](int k, int c, unsigned t) {
    if constexpr (TIMED) {
      __builtin_amdgcn_sched_barrier(0);
      tv[k] = lane == c ? t : tv[k];
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  const unsigned t_start = now();
  const TileIndex ti = tile_of_block(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m);
  const int mt_per_b = (p.M + BM - 1) / BM;
  const int b = ti.tm / mt_per_b;
  const int m0 = (ti.tm % mt_per_b) * BM, n0 = ti.tn * BN;
  const _Float16* A = (const _Float16*)p.A + (int64_t)b * p.sa;
  const _Float16* B = (const _Float16*)p.B + (int64_t)b * p.sb;
  const _Float16* Wm = (const _Float16*)p.W + (int64_t)b * p.sw;
  const int nch = (p.N1 + CW - 1) / CW;

  // this wave's A rows as the second operand of the first product:
  // fragment (i, kk) of lane l: row m0 + 32 RM w + 32 i + l % 32, k = 16 kk + 8 (l / 32)
  const RowK al = atom_ab_coord(lane);
  half8 af[RM][KSUB];
#pragma unroll
  for (int i = 0; i < RM; ++i) {
    const int m = min(m0 + 32 * RM * w + 32 * i + al.row, p.M - 1);
#pragma unroll
    for (int kk = 0; kk < KSUB; ++kk) {
      const uint4 u = load16(A + (int64_t)m * p.lda + 16 * kk + al.k);
      __builtin_memcpy(&af[i][kk], &u, 16);
    }
  }

  // ---- staging of slot s: B of chunk s+1 and W of chunk s, when they exist
  // DMA: one instruction moves 64 lanes x SZ bytes into consecutive LDS bytes;
  // each lane fetches the element its LDS bytes stand for
  constexpr int SZB = KD * H >= 64 ? 16 : 4;
  constexpr int NB = 2 * CW * KD / (64 * SZB) / WAVES, NW = 2 * CW * BN / 1024 / WAVES;
  static_assert(NB >= 1 && NW >= 1, "every wave issues B and W loads");
  // registers: 16-byte chunks q = tid + t * THREADS of each tile
  constexpr int BCH = CW * CH, WCH = BN * CW / 8;
  constexpr int BPT = (BCH + THREADS - 1) / THREADS, WPT = WCH / THREADS;
  static_assert(WCH % THREADS == 0, "W chunks divide over the threads");
  constexpr int NBI = DMA ? NB : BPT, NWI = DMA ? NW : WPT;
  int64_t boff[NBI], woff[NWI];   // element offsets within chunk 0
  int brow[NBI], wn1[NWI];        // (registers) N1 row / column within a chunk
  uint4 rb[DMA ? 1 : BPT], rw[DMA ? 1 : WPT];
  if constexpr (DMA) {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int byte = (w * NB + i) * 64 * SZB + SZB * lane;
      const int r = byte / (2 * KD), rb_ = byte % (2 * KD);
      const int k = 8 * ((rb_ / 16) ^ b_swz<KD>(r)) + (rb_ % 16) / 2;
      brow[i] = pi_inv(r);
      boff[i] = (int64_t)brow[i] * p.ldb + k;
    }
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const int byte = (w * NW + i) * 1024 + 16 * lane;
      const int r = byte / (2 * CW), q = (byte % (2 * CW)) / 16;
      const int n2 = min(n0 + w_col<RN>(r), p.N2 - 1);
      wn1[i] = 8 * (q ^ w_swz<CW>(r));
      woff[i] = (int64_t)n2 * p.ldw + wn1[i];
    }
  } else {
#pragma unroll
    for (int t = 0; t < BPT; ++t) {
      const int q = min(tid + t * THREADS, BCH - 1), r = q / CH;
      brow[t] = pi_inv(r);
      boff[t] = 8 * (q % CH);
    }
#pragma unroll
    for (int t = 0; t < WPT; ++t) {
      const int q = tid + t * THREADS, r = q / (CW / 8);
      const int n2 = min(n0 + w_col<RN>(r), p.N2 - 1);
      wn1[t] = 8 * (q % (CW / 8));
      woff[t] = (int64_t)n2 * p.ldw + wn1[t];
    }
  }
  auto stage_of = [](int slot) { return (slot + NST) % NST; };
  // DMA instruction j of slot s: B rows for j < NB, W rows after
  auto issue_one = [&](int s, int j) {
    _Float16* st = smem + stage_of(s) * STAGE;
    const int cb = s + 1, cw = s;
    if (j < NB) {
      if (cb < nch) {
        const void* g = B + (int64_t)(CW * cb) * p.ldb + boff[j];
        const lds_t l = (lds_t)(st + (w * NB + j) * 32 * SZB);
        if constexpr (SZB == 16)
          __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
        else
          __builtin_amdgcn_global_load_lds(g, l, 4, 0, 0);
      }
    } else if (cw >= 0 && cw < nch) {
      __builtin_amdgcn_global_load_lds((const void*)(Wm + CW * cw + woff[j - NB]),
                                       (lds_t)(st + BSTAGE + (w * NW + j - NB) * 512), 16, 0, 0);
    }
  };
  // issue the loads of slot s (DMA: straight into its stage)
  auto issue = [&](int s) {
    if constexpr (DMA) {
#pragma unroll
      for (int j = 0; j < NB + NW; ++j) issue_one(s, j);
    } else {
      const int cb = s + 1, cw = s;
      if (cb < nch) {
#pragma unroll
        for (int t = 0; t < BPT; ++t) {
          const int n1 = min(CW * cb + brow[t], p.N1 - 1);   // zeroed when written
          rb[t] = load16(B + (int64_t)n1 * p.ldb + boff[t]);
        }
      }
      if (cw >= 0 && cw < nch) {
#pragma unroll
        for (int t = 0; t < WPT; ++t)
          if (CW * cw + wn1[t] + 8 <= p.N1) rw[t] = load16(Wm + CW * cw + woff[t]);
      }
    }
  };
  // registers: write slot s to its stage, zero beyond N1
  auto stash = [&](int s) {
    if constexpr (!DMA) {
      _Float16* st = smem + stage_of(s) * STAGE;
      const int cb = s + 1, cw = s;
      if (cb < nch) {
#pragma unroll
        for (int t = 0; t < BPT; ++t) {
          const int q = tid + t * THREADS;
          if (BCH % THREADS == 0 || q < BCH) {
            const uint4 v = CW * cb + brow[t] < p.N1 ? rb[t] : make_uint4(0, 0, 0, 0);
            *(uint4*)&st[b_off<KD>(q / CH, (int)boff[t])] = v;
          }
        }
      }
      if (cw >= 0 && cw < nch) {
#pragma unroll
        for (int t = 0; t < WPT; ++t) {
          const int q = tid + t * THREADS, left = p.N1 - CW * cw - wn1[t];
          uint4 v = rw[t];
          if (left < 8)
            v = left > 0 ? load_partial(Wm + CW * cw + woff[t], left) : make_uint4(0, 0, 0, 0);
          *(uint4*)&st[BSTAGE + w_off<CW>(q / (CW / 8), wn1[t])] = v;
        }
      }
    }
  };
  // DMA: wait until every slot before s has landed (slots s and s+1 may be
  // in flight; a slot brings NB + NW instructions, only NW for the last
  // chunk's W, none past it)
  auto wait_before_two = [&](int s) {
    if constexpr (DMA) {
      if (s + 2 < nch) wait_vm<2 * (NB + NW)>();
      else if (s + 1 < nch) wait_vm<NB + 2 * NW>();
      else if (s < nch) wait_vm<NW>();
      else wait_vm<0>();
    }
  };

  floatx16 acc[RM][RN];
#pragma unroll
  for (int i = 0; i < RM; ++i)
#pragma unroll
    for (int j = 0; j < RN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // the accumulator, rounded once to fp16, is the next operand: values
  // 8 kc' .. 8 kc' + 7 of block h are K chunk kc = 2 h + kc'
  typedef half8 Frag[RM][2 * H];
  auto convert = [&](const floatx16 (&st)[RM][H], Frag& out) {
#pragma unroll
    for (int i = 0; i < RM; ++i)
#pragma unroll
      for (int kc = 0; kc < 2 * H; ++kc)
#pragma unroll
        for (int v = 0; v < 8; ++v) out[i][kc][v] = (_Float16)st[i][kc / 2][8 * (kc % 2) + v];   // RNE
  };
  // one piece of it, out[i][kc]; the empty asm keeps the piece where it is
  // made (beside the MFMAs it runs under) instead of sinking it to its use
  auto convert_one = [&](const floatx16 (&st)[RM][H], Frag& out, int i, int kc) {
#pragma unroll
    for (int v = 0; v < 8; ++v) out[i][kc][v] = (_Float16)st[i][kc / 2][8 * (kc % 2) + v];
    asm volatile("" : "+v"(out[i][kc]));
  };
  auto zero_st = [&](floatx16 (&st)[RM][H]) {
#pragma unroll
    for (int i = 0; i < RM; ++i)
#pragma unroll
      for (int h = 0; h < H; ++h)
#pragma unroll
        for (int v = 0; v < 16; ++v) st[i][h][v] = 0.0f;
  };
  auto read_b = [&](const _Float16* sb, int s) {   // step s: block s / KSUB, sub-step s % KSUB
    return *(const half8*)&sb[b_off<KD>(32 * (s / KSUB) + al.row, 16 * (s % KSUB) + al.k)];
  };
  auto read_w = [&](const _Float16* sw, int kc, half8 (&wf)[RN]) {
#pragma unroll
    for (int j = 0; j < RN; ++j)
      wf[j] = *(const half8*)&sw[w_off<CW>(32 * j + al.row, 16 * kc + al.k)];
  };
  // first product of B's block s / KSUB (S^T), K sub-step s % KSUB
  auto first_step = [&](floatx16 (&st)[RM][H], const half8& bf, int s) {
    const int h = s / KSUB, kk = s % KSUB;
#pragma unroll
    for (int i = 0; i < RM; ++i)
      st[i][h] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf, af[i][kk], st[i][h], 0, 0, 0);
  };
  auto second = [&](const Frag& pf, int kc, int g, const half8 (&wf)[RN]) {
    acc[g / RN][g % RN] = __builtin_amdgcn_mfma_f32_32x32x16_f16(pf[g / RN][kc], wf[g % RN],
                                                                 acc[g / RN][g % RN], 0, 0, 0);
  };

  // Iteration c on slot c: the second product of chunk c over its 2H K
  // chunks (P in registers) with the FS steps of the first product of chunk
  // c+1 spread over all but the last K chunk.  The barrier that closes the
  // slot comes before the last K chunk, which runs on fragments already in
  // registers while the first fragments of slot c+1 are read.  Direct-to-LDS,
  // slot c+3 goes to the stage of slot c-1, which every wave left at the
  // previous barrier, one DMA instruction at a time spread over the K chunks
  // before the barrier; it has two iterations to land.  Through registers,
  // slot c+2 is loaded after the barrier and written to its stage in the
  // next iteration.  P of chunk c+1 is converted piece by piece beside the
  // MFMAs: block h of S in K chunk 2H-2 (all but the last block, whose
  // first-product steps are done by then) or 2H-1 (the last block).
  constexpr int FS = KSUB * H, NPRE = (2 * H - 1) * RM * RN, NI = NB + NW;
  auto convert_at = [&](const floatx16 (&st)[RM][H], Frag& out, int kc, int g) {
#pragma unroll
    for (int h = 0; h < H; ++h)
      if ((h == H - 1 ? 2 * H - 1 : 2 * H - 2) == kc)
#pragma unroll
        for (int q = 0; q < 2 * RM; ++q)
          if (q * RM * RN / (2 * RM) == g) convert_one(st, out, q / 2, 2 * h + q % 2);
  };
  // Fragments are read ahead of their use, after the MFMAs of the slot they
  // follow: W of K chunk kc+1 after the first MFMA of K chunk kc, B of step
  // s1+RA after the MFMAs of step s1.  A wait for one is then a wait for reads
  // issued several MFMAs earlier, not for the read just issued.
  constexpr int RA = FS < 2 ? FS : 2;
  Frag pf, pn;
  half8 wf0[RN], bc[RA];   // carried: W of the next chunk, K chunk 0; its B, steps 0..RA-1
  auto iteration = [&](int c, auto more) {
    constexpr bool MORE = decltype(more)::value;
    const unsigned t0 = now();
    unsigned t1 = 0, t2 = 0, t3 = 0;
    const _Float16* sb = smem + stage_of(c) * STAGE;
    const _Float16* sw = sb + BSTAGE;
    floatx16 st[RM][H];
    zero_st(st);
    half8 wf[RN], wn[RN], bq[RA];
#pragma unroll
    for (int j = 0; j < RN; ++j) wf[j] = wf0[j];
#pragma unroll
    for (int kc = 0; kc < 2 * H; ++kc) {
      if (kc > 0) {
#pragma unroll
        for (int j = 0; j < RN; ++j) wf[j] = wn[j];
      }
      if (kc == 2 * H - 1) {
        if constexpr (MORE) {
          t1 = now();
          stash(c + 1);          // registers: slot c+1, loaded one iteration ago
          if constexpr (DMA)
            wait_before_two(c + 2);   // slot c+1 has landed; c+2 and c+3 may be in flight
          else
            wait_vm<0>();
          t2 = now();
          barrier();             // ... in every wave; slot c-1 is free
          t3 = now();
          keep(0, c, t0);
          keep(1, c, t1);
          keep(2, c, t2);
        }
      }
#pragma unroll
      for (int g = 0; g < RM * RN; ++g) {
        if constexpr (MORE) {
          if (kc < 2 * H - 1) {
#pragma unroll
            for (int s1 = 0; s1 < FS; ++s1)
              if (s1 * NPRE / FS == kc * RM * RN + g) {
                first_step(st, s1 < RA ? bc[s1] : bq[s1 % RA], s1);
                if (s1 + RA < FS) bq[s1 % RA] = read_b(sb, s1 + RA);
              }
          }
        }
        second(pf, kc, g, wf);
        if constexpr (MORE) {
          if (kc == 2 * H - 1) {
            if (g == 0) {
              // after the barrier: the next slot's first fragments (B of
              // chunk c+2 may not exist: its value is then stale and unused,
              // the last iteration has no first product)
              const _Float16* nb = smem + stage_of(c + 1) * STAGE;
              read_w(nb + BSTAGE, 0, wf0);
#pragma unroll
              for (int r = 0; r < RA; ++r) bc[r] = read_b(nb, r);
              if constexpr (!DMA) issue(c + 2);
            }
          } else if constexpr (DMA) {
#pragma unroll
            for (int j = 0; j < NI; ++j)
              if (j * NPRE / NI == kc * RM * RN + g) issue_one(c + 3, j);
          }
          convert_at(st, pn, kc, g);
        }
        if (g == 0 && kc + 1 < 2 * H) read_w(sw, kc + 1, wn);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (MORE) {
#pragma unroll
      for (int i = 0; i < RM; ++i)
#pragma unroll
        for (int kc = 0; kc < 2 * H; ++kc) pf[i][kc] = pn[i][kc];
      keep(3, c, t3);
    } else {
      keep(0, c, t0);
    }
  };

  // the whole main loop sits under this test, so on every path into it the
  // prologue has waited for A's fragments
  if (nch > 0) {
    issue(-1);
    stash(-1);
    issue(0);
    stash(0);
    issue(1);                        // registers: written in iteration 0
    if constexpr (DMA) {
      issue(2);
      wait_before_two(1);
    }
    barrier();
    {
      floatx16 st[RM][H];
      zero_st(st);
      const _Float16* sb = smem + stage_of(-1) * STAGE;
#pragma unroll
      for (int s1 = 0; s1 < FS; ++s1) first_step(st, read_b(sb, s1), s1);
      // direct-to-LDS: iteration 0 fetches slot 3 into this stage
      if constexpr (DMA) barrier();
      convert(st, pf);
      const _Float16* s0 = smem + stage_of(0) * STAGE;
      read_w(s0 + BSTAGE, 0, wf0);
#pragma unroll
      for (int r = 0; r < RA; ++r) bc[r] = read_b(s0, r);   // B of chunk 1, if it exists
    }
    for (int c = 0; c + 1 < nch; ++c) iteration(c, BoolC<true>{});
    iteration(nch - 1, BoolC<false>{});
  }
  const unsigned t_loop = now();

  // epilogue: acc[i][j][v] of lane l is D(m0 + 32 RM w + 32 i + atom_c(l, v).row,
  // n0 + 4 (l % 32) + j): one 4-element vector per (i, v)
  const RowK cl = atom_c_coord(lane, 0);
#pragma unroll
  for (int i = 0; i < RM; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = m0 + 32 * RM * w + 32 * i + atom_c_coord(lane, v).row;
      const int n = n0 + RN * cl.k;
      if (m >= p.M) continue;
      float x[RN];
#pragma unroll
      for (int j = 0; j < RN; ++j) x[j] = acc[i][j][v];
      const int64_t row = (int64_t)b * p.sd + (int64_t)m * p.ldd;
      if (p.d_vec && n + RN <= p.N2) {
        if constexpr (DK == 2) {
          typedef float fv __attribute__((ext_vector_type(RN)));
          fv y;
#pragma unroll
          for (int j = 0; j < RN; ++j) y[j] = x[j];
          __builtin_nontemporal_store(y, (fv*)((float*)p.D + row + n));
        } else {
          typedef _Float16 hv __attribute__((ext_vector_type(RN)));
          hv y;
#pragma unroll
          for (int j = 0; j < RN; ++j) y[j] = (_Float16)x[j];
          __builtin_nontemporal_store(y, (hv*)((_Float16*)p.D + row + n));
        }
      } else {
#pragma unroll
        for (int j = 0; j < RN; ++j) {
          if (n + j >= p.N2) continue;
          if constexpr (DK == 2)
            ((float*)p.D)[row + n + j] = x[j];
          else
            ((_Float16*)p.D)[row + n + j] = (_Float16)x[j];
        }
      }
    }
  if constexpr (TIMED) {
    const unsigned t_end = now();
    if (blockIdx.x < kStampBlocks) {
      unsigned* out = p.stamps + (blockIdx.x * kStampWaves + w) * kStampsPerWave;
      if (lane < kStampIters)
#pragma unroll
        for (int k = 0; k < 4; ++k) out[4 * lane + k] = tv[k];
      if (lane == 0) {
        out[4 * kStampIters] = t_start;
        out[4 * kStampIters + 1] = t_loop;
        out[4 * kStampIters + 2] = t_end;
      }
    }
  }
}

// host: kernel symbol for K, the D type (1 fp16, 2 fp32), the staging
// (direct-to-LDS or through registers) and the N2 tile width; nullptr if none
const void* chain_symbol(int kd, int dk, bool dma, int bn);
// the timed probe instance (K = 128, fp16 D, direct-to-LDS, 128-column tiles)
const void* chain_timed_symbol();

}  // namespace mfl

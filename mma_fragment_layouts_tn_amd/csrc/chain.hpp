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
// (converted to fp16); the sum over N1 does not care about order, so W's
// N1 axis takes the same permutation pi: K position p = 16 kc + 8 h + v of
// the second MMA is N1 column pi(p) of the first accumulator.  pi is derived
// below from the two atom TV layouts and checked at compile time; W is stored
// in LDS in pi order, so every lane reads its 8 values with one 16-byte read.
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
};

// ---------------------------------------------------------------- the pi map
// K position p (0..31) of the second MMA over one 32-wide N1 chunk -> N1
// column: lane l, chunk kc, value v of the operand (row atom_ab(l).row, k =
// 16 kc + atom_ab(l).k + v) takes accumulator value 8 kc + v of the same lane,
// which sits at (row n1, column m) = atom_c(l, 8 kc + v) of the transposed
// first product.  Requires: the accumulator's column is the operand's row (so
// the values stay in their lane), and every lane with the same k agrees on
// the N1 column (pi is a function of p) and pi is a bijection.
struct ChainPerm {
  int n1[32];     // pi
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

// runs of 4 consecutive N1 columns stay together under pi, so an 8-element
// global chunk is stored as two 8-byte pieces
MFL_HD constexpr bool chain_runs_of_4() {
  const ChainPerm r = chain_k_perm();
  for (int n = 0; n < 32; ++n)
    if (r.pos[n] != r.pos[n - n % 4] + n % 4 || r.pos[n - n % 4] % 4 != 0) return false;
  return true;
}

static_assert(chain_k_perm().ok, "the accumulator must read as the next operand");
static_assert(chain_runs_of_4(), "pi must keep runs of 4 N1 columns");

// ------------------------------------------------------------------ kernel
// Workgroup: 4 waves, 256 rows of M (64 per wave, RM = 2 atom rows) x 128
// columns of N2 (RN = 4 atom columns, N-permuted: repeat j of atom column c
// is column 4 c + j, so D leaves in 4-element vectors).  N1 is consumed in
// 32-wide chunks; the B chunk (32 x KD) and W chunk (128 x 32, pi order)
// of chunk c+1 are loaded into registers while chunk c computes and written
// to the other LDS stage.
namespace chain {
constexpr int BM = 256, BN = 128, RM = 2, RN = 4, WAVES = 4, THREADS = 256;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

// B chunk tile: 32 rows x KD halves, 16-byte chunks XOR-swizzled as the GEMM
// tiles (16 consecutive rows at one chunk land on distinct bank groups)
template <int KD>
__device__ __forceinline__ int b_off(int row, int k) {
  constexpr int CH = KD / 8;
  const int s = CH >= 16 ? (row & 15) : swz<CH>(row);
  return row * KD + (((k >> 3) ^ s) << 3) + (k & 7);
}

// W chunk tile: 128 rows x 32 halves (positions p in pi order), the four
// 16-byte chunks of a row XOR-swizzled by (row >> 2) & 3
__device__ __forceinline__ int w_off(int row, int p) {
  return row * 32 + (((p >> 3) ^ ((row >> 2) & 3)) << 3) + (p & 7);
}

__device__ __forceinline__ uint4 load16(const _Float16* p) {
  uint4 v;
  __builtin_memcpy(&v, p, 16);
  return v;
}

__device__ __forceinline__ uint4 load8_valid(const _Float16* p, int valid) {
  if (valid >= 8) return load16(p);
  union {
    uint4 u;
    _Float16 h[8];
  } r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r.h[e] = e < valid ? p[e] : (_Float16)0.0f;
  return r.u;
}
}  // namespace chain

template <int KD, int DK>
__global__ void __launch_bounds__(chain::THREADS, 1) gemm_chain(const ChainParams p) {
  using namespace chain;
  static_assert(KD == 32 || KD == 64 || KD == 128 || KD == 256, "K is 32, 64, 128 or 256");
  constexpr int KSUB = KD / 16;
  constexpr int BSTAGE = 32 * KD, WSTAGE = BN * 32, STAGE = BSTAGE + WSTAGE;   // halves
  constexpr int BCH = 32 * KD / 8, WCH = BN * 4;                              // 16-byte chunks
  constexpr int BPT = (BCH + THREADS - 1) / THREADS, WPT = WCH / THREADS;     // per thread
  static_assert(WCH % THREADS == 0, "W chunk divides over the threads");
  __shared__ __attribute__((aligned(1024))) _Float16 smem[2 * STAGE];
  constexpr ChainPerm kPi = chain_k_perm();
  // pi^-1 at a run start n (a multiple of 4): a select over the table's
  // compile-time entries, no indexed memory
  auto pi_pos = [&](int n) {
    int r = kPi.pos[0];
#pragma unroll
    for (int e = 4; e < 32; e += 4)
      if (n == e) r = kPi.pos[e];
    return r;
  };

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const TileIndex ti = tile_of_block(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m);
  const int mt_per_b = (p.M + BM - 1) / BM;
  const int b = ti.tm / mt_per_b;
  const int m0 = (ti.tm % mt_per_b) * BM, n0 = ti.tn * BN;
  const _Float16* A = (const _Float16*)p.A + (int64_t)b * p.sa;
  const _Float16* B = (const _Float16*)p.B + (int64_t)b * p.sb;
  const _Float16* Wm = (const _Float16*)p.W + (int64_t)b * p.sw;

  // this wave's A rows as the second operand of the first product:
  // fragment (i, kk) of lane l: row m0 + 64 w + 32 i + l % 32, k = 16 kk + 8 (l / 32)
  const RowK al = atom_ab_coord(lane);
  half8 af[RM][KSUB];
#pragma unroll
  for (int i = 0; i < RM; ++i) {
    const int m = min(m0 + 64 * w + 32 * i + al.row, p.M - 1);
#pragma unroll
    for (int kk = 0; kk < KSUB; ++kk) {
      const uint4 u = load16(A + (int64_t)m * p.lda + 16 * kk + al.k);
      __builtin_memcpy(&af[i][kk], &u, 16);
    }
  }

  // staging: thread's 16-byte chunks of the B chunk (row r, k chunk q) and of
  // the W chunk (LDS row r = 32 j + c holds N2 column n0 + 4 c + j; N1 piece q)
  uint4 rb[BPT], rw[WPT];
  auto load_chunk = [&](int c) {
    const int n1b = 32 * c;
#pragma unroll
    for (int t = 0; t < BPT; ++t) {
      const int q = tid + t * THREADS;
      if (q < BCH) {
        const int row = q / (KD / 8), kq = q % (KD / 8);
        const int n1 = n1b + row;
        rb[t] = n1 < p.N1 ? load16(B + (int64_t)n1 * p.ldb + 8 * kq) : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int t = 0; t < WPT; ++t) {
      const int q = tid + t * THREADS, row = q / 4, kq = q % 4;
      const int n2 = min(n0 + RN * (row % 32) + row / 32, p.N2 - 1);
      const int n1 = n1b + 8 * kq;
      rw[t] = n1 < p.N1 ? load8_valid(Wm + (int64_t)n2 * p.ldw + n1, p.N1 - n1)
                        : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_chunk = [&](int s) {
    _Float16* sb = smem + s * STAGE;
    _Float16* sw = sb + BSTAGE;
#pragma unroll
    for (int t = 0; t < BPT; ++t) {
      const int q = tid + t * THREADS;
      if (q < BCH) {
        const int row = q / (KD / 8), kq = q % (KD / 8);
        *(uint4*)&sb[b_off<KD>(row, 8 * kq)] = rb[t];
      }
    }
#pragma unroll
    for (int t = 0; t < WPT; ++t) {
      const int q = tid + t * THREADS, row = q / 4, kq = q % 4;
      // N1 columns 8 kq .. 8 kq + 3 and 8 kq + 4 .. + 7 go to their pi positions
      *(uint2*)&sw[w_off(row, pi_pos(8 * kq))] = make_uint2(rw[t].x, rw[t].y);
      *(uint2*)&sw[w_off(row, pi_pos(8 * kq + 4))] = make_uint2(rw[t].z, rw[t].w);
    }
  };

  floatx16 acc[RM][RN];
#pragma unroll
  for (int i = 0; i < RM; ++i)
#pragma unroll
    for (int j = 0; j < RN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int nch = (p.N1 + 31) / 32;
  if (nch > 0) {
    load_chunk(0);
    store_chunk(0);
    if (nch > 1) load_chunk(1);
  }
  __syncthreads();
  for (int c = 0; c < nch; ++c) {
    const int s = c & 1;
    const _Float16* sb = smem + s * STAGE;
    const _Float16* sw = sb + BSTAGE;
    // first product, transposed: S^T (32 N1 x 32 M per atom row i)
    floatx16 st[RM];
#pragma unroll
    for (int i = 0; i < RM; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) st[i][v] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < KSUB; ++kk) {
      const half8 bf = *(const half8*)&sb[b_off<KD>(al.row, 16 * kk + al.k)];
#pragma unroll
      for (int i = 0; i < RM; ++i)
        st[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf, af[i][kk], st[i], 0, 0, 0);
    }
    // the accumulator, rounded once to fp16, is the next operand: values
    // 8 kc .. 8 kc + 7 are K chunk kc (pi order)
    half8 pf[RM][2];
#pragma unroll
    for (int i = 0; i < RM; ++i)
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          const float x = st[i][8 * kc + v];
          pf[i][kc][v] = (_Float16)x;   // RNE
        }
    // second product: D += P W^T over this chunk's 32 N1 columns
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      half8 wf[RN];
#pragma unroll
      for (int j = 0; j < RN; ++j)
        wf[j] = *(const half8*)&sw[w_off(32 * j + al.row, 16 * kc + al.k)];
#pragma unroll
      for (int i = 0; i < RM; ++i)
#pragma unroll
        for (int j = 0; j < RN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(pf[i][kc], wf[j], acc[i][j], 0, 0, 0);
    }
    if (c + 1 < nch) store_chunk(s ^ 1);   // stage s^1 was last read before the previous barrier
    if (c + 2 < nch) load_chunk(c + 2);
    __syncthreads();
  }

  // epilogue: acc[i][j][v] of lane l is D(m0 + 64 w + 32 i + atom_c(l, v).row,
  // n0 + 4 (l % 32) + j): one 4-element vector per (i, v)
  const RowK cl = atom_c_coord(lane, 0);
#pragma unroll
  for (int i = 0; i < RM; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = m0 + 64 * w + 32 * i + atom_c_coord(lane, v).row;
      const int n = n0 + RN * cl.k;
      if (m >= p.M) continue;
      float x[RN];
#pragma unroll
      for (int j = 0; j < RN; ++j) x[j] = acc[i][j][v];
      const int64_t row = (int64_t)b * p.sd + (int64_t)m * p.ldd;
      if (p.d_vec && n + RN <= p.N2) {
        if constexpr (DK == 2) {
          typedef float f4 __attribute__((ext_vector_type(4)));
          const f4 y = {x[0], x[1], x[2], x[3]};
          __builtin_nontemporal_store(y, (f4*)((float*)p.D + row + n));
        } else {
          typedef _Float16 h4 __attribute__((ext_vector_type(4)));
          const h4 y = {(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3]};
          __builtin_nontemporal_store(y, (h4*)((_Float16*)p.D + row + n));
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
}

// host: kernel symbol for K and the D type (1 fp16, 2 fp32); nullptr if none
const void* chain_symbol(int kd, int dk);

}  // namespace mfl

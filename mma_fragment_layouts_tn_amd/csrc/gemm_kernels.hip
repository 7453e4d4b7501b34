// gfx950 kernels for D = C + A * B^T with fp16 A (M,K), B (N,K).
//
// Two kernel families (structure in gemm_tile.hpp):
//  * gemm_lds: block tile staged through LDS, double-buffered.  Each K-step
//    every thread fetches its share of the next A and B tiles from global
//    memory into registers (16-byte loads) while the waves run the MFMA
//    K-loop on the current LDS buffer; the fetched chunks are then written to
//    the other buffer and one barrier closes the step.  This is the
//    shared-memory GEMM the simple-GEMM page names as the faster successor of
//    its global-only kernel ("cute(7) simple_gemm" §10), with the block tile
//    and shared-memory layout choices of "CuTe Layout 到 Tensor Core" §4-5.
//  * gemm_direct: the global-only kernel of the simple-GEMM page (§1, §3.4):
//    every lane reads its operand fragments straight from global memory into
//    registers, no LDS at all.
// Both accumulate in fp32 with v_mfma_f32_32x32x16_f16 and finish with the
// epilogue D = acc + C, rounded once to fp16 (nearest even) when D is fp16.
//
// Edges (partial tiles, which the TiledMMA page leaves to the caller,
// section "打印布局，核对一次"): operand rows past M or N are clamped to the
// last row (they only feed outputs that are never stored); K past the end is
// zero in BOTH operands (0 * Inf would be NaN); stores are predicated.
#include <hip/hip_runtime.h>

#include "gemm_launch.hpp"
#include "gemm_tile.hpp"

namespace mfl {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

// 16-byte global load at any 2-byte alignment (gfx9 runs in unaligned access
// mode, so this is one global_load_dwordx4 either way).
__device__ __forceinline__ uint4 load16(const char* base, int64_t byte_off) {
  uint4 v;
  __builtin_memcpy(&v, base + byte_off, 16);
  return v;
}

// 8 consecutive elements (row-contiguous run) starting at element `e0` of a
// run whose valid length is `valid` (elements >= valid read as zero).
__device__ __forceinline__ uint4 load8_tail(const _Float16* p, int valid) {
  union {
    uint4 u;
    _Float16 h[8];
  } r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r.h[e] = e < valid ? p[e] : (_Float16)0.0f;
  return r.u;
}

__device__ __forceinline__ half8 as_half8(uint4 u) {
  half8 h;
  __builtin_memcpy(&h, &u, 16);
  return h;
}

template <int CK>
__device__ __forceinline__ float c_value(const GemmParams& p, int m, int n) {
  if constexpr (CK == 1) return (float)((const _Float16*)p.C)[(int64_t)m * p.ldc + n];
  if constexpr (CK == 2) return ((const float*)p.C)[(int64_t)m * p.ldc + n];
  return 0.0f;
}

template <int DK>
__device__ __forceinline__ void d_store(const GemmParams& p, int m, int n, float x) {
  if constexpr (DK == 1)
    ((_Float16*)p.D)[(int64_t)m * p.ldd + n] = (_Float16)x;   // v_cvt_f16_f32, RNE
  else
    ((float*)p.D)[(int64_t)m * p.ldd + n] = x;
}

// Epilogue shared by both kernels: acc[i][j] value v -> (m, n) from the
// accumulator TV layout.
template <class Cfg, int CK, int DK>
__device__ __forceinline__ void epilogue(const GemmParams& p, int w, int lane, int m0,
                                         int n0, const floatx16 (&acc)[Cfg::RM][Cfg::RN]) {
#pragma unroll
  for (int i = 0; i < Cfg::RM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::RN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const RowK c = frag_c_coord<Cfg>(w, lane, i, j, v);
        const int m = m0 + c.row, n = n0 + c.k;
        if (m < p.M && n < p.N) d_store<DK>(p, m, n, acc[i][j][v] + c_value<CK>(p, m, n));
      }
}

// ---------------------------------------------------------------------------
// LDS-staged kernel
// ---------------------------------------------------------------------------
template <class Cfg, bool A_MMAJOR, int CK, int DK>
__global__ void __launch_bounds__(Cfg::kThreads, 1) gemm_lds(const GemmParams p) {
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, CH = Cfg::CH;
  constexpr int T = Cfg::kThreads;
  constexpr int LA = BM * CH / T, LB = BN * CH / T;
  __shared__ __attribute__((aligned(16))) _Float16 sA[2][Cfg::kLdsA];
  __shared__ __attribute__((aligned(16))) _Float16 sB[2][Cfg::kLdsB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const TileIndex ti = tile_of_block(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m);
  const int m0 = ti.tm * BM, n0 = ti.tn * BN;
  const char* Ab = (const char*)p.A;
  const char* Bb = (const char*)p.B;

  // Per-thread staging chunks: chunk q = tid + i*T of the operand tile.
  // K-major: row = q / CH, 16-byte chunk c = q % CH.
  // M-major A: k-row kr = q / (BM/8), 8-element m-run mc = q % (BM/8).
  int a_off[LA], a_lds[LA], a_aux[LA];
  int b_off[LB], b_lds[LB], b_aux[LB];
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int q = tid + i * T;
    if constexpr (!A_MMAJOR) {
      const int row = q / CH, c = q % CH;
      const int gm = min(m0 + row, p.M - 1);
      a_off[i] = (int)((int64_t)gm * p.lda * 2) + c * 16;
      a_lds[i] = lds_offset<BK>(row, c * 8);
      a_aux[i] = c * 8;                         // k offset of the chunk in the tile
    } else {
      const int kr = q / (BM / 8), mc = q % (BM / 8);
      a_off[i] = (int)((int64_t)kr * p.lda * 2) + (m0 + mc * 8) * 2;
      a_lds[i] = kr | (mc << 16);               // unpacked at store time
      a_aux[i] = kr;
    }
  }
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    const int q = tid + i * T;
    const int row = q / CH, c = q % CH;
    const int gn = min(n0 + row, p.N - 1);
    b_off[i] = (int)((int64_t)gn * p.ldb * 2) + c * 16;
    b_lds[i] = lds_offset<BK>(row, c * 8);
    b_aux[i] = c * 8;
  }

  uint4 ra[LA], rb[LB];
  auto fetch = [&](int kt) {
    const int k0 = kt * BK;
    const bool tail = k0 + BK > p.K;
    if constexpr (!A_MMAJOR) {
      const int64_t step = (int64_t)k0 * 2;
#pragma unroll
      for (int i = 0; i < LA; ++i) {
        if (!tail) {
          ra[i] = load16(Ab, a_off[i] + step);
        } else {
          const int valid = p.K - (k0 + a_aux[i]);
          ra[i] = valid >= 8 ? load16(Ab, a_off[i] + step)
                  : valid <= 0 ? make_uint4(0, 0, 0, 0)
                               : load8_tail((const _Float16*)(Ab + a_off[i] + step), valid);
        }
      }
    } else {
      const int64_t step = (int64_t)k0 * p.lda * 2;
#pragma unroll
      for (int i = 0; i < LA; ++i) {
        const int kr = a_aux[i];
        const int mrun = m0 + (a_lds[i] >> 16) * 8;
        const bool kvalid = k0 + kr < p.K;
        const int mvalid = p.M - mrun;
        if (kvalid && mvalid >= 8)
          ra[i] = load16(Ab, a_off[i] + step);
        else if (!kvalid || mvalid <= 0)
          ra[i] = make_uint4(0, 0, 0, 0);
        else
          ra[i] = load8_tail((const _Float16*)(Ab + a_off[i] + step), mvalid);
      }
    }
    const int64_t stepb = (int64_t)k0 * 2;
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      if (!tail) {
        rb[i] = load16(Bb, b_off[i] + stepb);
      } else {
        const int valid = p.K - (k0 + b_aux[i]);
        rb[i] = valid >= 8 ? load16(Bb, b_off[i] + stepb)
                : valid <= 0 ? make_uint4(0, 0, 0, 0)
                             : load8_tail((const _Float16*)(Bb + b_off[i] + stepb), valid);
      }
    }
  };
  auto stash = [&](int st) {
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      if constexpr (!A_MMAJOR) {
        *(uint4*)&sA[st][a_lds[i]] = ra[i];
      } else {
        // transpose on the way in: 8 m values of one k go to 8 LDS rows
        const int kr = a_lds[i] & 0xffff, mc = a_lds[i] >> 16;
        union {
          uint4 u;
          _Float16 h[8];
        } x;
        x.u = ra[i];
#pragma unroll
        for (int e = 0; e < 8; ++e) sA[st][lds_offset<BK>(mc * 8 + e, kr)] = x.h[e];
      }
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) *(uint4*)&sB[st][b_lds[i]] = rb[i];
  };

  floatx16 acc[Cfg::RM][Cfg::RN];
#pragma unroll
  for (int i = 0; i < Cfg::RM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::RN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int nk = (p.K + BK - 1) / BK;
  if (nk > 0) {
    fetch(0);
    stash(0);
    __syncthreads();
  }
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) fetch(kt + 1);
#pragma unroll
    for (int kk = 0; kk < Cfg::KSUB; ++kk) {
      half8 af[Cfg::RM], bf[Cfg::RN];
#pragma unroll
      for (int i = 0; i < Cfg::RM; ++i) {
        const RowK a = frag_a_coord<Cfg>(w, lane, i, kk);
        af[i] = *(const half8*)&sA[cur][lds_offset<BK>(a.row, a.k)];
      }
#pragma unroll
      for (int j = 0; j < Cfg::RN; ++j) {
        const RowK b = frag_b_coord<Cfg>(w, lane, j, kk);
        bf[j] = *(const half8*)&sB[cur][lds_offset<BK>(b.row, b.k)];
      }
#pragma unroll
      for (int i = 0; i < Cfg::RM; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::RN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) stash(cur ^ 1);
    __syncthreads();
  }
  epilogue<Cfg, CK, DK>(p, w, lane, m0, n0, acc);
}

// ---------------------------------------------------------------------------
// LDS-staged kernel, direct-to-LDS fetch (K-contiguous, 16-byte aligned rows)
// ---------------------------------------------------------------------------
// Same tile structure as gemm_lds, different pipeline:
//  * operand tiles go global -> LDS with global_load_lds_dwordx4: lane l of
//    a wave writes LDS bytes [16 l, 16 l + 16) of a 1 KB run (8 rows of
//    BK=64 halves), so the XOR swizzle is applied by choosing which 16-byte
//    chunk of its row each lane fetches;
//  * the fetch of tile kt+2 is issued right after the barrier of step kt and
//    has a whole step to land; each step has one barrier, placed after the
//    third K sub-step so the fragment reads for the next stage and the
//    barrier wait overlap the MFMAs still queued;
//  * fragments are double-buffered across K sub-steps;
//  * a K remainder (K % BK) is staged once through registers with zero fill.
using lds_ptr_t = __attribute__((address_space(3))) void*;

template <class Cfg>
struct DmaPlan {
  // per wave: A and B runs of 8 rows each
  static constexpr int kRunsA = Cfg::BM / 8 / Cfg::kWaves;
  static constexpr int kRunsB = Cfg::BN / 8 / Cfg::kWaves;
  static_assert(Cfg::BK == 64, "one 1 KB run = 8 rows of 64 halves");
  static_assert(Cfg::BM % (8 * Cfg::kWaves) == 0 && Cfg::BN % (8 * Cfg::kWaves) == 0, "runs");
};

template <class Cfg, int CK, int DK>
__global__ void __launch_bounds__(Cfg::kThreads, 1) gemm_dma(const GemmParams p) {
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK;
  constexpr int RA = DmaPlan<Cfg>::kRunsA, RB = DmaPlan<Cfg>::kRunsB;
  constexpr int RM = Cfg::RM, RN = Cfg::RN, KSUB = Cfg::KSUB;
  static_assert(KSUB == 4, "the schedule below is written for 4 K sub-steps");
  // stage s: A at smem + s*kStage, B at smem + s*kStage + BM*BK (halves)
  constexpr int kStage = (BM + BN) * BK;
  __shared__ __attribute__((aligned(1024))) _Float16 smem[2 * kStage];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const TileIndex ti = tile_of_block(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m);
  const int m0 = ti.tm * BM, n0 = ti.tn * BN;

  // lane's 16-byte chunk within its 8-row run: row r = 8*run + lane/8 holds
  // physical chunk lane%8, i.e. logical chunk (lane%8) ^ swz(r)
  const int rsub = lane >> 3;
  unsigned a_off[RA], b_off[RB];
#pragma unroll
  for (int i = 0; i < RA; ++i) {
    const int row = 8 * (w * RA + i) + rsub;
    const int kchunk = ((lane & 7) ^ swz<Cfg::CH>(row)) * 8;
    a_off[i] = (unsigned)((int64_t)min(m0 + row, p.M - 1) * p.lda * 2) + kchunk * 2;
  }
#pragma unroll
  for (int i = 0; i < RB; ++i) {
    const int row = 8 * (w * RB + i) + rsub;
    const int kchunk = ((lane & 7) ^ swz<Cfg::CH>(row)) * 8;
    b_off[i] = (unsigned)((int64_t)min(n0 + row, p.N - 1) * p.ldb * 2) + kchunk * 2;
  }

  auto dma = [&](int kt, int stage) {
    const char* a = (const char*)p.A + (int64_t)kt * BK * 2;
    const char* b = (const char*)p.B + (int64_t)kt * BK * 2;
    _Float16* sa = smem + stage * kStage;
    _Float16* sb = sa + BM * BK;
#pragma unroll
    for (int i = 0; i < RA; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(a + (uint64_t)a_off[i]),
                                       (lds_ptr_t)(sa + (w * RA + i) * 8 * BK), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < RB; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(b + (uint64_t)b_off[i]),
                                       (lds_ptr_t)(sb + (w * RB + i) * 8 * BK), 16, 0, 0);
  };

  // fragment read offsets within a stage (halves), per K sub-step
  int fa_off[KSUB][RM], fb_off[KSUB][RN];
#pragma unroll
  for (int kk = 0; kk < KSUB; ++kk) {
#pragma unroll
    for (int i = 0; i < RM; ++i) {
      const RowK a = frag_a_coord<Cfg>(w, lane, i, kk);
      fa_off[kk][i] = lds_offset<BK>(a.row, a.k);
    }
#pragma unroll
    for (int j = 0; j < RN; ++j) {
      const RowK b = frag_b_coord<Cfg>(w, lane, j, kk);
      fb_off[kk][j] = BM * BK + lds_offset<BK>(b.row, b.k);
    }
  }

  half8 fa[2][RM], fb[2][RN];
  auto frags = [&](int buf, int kk, int stage) {
    const _Float16* st = smem + stage * kStage;
#pragma unroll
    for (int i = 0; i < RM; ++i) fa[buf][i] = *(const half8*)&st[fa_off[kk][i]];
#pragma unroll
    for (int j = 0; j < RN; ++j) fb[buf][j] = *(const half8*)&st[fb_off[kk][j]];
  };

  floatx16 acc[RM][RN];
#pragma unroll
  for (int i = 0; i < RM; ++i)
#pragma unroll
    for (int j = 0; j < RN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  auto mma = [&](int buf) {
#pragma unroll
    for (int i = 0; i < RM; ++i)
#pragma unroll
      for (int j = 0; j < RN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[buf][i], fb[buf][j], acc[i][j], 0, 0, 0);
  };
  // interleave: the group's fragment reads spread between its MFMAs
  constexpr int kReads = RM + RN, kMfma = RM * RN;
  auto interleave = [&]() {
#pragma unroll
    for (int g = 0; g < kReads; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, kMfma / kReads > 0 ? kMfma / kReads : 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kMfma, 0);
  };

  const int nfull = p.K / BK;
  if (nfull > 0) {
    dma(0, 0);
    if (nfull > 1) dma(1, 1);
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    frags(0, 0, 0);
  }
  for (int kt = 0; kt < nfull; ++kt) {
    const int cur = kt & 1;
    frags(1, 1, cur);
    mma(0);
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    frags(0, 2, cur);
    mma(1);
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    frags(1, 3, cur);
    mma(0);
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0);        // own reads of this stage and DMA of tile kt+1 done
    __builtin_amdgcn_s_barrier();         // ... in every wave: this stage is free, next is full
    __builtin_amdgcn_sched_barrier(0);
    if (kt + 2 < nfull) dma(kt + 2, cur);
    if (kt + 1 < nfull) frags(0, 0, cur ^ 1);
    mma(1);
    __builtin_amdgcn_sched_barrier(0);
  }

  // K remainder: one step staged through registers with zero fill
  if (p.K % BK != 0) {
    const int k0 = nfull * BK;
    _Float16* sA0 = smem;
    _Float16* sB0 = smem + BM * BK;
    __syncthreads();
    constexpr int T = Cfg::kThreads, CH = Cfg::CH;
#pragma unroll
    for (int i = 0; i < BM * CH / T; ++i) {
      const int q = tid + i * T, row = q / CH, c = q % CH;
      const int gm = min(m0 + row, p.M - 1);
      const _Float16* src = (const _Float16*)p.A + (int64_t)gm * p.lda + k0 + c * 8;
      const int valid = p.K - (k0 + c * 8);
      *(uint4*)&sA0[lds_offset<BK>(row, c * 8)] =
          valid >= 8 ? load16((const char*)src, 0)
                     : valid <= 0 ? make_uint4(0, 0, 0, 0) : load8_tail(src, valid);
    }
#pragma unroll
    for (int i = 0; i < BN * CH / T; ++i) {
      const int q = tid + i * T, row = q / CH, c = q % CH;
      const int gn = min(n0 + row, p.N - 1);
      const _Float16* src = (const _Float16*)p.B + (int64_t)gn * p.ldb + k0 + c * 8;
      const int valid = p.K - (k0 + c * 8);
      *(uint4*)&sB0[lds_offset<BK>(row, c * 8)] =
          valid >= 8 ? load16((const char*)src, 0)
                     : valid <= 0 ? make_uint4(0, 0, 0, 0) : load8_tail(src, valid);
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < KSUB; ++kk) {
      frags(0, kk, 0);
      mma(0);
    }
  }
  epilogue<Cfg, CK, DK>(p, w, lane, m0, n0, acc);
}

// ---------------------------------------------------------------------------
// Direct kernel: fragments from global memory, no LDS
// ---------------------------------------------------------------------------
template <class Cfg, int CK, int DK>
__global__ void __launch_bounds__(Cfg::kThreads, 1) gemm_direct(const GemmParams p) {
  constexpr int BK = Cfg::BK;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const TileIndex ti = tile_of_block(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m);
  const int m0 = ti.tm * Cfg::BM, n0 = ti.tn * Cfg::BN;
  const _Float16* A = (const _Float16*)p.A;
  const _Float16* B = (const _Float16*)p.B;

  floatx16 acc[Cfg::RM][Cfg::RN];
#pragma unroll
  for (int i = 0; i < Cfg::RM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::RN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int nk = (p.K + BK - 1) / BK;
  for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
    for (int kk = 0; kk < Cfg::KSUB; ++kk) {
      half8 af[Cfg::RM], bf[Cfg::RN];
#pragma unroll
      for (int i = 0; i < Cfg::RM; ++i) {
        const RowK a = frag_a_coord<Cfg>(w, lane, i, kk);
        const int m = min(m0 + a.row, p.M - 1);
        const int k = kt * BK + a.k;
        const _Float16* src = A + (int64_t)m * p.lda + k;
        const int valid = p.K - k;
        af[i] = as_half8(valid >= 8 ? load16((const char*)src, 0)
                         : valid <= 0 ? make_uint4(0, 0, 0, 0)
                                      : load8_tail(src, valid));
      }
#pragma unroll
      for (int j = 0; j < Cfg::RN; ++j) {
        const RowK b = frag_b_coord<Cfg>(w, lane, j, kk);
        const int n = min(n0 + b.row, p.N - 1);
        const int k = kt * BK + b.k;
        const _Float16* src = B + (int64_t)n * p.ldb + k;
        const int valid = p.K - k;
        bf[j] = as_half8(valid >= 8 ? load16((const char*)src, 0)
                         : valid <= 0 ? make_uint4(0, 0, 0, 0)
                                      : load8_tail(src, valid));
      }
#pragma unroll
      for (int i = 0; i < Cfg::RM; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::RN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  }
  epilogue<Cfg, CK, DK>(p, w, lane, m0, n0, acc);
}

// ---------------------------------------------------------------------------
// instantiation tables
// ---------------------------------------------------------------------------
using KernelFn = void (*)(const GemmParams);

// [a_mmajor][c_kind][d_kind-1]
template <class Cfg>
constexpr KernelFn lds_table[2][3][2] = {
    {{gemm_lds<Cfg, false, 0, 1>, gemm_lds<Cfg, false, 0, 2>},
     {gemm_lds<Cfg, false, 1, 1>, gemm_lds<Cfg, false, 1, 2>},
     {gemm_lds<Cfg, false, 2, 1>, gemm_lds<Cfg, false, 2, 2>}},
    {{gemm_lds<Cfg, true, 0, 1>, gemm_lds<Cfg, true, 0, 2>},
     {gemm_lds<Cfg, true, 1, 1>, gemm_lds<Cfg, true, 1, 2>},
     {gemm_lds<Cfg, true, 2, 1>, gemm_lds<Cfg, true, 2, 2>}}};

template <class Cfg>
constexpr KernelFn direct_table[3][2] = {
    {gemm_direct<Cfg, 0, 1>, gemm_direct<Cfg, 0, 2>},
    {gemm_direct<Cfg, 1, 1>, gemm_direct<Cfg, 1, 2>},
    {gemm_direct<Cfg, 2, 1>, gemm_direct<Cfg, 2, 2>}};

template <class Cfg>
constexpr KernelFn dma_table[3][2] = {
    {gemm_dma<Cfg, 0, 1>, gemm_dma<Cfg, 0, 2>},
    {gemm_dma<Cfg, 1, 1>, gemm_dma<Cfg, 1, 2>},
    {gemm_dma<Cfg, 2, 1>, gemm_dma<Cfg, 2, 2>}};

template <class Cfg>
KernelInfo info_of(int algo) {
  return KernelInfo{algo, Cfg::BM, Cfg::BN, Cfg::BK, Cfg::kThreads};
}

}  // namespace

KernelInfo kernel_info(int algo) {
  switch (algo) {
    case kAlgoDirect: return info_of<CfgDirect>(algo);
    case kAlgoLds128: return info_of<CfgLds128>(algo);
    case kAlgoLds256: return info_of<CfgLds256>(algo);
    case kAlgoDma256: return info_of<CfgDma256>(algo);
    case kAlgoDma256W8: return info_of<CfgDma256W8>(algo);
    default: return KernelInfo{-1, 0, 0, 0, 0};
  }
}

const void* kernel_symbol(int algo, bool a_mmajor, int c_kind, int d_kind) {
  if (c_kind < 0 || c_kind > 2 || d_kind < 1 || d_kind > 2) return nullptr;
  switch (algo) {
    case kAlgoDirect:
      return a_mmajor ? nullptr : (const void*)direct_table<CfgDirect>[c_kind][d_kind - 1];
    case kAlgoLds128: return (const void*)lds_table<CfgLds128>[a_mmajor][c_kind][d_kind - 1];
    case kAlgoLds256: return (const void*)lds_table<CfgLds256>[a_mmajor][c_kind][d_kind - 1];
    case kAlgoDma256:
      return a_mmajor ? nullptr : (const void*)dma_table<CfgDma256>[c_kind][d_kind - 1];
    case kAlgoDma256W8:
      return a_mmajor ? nullptr : (const void*)dma_table<CfgDma256W8>[c_kind][d_kind - 1];
    default: return nullptr;
  }
}

int launch_gemm(int algo, bool a_mmajor, int c_kind, int d_kind, const GemmParams& p,
                hipStream_t stream) {
  const void* fn = kernel_symbol(algo, a_mmajor, c_kind, d_kind);
  const KernelInfo ki = kernel_info(algo);
  if (!fn || ki.algo < 0) return -1;
  const int64_t nb = (int64_t)p.tiles_m * p.tiles_n;
  hipLaunchKernelGGL((KernelFn)fn, dim3((unsigned)nb), dim3(ki.threads), 0, stream, p);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // namespace mfl

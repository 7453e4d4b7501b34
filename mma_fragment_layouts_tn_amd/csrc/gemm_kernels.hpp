// gfx950 kernels for D = C + A * B^T with fp16 A (M,K), B (N,K).
//
// Two kernel families (tile structure in gemm_tile.hpp):
//  * gemm_tiled: the block tile is staged through LDS in two stages.  This is
//    the shared-memory GEMM the simple-GEMM page names as the faster
//    successor of its global-only kernel ("cute(7) simple_gemm" §10), with the
//    block tile and shared-memory layout choices of "CuTe Layout 到 Tensor
//    Core" §4-5.  Each operand is fetched by one of three policies:
//      DMA   global_load_lds_dwordx4 straight into LDS (K-contiguous rows,
//            16-byte aligned);
//      REG   16-byte loads into registers (any 2-byte alignment), written to
//            LDS one step later;
//      REGT  M-contiguous A: 4 k-rows x 8 m loaded into registers, transposed
//            in registers to 8 runs of 4 k, written with 8-byte LDS stores;
//      DMAT  M-contiguous A straight into an M-contiguous LDS tile, operand
//            fragments read with the transposing LDS read (ds_read_b64_tr_b16).
//    Per K-step: fragment reads for sub-step kk+1 overlap the MFMAs of kk;
//    register-staged tiles are written to the idle stage during the last
//    sub-step before the step's single barrier; after the barrier the fetch
//    of tile kt+2 (it has a whole step to land) and the first fragment reads
//    of the next stage are interleaved with the last sub-step's MFMAs.
//  * gemm_direct: the global-only kernel of the simple-GEMM page (§1, §3.4):
//    every lane reads its operand fragments straight from global memory into
//    registers, no LDS at all.
// Both accumulate in fp32 with v_mfma_f32_32x32x16_f16 and finish with the
// epilogue D = acc + C, rounded once to fp16 (nearest even) when D is fp16.
//
// Edges (partial tiles, which the TiledMMA page leaves to the caller,
// section "打印布局，核对一次"): operand rows past M or N are clamped to the
// last row (they only feed outputs that are never stored); a K remainder is
// staged once with zero fill in BOTH operands (0 * Inf would be NaN); stores
// are predicated.
#include <hip/hip_runtime.h>

#pragma once

#include "gemm_launch.hpp"
#include "gemm_tile.hpp"

namespace mfl {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
using lds_ptr_t = __attribute__((address_space(3))) void*;

// The matrix instruction of a configuration: acc += A B^T on one atom, with
// one 8-half operand fragment per lane for A and for B.
//  * 32x32x16: the compiler's builtin.
//  * 16x16x32: the instruction with its accumulator tied to one AGPR tuple.
//    With the builtin the compiler does not keep a wave's 64 four-register
//    accumulator tuples in place across the K loop and copies them around
//    every iteration (the sixteen-register tuples of the 32x32 form stay in
//    place).  The compiler cannot see hazards through the tied form: each
//    instruction carries two wait states ahead of it (operands assembled by
//    vector instructions), and mma_begin / mma_end below cover the
//    accumulators' zero fill and the first reads of the results.
template <int OP>
struct Mma;
template <>
struct Mma<kMfma32x32x16> {
  using Acc = floatx16;
  static __device__ __forceinline__ void run(const half8& a, const half8& b, Acc& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};
template <>
struct Mma<kMfma16x16x32> {
  using Acc = floatx4;
  static __device__ __forceinline__ void run(const half8& a, const half8& b, Acc& c) {
    asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_f16 %0, %1, %2, %0"
                 : "+a"(c)
                 : "v"(a), "v"(b));
  }
};
template <class Cfg>
using AccT = typename Mma<Cfg::kOp>::Acc;

template <class Cfg>
__device__ __forceinline__ void zero_acc(AccT<Cfg> (&acc)[Cfg::RM][Cfg::RN]) {
#pragma unroll
  for (int i = 0; i < Cfg::RM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::RN; ++j)
#pragma unroll
      for (int v = 0; v < Cfg::kNV; ++v) acc[i][j][v] = 0.0f;
}

// Before the first matrix instruction: every accumulator holds its zeros
// (the empty statements take each tuple as written), then wait states cover
// the vector writes of those zeros.
template <class Cfg>
__device__ __forceinline__ void mma_begin(AccT<Cfg> (&acc)[Cfg::RM][Cfg::RN]) {
#pragma unroll
  for (int i = 0; i < Cfg::RM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::RN; ++j) asm volatile("" : "+a"(acc[i][j]));
  asm volatile("s_nop 4" ::);
}

// After the last matrix instruction: 24 wait states (more than either
// instruction's latency), then the empty statements, so no read of an
// accumulator can be placed before the results are written.  Needed for the
// tied form, whose hazards the compiler cannot see, and for the builtin as
// well: where the last instructions sit in a conditional block (the K
// remainder) this compiler reads an accumulator in the following block, or
// spills it, with no wait states (measured: a stale value in one register of
// one tile, through the fp32-C epilogue of the one-wave 128x128 kernel).
template <class Cfg>
__device__ __forceinline__ void mma_end(AccT<Cfg> (&acc)[Cfg::RM][Cfg::RN]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::);
#pragma unroll
  for (int i = 0; i < Cfg::RM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::RN; ++j) asm volatile("" : "+a"(acc[i][j]));
}

// 16-byte global load at any 2-byte alignment (gfx9 runs in unaligned access
// mode, so this is one global_load_dwordx4 either way).
__device__ __forceinline__ uint4 load16(const char* base, int64_t byte_off) {
  uint4 v;
  __builtin_memcpy(&v, base + byte_off, 16);
  return v;
}

// 8 consecutive elements of which the first `valid` are read, the rest zero.
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

// The `nt` cache policy (non-temporal) on data the kernel touches once:
// the stores of D, which leaves D out of the L2s and shortens the write-back
// at the end of the kernel (about 1 % at 4096^3), and the C rows fetched
// straight into LDS (whole 1 KB runs per instruction), which leaves the L2s
// to the operand tiles that other workgroups read again (8192^2 x 2048 with
// an fp32 C: 4-5 % faster).  Per-lane C vectors keep the default policy:
// there a cache line is shared by neighbouring instructions, and with nt the
// aligned fp16 C case ran 3.5 % slower, the ragged one 9 %.  A and B keep it
// too: with nt on their fetch the 4096^3 kernel takes 121 us against 101.
constexpr int kNt = 2;   // cache-policy operand of the buffer and direct-to-LDS builtins: nt

template <int DK>
__device__ __forceinline__ void d_store(const GemmParams& p, int m, int n, float x) {
  if constexpr (DK == 1)
    __builtin_nontemporal_store((_Float16)x, (_Float16*)p.D + (int64_t)m * p.ldd + n);   // RNE
  else
    __builtin_nontemporal_store(x, (float*)p.D + (int64_t)m * p.ldd + n);
}

// Register epilogue.  The N permutation gives each lane, for a row block i
// and value v, its RN accumulators acc[i][0..RN-1][v] on RN adjacent columns
// of one row: one RN-element vector of D per (i, v), and for a fixed (i, v)
// the 64 lanes cover two rows of 32*RN consecutive columns.  Interior tiles
// with vector-aligned D (and C) go through buffer descriptors based at the
// wave's tile origin: the lane part of the accumulator layout is one per-lane
// offset and the row part of (i, v) a uniform scalar offset, so there is no
// vector address arithmetic and no per-element branch; C's 16 vectors of a
// row block are loaded before any of them is used.  Other tiles address each
// vector and fall back to elements where a vector would cross the right edge
// or the rows are not vector-aligned.  Only the row blocks own(i) accepts
// are written.
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

struct AllRows {
  __device__ bool operator()(int) const { return true; }
};

__device__ __forceinline__ unsigned pack_half2(float a, float b) {   // RNE
  return (unsigned)__builtin_bit_cast(unsigned short, (_Float16)a) |
         ((unsigned)__builtin_bit_cast(unsigned short, (_Float16)b) << 16);
}

__device__ __forceinline__ float half_lo(unsigned u) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(u & 0xffffu));
}
__device__ __forceinline__ float half_hi(unsigned u) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(u >> 16));
}

// RN values -> one D vector through a buffer descriptor (kNt: D is
// written once and not read back by this kernel)
template <int DK, int RN>
__device__ __forceinline__ void buffer_store_d(const float (&x)[RN], __amdgpu_buffer_rsrc_t r,
                                               int voff, int soff) {
  static_assert(RN == 2 || RN == 4, "vectors of 2 or 4 columns");
  if constexpr (DK == 2 && RN == 4) {
    const u32x4 d = {__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                     __float_as_uint(x[3])};
    __builtin_amdgcn_raw_buffer_store_b128(d, r, voff, soff, kNt);
  } else if constexpr (DK == 2) {
    const u32x2 d = {__float_as_uint(x[0]), __float_as_uint(x[1])};
    __builtin_amdgcn_raw_buffer_store_b64(d, r, voff, soff, kNt);
  } else if constexpr (RN == 4) {
    const u32x2 d = {pack_half2(x[0], x[1]), pack_half2(x[2], x[3])};
    __builtin_amdgcn_raw_buffer_store_b64(d, r, voff, soff, kNt);
  } else {
    __builtin_amdgcn_raw_buffer_store_b32(pack_half2(x[0], x[1]), r, voff, soff, kNt);
  }
}

template <int CK, int RN>
__device__ __forceinline__ void buffer_load_c(float (&c)[RN], __amdgpu_buffer_rsrc_t r, int voff,
                                              int soff) {
  if constexpr (CK == 2 && RN == 4) {
    const u32x4 d = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
#pragma unroll
    for (int e = 0; e < 4; ++e) c[e] = __uint_as_float(d[e]);
  } else if constexpr (CK == 2) {
    const u32x2 d = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
    c[0] = __uint_as_float(d[0]);
    c[1] = __uint_as_float(d[1]);
  } else if constexpr (RN == 4) {
    const u32x2 d = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
    c[0] = half_lo(d[0]);
    c[1] = half_hi(d[0]);
    c[2] = half_lo(d[1]);
    c[3] = half_hi(d[1]);
  } else {
    const unsigned d = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
    c[0] = half_lo(d);
    c[1] = half_hi(d);
  }
}

// the same through a plain address (rows not in reach of one descriptor, or
// edge tiles)
template <int DK, int RN>
__device__ __forceinline__ void store_d_vec(const GemmParams& p, int m, int n,
                                            const float (&x)[RN]) {
  if constexpr (DK == 2) {
    typedef float fv __attribute__((ext_vector_type(RN)));
    fv v;
#pragma unroll
    for (int e = 0; e < RN; ++e) v[e] = x[e];
    __builtin_nontemporal_store(v, (fv*)((float*)p.D + (int64_t)m * p.ldd + n));
  } else {
    typedef _Float16 hv __attribute__((ext_vector_type(RN)));
    hv v;
#pragma unroll
    for (int e = 0; e < RN; ++e) v[e] = (_Float16)x[e];
    __builtin_nontemporal_store(v, (hv*)((_Float16*)p.D + (int64_t)m * p.ldd + n));
  }
}

template <int CK, int RN>
__device__ __forceinline__ void load_c_vec(const GemmParams& p, int m, int n, float (&c)[RN]) {
  if constexpr (CK == 2) {
    typedef float fv __attribute__((ext_vector_type(RN)));
    fv v;
    __builtin_memcpy(&v, (const float*)p.C + (int64_t)m * p.ldc + n, sizeof(v));
#pragma unroll
    for (int e = 0; e < RN; ++e) c[e] = v[e];
  } else {
    typedef _Float16 hv __attribute__((ext_vector_type(RN)));
    hv v;
    __builtin_memcpy(&v, (const _Float16*)p.C + (int64_t)m * p.ldc + n, sizeof(v));
#pragma unroll
    for (int e = 0; e < RN; ++e) c[e] = (float)v[e];
  }
}

// every value of a lane lies in the lane's own column of the atom, so the
// column of acc[i][j][v] depends on (lane, j) only
template <int OP>
MFL_HD constexpr bool c_columns_per_lane() {
  for (int v = 0; v < AtomTraits<OP>::NV; ++v)
    if (atom_c_coord_of<OP>(0, v).k != 0) return false;
  return true;
}
static_assert(c_columns_per_lane<kMfma32x32x16>() && c_columns_per_lane<kMfma16x16x32>(),
              "accumulator column must not depend on the value");

// Wait until at most VM vector-memory operations of this wave are in flight
// and all its LDS operations are done (s_waitcnt vmcnt(VM) lgkmcnt(0); the
// export counter is not waited on).  Vector-memory loads complete in issue
// order, so this leaves exactly the VM most recent ones outstanding.
template <int VM>
__device__ __forceinline__ void wait_vm_lds() {
  static_assert(VM >= 0 && VM < 64, "vmcnt has 6 bits");
  __builtin_amdgcn_s_waitcnt((VM & 15) | (((VM >> 4) & 3) << 14) | (7 << 4));
}

// whole tile inside D, vector-aligned rows, and every row of the tile within
// reach of one buffer descriptor
template <class Cfg, int CK, int DK>
__device__ __forceinline__ bool register_epilogue_ok(const GemmParams& p, int m0, int n0) {
  constexpr int ES = DK == 1 ? 2 : 4, CS = CK == 1 ? 2 : 4;
  return p.d_vec && (CK == 0 || p.c_vec) && m0 + Cfg::BM <= p.M && n0 + Cfg::BN <= p.N &&
         (int64_t)Cfg::BM * p.ldd * ES < ((int64_t)1 << 31) &&
         (CK == 0 || (int64_t)Cfg::BM * p.ldc * CS < ((int64_t)1 << 31));
}

// the buffer-descriptor path alone (one straight block: the kernels with one
// wave per SIMD have no registers for a second path).  A lane's repeats j of
// row block i sit in RN / V runs g of V adjacent columns (jl = j % V), run g
// AN V columns after run 0: one V-element vector of D per (i, v, g).
template <class Cfg, int CK, int DK, class Own = AllRows>
__device__ __forceinline__ void epilogue_regs(const GemmParams& p, int w, int lane, int m0,
                                              int n0, const AccT<Cfg> (&acc)[Cfg::RM][Cfg::RN],
                                              Own own = Own()) {
  constexpr int RM = Cfg::RM, V = Cfg::kVec, NG = Cfg::RN / V, NV = Cfg::kNV;
  constexpr int AM = Cfg::kAtomM, AN = Cfg::kAtomN;
  constexpr int ES = DK == 1 ? 2 : 4, CS = CK == 1 ? 2 : 4;
  {
    const RowK cl = atom_c_coord_of<Cfg::kOp>(lane, 0);
    const RowK w0 = frag_c_coord<Cfg>(w, 0, 0, 0, 0);     // the wave's tile origin
    // raw buffers (stride 0), records up to 2^31 bytes, 32-bit data format
    const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(
        (char*)p.D + ((int64_t)(m0 + w0.row) * p.ldd + (n0 + w0.k)) * ES, (short)0, 0x7fffffff,
        0x00020000);
    const int voff = (cl.row * p.ldd + V * cl.k) * ES;
    __amdgpu_buffer_rsrc_t rc = rd;
    int cvoff = 0;
    if constexpr (CK != 0) {
      rc = __builtin_amdgcn_make_buffer_rsrc(
          (char*)p.C + ((int64_t)(m0 + w0.row) * p.ldc + (n0 + w0.k)) * CS, (short)0, 0x7fffffff,
          0x00020000);
      cvoff = (cl.row * p.ldc + V * cl.k) * CS;
    }
    constexpr int QB = NV < 8 ? NV : 8;   // values whose C vectors load before first use
#pragma unroll
    for (int i = 0; i < RM; ++i) {
      if (!own(i)) continue;
#pragma unroll
      for (int v0 = 0; v0 < NV; v0 += QB) {
        float c[QB][NG][V];
        if constexpr (CK != 0) {
#pragma unroll
          for (int q = 0; q < QB; ++q)
#pragma unroll
            for (int g = 0; g < NG; ++g)
              buffer_load_c<CK, V>(
                  c[q][g], rc, cvoff,
                  (i * AM + atom_c_coord_of<Cfg::kOp>(0, v0 + q).row) * p.ldc * CS +
                      g * AN * V * CS);
        }
#pragma unroll
        for (int q = 0; q < QB; ++q) {
          const int v = v0 + q;
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            float x[V];
#pragma unroll
            for (int jl = 0; jl < V; ++jl) {
              // (copied to a scalar first: a bit cast applied to a vector
              // element directly read element 0 with this compiler)
              x[jl] = acc[i][g * V + jl][v];
              if constexpr (CK != 0) x[jl] += c[q][g][jl];
            }
            buffer_store_d<DK, V>(
                x, rd, voff,
                (i * AM + atom_c_coord_of<Cfg::kOp>(0, v).row) * p.ldd * ES + g * AN * V * ES);
          }
        }
      }
    }
  }
}

// The register epilogue with fp32 C taken through LDS.  Loading C with
// per-lane vector loads leaves a few KB in flight per wave and waits for each
// batch, so the C read runs far below the memory's rate.  Here the operand
// stages hold a wave row band of C (CR = WTM rows) at a time: the WAVES_N
// waves of that band fetch its rows straight into LDS (one 1 KB run per
// instruction, all runs of the band in flight together, and no store of
// theirs queued ahead, so their wait covers loads alone), then add each
// accumulator to the C value at its position and store D as the register
// epilogue does.
template <class Cfg>
struct CViaLds {
  static constexpr int kBytes = Cfg::kStages * (Cfg::BM + Cfg::BN) * Cfg::BK * 2;
  static constexpr int CR = Cfg::WTM;          // rows per pass: one wave row band
  static constexpr int RPI = 256 / Cfg::BN;    // rows per 1 KB run
  static constexpr int kRuns = CR / RPI;       // runs per pass
  // (the 16x16x32 kernels tie their accumulators by hand and have no
  // registers to spare for this path)
  static constexpr bool ok = Cfg::WAVES_K == 1 && Cfg::kOp == kMfma32x32x16 &&
                             (Cfg::BN == 128 || Cfg::BN == 256) && CR * Cfg::BN * 4 <= kBytes &&
                             kRuns % Cfg::WAVES_N == 0;
};

template <class Cfg, int DK>
__device__ __forceinline__ void epilogue_c_lds(const GemmParams& p, _Float16* smem, int w,
                                               int lane, int m0, int n0,
                                               const AccT<Cfg> (&acc)[Cfg::RM][Cfg::RN]) {
  using X = CViaLds<Cfg>;
  static_assert(X::ok, "configuration without a C pass through LDS");
  constexpr int RM = Cfg::RM, V = Cfg::kVec, NG = Cfg::RN / V, NV = Cfg::kNV;
  constexpr int AM = Cfg::kAtomM, AN = Cfg::kAtomN, BN = Cfg::BN, ES = DK == 1 ? 2 : 4;
  const float* C = (const float*)p.C;
  float* cs = (float*)smem;
  const int wm = wave_m<Cfg>(w), wn = wave_n<Cfg>(w);
  const RowK cl = atom_c_coord_of<Cfg::kOp>(lane, 0);
  const RowK w0 = frag_c_coord<Cfg>(w, 0, 0, 0, 0);     // the wave's tile origin
  const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(
      (char*)p.D + ((int64_t)(m0 + w0.row) * p.ldd + (n0 + w0.k)) * ES, (short)0, 0x7fffffff,
      0x00020000);
  const int voff = (cl.row * p.ldd + V * cl.k) * ES;
  for (int band = 0; band < Cfg::WAVES_M; ++band) {
    __syncthreads();   // the stages, or the previous band's C, are no longer read
    if (wm == band) {
#pragma unroll
      for (int k = 0; k < X::kRuns / Cfg::WAVES_N; ++k) {
        const int run = wn + Cfg::WAVES_N * k;
        const int row = run * X::RPI + lane / (BN / 4), col = 4 * (lane % (BN / 4));
        const float* src = C + (int64_t)(m0 + band * X::CR + row) * p.ldc + n0 + col;
        __builtin_amdgcn_global_load_lds((const void*)src, (lds_ptr_t)((char*)cs + run * 1024),
                                         16, 0, kNt);
      }
      wait_vm_lds<0>();
    }
    __syncthreads();
    if (wm == band) {
#pragma unroll
      for (int i = 0; i < RM; ++i)
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          const int row = i * AM + atom_c_coord_of<Cfg::kOp>(lane, v).row;
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            typedef float fv __attribute__((ext_vector_type(V)));
            const int col = frag_c_coord<Cfg>(w, lane, i, g * V, v).k;   // start of the run
            const fv c = *(const fv*)&cs[row * BN + col];
            float x[V];
#pragma unroll
            for (int jl = 0; jl < V; ++jl) {
              x[jl] = acc[i][g * V + jl][v];
              x[jl] += c[jl];
            }
            buffer_store_d<DK, V>(
                x, rd, voff,
                (i * AM + atom_c_coord_of<Cfg::kOp>(0, v).row) * p.ldd * ES + g * AN * V * ES);
          }
        }
    }
  }
}

// any tile: one vector per (i, v, run) where it fits inside D and the rows
// are vector-aligned, elements otherwise
template <class Cfg, int CK, int DK, class Own = AllRows>
__device__ __forceinline__ void epilogue_any(const GemmParams& p, int w, int lane, int m0,
                                             int n0, const AccT<Cfg> (&acc)[Cfg::RM][Cfg::RN],
                                             Own own = Own()) {
  constexpr int RM = Cfg::RM, V = Cfg::kVec, NG = Cfg::RN / V, AN = Cfg::kAtomN;
  const bool vec = p.d_vec && (CK == 0 || p.c_vec);
#pragma unroll
  for (int i = 0; i < RM; ++i) {
    if (!own(i)) continue;
#pragma unroll
    for (int v = 0; v < Cfg::kNV; ++v) {
      const RowK c0 = frag_c_coord<Cfg>(w, lane, i, 0, v);   // run 0: columns n .. n+V-1
      const int m = m0 + c0.row;
      if (m >= p.M) continue;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const int n = n0 + c0.k + g * AN * V;
        float x[V];
#pragma unroll
        for (int jl = 0; jl < V; ++jl) x[jl] = acc[i][g * V + jl][v];
        if (vec && n + V <= p.N) {
          if constexpr (CK != 0) {
            float c[V];
            load_c_vec<CK, V>(p, m, n, c);
#pragma unroll
            for (int jl = 0; jl < V; ++jl) x[jl] += c[jl];
          }
          store_d_vec<DK, V>(p, m, n, x);
        } else {
#pragma unroll
          for (int jl = 0; jl < V; ++jl)
            if (n + jl < p.N) d_store<DK>(p, m, n + jl, x[jl] + c_value<CK>(p, m, n + jl));
        }
      }
    }
  }
}

// Split-K reduction (the K-direction thread groups of the TiledMMA page,
// section "K 方向的线程组，与 K 方向的循环": several groups hold partial sums
// for the same outputs and one of them must add the others, C once).  Row
// block i (atom blocks i*RN .. i*RN+RN-1, whole rows so the epilogue's
// vectors stay with one wave) of a wave is finished by the member of its
// K-group set with wave_k == i % WAVES_K; each other member writes its
// partial blocks into the freed operand stages and the owner adds them, so
// every member finishes RM/WAVES_K row blocks (a reduce-scatter inside the
// workgroup).  A block is
// NV values x 64 lanes, laid out [v/4][lane][v%4]: each lane moves 16-byte
// pieces and the 64 lanes of one access cover 1 KB contiguously.
template <class Cfg>
struct OwnedRows {
  int wk;
  __device__ bool operator()(int i) const { return i % Cfg::WAVES_K == wk; }
};

template <class Cfg>
__device__ __forceinline__ void reduce_k_groups(float* red, int w, int lane,
                                                AccT<Cfg> (&acc)[Cfg::RM][Cfg::RN]) {
  constexpr int RN = Cfg::RN, WK = Cfg::WAVES_K, NB = Cfg::RM * RN, NV = Cfg::kNV;
  const int wg = w % Cfg::kGroupWaves, wk = wave_k<Cfg>(w);
  auto block = [&](int b, int writer) {
    const int owner = (b / RN) % WK;
    const int slot = (writer - owner - 1 + WK) % WK;    // 0 .. WK-2
    return red + ((wg * NB + b) * (WK - 1) + slot) * (NV * 64) + lane * 4;
  };
  __syncthreads();   // every wave is done with the operand stages
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    if ((b / RN) % WK == wk) continue;
    float* dst = block(b, wk);
#pragma unroll
    for (int q = 0; q < NV / 4; ++q) {
      const AccT<Cfg>& a = acc[b / RN][b % RN];
      const float4 x = make_float4(a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]);
      *(float4*)(dst + q * 256) = x;
    }
  }
  __syncthreads();
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    if ((b / RN) % WK != wk) continue;
#pragma unroll
    for (int m = 1; m < WK; ++m) {
      const float* src = block(b, (wk + m) % WK);
#pragma unroll
      for (int q = 0; q < NV / 4; ++q) {
        const float4 x = *(const float4*)(src + q * 256);
        acc[b / RN][b % RN][4 * q] += x.x;
        acc[b / RN][b % RN][4 * q + 1] += x.y;
        acc[b / RN][b % RN][4 * q + 2] += x.z;
        acc[b / RN][b % RN][4 * q + 3] += x.w;
      }
    }
  }
}

// LDS-staged epilogue of the LDS kernels when C is read.  Accumulators leave
// the MFMA layout through LDS so that every global access is a row-contiguous
// run of 4 elements per lane: D = acc + C with one C load, four adds and one
// D store per run.  (Without C the register epilogue is faster: its stores
// need no staging.)  Interior tiles batch their C loads (no per-element
// branches); edge tiles check each run and fall back to elements at the
// right edge.  The runs of a D row are 16-byte (fp32) or 8-byte (fp16)
// stores when d_vec says D allows it, single elements otherwise.
__device__ __forceinline__ float4 load_c4_f32(const GemmParams& p, int m, int n) {
  float4 c;
  __builtin_memcpy(&c, (const float*)p.C + (int64_t)m * p.ldc + n, 16);
  return c;
}
__device__ __forceinline__ float4 load_c4_f16(const GemmParams& p, int m, int n) {
  typedef _Float16 half4v __attribute__((ext_vector_type(4)));
  half4v h;
  __builtin_memcpy(&h, (const _Float16*)p.C + (int64_t)m * p.ldc + n, 8);
  return make_float4((float)h[0], (float)h[1], (float)h[2], (float)h[3]);
}

template <int CK>
__device__ __forceinline__ float4 load_c4(const GemmParams& p, int m, int n) {
  if constexpr (CK == 2) return load_c4_f32(p, m, n);
  if constexpr (CK == 1) return load_c4_f16(p, m, n);
  return make_float4(0.f, 0.f, 0.f, 0.f);
}

template <int DK>
__device__ __forceinline__ void store_d4(const GemmParams& p, int m, int n, float4 x) {
  if (p.d_vec) {
    if constexpr (DK == 1) {
      typedef _Float16 half4v __attribute__((ext_vector_type(4)));
      const half4v h = {(_Float16)x.x, (_Float16)x.y, (_Float16)x.z, (_Float16)x.w};
      __builtin_nontemporal_store(h, (half4v*)((_Float16*)p.D + (int64_t)m * p.ldd + n));
    } else {
      typedef float float4v __attribute__((ext_vector_type(4)));
      const float4v v = {x.x, x.y, x.z, x.w};
      __builtin_nontemporal_store(v, (float4v*)((float*)p.D + (int64_t)m * p.ldd + n));
    }
  } else {
    d_store<DK>(p, m, n, x.x);
    d_store<DK>(p, m, n + 1, x.y);
    d_store<DK>(p, m, n + 2, x.z);
    d_store<DK>(p, m, n + 3, x.w);
  }
}

template <class Cfg, int CK, int DK>
__device__ __forceinline__ void epilogue_lds(const GemmParams& p, float* sm, int w, int lane,
                                             int m0, int n0,
                                             const AccT<Cfg> (&acc)[Cfg::RM][Cfg::RN]) {
  constexpr int RM = Cfg::RM, WTN = Cfg::WTN, IG = Cfg::kEpiRows, AM = Cfg::kAtomM;
  constexpr int V = Cfg::kVec, NG = Cfg::RN / V, AN = Cfg::kAtomN;
  constexpr int ROWS = IG * AM, V4 = WTN / 4, NQ = ROWS * V4 / 64, QB = 8;
  static_assert((ROWS * V4) % 64 == 0 && NQ % QB == 0, "runs must divide over the lanes");
  float* reg = sm + w * ROWS * WTN;
  const int wm = wave_m<Cfg>(w), wn = wave_n<Cfg>(w);
  const int mw = m0 + wm * Cfg::WTM, nw = n0 + wn * WTN;
  const bool interior = m0 + Cfg::BM <= p.M && n0 + Cfg::BN <= p.N;
  __syncthreads();   // every wave is done with the operand stages
#pragma unroll
  for (int i0 = 0; i0 < RM; i0 += IG) {
    // accumulators -> this wave's staging tile (rows i0*AM .. +ROWS), at
    // their physical columns: a lane's repeats come in runs of V adjacent
    // columns, one vector per run
#pragma unroll
    for (int ii = 0; ii < IG; ++ii)
#pragma unroll
      for (int v = 0; v < Cfg::kNV; ++v) {
        const RowK c = atom_c_coord_of<Cfg::kOp>(lane, v);
        typedef float fv __attribute__((ext_vector_type(V)));
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          fv x;
#pragma unroll
          for (int jl = 0; jl < V; ++jl) x[jl] = acc[i0 + ii][g * V + jl][v];
          *(fv*)&reg[epi_offset<WTN>(ii * AM + c.row, g * AN * V + V * c.k)] = x;
        }
      }
    // A wave's LDS operations complete in order, so the reads below see the
    // stores above, and the next pass's stores follow these reads.
#pragma unroll
    for (int q0 = 0; q0 < NQ; q0 += QB) {
      float4 x[QB], c[QB];
#pragma unroll
      for (int q = 0; q < QB; ++q) {
        const int t = lane + 64 * (q0 + q), r = t / V4, c4 = t % V4;
        x[q] = *(const float4*)&reg[epi_offset<WTN>(r, 4 * c4)];
      }
      if (interior) {
        if constexpr (CK != 0) {
#pragma unroll
          for (int q = 0; q < QB; ++q) {
            const int t = lane + 64 * (q0 + q);
            c[q] = load_c4<CK>(p, mw + i0 * AM + t / V4, nw + 4 * (t % V4));
          }
        }
#pragma unroll
        for (int q = 0; q < QB; ++q) {
          const int t = lane + 64 * (q0 + q);
          float4 y = x[q];
          if constexpr (CK != 0) {
            y.x += c[q].x;
            y.y += c[q].y;
            y.z += c[q].z;
            y.w += c[q].w;
          }
          store_d4<DK>(p, mw + i0 * AM + t / V4, nw + 4 * (t % V4), y);
        }
      } else {
#pragma unroll
        for (int q = 0; q < QB; ++q) {
          const int t = lane + 64 * (q0 + q);
          const int m = mw + i0 * AM + t / V4, n = nw + 4 * (t % V4);
          if (m < p.M) {
            if (n + 3 < p.N) {
              float4 y = x[q];
              if constexpr (CK != 0) {
                const float4 cc = load_c4<CK>(p, m, n);
                y.x += cc.x;
                y.y += cc.y;
                y.z += cc.z;
                y.w += cc.w;
              }
              store_d4<DK>(p, m, n, y);
            } else {
              const float xv[4] = {x[q].x, x[q].y, x[q].z, x[q].w};
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (n + e < p.N) d_store<DK>(p, m, n + e, xv[e] + c_value<CK>(p, m, n + e));
            }
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Operand fetchers: one operand tile (ROWS x BK halves) per stage
// ---------------------------------------------------------------------------
// Common interface:
//   init(row0, rows_valid, ld, tid, w, lane)   per-thread offsets, once
//   issue(base, kt, stage_ptr)                 start fetching K-tile kt
//   stash(stage_ptr)                           registers -> LDS (REG policies)

// DMA: global_load_lds_dwordx4 writes the 64 lanes' 16-byte chunks to 1 KB of
// LDS after M0, lane l at byte 16 l.  A 1 KB run holds RUN = 512/BK rows; lane
// l takes row RUN*run + l/CH, physical chunk l%CH, so it fetches logical chunk
// (l%CH) ^ swz(row) of that row.
// PERM: the operand's rows carry the N permutation (B): LDS row r holds
// global row row0 + perm_n(r).
template <class Cfg, int ROWS, bool PERM>
struct FetchDma {
  static constexpr int BK = Cfg::BK, CH = Cfg::CH, RUN = 512 / BK;
  static constexpr int kRuns = ROWS / RUN / Cfg::kWaves;
  static_assert(ROWS % (RUN * Cfg::kWaves) == 0, "runs must divide over the waves");
  static constexpr int kVmem = kRuns, kDsWrites = 0;   // instructions per issue / stash
  unsigned off[kRuns];
  int run0;
  __device__ void init(int row0, int rows_valid, int ld, int tid, int w, int lane) {
    (void)tid;
    run0 = w * kRuns;
    const int rsub = lane / CH;
#pragma unroll
    for (int i = 0; i < kRuns; ++i) {
      const int row = RUN * (run0 + i) + rsub;
      const int grow = PERM ? perm_n<Cfg>(row) : row;
      const int kc = ((lane % CH) ^ swz<CH>(row)) * 8;
      off[i] = (unsigned)((int64_t)min(row0 + grow, row0 + rows_valid - 1) * ld * 2) + kc * 2;
    }
  }
  __device__ void issue_one(int i, const void* base, int kt, _Float16* stage) {
    const char* b = (const char*)base + (int64_t)kt * BK * 2;
    __builtin_amdgcn_global_load_lds((const void*)(b + (uint64_t)off[i]),
                                     (lds_ptr_t)(stage + (run0 + i) * RUN * BK), 16, 0, 0);
  }
  __device__ void stash_one(int, _Float16*) {}
};

// REG: K-contiguous rows, 16-byte chunks q = tid + i*T (row q/CH, chunk q%CH)
template <class Cfg, int ROWS, bool PERM>
struct FetchReg {
  static constexpr int BK = Cfg::BK, CH = Cfg::CH, T = Cfg::kThreads;
  static constexpr int kChunks = ROWS * CH / T;
  static_assert((ROWS * CH) % T == 0, "chunks must divide over the threads");
  static constexpr int kVmem = kChunks, kDsWrites = kChunks;
  int off[kChunks], lds[kChunks];
  uint4 r[kChunks];
  __device__ void init(int row0, int rows_valid, int ld, int tid, int w, int lane) {
    (void)w;
    (void)lane;
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int q = tid + i * T, row = q / CH, c = q % CH;
      const int grow = PERM ? perm_n<Cfg>(row) : row;
      off[i] = (int)((int64_t)min(row0 + grow, row0 + rows_valid - 1) * ld * 2) + c * 16;
      lds[i] = lds_offset<BK>(row, c * 8);
    }
  }
  __device__ void issue_one(int i, const void* base, int kt, _Float16*) {
    r[i] = load16((const char*)base + (int64_t)kt * BK * 2, off[i]);
  }
  __device__ void stash_one(int i, _Float16* stage) { *(uint4*)&stage[lds[i]] = r[i]; }
};

// REGT: M-contiguous A.  Chunk = KR k-rows x 8 m (KR 16-byte loads, one
// per k-row); transposed in registers into 8 runs of KR k, one per m, and
// written with KR*2-byte LDS stores into the K-contiguous tile.  KR = 4 when
// the chunks divide over the threads, else 2.
template <class Cfg, int ROWS>
struct FetchRegT {
  static constexpr int BK = Cfg::BK, T = Cfg::kThreads;
  static constexpr int KR = ((BK / 4) * (ROWS / 8)) % T == 0 ? 4 : 2;
  static constexpr int kChunks = (BK / KR) * (ROWS / 8) / T;
  static_assert(((BK / KR) * (ROWS / 8)) % T == 0 && kChunks > 0,
                "chunks must divide over the threads");
  static constexpr int kVmem = kChunks * KR, kDsWrites = kChunks * 8;
  int off[kChunks], mvalid[kChunks], lds_k[kChunks], lds_m[kChunks];
  int ld;
  uint4 r[kChunks][KR];
  __device__ void init(int row0, int rows_valid, int ld_, int tid, int w, int lane) {
    (void)w;
    (void)lane;
    ld = ld_;
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int q = tid + i * T, kg = q / (ROWS / 8), mc = q % (ROWS / 8);
      off[i] = (int)((int64_t)kg * KR * ld * 2) + (row0 + mc * 8) * 2;
      mvalid[i] = rows_valid - mc * 8;
      lds_k[i] = kg * KR;
      lds_m[i] = mc * 8;
    }
  }
  // instruction v loads k-row v % KR of chunk v / KR
  __device__ void issue_one(int v, const void* base, int kt, _Float16*) {
    const int i = v / KR, rr = v % KR;
    const char* b = (const char*)base + (int64_t)kt * BK * ld * 2;
    const int64_t o = off[i] + (int64_t)rr * ld * 2;
    r[i][rr] = mvalid[i] >= 8 ? load16(b, o)
               : mvalid[i] <= 0 ? make_uint4(0, 0, 0, 0)
                                : load8_tail((const _Float16*)(b + o), mvalid[i]);
  }
  // halves e of two 8-half vectors x, y packed as (x[e], y[e])
  __device__ static unsigned pack(const uint4& x, const uint4& y, int e) {
    const unsigned* a = (const unsigned*)&x;
    const unsigned* b = (const unsigned*)&y;
    const int d = e >> 1;
    return (e & 1) ? ((a[d] >> 16) | (b[d] & 0xffff0000u)) : ((a[d] & 0xffffu) | (b[d] << 16));
  }
  // store d writes the KR k of m = lds_m + d % 8 of chunk d / 8
  __device__ void stash_one(int d, _Float16* stage) {
    const int i = d / 8, e = d % 8;
    _Float16* dst = &stage[lds_offset<BK>(lds_m[i] + e, lds_k[i])];
    if constexpr (KR == 4)
      *(uint2*)dst = make_uint2(pack(r[i][0], r[i][1], e), pack(r[i][2], r[i][3], e));
    else
      *(unsigned*)dst = pack(r[i][0], r[i][1], e);
  }
};

// DMAT: M-contiguous A straight into an M-contiguous LDS tile (BK rows of
// ROWS halves, lds_offset_mn).  A 1 KB run holds RUN = 512/ROWS k-rows; lane
// l takes k-row RUN*run + l/CPR, physical chunk l%CPR, so it fetches logical
// chunk (l%CPR) ^ mn_swz(krow), i.e. m = row0 + 8 * that.  Needs M % 8 == 0
// (chunks are all-valid or all-past-M; the latter are clamped to the last
// valid chunk and only feed outputs that are never stored).
template <class Cfg, int ROWS>
struct FetchDmaT {
  static constexpr int BK = Cfg::BK, CPR = ROWS / 8, RUN = 64 / CPR;
  static constexpr int kRuns = BK / RUN / Cfg::kWaves;
  static_assert(BK % (RUN * Cfg::kWaves) == 0 && kRuns > 0, "runs must divide over the waves");
  static constexpr int kVmem = kRuns, kDsWrites = 0;
  unsigned off[kRuns];
  int run0, ld;
  __device__ void init(int row0, int rows_valid, int ld_, int tid, int w, int lane) {
    (void)tid;
    ld = ld_;
    run0 = w * kRuns;
#pragma unroll
    for (int i = 0; i < kRuns; ++i) {
      const int krow = RUN * (run0 + i) + lane / CPR;
      const int c = (lane % CPR) ^ mn_swz(krow);
      const int m = min(8 * c, rows_valid - 8);
      off[i] = (unsigned)(((int64_t)krow * ld + row0 + m) * 2);
    }
  }
  __device__ void issue_one(int i, const void* base, int kt, _Float16* stage) {
    const char* b = (const char*)base + (int64_t)kt * BK * ld * 2;
    __builtin_amdgcn_global_load_lds((const void*)(b + (uint64_t)off[i]),
                                     (lds_ptr_t)(stage + (run0 + i) * RUN * ROWS), 16, 0, 0);
  }
  __device__ void stash_one(int, _Float16*) {}
};

template <class Cfg, int ROWS, int POLICY, bool PERM>
struct FetchSel;
template <class Cfg, int ROWS, bool PERM>
struct FetchSel<Cfg, ROWS, kFetchDma, PERM> {
  using type = FetchDma<Cfg, ROWS, PERM>;
};
template <class Cfg, int ROWS, bool PERM>
struct FetchSel<Cfg, ROWS, kFetchReg, PERM> {
  using type = FetchReg<Cfg, ROWS, PERM>;
};
template <class Cfg, int ROWS>
struct FetchSel<Cfg, ROWS, kFetchRegT, false> {   // A only
  using type = FetchRegT<Cfg, ROWS>;
};
template <class Cfg, int ROWS>
struct FetchSel<Cfg, ROWS, kFetchDmaT, false> {   // A only
  using type = FetchDmaT<Cfg, ROWS>;
};

// Two transposed LDS reads (k0 and k0 + 4 of an M-contiguous tile) -> one
// 8-half operand fragment.
typedef short short4v __attribute__((ext_vector_type(4)));
typedef short short8v __attribute__((ext_vector_type(8)));
__device__ __forceinline__ half8 read_tr_pair(const _Float16* p0, const _Float16* p1) {
  using lds_s4 = __attribute__((address_space(3))) short4v*;
  const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)(p0));
  const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)(p1));
  const short8v v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(half8, v);
}

template <bool B>
struct BoolC {
  static constexpr bool value = B;
};

// C kind of the test-only register dump instances (never a valid C dtype):
// instead of the epilogue, every thread writes its operand fragment
// registers and accumulators to p.D (as 32-bit words, see dump_words).
constexpr int kDumpC = 3;

// words per thread of a dump: NBUF x (RM + RN) fragments of 8 halves (4 words
// each), then RM x RN x NV accumulators
template <class Cfg>
constexpr int dump_words() {
  constexpr int nbuf = Cfg::kFragDist == 1 ? 2 : Cfg::KSUB_W;
  return nbuf * (Cfg::RM + Cfg::RN) * 4 + Cfg::RM * Cfg::RN * Cfg::kNV;
}

// ---------------------------------------------------------------------------
// LDS-staged pipelined kernel
// ---------------------------------------------------------------------------
// POISON (test-only instances): the whole LDS array is first filled with
// fp16 NaN, so a fragment or epilogue read of any location the kernel did
// not write shows up in D.
template <class Cfg, int FA, int FB, int CK, int DK, bool POISON = false>
__global__ void __launch_bounds__(Cfg::kThreads, 1) gemm_tiled(const GemmParams p) {
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK;
  // KSUB: this wave's K sub-steps of each stage (all of them unless the
  // workgroup splits K between groups of waves)
  constexpr int RM = Cfg::RM, RN = Cfg::RN, KSUB = Cfg::KSUB_W;
  static_assert(KSUB % 2 == 0, "fragment buffers alternate per K sub-step");
  constexpr int kDist = Cfg::kFragDist;
  constexpr int NBUF = kDist == 1 ? 2 : KSUB;     // fragment register buffers
  static_assert(FB != kFetchRegT && FB != kFetchDmaT, "B is always K-contiguous");
  constexpr bool kAT = FA == kFetchDmaT;   // A tile M-contiguous in LDS
  // stage s: A at smem + s*kStage, B at smem + s*kStage + BM*BK (halves)
  constexpr int NST = Cfg::kStages;
  constexpr int kStage = (BM + BN) * BK;
  __shared__ __attribute__((aligned(1024))) _Float16 smem[NST * kStage];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const TileIndex ti = tile_of_block(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.group_m);
  const int m0 = ti.tm * BM, n0 = ti.tn * BN;
  if constexpr (POISON) {
    for (int i = tid; i < NST * kStage / 2; i += Cfg::kThreads)
      ((unsigned*)smem)[i] = 0x7E007E00u;   // two fp16 NaNs
    __syncthreads();
  }

  using FetchA = typename FetchSel<Cfg, BM, FA, false>::type;
  using FetchB = typename FetchSel<Cfg, BN, FB, true>::type;   // rows in N-permuted order
  FetchA fa_;
  FetchB fb_;
  fa_.init(m0, p.M - m0, p.lda, tid, w, lane);
  fb_.init(n0, p.N - n0, p.ldb, tid, w, lane);
  auto stage_a = [&](int s) { return smem + s * kStage; };
  auto stage_b = [&](int s) { return smem + s * kStage + BM * BK; };
  // fetch instruction v / LDS store d of both operands (A first)
  constexpr int kVmem = FetchA::kVmem + FetchB::kVmem;
  constexpr int kDsW = FetchA::kDsWrites + FetchB::kDsWrites;
  auto issue_one = [&](int v, int kt, int s) {
    if (v < FetchA::kVmem)
      fa_.issue_one(v, p.A, kt, stage_a(s));
    else
      fb_.issue_one(v - FetchA::kVmem, p.B, kt, stage_b(s));
  };
  auto stash_one = [&](int d, int s) {
    if (d < FetchA::kDsWrites)
      fa_.stash_one(d, stage_a(s));
    else
      fb_.stash_one(d - FetchA::kDsWrites, stage_b(s));
  };
  auto issue = [&](int kt, int s) {
#pragma unroll
    for (int v = 0; v < kVmem; ++v) issue_one(v, kt, s);
  };
  auto stash = [&](int s) {
#pragma unroll
    for (int d = 0; d < kDsW; ++d) stash_one(d, s);
  };
  constexpr bool kAnyReg = FA != kFetchDma || FB != kFetchDma;
  // Three stages, both operands straight into LDS: a tile's fetch is split.
  // Its first kH1 instructions go out after the barrier that frees its stage
  // (the groups after the barrier of step kt fetch tile kt+NST into stage
  // cur), the rest in the groups before the next step's barrier, which write
  // the same stage (stage prv there).  A CU moves at most 64 B per clock into
  // LDS and an instruction that finds that path busy holds its wave, so a
  // whole tile's fetch between two barriers would stall the one wave of each
  // SIMD for longer than its MFMAs there.
  constexpr bool kSplitFetch = NST == 3 && !kAnyReg;
  constexpr int kH1 = kSplitFetch ? kVmem / 2 : kVmem;

  // fragment read offsets within a stage (halves), per K sub-step
  int fa_off[KSUB][RM], fb_off[KSUB][RN];
#pragma unroll
  for (int kk = 0; kk < KSUB; ++kk) {
#pragma unroll
    for (int i = 0; i < RM; ++i) {
      if constexpr (kAT) {
        // first of the two transposed reads; the second is 4 k-rows on
        const RowK t = frag_a_tr_coord<Cfg>(w, lane, i, kk);
        fa_off[kk][i] = lds_offset_mn<BM>(t.row, t.k);
      } else {
        const RowK a = frag_a_coord<Cfg>(w, lane, i, kk);
        fa_off[kk][i] = lds_offset<BK>(a.row, a.k);
      }
    }
#pragma unroll
    for (int j = 0; j < RN; ++j) {
      const RowK b = frag_b_coord<Cfg>(w, lane, j, kk);
      fb_off[kk][j] = BM * BK + lds_offset<BK>(b.row, b.k);
    }
  }

  half8 fa[NBUF][RM], fb[NBUF][RN];
  auto bufof = [](int kk) { return kDist == 1 ? (kk & 1) : kk; };   // buffer of sub-step kk
  // fragment read r in the order the MFMAs consume them (i-major, so A0,
  // then B0..B(RN-1), then A1..A(RM-1))
  constexpr int kReads = RM + RN, kMfma = RM * RN;
  auto read_a = [&](int i, int buf, int kk, const _Float16* st) {
    if constexpr (kAT)
      fa[buf][i] = read_tr_pair(&st[fa_off[kk][i]], &st[fa_off[kk][i] + 4 * BM]);
    else
      fa[buf][i] = *(const half8*)&st[fa_off[kk][i]];
  };
  auto read_one = [&](int r, int buf, int kk, int s) {
    const _Float16* st = smem + s * kStage;
    if (r == 0)
      read_a(0, buf, kk, st);
    else if (r <= RN)
      fb[buf][r - 1] = *(const half8*)&st[fb_off[kk][r - 1]];
    else
      read_a(r - RN, buf, kk, st);
  };
  auto frags = [&](int buf, int kk, int s) {
#pragma unroll
    for (int r = 0; r < kReads; ++r) read_one(r, buf, kk, s);
  };

  AccT<Cfg> acc[RM][RN];
  zero_acc<Cfg>(acc);
  mma_begin<Cfg>(acc);

  auto mma = [&](int buf) {
#pragma unroll
    for (int i = 0; i < RM; ++i)
#pragma unroll
      for (int j = 0; j < RN; ++j) Mma<Cfg::kOp>::run(fa[buf][i], fb[buf][j], acc[i][j]);
  };

  // One group: the RM x RN MFMAs on fragment buffer `buf`.  A wave can issue
  // other instructions while its previous MFMA occupies the matrix core, so
  // each MFMA is followed by its share of the group's memory instructions:
  // fragment reads (buffer rbuf, sub-step rkk of stage rs) in the first half
  // of the group, since they feed the next one; fetch instructions (tile fkt
  // into stage fs) and LDS stores of register-staged data (stage ss) over the
  // whole group.  The fences keep the compiler from regrouping them.
  auto group = [&](int buf, auto reads, int rbuf, int rkk, int rs, auto fetch, int fkt, int fs,
                   auto stores, int ss, int v0, int v1) {
    constexpr bool kR = decltype(reads)::value, kF = decltype(fetch)::value;
    constexpr bool kS = decltype(stores)::value;
    constexpr int rslots = kMfma / 2 > 0 ? kMfma / 2 : 1;
    // Two waves per SIMD on the 16x16x32 instruction: the SIMD issues for
    // the older wave first, which would finish each step well ahead of its
    // partner and wait at the barrier while the partner runs alone.  A wave
    // holds a raised priority for the first half of each group, so the one
    // that is behind catches up (measured on 4096^3: the wait at the barrier
    // halves, the cycles per K step drop 2.8 %).
    constexpr bool kBalance = Cfg::kOp == kMfma16x16x32 && Cfg::kWaves > 4;
#pragma unroll
    for (int g = 0; g < kMfma; ++g) {
      const int i = g / RN, j = g % RN;
      if constexpr (kBalance) {
        if (g == 0) __builtin_amdgcn_s_setprio(1);
        if (g == kMfma / 2) __builtin_amdgcn_s_setprio(0);
      }
      Mma<Cfg::kOp>::run(fa[buf][i], fb[buf][j], acc[i][j]);
      if constexpr (kR) {
        if (g < rslots) {
#pragma unroll
          for (int r = g * kReads / rslots; r < (g + 1) * kReads / rslots; ++r)
            read_one(r, rbuf, rkk, rs);
        }
      }
      if constexpr (kF) {
        // fetch instructions [v0, v1) spread over the group
#pragma unroll
        for (int v = v0 + g * (v1 - v0) / kMfma; v < v0 + (g + 1) * (v1 - v0) / kMfma; ++v)
          issue_one(v, fkt, fs);
      }
      if constexpr (kS) {
#pragma unroll
        for (int d = g * kDsW / kMfma; d < (g + 1) * kDsW / kMfma; ++d) stash_one(d, ss);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using Yes = BoolC<true>;
  using No = BoolC<false>;

  const int nfull = p.K / BK;
  if (nfull > 0) {
    // tiles 0 .. NST-1 into stages 0 .. NST-1.  Register-staged tiles other
    // than tile NST-1 are written to LDS at once; tile NST-1 waits in
    // registers and is written in step 0 (the steps write tile kt+NST-1).
    issue(0, 0);
    if constexpr (kAnyReg) stash(0);
    if (nfull > 1) {
      issue(1, 1);
      if constexpr (NST == 3 && kAnyReg) stash(1);
    }
    // Only tile 0 must have landed before the first barrier: the later tiles
    // are waited for by the step that reads them, before its own barrier.
    if constexpr (NST == 3) {
      if (nfull > 2) {
#pragma unroll
        for (int v = 0; v < kH1; ++v) issue_one(v, 2, 2);   // the rest in step 0
        wait_vm_lds<kVmem + kH1>();   // tiles 1 and 2 may be in flight
      } else if (nfull > 1) {
        wait_vm_lds<kVmem>();
      } else {
        wait_vm_lds<0>();
      }
    } else {
      if (nfull > 1)
        wait_vm_lds<kVmem>();       // tile 1 may be in flight
      else
        wait_vm_lds<0>();
    }
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    frags(bufof(0), 0, 0);
    if constexpr (kDist == 2) frags(bufof(1), 1, 0);
  }
  // One K-step on tile kt (stage kt % NST).  FETCH: tile kt+NST exists and is
  // fetched into this step's stage once every wave is done with it; NEXT:
  // tile kt+1 exists; LAST: tile kt+NST-1 exists (it was fetched NST-1 steps
  // ago; with registers as staging it is written to its stage in this step).
  // The last NST steps are peeled off the loop so its body is one straight
  // block.
  //
  // Fragment distance 1: sub-steps 0..KSUB-2 read sub-step kk+1 of stage cur;
  // the barrier; sub-step KSUB-1 fetches tile kt+NST and reads sub-step 0 of
  // the next stage.  Distance 2: sub-steps 0..KSUB-3 read sub-step kk+2; the
  // barrier; sub-steps KSUB-2 and KSUB-1 share the fetch and read sub-steps 0
  // and 1 of the next stage.  Either way register-staged tile kt+NST-1 goes to
  // its stage in the last group before the barrier, and the groups after the
  // barrier run on fragments already in registers.  Before the barrier each
  // wave waits for its fetch of tile kt+1; with three stages the fetch of
  // tile kt+2 (the most recent kVmem loads) stays in flight.
  auto step = [&](const int kt, auto fetch, auto next, auto last) {
    constexpr bool kLast = decltype(last)::value;
    const int cur = NST == 2 ? (kt & 1) : kt % NST;
    const int nxt = cur + 1 == NST ? 0 : cur + 1;
    const int prv = cur == 0 ? NST - 1 : cur - 1;   // stage of tile kt+NST-1
    constexpr int kPre = KSUB - kDist;   // groups before the barrier
    // split fetch: the second part of tile kt+NST-1 over the groups before
    // the barrier
    using PreFetch = BoolC<kSplitFetch && kLast>;
    constexpr int kRest = kVmem - kH1;
#pragma unroll
    for (int kk = 0; kk + 1 < kPre; ++kk)
      group(bufof(kk), Yes(), bufof(kk + kDist), kk + kDist, cur, PreFetch(), kt + NST - 1, prv,
            No(), 0, kH1 + kk * kRest / kPre, kH1 + (kk + 1) * kRest / kPre);
    group(bufof(kPre - 1), Yes(), bufof(KSUB - 1), KSUB - 1, cur, PreFetch(), kt + NST - 1, prv,
          BoolC<kAnyReg && kLast>(), prv, kH1 + (kPre - 1) * kRest / kPre, kVmem);
    wait_vm_lds<(NST == 3 && kLast) ? kVmem : 0>();   // own reads, stores, fetch of tile kt+1
    __builtin_amdgcn_s_barrier();                     // ... in every wave: stage cur is free
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int d = 0; d < kDist; ++d)
      group(bufof(kPre + d), next, bufof(d), d, nxt, fetch, kt + NST, cur, No(), 0,
            d * kH1 / kDist, (d + 1) * kH1 / kDist);
  };
  int kt = 0;
  for (; kt + NST < nfull; ++kt) step(kt, Yes(), Yes(), Yes());
  if constexpr (NST == 3) {
    if (kt + 2 < nfull) step(kt++, No(), Yes(), Yes());
  }
  if (kt + 1 < nfull) step(kt++, No(), Yes(), BoolC<NST == 2>());
  if (kt < nfull) step(kt, No(), No(), No());

  // K remainder: one step staged with zero fill past K.  K-contiguous rows go
  // by 16-byte chunks (a whole chunk in one load, the chunk that holds K's
  // edge element by element, zeros past it); M-contiguous A element by
  // element.
  if (p.K % BK != 0) {
    const int k0 = nfull * BK;
    __syncthreads();
    _Float16* sa = stage_a(0);
    _Float16* sb = stage_b(0);
    const _Float16* A = (const _Float16*)p.A;
    const _Float16* B = (const _Float16*)p.B;
    auto stage_rows = [&](const _Float16* X, int64_t ld, int rows, auto grow, _Float16* dst) {
      constexpr int CHK = BK / 8;
      for (int q = tid; q < rows * CHK; q += Cfg::kThreads) {
        const int row = q / CHK, c = q % CHK, gk = k0 + 8 * c;
        const _Float16* src = X + (int64_t)grow(row) * ld + gk;
        union {
          uint4 u;
          _Float16 h[8];
        } v;
        v.u = make_uint4(0, 0, 0, 0);
        if (gk + 8 <= p.K) {
          __builtin_memcpy(&v.u, src, 16);
        } else if (gk < p.K) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (gk + e < p.K) v.h[e] = src[e];
        }
        *(uint4*)&dst[lds_offset<BK>(row, 8 * c)] = v.u;
      }
    };
    if constexpr (FA == kFetchRegT || kAT) {
      for (int e = tid; e < BM * BK; e += Cfg::kThreads) {
        const int row = e / BK, k = e % BK, gk = k0 + k;
        const int gm = min(m0 + row, p.M - 1);
        const _Float16 v = gk < p.K ? A[(int64_t)gk * p.lda + gm] : (_Float16)0.0f;
        if constexpr (kAT)
          sa[lds_offset_mn<BM>(row, k)] = v;
        else
          sa[lds_offset<BK>(row, k)] = v;
      }
    } else {
      stage_rows(A, p.lda, BM, [&](int row) { return min(m0 + row, p.M - 1); }, sa);
    }
    stage_rows(B, p.ldb, BN, [&](int row) { return min(n0 + perm_n<Cfg>(row), p.N - 1); }, sb);
    __syncthreads();
    // this wave's sub-steps that start at or past K hold only zeros: skipped
    const int krem = p.K % BK;
#pragma unroll
    for (int kk = 0; kk < KSUB; ++kk) {
      if (sub_k<Cfg>(w, kk) < krem) {
        frags(0, kk, 0);
        mma(0);
      }
    }
  }
  mma_end<Cfg>(acc);
  if constexpr (CK == kDumpC) {
    // the registers as the compiled fetch, LDS layout, fragment reads and
    // matrix instructions left them: fragments [buf][A 0..RM-1, B 0..RN-1],
    // then accumulators [i][j][v]
    unsigned* out = (unsigned*)p.D + ((int64_t)blockIdx.x * Cfg::kThreads + tid) * dump_words<Cfg>();
    int o = 0;
#pragma unroll
    for (int b = 0; b < NBUF; ++b) {
#pragma unroll
      for (int r = 0; r < RM + RN; ++r) {
        const half8 h = r < RM ? fa[b][r] : fb[b][r - RM];
        unsigned u[4];
        __builtin_memcpy(u, &h, 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) out[o++] = u[e];
      }
    }
#pragma unroll
    for (int i = 0; i < RM; ++i)
#pragma unroll
      for (int j = 0; j < RN; ++j)
#pragma unroll
        for (int v = 0; v < Cfg::kNV; ++v) out[o++] = __float_as_uint(acc[i][j][v]);
    return;
  }
  // Interior tiles with vector-aligned rows: vectors straight from the
  // registers.  Other tiles: split-K owners address each vector; the other
  // kernels stage through LDS into row runs of 4 (one code path less in the
  // kernels that hold every register).
  if constexpr (Cfg::WAVES_K > 1) {
    reduce_k_groups<Cfg>((float*)smem, w, lane, acc);
    const OwnedRows<Cfg> own{wave_k<Cfg>(w)};
    if (register_epilogue_ok<Cfg, CK, DK>(p, m0, n0))
      epilogue_regs<Cfg, CK, DK>(p, w, lane, m0, n0, acc, own);
    else
      epilogue_any<Cfg, CK, DK>(p, w, lane, m0, n0, acc, own);
  } else {
    if (register_epilogue_ok<Cfg, CK, DK>(p, m0, n0)) {
      if constexpr (CK == 2 && CViaLds<Cfg>::ok)
        epilogue_c_lds<Cfg, DK>(p, smem, w, lane, m0, n0, acc);
      else
        epilogue_regs<Cfg, CK, DK>(p, w, lane, m0, n0, acc);
    } else
      epilogue_lds<Cfg, CK, DK>(p, (float*)smem, w, lane, m0, n0, acc);
  }
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

  AccT<Cfg> acc[Cfg::RM][Cfg::RN];
  zero_acc<Cfg>(acc);
  mma_begin<Cfg>(acc);

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
        const int n = min(n0 + perm_n<Cfg>(b.row), p.N - 1);   // N-permuted rows
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
        for (int j = 0; j < Cfg::RN; ++j) Mma<Cfg::kOp>::run(af[i], bf[j], acc[i][j]);
    }
  }
  mma_end<Cfg>(acc);
  if (register_epilogue_ok<Cfg, CK, DK>(p, m0, n0))
    epilogue_regs<Cfg, CK, DK>(p, w, lane, m0, n0, acc);
  else
    epilogue_any<Cfg, CK, DK>(p, w, lane, m0, n0, acc);
}

// ---------------------------------------------------------------------------
// instantiation tables (one translation unit per tile configuration)
// ---------------------------------------------------------------------------
using KernelFn = void (*)(const GemmParams);

// [c_kind][d_kind-1]
template <class Cfg, int FA, int FB>
constexpr KernelFn tiled_table[3][2] = {
    {gemm_tiled<Cfg, FA, FB, 0, 1>, gemm_tiled<Cfg, FA, FB, 0, 2>},
    {gemm_tiled<Cfg, FA, FB, 1, 1>, gemm_tiled<Cfg, FA, FB, 1, 2>},
    {gemm_tiled<Cfg, FA, FB, 2, 1>, gemm_tiled<Cfg, FA, FB, 2, 2>}};

// Fetch policy pairs a configuration offers.  The 16x16x32 configurations
// issue their instruction with the accumulator tied by hand (Mma above), so
// the compiler must never move an accumulator between the first and the last
// instruction; that holds only where registers are not short.  They do not
// offer the transposing register fetch of an M-contiguous A, and the one with
// two waves per SIMD (256 registers per lane) offers only direct-to-LDS fetch.
// The build checks the generated code of every instance for such moves.
template <class Cfg>
constexpr bool offers(int fa, int fb) {
  // The four-wave 256x256 kernel with M-contiguous A straight into LDS and
  // B through registers: this compiler moves accumulators in a block where
  // the preceding matrix instructions' results may not be written yet, and
  // the build's check rejects it; that case runs on the eight-wave kernel.
  if (Cfg::kOp == kMfma32x32x16)
    return !(Cfg::BM == 256 && Cfg::kWaves == 4 && fa == kFetchDmaT && fb == kFetchReg);
  if (fa == kFetchRegT) return false;
  if (Cfg::kWaves > 4) return fb == kFetchDma && (fa == kFetchDma || fa == kFetchDmaT);
  return true;
}

template <class Cfg, int FA, int FB>
const void* instance(int ck, int dk) {
  if constexpr (offers<Cfg>(FA, FB))
    return (const void*)tiled_table<Cfg, FA, FB>[ck][dk - 1];
  else
    return nullptr;
}

// fetch policy pairs used: (A, B) = (DMA, DMA), (REG, REG), (REG, DMA),
// (DMA, REG), (REGT, DMA), (REGT, REG), (DMAT, DMA), (DMAT, REG)
template <class Cfg>
const void* tiled_symbol(int fa, int fb, int ck, int dk) {
  if (ck < 0 || ck > 2 || dk < 1 || dk > 2) return nullptr;
  if (fa == kFetchDma && fb == kFetchDma) return instance<Cfg, kFetchDma, kFetchDma>(ck, dk);
  if (fa == kFetchReg && fb == kFetchReg) return instance<Cfg, kFetchReg, kFetchReg>(ck, dk);
  if (fa == kFetchReg && fb == kFetchDma) return instance<Cfg, kFetchReg, kFetchDma>(ck, dk);
  if (fa == kFetchDma && fb == kFetchReg) return instance<Cfg, kFetchDma, kFetchReg>(ck, dk);
  if (fa == kFetchRegT && fb == kFetchDma) return instance<Cfg, kFetchRegT, kFetchDma>(ck, dk);
  if (fa == kFetchRegT && fb == kFetchReg) return instance<Cfg, kFetchRegT, kFetchReg>(ck, dk);
  if (fa == kFetchDmaT && fb == kFetchDma) return instance<Cfg, kFetchDmaT, kFetchDma>(ck, dk);
  if (fa == kFetchDmaT && fb == kFetchReg) return instance<Cfg, kFetchDmaT, kFetchReg>(ck, dk);
  return nullptr;
}

}  // namespace
}  // namespace mfl

// Kernel registry shared by the C ABI (host) and the kernel file.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_tile.hpp"

namespace mfl {

// Kernel arguments (passed by value).  Offsets inside A and B are 32-bit
// byte offsets, so each operand's span must stay below 2^31 bytes (checked
// by the C ABI before launch).
struct GemmParams {
  int M, N, K;
  int lda, ldb, ldc, ldd;
  int tiles_m, tiles_n, group_m;
  int d_vec;   // 1: D rows take aligned 4-element vector stores (base and ldd)
  int c_vec;   // 1: C rows take aligned 4-element vector loads (base and ldc)
  const void* A;
  const void* B;
  const void* C;
  void* D;
};

// values match mfl_algo in include/mfl_gemm.h
enum Algo : int {
  kAlgoAuto = 0,
  kAlgoDirect = 1,
  kAlgoLds128 = 2,
  kAlgoLds256 = 3,      // 8 waves of 128x64
  kAlgoLds256W4 = 4,    // 4 waves of 128x128
  kAlgoLds128W1 = 5,    // 1 wave of 128x128 per workgroup, 4 workgroups per CU
  kAlgoLdsSplitK = 6,   // 128x64 tile, 4 waves each taking a quarter of every K stage
  kAlgoLds256W4x16 = 7,   // 4 waves of 128x128, 16x16x32 instructions
  kAlgoLds256x16 = 8,     // 8 waves of 128x64, 16x16x32 instructions
  kAlgoLds128x16 = 9,     // 128x128x64, 4 waves of 64x64, 16x16x32 instructions
  kAlgoLdsSplitK16 = 10,  // 128x64x128, 2 K-groups of 4 waves of 32x64, 16x16x32
  kAlgoCount = 11
};

// how an operand tile travels from global memory to LDS
enum Fetch : int {
  kFetchDma = 0,    // global_load_lds_dwordx4 (K-contiguous, 16-byte aligned rows)
  kFetchReg = 1,    // 16-byte loads into registers, any 2-byte alignment
  kFetchRegT = 2,   // M-contiguous A, transposed in registers
  kFetchDmaT = 3,   // M-contiguous A, global_load_lds into an M-contiguous tile,
                    // fragments read with the transposing LDS read
};

// direct-from-global: 128x128 block (the simple-GEMM page's CTA tile), 2x2 waves
using CfgDirect = TileCfg<128, 128, 32, 2, 2>;
// 128x128x32 block tile, 2x2 waves of 64x64
using CfgLds128 = TileCfg<128, 128, 32, 2, 2>;
// 256x256x64 block tile, 2x4 waves of 128x64 (two waves per SIMD)
using CfgLds256 = TileCfg<256, 256, 64, 2, 4>;
// 256x256x64 block tile, 2x2 waves of 128x128 (one wave per SIMD); with a
// single wave per SIMD the fragments are read two K sub-steps ahead
using CfgLds256W4 = TileCfg<256, 256, 64, 2, 2, 2>;
// 128x128x32 block tile owned by a single wave (128x128, 4x4 atoms): no
// workgroup barrier to wait on, and four such workgroups share a CU
using CfgLds128W1 = TileCfg<128, 128, 32, 1, 1>;
// 128x64x128 block tile, 4 K-groups of one wave each: every wave computes
// the whole 128x64 tile over 32 of each stage's 128 k, then the four partial
// tiles are reduced through LDS.  256 workgroups of 4 waves fill the chip
// when the output has only 256 such tiles (small M x N, long K).  A step is
// only 16 MFMAs per wave, so tiles are fetched two steps ahead (three
// stages, 144 KB of LDS).
using CfgLdsSplitK = TileCfg<128, 64, 128, 1, 1, 1, 4, 3>;

// The same block tiles on v_mfma_f32_16x16x32_f16, the instruction that
// holds a higher clock under the power limit on random data (measured with
// the MFMA issue-rate kernel): one 64-deep stage is two 32-deep sub-steps.
using CfgLds256W4x16 = TileCfg<256, 256, 64, 2, 2, 1, 1, 2, kMfma16x16x32>;
using CfgLds256x16 = TileCfg<256, 256, 64, 2, 4, 1, 1, 2, kMfma16x16x32>;
using CfgLds128x16 = TileCfg<128, 128, 64, 2, 2, 1, 1, 2, kMfma16x16x32>;
// The split-K tile on it with two waves per SIMD: 2 K-groups of 4 waves of
// 32x64, so while one wave of a SIMD is held by a direct-to-LDS instruction
// that finds the CU's fetch path busy, the other issues MFMAs.
using CfgLdsSplitK16 = TileCfg<128, 64, 128, 4, 1, 1, 2, 3, kMfma16x16x32>;

static_assert(frag_c_is_partition_c<CfgLds128>() && frag_c_is_partition_c<CfgLds256>() &&
                  frag_c_is_partition_c<CfgLds256W4>() && frag_c_is_partition_c<CfgLds128W1>() &&
                  frag_c_is_partition_c<CfgLdsSplitK>() &&
                  frag_c_is_partition_c<CfgLds256W4x16>() &&
                  frag_c_is_partition_c<CfgLds256x16>() && frag_c_is_partition_c<CfgLds128x16>() &&
                  frag_c_is_partition_c<CfgLdsSplitK16>(),
              "accumulator coordinates must be the tiled MMA's partition_C");

struct KernelInfo {
  int algo, bm, bn, bk, threads;
};

KernelInfo kernel_info(int algo);
const void* kernel_symbol(int algo, int fetch_a, int fetch_b, int c_kind, int d_kind);
// 0 ok, -1 no such kernel, -2 launch error
int launch_gemm(int algo, int fetch_a, int fetch_b, int c_kind, int d_kind, const GemmParams& p,
                hipStream_t stream);

}  // namespace mfl

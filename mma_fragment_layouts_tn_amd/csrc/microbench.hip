// Measurement-only kernels: the rates the GEMM kernels are priced against.
//
//  * MFMA issue rate: every wave of a full-chip launch issues a long run of
//    independent f16 matrix instructions on operand registers filled from a
//    host-supplied buffer (random or zero data), with no memory traffic in
//    the loop.  This is the ceiling a GEMM K loop can reach on the same data
//    at the clock the chip holds under that load.
//  * LDS read rate: every wave of a full-chip launch issues 16-byte LDS reads
//    that touch each bank once per pass, with no other work.
//  * Direct-to-LDS fetch rate: every wave issues global_load_lds_dwordx4 from
//    a region of global memory that stays in L2, with no other work.
//
// Both record, per workgroup, the shader-clock cycle counter (s_memtime) and
// the constant 100 MHz real-time counter (s_memrealtime) before and after the
// loop, so the host obtains the shader clock the chip actually held during
// the measurement from the kernel itself.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "../../include/mfl_probe.h"

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kSets = 2;   // operand register sets, alternated between instructions

__device__ __forceinline__ void stamp(uint64_t* clocks, int slot) {
  // lane 0 of wave 0 records (cycles, real time) of its workgroup
  const uint64_t c = __builtin_amdgcn_s_memtime();
  const uint64_t r = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    clocks[4 * blockIdx.x + 2 * slot] = c;
    clocks[4 * blockIdx.x + 2 * slot + 1] = r;
  }
}

// One wave holds R x R accumulator tiles (the 128 x 128 fp32 tile a GEMM
// wave holds with either instruction) and kSets sets of R A and R B operand
// fragments; each set is used for all R*R instructions before the next, as
// a GEMM K loop uses its fragments of one K sub-step.
template <int OP>
__global__ void __launch_bounds__(256, 1) mfma_rate(const uint16_t* ops, int nops, int iters,
                                                    float* sink, uint64_t* clocks) {
  constexpr int R = OP == 0 ? 4 : 8;    // 4x4 tiles of 32x32, or 8x8 of 16x16
  using Acc = typename std::conditional<OP == 0, floatx16, floatx4>::type;
  constexpr int NV = OP == 0 ? 16 : 4;
  const int tid = blockIdx.x * blockDim.x + threadIdx.x;
  half8 a[kSets][R], b[kSets][R];
#pragma unroll
  for (int s = 0; s < kSets; ++s)
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int base = ((tid * kSets + s) * 2 * R + 2 * i) * 8;
      uint16_t ha[8], hb[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ha[e] = ops[(base + e) % nops];
        hb[e] = ops[(base + 8 + e) % nops];
      }
      __builtin_memcpy(&a[s][i], ha, 16);
      __builtin_memcpy(&b[s][i], hb, 16);
    }
  Acc acc[R][R];
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int j = 0; j < R; ++j)
#pragma unroll
      for (int v = 0; v < NV; ++v) acc[i][j][v] = 0.0f;
  __syncthreads();
  stamp(clocks, 0);
  // With the builtin, the compiler keeps the 16 sixteen-register accumulator
  // tuples of the 32x32 form in place, but rotates the 64 four-register
  // tuples of the 16x16 form through copies inside the loop.  The 16x16 form
  // is therefore issued as an instruction with its accumulator tied to one
  // AGPR tuple.  The compiler cannot see hazards through it: the wait states
  // before the loop cover the accumulators' initialisation, those after it
  // the last instructions' results (24 cycles, more than the instruction's
  // latency).  Inside the loop consecutive instructions use different
  // accumulators and operands that do not change.
  if constexpr (OP == 1) asm volatile("s_nop 7\n\ts_nop 7" ::);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int s = 0; s < kSets; ++s)
#pragma unroll
      for (int i = 0; i < R; ++i)
#pragma unroll
        for (int j = 0; j < R; ++j) {
          if constexpr (OP == 0)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[s][i], b[s][j], acc[i][j], 0, 0, 0);
          else
            asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0"
                         : "+a"(acc[i][j])
                         : "v"(a[s][i]), "v"(b[s][j]));
        }
  }
  if constexpr (OP == 1) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::);
  float t = 0.0f;
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int j = 0; j < R; ++j)
#pragma unroll
      for (int v = 0; v < NV; ++v) t += acc[i][j][v];
  __syncthreads();
  stamp(clocks, 1);
  sink[tid] = t;
}

// LDS read rate.  The workgroup's LDS (kLdsBytes, more than half the CU's
// 160 KB so one workgroup runs per CU) is filled once; then each wave reads
// 1 KB runs (lane l at byte 16 l of the run, so every 16-lane pass of a
// ds_read_b128 covers the 64 banks once), 16 reads per iteration in groups of
// DEPTH: a group's reads go to distinct registers and are all issued before
// the first is consumed, so DEPTH reads are in flight per wave.  The run
// index is taken modulo a runtime mask so the compiler cannot reuse a load;
// an empty asm statement consumes each loaded value.
constexpr int kLdsBytes = 96 * 1024, kLdsReadsPerIter = 16;

template <int DEPTH>
__global__ void __launch_bounds__(1024, 1) lds_read_rate(int iters, int run_mask,
                                                          uint32_t* sink, uint64_t* clocks) {
  static_assert(kLdsReadsPerIter % DEPTH == 0, "groups divide an iteration");
  __shared__ __attribute__((aligned(1024))) uint32_t lds[kLdsBytes / 4];
  for (int i = threadIdx.x; i < kLdsBytes / 4; i += blockDim.x) lds[i] = i * 2654435761u;
  __syncthreads();
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const char* base = (const char*)lds + lane * 16;
  stamp(clocks, 0);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int g = 0; g < kLdsReadsPerIter / DEPTH; ++g) {
      u32x4 v[DEPTH];
#pragma unroll
      for (int u = 0; u < DEPTH; ++u) {
        const int run = ((it * kLdsReadsPerIter + g * DEPTH + u + w * 3) & run_mask);
        v[u] = *(const u32x4*)(base + run * 1024);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < DEPTH; ++u) asm volatile("" ::"v"(v[u]));
    }
  }
  __syncthreads();
  stamp(clocks, 1);
  if (threadIdx.x == 0) sink[blockIdx.x] = lds[blockIdx.x % (kLdsBytes / 4)];
}

// Direct-to-LDS fetch rate.  Workgroup g re-reads its own 64 KB region of
// `buf` (L2-resident after the first pass) in 1 KB runs, lane l taking bytes
// 16 l .. 16 l + 15 of a run, straight into 1 KB slots of a 96 KB LDS array
// (one workgroup per CU); each wave issues DEPTH instructions, then waits
// for all of them.
constexpr int kDmaRegion = 64 * 1024;

template <int DEPTH>
__global__ void __launch_bounds__(1024, 1) dma_rate(const uint8_t* buf, int iters, uint32_t* sink,
                                                     uint64_t* clocks) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsBytes];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint8_t* base = buf + (size_t)blockIdx.x * kDmaRegion + lane * 16;
  __syncthreads();
  stamp(clocks, 0);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) {
      const int run = (it * DEPTH + u + w * 7) & (kDmaRegion / 1024 - 1);
      const int slot = (w * DEPTH + u) % (kLdsBytes / 1024);
      __builtin_amdgcn_global_load_lds((const void*)(base + run * 1024),
                                       (__attribute__((address_space(3))) void*)(lds + slot * 1024),
                                       16, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));   // vmcnt(0)
  }
  __syncthreads();
  stamp(clocks, 1);
  if (threadIdx.x == 0) sink[blockIdx.x] = lds[blockIdx.x % kLdsBytes];
}

}  // namespace

extern "C" int mfl_bench_mfma(int32_t op, const uint16_t* operands, int32_t n_operands,
                              int32_t iters, int32_t nwg, float* sink, uint64_t* clocks,
                              void* stream) {
  if ((op != 0 && op != 1) || !operands || n_operands <= 0 || iters <= 0 || nwg <= 0 ||
      nwg > 65536 || !sink || !clocks)
    return -4;
  hipStream_t s = (hipStream_t)stream;
  if (op == 0)
    hipLaunchKernelGGL(mfma_rate<0>, dim3(nwg), dim3(256), 0, s, operands, n_operands, iters,
                       sink, clocks);
  else
    hipLaunchKernelGGL(mfma_rate<1>, dim3(nwg), dim3(256), 0, s, operands, n_operands, iters,
                       sink, clocks);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int mfl_bench_lds_read(int32_t threads, int32_t iters, int32_t nwg, int32_t depth,
                                  uint32_t* sink, uint64_t* clocks, void* stream) {
  if (threads <= 0 || threads > 1024 || threads % 64 != 0 || iters <= 0 || nwg <= 0 ||
      nwg > 65536 || !sink || !clocks)
    return -4;
  // runs of 1 KB inside the 96 KB array: the mask keeps run indices below 64
  hipStream_t s = (hipStream_t)stream;
  switch (depth) {
    case 1: hipLaunchKernelGGL(lds_read_rate<1>, dim3(nwg), dim3(threads), 0, s, iters, 63, sink, clocks); break;
    case 4: hipLaunchKernelGGL(lds_read_rate<4>, dim3(nwg), dim3(threads), 0, s, iters, 63, sink, clocks); break;
    case 8: hipLaunchKernelGGL(lds_read_rate<8>, dim3(nwg), dim3(threads), 0, s, iters, 63, sink, clocks); break;
    case 16: hipLaunchKernelGGL(lds_read_rate<16>, dim3(nwg), dim3(threads), 0, s, iters, 63, sink, clocks); break;
    default: return -4;
  }
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int mfl_bench_dma_rate(int32_t threads, int32_t iters, int32_t nwg, int32_t depth,
                                  const uint8_t* buf, uint32_t* sink, uint64_t* clocks,
                                  void* stream) {
  if (threads <= 0 || threads > 1024 || threads % 64 != 0 || iters <= 0 || nwg <= 0 ||
      nwg > 65536 || !buf || !sink || !clocks)
    return -4;
  hipStream_t s = (hipStream_t)stream;
  switch (depth) {
    case 4: hipLaunchKernelGGL(dma_rate<4>, dim3(nwg), dim3(threads), 0, s, buf, iters, sink, clocks); break;
    case 12: hipLaunchKernelGGL(dma_rate<12>, dim3(nwg), dim3(threads), 0, s, buf, iters, sink, clocks); break;
    case 24: hipLaunchKernelGGL(dma_rate<24>, dim3(nwg), dim3(threads), 0, s, buf, iters, sink, clocks); break;
    default: return -4;
  }
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int mfl_wall_clock_khz(int32_t* khz) {
  if (!khz) return -4;
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&v, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
    return -5;
  *khz = v;
  return 0;
}

// Test-only kernel: one matrix instruction on slot values supplied by the
// host, so a test can recover the instruction's lane/slot <-> matrix maps.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mfl_probe.h"

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

template <int OP>
__global__ void __launch_bounds__(64) probe_mfma(const uint16_t* a, const uint16_t* b,
                                                 const float* c, float* d) {
  const int l = threadIdx.x;
  constexpr int VA = (OP == 0 || OP == 1) ? 8 : 4;
  constexpr int VC = (OP == 0 || OP == 2) ? 16 : 4;
  _Float16 av[VA], bv[VA];
  for (int i = 0; i < VA; ++i) {
    uint16_t x = a[l * VA + i], y = b[l * VA + i];
    __builtin_memcpy(&av[i], &x, 2);
    __builtin_memcpy(&bv[i], &y, 2);
  }
  if constexpr (OP == 0 || OP == 1) {
    half8 A, B;
    __builtin_memcpy(&A, av, 16);
    __builtin_memcpy(&B, bv, 16);
    if constexpr (OP == 0) {
      floatx16 C;
      for (int i = 0; i < 16; ++i) C[i] = c[l * 16 + i];
      C = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, B, C, 0, 0, 0);
      for (int i = 0; i < 16; ++i) d[l * 16 + i] = C[i];
    } else {
      floatx4 C;
      for (int i = 0; i < 4; ++i) C[i] = c[l * 4 + i];
      C = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B, C, 0, 0, 0);
      for (int i = 0; i < 4; ++i) d[l * 4 + i] = C[i];
    }
  } else {
    half4 A, B;
    __builtin_memcpy(&A, av, 8);
    __builtin_memcpy(&B, bv, 8);
    if constexpr (OP == 2) {
      floatx16 C;
      for (int i = 0; i < 16; ++i) C[i] = c[l * 16 + i];
      C = __builtin_amdgcn_mfma_f32_32x32x8f16(A, B, C, 0, 0, 0);
      for (int i = 0; i < 16; ++i) d[l * 16 + i] = C[i];
    } else {
      floatx4 C;
      for (int i = 0; i < 4; ++i) C[i] = c[l * 4 + i];
      C = __builtin_amdgcn_mfma_f32_16x16x16f16(A, B, C, 0, 0, 0);
      for (int i = 0; i < 4; ++i) d[l * 4 + i] = C[i];
    }
  }
  (void)VC;
}

struct LaneOffsets {
  int32_t h[64];
};

typedef short short4v __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(64) probe_tr16(const LaneOffsets offs, const uint16_t* in,
                                                 uint16_t* out) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[4096];
  const int l = threadIdx.x;
  for (int i = l; i < 4096; i += 64) lds[i] = in[i];
  __syncthreads();
  using lds_s4 = __attribute__((address_space(3))) short4v*;
  const short4v r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)(lds + offs.h[l]));
  for (int e = 0; e < 4; ++e) out[l * 4 + e] = (uint16_t)r[e];
}

}  // namespace

extern "C" int mfl_probe_lds_tr16(const int32_t* lane_offsets, const uint16_t* lds_in,
                                  uint16_t* out, void* stream) {
  if (!lane_offsets || !lds_in || !out) return -4;
  LaneOffsets offs;
  for (int l = 0; l < 64; ++l) {
    const int32_t h = lane_offsets[l];
    if (h < 0 || h > 4092 || h % 4 != 0) return -4;
    offs.h[l] = h;
  }
  hipLaunchKernelGGL(probe_tr16, dim3(1), dim3(64), 0, (hipStream_t)stream, offs, lds_in, out);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int mfl_probe_mfma(int32_t op, const uint16_t* a_slots, const uint16_t* b_slots,
                              const float* c_slots, float* d_out, void* stream) {
  if (!a_slots || !b_slots || !c_slots || !d_out) return -4;
  hipStream_t s = (hipStream_t)stream;
  switch (op) {
    case 0: hipLaunchKernelGGL(probe_mfma<0>, dim3(1), dim3(64), 0, s, a_slots, b_slots, c_slots, d_out); break;
    case 1: hipLaunchKernelGGL(probe_mfma<1>, dim3(1), dim3(64), 0, s, a_slots, b_slots, c_slots, d_out); break;
    case 2: hipLaunchKernelGGL(probe_mfma<2>, dim3(1), dim3(64), 0, s, a_slots, b_slots, c_slots, d_out); break;
    case 3: hipLaunchKernelGGL(probe_mfma<3>, dim3(1), dim3(64), 0, s, a_slots, b_slots, c_slots, d_out); break;
    default: return -4;
  }
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// Each workgroup records the XCD (the accelerator die of the 8 on the
// package) it runs on, read from the XCC_ID hardware register; lane 0 stores
// it with an ordinary vector store.
__global__ void __launch_bounds__(64) probe_xcc(int32_t* out) {
  unsigned id;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(id));
  if (threadIdx.x == 0) out[blockIdx.x] = (int32_t)(id & 0xf);
}

extern "C" int mfl_probe_xcc(int32_t nblocks, int32_t* out, void* stream) {
  if (nblocks <= 0 || nblocks > 65536 || !out) return -4;
  hipLaunchKernelGGL(probe_xcc, dim3(nblocks), dim3(64), 0, (hipStream_t)stream, out);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

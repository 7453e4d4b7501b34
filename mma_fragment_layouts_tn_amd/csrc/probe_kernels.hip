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

}  // namespace

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

// Kernel instances of the back-to-back GEMM: K in {32, 64, 128, 256}, D fp16 or fp32.
#include <hip/hip_runtime.h>

#include "chain.hpp"

namespace mfl {
const void* chain_symbol(int kd, int dk) {
  if (dk != 1 && dk != 2) return nullptr;
  switch (kd) {
    case 32: return dk == 1 ? (const void*)gemm_chain<32, 1> : (const void*)gemm_chain<32, 2>;
    case 64: return dk == 1 ? (const void*)gemm_chain<64, 1> : (const void*)gemm_chain<64, 2>;
    case 128: return dk == 1 ? (const void*)gemm_chain<128, 1> : (const void*)gemm_chain<128, 2>;
    case 256: return dk == 1 ? (const void*)gemm_chain<256, 1> : (const void*)gemm_chain<256, 2>;
    default: return nullptr;
  }
}
}  // namespace mfl

// Kernel instances of the back-to-back GEMM: K in {32, 64, 128, 256}, D fp16
// or fp32, operands staged direct-to-LDS or through registers.
#include <hip/hip_runtime.h>

#include "chain.hpp"

namespace mfl {
namespace {
template <int KD>
const void* pick(int dk, bool dma) {
  if (dma) return dk == 1 ? (const void*)gemm_chain<KD, 1, true> : (const void*)gemm_chain<KD, 2, true>;
  return dk == 1 ? (const void*)gemm_chain<KD, 1, false> : (const void*)gemm_chain<KD, 2, false>;
}
}  // namespace

const void* chain_symbol(int kd, int dk, bool dma) {
  if (dk != 1 && dk != 2) return nullptr;
  switch (kd) {
    case 32: return pick<32>(dk, dma);
    case 64: return pick<64>(dk, dma);
    case 128: return pick<128>(dk, dma);
    case 256: return pick<256>(dk, dma);
    default: return nullptr;
  }
}
}  // namespace mfl

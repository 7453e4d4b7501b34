// Kernel instances of the back-to-back GEMM: K in {32, 64, 128, 256}, D fp16
// or fp32, operands staged direct-to-LDS or through registers, N2 tiles of
// 64 or 128 columns.
#include <hip/hip_runtime.h>

#include "chain.hpp"

namespace mfl {
namespace {
template <int KD, int BN>
const void* pick(int dk, bool dma) {
  if (dma)
    return dk == 1 ? (const void*)gemm_chain<KD, 1, true, BN> : (const void*)gemm_chain<KD, 2, true, BN>;
  return dk == 1 ? (const void*)gemm_chain<KD, 1, false, BN> : (const void*)gemm_chain<KD, 2, false, BN>;
}
template <int KD>
const void* pick(int dk, bool dma, int bn) {
  return bn == 64 ? pick<KD, 64>(dk, dma) : bn == 128 ? pick<KD, 128>(dk, dma) : nullptr;
}
}  // namespace

const void* chain_symbol(int kd, int dk, bool dma, int bn) {
  if (dk != 1 && dk != 2) return nullptr;
  switch (kd) {
    case 32: return pick<32>(dk, dma, bn);
    case 64: return pick<64>(dk, dma, bn);
    case 128: return pick<128>(dk, dma, bn);
    case 256: return pick<256>(dk, dma, bn);
    default: return nullptr;
  }
}
const void* chain_timed_symbol() { return (const void*)gemm_chain<128, 1, true, 128, true>; }
}  // namespace mfl

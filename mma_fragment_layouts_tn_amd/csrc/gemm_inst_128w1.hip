// Kernel instances for the single-wave 128x128x32 tile configuration.
#include <hip/hip_runtime.h>

#include "gemm_kernels.hpp"

namespace mfl {
const void* tiled_symbol_128w1(int fa, int fb, int ck, int dk) {
  return tiled_symbol<CfgLds128W1>(fa, fb, ck, dk);
}
}  // namespace mfl

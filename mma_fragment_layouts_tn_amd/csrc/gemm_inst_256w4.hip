// Kernel instances for the 256w4 tile configuration.
#include <hip/hip_runtime.h>

#include "gemm_kernels.hpp"

namespace mfl {
const void* tiled_symbol_256w4(int fa, int fb, int ck, int dk) {
  return tiled_symbol<CfgLds256W4>(fa, fb, ck, dk);
}
}  // namespace mfl

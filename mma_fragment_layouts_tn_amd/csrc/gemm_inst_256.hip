// Kernel instances for the 256 tile configuration.
#include <hip/hip_runtime.h>

#include "gemm_kernels.hpp"

namespace mfl {
const void* tiled_symbol_256(int fa, int fb, int ck, int dk) {
  return tiled_symbol<CfgLds256>(fa, fb, ck, dk);
}
}  // namespace mfl

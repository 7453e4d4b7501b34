// Kernel instances for the 128x128x64, 4 waves, 16x16x32 tile configuration.
#include <hip/hip_runtime.h>

#include "gemm_kernels.hpp"

namespace mfl {
const void* tiled_symbol_128x16(int fa, int fb, int ck, int dk) {
  return tiled_symbol<CfgLds128x16>(fa, fb, ck, dk);
}
}  // namespace mfl

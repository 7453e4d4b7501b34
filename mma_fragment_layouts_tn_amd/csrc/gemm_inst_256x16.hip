// Kernel instances for the 256x256x64, 8 waves, 16x16x32 tile configuration.
#include <hip/hip_runtime.h>

#include "gemm_kernels.hpp"

namespace mfl {
const void* tiled_symbol_256x16(int fa, int fb, int ck, int dk) {
  return tiled_symbol<CfgLds256x16>(fa, fb, ck, dk);
}
}  // namespace mfl

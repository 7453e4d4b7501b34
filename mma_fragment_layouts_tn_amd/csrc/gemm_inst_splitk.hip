// Kernel instances for the split-K 128x64x128 tile configuration.
#include <hip/hip_runtime.h>

#include "gemm_kernels.hpp"

namespace mfl {
const void* tiled_symbol_splitk(int fa, int fb, int ck, int dk) {
  return tiled_symbol<CfgLdsSplitK>(fa, fb, ck, dk);
}
}  // namespace mfl

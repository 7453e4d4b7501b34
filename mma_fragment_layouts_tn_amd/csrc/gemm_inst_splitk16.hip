// Kernel instances for the 128x64x128 split-K tile on 16x16x32 instructions:
// 2 K-groups of 4 waves of 32x64.
#include <hip/hip_runtime.h>

#include "gemm_kernels.hpp"

namespace mfl {
const void* tiled_symbol_splitk16(int fa, int fb, int ck, int dk) {
  return tiled_symbol<CfgLdsSplitK16>(fa, fb, ck, dk);
}
}  // namespace mfl

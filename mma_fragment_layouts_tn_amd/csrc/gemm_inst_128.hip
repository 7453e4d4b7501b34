// Kernel instances for the 128 tile configuration.
#include <hip/hip_runtime.h>

#include "gemm_kernels.hpp"

namespace mfl {
const void* tiled_symbol_128(int fa, int fb, int ck, int dk) {
  return tiled_symbol<CfgLds128>(fa, fb, ck, dk);
}

const void* direct_symbol(int ck, int dk) {
  static constexpr KernelFn table[3][2] = {
      {gemm_direct<CfgDirect, 0, 1>, gemm_direct<CfgDirect, 0, 2>},
      {gemm_direct<CfgDirect, 1, 1>, gemm_direct<CfgDirect, 1, 2>},
      {gemm_direct<CfgDirect, 2, 1>, gemm_direct<CfgDirect, 2, 2>}};
  if (ck < 0 || ck > 2 || dk < 1 || dk > 2) return nullptr;
  return (const void*)table[ck][dk - 1];
}
}  // namespace mfl

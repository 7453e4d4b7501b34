// Kernel registry: tile shapes, symbol lookup and launch.
#include <hip/hip_runtime.h>

#include "gemm_launch.hpp"

namespace mfl {

const void* tiled_symbol_128(int fa, int fb, int ck, int dk);
const void* tiled_symbol_256(int fa, int fb, int ck, int dk);
const void* tiled_symbol_256w4(int fa, int fb, int ck, int dk);
const void* tiled_symbol_128w1(int fa, int fb, int ck, int dk);
const void* tiled_symbol_splitk(int fa, int fb, int ck, int dk);
const void* tiled_symbol_256w4x16(int fa, int fb, int ck, int dk);
const void* tiled_symbol_256x16(int fa, int fb, int ck, int dk);
const void* tiled_symbol_128x16(int fa, int fb, int ck, int dk);
const void* tiled_symbol_splitk16(int fa, int fb, int ck, int dk);
const void* direct_symbol(int ck, int dk);

namespace {
template <class Cfg>
KernelInfo info_of(int algo) {
  return KernelInfo{algo, Cfg::BM, Cfg::BN, Cfg::BK, Cfg::kThreads};
}
}  // namespace

KernelInfo kernel_info(int algo) {
  switch (algo) {
    case kAlgoDirect: return info_of<CfgDirect>(algo);
    case kAlgoLds128: return info_of<CfgLds128>(algo);
    case kAlgoLds256: return info_of<CfgLds256>(algo);
    case kAlgoLds256W4: return info_of<CfgLds256W4>(algo);
    case kAlgoLds128W1: return info_of<CfgLds128W1>(algo);
    case kAlgoLdsSplitK: return info_of<CfgLdsSplitK>(algo);
    case kAlgoLds256W4x16: return info_of<CfgLds256W4x16>(algo);
    case kAlgoLds256x16: return info_of<CfgLds256x16>(algo);
    case kAlgoLds128x16: return info_of<CfgLds128x16>(algo);
    case kAlgoLdsSplitK16: return info_of<CfgLdsSplitK16>(algo);
    default: return KernelInfo{-1, 0, 0, 0, 0};
  }
}

const void* kernel_symbol(int algo, int fetch_a, int fetch_b, int c_kind, int d_kind) {
  switch (algo) {
    case kAlgoDirect:
      return fetch_a == kFetchRegT || fetch_a == kFetchDmaT ? nullptr : direct_symbol(c_kind, d_kind);
    case kAlgoLds128: return tiled_symbol_128(fetch_a, fetch_b, c_kind, d_kind);
    case kAlgoLds256: return tiled_symbol_256(fetch_a, fetch_b, c_kind, d_kind);
    case kAlgoLds256W4: return tiled_symbol_256w4(fetch_a, fetch_b, c_kind, d_kind);
    case kAlgoLds128W1: return tiled_symbol_128w1(fetch_a, fetch_b, c_kind, d_kind);
    case kAlgoLdsSplitK: return tiled_symbol_splitk(fetch_a, fetch_b, c_kind, d_kind);
    case kAlgoLds256W4x16: return tiled_symbol_256w4x16(fetch_a, fetch_b, c_kind, d_kind);
    case kAlgoLds256x16: return tiled_symbol_256x16(fetch_a, fetch_b, c_kind, d_kind);
    case kAlgoLds128x16: return tiled_symbol_128x16(fetch_a, fetch_b, c_kind, d_kind);
    case kAlgoLdsSplitK16: return tiled_symbol_splitk16(fetch_a, fetch_b, c_kind, d_kind);
    default: return nullptr;
  }
}

int launch_gemm(int algo, int fetch_a, int fetch_b, int c_kind, int d_kind, const GemmParams& p,
                hipStream_t stream) {
  const void* fn = kernel_symbol(algo, fetch_a, fetch_b, c_kind, d_kind);
  const KernelInfo ki = kernel_info(algo);
  if (!fn || ki.algo < 0) return -1;
  const int64_t nb = (int64_t)p.tiles_m * p.tiles_n;
  void* args[] = {(void*)&p};
  const hipError_t e = hipLaunchKernel(fn, dim3((unsigned)nb), dim3(ki.threads), args, 0, stream);
  return e == hipSuccess ? 0 : -2;
}

}  // namespace mfl

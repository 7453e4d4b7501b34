// Test-only instances of the LDS kernels in register-dump mode (C kind
// kDumpC): each configuration once with both operands straight into LDS, and
// the register and transposing fetch paths on the configurations that use
// them.  A test fills A and B with values that encode their coordinates and
// reads back, per lane, what the compiled fetch, LDS layout, fragment reads
// and matrix instructions put in each register (the per-thread coordinate
// dump the simple-GEMM page prints for thread 0, "cute(7) simple_gemm" §4).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mfl_probe.h"
#include "gemm_kernels.hpp"

namespace mfl {

namespace {
template <class Cfg, int FA, int FB>
const void* dump_of() {
  return (const void*)gemm_tiled<Cfg, FA, FB, kDumpC, 2>;
}
}  // namespace

template <int ALGO, class Cfg, int FA, int FB>
struct DumpEntry {
  static bool take(int algo, int fa, int fb, int* words, int* threads, const void** fn) {
    if (algo != ALGO || fa != FA || fb != FB) return false;
    *words = dump_words<Cfg>();
    *threads = Cfg::kThreads;
    *fn = dump_of<Cfg, FA, FB>();
    return true;
  }
};

template <class... E>
const void* dump_lookup(int algo, int fa, int fb, int* words, int* threads) {
  const void* fn = nullptr;
  (void)(E::take(algo, fa, fb, words, threads, &fn) || ...);
  return fn;
}

// nullptr where no dump instance exists; *words: words per thread
const void* dump_symbol(int algo, int fa, int fb, int* words, int* threads) {
  return dump_lookup<DumpEntry<kAlgoLds128, CfgLds128, kFetchDma, kFetchDma>,
                     DumpEntry<kAlgoLds256, CfgLds256, kFetchDma, kFetchDma>,
                     DumpEntry<kAlgoLds256W4, CfgLds256W4, kFetchDma, kFetchDma>,
                     DumpEntry<kAlgoLds128W1, CfgLds128W1, kFetchDma, kFetchDma>,
                     DumpEntry<kAlgoLdsSplitK, CfgLdsSplitK, kFetchDma, kFetchDma>,
                     DumpEntry<kAlgoLds256W4x16, CfgLds256W4x16, kFetchDma, kFetchDma>,
                     DumpEntry<kAlgoLds256x16, CfgLds256x16, kFetchDma, kFetchDma>,
                     DumpEntry<kAlgoLds128x16, CfgLds128x16, kFetchDma, kFetchDma>,
                     DumpEntry<kAlgoLdsSplitK16, CfgLdsSplitK16, kFetchDma, kFetchDma>,
                     DumpEntry<kAlgoLds256, CfgLds256, kFetchReg, kFetchReg>,
                     DumpEntry<kAlgoLds256, CfgLds256, kFetchRegT, kFetchDma>,
                     DumpEntry<kAlgoLds256, CfgLds256, kFetchDmaT, kFetchDma>,
                     DumpEntry<kAlgoLds256W4x16, CfgLds256W4x16, kFetchReg, kFetchReg>,
                     DumpEntry<kAlgoLds256W4x16, CfgLds256W4x16, kFetchDmaT, kFetchDma>>(
      algo, fa, fb, words, threads);
}

// LDS-poisoned instances (test-only): a few configurations and fetch paths,
// C absent / fp16 / fp32 with the matching D
namespace {
template <class Cfg, int FA, int FB>
const void* poisoned_of(int ck) {
  switch (ck) {
    case 0: return (const void*)gemm_tiled<Cfg, FA, FB, 0, 2, true>;
    case 1: return (const void*)gemm_tiled<Cfg, FA, FB, 1, 1, true>;
    case 2: return (const void*)gemm_tiled<Cfg, FA, FB, 2, 2, true>;
    default: return nullptr;
  }
}

template <int ALGO, class Cfg, int FA, int FB>
struct PoisonEntry {
  static bool take(int algo, int fa, int fb, int ck, const void** fn) {
    if (algo != ALGO || fa != FA || fb != FB) return false;
    *fn = poisoned_of<Cfg, FA, FB>(ck);
    return true;
  }
};

template <class... E>
const void* poison_lookup(int algo, int fa, int fb, int ck) {
  const void* fn = nullptr;
  (void)(E::take(algo, fa, fb, ck, &fn) || ...);
  return fn;
}
}  // namespace

// nullptr where no poisoned instance exists (d_kind must be 2 for ck 0 and 2,
// 1 for ck 1)
const void* poisoned_symbol(int algo, int fa, int fb, int ck, int dk) {
  if ((ck == 1) != (dk == 1)) return nullptr;
  return poison_lookup<PoisonEntry<kAlgoLds128, CfgLds128, kFetchDma, kFetchDma>,
                       PoisonEntry<kAlgoLds128, CfgLds128, kFetchReg, kFetchReg>,
                       PoisonEntry<kAlgoLds256, CfgLds256, kFetchDmaT, kFetchDma>,
                       PoisonEntry<kAlgoLds256, CfgLds256, kFetchRegT, kFetchReg>,
                       PoisonEntry<kAlgoLds128W1, CfgLds128W1, kFetchDma, kFetchReg>,
                       PoisonEntry<kAlgoLdsSplitK, CfgLdsSplitK, kFetchDma, kFetchDma>,
                       PoisonEntry<kAlgoLds256W4x16, CfgLds256W4x16, kFetchReg, kFetchReg>,
                       PoisonEntry<kAlgoLds256x16, CfgLds256x16, kFetchDma, kFetchDma>,
                       PoisonEntry<kAlgoLds128x16, CfgLds128x16, kFetchDmaT, kFetchDma>,
                       PoisonEntry<kAlgoLdsSplitK16, CfgLdsSplitK16, kFetchDma, kFetchDma>>(
      algo, fa, fb, ck);
}

}  // namespace mfl

extern "C" int mfl_probe_fragments(int32_t algo, int32_t fetch_a, int32_t fetch_b, int32_t M,
                                   int32_t N, int32_t K, const uint16_t* A, int32_t lda,
                                   const uint16_t* B, int32_t ldb, uint32_t* out,
                                   int64_t out_words, int32_t* words_per_thread,
                                   int32_t* threads, void* stream) {
  int words = 0, nthr = 0;
  const void* fn = mfl::dump_symbol(algo, fetch_a, fetch_b, &words, &nthr);
  if (!fn) return -6;
  if (words_per_thread) *words_per_thread = words;
  if (threads) *threads = nthr;
  if (!out) return 0;   // query only
  const mfl::KernelInfo ki = mfl::kernel_info(algo);
  const bool mm = fetch_a == mfl::kFetchDmaT || fetch_a == mfl::kFetchRegT;
  // one whole K-step of whole tiles, operands inside their leading dimensions
  if (!A || !B || M <= 0 || N <= 0 || K != ki.bk || M % ki.bm || N % ki.bn) return -4;
  if ((mm ? lda < M : lda < K) || ldb < K) return -4;
  if (((uintptr_t)A | (uintptr_t)B) % 16 || lda % 8 || ldb % 8) return -4;   // 16-byte rows
  if (fetch_a == mfl::kFetchDmaT && M % 8) return -4;
  const int64_t tiles = (int64_t)(M / ki.bm) * (N / ki.bn);
  if (out_words < tiles * nthr * words) return -4;
  mfl::GemmParams p{};
  p.M = M;
  p.N = N;
  p.K = K;
  p.lda = lda;
  p.ldb = ldb;
  p.ldd = 0;
  p.tiles_m = M / ki.bm;
  p.tiles_n = N / ki.bn;
  p.group_m = ki.bm >= 256 ? 4 : 8;
  p.A = A;
  p.B = B;
  p.D = out;
  void* args[] = {(void*)&p};
  const hipError_t e = hipLaunchKernel(fn, dim3((unsigned)tiles), dim3(ki.threads), args, 0,
                                       (hipStream_t)stream);
  return e == hipSuccess ? 0 : -5;
}

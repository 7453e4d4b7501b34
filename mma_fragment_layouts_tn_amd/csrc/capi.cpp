// C ABI: argument checks, kernel choice and launch for gemm_tn (mfl_gemm.h),
// and the text interface of the layout module (mfl_layout.h).
#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <string>
#include <vector>

#include "../../include/mfl_gemm.h"
#include "../../include/mfl_chain.h"
#include "../../include/mfl_layout.h"
#include "../../include/mfl_probe.h"
#include "chain.hpp"
#include "gemm_launch.hpp"
#include "gemm_tile.hpp"
#include "layout.hpp"
#include "mfma_atoms.hpp"

namespace mfl {
const void* poisoned_symbol(int algo, int fa, int fb, int ck, int dk);
}

namespace {

using mfl::GemmParams;

int gemm_launch(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                int64_t ldb, const void* C, int64_t ldc, void* D, int64_t ldd,
                gemm_dtypes_t dtypes, void* stream, bool poisoned);

bool dtype_ok_cd(int32_t c, int32_t d) {
  return (c == MFL_NONE || c == MFL_F16 || c == MFL_F32) && (d == MFL_F16 || d == MFL_F32);
}

int64_t elem_size(int32_t t) { return t == MFL_F32 ? 4 : 2; }

// Largest byte offset an operand's fetch can form, relative to its base:
// rows x ld storage with `cols` valid elements in the last row.
bool span_fits(int64_t rows, int64_t ld, int64_t cols) {
  if (rows <= 0 || cols <= 0) return true;
  const int64_t last = (rows - 1) * ld + cols;   // elements
  return last * 2 < ((int64_t)1 << 31) - 64;
}

// direct-to-LDS loads move whole 16-byte chunks: the base and every row
// start must be 16-byte aligned
bool dma_ok(const void* X, int64_t ld) { return ((uintptr_t)X % 16 == 0) && (ld % 8 == 0); }

// Large outputs take the 256x256 tile.  Below that the 128x128 tile, unless
// its grid leaves CUs idle (fewer tiles than the 256 CUs) while K is long:
// then the split-K tile (128x64, its K split between groups of waves inside
// the workgroup) runs twice as many workgroups.
int pick_algo(int64_t M, int64_t N, int64_t K) {
  const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256);
  if (t256 >= 192) return mfl::kAlgoLds256;
  const int64_t t128 = ((M + 127) / 128) * ((N + 127) / 128);
  return t128 < 256 && K >= 1024 ? mfl::kAlgoLdsSplitK : mfl::kAlgoLds128;
}

struct Plan {
  int algo, fetch_a, fetch_b;
};

int check(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
          int64_t ldb, const void* C, int64_t ldc, const void* D, int64_t ldd,
          gemm_dtypes_t dt, Plan* plan) {
  if (M < 0 || N < 0 || K < 0) return MFL_E_NEGATIVE_DIM;
  if (dt.a != MFL_F16 || dt.b != MFL_F16 || !dtype_ok_cd(dt.c, dt.d)) return MFL_E_UNSUPPORTED;
  if (dt.a_order != MFL_A_KMAJOR && dt.a_order != MFL_A_MMAJOR) return MFL_E_UNSUPPORTED;
  if (dt.algo & ~(MFL_ALGO_MASK | MFL_ALGO_REG_FETCH)) return MFL_E_UNSUPPORTED;
  int algo = dt.algo & MFL_ALGO_MASK;
  const bool force_reg = (dt.algo & MFL_ALGO_REG_FETCH) != 0;
  if (algo >= MFL_ALGO_COUNT) return MFL_E_UNSUPPORTED;
  const bool mm = dt.a_order == MFL_A_MMAJOR;
  const int64_t one = 1;
  if (lda < (mm ? (M > one ? M : one) : (K > one ? K : one))) return MFL_E_LEADING_DIM;
  if (ldb < (K > one ? K : one)) return MFL_E_LEADING_DIM;
  if (dt.c != MFL_NONE && ldc < (N > one ? N : one)) return MFL_E_LEADING_DIM;
  if (ldd < (N > one ? N : one)) return MFL_E_LEADING_DIM;
  if ((dt.c == MFL_NONE) != (C == nullptr)) return MFL_E_NULL_POINTER;
  if (M > 0 && N > 0) {
    if (!D) return MFL_E_NULL_POINTER;
    if (K > 0 && (!A || !B)) return MFL_E_NULL_POINTER;
  }
  if (((uintptr_t)A & 1) || ((uintptr_t)B & 1)) return MFL_E_MISALIGNED;
  if (C && ((uintptr_t)C % (uintptr_t)elem_size(dt.c))) return MFL_E_MISALIGNED;
  if (D && ((uintptr_t)D % (uintptr_t)elem_size(dt.d))) return MFL_E_MISALIGNED;
  if (C && C == D && (ldc != ldd || dt.c != dt.d)) return MFL_E_ALIAS;
  if (M > INT_MAX / 2 || N > INT_MAX / 2 || K > INT_MAX / 2 || lda > INT_MAX ||
      ldb > INT_MAX || ldc > INT_MAX || ldd > INT_MAX)
    return MFL_E_TOO_LARGE;
  if (mm ? !span_fits(K, lda, M) : !span_fits(M, lda, K)) return MFL_E_TOO_LARGE;
  if (!span_fits(N, ldb, K)) return MFL_E_TOO_LARGE;
  const bool auto_algo = algo == MFL_ALGO_AUTO;
  if (auto_algo) algo = pick_algo(M, N, K);
  if (algo == MFL_ALGO_DIRECT && mm) return MFL_E_ALGO_CASE;
  const mfl::KernelInfo ki = mfl::kernel_info(algo);
  if (ki.algo < 0) return MFL_E_UNSUPPORTED;
  const int64_t tiles = ((M + ki.bm - 1) / ki.bm) * ((N + ki.bn - 1) / ki.bn);
  if (tiles > INT_MAX) return MFL_E_TOO_LARGE;
  if (plan) {
    plan->algo = algo;
    // M-contiguous A: straight into LDS when rows are 16-byte aligned and M
    // splits into whole 16-byte chunks, else transposed through registers
    if (mm)
      plan->fetch_a = !force_reg && dma_ok(A, lda) && M % 8 == 0 ? mfl::kFetchDmaT
                                                                 : mfl::kFetchRegT;
    else
      plan->fetch_a = !force_reg && dma_ok(A, lda) ? mfl::kFetchDma : mfl::kFetchReg;
    plan->fetch_b = !force_reg && dma_ok(B, ldb) ? mfl::kFetchDma : mfl::kFetchReg;
    // With both operands straight into LDS and no C, the same 256x256 tile
    // on v_mfma_f32_16x16x32_f16: the chip holds a higher clock with it under
    // the power limit (measured by the MFMA issue-rate kernel) and the
    // eight-wave kernel is the fastest at 4096^3.  Register fetch and C reads
    // stay on the 32x32x16 kernel, which measured faster there.
    if (auto_algo && algo == mfl::kAlgoLds256 && plan->fetch_a == mfl::kFetchDma &&
        plan->fetch_b == mfl::kFetchDma && dt.c == MFL_NONE)
      plan->algo = mfl::kAlgoLds256x16;
    // likewise the split-K tile, whose second wave per SIMD issues MFMAs
    // while the first is held by a fetch instruction (measured 4 % faster on
    // the 512 x 4096 x 4096 shard)
    if (auto_algo && algo == mfl::kAlgoLdsSplitK && plan->fetch_a == mfl::kFetchDma &&
        plan->fetch_b == mfl::kFetchDma && dt.c == MFL_NONE)
      plan->algo = mfl::kAlgoLdsSplitK16;
    // a forced configuration without an instance for this fetch path
    if (plan->algo != mfl::kAlgoDirect &&
        !mfl::kernel_symbol(plan->algo, plan->fetch_a, plan->fetch_b, dt.c, dt.d))
      return MFL_E_ALGO_CASE;
  }
  return MFL_OK;
}

// ------------------------------------------------------- layout text form
struct Parser {
  const char* s;
  int pos = 0;
  bool ok = true;
  void ws() {
    while (s[pos] == ' ') ++pos;
  }
  bool number(int64_t& v) {
    ws();
    if (s[pos] == '_') ++pos;
    bool neg = false;
    if (s[pos] == '-') {
      neg = true;
      ++pos;
    }
    if (s[pos] < '0' || s[pos] > '9') return false;
    int64_t x = 0;
    while (s[pos] >= '0' && s[pos] <= '9') {
      x = x * 10 + (s[pos] - '0');
      if (x > ((int64_t)1 << 40)) return false;
      ++pos;
    }
    v = neg ? -x : x;
    return true;
  }
  // flatten everything below the top level into one list of leaves
  bool leaves(int64_t* out, int& n, int cap) {
    ws();
    if (s[pos] == '(') {
      ++pos;
      for (;;) {
        if (!leaves(out, n, cap)) return false;
        ws();
        if (s[pos] == ',') {
          ++pos;
          continue;
        }
        if (s[pos] == ')') {
          ++pos;
          return true;
        }
        return false;
      }
    }
    int64_t v;
    if (!number(v)) return false;
    if (n >= cap) return false;
    out[n++] = v;
    return true;
  }
  // top level: list of modes, each a flat leaf list; mode_len[] sizes
  bool top(int64_t* out, int& n, int* mode_len, int& nm) {
    ws();
    n = 0;
    nm = 0;
    if (s[pos] != '(') {
      int before = n;
      if (!leaves(out, n, mfl::kMaxLeaves)) return false;
      mode_len[nm++] = n - before;
      return true;
    }
    ++pos;
    for (;;) {
      if (nm >= mfl::kMaxModes) return false;
      int before = n;
      if (!leaves(out, n, mfl::kMaxLeaves)) return false;
      mode_len[nm++] = n - before;
      ws();
      if (s[pos] == ',') {
        ++pos;
        continue;
      }
      if (s[pos] == ')') {
        ++pos;
        return true;
      }
      return false;
    }
  }
};

int parse_layout(const char* text, mfl::Layout& L) {
  if (!text) return mfl::kLayoutBadText;
  const char* colon = strchr(text, ':');
  if (!colon) return mfl::kLayoutBadText;
  std::string shape_txt(text, colon - text), stride_txt(colon + 1);
  int64_t sh[mfl::kMaxLeaves], st[mfl::kMaxLeaves];
  int nsh = 0, nst = 0, ml_sh[mfl::kMaxModes], ml_st[mfl::kMaxModes], nm_sh = 0, nm_st = 0;
  Parser p1{shape_txt.c_str()}, p2{stride_txt.c_str()};
  if (!p1.top(sh, nsh, ml_sh, nm_sh) || !p2.top(st, nst, ml_st, nm_st))
    return mfl::kLayoutBadText;
  p1.ws();
  p2.ws();
  if (p1.s[p1.pos] != 0 || p2.s[p2.pos] != 0) return mfl::kLayoutBadText;
  if (nsh != nst || nm_sh != nm_st) return mfl::kLayoutBadText;
  for (int m = 0; m < nm_sh; ++m)
    if (ml_sh[m] != ml_st[m]) return mfl::kLayoutBadText;
  L = mfl::Layout{};
  int k = 0;
  for (int m = 0; m < nm_sh; ++m) {
    L.open_mode();
    for (int i = 0; i < ml_sh[m]; ++i, ++k) {
      if (sh[k] <= 0) return mfl::kLayoutBadText;
      L.push_leaf(sh[k], st[k]);
    }
  }
  // the size and every offset of the domain must fit int64 (then plain
  // evaluation inside the domain cannot overflow)
  int ovf = mfl::kLayoutOk;
  mfl::size(L, &ovf);
  int64_t reach = 0;
  for (int i = 0; i < L.nleaves; ++i)
    reach = mfl::ck_add(reach, mfl::ck_mul(L.shape[i] - 1, L.stride[i] < 0 ? -L.stride[i]
                                                                          : L.stride[i], ovf),
                        ovf);
  if (ovf != mfl::kLayoutOk) return ovf;
  return L.status;
}

std::string print_mode(const mfl::Layout& L, int m, bool strides) {
  const int b = L.mode_begin(m), e = L.mode_end[m];
  const int64_t* v = strides ? L.stride : L.shape;
  if (e - b == 1) return std::to_string(v[b]);
  std::string s = "(";
  for (int i = b; i < e; ++i) {
    if (i > b) s += ",";
    s += std::to_string(v[i]);
  }
  return s + ")";
}

std::string print_layout(const mfl::Layout& L) {
  auto part = [&](bool strides) {
    if (L.nmodes == 1) return print_mode(L, 0, strides);
    std::string s = "(";
    for (int m = 0; m < L.nmodes; ++m) {
      if (m) s += ",";
      s += print_mode(L, m, strides);
    }
    return s + ")";
  };
  return part(false) + ":" + part(true);
}

int emit(const mfl::Layout& L, char* out, int64_t cap) {
  if (L.status != mfl::kLayoutOk) return L.status;
  const std::string s = print_layout(L);
  if (!out || (int64_t)s.size() + 1 > cap) return mfl::kLayoutBadIndex;
  memcpy(out, s.c_str(), s.size() + 1);
  return 0;
}

// a shape alone, "(8,(2,4,2))": modes of leaves with unit strides
int parse_shape(const char* text, mfl::Layout& S) {
  if (!text) return mfl::kLayoutBadText;
  int64_t sh[mfl::kMaxLeaves];
  int n = 0, ml[mfl::kMaxModes], nm = 0;
  Parser p{text};
  if (!p.top(sh, n, ml, nm)) return mfl::kLayoutBadText;
  p.ws();
  if (p.s[p.pos] != 0) return mfl::kLayoutBadText;
  S = mfl::Layout{};
  int k = 0;
  for (int m = 0; m < nm; ++m) {
    S.open_mode();
    for (int i = 0; i < ml[m]; ++i, ++k) {
      if (sh[k] <= 0) return mfl::kLayoutBadText;
      S.push_leaf(sh[k], 1);
    }
  }
  return S.status;
}

// Tiler text: one layout (divide the whole layout), or "T0;T1;..." with one
// entry per top-level mode, "_" keeping that mode whole ("T0;" for a single
// per-mode entry).  `whole` tells which form was given.
int parse_tiler(const char* tiler, mfl::Layout* tl, bool* has, int& nt, bool& whole) {
  if (!tiler) return mfl::kLayoutBadText;
  const std::string t(tiler);
  nt = 0;
  whole = t.find(';') == std::string::npos && t.find('_') == std::string::npos;
  if (whole) {
    has[0] = true;
    nt = 1;
    return parse_layout(tiler, tl[0]);
  }
  size_t pos = 0;
  for (;;) {
    const size_t e = t.find(';', pos);
    std::string item = t.substr(pos, e == std::string::npos ? std::string::npos : e - pos);
    item.erase(0, item.find_first_not_of(' '));
    item.erase(item.find_last_not_of(' ') + 1);
    if (item.empty() && e == std::string::npos && nt > 0) break;   // "T0;": one entry
    if (nt >= mfl::kMaxModes) return mfl::kLayoutTooLarge;
    if (item == "_") {
      has[nt++] = false;
    } else {
      const int rc = parse_layout(item.c_str(), tl[nt]);
      if (rc) return rc;
      has[nt++] = true;
    }
    if (e == std::string::npos) break;
    pos = e + 1;
  }
  return 0;
}

int divide_text(const char* a, const char* tiler, bool zipped, char* out, int64_t cap) {
  mfl::Layout A;
  int rc = parse_layout(a, A);
  if (rc) return rc;
  mfl::Layout tl[mfl::kMaxModes];
  bool has[mfl::kMaxModes] = {};
  int nt = 0;
  bool whole = false;
  rc = parse_tiler(tiler, tl, has, nt, whole);
  if (rc) return rc;
  if (whole) return emit(mfl::logical_divide(A, tl[0], true), out, cap);
  if (nt > A.nmodes) return mfl::kLayoutBadIndex;
  return emit(zipped ? mfl::zipped_divide(A, tl, has, nt, true)
                     : mfl::logical_divide_modes(A, tl, has, nt, true),
              out, cap);
}

template <class Cfg>
int lds_offsets(int operand, int32_t* out, int64_t cap, int32_t* outer, int32_t* inner) {
  if (operand < 0 || operand > 2) return mfl::kLayoutBadIndex;
  // operands 0/1: (row, k) K-contiguous; 2: (k, m) of an M-contiguous A
  const int O = operand == 0 ? Cfg::BM : operand == 1 ? Cfg::BN : Cfg::BK;
  const int I = operand == 2 ? Cfg::BM : Cfg::BK;
  if (outer) *outer = O;
  if (inner) *inner = I;
  if (!out) return 0;
  if ((int64_t)O * I > cap) return mfl::kLayoutBadIndex;
  for (int o = 0; o < O; ++o)
    for (int i = 0; i < I; ++i)
      out[o * I + i] = operand == 2 ? mfl::lds_offset_mn<Cfg::BM>(i, o)
                                    : mfl::lds_offset<Cfg::BK>(o, i);
  return 0;
}

template <class Cfg>
int frag_coords(int operand, int32_t* out, int64_t cap, int32_t* threads, int32_t* slots) {
  // per thread: its own K sub-steps of one stage (KSUB_W; all of them unless
  // the tile splits K between groups of waves)
  int ns = 0;
  if (operand == 0) ns = Cfg::KSUB_W * Cfg::RM * 8;
  else if (operand == 1) ns = Cfg::KSUB_W * Cfg::RN * 8;
  else if (operand == 2) ns = Cfg::RM * Cfg::RN * Cfg::kNV;
  else if (operand == 3) ns = Cfg::KSUB_W * Cfg::RM;
  else return mfl::kLayoutBadIndex;
  if (threads) *threads = Cfg::kThreads;
  if (slots) *slots = ns;
  if (!out) return 0;
  if ((int64_t)2 * Cfg::kThreads * ns > cap) return mfl::kLayoutBadIndex;
  for (int t = 0; t < Cfg::kThreads; ++t) {
    const int w = t / 64, lane = t % 64;
    int s = 0;
    auto put = [&](int a, int b) {
      out[2 * ((int64_t)t * ns + s) + 0] = a;
      out[2 * ((int64_t)t * ns + s) + 1] = b;
      ++s;
    };
    if (operand == 3) {
      for (int kk = 0; kk < Cfg::KSUB_W; ++kk)
        for (int i = 0; i < Cfg::RM; ++i) {
          const mfl::RowK c = mfl::frag_a_tr_coord<Cfg>(w, lane, i, kk);
          put(c.row, c.k);
        }
    } else if (operand == 2) {
      for (int i = 0; i < Cfg::RM; ++i)
        for (int j = 0; j < Cfg::RN; ++j)
          for (int v = 0; v < Cfg::kNV; ++v) {
            const mfl::RowK c = mfl::frag_c_coord<Cfg>(w, lane, i, j, v);
            put(c.row, c.k);
          }
    } else {
      const int R = operand == 0 ? Cfg::RM : Cfg::RN;
      for (int kk = 0; kk < Cfg::KSUB_W; ++kk)
        for (int i = 0; i < R; ++i)
          for (int v = 0; v < 8; ++v) {
            const mfl::RowK c = operand == 0 ? mfl::frag_a_coord<Cfg>(w, lane, i, kk)
                                             : mfl::frag_b_coord<Cfg>(w, lane, i, kk);
            put(c.row, c.k + v);
          }
    }
  }
  return 0;
}

}  // namespace

// back-to-back GEMM: argument checks shared by launch and validate
int chain_check(int64_t batch, int64_t M, int64_t N1, int64_t N2, int64_t K, const void* A,
                int64_t lda, int64_t sa, const void* B, int64_t ldb, int64_t sb, const void* W,
                int64_t ldw, int64_t sw, const void* D, int64_t ldd, int64_t sd, int32_t dk) {
  if (batch < 0 || M < 0 || N1 < 0 || N2 < 0 || K < 0) return MFL_E_NEGATIVE_DIM;
  if (K != 32 && K != 64 && K != 128 && K != 256) return MFL_E_UNSUPPORTED;
  if (dk != MFL_F16 && dk != MFL_F32) return MFL_E_UNSUPPORTED;
  const int64_t one = 1;
  if (lda < K || ldb < K || ldw < (N1 > one ? N1 : one) || ldd < (N2 > one ? N2 : one))
    return MFL_E_LEADING_DIM;
  if (sa < 0 || sb < 0 || sw < 0 || sd < 0) return MFL_E_LEADING_DIM;
  // bounds that keep every offset below (row * ld, batch * stride, M * ldd)
  // far inside int64: 2^48 elements is beyond any device's memory
  if (M > INT_MAX / 2 || N1 > INT_MAX / 2 || N2 > INT_MAX / 2 || batch > INT_MAX ||
      lda > INT_MAX || ldb > INT_MAX || ldw > INT_MAX || ldd > INT_MAX)
    return MFL_E_TOO_LARGE;
  const int64_t span = int64_t(1) << 48;
  for (const int64_t st : {sa, sb, sw, sd})
    if (st > 0 && batch > span / st) return MFL_E_TOO_LARGE;
  if (batch > 1 && M > 0 && N2 > 0 && sd < M * ldd) return MFL_E_ALIAS;
  const bool work = batch > 0 && M > 0 && N2 > 0;
  if (work && !D) return MFL_E_NULL_POINTER;
  if (work && N1 > 0 && (!A || !B || !W)) return MFL_E_NULL_POINTER;
  if (((uintptr_t)A & 1) || ((uintptr_t)B & 1) || ((uintptr_t)W & 1)) return MFL_E_MISALIGNED;
  if (D && ((uintptr_t)D % (uintptr_t)elem_size(dk))) return MFL_E_MISALIGNED;
  const int64_t bn = mfl::chain::tile_n(N2);
  const int64_t tiles = batch * ((M + mfl::chain::BM - 1) / mfl::chain::BM) * ((N2 + bn - 1) / bn);
  if (tiles > INT_MAX) return MFL_E_TOO_LARGE;
  return MFL_OK;
}

// direct-to-LDS staging: whole N1 chunks (64 columns, 32 at K = 256) and
// 16-byte aligned rows of B and W in every batch
bool chain_dma(int64_t K, int64_t N1, const void* B, int64_t ldb, int64_t sb, const void* W,
               int64_t ldw, int64_t sw) {
  return N1 % mfl::chain::chunk_width((int)K) == 0 && dma_ok(B, ldb) && dma_ok(W, ldw) &&
         sb % 8 == 0 && sw % 8 == 0;
}

// launch of the back-to-back GEMM; `timed` takes the phase-stamp instance
// (K = 128, fp16 D, direct-to-LDS staging, 128-column N2 tiles only)
int chain_launch(bool timed, int64_t batch, int64_t M, int64_t N1, int64_t N2, int64_t K,
                 const void* A, int64_t lda, int64_t stride_a, const void* B, int64_t ldb,
                 int64_t stride_b, const void* W, int64_t ldw, int64_t stride_w, void* D,
                 int64_t ldd, int64_t stride_d, int32_t d_dtype, uint32_t* stamps, void* stream) {
  const int rc = chain_check(batch, M, N1, N2, K, A, lda, stride_a, B, ldb, stride_b, W, ldw,
                             stride_w, D, ldd, stride_d, d_dtype);
  if (rc != MFL_OK) return rc;
  if (batch == 0 || M == 0 || N2 == 0) return MFL_OK;
  const int bn = mfl::chain::tile_n(N2);
  const bool dma = chain_dma(K, N1, B, ldb, stride_b, W, ldw, stride_w);
  const void* fn = timed ? (K == 128 && d_dtype == MFL_F16 && dma && bn == 128
                                ? mfl::chain_timed_symbol()
                                : nullptr)
                         : mfl::chain_symbol((int)K, d_dtype, dma, bn);
  if (!fn) return MFL_E_UNSUPPORTED;
  mfl::ChainParams p{};
  p.batch = (int)batch;
  p.M = (int)M;
  p.N1 = (int)N1;
  p.N2 = (int)N2;
  p.lda = lda;
  p.ldb = ldb;
  p.ldw = ldw;
  p.ldd = ldd;
  p.sa = stride_a;
  p.sb = stride_b;
  p.sw = stride_w;
  p.sd = stride_d;
  p.tiles_m = (int)(batch * ((M + mfl::chain::BM - 1) / mfl::chain::BM));
  p.tiles_n = (int)((N2 + bn - 1) / bn);
  p.group_m = 8;
  p.d_vec = ((uintptr_t)D % (uintptr_t)(4 * elem_size(d_dtype)) == 0) && (ldd % 4 == 0) &&
            (stride_d % 4 == 0);
  p.A = A;
  p.B = B;
  p.W = W;
  p.D = D;
  p.stamps = stamps;
  void* args[] = {(void*)&p};
  const int64_t nb = (int64_t)p.tiles_m * p.tiles_n;
  const hipError_t e = hipLaunchKernel(fn, dim3((unsigned)nb), dim3(mfl::chain::threads((int)K)), args, 0,
                                       (hipStream_t)stream);
  return e == hipSuccess ? MFL_OK : MFL_E_LAUNCH;
}


extern "C" {

int gemm_tn_validate(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                     const void* B, int64_t ldb, const void* C, int64_t ldc, const void* D,
                     int64_t ldd, gemm_dtypes_t dtypes, int32_t* algo_out) {
  Plan plan{};
  const int rc = check(M, N, K, A, lda, B, ldb, C, ldc, D, ldd, dtypes, &plan);
  if (rc == MFL_OK && algo_out) *algo_out = plan.algo;
  return rc;
}

int gemm_tn_plan(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                 int64_t ldb, const void* C, int64_t ldc, const void* D, int64_t ldd,
                 gemm_dtypes_t dtypes, int32_t* algo, int32_t* fetch_a, int32_t* fetch_b) {
  Plan plan{};
  const int rc = check(M, N, K, A, lda, B, ldb, C, ldc, D, ldd, dtypes, &plan);
  if (rc == MFL_OK) {
    if (algo) *algo = plan.algo;
    if (fetch_a) *fetch_a = plan.fetch_a;
    if (fetch_b) *fetch_b = plan.fetch_b;
  }
  return rc;
}

int gemm_tn(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
            int64_t ldb, const void* C, int64_t ldc, void* D, int64_t ldd,
            gemm_dtypes_t dtypes, void* stream) {
  return gemm_launch(M, N, K, A, lda, B, ldb, C, ldc, D, ldd, dtypes, stream, false);
}

int mfl_probe_gemm_poisoned(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                            const void* B, int64_t ldb, const void* C, int64_t ldc, void* D,
                            int64_t ldd, gemm_dtypes_t dtypes, void* stream) {
  return gemm_launch(M, N, K, A, lda, B, ldb, C, ldc, D, ldd, dtypes, stream, true);
}
}  // extern "C"

namespace {
int gemm_launch(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                int64_t ldb, const void* C, int64_t ldc, void* D, int64_t ldd,
                gemm_dtypes_t dtypes, void* stream, bool poisoned) {
  Plan plan{};
  const int rc = check(M, N, K, A, lda, B, ldb, C, ldc, D, ldd, dtypes, &plan);
  if (rc != MFL_OK) return rc;
  if (M == 0 || N == 0) return MFL_OK;
  const mfl::KernelInfo ki = mfl::kernel_info(plan.algo);
  GemmParams p{};
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  p.lda = (int)lda;
  p.ldb = (int)ldb;
  p.ldc = (int)(dtypes.c == MFL_NONE ? 0 : ldc);
  p.ldd = (int)ldd;
  p.tiles_m = (int)((M + ki.bm - 1) / ki.bm);
  p.tiles_n = (int)((N + ki.bn - 1) / ki.bn);
  p.group_m = ki.bm >= 256 ? 4 : 8;
  p.d_vec = ((uintptr_t)D % (uintptr_t)(4 * elem_size(dtypes.d)) == 0) && (ldd % 4 == 0);
  p.c_vec = C && ((uintptr_t)C % (uintptr_t)(4 * elem_size(dtypes.c)) == 0) && (ldc % 4 == 0);
  p.A = A;
  p.B = B;
  p.C = C;
  p.D = D;
  if (poisoned) {
    const void* fn = mfl::poisoned_symbol(plan.algo, plan.fetch_a, plan.fetch_b, dtypes.c,
                                          dtypes.d);
    if (!fn) return MFL_E_ALGO_CASE;
    void* args[] = {(void*)&p};
    const hipError_t e = hipLaunchKernel(fn, dim3((unsigned)(p.tiles_m * p.tiles_n)),
                                         dim3(ki.threads), args, 0, (hipStream_t)stream);
    return e == hipSuccess ? MFL_OK : MFL_E_LAUNCH;
  }
  const int lr = mfl::launch_gemm(plan.algo, plan.fetch_a, plan.fetch_b, dtypes.c, dtypes.d, p,
                                  (hipStream_t)stream);
  return lr == 0 ? MFL_OK : (lr == -1 ? MFL_E_UNSUPPORTED : MFL_E_LAUNCH);
}
}  // namespace

namespace {

// retile_D's regrouping (retile page, "读懂 CuTe 的 retile_D", sections
// "先确定要从哪些 fragment 位置取值" to "两个 K fragment 怎样连成一组"), from
// where each value lies in the copy's reference tile.
//
// The copy's TV layout maps thread t's copy value c to a position of the
// reference tile (positions numbered first coordinate fastest) and must cover
// the tile once.  The tiled copy orders a thread's values as the MMA orders
// its fragment: copy values c of one block b = c / V (V = the fragment's
// value count, mode 0) are the V values of one MMA, value c % V.  Which
// fragment repeat that block is follows from where the block lies: walking
// each tile axis from the origin, the block numbers met, in order of first
// appearance, are the repeat coordinates along that axis (block numbers are
// additive over the axes).  So copy value c of a thread is the fragment
// element (c % V, g_1 + e_1 r_1, ..., g_n + e_n r_n), with (g_d) the block's
// axis coordinates, e_d the blocks along axis d, and (r_d) the repeats the
// copy leaves (fragment mode d / e_d).  The result has mode 0 = (value of one
// copy instruction, instruction) -> register slot, then one mode per r_d;
// each part is factored from the table and the whole table is compared.
mfl::Layout retile_by_position(const mfl::Layout& frag, const mfl::Layout& tv,
                               const mfl::Layout& shape, int64_t nthr, int64_t nval) {
  mfl::Layout bad;
  bad.status = mfl::kLayoutBadIndex;
  const int nd = shape.nmodes;
  if (frag.nmodes != nd + 1 || nd < 1 || nd > mfl::kMaxModes - 1) return bad;
  const int64_t P = mfl::size(shape);
  if (P <= 0 || P > (int64_t(1) << 20) || mfl::size(tv) != P || P % nthr != 0) return bad;
  const int64_t V = mfl::size_mode(frag, 0);
  const int64_t per_thr = P / nthr;
  if (V < 1 || per_thr % V != 0 || per_thr % nval != 0) return bad;
  const int64_t K = per_thr / V;   // blocks (MMAs) per thread
  // position -> TV index, and its block number
  std::vector<int64_t> blk(P, -1);
  for (int64_t q = 0; q < P; ++q) {
    const int64_t p = mfl::eval(tv, q);
    if (p < 0 || p >= P || blk[p] >= 0) return bad;   // not a cover of the tile
    blk[p] = (q / nthr) / V;
  }
  // block numbers met along each axis, in order of first appearance
  int64_t ext[mfl::kMaxModes] = {}, stride[mfl::kMaxModes] = {};
  std::vector<std::vector<int64_t>> seen(nd);
  int64_t st = 1, nblocks = 1;
  for (int d = 0; d < nd; ++d) {
    ext[d] = mfl::size_mode(shape, d);
    stride[d] = st;
    st *= ext[d];
    for (int64_t x = 0; x < ext[d]; ++x) {
      const int64_t b = blk[x * stride[d]];
      bool have = false;
      for (int64_t y : seen[d]) have = have || y == b;
      if (!have) seen[d].push_back(b);
    }
    nblocks *= (int64_t)seen[d].size();
  }
  if (nblocks != K) return bad;
  // additivity: the block of a position is the sum of its axis blocks
  for (int64_t p = 0; p < P; ++p) {
    int64_t sum = 0, rem = p;
    for (int d = 0; d < nd; ++d) {
      sum += blk[(rem % ext[d]) * stride[d]];
      rem /= ext[d];
    }
    if (sum != blk[p]) {
      mfl::Layout nc;
      nc.status = mfl::kLayoutNotComposable;
      return nc;
    }
  }
  // axis coordinates of every block
  std::vector<std::vector<int64_t>> gcoord(K, std::vector<int64_t>(nd, -1));
  std::vector<int64_t> g(nd, 0);
  for (int64_t cell = 0; cell < K; ++cell) {
    int64_t rem = cell, b = 0;
    for (int d = 0; d < nd; ++d) {
      g[d] = rem % (int64_t)seen[d].size();
      rem /= (int64_t)seen[d].size();
      b += seen[d][g[d]];
    }
    if (b < 0 || b >= K || gcoord[b][0] >= 0) return bad;
    gcoord[b] = g;
  }
  // repeats the copy leaves along each fragment mode
  int64_t reps[mfl::kMaxModes] = {};
  for (int d = 0; d < nd; ++d) {
    const int64_t fm = mfl::size_mode(frag, d + 1), e = (int64_t)seen[d].size();
    if (fm % e != 0) return bad;
    reps[d] = fm / e;
  }
  // register slot of copy value c with leftover repeats given as one index
  auto slot = [&](int64_t c, const int64_t* r) {
    const int64_t b = c / V;
    int64_t off = mfl::eval_mode(frag, 0, c % V);
    for (int d = 0; d < nd; ++d)
      off += mfl::eval_mode(frag, d + 1, gcoord[b][d] + (int64_t)seen[d].size() * r[d]);
    return off;
  };
  const int64_t zero[mfl::kMaxModes] = {};
  const int64_t base = slot(0, zero);
  mfl::Layout out;
  // mode 0: values of one instruction, then instructions (kept as two parts)
  mfl::append_factored(out, nval, [&](int64_t j) { return slot(j, zero) - base; });
  mfl::Layout groups;
  mfl::append_factored(groups, per_thr / nval,
                       [&](int64_t gi) { return slot(nval * gi, zero) - base; });
  for (int i = 0; i < groups.nleaves; ++i) out.push_leaf(groups.shape[i], groups.stride[i]);
  for (int d = 0; d < nd; ++d) {
    mfl::append_factored(out, reps[d], [&](int64_t rd) {
      int64_t r[mfl::kMaxModes] = {};
      r[d] = rd;
      return slot(0, r) - base;
    });
  }
  if (out.status != mfl::kLayoutOk || groups.status != mfl::kLayoutOk) return bad;
  if (base != 0) {
    mfl::Layout nc;
    nc.status = mfl::kLayoutNotComposable;
    return nc;
  }
  // the whole table: every copy value of every leftover repeat
  int64_t nrest = 1;
  for (int d = 0; d < nd; ++d) nrest *= reps[d];
  for (int64_t ri = 0; ri < nrest; ++ri) {
    int64_t r[mfl::kMaxModes] = {}, rem = ri, idx = 0;
    for (int d = 0; d < nd; ++d) {
      r[d] = rem % reps[d];
      rem /= reps[d];
    }
    for (int64_t c = 0; c < per_thr; ++c) {
      int64_t got = mfl::eval_mode(out, 0, c);
      for (int d = 0; d < nd; ++d) got += mfl::eval_mode(out, d + 1, r[d]);
      (void)idx;
      if (got != slot(c, r)) {
        mfl::Layout nc;
        nc.status = mfl::kLayoutNotComposable;
        return nc;
      }
    }
  }
  return out;
}

}  // namespace

extern "C" {

const char* gemm_strerror(int code) {
  switch (code) {
    case MFL_OK: return "ok";
    case MFL_E_NEGATIVE_DIM: return "negative dimension";
    case MFL_E_LEADING_DIM: return "leading dimension too small";
    case MFL_E_NULL_POINTER: return "null pointer (or C pointer inconsistent with its dtype)";
    case MFL_E_UNSUPPORTED: return "unsupported dtype, A order or algorithm";
    case MFL_E_LAUNCH: return "HIP kernel launch failed";
    case MFL_E_ALGO_CASE: return "the forced algorithm cannot run this case";
    case MFL_E_MISALIGNED: return "pointer not aligned to its element size";
    case MFL_E_ALIAS: return "D aliases C with a different leading dimension or dtype";
    case MFL_E_TOO_LARGE: return "size beyond the supported index range";
    default: return "unknown error code";
  }
}

int mfl_kernel_info(int32_t algo, gemm_dtypes_t dt, int32_t* bm, int32_t* bn, int32_t* bk,
                    int32_t* threads, int32_t* lds_bytes, int32_t* vgprs_spilled) {
  algo &= MFL_ALGO_MASK;
  const mfl::KernelInfo ki = mfl::kernel_info(algo);
  if (ki.algo < 0 || !dtype_ok_cd(dt.c, dt.d)) return MFL_E_UNSUPPORTED;
  if (bm) *bm = ki.bm;
  if (bn) *bn = ki.bn;
  if (bk) *bk = ki.bk;
  if (threads) *threads = ki.threads;
  const int fa = dt.a_order == MFL_A_MMAJOR ? mfl::kFetchDmaT : mfl::kFetchDma;
  const void* fn = mfl::kernel_symbol(algo, fa, mfl::kFetchDma, dt.c, dt.d);
  if (!fn) return MFL_E_ALGO_CASE;
  if (lds_bytes || vgprs_spilled) {
    hipFuncAttributes attr{};
    if (hipFuncGetAttributes(&attr, fn) != hipSuccess) return MFL_E_LAUNCH;
    if (lds_bytes) *lds_bytes = (int32_t)attr.sharedSizeBytes;
    if (vgprs_spilled) *vgprs_spilled = (int32_t)attr.localSizeBytes;
  }
  return MFL_OK;
}

// ------------------------------------------------------------ layout C ABI
int mfl_layout_size(const char* layout, int64_t* out) {
  mfl::Layout L;
  const int rc = parse_layout(layout, L);
  if (rc) return rc;
  if (out) *out = mfl::size(L);
  return 0;
}

int mfl_layout_cosize(const char* layout, int64_t* out) {
  mfl::Layout L;
  const int rc = parse_layout(layout, L);
  if (rc) return rc;
  for (int i = 0; i < L.nleaves; ++i)
    if (L.stride[i] < 0) return mfl::kLayoutNegativeStride;
  if (out) *out = mfl::cosize(L);
  return 0;
}

int mfl_layout_eval(const char* layout, int64_t idx, int64_t* out) {
  mfl::Layout L;
  const int rc = parse_layout(layout, L);
  if (rc) return rc;
  if (idx < 0 || idx >= mfl::size(L)) return mfl::kLayoutBadIndex;
  if (out) *out = mfl::eval(L, idx);
  return 0;
}

int mfl_layout_table(const char* layout, int64_t* out, int64_t cap) {
  mfl::Layout L;
  const int rc = parse_layout(layout, L);
  if (rc) return rc;
  const int64_t n = mfl::size(L);
  if (!out || n > cap) return mfl::kLayoutBadIndex;
  for (int64_t i = 0; i < n; ++i) out[i] = mfl::eval(L, i);
  return 0;
}

int mfl_layout_coalesce(const char* layout, char* out, int64_t cap) {
  mfl::Layout L;
  const int rc = parse_layout(layout, L);
  if (rc) return rc;
  return emit(mfl::coalesce(L), out, cap);
}

int mfl_layout_compose(const char* a, const char* b, char* out, int64_t cap) {
  mfl::Layout A, B;
  int rc = parse_layout(a, A);
  if (rc) return rc;
  rc = parse_layout(b, B);
  if (rc) return rc;
  // inputs whose leaves interact (the result would not be A o B) are rejected
  return emit(mfl::compose_v(A, B, true), out, cap);
}

int mfl_layout_complement(const char* layout, int64_t cotarget, char* out, int64_t cap) {
  mfl::Layout L;
  const int rc = parse_layout(layout, L);
  if (rc) return rc;
  if (cotarget < 1 || cotarget > ((int64_t)1 << 40)) return mfl::kLayoutBadIndex;
  return emit(mfl::complement(L, cotarget), out, cap);
}

int mfl_layout_logical_divide(const char* a, const char* tiler, char* out, int64_t cap) {
  return divide_text(a, tiler, false, out, cap);
}

int mfl_layout_zipped_divide(const char* a, const char* tiler, char* out, int64_t cap) {
  return divide_text(a, tiler, true, out, cap);
}

int mfl_layout_logical_product(const char* a, const char* b, char* out, int64_t cap) {
  mfl::Layout A, B;
  int rc = parse_layout(a, A);
  if (rc) return rc;
  rc = parse_layout(b, B);
  if (rc) return rc;
  return emit(mfl::logical_product(A, B, true), out, cap);
}

int mfl_layout_tiled_product(const char* a, const char* b, char* out, int64_t cap) {
  mfl::Layout A, B;
  int rc = parse_layout(a, A);
  if (rc) return rc;
  rc = parse_layout(b, B);
  if (rc) return rc;
  return emit(mfl::tiled_product(A, B, true), out, cap);
}

int mfl_layout_upcast(const char* layout, int64_t n, char* out, int64_t cap) {
  mfl::Layout L;
  const int rc = parse_layout(layout, L);
  if (rc) return rc;
  if (n < 1) return mfl::kLayoutBadIndex;
  return emit(mfl::upcast(L, n), out, cap);
}

int mfl_layout_with_shape(const char* layout, const char* shape, char* out, int64_t cap) {
  mfl::Layout L, S;
  int rc = parse_layout(layout, L);
  if (rc) return rc;
  rc = parse_shape(shape, S);
  if (rc) return rc;
  if (mfl::size(S) != mfl::size(L)) return mfl::kLayoutBadIndex;
  return emit(mfl::with_shape(L, S, true), out, cap);
}

int mfl_layout_partition_c(const char* c, const char* tile, const char* atom_tv, int64_t atom_m,
                           int64_t atom_n, int64_t warps_m, int64_t warps_n, char* thr_out,
                           char* val_out, int64_t cap) {
  mfl::Layout C, TV;
  int rc = parse_layout(c, C);
  if (rc) return rc;
  rc = parse_layout(atom_tv, TV);
  if (rc) return rc;
  if (C.nmodes != 2 || atom_m < 1 || atom_n < 1 || warps_m < 1 || warps_n < 1)
    return mfl::kLayoutBadIndex;
  mfl::Layout tl[mfl::kMaxModes];
  const mfl::Layout* tp = nullptr;
  if (tile && *tile) {
    bool has[mfl::kMaxModes] = {}, whole = false;
    int nt = 0;
    rc = parse_tiler(tile, tl, has, nt, whole);
    if (rc) return rc;
    if (whole || nt != 2) return mfl::kLayoutBadText;
    for (int m = 0; m < 2; ++m)
      if (!has[m]) tl[m] = mfl::unit_leaf(m == 0 ? atom_m * warps_m : atom_n * warps_n);
    tp = tl;
  }
  const mfl::CPartition p = mfl::partition_c(C, tp, TV, atom_m, atom_n, warps_m, warps_n, true);
  rc = emit(p.thr, thr_out, cap);
  if (rc) return rc;
  return emit(p.val, val_out, cap);
}

int mfl_layout_retile(const char* frag, const char* tv, const char* tile_shape, int64_t nthr,
                      int64_t atom_nval, char* out, int64_t cap) {
  mfl::Layout F, TV, S;
  int rc = parse_layout(frag, F);
  if (rc) return rc;
  rc = parse_layout(tv, TV);
  if (rc) return rc;
  rc = parse_shape(tile_shape, S);
  if (rc) return rc;
  if (nthr < 1 || atom_nval < 1) return mfl::kLayoutBadIndex;
  return emit(retile_by_position(F, TV, S, nthr, atom_nval), out, cap);
}

int mfl_layout_right_inverse(const char* layout, char* out, int64_t cap) {
  mfl::Layout L;
  const int rc = parse_layout(layout, L);
  if (rc) return rc;
  return emit(mfl::right_inverse(L), out, cap);
}

int mfl_layout_mfma_tv(int32_t op, int32_t operand, char* out, int64_t cap) {
  if (op < 0 || op >= mfl::kMfmaOpCount || operand < 0 || operand > 2)
    return mfl::kLayoutBadIndex;
  return emit(mfl::mfma_tv(op, operand), out, cap);
}

int mfl_lds_tile_offsets(int32_t algo, int32_t operand, int32_t* out, int64_t cap,
                         int32_t* outer, int32_t* inner) {
  switch (algo & MFL_ALGO_MASK) {
    case mfl::kAlgoLds128: return lds_offsets<mfl::CfgLds128>(operand, out, cap, outer, inner);
    case mfl::kAlgoLds256: return lds_offsets<mfl::CfgLds256>(operand, out, cap, outer, inner);
    case mfl::kAlgoLds256W4:
      return lds_offsets<mfl::CfgLds256W4>(operand, out, cap, outer, inner);
    case mfl::kAlgoLds128W1:
      return lds_offsets<mfl::CfgLds128W1>(operand, out, cap, outer, inner);
    case mfl::kAlgoLdsSplitK:
      return lds_offsets<mfl::CfgLdsSplitK>(operand, out, cap, outer, inner);
    case mfl::kAlgoLds256W4x16:
      return lds_offsets<mfl::CfgLds256W4x16>(operand, out, cap, outer, inner);
    case mfl::kAlgoLds256x16:
      return lds_offsets<mfl::CfgLds256x16>(operand, out, cap, outer, inner);
    case mfl::kAlgoLds128x16:
      return lds_offsets<mfl::CfgLds128x16>(operand, out, cap, outer, inner);
    case mfl::kAlgoLdsSplitK16:
      return lds_offsets<mfl::CfgLdsSplitK16>(operand, out, cap, outer, inner);
    default: return mfl::kLayoutBadIndex;
  }
}

int mfl_chain_k_perm(int32_t* out) {
  constexpr mfl::ChainPerm pi = mfl::chain_k_perm();
  static_assert(pi.ok, "accumulator -> operand map");
  if (!out) return mfl::kLayoutBadIndex;
  for (int p = 0; p < 32; ++p) out[p] = pi.n1[p];
  return 0;
}

int mfl_tile_order(int32_t tiles_m, int32_t tiles_n, int32_t group_m, int32_t* tm, int32_t* tn) {
  if (tiles_m <= 0 || tiles_n <= 0 || group_m <= 0 || !tm || !tn) return mfl::kLayoutBadIndex;
  const int nb = tiles_m * tiles_n;
  for (int b = 0; b < nb; ++b) {
    const mfl::TileIndex t = mfl::tile_of_block(b, nb, tiles_m, tiles_n, group_m);
    tm[b] = t.tm;
    tn[b] = t.tn;
  }
  return 0;
}

int mfl_fragment_coords(int32_t algo, int32_t operand, int32_t* out, int64_t cap,
                        int32_t* threads, int32_t* slots) {
  switch (algo & MFL_ALGO_MASK) {
    case mfl::kAlgoDirect: return frag_coords<mfl::CfgDirect>(operand, out, cap, threads, slots);
    case mfl::kAlgoLds128: return frag_coords<mfl::CfgLds128>(operand, out, cap, threads, slots);
    case mfl::kAlgoLds256: return frag_coords<mfl::CfgLds256>(operand, out, cap, threads, slots);
    case mfl::kAlgoLds256W4: return frag_coords<mfl::CfgLds256W4>(operand, out, cap, threads, slots);
    case mfl::kAlgoLds128W1: return frag_coords<mfl::CfgLds128W1>(operand, out, cap, threads, slots);
    case mfl::kAlgoLdsSplitK: return frag_coords<mfl::CfgLdsSplitK>(operand, out, cap, threads, slots);
    case mfl::kAlgoLds256W4x16:
      return frag_coords<mfl::CfgLds256W4x16>(operand, out, cap, threads, slots);
    case mfl::kAlgoLds256x16:
      return frag_coords<mfl::CfgLds256x16>(operand, out, cap, threads, slots);
    case mfl::kAlgoLds128x16:
      return frag_coords<mfl::CfgLds128x16>(operand, out, cap, threads, slots);
    case mfl::kAlgoLdsSplitK16:
      return frag_coords<mfl::CfgLdsSplitK16>(operand, out, cap, threads, slots);
    default: return mfl::kLayoutBadIndex;
  }
}

int gemm_tn_chain_validate(int64_t batch, int64_t M, int64_t N1, int64_t N2, int64_t K,
                           const void* A, int64_t lda, int64_t stride_a, const void* B,
                           int64_t ldb, int64_t stride_b, const void* W, int64_t ldw,
                           int64_t stride_w, const void* D, int64_t ldd, int64_t stride_d,
                           int32_t d_dtype) {
  return chain_check(batch, M, N1, N2, K, A, lda, stride_a, B, ldb, stride_b, W, ldw, stride_w,
                     D, ldd, stride_d, d_dtype);
}

int gemm_tn_chain_plan(int64_t batch, int64_t M, int64_t N1, int64_t N2, int64_t K,
                       const void* A, int64_t lda, int64_t stride_a, const void* B, int64_t ldb,
                       int64_t stride_b, const void* W, int64_t ldw, int64_t stride_w,
                       const void* D, int64_t ldd, int64_t stride_d, int32_t d_dtype,
                       int32_t* staging, int32_t* tile_n) {
  const int rc = chain_check(batch, M, N1, N2, K, A, lda, stride_a, B, ldb, stride_b, W, ldw,
                             stride_w, D, ldd, stride_d, d_dtype);
  if (rc == MFL_OK && staging)
    *staging = chain_dma(K, N1, B, ldb, stride_b, W, ldw, stride_w) ? MFL_CHAIN_STAGE_DMA
                                                                  : MFL_CHAIN_STAGE_REGS;
  if (rc == MFL_OK && tile_n) *tile_n = mfl::chain::tile_n(N2);
  return rc;
}

int gemm_tn_chain(int64_t batch, int64_t M, int64_t N1, int64_t N2, int64_t K, const void* A,
                  int64_t lda, int64_t stride_a, const void* B, int64_t ldb, int64_t stride_b,
                  const void* W, int64_t ldw, int64_t stride_w, void* D, int64_t ldd,
                  int64_t stride_d, int32_t d_dtype, void* stream) {
  return chain_launch(false, batch, M, N1, N2, K, A, lda, stride_a, B, ldb, stride_b, W, ldw,
                      stride_w, D, ldd, stride_d, d_dtype, nullptr, stream);
}

int mfl_probe_chain_phases(int64_t batch, int64_t M, int64_t N1, int64_t N2, int64_t K,
                           const void* A, int64_t lda, int64_t stride_a, const void* B,
                           int64_t ldb, int64_t stride_b, const void* W, int64_t ldw,
                           int64_t stride_w, void* D, int64_t ldd, int64_t stride_d,
                           int32_t d_dtype, uint32_t* stamps, void* stream) {
  if (!stamps) return MFL_E_NULL_POINTER;
  return chain_launch(true, batch, M, N1, N2, K, A, lda, stride_a, B, ldb, stride_b, W, ldw,
                      stride_w, D, ldd, stride_d, d_dtype, stamps, stream);
}

}  // extern "C"

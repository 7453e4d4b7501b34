// AddressSanitizer / UndefinedBehaviorSanitizer driver for the C ABI's host
// code (capi.cpp, built with sanitizers on its host part only): every layout
// text operation on valid and malformed text with exact and too-small output
// capacities, the fragment-coordinate, LDS-offset and tile-order exports at
// the exact sizes they report, and the GEMM and chain argument checks over
// many argument combinations.  Nothing is launched and no GPU is touched.
// Exit 0 when every expected result holds.
#include <stdint.h>
#include <limits.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <string>
#include <vector>

#include "../../include/mfl_chain.h"
#include "../../include/mfl_gemm.h"
#include "../../include/mfl_layout.h"

static int fails = 0;
#define EXPECT(c)                                                        \
  do {                                                                   \
    if (!(c)) {                                                          \
      ++fails;                                                           \
      fprintf(stderr, "failed at line %d: %s\n", __LINE__, #c);          \
    }                                                                    \
  } while (0)

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u() {
  state ^= state << 13;
  state ^= state >> 7;
  state ^= state << 17;
  return state;
}
static int64_t rnd(int64_t n) { return n > 0 ? (int64_t)(next_u() % (uint64_t)n) : 0; }

// a dimension: mostly small, sometimes at the edges of the int32 / int64 range
static int64_t dim(int64_t small) {
  static const int64_t edge[] = {0, 1, -1, (1ll << 31) - 1, 1ll << 31, 1ll << 40, 1ll << 62,
                                 INT64_MAX, INT64_MIN};
  return rnd(8) ? rnd(small) - 5 : edge[rnd(9)];
}

static std::string random_layout() {
  const int nm = 1 + (int)rnd(3);
  std::string sh = nm > 1 ? "(" : "", st = nm > 1 ? "(" : "";
  for (int m = 0; m < nm; ++m) {
    const int nl = 1 + (int)rnd(3);
    if (m) {
      sh += ",";
      st += ",";
    }
    if (nl > 1) {
      sh += "(";
      st += "(";
    }
    for (int l = 0; l < nl; ++l) {
      if (l) {
        sh += ",";
        st += ",";
      }
      static const int64_t big[] = {1ll << 20, 1ll << 31, 3037000500ll, 1ll << 40, 1ll << 62,
                                    INT64_MAX};
      sh += std::to_string(rnd(40) ? 1 + rnd(6) : big[rnd(6)]);
      st += std::to_string(rnd(40) ? rnd(40) : (rnd(2) ? 1 : -1) * big[rnd(6)]);
    }
    if (nl > 1) {
      sh += ")";
      st += ")";
    }
  }
  if (nm > 1) {
    sh += ")";
    st += ")";
  }
  return sh + ":" + st;
}

static std::string mangle(std::string s) {
  switch (rnd(6)) {
    case 0: if (!s.empty()) s.erase(rnd((int64_t)s.size()), 1); break;
    case 1: s.insert(rnd((int64_t)s.size() + 1), 1, "(),:_-x 9"[rnd(9)]); break;
    case 2: s += "99999999999999999999"; break;
    case 3: s = s.substr(0, rnd((int64_t)s.size() + 1)); break;
    default: break;
  }
  return s;
}

int main(int argc, char** argv) {
  if (argc > 1) state += strtoull(argv[1], nullptr, 10) * 0x2545F4914F6CDD1Dull;
  char out[4096], out2[4096];
  // text operations: any outcome but a crash or an out-of-bounds access
  for (int it = 0; it < 3000; ++it) {
    const std::string a = mangle(random_layout()), b = mangle(random_layout());
    int64_t v = 0;
    mfl_layout_size(a.c_str(), &v);
    mfl_layout_cosize(a.c_str(), &v);
    mfl_layout_eval(a.c_str(), rnd(200) - 10, &v);
    const int64_t cap = rnd(6) == 0 ? rnd(8) : (int64_t)sizeof(out);
    mfl_layout_coalesce(a.c_str(), out, cap);
    mfl_layout_compose(a.c_str(), b.c_str(), out, cap);
    mfl_layout_right_inverse(a.c_str(), out, cap);
    mfl_layout_complement(a.c_str(), rnd(300), out, cap);
    mfl_layout_logical_divide(a.c_str(), b.c_str(), out, cap);
    mfl_layout_zipped_divide(a.c_str(), b.c_str(), out, cap);
    mfl_layout_logical_product(a.c_str(), b.c_str(), out, cap);
    mfl_layout_tiled_product(a.c_str(), b.c_str(), out, cap);
    mfl_layout_upcast(a.c_str(), 1 + rnd(16), out, cap);
    mfl_layout_with_shape(a.c_str(), "(8,(2,4,2))", out, cap);
    int64_t n = 0;
    if (mfl_layout_size(a.c_str(), &n) == 0 && n > 0 && n < 100000) {
      std::vector<int64_t> t((size_t)n);
      EXPECT(mfl_layout_table(a.c_str(), t.data(), n) == 0);
      EXPECT(mfl_layout_table(a.c_str(), t.data(), n - 1) != 0);   // one short
    }
  }
  // partition_C and retile on the instruction layouts, then on mangled text
  for (int op = 0; op < 2; ++op) {
    char tv[1024];
    EXPECT(mfl_layout_mfma_tv(op, 2, tv, sizeof(tv)) == 0);
    const int am = op == 0 ? 32 : 16;
    for (int wm = 1; wm <= 4; wm *= 2)
      for (int wn = 1; wn <= 4; wn *= 2) {
        const std::string c = "(" + std::to_string(am * wm * 2) + "," +
                              std::to_string(am * wn * 2) + "):(" +
                              std::to_string(am * wn * 2) + ",1)";
        EXPECT(mfl_layout_partition_c(c.c_str(), "", tv, am, am, wm, wn, out, out2,
                                      sizeof(out)) == 0);
        EXPECT(mfl_layout_partition_c(c.c_str(), "", tv, am, am, wm, wn, out, out2, 3) != 0);
        for (int it = 0; it < 20; ++it)
          mfl_layout_partition_c(mangle(c).c_str(), rnd(3) ? "" : mangle(random_layout()).c_str(),
                                 mangle(tv).c_str(), am, am, wm + rnd(3) - 1, wn, out, out2,
                                 rnd(4) ? (int64_t)sizeof(out) : rnd(16));
      }
  }
  const char* frag = "((2,2,2),1,1):((1,2,4),0,0)";
  const char* ctv = "((4,8),(2,2)):((16,1),(8,128))";
  for (int it = 0; it < 500; ++it)
    mfl_layout_retile(rnd(2) ? frag : mangle(frag).c_str(), rnd(2) ? ctv : mangle(ctv).c_str(),
                      rnd(2) ? "(16,8)" : mangle("(16,8)").c_str(), 32 * (1 + rnd(2)), 1 + rnd(4),
                      out, rnd(4) ? (int64_t)sizeof(out) : rnd(16));
  for (int op = -1; op < 5; ++op)
    for (int operand = -1; operand < 4; ++operand) mfl_layout_mfma_tv(op, operand, out, 16);

  // kernel maps at the sizes they report
  for (int algo = 0; algo < 12; ++algo) {
    for (int operand = -1; operand < 5; ++operand) {
      int32_t th = 0, sl = 0;
      if (mfl_fragment_coords(algo, operand, nullptr, 0, &th, &sl) == 0 && th > 0 && sl > 0) {
        std::vector<int32_t> f((size_t)2 * th * sl);
        EXPECT(mfl_fragment_coords(algo, operand, f.data(), (int64_t)f.size(), &th, &sl) == 0);
        EXPECT(mfl_fragment_coords(algo, operand, f.data(), (int64_t)f.size() - 1, &th, &sl) !=
               0);
      }
      int32_t o = 0, i = 0;
      if (mfl_lds_tile_offsets(algo, operand, nullptr, 0, &o, &i) == 0 && o > 0 && i > 0) {
        std::vector<int32_t> f((size_t)o * i);
        EXPECT(mfl_lds_tile_offsets(algo, operand, f.data(), (int64_t)f.size(), &o, &i) == 0);
      }
    }
  }
  for (int it = 0; it < 200; ++it) {
    const int tm = 1 + (int)rnd(40), tn = 1 + (int)rnd(40), g = 1 + (int)rnd(9);
    std::vector<int32_t> a((size_t)tm * tn), b((size_t)tm * tn);
    EXPECT(mfl_tile_order(tm, tn, g, a.data(), b.data()) == 0);
  }
  std::vector<int32_t> perm(64);
  EXPECT(mfl_chain_k_perm(perm.data()) == 0);

  // argument checks (no launch)
  const uintptr_t P = 1 << 20;
  for (int it = 0; it < 20000; ++it) {
    gemm_dtypes_t dt{};
    dt.a = (int32_t)rnd(4);
    dt.b = (int32_t)rnd(4);
    dt.c = (int32_t)rnd(4);
    dt.d = (int32_t)rnd(4);
    dt.a_order = (int32_t)rnd(3);
    dt.algo = (int32_t)(rnd(12) | (rnd(3) == 0 ? 0x100 : 0));
    const int64_t M = dim(600), N = dim(600), K = dim(600);
    const void* C = dt.c == MFL_NONE && rnd(4) ? nullptr : (const void*)(P + 16 * rnd(3));
    int32_t al = 0, fa = 0, fb = 0;
    gemm_tn_validate(M, N, K, (const void*)(P + rnd(3)), rnd(4) ? dim(640) : M,
                     (const void*)(P * 2 + 2 * rnd(9)), rnd(4) ? dim(640) : K, C,
                     rnd(4) ? dim(610) : N, (void*)(P * 3), rnd(4) ? dim(610) : N, dt,
                     rnd(2) ? &al : nullptr);
    gemm_tn_plan(M, N, K, (const void*)P, K, (const void*)(2 * P), K, C, N, (void*)(3 * P), N,
                 dt, &al, &fa, &fb);
  }
  for (int it = 0; it < 5000; ++it) {
    const int64_t bt = rnd(8) ? rnd(5) - 1 : dim(5), M = dim(600), N1 = dim(600),
                  N2 = dim(300), K = rnd(8) ? 32 << rnd(5) : dim(600);
    int32_t stg = 0, tn = 0;
    gemm_tn_chain_validate(bt, M, N1, N2, K, (const void*)P, rnd(2) ? K : dim(700),
                           rnd(2) ? 0 : dim(1 << 20), (const void*)(2 * P), rnd(2) ? K : dim(700),
                           rnd(2) ? 0 : dim(1 << 20), (const void*)(3 * P),
                           rnd(2) ? N1 : dim(700), rnd(2) ? 0 : dim(1 << 20), (void*)(4 * P),
                           rnd(2) ? N2 : dim(400), rnd(2) ? 0 : dim(1 << 20), (int32_t)rnd(4));
    gemm_tn_chain_plan(bt, M, N1, N2, K, (const void*)P, K, 0, (const void*)(2 * P), K, 0,
                       (const void*)(3 * P), N1, 0, (void*)(4 * P), N2, 0, MFL_F16, &stg, &tn);
  }
  for (int code = -20; code < 5; ++code) EXPECT(gemm_strerror(code) != nullptr);
  printf("capi driver: %d failures\n", fails);
  return fails != 0;
}

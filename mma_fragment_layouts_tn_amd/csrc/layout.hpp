// Shape:stride layout algebra, usable on the host and inside kernels.
//
// A layout maps a coordinate to an integer offset: each top-level mode holds
// one or more leaves (shape, stride); an integer index is split over all
// leaves with the first leaf varying fastest, and the offset is the sum of
// leaf-coordinate times leaf-stride.  This is the reading of the TiledMMA
// page ("读懂 CuTe 的 make_tiled_mma：一条 MMA 怎样铺成一块矩阵", sections
// "先固定矩阵和方向" and "从 C 的四个值开始读") and of "CuTe Layout 到 Tensor
// Core" (§1 shape+stride, §3 size vs cosize).  Nesting is kept to two
// levels (top-level modes of flat leaves), which covers every layout the
// pages print; as functions of an integer, deeper nesting is equivalent.
//
// Operations:
//   eval / eval2        evaluate at an integer, or at one integer per mode
//   size / cosize       domain size; largest offset + 1 (strides >= 0)
//   coalesce            merge leaves that continue each other, drop size-1
//   compose(A, B)       (A o B)(c) = A(B(c)), B's integer decoded in A's
//                       shape, A's last leaf taken as unbounded (retile page
//                       "读懂 CuTe 的 retile_D", section "把编号接到原来的存储上")
//   right_inverse(L)    R with L(R(j)) = j on the longest prefix 0..n-1 the
//                       layout covers (retile page, section "先确定要从哪些
//                       fragment 位置取值")
//   complement(L, M)    the layout R, strides increasing, that fills the gaps
//                       between L's strides so (L, R) tiles [0, M)
//   logical_divide      A o (B, complement(B, |A|)): (tile, rest), whole
//                       layout or mode by mode (partition_C's first step,
//                       TiledMMA page "先按第三个参数划分 M、N")
//   zipped_divide       mode-by-mode divide with all tile parts gathered in
//                       mode 0 and all rest parts in mode 1 ("再切出单条指令
//                       的输出块")
//   logical_product     (A, complement(A, |A| cosize(B)) o B) (retile page,
//                       "建立 Copy 的分组编号")
//   upcast(L, N)        L viewed in units of N elements, leaf by leaf
//   with_shape(L, S)    L o make_layout(S): the same function on a domain
//                       reshaped to S
//   tiled_product       logical_product with B's modes kept apart
//   partition_c         a tiled MMA's C partition, from the element each
//                       (thread, value) holds, factored into layouts
// Results that would nest three levels deep keep their leaves flattened
// inside a top-level mode; as functions they are unchanged.
// All functions are constexpr so kernels can fold them at compile time.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define MFL_HD __host__ __device__
#else
#define MFL_HD
#endif

namespace mfl {

constexpr int kMaxLeaves = 16;
constexpr int kMaxModes = 8;

enum LayoutStatus : int {
  kLayoutOk = 0,
  kLayoutTooLarge = -10,     // more leaves or modes than supported
  kLayoutNotComposable = -11,  // divisibility condition of composition fails
  kLayoutBadText = -12,
  kLayoutBadIndex = -13,
  kLayoutNegativeStride = -14,
};

struct Layout {
  int nmodes = 0;
  int nleaves = 0;
  int status = kLayoutOk;
  int mode_end[kMaxModes] = {};   // one past the last leaf of each mode
  int64_t shape[kMaxLeaves] = {};
  int64_t stride[kMaxLeaves] = {};

  MFL_HD constexpr int mode_begin(int m) const { return m == 0 ? 0 : mode_end[m - 1]; }

  // append a leaf to the last mode (opening a first mode if needed)
  MFL_HD constexpr void push_leaf(int64_t s, int64_t d) {
    if (nmodes == 0) open_mode();
    if (nleaves >= kMaxLeaves) {
      status = kLayoutTooLarge;
      return;
    }
    shape[nleaves] = s;
    stride[nleaves] = d;
    ++nleaves;
    mode_end[nmodes - 1] = nleaves;
  }
  MFL_HD constexpr void open_mode() {
    if (nmodes >= kMaxModes) {
      status = kLayoutTooLarge;
      return;
    }
    mode_end[nmodes] = nleaves;
    ++nmodes;
  }
};

// ------------------------------------------------------ checked arithmetic
// Text input can describe layouts whose sizes or offsets leave int64.  The
// algebra's products and sums below go through these: an overflow (or the
// value INT64_MIN, which has no negation) sets `st` to kLayoutTooLarge and
// yields INT64_MAX, never 0, so later divisions stay defined.  The per-lane
// evaluation that kernels run (eval, eval2) stays plain; it only ever sees
// the small layouts of the instructions and tiles.
constexpr int64_t kInt64Max = int64_t(~uint64_t(0) >> 1);

MFL_HD constexpr int64_t ck_mul(int64_t a, int64_t b, int& st) {
  int64_t r = 0;
  if (__builtin_mul_overflow(a, b, &r) || r == -kInt64Max - 1) {
    st = kLayoutTooLarge;
    return kInt64Max;
  }
  return r;
}

MFL_HD constexpr int64_t ck_add(int64_t a, int64_t b, int& st) {
  int64_t r = 0;
  if (__builtin_add_overflow(a, b, &r) || r == -kInt64Max - 1) {
    st = kLayoutTooLarge;
    return kInt64Max;
  }
  return r;
}

// ---------------------------------------------------------------- builders
MFL_HD constexpr Layout make_flat(int n, const int64_t* s, const int64_t* d) {
  Layout L;
  L.open_mode();
  for (int i = 0; i < n; ++i) L.push_leaf(s[i], d[i]);
  return L;
}

// one top-level mode per leaf: (s0,s1,...):(d0,d1,...)
MFL_HD constexpr Layout make_modes(int n, const int64_t* s, const int64_t* d) {
  Layout L;
  for (int i = 0; i < n; ++i) {
    L.open_mode();
    L.push_leaf(s[i], d[i]);
  }
  return L;
}

// ------------------------------------------------------------- evaluation
// size and cosize saturate at INT64_MAX and report that in *st, if given
MFL_HD constexpr int64_t size(const Layout& L, int* st = nullptr) {
  int s = kLayoutOk;
  int64_t n = 1;
  for (int i = 0; i < L.nleaves; ++i) n = ck_mul(n, L.shape[i], s);
  if (st && s != kLayoutOk) *st = s;
  return n;
}

MFL_HD constexpr int64_t size_mode(const Layout& L, int m, int* st = nullptr) {
  int s = kLayoutOk;
  int64_t n = 1;
  for (int i = L.mode_begin(m); i < L.mode_end[m]; ++i) n = ck_mul(n, L.shape[i], s);
  if (st && s != kLayoutOk) *st = s;
  return n;
}

// evaluate leaves [b, e) at integer idx (first leaf fastest)
MFL_HD constexpr int64_t eval_leaves(const Layout& L, int b, int e, int64_t idx) {
  int64_t off = 0;
  for (int i = b; i < e; ++i) {
    const int64_t s = L.shape[i];
    off += (idx % s) * L.stride[i];
    idx /= s;
  }
  return off;
}

MFL_HD constexpr int64_t eval(const Layout& L, int64_t idx) {
  return eval_leaves(L, 0, L.nleaves, idx);
}

// eval with checked arithmetic, for layouts built from arbitrary input
MFL_HD constexpr int64_t eval_ck(const Layout& L, int64_t idx, int& st) {
  int64_t off = 0;
  for (int i = 0; i < L.nleaves; ++i) {
    off = ck_add(off, ck_mul(idx % L.shape[i], L.stride[i], st), st);
    idx /= L.shape[i];
  }
  return off;
}

// as eval_ck, but the last leaf takes whatever index remains (indices past
// size(L) continue along the last leaf), the reading composition uses
MFL_HD constexpr int64_t eval_unbounded(const Layout& L, int64_t idx, int& st) {
  int64_t off = 0;
  for (int i = 0; i < L.nleaves; ++i) {
    if (i == L.nleaves - 1) return ck_add(off, ck_mul(idx, L.stride[i], st), st);
    off = ck_add(off, ck_mul(idx % L.shape[i], L.stride[i], st), st);
    idx /= L.shape[i];
  }
  return off;
}

MFL_HD constexpr int64_t eval_mode(const Layout& L, int m, int64_t idx) {
  return eval_leaves(L, L.mode_begin(m), L.mode_end[m], idx);
}

// coordinates given per top-level mode
MFL_HD constexpr int64_t eval2(const Layout& L, int64_t c0, int64_t c1) {
  return eval_mode(L, 0, c0) + eval_mode(L, 1, c1);
}

MFL_HD constexpr int64_t cosize(const Layout& L, int* st = nullptr) {
  int s = kLayoutOk;
  int64_t hi = 0;
  for (int i = 0; i < L.nleaves; ++i) hi = ck_add(hi, ck_mul(L.shape[i] - 1, L.stride[i], s), s);
  hi = ck_add(hi, 1, s);
  if (st && s != kLayoutOk) *st = s;
  return hi;
}

// ------------------------------------------------------------- coalesce
// One flat mode with equal function: drops size-1 leaves and merges a leaf
// into its predecessor when stride_next == shape_prev * stride_prev.
MFL_HD constexpr Layout coalesce(const Layout& L) {
  Layout out;
  out.open_mode();
  int ovf = kLayoutOk;
  for (int i = 0; i < L.nleaves; ++i) {
    const int64_t s = L.shape[i], d = L.stride[i];
    if (s == 1) continue;
    const int n = out.nleaves;
    int st = kLayoutOk;
    if (n > 0 && ck_mul(out.stride[n - 1], out.shape[n - 1], st) == d && st == kLayoutOk) {
      out.shape[n - 1] = ck_mul(out.shape[n - 1], s, ovf);
      continue;
    }
    out.push_leaf(s, d);
  }
  if (out.nleaves == 0) out.push_leaf(1, 0);
  out.status = L.status != kLayoutOk ? L.status : ovf != kLayoutOk ? ovf : out.status;
  return out;
}

// ---------------------------------------------------------- composition
// Compose a coalesced flat layout A with one leaf s:d; appends the resulting
// leaves to `out` (in its current last mode).  A's last leaf is unbounded.
MFL_HD constexpr void compose_leaf(const Layout& A, int64_t s, int64_t d, Layout& out) {
  if (s == 1) {
    out.push_leaf(1, 0);
    return;
  }
  if (d == 0) {
    out.push_leaf(s, 0);
    return;
  }
  if (d < 0) {   // the division of A by d below is defined for d > 0 only
    out.status = kLayoutNegativeStride;
    return;
  }
  const int n = A.nleaves;
  int i = 0;
  int64_t rest = d;
  // divide A by d: skip whole leaves, then start inside leaf i
  while (i < n - 1 && rest > 1) {
    if (rest % A.shape[i] == 0) {
      rest /= A.shape[i];
      ++i;
    } else if (A.shape[i] % rest == 0) {
      break;
    } else {
      out.status = kLayoutNotComposable;
      return;
    }
  }
  bool last = (i == n - 1);
  int64_t cur_shape = last ? 0 : A.shape[i] / rest;
  int64_t cur_stride = ck_mul(A.stride[i], rest, out.status);
  int64_t need = s;
  while (need > 1) {
    if (last) {
      out.push_leaf(need, cur_stride);
      return;
    }
    if (cur_shape >= need) {
      if (cur_shape % need != 0) {
        out.status = kLayoutNotComposable;
        return;
      }
      out.push_leaf(need, cur_stride);
      return;
    }
    if (need % cur_shape != 0) {
      out.status = kLayoutNotComposable;
      return;
    }
    if (cur_shape > 1) out.push_leaf(cur_shape, cur_stride);
    need /= cur_shape;
    ++i;
    last = (i == n - 1);
    cur_shape = last ? 0 : A.shape[i];
    cur_stride = A.stride[i];
  }
}

// (A o B): one result mode per top-level mode of B.  The leaf-by-leaf
// construction equals A(B(c)) when B's leaves address separate digit ranges
// of A's shape (no carries between them); callers that accept arbitrary
// input check the result with compose_is_exact.
MFL_HD constexpr Layout compose(const Layout& A, const Layout& B) {
  const Layout a = coalesce(A);
  Layout out;
  for (int m = 0; m < B.nmodes; ++m) {
    out.open_mode();
    const int before = out.nleaves;
    for (int i = B.mode_begin(m); i < B.mode_end[m]; ++i)
      compose_leaf(a, B.shape[i], B.stride[i], out);
    if (out.nleaves == before) out.push_leaf(1, 0);
  }
  if (a.status != kLayoutOk) out.status = a.status;
  if (B.status != kLayoutOk) out.status = B.status;
  return out;
}

// true when compose(A, B) equals A(B(c)) at every c (brute force; for
// checks of arbitrary inputs)
MFL_HD constexpr bool compose_is_exact(const Layout& A, const Layout& B, const Layout& AB) {
  int st = kLayoutOk;
  const int64_t n = size(B, &st);
  if (size(AB, &st) != n || st != kLayoutOk) return false;
  for (int64_t i = 0; i < n; ++i)
    if (eval_ck(AB, i, st) != eval_unbounded(A, eval_ck(B, i, st), st) || st != kLayoutOk)
      return false;
  return true;
}

// largest domain compose_v checks point by point
constexpr int64_t kVerifyMax = int64_t(1) << 22;

// compose; with `verify`, a result that differs from A(B(c)) anywhere is
// marked not composable (and a domain too large to check, too large).  The
// operations below take the same flag: callers with arbitrary input set it,
// kernels folding known-good layouts at compile time leave it off.
MFL_HD constexpr Layout compose_v(const Layout& A, const Layout& B, bool verify) {
  Layout AB = compose(A, B);
  if (!verify || AB.status != kLayoutOk) return AB;
  if (size(B) > kVerifyMax)
    AB.status = kLayoutTooLarge;
  else if (!compose_is_exact(A, B, AB))
    AB.status = kLayoutNotComposable;
  return AB;
}

// -------------------------------------------------------- right inverse
MFL_HD constexpr Layout right_inverse(const Layout& L) {
  const Layout c = coalesce(L);
  int64_t dom[kMaxLeaves] = {};  // domain stride of each leaf
  int64_t p = 1;
  int ovf = kLayoutOk;
  for (int i = 0; i < c.nleaves; ++i) {
    dom[i] = p;
    p = ck_mul(p, c.shape[i], ovf);
    if (c.stride[i] < 0) {
      Layout bad;
      bad.status = kLayoutNegativeStride;
      return bad;
    }
  }
  bool used[kMaxLeaves] = {};
  Layout out;
  out.open_mode();
  int64_t cur = 1;
  for (;;) {
    int pick = -1;
    for (int i = 0; i < c.nleaves; ++i)
      if (!used[i] && c.shape[i] > 1 && c.stride[i] == cur) {
        pick = i;
        break;
      }
    if (pick < 0) break;
    used[pick] = true;
    out.push_leaf(c.shape[pick], dom[pick]);
    cur = ck_mul(cur, c.shape[pick], ovf);
  }
  if (out.nleaves == 0) out.push_leaf(1, 0);
  out.status = c.status != kLayoutOk ? c.status : ovf != kLayoutOk ? ovf : out.status;
  return out;
}

// ------------------------------------------------------------ complement
MFL_HD constexpr Layout complement(const Layout& L, int64_t cotarget) {
  // leaves that move (shape > 1, stride != 0), sorted by stride
  int64_t sh[kMaxLeaves] = {}, st[kMaxLeaves] = {};
  int n = 0;
  Layout out;
  out.open_mode();
  for (int i = 0; i < L.nleaves; ++i) {
    if (L.shape[i] == 1 || L.stride[i] == 0) continue;
    if (L.stride[i] < 0) {
      out.status = kLayoutNegativeStride;
      return out;
    }
    int j = n++;
    while (j > 0 && st[j - 1] > L.stride[i]) {
      sh[j] = sh[j - 1];
      st[j] = st[j - 1];
      --j;
    }
    sh[j] = L.shape[i];
    st[j] = L.stride[i];
  }
  int64_t cur = 1;   // extent covered so far
  for (int i = 0; i < n; ++i) {
    if (st[i] < cur || st[i] % cur != 0) {   // overlapping or non-divisible leaves
      out.status = kLayoutNotComposable;
      return out;
    }
    if (st[i] / cur > 1) out.push_leaf(st[i] / cur, cur);
    cur = ck_mul(sh[i], st[i], out.status);
  }
  const int64_t rest = cotarget / cur + (cotarget % cur > 0 ? 1 : 0);   // ceil, no overflow
  if (rest > 1) out.push_leaf(rest, cur);
  Layout c = coalesce(out);
  if (L.status != kLayoutOk) c.status = L.status;
  return c;
}

// one top-level mode of L as a layout of its own
MFL_HD constexpr Layout mode_of(const Layout& L, int m) {
  Layout out;
  out.open_mode();
  for (int i = L.mode_begin(m); i < L.mode_end[m]; ++i) out.push_leaf(L.shape[i], L.stride[i]);
  out.status = L.status;
  return out;
}

// append all leaves of `src` to the last mode of `dst`
MFL_HD constexpr void append_leaves(Layout& dst, const Layout& src) {
  for (int i = 0; i < src.nleaves; ++i) dst.push_leaf(src.shape[i], src.stride[i]);
  if (src.status != kLayoutOk) dst.status = src.status;
}

// -------------------------------------------------------------- divides
// A divided by the single layout B over A's whole domain: mode 0 the tile
// (B's leaves composed into A), mode 1 the rest (B's complement)
MFL_HD constexpr Layout logical_divide(const Layout& A, const Layout& B, bool verify = false) {
  int ovf = kLayoutOk;
  Layout R = complement(B, size(A, &ovf));
  if (ovf != kLayoutOk) R.status = ovf;
  Layout BR;
  BR.open_mode();
  append_leaves(BR, B);
  BR.open_mode();
  append_leaves(BR, R);
  const Layout q = compose_v(A, BR, verify);
  Layout out;
  for (int m = 0; m < q.nmodes; ++m) {
    out.open_mode();
    append_leaves(out, mode_of(q, m));
  }
  if (q.status != kLayoutOk) out.status = q.status;
  return out;
}

// Mode-by-mode tilers: tilers[m] divides mode m of A (has_tiler[m] false or
// m >= ntilers: the mode is kept whole as the tile, rest 1).  `tile[m]` and
// `rest[m]` receive the parts.
MFL_HD constexpr void divide_modes(const Layout& A, const Layout* tilers, const bool* has_tiler,
                                   int ntilers, Layout* tile, Layout* rest, bool verify = false) {
  for (int m = 0; m < A.nmodes; ++m) {
    const Layout am = mode_of(A, m);
    if (m < ntilers && has_tiler[m]) {
      const Layout q = logical_divide(am, tilers[m], verify);
      tile[m] = mode_of(q, 0);
      rest[m] = mode_of(q, 1);
      if (q.status != kLayoutOk) tile[m].status = q.status;
    } else {
      tile[m] = am;
      Layout one;
      one.open_mode();
      one.push_leaf(1, 0);
      rest[m] = one;
    }
  }
}

// mode m of the result is (tile_m, rest_m), flattened into one mode; modes
// without a tiler are returned unchanged
MFL_HD constexpr Layout logical_divide_modes(const Layout& A, const Layout* tilers,
                                             const bool* has_tiler, int ntilers,
                                             bool verify = false) {
  Layout tile[kMaxModes], rest[kMaxModes];
  divide_modes(A, tilers, has_tiler, ntilers, tile, rest, verify);
  Layout out;
  for (int m = 0; m < A.nmodes; ++m) {
    out.open_mode();
    append_leaves(out, tile[m]);
    if (m < ntilers && has_tiler[m]) append_leaves(out, rest[m]);
  }
  if (A.status != kLayoutOk) out.status = A.status;
  return out;
}

// ((tile_0, tile_1, ...), (rest_0, rest_1, ...)), each part flattened
MFL_HD constexpr Layout zipped_divide(const Layout& A, const Layout* tilers, const bool* has_tiler,
                                      int ntilers, bool verify = false) {
  Layout tile[kMaxModes], rest[kMaxModes];
  divide_modes(A, tilers, has_tiler, ntilers, tile, rest, verify);
  Layout out;
  out.open_mode();
  for (int m = 0; m < A.nmodes; ++m) append_leaves(out, tile[m]);
  out.open_mode();
  for (int m = 0; m < A.nmodes; ++m) append_leaves(out, rest[m]);
  if (A.status != kLayoutOk) out.status = A.status;
  return out;
}

// ------------------------------------------------------------- product
MFL_HD constexpr Layout logical_product(const Layout& A, const Layout& B, bool verify = false) {
  int ovf = kLayoutOk;
  const Layout C = complement(A, ck_mul(size(A, &ovf), cosize(B, &ovf), ovf));
  const Layout CB = compose_v(C, B, verify);
  Layout out;
  out.open_mode();
  append_leaves(out, A);
  out.open_mode();
  append_leaves(out, CB);
  if (A.status != kLayoutOk) out.status = A.status;
  if (ovf != kLayoutOk) out.status = ovf;
  return out;
}

// logical_product with B's top-level modes kept apart: (A, (C o B)_0,
// (C o B)_1, ...).  With A the atom's thread ids and B the arrangement of
// atoms over M, N, K this is the tiled MMA's thread layout (TiledMMA page,
// "第二个参数怎样把一个 warp 扩展成四个")
MFL_HD constexpr Layout tiled_product(const Layout& A, const Layout& B, bool verify = false) {
  int ovf = kLayoutOk;
  const Layout C = complement(A, ck_mul(size(A, &ovf), cosize(B, &ovf), ovf));
  const Layout CB = compose_v(C, B, verify);
  Layout out;
  out.open_mode();
  append_leaves(out, A);
  for (int m = 0; m < CB.nmodes; ++m) {
    out.open_mode();
    append_leaves(out, mode_of(CB, m));
  }
  if (A.status != kLayoutOk) out.status = A.status;
  if (C.status != kLayoutOk) out.status = C.status;
  if (CB.status != kLayoutOk) out.status = CB.status;
  if (ovf != kLayoutOk) out.status = ovf;
  return out;
}

// ------------------------------------------------------------- upcast
// a / b when b divides a, 1 when a divides b, else not representable
MFL_HD constexpr int64_t shape_div(int64_t a, int64_t b, int& status) {
  if (b != 0 && a % b == 0) return a / b;
  if (a != 0 && b % a == 0) return 1;
  status = kLayoutNotComposable;
  return 1;
}

// leaf (s, d) -> (s / (N / d), d / N), 1 where the unit exceeds the extent;
// stride-0 leaves unchanged
MFL_HD constexpr Layout upcast(const Layout& L, int64_t n) {
  Layout out;
  for (int m = 0; m < L.nmodes; ++m) {
    out.open_mode();
    for (int i = L.mode_begin(m); i < L.mode_end[m]; ++i) {
      const int64_t s = L.shape[i], d = L.stride[i];
      if (d == 0) {
        out.push_leaf(s, 0);
        continue;
      }
      int st = kLayoutOk;
      const int64_t ad = d < 0 ? -d : d;
      const int64_t ns = shape_div(s, shape_div(n, ad, st), st);
      const int64_t nd = shape_div(ad, n, st) * (d < 0 ? -1 : 1);
      out.push_leaf(ns, nd);
      if (st != kLayoutOk) out.status = st;
    }
  }
  if (L.status != kLayoutOk) out.status = L.status;
  return out;
}

// --------------------------------------------------------- with_shape
// make_layout(shape) for a shape given as modes of leaves: column-major
MFL_HD constexpr Layout compact(const Layout& shape_only) {
  Layout out;
  int64_t d = 1;
  int ovf = kLayoutOk;
  for (int m = 0; m < shape_only.nmodes; ++m) {
    out.open_mode();
    for (int i = shape_only.mode_begin(m); i < shape_only.mode_end[m]; ++i) {
      out.push_leaf(shape_only.shape[i], d);
      d = ck_mul(d, shape_only.shape[i], ovf);
    }
  }
  out.status = shape_only.status != kLayoutOk ? shape_only.status
               : ovf != kLayoutOk             ? ovf
                                              : out.status;
  return out;
}

MFL_HD constexpr Layout with_shape(const Layout& L, const Layout& shape_only, bool verify = false) {
  return compose_v(L, compact(shape_only), verify);
}

MFL_HD constexpr Layout unit_leaf(int64_t n) {
  Layout out;
  out.open_mode();
  out.push_leaf(n, n == 1 ? 0 : 1);
  return out;
}

// all leaves of the listed layouts, in order, as one top-level mode
MFL_HD constexpr Layout flat_join(const Layout* parts, int n) {
  Layout out;
  out.open_mode();
  for (int i = 0; i < n; ++i) append_leaves(out, parts[i]);
  return out;
}

// ------------------------------------------------------------- factoring
// One mode of a layout for a function f on [0, n) with f(0) = 0: the index
// is split into prime digits, smallest prime first, and each digit becomes a
// leaf whose stride is f at that digit's unit; a digit that continues the
// previous leaf's progression (stride = that leaf's shape x stride) widens
// it instead.  The mode equals f exactly when f is linear over these digits,
// which holds for every layout whose leaves have power-of-two shapes; other
// inputs are checked by the caller against the whole table.
template <class F>
MFL_HD constexpr void append_factored(Layout& out, int64_t n, const F& f) {
  out.open_mode();
  const int first = out.nleaves;
  int64_t rest = n, unit = 1;
  while (rest > 1) {
    int64_t p = 2;
    while (rest % p != 0) ++p;
    const int64_t d = f(unit);
    const int k = out.nleaves;
    int st = kLayoutOk;
    if (k > first && ck_mul(out.shape[k - 1], out.stride[k - 1], st) == d && st == kLayoutOk)
      out.shape[k - 1] = ck_mul(out.shape[k - 1], p, out.status);
    else
      out.push_leaf(p, d);
    unit = ck_mul(unit, p, out.status);
    rest /= p;
  }
  if (out.nleaves == first) out.push_leaf(1, 0);
}

// ------------------------------------------------------------ partition_C
// The C partition of a tiled MMA (TiledMMA page, "partition_C 怎样把分工应
// 用到一个 Tensor"), computed from the element each (thread, value, repeat)
// holds and then written as layouts.
//
// The tiled MMA repeats an atom_m x atom_n atom over warps_m x warps_n warps
// (warp w = wm + warps_m wn; thread t = lane + nlanes w).  C (mode 0 = M,
// mode 1 = N, its storage layout) is cut into tiles of tile_m x tile_n
// (the sizes of the tile entries, or atom x warps); inside a tile, logical
// row i sits at physical row tile_m(i) (the entry permutes the tile's rows,
// section "用 Layout 改变 M 方向的坐标顺序"; compact when absent).  Along M
// the atom-row blocks are numbered down each tile and then across tiles
// (block b: tile b / (tile_m/atom_m), logical rows atom_m (b % (tile_m/
// atom_m)) + 0 .. atom_m-1), and warp row wm takes blocks wm, wm + warps_m,
// wm + 2 warps_m, ...: its rm-th repeat is block wm + warps_m rm.  Likewise
// along N.  Value v of lane l is the atom element q = atom_tv(l + nlanes v),
// at (q % atom_m, q / atom_m) inside its block.  So thread t's value v of
// repeat (rm, rn) is C at
//   m = tile_m(q % atom_m + atom_m (bm % (tile_m/atom_m))) + tile_m_size (bm / (tile_m/atom_m)),
//   bm = wm + warps_m rm, and n the same way.
// The results: `thr`, one mode, thread -> offset of its first value (value
// 0 of repeat (0, 0)); `val`, (value, rest M, rest N) -> offset from it.
// Each mode is factored from that function (append_factored); with `verify`
// every (thread, value) is compared, and the tile entries must permute
// their tiles' rows.
struct CPartition {
  Layout thr;
  Layout val;
};

MFL_HD constexpr CPartition partition_c(const Layout& C, const Layout* tile, const Layout& atom_tv,
                                        int64_t atom_m, int64_t atom_n, int64_t warps_m,
                                        int64_t warps_n, bool verify = false) {
  CPartition r;
  auto fail = [&](int st) {
    r.thr = Layout{};
    r.val = Layout{};
    r.thr.status = r.val.status = st;
    return r;
  };
  if (C.status != kLayoutOk) return fail(C.status);
  if (atom_tv.status != kLayoutOk) return fail(atom_tv.status);
  if (tile && (tile[0].status != kLayoutOk || tile[1].status != kLayoutOk))
    return fail(tile[0].status != kLayoutOk ? tile[0].status : tile[1].status);
  if (C.nmodes != 2 || atom_tv.nmodes != 2 || atom_m < 1 || atom_n < 1 || warps_m < 1 ||
      warps_n < 1)
    return fail(kLayoutBadIndex);
  int ovf = kLayoutOk;
  const int64_t ext[2] = {size_mode(C, 0, &ovf), size_mode(C, 1, &ovf)};
  const int64_t atom[2] = {atom_m, atom_n}, warps[2] = {warps_m, warps_n};
  const int64_t nlanes = size_mode(atom_tv, 0, &ovf), nvals = size_mode(atom_tv, 1, &ovf);
  int64_t tsz[2] = {0, 0}, per_tile[2] = {0, 0}, reps[2] = {0, 0};
  for (int d = 0; d < 2; ++d) {
    tsz[d] = tile ? size(tile[d], &ovf) : ck_mul(atom[d], warps[d], ovf);
    // the tile must divide C, the atom the tile and the warps the atom blocks
    if (ovf != kLayoutOk) return fail(ovf);
    if (tsz[d] < 1 || ext[d] % tsz[d] != 0 || tsz[d] % atom[d] != 0) return fail(kLayoutBadIndex);
    per_tile[d] = tsz[d] / atom[d];
    const int64_t blocks = ck_mul(per_tile[d], ext[d] / tsz[d], ovf);
    if (blocks % warps[d] != 0) return fail(kLayoutBadIndex);
    reps[d] = blocks / warps[d];
  }
  if (ck_mul(atom_m, atom_n, ovf) != size(atom_tv, &ovf)) return fail(kLayoutBadIndex);
  const int64_t nthr = ck_mul(nlanes, ck_mul(warps_m, warps_n, ovf), ovf);
  const int64_t nval = ck_mul(nvals, ck_mul(reps[0], reps[1], ovf), ovf);
  if (ovf != kLayoutOk) return fail(ovf);

  // the C offset of thread t's value u = v + nvals (rm + reps_m rn)
  auto coord = [&](int d, int64_t a, int64_t w, int64_t rep) {   // a: atom coordinate
    const int64_t b = w + warps[d] * rep;
    const int64_t i = a + atom[d] * (b % per_tile[d]);
    return (tile ? eval(tile[d], i) : i) + tsz[d] * (b / per_tile[d]);
  };
  auto offset = [&](int64_t t, int64_t u) {
    const int64_t lane = t % nlanes, w = t / nlanes;
    const int64_t v = u % nvals, ru = u / nvals;
    const int64_t q = eval(atom_tv, lane + nlanes * v);
    const int64_t m = coord(0, q % atom_m, w % warps_m, ru % reps[0]);
    const int64_t n = coord(1, q / atom_m, w / warps_m, ru / reps[0]);
    return eval_mode(C, 0, m) + eval_mode(C, 1, n);
  };
  if (offset(0, 0) != 0) return fail(kLayoutNotComposable);   // not a layout
  append_factored(r.thr, nthr, [&](int64_t t) { return offset(t, 0); });
  append_factored(r.val, nvals, [&](int64_t v) { return offset(0, v); });
  append_factored(r.val, reps[0], [&](int64_t rm) { return offset(0, nvals * rm); });
  append_factored(r.val, reps[1], [&](int64_t rn) { return offset(0, nvals * reps[0] * rn); });
  if (r.thr.status != kLayoutOk || r.val.status != kLayoutOk)
    return fail(r.thr.status != kLayoutOk ? r.thr.status : r.val.status);
  if (verify) {
    if (ck_mul(nthr, nval, ovf) > kVerifyMax || ovf != kLayoutOk) return fail(kLayoutTooLarge);
    if (tile) {   // each entry permutes its tile's rows
      for (int d = 0; d < 2; ++d) {
        if (tsz[d] > 4096) return fail(kLayoutTooLarge);
        bool seen[4096] = {};
        for (int64_t i = 0; i < tsz[d]; ++i) {
          const int64_t x = eval(tile[d], i);
          if (x < 0 || x >= tsz[d] || seen[x]) return fail(kLayoutNotComposable);
          seen[x] = true;
        }
      }
    }
    // the C coordinates stay inside C, and the layouts equal the rule
    for (int64_t t = 0; t < nthr; ++t)
      for (int64_t u = 0; u < nval; ++u)
        if (eval(r.thr, t) + eval(r.val, u) != offset(t, u)) return fail(kLayoutNotComposable);
  }
  return r;
}

}  // namespace mfl

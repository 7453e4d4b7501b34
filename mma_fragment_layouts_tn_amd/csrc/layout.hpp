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
MFL_HD constexpr int64_t size(const Layout& L) {
  int64_t n = 1;
  for (int i = 0; i < L.nleaves; ++i) n *= L.shape[i];
  return n;
}

MFL_HD constexpr int64_t size_mode(const Layout& L, int m) {
  int64_t n = 1;
  for (int i = L.mode_begin(m); i < L.mode_end[m]; ++i) n *= L.shape[i];
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

// as eval, but the last leaf takes whatever index remains (indices past
// size(L) continue along the last leaf), the reading composition uses
MFL_HD constexpr int64_t eval_unbounded(const Layout& L, int64_t idx) {
  int64_t off = 0;
  for (int i = 0; i < L.nleaves; ++i) {
    if (i == L.nleaves - 1) return off + idx * L.stride[i];
    off += (idx % L.shape[i]) * L.stride[i];
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

MFL_HD constexpr int64_t cosize(const Layout& L) {
  int64_t hi = 0;
  for (int i = 0; i < L.nleaves; ++i) hi += (L.shape[i] - 1) * L.stride[i];
  return hi + 1;
}

// ------------------------------------------------------------- coalesce
// One flat mode with equal function: drops size-1 leaves and merges a leaf
// into its predecessor when stride_next == shape_prev * stride_prev.
MFL_HD constexpr Layout coalesce(const Layout& L) {
  Layout out;
  out.open_mode();
  for (int i = 0; i < L.nleaves; ++i) {
    const int64_t s = L.shape[i], d = L.stride[i];
    if (s == 1) continue;
    const int n = out.nleaves;
    if (n > 0 && out.stride[n - 1] * out.shape[n - 1] == d) {
      out.shape[n - 1] *= s;
      continue;
    }
    out.push_leaf(s, d);
  }
  if (out.nleaves == 0) out.push_leaf(1, 0);
  out.status = L.status;
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
  int64_t cur_stride = A.stride[i] * rest;
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
// host-side checks of arbitrary inputs)
inline bool compose_is_exact(const Layout& A, const Layout& B, const Layout& AB) {
  const int64_t n = size(B);
  if (size(AB) != n) return false;
  for (int64_t i = 0; i < n; ++i)
    if (eval(AB, i) != eval_unbounded(A, eval(B, i))) return false;
  return true;
}

// -------------------------------------------------------- right inverse
MFL_HD constexpr Layout right_inverse(const Layout& L) {
  const Layout c = coalesce(L);
  int64_t dom[kMaxLeaves] = {};  // domain stride of each leaf
  int64_t p = 1;
  for (int i = 0; i < c.nleaves; ++i) {
    dom[i] = p;
    p *= c.shape[i];
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
    cur *= c.shape[pick];
  }
  if (out.nleaves == 0) out.push_leaf(1, 0);
  out.status = c.status;
  return out;
}

}  // namespace mfl

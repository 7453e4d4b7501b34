// gfx950 (CDNA4) f16 matrix-instruction atoms as thread/value layouts.
//
// The pages build every fragment map from an atom's (thread, value) ->
// matrix-coordinate layout (TiledMMA page "读懂 CuTe 的 make_tiled_mma",
// sections "从 C 的四个值开始读" and "A 的八个值和 B 的四个值").  This file
// states the same kind of layout for the wave64 MFMA instructions the kernels
// issue.  Operand layouts map (lane, value) to q = row + ROWS*k (row is m for
// A, n for B); accumulator layouts map (lane, value) to q = m + M*n.  Thread
// index = lane in 0..63; flattened TV index = lane + 64*value.
//
//   v_mfma_f32_32x32x16_f16:  A/B ((32,2),8):((1,256),32)
//                             C   ((32,2),(4,4)):((32,4),(1,8))
//   v_mfma_f32_16x16x32_f16:  A/B ((16,4),8):((1,128),16)
//                             C   ((16,4),4):((16,4),1)
//
// Value v of an operand sits in half v%2 (low half first) of VGPR v/2 of the
// operand register tuple, as the pages' 32-bit packing does (retile page
// "读懂 CuTe 的 retile_D", section "Copy 与 MMA 怎样使用同一份寄存器").  The
// K order inside a lane is only observable up to a permutation shared by A
// and B; the layouts pick 8 contiguous k per lane so one 16-byte read fills
// one operand.  The hardware mapping is checked by the GPU probe test.
#pragma once

#include "layout.hpp"

namespace mfl {

struct AtomShape {
  int m, n, k, vals_ab, vals_c;
};

// TV layout of the A/B operand: lane = (row-in-atom, k-group), value = k
MFL_HD constexpr Layout mfma_ab_tv(int rows, int kgroups, int vals) {
  Layout L;
  L.open_mode();
  L.push_leaf(rows, 1);
  L.push_leaf(kgroups, (int64_t)rows * vals);
  L.open_mode();
  L.push_leaf(vals, rows);
  return L;
}

// TV layout of the accumulator for the 32x32 family
MFL_HD constexpr Layout mfma32_c_tv() {
  Layout L;
  L.open_mode();
  L.push_leaf(32, 32);
  L.push_leaf(2, 4);
  L.open_mode();
  L.push_leaf(4, 1);
  L.push_leaf(4, 8);
  return L;
}

// TV layout of the accumulator for the 16x16 family
MFL_HD constexpr Layout mfma16_c_tv() {
  Layout L;
  L.open_mode();
  L.push_leaf(16, 16);
  L.push_leaf(4, 4);
  L.open_mode();
  L.push_leaf(4, 1);
  return L;
}

enum MfmaOp : int {
  kMfma32x32x16 = 0,   // v_mfma_f32_32x32x16_f16
  kMfma16x16x32 = 1,   // v_mfma_f32_16x16x32_f16
  kMfma32x32x8 = 2,    // v_mfma_f32_32x32x8_f16
  kMfma16x16x16 = 3,   // v_mfma_f32_16x16x16_f16
  kMfmaOpCount = 4,
};

MFL_HD constexpr AtomShape mfma_shape(int op) {
  return op == kMfma32x32x16   ? AtomShape{32, 32, 16, 8, 16}
         : op == kMfma16x16x32 ? AtomShape{16, 16, 32, 8, 4}
         : op == kMfma32x32x8  ? AtomShape{32, 32, 8, 4, 16}
                               : AtomShape{16, 16, 16, 4, 4};
}

MFL_HD constexpr Layout mfma_tv(int op, int operand /*0 A, 1 B, 2 C*/) {
  const AtomShape s = mfma_shape(op);
  if (operand == 2) return s.m == 32 ? mfma32_c_tv() : mfma16_c_tv();
  return mfma_ab_tv(s.m, 64 / s.m, s.vals_ab);
}

}  // namespace mfl

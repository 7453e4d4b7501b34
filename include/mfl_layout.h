/*
 * mfl_layout.h — C ABI of the host layout-algebra module.
 *
 * Layouts cross this boundary as text "shape:stride" with nested tuples, e.g.
 * "((4,8),(2,2)):((32,1),(16,8))" (CuTe's printed form; a leading '_' on an
 * integer is accepted).  Two nesting levels are supported: top-level modes,
 * each an integer or a tuple of integers.  Semantics:
 *   - an integer index is split over the leaves with the first leaf varying
 *     fastest; the offset is sum(leaf coordinate * leaf stride)
 *     (TiledMMA page "读懂 CuTe 的 make_tiled_mma：一条 MMA 怎样铺成一块矩阵",
 *     sections "先固定矩阵和方向", "从 C 的四个值开始读");
 *   - size = product of shapes; cosize = largest offset + 1 ("CuTe Layout 到
 *     Tensor Core" §3);
 *   - compose(A, B)(c) = A(B(c)), B's integer decoded in A's shape with A's
 *     last leaf unbounded (retile page "读懂 CuTe 的 retile_D", section
 *     "把编号接到原来的存储上"); the result has one mode per mode of B;
 *     inputs whose leaves of B would interact through carries in A's shape
 *     are rejected (-11): every returned layout equals A(B(c)) at every c,
 *     checked by brute force (size(B) <= 2^22);
 *   - right_inverse(L) = R with L(R(j)) = j for j < size(R), over the
 *     longest prefix 0..n-1 that L reaches (retile page, section
 *     "先确定要从哪些 fragment 位置取值"; route page "ldmatrix 怎样对上 MMA
 *     的寄存器", 第二步).
 * Output text is written into a caller buffer `out` of `cap` bytes (NUL
 * terminated).  Every function returns 0 or a negative code:
 *   -10 too many leaves/modes (16 leaves, 8 modes), -11 not composable
 *   (divisibility fails), -12 malformed text, -13 index out of range or
 *   buffer too small, -14 negative stride where not supported.
 * Pure host code: no GPU is touched.
 */
#ifndef MFL_LAYOUT_H
#define MFL_LAYOUT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int mfl_layout_size(const char* layout, int64_t* out);
int mfl_layout_cosize(const char* layout, int64_t* out);
/* L(idx) for 0 <= idx < size */
int mfl_layout_eval(const char* layout, int64_t idx, int64_t* out);
/* L(i) for all i < size into out[0..size); fails if size > cap */
int mfl_layout_table(const char* layout, int64_t* out, int64_t cap);
int mfl_layout_coalesce(const char* layout, char* out, int64_t cap);
int mfl_layout_compose(const char* a, const char* b, char* out, int64_t cap);
int mfl_layout_right_inverse(const char* layout, char* out, int64_t cap);

/* Thread/value layout of a gfx950 matrix instruction operand.
 * op: 0 v_mfma_f32_32x32x16_f16, 1 v_mfma_f32_16x16x32_f16,
 *     2 v_mfma_f32_32x32x8_f16,  3 v_mfma_f32_16x16x16_f16.
 * operand: 0 A (q = m + M*k), 1 B (q = n + N*k), 2 C/D (q = m + M*n).
 * Domain: (lane 0..63, value); flattened index lane + 64*value. */
int mfl_layout_mfma_tv(int32_t op, int32_t operand, char* out, int64_t cap);

/* Per-lane fragment addressing of a GEMM kernel, computed by the same code
 * the kernel runs: for every thread t of one workgroup and every fragment
 * slot s of one K-step, the (row, k) (operand 0 A, 1 B) or (m, n)
 * (operand 2, accumulators) within the workgroup tile, written as pairs into
 * out[2*(t*slots + s) + {0,1}].  Operand 3: for an M-contiguous A, the
 * (m, k) each lane addresses with the first of the two transposing LDS reads
 * (ds_read_b64_tr_b16; 4 consecutive m, the second read 4 k further) per K
 * sub-step and repeat, slot = kk*RM + i.  *threads and *slots receive the counts; the
 * call fails with -13 when 2*threads*slots > cap.  algo is an mfl_algo value
 * other than AUTO.  Pure host code. */
int mfl_fragment_coords(int32_t algo, int32_t operand, int32_t* out, int64_t cap,
                        int32_t* threads, int32_t* slots);

/* LDS operand-tile layout of a kernel: out[o*inner + i] = element offset
 * (halves) inside one operand stage.  Operand 0 (A) and 1 (B): (o, i) =
 * (row, k), row < BM or BN, k < BK, the XOR-swizzled K-contiguous tile.
 * Operand 2: (o, i) = (k, m) of the M-contiguous A tile, k < BK, m < BM.
 * *outer and *inner receive the tile shape; fails with -13 if
 * outer*inner > cap.  Pure host code. */
int mfl_lds_tile_offsets(int32_t algo, int32_t operand, int32_t* out, int64_t cap,
                         int32_t* outer, int32_t* inner);

/* Workgroup -> output tile order the kernels use for a grid of
 * tiles_m x tiles_n tiles (XCD-aware grouping, band height group_m):
 * tm[b], tn[b] for every workgroup id b < tiles_m*tiles_n.  Pure host code. */
int mfl_tile_order(int32_t tiles_m, int32_t tiles_n, int32_t group_m, int32_t* tm, int32_t* tn);

#ifdef __cplusplus
}
#endif
#endif /* MFL_LAYOUT_H */

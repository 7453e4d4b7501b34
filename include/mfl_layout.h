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
 *     checked by brute force (size(B) <= 2^22, else -10);
 *   - right_inverse(L) = R with L(R(j)) = j for j < size(R), over the
 *     longest prefix 0..n-1 that L reaches (retile page, section
 *     "先确定要从哪些 fragment 位置取值"; route page "ldmatrix 怎样对上 MMA
 *     的寄存器", 第二步).
 * Output text is written into a caller buffer `out` of `cap` bytes (NUL
 * terminated).  Every function returns 0 or a negative code:
 *   -10 too many leaves/modes (16 leaves, 8 modes), or a size, offset or
 *   intermediate value beyond int64 (inputs: integers up to 2^40 in
 *   magnitude, size and reach of every offset within int64), -11 not
 *   composable (divisibility fails), -12 malformed text, -13 index out of
 *   range or buffer too small, -14 negative stride where not supported.
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

/* Tiling algebra (the operations partition_C and retile are built from:
 * TiledMMA page "读懂 CuTe 的 make_tiled_mma", section "partition_C 怎样把分工
 * 应用到一个 Tensor"; retile page "读懂 CuTe 的 retile_D", sections "带着 8 和
 * 2，读一遍 retile 的源码" and "两个 K fragment 怎样连成一组").  Text in and out
 * as above; results nesting deeper than modes of leaves keep their leaves
 * flattened inside a top-level mode (the same function).
 *   complement(L, M): the layout R, strides increasing, filling the gaps
 *     between L's strides so that (L, R) tiles [0, M).  -11 when L's leaves
 *     overlap or do not divide each other.
 *   logical_divide(A, tiler): tiler is one layout B (A o (B, complement(B,
 *     |A|)), result (tile, rest)) or "T0;T1;..." dividing mode m by Tm ("_"
 *     keeps the mode; "T0;" for a single entry; result mode m = (tile_m,
 *     rest_m)).
 *   zipped_divide(A, tiler): as logical_divide, then all tile parts in mode
 *     0 and all rest parts in mode 1.
 *   logical_product(A, B): (A, complement(A, |A| cosize(B)) o B).
 *   upcast(L, n): each leaf (s, d) -> (s / (n / d), d / n), 1 where the unit
 *     exceeds the extent; -11 when the sizes do not divide.
 *   with_shape(L, shape): L o make_layout(shape); shape text like
 *     "(8,(2,4,2))" must have L's size.
 *   tiled_product(A, B): logical_product with B's top-level modes kept
 *     apart, (A, (C o B)_0, (C o B)_1, ...), C = complement(A, |A| cosize(B));
 *     with A the atom's thread ids and B the atoms' arrangement over M, N, K
 *     it is the tiled MMA's thread layout (TiledMMA page, section "第二个参数
 *     怎样把一个 warp 扩展成四个").
 * Compositions inside these are checked against A(B(c)) at every c; -11 when
 * the shape:stride form would not equal it. */
int mfl_layout_complement(const char* layout, int64_t cotarget, char* out, int64_t cap);
int mfl_layout_logical_divide(const char* a, const char* tiler, char* out, int64_t cap);
int mfl_layout_zipped_divide(const char* a, const char* tiler, char* out, int64_t cap);
int mfl_layout_logical_product(const char* a, const char* b, char* out, int64_t cap);
int mfl_layout_upcast(const char* layout, int64_t n, char* out, int64_t cap);
int mfl_layout_with_shape(const char* layout, const char* shape, char* out, int64_t cap);
int mfl_layout_tiled_product(const char* a, const char* b, char* out, int64_t cap);

/* partition_C of a tiled MMA (TiledMMA page, section "partition_C 怎样把分工
 * 应用到一个 Tensor"), from the element each thread holds.  The atom
 * (atom_m x atom_n, C TV layout `atom_tv`: lane + nlanes*value -> m +
 * atom_m*n) is repeated over warps_m x warps_n warps; the output tensor `c`
 * (two modes, M then N: its storage layout) is covered by tiles whose rows
 * (columns) are permuted by the tile entries; `tile` is "" (compact
 * atom*warps per direction) or "Lm;Ln" (section "用 Layout 改变 M 方向的坐标
 * 顺序"; "_" for an unpermuted direction; each entry must permute its tile).
 * Along M the atom-row blocks are numbered down a tile, then across tiles,
 * and warp row wm holds blocks wm, wm + warps_m, ...; likewise along N.
 * Outputs, each `cap` bytes: thr_out, one mode, thread lane + nlanes*(wm +
 * warps_m*wn) -> storage offset of that thread's first value; val_out,
 * (value, rest M, rest N) -> offset relative to it.  Each mode is factored
 * from that element map and the whole map is checked.  -13 when c is not
 * rank 2, the tile does not divide c, the atom the tile, or the warp counts
 * the atom blocks; -11 when a tile entry is not a permutation or the map is
 * not a layout. */
int mfl_layout_partition_c(const char* c, const char* tile, const char* atom_tv, int64_t atom_m,
                           int64_t atom_n, int64_t warps_m, int64_t warps_n, char* thr_out,
                           char* val_out, int64_t cap);

/* retile_D's regrouping of a register fragment (retile page, sections "先确
 * 定要从哪些 fragment 位置取值" to "两个 K fragment 怎样连成一组"): `frag` is
 * one thread's fragment layout (mode 0 the V values of one MMA, then one mode
 * per repeat direction, values = register slots), `tv` the copy's tiled TV
 * layout over the reference tile of shape `tile_shape` (thread + nthr*value
 * -> position, first coordinate fastest; it must cover the tile once) and
 * atom_nval the values one copy instruction writes per thread.  The copy
 * orders a thread's values as the MMA orders its fragment: values c of block
 * c / V are the V values of one MMA; a block's fragment repeat is where the
 * block lies in the tile (the blocks met walking each tile axis, in order of
 * first appearance).  Returns mode 0 = (values of one copy, copy groups) ->
 * register slot, then the repeats the copy leaves.  -13 when frag's rank is
 * not rank(tile_shape)+1, tv does not cover the tile once, or the counts do
 * not divide; -11 when the blocks do not form a grid. */
int mfl_layout_retile(const char* frag, const char* tv, const char* tile_shape, int64_t nthr,
                      int64_t atom_nval, char* out, int64_t cap);

/* Thread/value layout of a gfx950 matrix instruction operand.
 * op: 0 v_mfma_f32_32x32x16_f16, 1 v_mfma_f32_16x16x32_f16,
 *     2 v_mfma_f32_32x32x8_f16,  3 v_mfma_f32_16x16x16_f16.
 * operand: 0 A (q = m + M*k), 1 B (q = n + N*k), 2 C/D (q = m + M*n).
 * Domain: (lane 0..63, value); flattened index lane + 64*value. */
int mfl_layout_mfma_tv(int32_t op, int32_t operand, char* out, int64_t cap);

/* Per-lane fragment addressing of a GEMM kernel, computed by the same code
 * the kernel runs.  B coordinates are LDS rows: the kernels store B in
 * N-permuted row order (LDS row r of a wave's WTN rows holds tile row
 * RN*(r % 32) + r / 32, RN = WTN / 32), and accumulator coordinates are the
 * physical (m, n).  For every thread t of one workgroup and every fragment
 * slot s of the K sub-steps it takes from one stage (all of them, or its
 * K-group's share when the tile splits K), the (row, k) (operand 0 A, 1 B)
 * or (m, n)
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

/* The back-to-back GEMM's accumulator -> operand map (mfl_chain.h): out[p]
 * = row (0..31 within a 32-row block) of the first, transposed product's
 * accumulator that feeds K position p of the second product's operand,
 * derived at compile time from the 32x32x16 atom's accumulator and operand
 * TV layouts.  The kernel stages B's rows by its inverse, so the operand
 * arrives in natural N1 order.  Pure host code. */
int mfl_chain_k_perm(int32_t* out);

/* Workgroup -> output tile order the kernels use for a grid of
 * tiles_m x tiles_n tiles (XCD-aware grouping, band height group_m):
 * tm[b], tn[b] for every workgroup id b < tiles_m*tiles_n.  Pure host code. */
int mfl_tile_order(int32_t tiles_m, int32_t tiles_n, int32_t group_m, int32_t* tm, int32_t* tn);

#ifdef __cplusplus
}
#endif
#endif /* MFL_LAYOUT_H */

/*
 * mfl_gemm.h — C ABI of the MI355X (gfx950) fp16 "TN" GEMM library.
 *
 * Operation.  D(m,n) = C(m,n) + sum_{k<K} A(m,k) * B(n,k), with A indexed
 * (M,K), B indexed (N,K) and C, D indexed (M,N): the operand directions the
 * TiledMMA page fixes ("读懂 CuTe 的 make_tiled_mma：一条 MMA 怎样铺成一块矩阵",
 * section "先固定矩阵和方向").  "TN" names that operand form (both inputs
 * K-contiguous), as the same section and the retile page ("读懂 CuTe 的
 * retile_D", section "从 CuTe 的名字找到实际指令") explain; it is not a
 * transpose switch.  The kernel structure (tile per workgroup, operand tiles
 * staged through LDS, per-lane fragments taken from the matrix instruction's
 * thread/value layout, K loop of matrix instructions, epilogue) follows the
 * simple-GEMM page ("cute(7) simple_gemm", sections 1–4) and the Tensor
 * Core page ("CuTe Layout 到 Tensor Core", §4–5 CTA tiles and shared-memory
 * layouts), redone for CDNA4 wave64 MFMA instructions.
 *
 * Addressing (element offsets, all row-major in the sense below):
 *   A(m,k) = A[m*lda + k]            a_order = MFL_A_KMAJOR (K contiguous)
 *   A(m,k) = A[m + k*lda]            a_order = MFL_A_MMAJOR (the (M,K):(1,ldA)
 *                                    form of "CuTe Layout 到 Tensor Core" §1)
 *   B(n,k) = B[n*ldb + k]
 *   C(m,n) = C[m*ldc + n],  D(m,n) = D[m*ldd + n]
 *
 * Types.  A and B are fp16 (IEEE binary16).  C is absent (C == NULL, read as
 * 0), fp16 or fp32.  D is fp16 or fp32.  Products are accumulated in fp32;
 * an fp16 D is rounded once, to nearest even, at the end.
 *
 * Ownership and execution.  All pointers are device pointers owned by the
 * caller.  The library never allocates, frees or synchronises, and keeps no
 * pointer after the call returns.  Work is enqueued on `stream` (a
 * hipStream_t; NULL = the null stream) and runs asynchronously; completion
 * is the stream's.  D may equal C only when ldd == ldc and the two dtypes
 * are equal (in-place accumulate); any other overlap is undefined.
 *
 * Errors.  Every function returns 0 on success or a negative MFL_E* code;
 * on error nothing is enqueued.  gemm_strerror() names a code.
 *
 * Degenerate sizes.  M == 0 or N == 0: nothing to do, returns 0.  K == 0:
 * D = C (or 0 when C is absent).
 */
#ifndef MFL_GEMM_H
#define MFL_GEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MFL_NONE = 0, MFL_F16 = 1, MFL_F32 = 2 } mfl_dtype;
typedef enum { MFL_A_KMAJOR = 0, MFL_A_MMAJOR = 1 } mfl_a_order;

/* Kernel choice (low 8 bits of gemm_dtypes_t.algo).  AUTO picks per shape:
 * LDS_256 (LDS_256_16 when both operands go straight into LDS and C is
 * absent) once the grid has at least 192 tiles of 256x256; else LDS_SPLITK
 * when the grid has fewer than 256 tiles of 128x128 and K >= 1024; else
 * LDS_128.
 * DIRECT reads fragments straight from global memory into registers (no
 * LDS; the simple-GEMM page's "不用 Shared Memory" kernel).  LDS_128 stages
 * 128x128x32 block tiles through LDS (the block tile of "CuTe Layout 到
 * Tensor Core" §4) with 4 waves of 64x64.  LDS_256 stages 256x256x64 block
 * tiles with 8 waves of 128x64; LDS_256_W4 the same tile with 4 waves of
 * 128x128.  LDS_128_W1 stages 128x128x32 tiles owned by one wave each (a
 * workgroup of 64 threads, four per CU).  LDS_SPLITK stages 128x64x128
 * tiles with 4 waves that each compute the whole 128x64 tile over their own
 * quarter of every stage's K (the K-direction thread groups of the TiledMMA
 * page, section "K 方向的线程组，与 K 方向的循环"); the four partial tiles are
 * reduced through LDS, every wave finishing a quarter of the tile and adding
 * C once.  The LDS kernels fetch each K-contiguous operand straight into
 * LDS (global_load_lds_dwordx4) when its base and leading dimension are
 * 16-byte aligned, else through registers with 16-byte loads at any 2-byte
 * alignment.  An M-contiguous A goes straight into an M-contiguous LDS tile
 * when its base and lda are 16-byte aligned and M % 8 == 0, and its operand
 * fragments are read with the transposing LDS read; otherwise it is
 * transposed in registers.  MFL_ALGO_REG_FETCH or-ed into algo forces
 * register fetch.
 * The *_16 kernels run the same block tiles on v_mfma_f32_16x16x32_f16
 * (the others on v_mfma_f32_32x32x16_f16): LDS_256_W4_16 with 4 waves of
 * 128x128, LDS_256_16 with 8 waves of 128x64, LDS_128_16 128x128x64 tiles
 * with 4 waves of 64x64, LDS_SPLITK_16 the 128x64x128 split-K tile as 2
 * K-groups of 4 waves of 32x64.  They do not transpose an M-contiguous A in
 * registers, and LDS_256_16 and LDS_SPLITK_16 fetch only straight into LDS;
 * LDS_256_W4 does not combine an M-contiguous A straight into LDS with B
 * through registers.
 * A forced kernel that does not offer the fetch path a call needs returns
 * MFL_E_ALGO_CASE. */
typedef enum {
  MFL_ALGO_AUTO = 0,
  MFL_ALGO_DIRECT = 1,
  MFL_ALGO_LDS_128 = 2,
  MFL_ALGO_LDS_256 = 3,
  MFL_ALGO_LDS_256_W4 = 4,
  MFL_ALGO_LDS_128_W1 = 5,
  MFL_ALGO_LDS_SPLITK = 6,
  MFL_ALGO_LDS_256_W4_16 = 7,
  MFL_ALGO_LDS_256_16 = 8,
  MFL_ALGO_LDS_128_16 = 9,
  MFL_ALGO_LDS_SPLITK_16 = 10,
  MFL_ALGO_COUNT = 11,
  MFL_ALGO_MASK = 0xff,
  MFL_ALGO_REG_FETCH = 0x100
} mfl_algo;

typedef struct {
  int32_t a;        /* mfl_dtype of A: must be MFL_F16 */
  int32_t b;        /* mfl_dtype of B: must be MFL_F16 */
  int32_t c;        /* MFL_NONE (C must be NULL), MFL_F16 or MFL_F32 */
  int32_t d;        /* MFL_F16 or MFL_F32 */
  int32_t a_order;  /* mfl_a_order */
  int32_t algo;     /* mfl_algo */
} gemm_dtypes_t;

enum {
  MFL_OK = 0,
  MFL_E_NEGATIVE_DIM = -1,   /* M, N or K < 0 */
  MFL_E_LEADING_DIM = -2,    /* lda < K (K-major) or < M (M-major); ldb < K;
                                ldc < N with C present; ldd < N */
  MFL_E_NULL_POINTER = -3,   /* A, B or D NULL when M*N*K > 0 (D when M*N > 0);
                                C NULL with c != NONE or non-NULL with NONE */
  MFL_E_UNSUPPORTED = -4,    /* dtype, a_order or algo value (or flag) not supported */
  MFL_E_LAUNCH = -5,         /* the HIP launch reported an error */
  MFL_E_ALGO_CASE = -6,      /* the forced algo cannot run this case */
  MFL_E_MISALIGNED = -7,     /* a pointer not aligned to its element size */
  MFL_E_ALIAS = -8,          /* D == C with different ld or dtype */
  MFL_E_TOO_LARGE = -9       /* a dimension or offset beyond the 2^31 grid /
                                index range the kernels support */
};

/* Enqueue D = C + A * B^T (see above).  `stream` is a hipStream_t. */
int gemm_tn(int64_t M, int64_t N, int64_t K,
            const void* A, int64_t lda,
            const void* B, int64_t ldb,
            const void* C, int64_t ldc,
            void* D, int64_t ldd,
            gemm_dtypes_t dtypes, void* stream);

/* The same argument checks as gemm_tn, without touching the GPU.  Returns
 * the code gemm_tn would return before launching; *algo_out (if not NULL)
 * receives the algorithm AUTO would pick (or the forced one). */
int gemm_tn_validate(int64_t M, int64_t N, int64_t K,
                     const void* A, int64_t lda,
                     const void* B, int64_t ldb,
                     const void* C, int64_t ldc,
                     const void* D, int64_t ldd,
                     gemm_dtypes_t dtypes, int32_t* algo_out);

/* The same checks; on success also reports the kernel the call would run:
 * *algo (mfl_algo without flags) and the fetch policy of A and B
 * (0 direct-to-LDS, 1 through registers, 2 M-contiguous A through registers
 * with transpose, 3 M-contiguous A direct-to-LDS with transposing reads).
 * Any out pointer may be NULL. */
int gemm_tn_plan(int64_t M, int64_t N, int64_t K,
                 const void* A, int64_t lda,
                 const void* B, int64_t ldb,
                 const void* C, int64_t ldc,
                 const void* D, int64_t ldd,
                 gemm_dtypes_t dtypes, int32_t* algo, int32_t* fetch_a, int32_t* fetch_b);

/* Static text for an MFL_* code (never NULL). */
const char* gemm_strerror(int code);

/* Kernel properties of an algorithm for the given dtypes: block tile
 * (bm, bn, bk), threads per workgroup, and the static LDS bytes of the
 * kernel (0 for DIRECT), read from the compiled code object.  Needs a GPU.
 * Any out pointer may be NULL. */
int mfl_kernel_info(int32_t algo, gemm_dtypes_t dtypes, int32_t* bm, int32_t* bn,
                    int32_t* bk, int32_t* threads, int32_t* lds_bytes,
                    int32_t* vgprs_spilled);

#ifdef __cplusplus
}
#endif
#endif /* MFL_GEMM_H */

/*
 * mfl_chain.h — C ABI of the back-to-back GEMM (first accumulator reused as
 * the second operand in registers).
 *
 * For each batch b < batch, with fp16 operands whose rows are contiguous
 * along the summed index (the "TN" form):
 *
 *   S_b(m, n1) = sum_{k < K}  A_b(m, k)  * B_b(n1, k)     fp32 sums
 *   P_b(m, n1) = S_b(m, n1) rounded once to fp16 (nearest, ties to even)
 *   D_b(m, n2) = sum_{n1 < N1} P_b(m, n1) * W_b(n2, n1)    fp32 sums, D fp16 or fp32
 *
 * the attention-style chain of "CuTe Layout 到 Tensor Core" (§17, "为什么这套
 * 抽象对 FlashAttention 特别重要": the first MMA's accumulator, after an
 * element-wise step, is the second MMA's operand; here the step is the
 * rounding to fp16, no softmax).  Addressing (elements):
 *   A_b(m, k)   = A[b*stride_a + m*lda + k]     (M, K)
 *   B_b(n1, k)  = B[b*stride_b + n1*ldb + k]    (N1, K)
 *   W_b(n2, n1) = W[b*stride_w + n2*ldw + n1]   (N2, N1)
 *   D_b(m, n2)  = D[b*stride_d + m*ldd + n2]    (M, N2)
 * Input strides may be 0 (the batch shares the operand).  The summation
 * order over K and over N1 is the kernels' own (fp32); integer-valued inputs
 * whose sums stay below 2^11 in S and 2^24 in D are exact.
 *
 * K must be 32, 64, 128 or 256 (the head dimensions of attention; other K
 * return MFL_E_UNSUPPORTED).  M, N1, N2 and batch are free (N1 == 0 gives
 * D = 0).  Buffers are device pointers owned by the caller; the call is
 * asynchronous on `stream` and allocates nothing.  D must not overlap A, B
 * or W, nor its own batches (stride_d >= M*ldd when batch > 1: else
 * MFL_E_ALIAS).  Error codes are those of mfl_gemm.h; nothing is launched
 * on an error.
 */
#ifndef MFL_CHAIN_H
#define MFL_CHAIN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* d_dtype: MFL_F16 (1) or MFL_F32 (2) */
int gemm_tn_chain(int64_t batch, int64_t M, int64_t N1, int64_t N2, int64_t K,
                  const void* A, int64_t lda, int64_t stride_a,
                  const void* B, int64_t ldb, int64_t stride_b,
                  const void* W, int64_t ldw, int64_t stride_w,
                  void* D, int64_t ldd, int64_t stride_d, int32_t d_dtype, void* stream);

/* the same checks without launching */
int gemm_tn_chain_validate(int64_t batch, int64_t M, int64_t N1, int64_t N2, int64_t K,
                           const void* A, int64_t lda, int64_t stride_a,
                           const void* B, int64_t ldb, int64_t stride_b,
                           const void* W, int64_t ldw, int64_t stride_w,
                           const void* D, int64_t ldd, int64_t stride_d, int32_t d_dtype);

/* how gemm_tn_chain stages B and W for these arguments: the same checks,
 * then *staging = MFL_CHAIN_STAGE_DMA (direct global-to-LDS loads: N1 a
 * multiple of the kernel's N1 chunk, 64 columns, 32 at K = 256; B and W
 * 16-byte aligned with ldb, ldw, stride_b, stride_w multiples of 8) or
 * MFL_CHAIN_STAGE_REGS (through registers, any layout), and *tile_n = the
 * N2 columns per workgroup (64 when N2 <= 64, else 128); either pointer may
 * be NULL.  Every choice gives the same D. */
#define MFL_CHAIN_STAGE_REGS 0
#define MFL_CHAIN_STAGE_DMA 1
int gemm_tn_chain_plan(int64_t batch, int64_t M, int64_t N1, int64_t N2, int64_t K,
                       const void* A, int64_t lda, int64_t stride_a,
                       const void* B, int64_t ldb, int64_t stride_b,
                       const void* W, int64_t ldw, int64_t stride_w,
                       const void* D, int64_t ldd, int64_t stride_d, int32_t d_dtype,
                       int32_t* staging, int32_t* tile_n);

#ifdef __cplusplus
}
#endif
#endif /* MFL_CHAIN_H */

/*
 * Float64 reference for D(m,n) = C(m,n) + sum_k A(m,k) * B(n,k).
 *
 * TEST INFRASTRUCTURE ONLY: called from tests/, the smoke check and the
 * cpu_baseline leg of bench.py; never from the product library.  Shares no
 * header or code with the HIP implementation.
 *
 * The operation is the one the TiledMMA page ("读懂 CuTe 的 make_tiled_mma：
 * 一条 MMA 怎样铺成一块矩阵", section "先固定矩阵和方向") fixes: A is indexed
 * (M,K), B is indexed (N,K), C and D (M,N).  Steps, in this order:
 *   1. every fp16 input bit pattern is decoded exactly to double (binary16:
 *      bias 15, 10 fraction bits, subnormals kept);
 *   2. for each (m,n): s = C(m,n) (0 when C is absent), then
 *      s += A(m,k) * B(n,k) for k = 0, 1, ..., K-1 in that order;
 *   3. D(m,n) = s, unrounded double.
 * A product of two fp16 values has at most 22 significant bits, so each
 * product is exact in double; whether the compiler fuses the add changes
 * nothing.
 *
 * Addressing: A(m,k) = A[m*lda + k] (K-contiguous) or A[m + k*lda] when
 * a_mmajor != 0; B(n,k) = B[n*ldb + k]; C(m,n) = C[m*ldc + n] with C of
 * kind 0 = absent, 1 = fp16 bits, 2 = fp32; D is written densely
 * D[m*ldd + n].
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC gemm_ref.c -o libgemm_ref.so
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double f16_decode(uint16_t h) {
  const double sign = (h & 0x8000u) ? -1.0 : 1.0;
  const int e = (h >> 10) & 0x1f;
  const int f = h & 0x3ff;
  if (e == 0x1f) return f ? NAN : sign * INFINITY;
  if (e == 0) return sign * ldexp((double)f, -24);
  return sign * ldexp((double)(1024 + f), e - 25);
}

static double c_at(const void* C, int c_kind, int64_t ldc, int64_t m, int64_t n) {
  if (c_kind == 1) return f16_decode(((const uint16_t*)C)[m * ldc + n]);
  if (c_kind == 2) return (double)((const float*)C)[m * ldc + n];
  return 0.0;
}

/* number of threads the next parallel region will use */
int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* decode a (rows x K) operand into a dense row-major double array */
static double* decode_operand(const uint16_t* X, int64_t rows, int64_t K,
                              int64_t ld, int mmajor) {
  double* out = (double*)malloc(sizeof(double) * (size_t)(rows > 0 ? rows : 1) *
                                (size_t)(K > 0 ? K : 1));
  if (!out) return NULL;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t k = 0; k < K; ++k)
      out[r * K + k] = f16_decode(mmajor ? X[r + k * ld] : X[r * ld + k]);
  return out;
}

/* Full reference over rows [m0, m1) of D.  Returns 0, or -1 on allocation
 * failure.  nthreads <= 0 keeps the OpenMP default. */
int oracle_gemm_f64(int64_t M, int64_t N, int64_t K,
                    const uint16_t* A, int64_t lda, int a_mmajor,
                    const uint16_t* B, int64_t ldb,
                    const void* C, int c_kind, int64_t ldc,
                    double* D, int64_t ldd, int64_t m0, int64_t m1,
                    int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  if (m1 > M) m1 = M;
  if (m0 < 0) m0 = 0;
  if (m1 <= m0 || N <= 0) return 0;
  const int64_t rows = m1 - m0;
  const uint16_t* Ablk = a_mmajor ? A + m0 : A + m0 * lda;
  double* a = decode_operand(Ablk, rows, K, lda, a_mmajor);
  double* b = decode_operand(B, N, K, ldb, 0);
  if (!a || !b) {
    free(a);
    free(b);
    return -1;
  }
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < rows; ++i) {
    const double* arow = a + i * K;
    for (int64_t n = 0; n < N; ++n) {
      const double* brow = b + n * K;
      double s = c_at(C, c_kind, ldc, m0 + i, n);
      for (int64_t k = 0; k < K; ++k) s += arow[k] * brow[k];
      D[(m0 + i) * ldd + n] = s;
    }
  }
  free(a);
  free(b);
  return 0;
}

/* The same definition evaluated at listed (m,n) pairs only, decoding on the
 * fly (for sampled checks at sizes the full loop cannot afford). */
int oracle_gemm_f64_sampled(int64_t M, int64_t N, int64_t K,
                            const uint16_t* A, int64_t lda, int a_mmajor,
                            const uint16_t* B, int64_t ldb,
                            const void* C, int c_kind, int64_t ldc,
                            int64_t nsamp, const int64_t* ms, const int64_t* ns,
                            double* out, int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 16) reduction(| : bad)
  for (int64_t i = 0; i < nsamp; ++i) {
    const int64_t m = ms[i], n = ns[i];
    if (m < 0 || m >= M || n < 0 || n >= N) {
      bad = 1;
      out[i] = NAN;
      continue;
    }
    double s = c_at(C, c_kind, ldc, m, n);
    for (int64_t k = 0; k < K; ++k) {
      const double av = f16_decode(a_mmajor ? A[m + k * lda] : A[m * lda + k]);
      const double bv = f16_decode(B[n * ldb + k]);
      s += av * bv;
    }
    out[i] = s;
  }
  return bad ? -2 : 0;
}

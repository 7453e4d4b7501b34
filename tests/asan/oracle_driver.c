/* AddressSanitizer / UndefinedBehaviorSanitizer driver for the oracle's C
 * reference (oracle/gemm_ref.c, compiled into this file): random small
 * shapes, both A orders, every C kind, row ranges and sampled positions,
 * buffers allocated to their exact extent so a read past any operand is
 * reported.  Results are compared with a plain loop written here.  Exit 0
 * when every comparison holds. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/gemm_ref.c"

static uint64_t state = 88172645463325252ull;
static uint64_t next_u(void) {   /* xorshift64 */
  state ^= state << 13;
  state ^= state >> 7;
  state ^= state << 17;
  return state;
}
static int64_t rnd(int64_t n) { return n > 0 ? (int64_t)(next_u() % (uint64_t)n) : 0; }

/* small integers in [-2, 2] as binary16 bit patterns */
static uint16_t h_of(int v) {
  static const uint16_t t[5] = {0xC000, 0xBC00, 0x0000, 0x3C00, 0x4000};
  return t[v + 2];
}

int main(int argc, char** argv) {
  if (argc > 1) state += strtoull(argv[1], NULL, 10) * 0x2545F4914F6CDD1Dull;
  int fails = 0;
  for (int it = 0; it < 300; ++it) {
    const int64_t M = rnd(9), N = rnd(9), K = rnd(12);
    const int mm = (int)rnd(2), ck = (int)rnd(3);
    const int64_t lda = (mm ? M : K) + rnd(3), ldb = K + rnd(3), ldc = N + rnd(2),
                  ldd = N + rnd(2);
    const int64_t arows = mm ? K : M;
    /* exact extents: the last row holds only the valid elements */
    const int64_t asz = arows > 0 ? (arows - 1) * lda + (mm ? M : K) : 0;
    const int64_t bsz = N > 0 ? (N - 1) * ldb + K : 0;
    uint16_t* A = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(asz > 0 ? asz : 1));
    uint16_t* B = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(bsz > 0 ? bsz : 1));
    int* av = (int*)malloc(sizeof(int) * (size_t)(M * K + 1));
    int* bv = (int*)malloc(sizeof(int) * (size_t)(N * K + 1));
    for (int64_t m = 0; m < M; ++m)
      for (int64_t k = 0; k < K; ++k) {
        const int v = (int)rnd(5) - 2;
        av[m * K + k] = v;
        A[mm ? m + k * lda : m * lda + k] = h_of(v);
      }
    for (int64_t n = 0; n < N; ++n)
      for (int64_t k = 0; k < K; ++k) {
        const int v = (int)rnd(5) - 2;
        bv[n * K + k] = v;
        B[n * ldb + k] = h_of(v);
      }
    const int64_t csz = M > 0 ? (M - 1) * ldc + N : 0;
    void* C = NULL;
    int* cv = (int*)calloc((size_t)(M * N + 1), sizeof(int));
    if (ck != 0) {
      C = malloc((ck == 1 ? 2 : 4) * (size_t)(csz > 0 ? csz : 1));
      for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
          const int v = (int)rnd(5) - 2;
          cv[m * N + n] = v;
          if (ck == 1)
            ((uint16_t*)C)[m * ldc + n] = h_of(v);
          else
            ((float*)C)[m * ldc + n] = (float)v;
        }
    }
    const int64_t dsz = M > 0 ? (M - 1) * ldd + N : 0;
    double* D = (double*)malloc(sizeof(double) * (size_t)(dsz > 0 ? dsz : 1));
    const int64_t m0 = rnd(M + 1), m1 = m0 + rnd(M - m0 + 1);
    if (oracle_gemm_f64(M, N, K, A, lda, mm, B, ldb, C, ck, ldc, D, ldd, m0, m1, 1) != 0) ++fails;
    for (int64_t m = m0; m < m1; ++m)
      for (int64_t n = 0; n < N; ++n) {
        long s = cv[m * N + n];
        for (int64_t k = 0; k < K; ++k) s += (long)av[m * K + k] * bv[n * K + k];
        if (D[m * ldd + n] != (double)s) ++fails;
      }
    const int64_t ns = 1 + rnd(6);
    int64_t ms[8], nsv[8];
    double out[8];
    int oob = 0;
    for (int64_t i = 0; i < ns; ++i) {
      ms[i] = rnd(M + 2) - 1;   /* includes -1 and M: out of range */
      nsv[i] = rnd(N + 2) - 1;
      if (ms[i] < 0 || ms[i] >= M || nsv[i] < 0 || nsv[i] >= N) oob = 1;
    }
    const int rc = oracle_gemm_f64_sampled(M, N, K, A, lda, mm, B, ldb, C, ck, ldc, ns, ms, nsv,
                                           out, 1);
    if (rc != (oob ? -2 : 0)) ++fails;
    for (int64_t i = 0; i < ns; ++i) {
      if (ms[i] < 0 || ms[i] >= M || nsv[i] < 0 || nsv[i] >= N) {
        if (!isnan(out[i])) ++fails;
        continue;
      }
      long s = cv[ms[i] * N + nsv[i]];
      for (int64_t k = 0; k < K; ++k) s += (long)av[ms[i] * K + k] * bv[nsv[i] * K + k];
      if (out[i] != (double)s) ++fails;
    }
    free(A); free(B); free(av); free(bv); free(C); free(cv); free(D);
  }
  printf("oracle driver: %d mismatches\n", fails);
  return fails != 0;
}

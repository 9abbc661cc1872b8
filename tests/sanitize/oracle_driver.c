/* Drives the oracle's C loop (oracle/oracle.c) under AddressSanitizer and
 * UBSan (built by tests/test_sanitizers.py): closed forms that pin it
 * (identity, all-ones, a hand-worked 2 x 3 by 3 x 2 product), sub-blocks at
 * the matrix edges, empty blocks and rejected arguments. Exit status 0:
 * every expectation held. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_gemm_f32(const float *A, const float *B, double *R, int64_t M, int64_t N, int64_t K,
                    int64_t i0, int64_t i1, int64_t j0, int64_t j1, int nthreads);
int oracle_gemm_bf16(const uint16_t *A, const uint16_t *B, double *R, int64_t M, int64_t N,
                     int64_t K, int64_t i0, int64_t i1, int64_t j0, int64_t j1, int nthreads);
int oracle_gemm_f64(const double *A, const double *B, double *R, int64_t M, int64_t N, int64_t K,
                    int64_t i0, int64_t i1, int64_t j0, int64_t j1, int nthreads);

static int failures = 0;
#define EXPECT(cond)                                                               \
  do {                                                                             \
    if (!(cond)) {                                                                 \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                                  \
    }                                                                              \
  } while (0)

int main(void) {
  /* hand-worked: [[1,2,3],[4,5,6]] x [[1,0],[0,1],[1,1]] = [[4,5],[10,11]] */
  const float a[6] = {1, 2, 3, 4, 5, 6}, b[6] = {1, 0, 0, 1, 1, 1};
  double r[4];
  EXPECT(oracle_gemm_f32(a, b, r, 2, 2, 3, 0, 2, 0, 2, 2) == 0);
  EXPECT(r[0] == 4 && r[1] == 5 && r[2] == 10 && r[3] == 11);
  /* identity and all-ones, fp32 and bf16, with edge sub-blocks */
  enum { n = 37 };
  float *I = calloc(n * n, sizeof(float)), *X = malloc(n * n * sizeof(float));
  uint16_t *ones = malloc(n * n * sizeof(uint16_t));
  double *R = malloc(n * n * sizeof(double));
  for (int i = 0; i < n * n; ++i) X[i] = (float)((i * 7919) % 13) - 6.0f;
  for (int i = 0; i < n; ++i) I[i * n + i] = 1.0f;
  for (int i = 0; i < n * n; ++i) ones[i] = 0x3F80; /* bf16 1.0 */
  EXPECT(oracle_gemm_f32(I, X, R, n, n, n, 0, n, 0, n, 4) == 0);
  for (int i = 0; i < n * n; ++i) EXPECT(R[i] == (double)X[i]);
  EXPECT(oracle_gemm_bf16(ones, ones, R, n, n, n, 30, n, 20, n, 3) == 0);
  for (int i = 0; i < (n - 30) * (n - 20); ++i) EXPECT(R[i] == n);
  double *D = malloc(n * n * sizeof(double));
  for (int i = 0; i < n * n; ++i) D[i] = X[i];
  EXPECT(oracle_gemm_f64(D, D, R, n, n, n, n - 1, n, 0, n, 1) == 0);
  /* empty blocks and K = 0 */
  EXPECT(oracle_gemm_f32(I, X, R, n, n, n, 5, 5, 0, n, 2) == 0);
  EXPECT(oracle_gemm_f32(NULL, NULL, R, n, n, 0, 0, n, 0, n, 2) == 0);
  for (int i = 0; i < n * n; ++i) EXPECT(R[i] == 0.0);
  /* rejected arguments */
  EXPECT(oracle_gemm_f32(I, X, R, n, n, n, 0, n + 1, 0, n, 2) == 1);
  EXPECT(oracle_gemm_f32(I, X, R, -1, n, n, 0, 0, 0, 0, 2) == 1);
  EXPECT(oracle_gemm_f32(I, X, NULL, n, n, n, 0, 1, 0, 1, 2) == 1);
  free(I); free(X); free(ones); free(R); free(D);
  if (failures) fprintf(stderr, "%d expectation(s) failed\n", failures);
  else printf("oracle driver: all expectations held\n");
  return failures ? 1 : 0;
}

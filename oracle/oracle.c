/*
 * CPU oracle for the dense matrix product C = A * B (test infrastructure).
 *
 * Only the tests, the smoke check and the CPU-baseline leg of the benchmark
 * use this file. It shares no code with the HIP library.
 *
 * Definition followed: each output element is the sum over k of
 * A[i,k] * B[k,j], one multiply and one add per term
 * ("09 计算受限还是访存受限" (compute- vs memory-bound), section on counting
 * a matrix multiply; CS336 Lecture 5 GPU notes, §4.2, the naive per-thread
 * snippet). Matrices are row-major: A[i,k] lives at A + i*K + k
 * (CS336 Lecture 5 GPU notes, §4.1, the warning on row-major layout).
 *
 * Arithmetic: every input is widened exactly to double and the sum is taken
 * in double, k ascending for every element, with no fused multiply-add
 * (build with -ffp-contract=off). A product of two fp32 (or bf16) values is
 * exact in double, so the only error is the double-precision summation,
 * bounded by K * 2^-53 * sum_k |A[i,k] * B[k,j]|.
 *
 * Loop order is i, k, j: element (i,j) still receives its terms in
 * ascending k, so the result equals the textbook i, j, k loop bit for bit;
 * the order only makes the row of B contiguous in the inner loop. Rows are
 * shared among OpenMP threads; each element is owned by one thread.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

static double widen_f32(float x) { return (double)x; }

/* bf16 is the upper half of an IEEE fp32 word (CS336 Lecture 5 GPU notes,
 * §3.1, table of floating-point formats). */
static double widen_bf16(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static int bad_args(const void *A, const void *B, const double *R, int64_t M,
                    int64_t N, int64_t K, int64_t i0, int64_t i1, int64_t j0,
                    int64_t j1) {
  if (M < 0 || N < 0 || K < 0) return 1;
  if (i0 < 0 || i1 < i0 || i1 > M || j0 < 0 || j1 < j0 || j1 > N) return 1;
  if ((i1 > i0 && j1 > j0) && R == NULL) return 1;
  if (K > 0 && (i1 > i0 && j1 > j0) && (A == NULL || B == NULL)) return 1;
  return 0;
}

/* R[(i-i0)*(j1-j0) + (j-j0)] = sum_k A[i,k]*B[k,j] for i0<=i<i1, j0<=j<j1.
 * Returns 0 on success, 1 on bad arguments. */
#define ORACLE_BODY(WIDEN_A, WIDEN_B)                                          \
  const int64_t rows = i1 - i0, cols = j1 - j0;                                \
  if (bad_args(A, B, R, M, N, K, i0, i1, j0, j1)) return 1;                    \
  if (rows == 0 || cols == 0) return 0;                                        \
  if (nthreads <= 0) nthreads = 1;                                             \
  _Pragma("omp parallel for schedule(dynamic, 1) num_threads(nthreads)")       \
  for (int64_t i = i0; i < i1; ++i) {                                          \
    double *r = R + (i - i0) * cols;                                           \
    for (int64_t j = 0; j < cols; ++j) r[j] = 0.0;                             \
    for (int64_t k = 0; k < K; ++k) {                                          \
      const double a = WIDEN_A(A[i * K + k]);                                  \
      const int64_t brow = k * N + j0;                                         \
      for (int64_t j = 0; j < cols; ++j) r[j] = r[j] + a * WIDEN_B(B[brow + j]); \
    }                                                                          \
  }                                                                            \
  return 0;

int oracle_gemm_f32(const float *A, const float *B, double *R, int64_t M,
                    int64_t N, int64_t K, int64_t i0, int64_t i1, int64_t j0,
                    int64_t j1, int nthreads) {
  ORACLE_BODY(widen_f32, widen_f32)
}

int oracle_gemm_bf16(const uint16_t *A, const uint16_t *B, double *R,
                     int64_t M, int64_t N, int64_t K, int64_t i0, int64_t i1,
                     int64_t j0, int64_t j1, int nthreads) {
  ORACLE_BODY(widen_bf16, widen_bf16)
}

/* Same sum over operands already widened to double: the FP8 product, whose
 * codes and block scales the Python side decodes to their exact values
 * first. */
static double widen_f64(double x) { return x; }

int oracle_gemm_f64(const double *A, const double *B, double *R, int64_t M,
                    int64_t N, int64_t K, int64_t i0, int64_t i1, int64_t j0,
                    int64_t j1, int nthreads) {
  ORACLE_BODY(widen_f64, widen_f64)
}

/* Threads OpenMP would use by default (for reporting). */
int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Drives the C ABI's host-side validation of every entry point in
 * include/tdm.h under AddressSanitizer and UBSan (built by
 * tests/test_sanitizers.py; no GPU). Device pointers are fake addresses:
 * every call either fails validation or, once its arguments are valid,
 * stops at the device check (TDM_ERROR_NO_DEVICE) before any HIP call that
 * would touch them. Exit status 0: every expectation held. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "tdm.h"

static int failures = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__,     \
              __LINE__, #cond);                                        \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

#define P(x) ((void*)(uintptr_t)(x))
static const uintptr_t A = 0x10000, B = (uintptr_t)1 << 40, C = (uintptr_t)1 << 44,
                       BIAS = (uintptr_t)1 << 42, RES = (uintptr_t)1 << 43;

int main(void) {
  const tdm_status INV = TDM_ERROR_INVALID_VALUE, NS = TDM_ERROR_NOT_SUPPORTED,
                   ND = TDM_ERROR_NO_DEVICE, OK = TDM_SUCCESS;
  /* plain products */
  EXPECT(gemm_f32(P(A), P(B), P(C), -1, 4, 4, NULL) == INV);
  EXPECT(gemm_f32(NULL, P(B), P(C), 4, 4, 4, NULL) == INV);
  EXPECT(gemm_f32(P(A), P(B), P(C + 2), 4, 4, 4, NULL) == INV);
  EXPECT(gemm_f32(P(A), P(B), P(A + 8), 4, 4, 4, NULL) == INV);
  EXPECT(gemm_f32(P(A), P(B), P(C), (int64_t)1 << 32, 1 << 20, 4, NULL) == NS);
  EXPECT(gemm_f32(P(A), P(B), P(C), 0, 4, 4, NULL) == OK);
  EXPECT(gemm_f32(P(A), P(B), P(C), 64, 64, 64, NULL) == ND);
  EXPECT(gemm_bf16_f32acc(P(A), P(B), P(C), 16, 8192, 8192, NULL) == ND);
  EXPECT(gemm_bf16_f32acc(P(A + 1), P(B), P(C), 16, 64, 64, NULL) == INV);
  EXPECT(tdm_gemm_f32_path(P(A), P(B), P(C), 64, 64, 64, (tdm_path)9, NULL) == INV);
  EXPECT(tdm_gemm_f32_path(P(A), P(B), P(C), 64, 64, 64, TDM_PATH_SKINNY, NULL) == NS);
  EXPECT(tdm_gemm_bf16_f32acc_path(P(A), P(B), P(C), 64, 64, 64, TDM_PATH_VALU, NULL) == NS);
  EXPECT(tdm_gemm_bf16_f32acc_path(P(A), P(B), P(C), 64, 64, 64, TDM_PATH_MFMA, NULL) == ND);
  /* epilogue and layouts */
  EXPECT(gemm_bf16_epilogue(P(A), P(B), P(C), (tdm_dtype)7, NULL, NULL, 0, 64, 64, 64, NULL) ==
         INV);
  EXPECT(gemm_bf16_epilogue(P(A), P(B), P(C), TDM_DTYPE_BF16, P(BIAS + 1), NULL, 1, 64, 64, 64,
                            NULL) == INV);
  EXPECT(gemm_bf16_epilogue(P(A), P(B), P(C), TDM_DTYPE_BF16, P(BIAS), P(C), 1, 64, 64, 64,
                            NULL) == ND);
  EXPECT(tdm_gemm_bf16_epilogue_path(P(A), P(B), P(C), TDM_DTYPE_F32, NULL, NULL, 0, 64, 64, 64,
                                     TDM_PATH_VALU, NULL) == NS);
  for (int l = 0; l < 4; ++l) {
    EXPECT(gemm_bf16_ex(P(A), P(B), (tdm_layout)l, P(C), TDM_DTYPE_F32, NULL, NULL, 0, 64, 64,
                        64, NULL) == ND);
    EXPECT(gemm_bf16_ex_noalloc(P(A), P(B), (tdm_layout)l, P(C), TDM_DTYPE_BF16, P(BIAS), NULL,
                                1, 16, 1024, 2048, NULL) == ND);
  }
  EXPECT(gemm_bf16_ex(P(A), P(B), (tdm_layout)4, P(C), TDM_DTYPE_F32, NULL, NULL, 0, 64, 64, 64,
                      NULL) == INV);
  EXPECT(tdm_gemm_bf16_ex_path(P(A), P(B), TDM_LAYOUT_KM_KN, P(C), TDM_DTYPE_F32, NULL, NULL, 0,
                               16, 1024, 2048, TDM_PATH_SKINNY, NULL) == NS);
  EXPECT(tdm_path_supports_ex(TDM_KIND_BF16_F32ACC, TDM_LAYOUT_KM_NK, TDM_PATH_MFMA, 256, 257,
                              520, 0, 0, 0) == 1);
  EXPECT(tdm_select_path_ex(TDM_KIND_BF16_F32ACC, TDM_LAYOUT_KN, 16, 8192, 8192) ==
         TDM_PATH_SKINNY);
  EXPECT(tdm_select_path_ex(TDM_KIND_F32, (tdm_layout)3, 64, 64, 64) == TDM_PATH_EDGE);
  for (int l = 0; l < 4; ++l)
    EXPECT(gemm_f32_ex(P(A), P(B), (tdm_layout)l, P(C), 64, 64, 64, NULL) == ND);
  EXPECT(gemm_f32_ex(P(A), P(B), (tdm_layout)4, P(C), 64, 64, 64, NULL) == INV);
  EXPECT(gemm_f32_ex(P(A), P(B), TDM_LAYOUT_NK, P(A + 8), 4, 4, 4, NULL) == INV);
  EXPECT(tdm_gemm_f32_ex_path(P(A), P(B), TDM_LAYOUT_KM_KN, P(C), 64, 64, 64, TDM_PATH_VALU,
                              NULL) == NS);
  EXPECT(tdm_gemm_f32_ex_path(P(A), P(B), TDM_LAYOUT_KM_NK, P(C), 64, 64, 64, (tdm_path)9,
                              NULL) == INV);
  EXPECT(tdm_select_path_ex(TDM_KIND_F32, TDM_LAYOUT_KM_NK, 4096, 4096, 4096) == TDM_PATH_MFMA);
  /* FP8 */
  EXPECT(gemm_fp8(P(A), TDM_FP8_E4M3, NULL, P(B), TDM_FP8_E5M2, NULL, P(C), TDM_DTYPE_F32, NULL,
                  NULL, 0, 64, 64, 96, NULL) == ND);
  EXPECT(gemm_fp8(P(A), (tdm_fp8_format)2, NULL, P(B), TDM_FP8_E5M2, NULL, P(C), TDM_DTYPE_F32,
                  NULL, NULL, 0, 64, 64, 96, NULL) == INV);
  EXPECT(gemm_fp8(P(A), TDM_FP8_E4M3, P(BIAS), P(B), TDM_FP8_E5M2, NULL, P(C), TDM_DTYPE_F32,
                  NULL, NULL, 0, 64, 64, 96, NULL) == INV);
  EXPECT(gemm_fp8(P(A), TDM_FP8_E4M3, NULL, P(B), TDM_FP8_E5M2, NULL, P(C), TDM_DTYPE_F32, NULL,
                  NULL, 0, 64, 64, 100, NULL) == NS);
  EXPECT(tdm_fp8_supports(64, 64, 96, 0, 0) == 1 && tdm_fp8_supports(64, 64, 96, 8, 0) == 0);
  /* attention */
  EXPECT(attention_fwd(P(A), P(B), P(BIAS), P(C), NULL, 4, 128, 128, 128, 0.088f, 0, NULL) == ND);
  EXPECT(attention_fwd(P(A), P(B), P(BIAS), P(C), P(A + 256), 4, 128, 128, 128, 0.088f, 0,
                       NULL) == INV);
  EXPECT(attention_fwd(P(A), P(B), P(BIAS), P(C), NULL, 4, 128, 128, 96, 0.088f, 0, NULL) == NS);
  EXPECT(attention_fwd(P(A), P(B), P(BIAS), P(C), NULL, 4, 128, 64, 128, 0.088f, 1, NULL) == INV);
  /* host-only queries */
  tdm_roofline r;
  EXPECT(gemm_roofline(TDM_KIND_F32, 4096, 4096, 4096, &r) == OK);
  EXPECT(r.flops == 137438953472.0 && r.bytes == 201326592.0);
  EXPECT(gemm_roofline(TDM_KIND_F32, 4, 4, 4, NULL) == INV);
  EXPECT(gemm_roofline((tdm_kind)5, 4, 4, 4, &r) == INV);
  for (int s = -1; s < 7; ++s) EXPECT(strlen(tdm_status_string((tdm_status)s)) > 0);
  for (int p = -1; p < 7; ++p) EXPECT(strlen(tdm_path_name((tdm_path)p)) > 0);
  EXPECT(tdm_select_path(TDM_KIND_BF16_F32ACC, 8192, 8192, 8192) == TDM_PATH_MFMA);
  EXPECT(tdm_path_supports(TDM_KIND_F32, TDM_PATH_VALU, 4096, 4096, 4096, 0, 0, 0) == 1);
  EXPECT(tdm_version() == TDM_VERSION);
  if (failures) fprintf(stderr, "%d expectation(s) failed\n", failures);
  else printf("abi driver: all expectations held\n");
  return failures ? 1 : 0;
}

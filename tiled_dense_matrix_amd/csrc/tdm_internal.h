// Internal interface between the C ABI (tdm_api.hip) and the kernel files.
// Every launcher enqueues on `stream` and returns hipGetLastError() after
// the launch. Callers have validated sizes and pointers beforehand.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tdm {

// --- shape requirements of each kernel family --------------------------
// Sizes are already known to be >= 1 and each matrix < 2^31 elements.

// 32x32 LDS-tiled kernel: any shape, element-aligned pointers.
inline bool edge_supports(int64_t, int64_t, int64_t) { return true; }

// fp32 register/LDS-tiled VALU kernel: 16-byte chunks along K and N.
bool valu_f32_supports(int64_t M, int64_t N, int64_t K, int mis_a, int mis_b,
                       int mis_c);

// fp32 MFMA kernel: 16-byte chunks along K and N.
bool mfma_f32_supports(int64_t M, int64_t N, int64_t K, int mis_a, int mis_b,
                       int mis_c);

// bf16 MFMA kernel: 16-byte chunks (8 elements) along K and N.
bool mfma_bf16_supports(int64_t M, int64_t N, int64_t K, int mis_a, int mis_b,
                        int mis_c);

// bf16 small-M streaming kernel.
bool skinny_bf16_supports(int64_t M, int64_t N, int64_t K, int mis_a,
                          int mis_b, int mis_c);

// --- launchers ----------------------------------------------------------
hipError_t launch_fill_zero_f32(float* C, int64_t count, hipStream_t s);

hipError_t launch_edge_f32(const float* A, const float* B, float* C, int M,
                           int N, int K, hipStream_t s);
hipError_t launch_edge_bf16(const uint16_t* A, const uint16_t* B, float* C,
                            int M, int N, int K, hipStream_t s);

hipError_t launch_valu_f32(const float* A, const float* B, float* C, int M,
                           int N, int K, hipStream_t s);

hipError_t launch_mfma_f32(const float* A, const float* B, float* C, int M,
                           int N, int K, hipStream_t s);

hipError_t launch_mfma_bf16(const uint16_t* A, const uint16_t* B, float* C,
                            int M, int N, int K, hipStream_t s);

hipError_t launch_skinny_bf16(const uint16_t* A, const uint16_t* B, float* C,
                              int M, int N, int K, hipStream_t s);

}  // namespace tdm

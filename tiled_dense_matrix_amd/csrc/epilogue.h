// Fused epilogue of the bf16-input product, applied where a tile writes C
// (CS336 Lecture 5 GPU notes, §4.3: fusing elementwise work into the kernel
// that produces its input, so the intermediate never goes through HBM; LLM
// course ch. 15, the GELU + residual example).
//
// Per output element, in fp32, after the K sum t of row i, column j:
//   t += bias[j]          (bias != nullptr)
//   t  = GELU(t)          (gelu != 0; t * Phi(t) = t/2 * (1 + erf(t/sqrt 2)),
//                          erf within 1.5e-7, see epi_erf)
//   t += residual[i][j]   (residual != nullptr)
//   D[i][j] = t           as fp32, or as bf16 rounded to nearest even
// bias and residual have D's element type.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tdm {

struct Epilogue {
  const void* bias = nullptr;      // N elements of D's type, or none
  const void* residual = nullptr;  // M x N of D's type (row-major), or none
  int gelu = 0;
  int d_bf16 = 0;                  // D, bias and residual are bf16 (else fp32)
};

__device__ __forceinline__ float epi_bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest, ties to even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t epi_f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  return static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// erf(z) for the GELU, branch-free: Abramowitz and Stegun, Handbook of
// Mathematical Functions, formula 7.1.26 (|error| <= 1.5e-7 for z >= 0),
// with erf(-z) = -erf(z). One reciprocal, one exponential and a degree-5
// polynomial; the library erff branches on the argument's range, and a wave
// whose lanes span several ranges runs every branch.
__device__ __forceinline__ float epi_erf(float z) {
  const float az = fabsf(z);
  const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * az);  // v_rcp_f32 (1 ulp)
  float p = 1.061405429f;
  p = fmaf(p, t, -1.453152027f);
  p = fmaf(p, t, 1.421413741f);
  p = fmaf(p, t, -0.284496736f);
  p = fmaf(p, t, 0.254829592f);
  // exp(-z^2) = 2^(-z^2 log2 e) with v_exp_f32; it underflows to 0 where erf = 1.
  const float e = 1.0f - p * t * __builtin_amdgcn_exp2f(-az * az * 1.44269504088896341f);
  return copysignf(e, z);
}

__device__ __forceinline__ float epi_gelu(float x) {
  return 0.5f * x * (1.0f + epi_erf(x * 0.707106781186547524f));
}

// Finish output element idx = i*N + j (column j) from its K sum t.
__device__ __forceinline__ void epi_store(void* D, int64_t idx, int col, float t,
                                          const Epilogue& e) {
  if (e.d_bf16) {
    if (e.bias) t += epi_bf16_to_f32(static_cast<const uint16_t*>(e.bias)[col]);
    if (e.gelu) t = epi_gelu(t);
    if (e.residual) t += epi_bf16_to_f32(static_cast<const uint16_t*>(e.residual)[idx]);
    static_cast<uint16_t*>(D)[idx] = epi_f32_to_bf16(t);
  } else {
    if (e.bias) t += static_cast<const float*>(e.bias)[col];
    if (e.gelu) t = epi_gelu(t);
    if (e.residual) t += static_cast<const float*>(e.residual)[idx];
    static_cast<float*>(D)[idx] = t;
  }
}

// Four consecutive outputs of one row: columns col..col+3 (those below N
// are stored), element index idx of column col. t holds their K sums, b
// their bias (zeros without one, see epi_bias4). The residual is read and D
// written with one vector access when all four columns exist and the address
// allows it.
typedef float epi_f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t epi_u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t epi_u16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ epi_f32x4 epi_bias4(int col, int N, const Epilogue& e) {
  epi_f32x4 b = {0.f, 0.f, 0.f, 0.f};
  if (e.bias == nullptr) return b;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (col + k < N)
      b[k] = e.d_bf16 ? epi_bf16_to_f32(static_cast<const uint16_t*>(e.bias)[col + k])
                      : static_cast<const float*>(e.bias)[col + k];
  return b;
}

__device__ __forceinline__ void epi_store4(void* D, int64_t idx, int col, int N, epi_f32x4 t,
                                           epi_f32x4 b, const Epilogue& e) {
  const bool all4 = col + 4 <= N;
  const int esize = e.d_bf16 ? 2 : 4;
  const bool vec = all4 && (reinterpret_cast<uintptr_t>(D) + idx * esize) % (4 * esize) == 0 &&
                   (e.residual == nullptr ||
                    (reinterpret_cast<uintptr_t>(e.residual) + idx * esize) % (4 * esize) == 0);
  epi_f32x4 r = {0.f, 0.f, 0.f, 0.f};
  if (e.residual != nullptr) {
    if (vec && e.d_bf16) {
      const epi_u16x4 h = *reinterpret_cast<const epi_u16x4*>(
          static_cast<const uint16_t*>(e.residual) + idx);
#pragma unroll
      for (int k = 0; k < 4; ++k) r[k] = epi_bf16_to_f32(h[k]);
    } else if (vec) {
      r = *reinterpret_cast<const epi_f32x4*>(static_cast<const float*>(e.residual) + idx);
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (col + k < N)
          r[k] = e.d_bf16 ? epi_bf16_to_f32(static_cast<const uint16_t*>(e.residual)[idx + k])
                          : static_cast<const float*>(e.residual)[idx + k];
    }
  }
  epi_f32x4 v;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float x = t[k];
    if (e.bias != nullptr) x += b[k];
    if (e.gelu) x = epi_gelu(x);
    if (e.residual != nullptr) x += r[k];
    v[k] = x;  // no term added: the sum itself, -0.0 included
  }
  if (e.d_bf16) {
    epi_u16x4 h;
#pragma unroll
    for (int k = 0; k < 4; ++k) h[k] = epi_f32_to_bf16(v[k]);
    if (vec) {
      *reinterpret_cast<epi_u16x4*>(static_cast<uint16_t*>(D) + idx) = h;
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (col + k < N) static_cast<uint16_t*>(D)[idx + k] = h[k];
    }
  } else if (vec) {
    *reinterpret_cast<epi_f32x4*>(static_cast<float*>(D) + idx) = v;
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (col + k < N) static_cast<float*>(D)[idx + k] = v[k];
  }
}

}  // namespace tdm

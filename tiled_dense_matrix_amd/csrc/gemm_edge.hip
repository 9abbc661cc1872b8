// Edge path: a plain shared-memory tiled product that is correct for every
// shape and every element-aligned pointer.
//
// Scheme (CS336 Lecture 5 GPU notes, §4.2, tiling): one workgroup owns a
// 32 x 32 tile of C and walks K in steps of 32. Each step the workgroup
// loads a 32 x 32 tile of A and of B into LDS with neighbouring lanes on
// neighbouring addresses (§4.1, coalescing), waits at a barrier, and every
// lane accumulates its 2 x 2 outputs from LDS. Elements outside the matrix
// load as zero, so partial tiles need no other special case.
//
// This kernel carries the ragged remainders the fast paths leave, tiny
// products, and any call whose pointers are not 16-byte aligned.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tdm_internal.h"

namespace tdm {
namespace {

constexpr int kT = 32;        // tile edge
constexpr int kThreads = 256; // 16 x 16 lanes, 2 x 2 outputs each

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// kEpi: finish each output with the fused epilogue and write it to C as the
// epilogue's type says (C is then the epilogue's D); else store the fp32 sum.
// kBNK: B is stored N x K (op(B) = B^T). kAKM: A is stored K x M (op(A) = A^T).
template <typename T, bool kEpi, bool kBNK, bool kAKM = false>
__global__ __launch_bounds__(kThreads) void edge_kernel(
    const T* __restrict__ A, const T* __restrict__ B, void* C,
    int M, int N, int K, int tiles_n, Epilogue epi) {
  __shared__ float As[kT][kT + 1];
  __shared__ float Bs[kT][kT + 1];

  const int tid = threadIdx.x;
  const int tm = blockIdx.x / tiles_n;
  const int tn = blockIdx.x - tm * tiles_n;
  const int m0 = tm * kT;
  const int n0 = tn * kT;

  const int lc = tid & 31;  // loading column inside the tile
  const int lr = tid >> 5;  // loading row (0..7), +8 per pass

  const int ty = tid >> 4;  // output rows ty and ty + 16
  const int tx = tid & 15;  // output cols tx and tx + 16
  float acc00 = 0.f, acc01 = 0.f, acc10 = 0.f, acc11 = 0.f;

  for (int k0 = 0; k0 < K; k0 += kT) {
#pragma unroll
    for (int p = 0; p < kT / 8; ++p) {
      const int r = lr + 8 * p;
      if constexpr (kAKM) {  // lanes along m (contiguous in A), stored transposed
        const int ak = k0 + r, am = m0 + lc;
        As[lc][r] = (am < M && ak < K)
                        ? to_f32(A[static_cast<int64_t>(ak) * M + am]) : 0.f;
      } else {
        const int am = m0 + r, ak = k0 + lc;
        As[r][lc] = (am < M && ak < K)
                        ? to_f32(A[static_cast<int64_t>(am) * K + ak]) : 0.f;
      }
      if constexpr (kBNK) {  // lanes along k (contiguous in B), stored transposed
        const int bn = n0 + r, bk = k0 + lc;
        Bs[lc][r] = (bk < K && bn < N)
                        ? to_f32(B[static_cast<int64_t>(bn) * K + bk]) : 0.f;
      } else {
        const int bk = k0 + r, bn = n0 + lc;
        Bs[r][lc] = (bk < K && bn < N)
                        ? to_f32(B[static_cast<int64_t>(bk) * N + bn]) : 0.f;
      }
    }
    __syncthreads();
#pragma unroll 8
    for (int k = 0; k < kT; ++k) {
      const float a0 = As[ty][k], a1 = As[ty + 16][k];
      const float b0 = Bs[k][tx], b1 = Bs[k][tx + 16];
      acc00 = fmaf(a0, b0, acc00);
      acc01 = fmaf(a0, b1, acc01);
      acc10 = fmaf(a1, b0, acc10);
      acc11 = fmaf(a1, b1, acc11);
    }
    __syncthreads();
  }

  const int r0 = m0 + ty, r1 = m0 + ty + 16;
  const int c0 = n0 + tx, c1 = n0 + tx + 16;
  auto put = [&](int r, int c, float v) {
    if (r >= M || c >= N) return;
    const int64_t idx = static_cast<int64_t>(r) * N + c;
    if constexpr (kEpi)
      epi_store(C, idx, c, v, epi);
    else
      static_cast<float*>(C)[idx] = v;
  };
  put(r0, c0, acc00);
  put(r0, c1, acc01);
  put(r1, c0, acc10);
  put(r1, c1, acc11);
}

__global__ void fill_zero_kernel(float* __restrict__ C, int64_t count) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
       i < count; i += stride)
    C[i] = 0.f;
}

template <typename T, bool kEpi, bool kBNK, bool kAKM = false>
hipError_t launch_edge(const T* A, const T* B, void* C, int M, int N, int K, const Epilogue& e,
                       hipStream_t s) {
  const int tiles_m = (M + kT - 1) / kT;
  const int tiles_n = (N + kT - 1) / kT;
  const int64_t tiles = static_cast<int64_t>(tiles_m) * tiles_n;
  if (tiles > 0x7fffffff) return hipErrorInvalidValue;
  return launch(edge_kernel<T, kEpi, kBNK, kAKM>, dim3(static_cast<unsigned>(tiles)),
                dim3(kThreads), 0, s, A, B, C, M, N, K, tiles_n, e);
}

}  // namespace

hipError_t launch_fill_zero_f32(float* C, int64_t count, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  int64_t blocks = (count + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  return launch(fill_zero_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, C, count);
}

hipError_t launch_edge_f32(const float* A, const float* B, float* C, int M,
                           int N, int K, hipStream_t s) {
  return launch_edge<float, false, false>(A, B, C, M, N, K, Epilogue{}, s);
}

hipError_t launch_edge_f32_layout(const float* A, const float* B, bool b_nk, bool a_km, float* C,
                                  int M, int N, int K, hipStream_t s) {
  if (a_km)
    return b_nk ? launch_edge<float, false, true, true>(A, B, C, M, N, K, Epilogue{}, s)
                : launch_edge<float, false, false, true>(A, B, C, M, N, K, Epilogue{}, s);
  if (b_nk) return launch_edge<float, false, true>(A, B, C, M, N, K, Epilogue{}, s);
  return launch_edge<float, false, false>(A, B, C, M, N, K, Epilogue{}, s);
}

hipError_t launch_edge_bf16(const uint16_t* A, const uint16_t* B, float* C,
                            int M, int N, int K, hipStream_t s) {
  return launch_edge<uint16_t, false, false>(A, B, C, M, N, K, Epilogue{}, s);
}

hipError_t launch_edge_bf16_epi(const uint16_t* A, const uint16_t* B, bool b_nk, bool a_km,
                                void* D, int M, int N, int K, const Epilogue& e, hipStream_t s) {
  if (a_km)
    return b_nk ? launch_edge<uint16_t, true, true, true>(A, B, D, M, N, K, e, s)
                : launch_edge<uint16_t, true, false, true>(A, B, D, M, N, K, e, s);
  if (b_nk) return launch_edge<uint16_t, true, true>(A, B, D, M, N, K, e, s);
  return launch_edge<uint16_t, true, false>(A, B, D, M, N, K, e, s);
}

}  // namespace tdm

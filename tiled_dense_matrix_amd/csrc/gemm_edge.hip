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
//
// Small fp32 products (M and N up to 512, K up to 512, A M x K and B K x N,
// 16-byte rows): the kernel above walks K in eight or more dependent steps,
// each waiting on a global load, and puts few workgroups on the CUs (8 x 8
// for 256^3). small_f32_kernel instead gives each workgroup a 16 x 16 tile
// of C, loads its whole 16 x K panel of A and K x 16 panel of B into LDS at
// once (all loads in flight together), lets its four waves take every
// fourth k, and adds the four partial sums in wave order.
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

constexpr int kSmallT = 16;       // small_f32_kernel: C tile edge
constexpr int kSmallMaxMN = 512;  // largest M and N it takes
constexpr int kSmallMaxK = 512;   // largest K (the panels fill 66 KB of LDS)

// LDS: A panel [16][K + 4] (the row pad puts the 16 rows in different banks),
// then B panel [K][16].
__global__ __launch_bounds__(kThreads) void small_f32_kernel(
    const float* __restrict__ A, const float* __restrict__ B, float* __restrict__ C, int M,
    int N, int K, int tiles_n) {
  extern __shared__ __attribute__((aligned(16))) float small_lds[];
  const int tid = threadIdx.x;
  const int tm = blockIdx.x / tiles_n;
  const int tn = blockIdx.x - tm * tiles_n;
  const int m0 = tm * kSmallT, n0 = tn * kSmallT;
  const int lda = K + 4;
  float* As = small_lds;
  float* Bs = small_lds + kSmallT * lda;
  typedef float f4 __attribute__((ext_vector_type(4)));
  const f4 zero = {0.f, 0.f, 0.f, 0.f};

  // Panels: rows past M and columns past N load as zero. K and N are
  // multiples of 4 and the rows 16-byte aligned, so every float4 lies wholly
  // inside a row, and wholly inside or outside the matrix. Every load of the
  // thread is issued before the first is used (addresses clamped inside the
  // matrix, unused values replaced by zero), so the panels cost one memory
  // latency rather than one per load.
  // A: thread t loads row t/16, float4 columns t%16 + 16j (16 lanes cover
  // 256 contiguous bytes of a row). B: row t/4 + 64j, float4 column t%4.
  constexpr int kJ = kSmallMaxK / 64;  // loads per thread and panel at the largest K
  const int k4 = K / 4;
  const int ar = tid >> 4, ac = tid & 15;
  const int arow = min(m0 + ar, M - 1);
  f4 va[kJ], vb[kJ];
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    const int c = min(ac + 16 * j, k4 - 1);
    va[j] = *reinterpret_cast<const f4*>(A + static_cast<int64_t>(arow) * K + 4 * c);
  }
  const int bc = tid & 3, bk0 = tid >> 2;
  const int bn = min(n0 + 4 * bc, N - 4);
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    const int k = min(bk0 + 64 * j, K - 1);
    vb[j] = *reinterpret_cast<const f4*>(B + static_cast<int64_t>(k) * N + bn);
  }
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    const int c = ac + 16 * j;
    if (c < k4) *reinterpret_cast<f4*>(As + ar * lda + 4 * c) = m0 + ar < M ? va[j] : zero;
  }
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    const int k = bk0 + 64 * j;
    if (k < K) *reinterpret_cast<f4*>(Bs + k * kSmallT + 4 * bc) = n0 + 4 * bc < N ? vb[j] : zero;
  }
  __syncthreads();

  // Wave w takes k = w, w+4, ...; lane l the outputs (l/4, 4(l%4) .. +3).
  const int wave = tid >> 6, lane = tid & 63;
  const int r = lane >> 2, c = 4 * (lane & 3);
  f4 acc = zero;
#pragma unroll 4
  for (int k = wave; k < K; k += 4) {
    const float a = As[r * lda + k];
    const f4 b = *reinterpret_cast<const f4*>(Bs + k * kSmallT + c);
    acc.x = fmaf(a, b.x, acc.x);
    acc.y = fmaf(a, b.y, acc.y);
    acc.z = fmaf(a, b.z, acc.z);
    acc.w = fmaf(a, b.w, acc.w);
  }
  __syncthreads();  // every wave is done with the panels
  float* red = small_lds;  // [wave][16 x 16], over the panels
  *reinterpret_cast<f4*>(red + wave * kSmallT * kSmallT + r * kSmallT + c) = acc;
  __syncthreads();
  const int orow = tid / kSmallT, ocol = tid % kSmallT;
  float sum = 0.f;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) sum += red[w * kSmallT * kSmallT + tid];
  if (m0 + orow < M && n0 + ocol < N) C[static_cast<int64_t>(m0 + orow) * N + n0 + ocol] = sum;
}

bool small_f32_fits(const float* A, const float* B, int M, int N, int K) {
  const bool aligned = (reinterpret_cast<uintptr_t>(A) & 15) == 0 &&
                       (reinterpret_cast<uintptr_t>(B) & 15) == 0;
  return aligned && K % 4 == 0 && N % 4 == 0 && K >= 4 && K <= kSmallMaxK && M >= 1 &&
         M <= kSmallMaxMN && N >= 4 && N <= kSmallMaxMN;
}

hipError_t launch_small_f32(const float* A, const float* B, float* C, int M, int N, int K,
                            hipStream_t s) {
  static std::atomic<uint64_t> lds_ok{0};  // devices already opted in
  // The panels, or the four waves' 16 x 16 partial sums if K is tiny.
  const int lds_bytes = max((kSmallT * (K + 4) + K * kSmallT) * 4, 4 * kSmallT * kSmallT * 4);
  hipError_t e = allow_lds(lds_ok, reinterpret_cast<const void*>(small_f32_kernel),
                           (kSmallT * (kSmallMaxK + 4) + kSmallMaxK * kSmallT) * 4);
  if (e != hipSuccess) return e;
  const int tiles_m = (M + kSmallT - 1) / kSmallT;
  const int tiles_n = (N + kSmallT - 1) / kSmallT;
  return launch(small_f32_kernel, dim3(tiles_m * tiles_n), dim3(kThreads), lds_bytes, s, A, B, C,
                M, N, K, tiles_n);
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
  if (small_f32_fits(A, B, M, N, K)) return launch_small_f32(A, B, C, M, N, K, s);
  return launch_edge<float, false, false>(A, B, C, M, N, K, Epilogue{}, s);
}

hipError_t launch_edge_f32_layout(const float* A, const float* B, bool b_nk, bool a_km, float* C,
                                  int M, int N, int K, hipStream_t s) {
  if (a_km)
    return b_nk ? launch_edge<float, false, true, true>(A, B, C, M, N, K, Epilogue{}, s)
                : launch_edge<float, false, false, true>(A, B, C, M, N, K, Epilogue{}, s);
  if (b_nk) return launch_edge<float, false, true>(A, B, C, M, N, K, Epilogue{}, s);
  return launch_edge_f32(A, B, C, M, N, K, s);
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

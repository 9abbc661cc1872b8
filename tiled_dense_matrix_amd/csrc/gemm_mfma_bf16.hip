// bf16-input / fp32-accumulate product on the gfx950 matrix cores.
//
// Method (CS336 Lecture 5 GPU notes, §4.2 tiling, register blocking and
// double buffering; §3.2 low-precision products with fp32 accumulation;
// LLM course ch. 15 "GPU", §15.6 table of GEMM techniques):
//   * one workgroup owns a 256 x 256 tile of C and walks K in steps of 64;
//   * each step it copies a 256 x 64 slice of A and a 64 x 256 slice of B
//     from HBM into LDS with 16-byte, row-contiguous loads (coalesced);
//   * the four waves (2 x 2) each hold a 128 x 128 block of C in registers
//     (4 x 4 blocks of 32 x 32) and feed v_mfma_f32_32x32x16_bf16 from LDS;
//   * LDS is double-buffered: while the waves multiply slice t, the loads of
//     slice t+1 are in flight, and a single barrier per step separates them.
//
// MFMA wants, in every lane, eight consecutive K values of one row of A and
// of one column of B. A is row-major, so its rows are already K-contiguous.
// B is row-major [K, N] (N-contiguous), so each lane loads an 8 x 8 block of
// B (8 rows, 8 adjacent columns), transposes it in registers, and writes it
// to LDS as Bt[n][k]. Both LDS tiles are therefore [row][64 k] arrays of
// eight 16-byte chunks, and chunk c of row r is stored at c ^ swz(r), an XOR
// swizzle that keeps 8 consecutive rows (the MFMA read) and 8 rows 8 apart
// (the transposed write) on distinct LDS banks.
//
// Partial tiles (M or N not a multiple of 256, K not a multiple of 64) run the
// same loop with clamped, zero-masked loads and masked stores.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tdm_internal.h"
#include "tile_map.h"

namespace tdm {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef float f32x16 __attribute__((ext_vector_type(16)));
// Native 16-byte vector: HIP's uint4 is a struct, which kept the staging
// arrays out of registers.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kBK = 64;
constexpr int kThreads = 256;
constexpr int kChunks = kBK / 8;                  // 16-byte chunks per row
constexpr int kBufChunks = (kBM + kBN) * kChunks; // one stage: A then Bt
constexpr int kLdsBytes = 2 * kBufChunks * 16;    // double-buffered
constexpr int kWaveM = 128, kWaveN = 128;         // per-wave block of C
constexpr int kFragM = kWaveM / 32, kFragN = kWaveN / 32;
constexpr int kGroupM = 4;

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

// 16-bit element e (0..7) of a 16-byte chunk.
__device__ __forceinline__ uint32_t elem(const u32x4& v, int e) {
  const uint32_t d = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y
                   : (e >> 1) == 2 ? v.z : v.w;
  return (e & 1) ? (d >> 16) : (d & 0xffffu);
}

template <bool kGuard>
__device__ __forceinline__ void load_a(const uint16_t* __restrict__ A, int M,
                                       int K, int m0, int k0, int tid,
                                       u32x4 (&ra)[8]) {
  const int c = tid & 7;
  const int r = tid >> 3;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int gm = m0 + r + 32 * i;
    int gk = k0 + c * 8;
    if (!kGuard) {
      ra[i] = *reinterpret_cast<const u32x4*>(A + static_cast<int64_t>(gm) * K + gk);
    } else {
      const bool ok = gm < M && gk < K;
      gm = gm < M ? gm : M - 1;
      gk = gk < K ? gk : K - 8;
      const u32x4 v = *reinterpret_cast<const u32x4*>(A + static_cast<int64_t>(gm) * K + gk);
      ra[i] = ok ? v : u32x4{0u, 0u, 0u, 0u};
    }
  }
}

template <bool kGuard>
__device__ __forceinline__ void load_b(const uint16_t* __restrict__ B, int N,
                                       int K, int n0, int k0, int tid,
                                       u32x4 (&rb)[8]) {
  const int nc = tid & 31;
  const int kb = tid >> 5;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    int gk = k0 + kb * 8 + r;
    int gn = n0 + nc * 8;
    if (!kGuard) {
      rb[r] = *reinterpret_cast<const u32x4*>(B + static_cast<int64_t>(gk) * N + gn);
    } else {
      const bool ok = gk < K && gn < N;
      gk = gk < K ? gk : K - 1;
      gn = gn < N ? gn : N - 8;
      const u32x4 v = *reinterpret_cast<const u32x4*>(B + static_cast<int64_t>(gk) * N + gn);
      rb[r] = ok ? v : u32x4{0u, 0u, 0u, 0u};
    }
  }
}

__device__ __forceinline__ void store_a(u32x4* __restrict__ stage, int tid,
                                        const u32x4 (&ra)[8]) {
  const int c = tid & 7;
  const int r = tid >> 3;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = r + 32 * i;
    stage[row * kChunks + (c ^ swz(row))] = ra[i];
  }
}

// Transpose the lane's 8 (k) x 8 (n) block and store it as Bt[n][k].
__device__ __forceinline__ void store_bt(u32x4* __restrict__ stage, int tid,
                                         const u32x4 (&rb)[8]) {
  const int nc = tid & 31;
  const int kb = tid >> 5;
  u32x4* bt = stage + kBM * kChunks;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    u32x4 o;
    o.x = elem(rb[0], c) | (elem(rb[1], c) << 16);
    o.y = elem(rb[2], c) | (elem(rb[3], c) << 16);
    o.z = elem(rb[4], c) | (elem(rb[5], c) << 16);
    o.w = elem(rb[6], c) | (elem(rb[7], c) << 16);
    const int n = nc * 8 + c;
    bt[n * kChunks + (kb ^ swz(n))] = o;
  }
}

template <bool kGuard>
__device__ __forceinline__ void tile_product(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
    float* __restrict__ C, int M, int N, int K, int m0, int n0,
    u32x4* __restrict__ lds) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lg = lane >> 5;

  f32x16 acc[kFragM][kFragN];
#pragma unroll
  for (int i = 0; i < kFragM; ++i)
#pragma unroll
    for (int j = 0; j < kFragN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int steps = (K + kBK - 1) / kBK;
  u32x4 ra[8], rb[8];
  load_a<kGuard>(A, M, K, m0, 0, tid, ra);
  load_b<kGuard>(B, N, K, n0, 0, tid, rb);
  store_a(lds, tid, ra);
  store_bt(lds, tid, rb);
  __syncthreads();

  for (int t = 0; t < steps; ++t) {
    u32x4* cur = lds + (t & 1) * kBufChunks;
    u32x4* nxt = lds + ((t + 1) & 1) * kBufChunks;
    const bool more = t + 1 < steps;
    if (more) {
      load_a<kGuard>(A, M, K, m0, (t + 1) * kBK, tid, ra);
      load_b<kGuard>(B, N, K, n0, (t + 1) * kBK, tid, rb);
    }
    const u32x4* as = cur;
    const u32x4* bt = cur + kBM * kChunks;
#pragma unroll
    for (int s = 0; s < kBK / 16; ++s) {
      const int chunk = 2 * s + lg;
      bf16x8 a[kFragM], b[kFragN];
#pragma unroll
      for (int i = 0; i < kFragM; ++i) {
        const int row = wm * kWaveM + i * 32 + lr;
        a[i] = as_bf16x8(as[row * kChunks + (chunk ^ swz(row))]);
      }
#pragma unroll
      for (int j = 0; j < kFragN; ++j) {
        const int n = wn * kWaveN + j * 32 + lr;
        b[j] = as_bf16x8(bt[n * kChunks + (chunk ^ swz(n))]);
      }
#pragma unroll
      for (int i = 0; i < kFragM; ++i)
#pragma unroll
        for (int j = 0; j < kFragN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      store_a(nxt, tid, ra);
      store_bt(nxt, tid, rb);
    }
    __syncthreads();
  }

  // Epilogue: element v of a 32 x 32 accumulator sits at
  // row 8*(v/4) + 4*(lane/32) + v%4, column lane%32.
#pragma unroll
  for (int i = 0; i < kFragM; ++i) {
#pragma unroll
    for (int j = 0; j < kFragN; ++j) {
      const int col = n0 + wn * kWaveN + j * 32 + lr;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm * kWaveM + i * 32 + (v >> 2) * 8 + lg * 4 + (v & 3);
        if (!kGuard || (row < M && col < N))
          C[static_cast<int64_t>(row) * N + col] = acc[i][j][v];
      }
    }
  }
}

__global__ __launch_bounds__(kThreads, 1) void mfma_bf16_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
    float* __restrict__ C, int M, int N, int K, int tiles_m, int tiles_n) {
  extern __shared__ u32x4 lds[];
  int tm, tn;
  xcd_tile(blockIdx.x, tiles_m, tiles_n, kGroupM, tm, tn);
  const int m0 = tm * kBM, n0 = tn * kBN;
  const bool full = (m0 + kBM <= M) && (n0 + kBN <= N) && (K % kBK == 0);
  if (full)
    tile_product<false>(A, B, C, M, N, K, m0, n0, lds);
  else
    tile_product<true>(A, B, C, M, N, K, m0, n0, lds);
}

}  // namespace

bool mfma_bf16_supports(int64_t M, int64_t N, int64_t K, int mis_a, int mis_b,
                        int mis_c) {
  (void)M;
  (void)mis_c;
  return K % 8 == 0 && N % 8 == 0 && K >= 8 && mis_a == 0 && mis_b == 0;
}

hipError_t launch_mfma_bf16(const uint16_t* A, const uint16_t* B, float* C,
                            int M, int N, int K, hipStream_t s) {
  // Opt in to more than 64 KB of dynamic LDS (done once per process).
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(mfma_bf16_kernel),
      hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
  if (attr != hipSuccess) return attr;
  const int tiles_m = (M + kBM - 1) / kBM;
  const int tiles_n = (N + kBN - 1) / kBN;
  hipLaunchKernelGGL(mfma_bf16_kernel, dim3(tiles_m * tiles_n), dim3(kThreads),
                     kLdsBytes, s, A, B, C, M, N, K, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace tdm

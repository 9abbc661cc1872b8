// fp32 product on the gfx950 matrix cores (v_mfma_f32_32x32x2_f32).
//
// The same tiling as the bf16 kernel (CS336 Lecture 5 GPU notes, §4.2:
// tiles in shared memory, register blocking, double buffering), with fp32
// operands: each 32 x 32 x 2 MFMA takes one A value and one B value per lane
// and accumulates in fp32.
//   * one workgroup of 8 waves (2 x 4) owns a BM x BN tile of C (256 x 256,
//     or 128 x 128 when a product has too few large tiles to occupy the CUs)
//     and walks K in steps of 32; each wave keeps a (BM/2) x (BN/4) block of C
//     in registers, and two waves per SIMD let one issue matrix instructions
//     while the other waits on LDS or the barrier;
//   * each step's BM x 32 slice of A and 32 x BN slice of B are loaded with
//     16-byte row-contiguous loads into registers one step ahead, then
//     written to the other half of a double-buffered LDS tile;
//   * LDS holds A k-major (As[k][m]) and B as is (Bs[k][n]), so the MFMA
//     operands -- lane l takes row/column l%32 at k = l/32 -- are two rows of
//     32 consecutive floats, read without bank conflicts (the row pitch puts
//     rows k and k+1 in different bank halves).
// fp32 matrix throughput is an eighth of bf16, so per FLOP the tile needs
// little bandwidth; the kernel is bound by MFMA issue.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tdm_internal.h"
#include "tile_map.h"

namespace tdm {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define LDS_PTR(T) __attribute__((address_space(3))) T*

constexpr int kBK = 32;
constexpr int kGroupM = 4;

template <int BM, int BN, int WM, int WN>
struct Tile {
  static constexpr int kBM = BM, kBN = BN, kWN = WN, kThreads = 64 * WM * WN;
  static constexpr int kPitchA = BM + 32;          // floats per LDS row: rows k and
  static constexpr int kPitchB = BN + 32;          // k+1 fall in different bank halves
  static constexpr int kArrayA = kBK * kPitchA;
  static constexpr int kStage = kArrayA + kBK * kPitchB;  // As then Bs
  static constexpr int kLdsBytes = 2 * kStage * 4;        // double-buffered
  static constexpr int kWaveM = BM / WM, kWaveN = BN / WN;
  static constexpr int kFragM = kWaveM / 32, kFragN = kWaveN / 32;
  static constexpr int kLoadsA = BM * kBK / 4 / kThreads;  // 16-byte loads per lane
  static constexpr int kLoadsB = BN * kBK / 4 / kThreads;
};

template <class T, bool kGuard>
__device__ __forceinline__ void load_step(const float* __restrict__ A, const float* __restrict__ B,
                                          int M, int N, int K, int m0, int n0, int k0, int tid,
                                          f32x4 (&ra)[T::kLoadsA], f32x4 (&rb)[T::kLoadsB]) {
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < T::kLoadsA; ++i) {
    const int id = tid + T::kThreads * i;
    int gm = m0 + (id >> 3);
    int gk = k0 + (id & 7) * 4;
    if (!kGuard) {
      ra[i] = *reinterpret_cast<const f32x4*>(A + static_cast<int64_t>(gm) * K + gk);
    } else {
      const bool ok = gm < M && gk < K;
      gm = gm < M ? gm : M - 1;
      gk = gk < K ? gk : K - 4;
      const f32x4 v = *reinterpret_cast<const f32x4*>(A + static_cast<int64_t>(gm) * K + gk);
      ra[i] = ok ? v : zero;
    }
  }
#pragma unroll
  for (int i = 0; i < T::kLoadsB; ++i) {
    const int id = tid + T::kThreads * i;
    int gk = k0 + id / (T::kBN / 4);
    int gn = n0 + (id % (T::kBN / 4)) * 4;
    if (!kGuard) {
      rb[i] = *reinterpret_cast<const f32x4*>(B + static_cast<int64_t>(gk) * N + gn);
    } else {
      const bool ok = gk < K && gn < N;
      gk = gk < K ? gk : K - 1;
      gn = gn < N ? gn : N - 4;
      const f32x4 v = *reinterpret_cast<const f32x4*>(B + static_cast<int64_t>(gk) * N + gn);
      rb[i] = ok ? v : zero;
    }
  }
}

template <class T>
__device__ __forceinline__ void store_step(LDS_PTR(float) stage, int tid,
                                           const f32x4 (&ra)[T::kLoadsA],
                                           const f32x4 (&rb)[T::kLoadsB]) {
  LDS_PTR(float) as = stage;
  LDS_PTR(float) bs = stage + T::kArrayA;
#pragma unroll
  for (int i = 0; i < T::kLoadsA; ++i) {
    const int id = tid + T::kThreads * i;
    const int m = id >> 3, k = (id & 7) * 4;
    as[(k + 0) * T::kPitchA + m] = ra[i].x;
    as[(k + 1) * T::kPitchA + m] = ra[i].y;
    as[(k + 2) * T::kPitchA + m] = ra[i].z;
    as[(k + 3) * T::kPitchA + m] = ra[i].w;
  }
#pragma unroll
  for (int i = 0; i < T::kLoadsB; ++i) {
    const int id = tid + T::kThreads * i;
    *(LDS_PTR(f32x4))(bs + (id / (T::kBN / 4)) * T::kPitchB + (id % (T::kBN / 4)) * 4) = rb[i];
  }
}

template <class T, bool kGuard>
__device__ __forceinline__ void tile_product(const float* __restrict__ A,
                                             const float* __restrict__ B, float* __restrict__ C,
                                             int M, int N, int K, int m0, int n0,
                                             LDS_PTR(float) lds) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave / T::kWN, wn = wave % T::kWN;
  const int lr = lane & 31, lg = lane >> 5;

  f32x16 acc[T::kFragM][T::kFragN];
#pragma unroll
  for (int i = 0; i < T::kFragM; ++i)
#pragma unroll
    for (int j = 0; j < T::kFragN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int steps = (K + kBK - 1) / kBK;
  f32x4 ra[T::kLoadsA], rb[T::kLoadsB];
  load_step<T, kGuard>(A, B, M, N, K, m0, n0, 0, tid, ra, rb);
  store_step<T>(lds, tid, ra, rb);
  __syncthreads();

  for (int t = 0; t < steps; ++t) {
    LDS_PTR(const float) as = lds + (t & 1) * T::kStage;
    LDS_PTR(const float) bs = as + T::kArrayA;
    const bool more = t + 1 < steps;
    if (more) load_step<T, kGuard>(A, B, M, N, K, m0, n0, (t + 1) * kBK, tid, ra, rb);
#pragma unroll 4
    for (int kp = 0; kp < kBK / 2; ++kp) {
      const int k = 2 * kp + lg;
      float a[T::kFragM], b[T::kFragN];
#pragma unroll
      for (int i = 0; i < T::kFragM; ++i) a[i] = as[k * T::kPitchA + wm * T::kWaveM + i * 32 + lr];
#pragma unroll
      for (int j = 0; j < T::kFragN; ++j) b[j] = bs[k * T::kPitchB + wn * T::kWaveN + j * 32 + lr];
#pragma unroll
      for (int i = 0; i < T::kFragM; ++i)
#pragma unroll
        for (int j = 0; j < T::kFragN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (more) store_step<T>(lds + ((t + 1) & 1) * T::kStage, tid, ra, rb);
    __syncthreads();
  }

  // Element v of a 32 x 32 accumulator: row 8*(v/4) + 4*(lane/32) + v%4,
  // column lane%32.
#pragma unroll
  for (int i = 0; i < T::kFragM; ++i)
#pragma unroll
    for (int j = 0; j < T::kFragN; ++j) {
      const int col = n0 + wn * T::kWaveN + j * 32 + lr;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm * T::kWaveM + i * 32 + (v >> 2) * 8 + lg * 4 + (v & 3);
        if (!kGuard || (row < M && col < N)) C[static_cast<int64_t>(row) * N + col] = acc[i][j][v];
      }
    }
}

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN, 1) void mfma_f32_kernel(
    const float* __restrict__ A, const float* __restrict__ B, float* __restrict__ C, int M,
    int N, int K, int tiles_m, int tiles_n) {
  using T = Tile<BM, BN, WM, WN>;
  extern __shared__ __attribute__((aligned(16))) float lds_raw[];
  LDS_PTR(float) lds = (LDS_PTR(float))lds_raw;
  int tm, tn;
  xcd_tile(blockIdx.x, tiles_m, tiles_n, kGroupM, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const bool full = (m0 + BM <= M) && (n0 + BN <= N) && (K % kBK == 0);
  if (full)
    tile_product<T, false>(A, B, C, M, N, K, m0, n0, lds);
  else
    tile_product<T, true>(A, B, C, M, N, K, m0, n0, lds);
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_tile(const float* A, const float* B, float* C, int M, int N, int K,
                       hipStream_t s) {
  using T = Tile<BM, BN, WM, WN>;
  static std::atomic<uint64_t> lds_ok{0};  // devices already opted in
  hipError_t e = allow_lds(lds_ok, reinterpret_cast<const void*>(mfma_f32_kernel<BM, BN, WM, WN>),
                           T::kLdsBytes);
  if (e != hipSuccess) return e;
  const int tiles_m = (M + BM - 1) / BM;
  const int tiles_n = (N + BN - 1) / BN;
  return launch(mfma_f32_kernel<BM, BN, WM, WN>, dim3(tiles_m * tiles_n), dim3(T::kThreads),
                T::kLdsBytes, s, A, B, C, M, N, K, tiles_m, tiles_n);
}

}  // namespace

bool mfma_f32_supports(int64_t M, int64_t N, int64_t K, int mis_a, int mis_b, int mis_c) {
  (void)M;
  (void)mis_c;
  return K % 4 == 0 && N % 4 == 0 && K >= 4 && mis_a == 0 && mis_b == 0;
}

hipError_t launch_mfma_f32(const float* A, const float* B, float* C, int M, int N, int K,
                           hipStream_t s) {
  if (use_large_tiles(M, N, kLargeTileFillF32))
    return launch_tile<256, 256, 2, 4>(A, B, C, M, N, K, s);
  return launch_tile<128, 128, 2, 4>(A, B, C, M, N, K, s);
}

}  // namespace tdm

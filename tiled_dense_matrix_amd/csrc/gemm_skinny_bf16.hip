// Small-M bf16 product (M <= 16): a bandwidth path.
//
// With a handful of rows in A the product does ~2*M FLOPs per byte of B, far
// below the ridge point, so its time is the time to stream B from HBM once
// (CS336 Lecture 5 GPU notes, §2.2 roofline; compute- vs memory-bound lesson,
// what to optimise when memory-bound: read every byte once, in large aligned
// coalesced blocks; LLM course ch. 15, §15.9 on decode-like steps).
//
// Layout of the work:
//   * a workgroup of 16 waves owns a 64-column panel of C (all M rows) and
//     the whole K range; wave w takes a contiguous 1/16 of K;
//   * per step of 32 rows of K a wave loads a 32 x 64 block of B with 16-byte
//     row-contiguous loads (8 lanes per 128-byte row), keeping the next
//     step's loads in flight while it works on the current one;
//   * the block is transposed through a wave-private LDS buffer (16-byte
//     chunks XOR-swizzled so the transposed 2-byte reads hit distinct banks)
//     into the K-contiguous operand layout of v_mfma_f32_16x16x32_bf16;
//     four MFMAs cover the 64 columns, with the rows of A (zero beyond M)
//     as the other operand, read straight from L2 (A is tiny);
//   * the 16 per-wave partial sums are added in LDS in fixed wave order, so
//     results are bitwise reproducible.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tdm_internal.h"

namespace tdm {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 16;
constexpr int kThreads = kWaves * 64;
constexpr int kPanel = 64;      // columns of C per workgroup
constexpr int kStepK = 32;      // K rows per MFMA step
constexpr int kMaxM = 16;
constexpr int kStageBytes = kStepK * kPanel * 2;  // one wave's staging block

// Physical 16-byte chunk of logical chunk c in staging row k.
__device__ __forceinline__ int chunk_pos(int k, int c) {
  return c ^ (((k >> 3) & 3) << 1);
}

template <bool kGuard>
__device__ __forceinline__ void load_step(const uint16_t* __restrict__ B,
                                          int N, int K, int n0, int k0,
                                          int lane, u32x4 (&rb)[4]) {
  const int c = lane & 7;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int gk = k0 + (lane >> 3) + 8 * i;
    int gn = n0 + c * 8;
    if (!kGuard) {
      rb[i] = *reinterpret_cast<const u32x4*>(B + static_cast<int64_t>(gk) * N + gn);
    } else {
      const bool ok = gk < K && gn < N;
      gk = gk < K ? gk : K - 1;
      gn = gn < N ? gn : N - 8;
      const u32x4 v = *reinterpret_cast<const u32x4*>(B + static_cast<int64_t>(gk) * N + gn);
      rb[i] = ok ? v : u32x4{0u, 0u, 0u, 0u};
    }
  }
}

__device__ __forceinline__ u32x4 load_a(const uint16_t* __restrict__ A, int M,
                                        int K, int k0, int lane) {
  const int m = lane & 15;
  const int k = k0 + (lane >> 4) * 8;
  if (m < M && k < K)
    return *reinterpret_cast<const u32x4*>(A + static_cast<int64_t>(m) * K + k);
  return u32x4{0u, 0u, 0u, 0u};
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

template <bool kGuard>
__device__ __forceinline__ void panel_product(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
    float* __restrict__ C, int M, int N, int K, int n0, uint8_t* lds) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;

  // This wave's share of K, in whole steps.
  const int steps_total = (K + kStepK - 1) / kStepK;
  const int per_wave = (steps_total + kWaves - 1) / kWaves;
  const int s_begin = wave * per_wave;
  const int s_end = min(steps_total, s_begin + per_wave);

  uint8_t* stage = lds + wave * kStageBytes;
  f32x4 acc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 rb[4];
  if (s_begin < s_end) load_step<kGuard>(B, N, K, n0, s_begin * kStepK, lane, rb);
  for (int s = s_begin; s < s_end; ++s) {
    const int k0 = s * kStepK;
    // Stage this step's block; row k of the block, chunk c at chunk_pos.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = (lane >> 3) + 8 * i;
      const int c = lane & 7;
      *reinterpret_cast<u32x4*>(stage + k * 128 + chunk_pos(k, c) * 16) = rb[i];
    }
    wave_sync();
    if (s + 1 < s_end) load_step<kGuard>(B, N, K, n0, k0 + kStepK, lane, rb);
    const bf16x8 a = __builtin_bit_cast(bf16x8, load_a(A, M, K, k0, lane));
    // Operand of MFMA q: column 16q + lane%16, rows 8*(lane/16) .. +7.
    const int kb = (lane >> 4) * 8;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int col = q * 16 + (lane & 15);
      const int c = col >> 3, e = col & 7;
      uint32_t w[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int k_lo = kb + 2 * p, k_hi = kb + 2 * p + 1;
        const uint32_t lo = *reinterpret_cast<const uint16_t*>(
            stage + k_lo * 128 + chunk_pos(k_lo, c) * 16 + e * 2);
        const uint32_t hi = *reinterpret_cast<const uint16_t*>(
            stage + k_hi * 128 + chunk_pos(k_hi, c) * 16 + e * 2);
        w[p] = lo | (hi << 16);
      }
      const u32x4 bw = {w[0], w[1], w[2], w[3]};
      acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, bw),
                                                       acc[q], 0, 0, 0);
    }
    wave_sync();
  }

  // Cross-wave sum in LDS: wave w writes its 16 x 64 partial block.
  __syncthreads();
  float* red = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = (lane >> 4) * 4 + v;
      const int col = q * 16 + (lane & 15);
      red[(wave * kMaxM + row) * kPanel + col] = acc[q][v];
    }
  __syncthreads();
  const int row = tid / kPanel, col = tid % kPanel;
  float sum = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) sum += red[(w * kMaxM + row) * kPanel + col];
  if (row < M && n0 + col < N) C[static_cast<int64_t>(row) * N + n0 + col] = sum;
}

__global__ __launch_bounds__(kThreads, 1) void skinny_bf16_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
    float* __restrict__ C, int M, int N, int K) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kWaves * kStageBytes];
  const int n0 = blockIdx.x * kPanel;
  const bool full = (n0 + kPanel <= N) && (K % kStepK == 0);
  if (full)
    panel_product<false>(A, B, C, M, N, K, n0, lds);
  else
    panel_product<true>(A, B, C, M, N, K, n0, lds);
}

static_assert(kWaves * kMaxM * kPanel * 4 <= kWaves * kStageBytes,
              "reduction buffer must fit in the staging LDS");
static_assert(kThreads == kMaxM * kPanel, "one thread per output of the panel");

}  // namespace

bool skinny_bf16_supports(int64_t M, int64_t N, int64_t K, int mis_a,
                          int mis_b, int mis_c) {
  (void)mis_c;
  return M >= 1 && M <= kMaxM && N % 8 == 0 && K % 8 == 0 && K >= 8 &&
         mis_a == 0 && mis_b == 0;
}

hipError_t launch_skinny_bf16(const uint16_t* A, const uint16_t* B, float* C,
                              int M, int N, int K, hipStream_t s) {
  const int panels = (N + kPanel - 1) / kPanel;
  hipLaunchKernelGGL(skinny_bf16_kernel, dim3(panels), dim3(kThreads), 0, s, A,
                     B, C, M, N, K);
  return hipGetLastError();
}

}  // namespace tdm

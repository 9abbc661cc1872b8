// Small-M bf16 product with B stored N x K (C = A * B^T, a linear layer's
// weight as PyTorch keeps it): the decode-like shape of the pages (LLM course
// ch. 15, small batches are bound by reading the weights; CS336 Lecture 5 GPU
// notes, §2.1: the time is the bytes).
//
// With B's rows K-contiguous, each output column j is a dot product of row j
// of B with the rows of A, so a workgroup can take whole rows of B:
//   * workgroup g owns R tiles of 16 consecutive rows of B (R = 1 or 2, the
//     fewest that keep the grid at two workgroups per CU or less) over the
//     full K, and streams them -- one contiguous region of R*16*K*2 bytes --
//     through a 72 KB LDS ring with global_load_lds, 256 k per step (512
//     contiguous bytes of each row), together with the matching 16 x 256
//     slice of A (A is M <= 16 rows; rows past M repeat row M-1). B's copies
//     are marked non-temporal (read once), A's are not (every workgroup
//     reads all of A);
//   * the K loop of workgroup g starts at step g mod (K / 256) and wraps
//     round. Rows of B lie K*2 bytes apart, so with every workgroup at the
//     same step the reads of the whole grid pile onto the few HBM channels
//     that one offset within a row maps to; staggered starts spread them.
//     (16 x 8192 x 8192: 31 us with a common start, 25 us staggered.) The
//     order of the K sum depends on g only, so results are reproducible;
//   * the four waves take two of each step's eight 32-k blocks and run one
//     v_mfma_f32_16x16x32_bf16 per tile and block: A and B operands are both
//     16-byte LDS reads (8 consecutive k of one row);
//   * after the K loop the four waves' sums meet in LDS and are added in wave
//     order, then finished by the epilogue (epilogue.h) and stored. No partial
//     sums leave the workgroup, so there is no workspace and no second kernel.
// LDS rows are 512 bytes (256 k); chunk c (8 k) of row r sits at slot
// c ^ (r % 16), so the 16 rows one read phase touches fall in 16 different
// bank groups. A K that is not a multiple of 256 loads its last step through
// registers, with zeros beyond K, after the wrapped full steps.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lds_copy.h"
#include "tdm_internal.h"

namespace tdm {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxM = 16;
constexpr int kWaves = 4, kThreads = 64 * kWaves;
constexpr int kStepK = 256;                 // k per step
constexpr int kRow = kStepK * 2;            // bytes per LDS row
constexpr int kChunks = kRow / 16;          // 16-byte chunks per row
constexpr int kRowsPerCopy = 1024 / kRow;   // rows one 1 KB copy fills
constexpr int kBlocks = kStepK / 32;        // 32-k MFMA blocks per step
constexpr int kStageA = kMaxM * kRow;
constexpr int kCopyA = kStageA / 1024 / kWaves;  // A copies per wave and step
constexpr int kTargetGroups = 512;           // two workgroups per CU
constexpr int kLdsBudget = 72 * 1024;        // ring bytes per workgroup
static_assert(kRowsPerCopy >= 1 && kCopyA >= 1 && kBlocks % kWaves == 0, "step geometry");

template <int R>
struct NkCfg {
  static constexpr int kRowsB = 16 * R;
  static constexpr int kStageB = kRowsB * kRow;
  static constexpr int kStage = kStageA + kStageB;
  static constexpr int kStages = kLdsBudget / kStage < 8 ? kLdsBudget / kStage : 8;
  static constexpr int kLdsBytes = kStages * kStage;
  static constexpr int kCopyB = kStageB / 1024 / kWaves;  // B copies per wave and step
  static constexpr int kCopies = kCopyA + kCopyB;
  static_assert(kCopyA * kWaves * 1024 == kStageA && kCopyB * kWaves * 1024 == kStageB,
                "whole 1 KB copies");
  static_assert(kStages >= 3 && (kStages - 2) * kCopies <= 63, "ring depth and vmcnt range");
  static_assert(kLdsBytes <= 160 * 1024, "LDS per workgroup");
  static_assert(4 * R * 1024 <= kLdsBytes, "cross-wave reduction fits the ring");
};

__device__ __forceinline__ int slot_of(int row, int c) { return c ^ (row & 15); }

template <int R>
__global__ __launch_bounds__(kThreads, 1) void skinny_nk_bf16_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, void* D, int M, int N,
    int K, Epilogue epi) {
  using T = NkCfg<R>;
  constexpr int S = T::kStages;
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[];
  LDS_PTR(uint8_t) lds = (LDS_PTR(uint8_t))lds_raw;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n_base = blockIdx.x * T::kRowsB;  // first row of B (= column of C)

  // Per-lane copy offsets (bytes from A + k0 and B + k0): copy q fills LDS
  // bytes [1024q, 1024q + 1024) of its operand's stage, lane L row
  // q*kRowsPerCopy + L/kChunks, slot L%kChunks. Wave w does copies w, w+4, ...
  const int crow = lane / kChunks, cslot = lane % kChunks;
  uint32_t off_a[kCopyA], off_b[T::kCopyB];
#pragma unroll
  for (int j = 0; j < kCopyA; ++j) {
    const int r = (wave + kWaves * j) * kRowsPerCopy + crow;
    const int c = slot_of(r, cslot);
    off_a[j] = static_cast<uint32_t>((static_cast<int64_t>(min(r, M - 1)) * K + 8 * c) * 2);
  }
#pragma unroll
  for (int j = 0; j < T::kCopyB; ++j) {
    const int r = (wave + kWaves * j) * kRowsPerCopy + crow;  // row within the B block
    const int c = slot_of(r, cslot);
    const int gn = min(n_base + r, N - 1);
    off_b[j] = static_cast<uint32_t>((static_cast<int64_t>(gn) * K + 8 * c) * 2);
  }

  const int steps = (K + kStepK - 1) / kStepK;
  const int full_steps = K / kStepK;
  const int rot = full_steps > 0 ? static_cast<int>(blockIdx.x % static_cast<unsigned>(full_steps)) : 0;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_offset(lds));

  auto issue = [&](int st, int slot) {
    if (st >= steps) return;
    int ks = st;  // full steps run from step rot, wrapping; the partial one stays last
    if (st < full_steps) {
      ks += rot;
      if (ks >= full_steps) ks -= full_steps;
    }
    const int k0 = ks * kStepK;
    const uint32_t stage = lds0 + slot * T::kStage;
    if (st < full_steps) {
#pragma unroll
      for (int j = 0; j < kCopyA; ++j)
        dma16(A + k0, off_a[j], stage + (wave + kWaves * j) * 1024);
#pragma unroll
      for (int j = 0; j < T::kCopyB; ++j)
        dma16_stream(B + k0, off_b[j], stage + kStageA + (wave + kWaves * j) * 1024);
      return;
    }
    // Partial last step, through registers: zeros beyond K.
    LDS_PTR(uint8_t) st_ptr = lds + slot * T::kStage;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    for (int id = tid; id < (kMaxM + T::kRowsB) * kChunks; id += kThreads) {
      const int row = id / kChunks, c = id % kChunks;
      const int gk = k0 + 8 * c;
      u32x4 v = zero;
      if (row < kMaxM) {
        if (gk < K)
          v = *reinterpret_cast<const u32x4*>(A + static_cast<int64_t>(min(row, M - 1)) * K + gk);
        *(LDS_PTR(u32x4))(st_ptr + row * kRow + (slot_of(row, c) << 4)) = v;
      } else {
        const int r = row - kMaxM;
        if (gk < K)
          v = *reinterpret_cast<const u32x4*>(
              B + static_cast<int64_t>(min(n_base + r, N - 1)) * K + gk);
        *(LDS_PTR(u32x4))(st_ptr + kStageA + r * kRow + (slot_of(r, c) << 4)) = v;
      }
    }
  };
  auto wait_step = [&](int next) {
    if (next + S - 2 < full_steps)
      wait_vm<(S - 2) * T::kCopies>();
    else
      wait_vm<0>();
  };

  f32x4 acc[R];
#pragma unroll
  for (int t = 0; t < R; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Operand reads: lane l takes row l%16 (of A, or of tile t of B) and, in
  // each of this wave's 32-k blocks b, the 8 k at 32*b + 8*(l/16).
  const int orow = lane & 15;

#pragma unroll
  for (int st = 0; st < S - 1; ++st) issue(st, st);
  int cur = 0;
  for (int t = 0; t < steps; ++t) {
    wait_step(t);
    __syncthreads();  // step t has landed; every wave is done with step t-1's slot
    issue(t + S - 1, cur == 0 ? S - 1 : cur - 1);
    LDS_PTR(const uint8_t) sa = lds + cur * T::kStage;
    LDS_PTR(const uint8_t) sb = sa + kStageA;
#pragma unroll
    for (int bb = 0; bb < kBlocks / kWaves; ++bb) {
      const int ochunk = 4 * (wave + kWaves * bb) + (lane >> 4);
      const u32x4 av =
          *(LDS_PTR(const u32x4))(sa + orow * kRow + (slot_of(orow, ochunk) << 4));
      const bf16x8 a = __builtin_bit_cast(bf16x8, av);
#pragma unroll
      for (int tt = 0; tt < R; ++tt) {
        const int r = 16 * tt + orow;
        const u32x4 bv = *(LDS_PTR(const u32x4))(sb + r * kRow + (slot_of(r, ochunk) << 4));
        acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, bv),
                                                          acc[tt], 0, 0, 0);
      }
    }
    cur = cur + 1 == S ? 0 : cur + 1;
  }

  // Cross-wave sum: element v of tile tt sits at row 4*(lane/16) + v, column
  // 16*tt + lane%16 of the block.
  __syncthreads();  // every wave is done with the ring
  LDS_PTR(float) red = (LDS_PTR(float))lds;  // [wave][tile][v][lane]
#pragma unroll
  for (int tt = 0; tt < R; ++tt)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[((wave * R + tt) * 4 + v) * 64 + lane] = acc[tt][v];
  __syncthreads();
  for (int e = tid; e < kMaxM * T::kRowsB; e += kThreads) {
    const int m = e / T::kRowsB, cn = e % T::kRowsB;
    const int tt = cn / 16, l = 16 * (m / 4) + (cn % 16), v = m % 4;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) sum += red[((w * R + tt) * 4 + v) * 64 + l];
    const int n = n_base + cn;
    if (m < M && n < N) epi_store(D, static_cast<int64_t>(m) * N + n, n, sum, epi);
  }
}

template <int R>
hipError_t launch_r(const uint16_t* A, const uint16_t* B, void* D, int M, int N, int K,
                    const Epilogue& e, hipStream_t s) {
  static std::atomic<uint64_t> lds_ok{0};  // devices already opted in
  hipError_t err = allow_lds(lds_ok, reinterpret_cast<const void*>(skinny_nk_bf16_kernel<R>),
                             NkCfg<R>::kLdsBytes);
  if (err != hipSuccess) return err;
  const int groups = (N + NkCfg<R>::kRowsB - 1) / NkCfg<R>::kRowsB;
  return launch(skinny_nk_bf16_kernel<R>, dim3(groups), dim3(kThreads), NkCfg<R>::kLdsBytes, s,
                A, B, D, M, N, K, e);
}

}  // namespace

bool skinny_bf16_nk_supports(int64_t M, int64_t N, int64_t K, int mis_a, int mis_b,
                             int mis_c) {
  (void)N;
  (void)mis_c;
  return M >= 1 && M <= kMaxM && K % 8 == 0 && K >= 8 && mis_a == 0 && mis_b == 0;
}

hipError_t launch_skinny_nk_bf16(const uint16_t* A, const uint16_t* B, void* D, int M, int N,
                                 int K, const Epilogue& e, hipStream_t s) {
  // One tile of 16 rows per workgroup while that keeps the grid at two
  // workgroups per CU or less, else two (four would leave the 72 KB ring
  // fewer than three stages).
  const int tiles = (N + 15) / 16;
  if (tiles <= kTargetGroups) return launch_r<1>(A, B, D, M, N, K, e, s);
  return launch_r<2>(A, B, D, M, N, K, e, s);
}

}  // namespace tdm

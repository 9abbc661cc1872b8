// fp32 product on the gfx950 matrix cores (v_mfma_f32_32x32x2_f32).
//
// The tiling of the bf16 kernel (CS336 Lecture 5 GPU notes, §4.2: tiles in
// shared memory, register blocking, a pipelined K loop), with fp32 operands:
//   * one workgroup of 8 waves (2 x 4) owns a BM x BN tile of C (256 x 256,
//     or 128 x 128 when a product has too few large tiles to occupy the CUs)
//     and walks K in steps of 32; each wave keeps a (BM/2) x (BN/4) block of C
//     in registers as 32 x 32 accumulators, two waves per SIMD;
//   * each step's BM x 32 slice of A and 32 x BN slice of B are copied from
//     HBM straight into LDS (global_load_lds, 16 bytes per lane), with no
//     registers and no LDS store instructions on the way; LDS holds a ring of
//     STAGES steps and the copy of step t+STAGES-1 is issued while step t is
//     multiplied; one barrier per step.
//
// Operand layouts. A 32 x 32 x 2 MFMA takes one A value (row l%32) and one B
// value (column l%32) per lane l, at the MFMA's k index l/32. Which two
// K values an MFMA covers is free, so each group of 8 consecutive k feeds
// four MFMAs r = 0..3 that cover k = 8q + r (lanes 0-31) and 8q + 4 + r
// (lanes 32-63). A lane then needs four consecutive k of its row of A: one
// 16-byte LDS read.
//   A stays row-major in LDS, As[m][k] (128 bytes per row). Chunk c (4 k) of
//   row m sits at chunk c ^ swz_a(m), so the 16 rows a 16-lane read phase
//   touches fill all 64 banks once.
//   B stays row-major too, Bs[k][n]; a lane reads four single floats of its
//   column. Chunk c of row k sits at chunk c ^ swz_b(k): the rows k and k+4
//   that the two halves of a wave read at once land in opposite bank halves.
// Each output is a sum over k in fp32; the order of the terms differs from a
// plain k-ascending loop only by rounding.
//
// Transposed operands (CS336 Lecture 5 GPU notes, review question 5 and the
// §4.1 warning: a transposed operand is another memory layout). A B stored
// N x K has k-contiguous rows like A, so its tile is staged and read as A's
// is (one 16-byte read per lane and group); an A stored K x M has rows of k
// like B, so its tile is staged and read as B's is (four single floats).
// Either way a tile holds the same BK x BM (or BK x BN) elements, so the
// ring's size does not change.
//
// Partial tiles in M or N load clamped (in-bounds) rows/columns whose
// products only reach outputs that are not stored. A K that is not a
// multiple of 32 has its last step loaded through registers with the
// out-of-range elements set to zero.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lds_copy.h"
#include "tdm_internal.h"
#include "tile_map.h"

namespace tdm {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kGroupM = 4;
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

// BNK_: B is stored N x K (C = A * B^T); AKM_: A is stored K x M (C = A^T * B).
template <int BM_, int BN_, int WM_, int WN_, int STAGES_, bool BNK_ = false, bool AKM_ = false>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, BK = 32;
  static constexpr bool kBNK = BNK_, kAKM = AKM_;
  static constexpr int kStages = STAGES_;
  static constexpr int kWaves = WM * WN, kThreads = 64 * kWaves;
  // Bytes per LDS row: a k-contiguous row holds BK floats, a row of k holds
  // the tile's BM (A) or BN (B) floats.
  static constexpr int kRowA = kAKM ? BM * 4 : BK * 4;
  static constexpr int kChunksA = kRowA / 16;
  static constexpr int kRowB = kBNK ? BK * 4 : BN * 4;
  static constexpr int kChunksB = kRowB / 16;
  static constexpr int kStageA = BM * BK * 4;
  static constexpr int kStageB = BN * BK * 4;
  static constexpr int kStage = kStageA + kStageB;
  static constexpr int kLdsBytes = kStages * kStage;
  static constexpr int kWaveM = BM / WM, kWaveN = BN / WN;
  static constexpr int kFragM = kWaveM / 32, kFragN = kWaveN / 32;
  static constexpr int kCopyA = kStageA / 1024 / kWaves;  // copies per wave and step
  static constexpr int kCopyB = kStageB / 1024 / kWaves;
  static constexpr int kCopies = kCopyA + kCopyB;
  static constexpr int kRowsPerCopyA = 1024 / kRowA;
  static constexpr int kRowsPerCopyB = 1024 / kRowB;
  static constexpr int kGroups = BK / 8;                 // 8-k groups per step
  static constexpr int kMfmas = 4 * kFragM * kFragN;     // MFMAs per group
  static constexpr int kReads = (kAKM ? 4 : 1) * kFragM + (kBNK ? 1 : 4) * kFragN;  // per group
  static_assert(kCopyA * kWaves * 1024 == kStageA && kCopyB * kWaves * 1024 == kStageB,
                "each wave copies whole 1 KB blocks");
  static_assert(kRowsPerCopyA >= 1 && kRowsPerCopyB >= 1 && BM % 64 == 0 && BN % 64 == 0,
                "LDS rows of 1 KB or less that divide a 1 KB copy");
  static_assert(kStageA % (16 * kThreads) == 0 && kStageB % (16 * kThreads) == 0,
                "masked copy: whole 16-byte chunks per lane");
  static_assert(kGroups % 2 == 0, "fragment double buffer alternates per group");
  static_assert(kStages >= 2 && (kStages - 2) * kCopies <= 63, "vmcnt range");
  static_assert(kLdsBytes <= 160 * 1024, "LDS per workgroup");
};

__device__ __forceinline__ int swz_a(int m) { return (m >> 1) & 7; }
__device__ __forceinline__ int swz_b(int k) { return ((k >> 2) & 1) << 3; }

// Byte offset of a lane's 16-byte chunk in copy `copy` of one operand's
// tile, relative to the tile's first element at k0. kKMajor: the operand is
// stored K x ext (rows of k; the lane takes 4 columns, clamped to the last
// whole group of 4 below ext); else it is stored ext x K (k-contiguous rows
// of the tile's `rows` rows, clamped to ext - 1). o0: the tile's first
// row/column; ld: the stored row length.
template <bool kKMajor, int kRowsPerCopy, int kChunks>
__device__ __forceinline__ uint32_t plan_off(int copy, int lane, int o0, int ext, int ld) {
  const int row = copy * kRowsPerCopy + lane / kChunks;
  if constexpr (kKMajor) {
    const int c = (lane % kChunks) ^ swz_b(row);
    const int d = min(o0 + c * 4, ext - 4) - o0;
    return static_cast<uint32_t>((static_cast<int64_t>(row) * ld + d) * 4);
  } else {
    const int c = (lane % kChunks) ^ swz_a(row);
    const int d = min(o0 + row, ext - 1) - o0;
    return static_cast<uint32_t>((static_cast<int64_t>(d) * ld + c * 4) * 4);
  }
}

// Per-lane byte offsets of this wave's copies, relative to each operand
// tile's first element at k0 (tile_a / tile_b below).
template <class T>
struct CopyPlan {
  uint32_t a[T::kCopyA];
  uint32_t b[T::kCopyB];
};

template <class T>
__device__ __forceinline__ CopyPlan<T> make_plan(int M, int N, int K, int m0, int n0, int wave,
                                                 int lane) {
  CopyPlan<T> p;
#pragma unroll
  for (int j = 0; j < T::kCopyA; ++j)
    p.a[j] = plan_off<T::kAKM, T::kRowsPerCopyA, T::kChunksA>(wave * T::kCopyA + j, lane, m0, M,
                                                              T::kAKM ? M : K);
#pragma unroll
  for (int j = 0; j < T::kCopyB; ++j)
    p.b[j] = plan_off<!T::kBNK, T::kRowsPerCopyB, T::kChunksB>(wave * T::kCopyB + j, lane, n0, N,
                                                               T::kBNK ? K : N);
  return p;
}

// First element of each operand's tile at k0.
template <class T>
__device__ __forceinline__ const float* tile_a(const float* A, int M, int K, int m0, int k0) {
  return T::kAKM ? A + static_cast<int64_t>(k0) * M + m0 : A + static_cast<int64_t>(m0) * K + k0;
}
template <class T>
__device__ __forceinline__ const float* tile_b(const float* B, int N, int K, int n0, int k0) {
  return T::kBNK ? B + static_cast<int64_t>(n0) * K + k0 : B + static_cast<int64_t>(k0) * N + n0;
}

template <class T>
__device__ __forceinline__ void copy_step_dma(const float* A, const float* B, int M, int N, int K,
                                              int m0, int n0, int k0, int wave,
                                              const CopyPlan<T>& p, uint32_t stage) {
  const float* a_base = tile_a<T>(A, M, K, m0, k0);
  const float* b_base = tile_b<T>(B, N, K, n0, k0);
#pragma unroll
  for (int j = 0; j < T::kCopyA; ++j)
    dma16(a_base, p.a[j], stage + (wave * T::kCopyA + j) * 1024);
#pragma unroll
  for (int j = 0; j < T::kCopyB; ++j)
    dma16(b_base, p.b[j], stage + T::kStageA + (wave * T::kCopyB + j) * 1024);
}

// One operand's tile through registers, with zeros beyond K (the partial
// last step), in the layout the copies give it (plan_off).
template <bool kKMajor, int kStage, int kRow, int kChunks, int kThreads>
__device__ __forceinline__ void masked_tile(const float* __restrict__ X, int o0, int ext, int K,
                                            int k0, int tid, LDS_PTR(uint8_t) dst) {
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kStage / 16 / kThreads; ++i) {
    const int id = tid + kThreads * i;
    const int row = id / kChunks, c = id % kChunks;
    f32x4 v = zero;
    if constexpr (kKMajor) {  // row = k, 4 columns
      const int gk = k0 + row, g = min(o0 + c * 4, ext - 4);
      if (gk < K) v = *reinterpret_cast<const f32x4*>(X + static_cast<int64_t>(gk) * ext + g);
      *(LDS_PTR(f32x4))(dst + row * kRow + ((c ^ swz_b(row)) << 4)) = v;
    } else {  // row of the operand, 4 k
      const int gk = k0 + c * 4, g = min(o0 + row, ext - 1);
      if (gk < K) v = *reinterpret_cast<const f32x4*>(X + static_cast<int64_t>(g) * K + gk);
      *(LDS_PTR(f32x4))(dst + row * kRow + ((c ^ swz_a(row)) << 4)) = v;
    }
  }
}

template <class T>
__device__ __forceinline__ void copy_step_masked(const float* __restrict__ A,
                                                 const float* __restrict__ B, int M, int N, int K,
                                                 int m0, int n0, int k0, int tid,
                                                 LDS_PTR(uint8_t) stage) {
  masked_tile<T::kAKM, T::kStageA, T::kRowA, T::kChunksA, T::kThreads>(A, m0, M, K, k0, tid, stage);
  masked_tile<!T::kBNK, T::kStageB, T::kRowB, T::kChunksB, T::kThreads>(B, n0, N, K, k0, tid,
                                                                      stage + T::kStageA);
}

// k = 8q + 4*(lane/32) + 0..3 of row `row` of a k-contiguous tile: one
// 16-byte read.
template <int kRow>
__device__ __forceinline__ f32x4 read_rows(LDS_PTR(const uint8_t) s, int row, int q, int lg) {
  const int chunk = 2 * q + lg;
  return *(LDS_PTR(const f32x4))(s + row * kRow + ((chunk ^ swz_a(row)) << 4));
}

// Rows k = 8q + 4*(lane/32) + 0..3 of column `col` of a tile of k rows:
// four single floats.
template <int kRow>
__device__ __forceinline__ f32x4 read_cols(LDS_PTR(const uint8_t) s, int col, int q, int lg) {
  const int k = 8 * q + 4 * lg;
  LDS_PTR(const uint8_t) p = s + (((col >> 2) ^ swz_b(k)) << 4) + ((col & 3) << 2);
  f32x4 v;
  v.x = *(LDS_PTR(const float))(p + (k + 0) * kRow);
  v.y = *(LDS_PTR(const float))(p + (k + 1) * kRow);
  v.z = *(LDS_PTR(const float))(p + (k + 2) * kRow);
  v.w = *(LDS_PTR(const float))(p + (k + 3) * kRow);
  return v;
}

// The lane's four k of row `row` of op(A) / column `col` of op(B).
template <class T>
__device__ __forceinline__ f32x4 read_a(LDS_PTR(const uint8_t) sa, int row, int q, int lg) {
  if constexpr (T::kAKM) return read_cols<T::kRowA>(sa, row, q, lg);
  return read_rows<T::kRowA>(sa, row, q, lg);
}
template <class T>
__device__ __forceinline__ f32x4 read_b(LDS_PTR(const uint8_t) sb, int col, int q, int lg) {
  if constexpr (T::kBNK) return read_rows<T::kRowB>(sb, col, q, lg);
  return read_cols<T::kRowB>(sb, col, q, lg);
}

// One read of the next group's operands after each MFMA, leftovers after.
template <class T>
__device__ __forceinline__ void interleave_hint() {
  constexpr int kPairs = T::kReads < T::kMfmas ? T::kReads : T::kMfmas;
#pragma unroll
  for (int r = 0; r < kPairs; ++r) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
  }
  if (T::kMfmas > kPairs) __builtin_amdgcn_sched_group_barrier(kSchedMfma, T::kMfmas - kPairs, 0);
  if (T::kReads > kPairs) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, T::kReads - kPairs, 0);
}

template <class T>
__global__ __launch_bounds__(T::kThreads, 1) void mfma_f32_kernel(
    const float* __restrict__ A, const float* __restrict__ B, float* __restrict__ C, int M, int N,
    int K, int tiles_m, int tiles_n) {
  constexpr int S = T::kStages;
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[];
  LDS_PTR(uint8_t) lds = (LDS_PTR(uint8_t))lds_raw;

  int tm, tn;
  xcd_tile(blockIdx.x, tiles_m, tiles_n, kGroupM, tm, tn);
  const int m0 = tm * T::BM, n0 = tn * T::BN;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int wm = wave / T::WN, wn = wave % T::WN;
  const int lr = lane & 31, lg = lane >> 5;
  const int row_a = wm * T::kWaveM + lr;  // + 32 i: this lane's rows of A
  const int col_b = wn * T::kWaveN + lr;  // + 32 j: this lane's columns of B

  f32x16 acc[T::kFragM][T::kFragN];
#pragma unroll
  for (int i = 0; i < T::kFragM; ++i)
#pragma unroll
    for (int j = 0; j < T::kFragN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int steps = (K + T::BK - 1) / T::BK;
  const int full_steps = K / T::BK;
  const CopyPlan<T> plan = make_plan<T>(M, N, K, m0, n0, wave, lane);
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_offset(lds));

  auto issue = [&](int st, int slot) {
    if (st < full_steps)
      copy_step_dma<T>(A, B, M, N, K, m0, n0, st * T::BK, wave, plan, lds0 + slot * T::kStage);
    else if (st < steps)
      copy_step_masked<T>(A, B, M, N, K, m0, n0, st * T::BK, tid, lds + slot * T::kStage);
  };
  auto wait_step = [&](int next) {
    if (S > 2 && next + S - 2 < full_steps)
      wait_vm<(S > 2 ? (S - 2) * T::kCopies : 0)>();
    else
      wait_vm<0>();
  };

#pragma unroll
  for (int st = 0; st < S - 1; ++st) issue(st, st);
  wait_step(0);
  __syncthreads();

  f32x4 a[2][T::kFragM], b[2][T::kFragN];
#pragma unroll
  for (int i = 0; i < T::kFragM; ++i) a[0][i] = read_a<T>(lds, row_a + 32 * i, 0, lg);
#pragma unroll
  for (int j = 0; j < T::kFragN; ++j) b[0][j] = read_b<T>(lds + T::kStageA, col_b + 32 * j, 0, lg);

  int cur = 0;
  for (int t = 0; t < steps; ++t) {
    const int nxt = cur + 1 == S ? 0 : cur + 1;
    issue(t + S - 1, cur == 0 ? S - 1 : cur - 1);
    LDS_PTR(const uint8_t) sa = lds + cur * T::kStage;
    LDS_PTR(const uint8_t) sb = sa + T::kStageA;
#pragma unroll
    for (int q = 0; q < T::kGroups; ++q) {
      const int c = q & 1, n = c ^ 1;
      if (q + 1 < T::kGroups) {
#pragma unroll
        for (int i = 0; i < T::kFragM; ++i) a[n][i] = read_a<T>(sa, row_a + 32 * i, q + 1, lg);
#pragma unroll
        for (int j = 0; j < T::kFragN; ++j) b[n][j] = read_b<T>(sb, col_b + 32 * j, q + 1, lg);
      } else {
        // Step t+1's copies have landed and every wave is done with the slot
        // the next issue overwrites; its first operands are read while the
        // last MFMAs of step t run. After the last step these reads fetch
        // stale values that are never used.
        wait_step(t + 1);
        __syncthreads();
        LDS_PTR(const uint8_t) na = lds + nxt * T::kStage;
#pragma unroll
        for (int i = 0; i < T::kFragM; ++i) a[n][i] = read_a<T>(na, row_a + 32 * i, 0, lg);
#pragma unroll
        for (int j = 0; j < T::kFragN; ++j)
          b[n][j] = read_b<T>(na + T::kStageA, col_b + 32 * j, 0, lg);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int i = 0; i < T::kFragM; ++i)
#pragma unroll
          for (int j = 0; j < T::kFragN; ++j)
            acc[i][j] =
                __builtin_amdgcn_mfma_f32_32x32x2f32(a[c][i][r], b[c][j][r], acc[i][j], 0, 0, 0);
      interleave_hint<T>();
    }
    cur = nxt;
  }

  // Element v of a 32 x 32 accumulator: row 8*(v/4) + 4*(lane/32) + v%4,
  // column lane%32.
  const bool full = (m0 + T::BM <= M) && (n0 + T::BN <= N);
#pragma unroll
  for (int i = 0; i < T::kFragM; ++i)
#pragma unroll
    for (int j = 0; j < T::kFragN; ++j) {
      const int col = n0 + col_b + 32 * j;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm * T::kWaveM + i * 32 + (v >> 2) * 8 + lg * 4 + (v & 3);
        if (full || (row < M && col < N)) C[static_cast<int64_t>(row) * N + col] = acc[i][j][v];
      }
    }
}

template <class T>
hipError_t launch_tile(const float* A, const float* B, float* C, int M, int N, int K,
                       hipStream_t s) {
  static std::atomic<uint64_t> lds_ok{0};  // devices already opted in
  hipError_t e = allow_lds(lds_ok, reinterpret_cast<const void*>(mfma_f32_kernel<T>),
                           T::kLdsBytes);
  if (e != hipSuccess) return e;
  const int tiles_m = (M + T::BM - 1) / T::BM;
  const int tiles_n = (N + T::BN - 1) / T::BN;
  return launch(mfma_f32_kernel<T>, dim3(tiles_m * tiles_n), dim3(T::kThreads), T::kLdsBytes, s,
                A, B, C, M, N, K, tiles_m, tiles_n);
}

template <bool BNK, bool AKM>
using LargeTile = Cfg<256, 256, 2, 4, 2, BNK, AKM>;
template <bool BNK, bool AKM>
using SmallTile = Cfg<128, 128, 2, 4, 4, BNK, AKM>;

template <bool BNK, bool AKM>
hipError_t launch_layout(const float* A, const float* B, float* C, int M, int N, int K,
                         hipStream_t s) {
  if (use_large_tiles(M, N, kLargeTileFillF32))
    return launch_tile<LargeTile<BNK, AKM>>(A, B, C, M, N, K, s);
  return launch_tile<SmallTile<BNK, AKM>>(A, B, C, M, N, K, s);
}

}  // namespace

bool mfma_f32_supports(int64_t M, int64_t N, int64_t K, int mis_a, int mis_b, int mis_c,
                       bool b_nk, bool a_km) {
  (void)mis_c;
  // 16-byte chunks along K of k-contiguous rows, along N or M of rows of k;
  // 32-bit per-lane copy offsets: 256 k-contiguous rows (K floats each) or
  // 32 rows of k (N or M floats each) stay below 4 GiB from a tile's first
  // element.
  if (K % 4 != 0 || K < 4 || K >= (1 << 22) || mis_a != 0 || mis_b != 0) return false;
  if (!b_nk && (N % 4 != 0 || N >= (1 << 25))) return false;
  if (a_km && (M % 4 != 0 || M >= (1 << 25))) return false;
  return true;
}

hipError_t launch_mfma_f32(const float* A, const float* B, float* C, int M, int N, int K,
                           hipStream_t s) {
  return launch_layout<false, false>(A, B, C, M, N, K, s);
}

hipError_t launch_mfma_f32_layout(const float* A, const float* B, bool b_nk, bool a_km, float* C,
                                  int M, int N, int K, hipStream_t s) {
  if (a_km)
    return b_nk ? launch_layout<true, true>(A, B, C, M, N, K, s)
                : launch_layout<false, true>(A, B, C, M, N, K, s);
  return b_nk ? launch_layout<true, false>(A, B, C, M, N, K, s)
              : launch_layout<false, false>(A, B, C, M, N, K, s);
}

}  // namespace tdm

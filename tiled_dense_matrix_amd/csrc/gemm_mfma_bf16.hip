// bf16-input / fp32-accumulate product on the gfx950 matrix cores.
//
// Method (CS336 Lecture 5 GPU notes, §4.2 tiling, register blocking and
// double buffering; §3.2 low-precision products with fp32 accumulation;
// LLM course ch. 15 "GPU", §15.6 table of GEMM techniques):
//   * one workgroup owns a BM x BN tile of C (256 x 256, or 128 x 128 when a
//     product has too few large tiles to occupy the CUs) and walks K in steps
//     of BK, from a start staggered by up to fifteen steps between
//     neighbouring workgroups (spreads the L2 channels a step's loads hit);
//   * each step copies a BM x BK slice of A and a BK x BN slice of B from HBM
//     into LDS with 16-byte row-contiguous loads that write LDS directly
//     (global_load_lds), so the copy costs no registers and no LDS stores;
//   * eight waves (2 x 4) each hold a (BM/2) x (BN/4) block of C in registers
//     as 16 x 16 accumulators fed by v_mfma_f32_16x16x32_bf16 (on normal
//     operands, where the part runs at its power limit, a loop of these
//     sustained 13% more FLOPs than one of 32 x 32 x 16 MFMAs); each SIMD
//     holds two waves, one of each half of the workgroup;
//   * LDS holds a ring of STAGES steps: the copy of step t+STAGES-1 is issued
//     while the waves multiply step t, so a copy has STAGES-1 steps to land
//     (data that misses the XCD's L2 comes from the last-level cache or HBM,
//     whose latency one step does not cover);
//   * the two halves of the workgroup take turns (ping-pong): while waves
//     0-3 run a step's MFMAs on fragments already in registers, waves 4-7
//     read theirs from LDS and issue their copies, then they swap, with a
//     workgroup barrier between phases. Rings of two slots and a partial
//     last K step use one loop per wave instead, which reads the next
//     sub-step's fragments while the current one is multiplied;
//   * C is written through LDS in row-contiguous groups of four, where the
//     optional fused epilogue (bias, GELU, residual, bf16 output; §4.3
//     operator fusion) finishes each output.
//
// Operand layouts. MFMA wants, in every lane, eight consecutive K values of
// one row of A and of one column of B.
//   A stays row-major in LDS, As[m][k] (2*BK bytes per row), and is read with
//   16-byte loads. Chunk c (8 k values) of row m sits at chunk c ^ swz_a(m).
//   An A stored K x M (the product is then A^T B for the stored matrix, the
//   pages' x = A.T @ B) is staged k-major like a K x N B, As[k][m], and read
//   with the same transposing reads as B below.
//   B stays row-major too, Bs[k][n] (2*BN bytes per row), and is read with
//   ds_read_b64_tr_b16: within each group of 16 lanes, lane j receives
//   element e from the address of lane 4e + j/4, so lanes that point at four
//   consecutive n of rows k..k+3 come back holding four consecutive k of one
//   column. Chunk c of row k sits at chunk c ^ swz_b(k).
// Both swizzles spread the rows each read touches over distinct LDS banks.
//
// Partial tiles in M or N load clamped (in-bounds) rows/columns whose
// products only reach outputs that are not stored. A K that is not a
// multiple of BK has its last step loaded through registers with the
// out-of-range elements set to zero.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lds_copy.h"
#include "tdm_internal.h"
#include "tile_map.h"

namespace tdm {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kGroupM = 8;
// Instruction classes of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

// Tile geometry. Copies move 1 KB of LDS per wave instruction. BNK_: B is
// stored N x K (C = A * B^T, a linear layer's weight) and is then kept in LDS
// like A, one K-contiguous row per column n; otherwise B is K x N. AKM_: A is
// stored K x M and kept in LDS k-major, one M-contiguous row per k, like a
// K x N B; otherwise A is M x K.
template <int BM_, int BN_, int WM_, int WN_, int BK_, int STAGES_, bool BNK_ = false,
          bool AKM_ = false>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, BK = BK_;
  static constexpr int kStages = STAGES_;
  static constexpr bool kBNK = BNK_;
  static constexpr bool kAKM = AKM_;
  static constexpr int kWaves = WM * WN, kThreads = 64 * kWaves;
  static constexpr int kRowA = kAKM ? BM * 2 : BK * 2;  // bytes per LDS row of A
  static constexpr int kChunksA = kRowA / 16;         // 16-byte chunks per row of A
  static constexpr int kRowB = kBNK ? BK * 2 : BN * 2;  // bytes per LDS row of B
  static constexpr int kChunksB = kRowB / 16;
  static constexpr int kStageA = BM * BK * 2;
  static constexpr int kStageB = BK * BN * 2;
  static constexpr int kStage = kStageA + kStageB;
  static constexpr int kLdsBytes = kStages * kStage;
  static constexpr int kWaveM = BM / WM, kWaveN = BN / WN;
  static constexpr int kFragM = kWaveM / 16, kFragN = kWaveN / 16;  // 16 x 16 MFMA tiles
  static constexpr int kCopyA = kStageA / 1024 / kWaves;  // copies per wave and step
  static constexpr int kCopyB = kStageB / 1024 / kWaves;
  static constexpr int kCopies = kCopyA + kCopyB;
  static constexpr int kRowsPerCopyA = 1024 / kRowA;
  static constexpr int kRowsPerCopyB = 1024 / kRowB;
  static constexpr int kSub = BK / 32;                // MFMA k-steps per K step
  // LDS read instructions per sub-step (a transposing fragment read takes two)
  static constexpr int kReads = (kAKM ? 2 : 1) * kFragM + (kBNK ? 1 : 2) * kFragN;
  static constexpr int kMfmas = kFragM * kFragN;      // MFMAs per sub-step
  static_assert(kCopyA * kWaves * 1024 == kStageA && kCopyB * kWaves * 1024 == kStageB,
                "each wave copies whole 1 KB blocks");
  static_assert(kStageA % (16 * kThreads) == 0 && kStageB % (16 * kThreads) == 0,
                "masked copy: whole 16-byte chunks per lane");
  static_assert(kAKM || kChunksA == 4 || kChunksA == 8, "swizzle of A rows");
  static_assert(!kAKM || kChunksA >= 16, "k-major A rows take the swizzle of B's");
  static_assert(!kBNK || kChunksB == BK / 8, "N x K rows of B like A's");
  static_assert(kStages >= 2 && (kStages - 2) * kCopies <= 63, "vmcnt range");
  static_assert(kLdsBytes <= 160 * 1024, "LDS per workgroup");
};

// Row m of A, chunk c (8 k values) is stored at chunk c ^ swz_a(m). A
// fragment read takes 16 rows x 4 chunks (lane l: row l%16, chunk l/16);
// with 64-byte rows a probe counting SQ_LDS_BANK_CONFLICT found this pattern
// conflict-free with the swizzle on row bits 1-2, and twice the cycles with
// it on bits 2-3 (right for a 32-row x 2-chunk pattern) or on bits 0-1.
template <int kChunks>
__device__ __forceinline__ int swz_a(int m) {
  if constexpr (kChunks == 8)
    return (m ^ (m >> 3)) & 7;
  else
    return (m >> 1) & 3;
}
// Row k of a k-major tile (B stored K x N, or A stored K x M), chunk c at
// c ^ swz_b(k). A transposing read serves 16 lanes (128 bytes) at a time;
// each 16-lane group touches 16 columns (two chunks) of rows k..k+3, which
// bits 0-1 of k place in four different chunk pairs of one 128-byte bank
// window. The groups reading rows k and k+8 differ in bit 3, which moves
// the second to the other half of a 256-byte window. (Without the bit-1
// term, rows k and k+2 shared banks: 40% of the LDS cycles were conflicts.)
__device__ __forceinline__ int swz_b(int k) {
  return ((k & 3) << 2) ^ (((k >> 1) & 1) << 1) ^ (((k >> 3) & 1) << 3);
}

// Per-lane byte offsets of this wave's copy instructions; the K step only
// moves the scalar base pointers.
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
  for (int j = 0; j < T::kCopyA; ++j) {  // A: blocks of kRowsPerCopyA rows
    const int row = (wave * T::kCopyA + j) * T::kRowsPerCopyA + lane / T::kChunksA;
    if constexpr (T::kAKM) {  // row = k of the step, chunk c = 8 rows m of A
      const int c = (lane % T::kChunksA) ^ swz_b(row);
      const int gm = min(m0 + c * 8, M - 8);
      p.a[j] = static_cast<uint32_t>((static_cast<int64_t>(row) * M + gm) * 2);
    } else {
      const int c = (lane % T::kChunksA) ^ swz_a<T::kChunksA>(row);
      const int gm = min(m0 + row, M - 1);
      p.a[j] = static_cast<uint32_t>((static_cast<int64_t>(gm) * K + c * 8) * 2);
    }
  }
#pragma unroll
  for (int j = 0; j < T::kCopyB; ++j) {  // B: blocks of kRowsPerCopyB rows
    const int row = (wave * T::kCopyB + j) * T::kRowsPerCopyB + lane / T::kChunksB;
    if constexpr (T::kBNK) {  // row = column n of the tile, chunk c = 8 k
      const int c = (lane % T::kChunksB) ^ swz_a<T::kChunksB>(row);
      const int gn = min(n0 + row, N - 1);
      p.b[j] = static_cast<uint32_t>((static_cast<int64_t>(gn) * K + c * 8) * 2);
    } else {  // row = k of the step, chunk c = 8 columns
      const int c = (lane % T::kChunksB) ^ swz_b(row);
      const int gn = min(n0 + c * 8, N - 8);
      p.b[j] = static_cast<uint32_t>((static_cast<int64_t>(row) * N + gn) * 2);
    }
  }
  return p;
}

// --- global -> LDS copy of one full K step (clamped M/N) -----------------
template <class T>
__device__ __forceinline__ void copy_step_dma(const uint16_t* __restrict__ A,
                                              const uint16_t* __restrict__ B, int M, int N,
                                              int k0, int wave, const CopyPlan<T>& p,
                                              uint32_t stage) {
  const uint16_t* a_base = T::kAKM ? A + static_cast<int64_t>(k0) * M : A + k0;
  const uint16_t* b_base = T::kBNK ? B + k0 : B + static_cast<int64_t>(k0) * N;
#pragma unroll
  for (int j = 0; j < T::kCopyA; ++j)
    dma16(a_base, p.a[j], stage + (wave * T::kCopyA + j) * 1024);
#pragma unroll
  for (int j = 0; j < T::kCopyB; ++j)
    dma16(b_base, p.b[j], stage + T::kStageA + (wave * T::kCopyB + j) * 1024);
}

// Same layout, through registers, with zeros beyond K (the partial last step).
template <class T>
__device__ __forceinline__ void copy_step_masked(const uint16_t* __restrict__ A,
                                                 const uint16_t* __restrict__ B, int M, int N,
                                                 int K, int m0, int n0, int k0, int tid,
                                                 LDS_PTR(uint8_t) stage) {
  const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < T::kStageA / 16 / T::kThreads; ++i) {  // A chunks
    const int id = tid + T::kThreads * i;
    const int row = id / T::kChunksA, c = id % T::kChunksA;
    u32x4 v = zero;
    if constexpr (T::kAKM) {  // row = k, chunk c = 8 rows m
      const int gk = k0 + row;
      const int gm = min(m0 + c * 8, M - 8);
      if (gk < K) v = *reinterpret_cast<const u32x4*>(A + static_cast<int64_t>(gk) * M + gm);
      *(LDS_PTR(u32x4))(stage + row * T::kRowA + ((c ^ swz_b(row)) << 4)) = v;
    } else {
      const int gk = k0 + c * 8;
      const int gm = min(m0 + row, M - 1);
      if (gk < K) v = *reinterpret_cast<const u32x4*>(A + static_cast<int64_t>(gm) * K + gk);
      *(LDS_PTR(u32x4))(stage + row * T::kRowA + ((c ^ swz_a<T::kChunksA>(row)) << 4)) = v;
    }
  }
  LDS_PTR(uint8_t) sb = stage + T::kStageA;
#pragma unroll
  for (int i = 0; i < T::kStageB / 16 / T::kThreads; ++i) {  // B chunks
    const int id = tid + T::kThreads * i;
    const int row = id / T::kChunksB, c = id % T::kChunksB;
    u32x4 v = zero;
    if constexpr (T::kBNK) {
      const int gk = k0 + c * 8;
      const int gn = min(n0 + row, N - 1);
      if (gk < K) v = *reinterpret_cast<const u32x4*>(B + static_cast<int64_t>(gn) * K + gk);
      *(LDS_PTR(u32x4))(sb + row * T::kRowB + ((c ^ swz_a<T::kChunksB>(row)) << 4)) = v;
    } else {
      const int gk = k0 + row;
      const int gn = min(n0 + c * 8, N - 8);
      if (gk < K) v = *reinterpret_cast<const u32x4*>(B + static_cast<int64_t>(gk) * N + gn);
      *(LDS_PTR(u32x4))(sb + row * T::kRowB + ((c ^ swz_b(row)) << 4)) = v;
    }
  }
}

// From a k-major LDS tile (rows of kRow bytes, chunk c of row k at
// c ^ swz_b(k)): eight consecutive k (32s + 8*(lane/16) + 0..7) of column
// n_base + lane%16, with two transposing reads.
template <int kRow>
__device__ __forceinline__ bf16x8 read_kmajor(LDS_PTR(const uint8_t) base, int n_base, int s,
                                              int lane) {
  const int g = lane >> 4, i = lane & 15;
  const int col = n_base + 4 * (i & 3);
  const int c = col >> 3, half = (col & 7) << 1;
  const int r0 = 32 * s + 8 * g + (i >> 2);
  const int r1 = r0 + 4;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (LDS_PTR(s16x4))(base + r0 * kRow + ((c ^ swz_b(r0)) << 4) + half));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (LDS_PTR(s16x4))(base + r1 * kRow + ((c ^ swz_b(r1)) << 4) + half));
  const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
  const u32x4 v = {l2.x, l2.y, h2.x, h2.y};
  return __builtin_bit_cast(bf16x8, v);
}

// Eight consecutive k (32s + 8*(lane/16) + 0..7) of row m_base + lane%16 of A.
template <class T>
__device__ __forceinline__ bf16x8 read_a(LDS_PTR(const uint8_t) sa, int m_base, int s,
                                         int lane) {
  if constexpr (T::kAKM) return read_kmajor<T::kRowA>(sa, m_base, s, lane);
  const int row = m_base + (lane & 15), chunk = 4 * s + (lane >> 4);
  const u32x4 v = *(LDS_PTR(const u32x4))(sa + row * T::kRowA +
                                           ((chunk ^ swz_a<T::kChunksA>(row)) << 4));
  return __builtin_bit_cast(bf16x8, v);
}

// Eight consecutive k (32s + 8*(lane/16) + 0..7) of column n_base + lane%16.
template <class T>
__device__ __forceinline__ bf16x8 read_b(LDS_PTR(const uint8_t) sb, int n_base, int s,
                                         int lane) {
  if constexpr (T::kBNK) {  // a K-contiguous row per column: read as A
    const int row = n_base + (lane & 15), chunk = 4 * s + (lane >> 4);
    const u32x4 v = *(LDS_PTR(const u32x4))(sb + row * T::kRowB +
                                             ((chunk ^ swz_a<T::kChunksB>(row)) << 4));
    return __builtin_bit_cast(bf16x8, v);
  }
  return read_kmajor<T::kRowB>(sb, n_base, s, lane);
}

// Instruction order for the scheduler within one sub-step: one read of the
// next fragments after each MFMA, leftovers after.
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

// C receives the sums finished by `epi` (epilogue.h), in the epilogue's
// element type; an empty epilogue stores the fp32 sums themselves.
template <class T>
__global__ __launch_bounds__(T::kThreads, 1) void mfma_bf16_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, void* C, int M, int N,
    int K, int tiles_m, int tiles_n, Epilogue epi) {
  constexpr int S = T::kStages;
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[];
  LDS_PTR(uint8_t) lds = (LDS_PTR(uint8_t))lds_raw;

  int tm, tn;
  xcd_tile(blockIdx.x, tiles_m, tiles_n, kGroupM, tm, tn);
  const int m0 = tm * T::BM, n0 = tn * T::BN;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int lane = tid & 63;
  const int wm = wave / T::WN, wn = wave % T::WN;
  const int lr = lane & 15, lg = lane >> 4;
  const int row_a = wm * T::kWaveM;  // + 16 i: this wave's rows of A
  const int col_b = wn * T::kWaveN;  // + 16 j: this wave's columns of B

  f32x4 acc[T::kFragM][T::kFragN];
#pragma unroll
  for (int i = 0; i < T::kFragM; ++i)
#pragma unroll
    for (int j = 0; j < T::kFragN; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[i][j][v] = 0.f;

  const int steps = (K + T::BK - 1) / T::BK;
  const int full_steps = K / T::BK;  // steps whose BK k are all in range
  // Staggered start: the full steps run from step rot and wrap round (the
  // partial step stays last). Workgroups are dealt round-robin to the eight
  // XCDs, so blockIdx/8 numbers the workgroups of one XCD; sixteen
  // neighbours there start up to fifteen steps apart (4096^3 with B stored
  // N x K: 150 us with eight, 137 us with sixteen). Rows of A (and of an N x K B) lie
  // K*2 bytes apart, so with one common start every line a step fetches sits
  // at the same offset of its row and the requests crowd into a few L2
  // channels; a small stagger spreads them while workgroups that share
  // operand rows stay within a few steps of each other, which keeps their
  // reuse in L2 (a stagger over the whole K range loses it and is slower).
  // When every tile of a K x N product is resident at once (one round of
  // workgroups), a common start is faster (4096^3: 109.9 against 111.2 us);
  // N x K and K x M operands keep the stagger.
  const bool stagger = T::kBNK || T::kAKM || gridDim.x > static_cast<unsigned>(kCUs);
  const int rot = stagger && full_steps > 0
                      ? static_cast<int>(((blockIdx.x >> 3) & 15u) % static_cast<unsigned>(full_steps))
                      : 0;
  const CopyPlan<T> plan = make_plan<T>(M, N, K, m0, n0, wave, lane);
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_offset(lds));

  // Copy the K step taken at position `st` of the loop into ring slot
  // `slot`: asynchronously when all its k are in range, else through
  // registers.
  auto issue = [&](int st, int slot) {
    if (st < full_steps) {
      int ks = st + rot;
      if (ks >= full_steps) ks -= full_steps;
      copy_step_dma<T>(A, B, M, N, ks * T::BK, wave, plan, lds0 + slot * T::kStage);
    } else if (st < steps) {
      copy_step_masked<T>(A, B, M, N, K, m0, n0, st * T::BK, tid, lds + slot * T::kStage);
    }
  };
  // Before reading step `next`: its copies, and all earlier ones, have landed.
  // The S-2 later steps may still be in flight when all of them are
  // asynchronous copies.
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

  // Ping-pong between the two halves of the workgroup (waves 0-3 and 4-7;
  // wave w runs on SIMD w % 4, so each SIMD holds one wave of each). Every K
  // step takes two phases separated by workgroup barriers: in one, a group
  // issues its share of the copies and reads all of the step's fragments
  // from LDS into registers; in the next, it runs the step's MFMAs while the
  // other group does its reads. The matrix core of a SIMD is then fed by one
  // wave whose operands are already in registers, and LDS reads never stall
  // its issue. Step t's slot is read in phases 2t (group 0) and 2t+1 (group
  // 1) and refilled from phase 2t+2 on, so its copies still have S-1 steps
  // to land. Measured on 8192^3 and 4096^3 (the same sums, bit for bit):
  // 844 / 111.8 us against 869 / 115.2 us for the interleaved loop below,
  // which remains for a partial last step and for two-slot rings.
  constexpr bool kPingPong = T::WM == 2 && T::WN == 4 && T::kSub == 1 && S >= 3;
  if (kPingPong && steps == full_steps) {
    if constexpr (kPingPong) {
      const int group = wave >> 2;
      bf16x8 fa[T::kSub][T::kFragM], fb[T::kSub][T::kFragN];
      auto load_frags = [&](int slot) __attribute__((always_inline)) {
        LDS_PTR(const uint8_t) pa = lds + slot * T::kStage;
        LDS_PTR(const uint8_t) pb = pa + T::kStageA;
#pragma unroll
        for (int s = 0; s < T::kSub; ++s) {
#pragma unroll
          for (int i = 0; i < T::kFragM; ++i) fa[s][i] = read_a<T>(pa, row_a + 16 * i, s, lane);
#pragma unroll
          for (int j = 0; j < T::kFragN; ++j) fb[s][j] = read_b<T>(pb, col_b + 16 * j, s, lane);
        }
      };
      auto multiply = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < T::kSub; ++s)
#pragma unroll
          for (int i = 0; i < T::kFragM; ++i)
#pragma unroll
            for (int j = 0; j < T::kFragN; ++j)
              acc[i][j] =
                  __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[s][i], fb[s][j], acc[i][j], 0, 0, 0);
      };
      // A workgroup barrier the scheduler moves nothing across (it had
      // hoisted an MFMA of the next phase above it).
      auto phase_end = []() __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
      };
      // Both groups pass 2*steps barriers here, then meet again at the
      // first barrier of the store.
      if (group == 0) {
        for (int t = 0; t < steps; ++t) {
          issue(t + S - 1, (t + S - 1) % S);  // into the slot step t-1 used
          load_frags(t % S);
          phase_end();  // phase 2t: reads
          multiply();
          wait_step(t + 1);
          phase_end();  // phase 2t+1: MFMAs
        }
      } else {
        phase_end();  // phase 0: group 0's first reads
        for (int t = 0; t < steps; ++t) {
          issue(t + S - 1, (t + S - 1) % S);
          load_frags(t % S);
          wait_step(t + 1);
          phase_end();  // phase 2t+1: reads
          multiply();   // phase 2t+2: MFMAs
          if (t + 1 < steps) phase_end();
        }
      }
    }
  } else {
    bf16x8 a[2][T::kFragM], b[2][T::kFragN];
#pragma unroll
    for (int i = 0; i < T::kFragM; ++i) a[0][i] = read_a<T>(lds, row_a + 16 * i, 0, lane);
#pragma unroll
    for (int j = 0; j < T::kFragN; ++j)
      b[0][j] = read_b<T>(lds + T::kStageA, col_b + 16 * j, 0, lane);

    int cur = 0;  // ring slot of step t
    for (int t = 0; t < steps; ++t) {
      const int nxt = cur + 1 == S ? 0 : cur + 1;
      issue(t + S - 1, cur == 0 ? S - 1 : cur - 1);  // the slot step t-1 used
      LDS_PTR(const uint8_t) sa = lds + cur * T::kStage;
      LDS_PTR(const uint8_t) sb = sa + T::kStageA;
#pragma unroll
      for (int s = 0; s < T::kSub; ++s) {
        const int c = s & 1, n = c ^ 1;
        if (s + 1 < T::kSub) {
#pragma unroll
          for (int i = 0; i < T::kFragM; ++i) a[n][i] = read_a<T>(sa, row_a + 16 * i, s + 1, lane);
#pragma unroll
          for (int j = 0; j < T::kFragN; ++j) b[n][j] = read_b<T>(sb, col_b + 16 * j, s + 1, lane);
        } else {
          // Step t+1's copies land and every wave is done with the slot the
          // next issue overwrites; then its first fragments are read while the
          // last MFMAs of step t run. After the last step these reads fetch
          // stale values that are never used.
          wait_step(t + 1);
          __syncthreads();
          LDS_PTR(const uint8_t) na = lds + nxt * T::kStage;
#pragma unroll
          for (int i = 0; i < T::kFragM; ++i) a[n][i] = read_a<T>(na, row_a + 16 * i, 0, lane);
#pragma unroll
          for (int j = 0; j < T::kFragN; ++j)
            b[n][j] = read_b<T>(na + T::kStageA, col_b + 16 * j, 0, lane);
        }
#pragma unroll
        for (int i = 0; i < T::kFragM; ++i)
#pragma unroll
          for (int j = 0; j < T::kFragN; ++j)
            acc[i][j] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[c][i], b[c][j], acc[i][j], 0, 0, 0);
        interleave_hint<T>();
      }
      if constexpr (T::kSub % 2 == 1) {  // the next step's fragments are in buffer 1
#pragma unroll
        for (int i = 0; i < T::kFragM; ++i) a[0][i] = a[1][i];
#pragma unroll
        for (int j = 0; j < T::kFragN; ++j) b[0][j] = b[1][j];
      }
      cur = nxt;
    }
  }

  // Writing C. Each wave stages its block through its share of the (now
  // idle) LDS ring, kPassRows rows at a time, then finishes the outputs in
  // row-contiguous groups of four: one compact loop for the epilogue instead
  // of one inlined per accumulator, coalesced residual reads, and 8- or
  // 16-byte stores (measured faster than storing from the accumulators'
  // layout even with no epilogue). Element v of a 16 x 16 accumulator sits
  // at row 4*(lane/16) + v, column lane%16. Staged rows are padded by four
  // floats, so the four rows (4 apart) one store instruction writes fall in
  // different banks.
  {
    constexpr int kWaveLds = T::kLdsBytes / T::kWaves;
    constexpr int kStride = T::kWaveN + 4;                 // floats per staged row
    constexpr int kFit = kWaveLds / (16 * kStride * 4);   // 16-row fragments per pass
    constexpr int kPassFrags = kFit >= T::kFragM ? T::kFragM : kFit >= 4 ? 4 : kFit >= 2 ? 2 : 1;
    static_assert(kFit >= 1 && T::kFragM % kPassFrags == 0, "epilogue staging");
    constexpr int kPassRows = 16 * kPassFrags;
    constexpr int kLanesPerRow = T::kWaveN / 4;
    constexpr int kRowsPerIter = 64 / kLanesPerRow;
    LDS_PTR(float) stage = (LDS_PTR(float))(lds + wave * kWaveLds);
    const int c4 = (lane % kLanesPerRow) * 4;
    const int col = n0 + wn * T::kWaveN + c4;
    const f32x4 bias4 = epi_bias4(col, N, epi);  // this lane's columns never change
    __syncthreads();  // every wave is done with the ring
#pragma unroll
    for (int i0 = 0; i0 < T::kFragM; i0 += kPassFrags) {
#pragma unroll
      for (int i = 0; i < kPassFrags; ++i)
#pragma unroll
        for (int j = 0; j < T::kFragN; ++j)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            stage[(i * 16 + lg * 4 + v) * kStride + j * 16 + lr] = acc[i0 + i][j][v];
      __syncthreads();
#pragma unroll 4
      for (int r = lane / kLanesPerRow; r < kPassRows; r += kRowsPerIter) {
        const f32x4 t = *(LDS_PTR(const f32x4))(stage + r * kStride + c4);
        const int row = m0 + wm * T::kWaveM + i0 * 16 + r;
        if (row < M && col < N)
          epi_store4(C, static_cast<int64_t>(row) * N + col, col, N, t, bias4, epi);
      }
      __syncthreads();
    }
  }
}

template <class T>
hipError_t launch_tile(const uint16_t* A, const uint16_t* B, void* C, int M, int N, int K,
                       const Epilogue& epi, hipStream_t s) {
  static std::atomic<uint64_t> lds_ok{0};  // devices already opted in
  hipError_t e =
      allow_lds(lds_ok, reinterpret_cast<const void*>(mfma_bf16_kernel<T>), T::kLdsBytes);
  if (e != hipSuccess) return e;
  const int tiles_m = (M + T::BM - 1) / T::BM;
  const int tiles_n = (N + T::BN - 1) / T::BN;
  return launch(mfma_bf16_kernel<T>, dim3(tiles_m * tiles_n), dim3(T::kThreads), T::kLdsBytes,
                s, A, B, C, M, N, K, tiles_m, tiles_n, epi);
}

}  // namespace

bool mfma_bf16_supports(int64_t M, int64_t N, int64_t K, int mis_a, int mis_b,
                        int mis_c) {
  (void)M;
  (void)mis_c;
  // 32-bit per-lane copy offsets: 130 rows of B stay below 4 GiB.
  return K % 8 == 0 && N % 8 == 0 && K >= 8 && N <= (1 << 24) && mis_a == 0 &&
         mis_b == 0;
}

bool mfma_bf16_akm_supports(int64_t M, int64_t N, int64_t K, bool b_nk, int mis_a, int mis_b,
                            int mis_c) {
  (void)mis_c;
  // A stored K x M: 16-byte chunks along M, and 32-bit per-lane copy
  // offsets (a step's rows of A and of a K x N B stay below 4 GiB).
  if (M % 8 != 0 || M > (1 << 24) || K % 8 != 0 || K < 8 || mis_a != 0 || mis_b != 0)
    return false;
  return b_nk || (N % 8 == 0 && N <= (1 << 24));
}

bool mfma_bf16_nk_supports(int64_t M, int64_t N, int64_t K, int mis_a, int mis_b,
                           int mis_c) {
  (void)M;
  (void)N;  // columns are rows of B: any count, clamped like the rows of A
  (void)mis_c;
  // Offsets gn*K*2 stay below 4 GiB because B has fewer than 2^31 elements.
  return K % 8 == 0 && K >= 8 && mis_a == 0 && mis_b == 0;
}

// 32 k per step over four slots (the ping-pong schedule) for every layout.
// For an N x K B this replaced 64 k per step over two slots, whose 128-byte
// row pieces of both operands (one cache line each) had been 2-9% faster in
// the interleaved loop (8192^3: 899.6 against 926.5 us with the ping-pong;
// 4096^3 115.7 against 114.1).
template <bool BNK, bool AKM>
using LargeTile = Cfg<256, 256, 2, 4, 32, 4, BNK, AKM>;
template <bool BNK, bool AKM>
using SmallTile = Cfg<128, 128, 2, 4, 32, 4, BNK, AKM>;

hipError_t launch_mfma_bf16(const uint16_t* A, const uint16_t* B, float* C,
                            int M, int N, int K, hipStream_t s) {
  // The plain product goes through the staged store too, with no epilogue
  // terms: its row-contiguous 16-byte stores write C faster than the
  // accumulators' own layout does.
  return launch_mfma_bf16_epi(A, B, false, false, C, M, N, K, Epilogue{}, s);
}

template <bool BNK, bool AKM>
hipError_t launch_layout(const uint16_t* A, const uint16_t* B, void* D, int M, int N, int K,
                         const Epilogue& e, hipStream_t s) {
  return use_large_tiles(M, N, kLargeTileFillBf16)
             ? launch_tile<LargeTile<BNK, AKM>>(A, B, D, M, N, K, e, s)
             : launch_tile<SmallTile<BNK, AKM>>(A, B, D, M, N, K, e, s);
}

hipError_t launch_mfma_bf16_epi(const uint16_t* A, const uint16_t* B, bool b_nk, bool a_km,
                                void* D, int M, int N, int K, const Epilogue& e, hipStream_t s) {
  if (a_km)
    return b_nk ? launch_layout<true, true>(A, B, D, M, N, K, e, s)
                : launch_layout<false, true>(A, B, D, M, N, K, e, s);
  return b_nk ? launch_layout<true, false>(A, B, D, M, N, K, e, s)
              : launch_layout<false, false>(A, B, D, M, N, K, e, s);
}

}  // namespace tdm

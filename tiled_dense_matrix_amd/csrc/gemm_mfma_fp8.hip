// FP8 product on the gfx950 matrix cores, with optional per-block scales.
//
// What is computed (CS336 Lecture 5 GPU notes, §3.1: the two 8-bit formats,
// E4M3 with 4 exponent and 3 mantissa bits, range +-448, and E5M2 with 5 and
// 2, range +-57344; FP8 training needs fine-grained per-tile scaling; every
// halving of the element width doubles the peak):
//   C[i,j] = sum_k (sa[i,k/32] A[i,k]) (sb[j,k/32] B[j,k])
// for A (M x K) and B (N x K, the layout of a linear layer's weight) stored
// as FP8 codes, each operand E4M3 or E5M2, and the scales one power of two
// 2^(e-127) per 32 consecutive k of each row, stored as the 8-bit exponent e
// (OCP Microscaling block scales); without scales every factor is 1. The
// sum is taken in fp32 and finished by the fused epilogue (epilogue.h).
//
// Method -- the tiling of the bf16 kernel (gemm_mfma_bf16.hip), re-cut for
// one-byte elements:
//   * one workgroup owns a 256 x 256 tile of C (128 x 128 when the large
//     tiles cannot fill the CUs); eight waves (2 x 4) each hold a
//     (BM/2) x (BN/4) block as 32 x 32 fp32 accumulators;
//   * K advances 128 per step: each step copies a BM x 128 slice of A and a
//     BN x 128 slice of B (one 128-byte cache line per row, since both
//     operands are K-contiguous) from HBM into LDS with global_load_lds,
//     double-buffered, from a start staggered between neighbouring
//     workgroups as in the bf16 kernel;
//   * v_mfma_scale_f32_32x32x64_f8f6f4 multiplies 32 x 64 by 64 x 32. Lane l
//     holds row l%32 of the A fragment and row (= column of C) l%32 of the B
//     fragment: in bytes 0-15 the k 16*(l/32) + 0..15 and in bytes 16-31 the
//     k 32 + 16*(l/32) + 0..15 of the 64 (two 16-byte LDS reads each), and,
//     with scales, the exponent of 32-k block l/32 of its row of A and of B.
//     Block 0 (k 0..31) is thus bytes 0-15 of lanes r and r+32, block 1
//     bytes 16-31 of both; the instruction applies both scales itself (this
//     grouping was measured: with 2^1 in lanes 0-31 and 2^2 in lanes 32-63, a
//     single nonzero input in bytes 0-15 of either lane came out doubled,
//     one in bytes 16-31 quadrupled). The unscaled form is the same
//     instruction without scales;
//   * with scales, each step also copies the tile's scale words -- for every
//     row of A and of B the four exponents of the step's 128 k, one 4-byte
//     word -- into LDS beside the data (global_load_lds_dword, one 64-row
//     copy per wave), and each lane reads the words of its rows there.
// LDS rows are 128 bytes; chunk c (16 bytes) of row m sits at chunk
// c ^ ((m >> 1) & 7). The 16 consecutive rows of one read phase then cover
// all 64 banks (two rows share a 256-byte bank window, and each pair takes
// another chunk), and the swizzle is the same for rows 16 apart, so one
// per-lane offset serves every fragment and both operands.
//
// Partial tiles in M or N load clamped rows whose products only reach outputs
// that are not stored. K is a multiple of 32 (one scale block); a K that is
// not a multiple of 128 loads its partial step (taken first) through
// registers, zeros beyond K, and its missing scale blocks as 2^0.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lds_copy.h"
#include "tdm_internal.h"
#include "tile_map.h"

namespace tdm {
namespace {

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kGroupM = 8;
constexpr int kSpanK = 128;        // k covered by one 4-byte scale word (four blocks)
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

// BK: k (= bytes) per step and LDS row, 64 or 128; STAGES: ring slots.
template <int BM_, int BN_, int WM_, int WN_, int BK_, int STAGES_>
struct Fp8Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, BK = BK_;
  static constexpr int kStages = STAGES_;
  static constexpr int kChunks = BK / 16;  // 16-byte chunks per row
  static constexpr int kWaves = WM * WN, kThreads = 64 * kWaves;
  static constexpr int kStageA = BM * BK, kStageB = BN * BK;
  static constexpr int kScaleOff = kStageA + kStageB;  // scale words: A rows, then B rows
  static constexpr int kStage = kScaleOff + 4 * (BM + BN);
  static constexpr int kScaleCopies = (BM + BN) / 64;  // 64 words per copy
  static constexpr int kScaleCopiesPerWave = (kScaleCopies + kWaves - 1) / kWaves;
  static constexpr int kLdsBytes = kStages * kStage;
  static constexpr int kWaveM = BM / WM, kWaveN = BN / WN;
  static constexpr int kFragM = kWaveM / 32, kFragN = kWaveN / 32;
  static constexpr int kCopyA = kStageA / 1024 / kWaves;  // 1 KB copies per wave and step
  static constexpr int kCopyB = kStageB / 1024 / kWaves;
  static constexpr int kCopies = kCopyA + kCopyB;         // (every wave; scale copies extra)
  static constexpr int kRowsPerCopy = 1024 / BK;
  static constexpr int kSub = BK / 64;  // MFMA k-steps per step
  static constexpr int kReads = 2 * (kFragM + kFragN);  // 16-byte LDS reads per sub-step
  static constexpr int kMfmas = kFragM * kFragN;
  static_assert(kChunks == 4 || kChunks == 8, "64- or 128-byte rows");
  static_assert(kCopyA * kWaves * 1024 == kStageA && kCopyB * kWaves * 1024 == kStageB,
                "whole 1 KB copies per wave");
  static_assert(kStageA % (16 * kThreads) == 0 && kStageB % (16 * kThreads) == 0,
                "masked copy: whole 16-byte chunks per lane");
  static_assert(BM % 64 == 0 && BN % 64 == 0, "whole 64-row scale copies");
  static_assert(kStages >= 2 && (kStages - 2) * (kCopies + kScaleCopiesPerWave) <= 63,
                "vmcnt range");
  static_assert(kLdsBytes <= 160 * 1024, "LDS per workgroup");
};

// 128 k per step, double-buffered: whole 128-byte lines per row. (64 k with
// four slots, three steps of copies in flight, measured 15% slower on
// 8192 x 14336 x 4096: the half-line row pieces double the L2 requests per
// byte, and the copies were not waiting on latency.)
using LargeTile = Fp8Cfg<256, 256, 2, 4, 128, 2>;
using SmallTile = Fp8Cfg<128, 128, 2, 4, 128, 2>;

// Chunk c of row m sits at chunk c ^ swz(m). 128-byte rows: two rows share
// a 256-byte bank window, rows that differ in bits 1-3 take different
// chunks; 64-byte rows: four rows share it, bits 2-3 decide. Either way the
// 16 rows one read phase touches cover all 64 banks, and the swizzle is the
// same for rows 16 apart.
template <int kChunks>
__device__ __forceinline__ int swz(int m) {
  if constexpr (kChunks == 8)
    return (m >> 1) & 7;
  else
    return (m >> 2) & 3;
}

// Per-lane byte offsets of this wave's copies from A + k0 and B + k0: copy q
// fills LDS bytes [1024q, 1024q + 1024) of its operand's stage with rows
// 8q..8q+7; lane L takes row 8q + L/8, LDS chunk L%8, which holds global
// chunk (L%8) ^ swz(row).
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
  for (int j = 0; j < T::kCopyA; ++j) {
    const int row = (wave * T::kCopyA + j) * T::kRowsPerCopy + lane / T::kChunks;
    const int c = (lane % T::kChunks) ^ swz<T::kChunks>(row);
    p.a[j] = static_cast<uint32_t>(static_cast<int64_t>(min(m0 + row, M - 1)) * K + 16 * c);
  }
#pragma unroll
  for (int j = 0; j < T::kCopyB; ++j) {
    const int row = (wave * T::kCopyB + j) * T::kRowsPerCopy + lane / T::kChunks;
    const int c = (lane % T::kChunks) ^ swz<T::kChunks>(row);
    p.b[j] = static_cast<uint32_t>(static_cast<int64_t>(min(n0 + row, N - 1)) * K + 16 * c);
  }
  return p;
}

template <class T>
__device__ __forceinline__ void copy_step_dma(const uint8_t* __restrict__ A,
                                              const uint8_t* __restrict__ B, int k0, int wave,
                                              const CopyPlan<T>& p, uint32_t stage) {
#pragma unroll
  for (int j = 0; j < T::kCopyA; ++j)
    dma16(A + k0, p.a[j], stage + (wave * T::kCopyA + j) * 1024);
#pragma unroll
  for (int j = 0; j < T::kCopyB; ++j)
    dma16(B + k0, p.b[j], stage + T::kStageA + (wave * T::kCopyB + j) * 1024);
}

// The partial last step through registers: chunks at or beyond K are zero.
template <class T>
__device__ __forceinline__ void copy_step_masked(const uint8_t* __restrict__ A,
                                                 const uint8_t* __restrict__ B, int M, int N,
                                                 int K, int m0, int n0, int k0, int tid,
                                                 LDS_PTR(uint8_t) stage) {
  const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < (T::kStageA + T::kStageB) / 16 / T::kThreads; ++i) {
    const int id = tid + T::kThreads * i;
    const int row = id / T::kChunks, c = id % T::kChunks;  // rows of A, then rows of B
    const int gk = k0 + 16 * c;
    u32x4 v = zero;
    if (row < T::BM) {
      if (gk < K)
        v = *reinterpret_cast<const u32x4*>(A + static_cast<int64_t>(min(m0 + row, M - 1)) * K + gk);
    } else if (gk < K) {
      v = *reinterpret_cast<const u32x4*>(
          B + static_cast<int64_t>(min(n0 + row - T::BM, N - 1)) * K + gk);
    }
    *(LDS_PTR(u32x4))(stage + row * T::BK + ((c ^ swz<T::kChunks>(row)) << 4)) = v;
  }
}

// Byte offset, from the first row of a 32-row fragment, of the 16-byte
// chunk the lane feeds to byte 16x..16x+15 of its operand in sub-step s:
// k 64s + 32x + 16*lg + 0..15 of the fragment's row lr, i.e. chunk
// 4s + 2x + lg. Every fragment starts at a multiple of 16 rows, so the
// swizzle only sees lr.
template <class T>
__device__ __forceinline__ int frag_off(int lr, int lg, int s, int x) {
  return lr * T::BK + (((4 * s + 2 * x + lg) ^ swz<T::kChunks>(lr)) << 4);
}

// The lane's 32 k of a fragment starting at `frag` (off0/off1: frag_off for
// x = 0 and 1).
__device__ __forceinline__ i32x8 read_frag(LDS_PTR(const uint8_t) frag, int off0, int off1) {
  const u32x4 lo = *(LDS_PTR(const u32x4))(frag + off0);
  const u32x4 hi = *(LDS_PTR(const u32x4))(frag + off1);
  return i32x8{static_cast<int32_t>(lo.x), static_cast<int32_t>(lo.y),
               static_cast<int32_t>(lo.z), static_cast<int32_t>(lo.w),
               static_cast<int32_t>(hi.x), static_cast<int32_t>(hi.y),
               static_cast<int32_t>(hi.z), static_cast<int32_t>(hi.w)};
}

// Exponents of the four scale blocks kb0 .. kb0 + 3 (128 k) of one row,
// byte q = block kb0 + q; blocks beyond K read as 127 (2^0).
__device__ __forceinline__ uint32_t scale_word(const uint8_t* __restrict__ row_scales, int kb0,
                                               int nkb, bool dword_ok) {
  if (dword_ok && kb0 + 4 <= nkb)
    return *reinterpret_cast<const uint32_t*>(row_scales + kb0);
  uint32_t w = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    w |= (kb0 + q < nkb ? static_cast<uint32_t>(row_scales[kb0 + q]) : 127u) << (8 * q);
  return w;
}

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

// FA, FB: formats of A and B (0 = E4M3, 1 = E5M2, the instruction's codes).
// SA, SB: scale exponents [M][K/32] and [N][K/32] (kScaled only); scale_dw:
// rows of scales may be read as aligned 32-bit words.
template <class T, int FA, int FB, bool kScaled>
__global__ __launch_bounds__(T::kThreads, 1) void mfma_fp8_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ SA, const uint8_t* __restrict__ SB, int scale_dw, void* C, int M,
    int N, int K, int tiles_m, int tiles_n, Epilogue epi) {
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
  const int row_a = wm * T::kWaveM + lr;            // + 32 i: this lane's rows of A (in the tile)
  const int row_b = T::BM + wn * T::kWaveN + lr;    // + 32 j: its rows of B, after A's in LDS
  // LDS offsets of the wave's first A and B fragment rows (uniform) and the
  // lane's chunk offsets for sub-steps 0 and 1.
  const int frag_a0 = wm * T::kWaveM * T::BK, frag_b0 = (T::BM + wn * T::kWaveN) * T::BK;
  int offs[T::kSub][2];
#pragma unroll
  for (int s = 0; s < T::kSub; ++s)
#pragma unroll
    for (int x = 0; x < 2; ++x) offs[s][x] = frag_off<T>(lr, lg, s, x);
  auto frag_a = [&](LDS_PTR(const uint8_t) slot, int i, int s) {
    return read_frag(slot + frag_a0 + 32 * i * T::BK, offs[s][0], offs[s][1]);
  };
  auto frag_b = [&](LDS_PTR(const uint8_t) slot, int j, int s) {
    return read_frag(slot + frag_b0 + 32 * j * T::BK, offs[s][0], offs[s][1]);
  };

  f32x16 acc[T::kFragM][T::kFragN];
#pragma unroll
  for (int i = 0; i < T::kFragM; ++i)
#pragma unroll
    for (int j = 0; j < T::kFragN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // Order of the K steps: a partial step (K not a multiple of BK) comes
  // first, in the prologue, so the masked register copy stays out of the
  // loop; then the full steps from a staggered start, wrapping round. As in
  // the bf16 kernel, rows lie K bytes apart and a common start sends a
  // step's lines to a few L2 channels; here 16 neighbours on one XCD begin
  // up to 15 steps apart (8192 x 14336 x 4096: 0.574 ms with no stagger,
  // 0.551 ms over 8 steps, 0.542 ms over 16, 0.560 ms over 32).
  const int steps = (K + T::BK - 1) / T::BK;
  const int full_steps = K / T::BK;
  const int partial = steps - full_steps;  // 0 or 1
  const int rot = full_steps > 0
                      ? static_cast<int>(((blockIdx.x >> 3) & 15u) % static_cast<unsigned>(full_steps))
                      : 0;
  auto step_k0 = [&](int st) {  // k0 of the step at loop position st
    if (st < partial) return full_steps * T::BK;
    int ks = st - partial + rot;
    if (ks >= full_steps) ks -= full_steps;
    return ks * T::BK;
  };
  const CopyPlan<T> plan = make_plan<T>(M, N, K, m0, n0, wave, lane);
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_offset(lds));

  // Scale words. Copy q (by wave q % kWaves) moves rows 64q..64q+63 of the
  // tile's scale rows (A's BM rows, then B's BN rows); in the register path
  // thread t assembles rows t, t + kThreads, ...
  const int nkb = K / 32;
  uint32_t sc_off[T::kScaleCopiesPerWave];
  if constexpr (kScaled) {
#pragma unroll
    for (int j = 0; j < T::kScaleCopiesPerWave; ++j) {
      const int q = wave + T::kWaves * j;
      const bool of_b = q * 64 >= T::BM;
      const int r = q * 64 + lane - (of_b ? T::BM : 0);
      sc_off[j] = static_cast<uint32_t>(of_b ? min(n0 + r, N - 1) : min(m0 + r, M - 1)) *
                  static_cast<uint32_t>(nkb);
    }
  }

  // Copy the step at loop position st into ring slot `slot`; `masked`: it
  // is the partial step.
  auto issue = [&](int st, int slot, bool masked) {
    if (st >= steps) return;
    if (!masked)
      copy_step_dma<T>(A, B, step_k0(st), wave, plan, lds0 + slot * T::kStage);
    else
      copy_step_masked<T>(A, B, M, N, K, m0, n0, step_k0(st), tid, lds + slot * T::kStage);
    if constexpr (kScaled) {
      // The word of the 128-k span the step lies in (a 64-k step uses half).
      const int kb0 = step_k0(st) / kSpanK * 4;
      if (scale_dw != 0 && !masked) {
#pragma unroll
        for (int j = 0; j < T::kScaleCopiesPerWave; ++j) {
          const int q = wave + T::kWaves * j;  // wave-uniform
          if (q < T::kScaleCopies)
            dma4((q * 64 >= T::BM ? SB : SA) + kb0, sc_off[j],
                 lds0 + slot * T::kStage + T::kScaleOff + q * 256);
        }
      } else {
        for (int t = tid; t < T::BM + T::BN; t += T::kThreads) {
          const uint8_t* row = t < T::BM
              ? SA + static_cast<int64_t>(min(m0 + t, M - 1)) * nkb
              : SB + static_cast<int64_t>(min(n0 + t - T::BM, N - 1)) * nkb;
          *(LDS_PTR(uint32_t))(lds + slot * T::kStage + T::kScaleOff + 4 * t) =
              scale_word(row, kb0, nkb, scale_dw != 0);
        }
      }
    }
  };
  // This lane's scale words of one step (rows row_a + 32i and row_b + 32j).
  uint32_t sa_w[T::kFragM], sb_w[T::kFragN];
  auto read_scales = [&](int slot) {
    if constexpr (kScaled) {
      LDS_PTR(const uint32_t) w = (LDS_PTR(const uint32_t))(lds + slot * T::kStage + T::kScaleOff);
#pragma unroll
      for (int i = 0; i < T::kFragM; ++i) sa_w[i] = w[row_a + 32 * i];
#pragma unroll
      for (int j = 0; j < T::kFragN; ++j) sb_w[j] = w[row_b + 32 * j];
    }
  };

  // Before reading the step at position `next`: its copies, and all earlier
  // ones, have landed. Copies complete in issue order; the S-2 later steps
  // may still be in flight when they have all been issued (a wave with
  // scale copies has more in flight than counted, which only waits longer).
  constexpr int S = T::kStages;
  auto wait_step = [&](int next) {
    if (S > 2 && next + S - 2 < steps)
      wait_vm<(S > 2 ? (S - 2) * T::kCopies : 0)>();
    else
      wait_vm<0>();
  };

#pragma unroll
  for (int st = 0; st < S - 1; ++st) issue(st, st, st < partial);
  wait_step(0);
  __syncthreads();

  // Fragments of the next sub-step are read while the current one is
  // multiplied. B's are double-buffered; each A fragment is reloaded into
  // its own registers right after its last MFMA of the sub-step has read
  // them (an A fragment takes 8 VGPRs: double-buffering both would not fit
  // next to the 128 accumulator registers).
  i32x8 a[T::kFragM], b[2][T::kFragN];
#pragma unroll
  for (int i = 0; i < T::kFragM; ++i) a[i] = frag_a(lds, i, 0);
#pragma unroll
  for (int j = 0; j < T::kFragN; ++j) b[0][j] = frag_b(lds, j, 0);

  read_scales(0);
  int cur = 0;
  for (int t = 0; t < steps; ++t) {
    const int nxt = cur + 1 == S ? 0 : cur + 1;
    // Step t+S-1 goes into the slot step t-1 used, which every wave finished
    // reading before the barrier that ended step t-1.
    const int kq = step_k0(t) % kSpanK / 32;  // first block of this step in its word
    issue(t + S - 1, cur == 0 ? S - 1 : cur - 1, false);
#pragma unroll
    for (int s = 0; s < T::kSub; ++s) {
      const int c = s & 1, n = c ^ 1;
      const bool last = s + 1 == T::kSub;
      LDS_PTR(const uint8_t) rb = lds + cur * T::kStage;
      if (!last) {
#pragma unroll
        for (int j = 0; j < T::kFragN; ++j) b[n][j] = frag_b(rb, j, s + 1);
      }
      // The lane's block: kq + 2s + lg of the word; the instruction takes the
      // scale from the low byte of its operand.
      const int sh = 8 * (kq + 2 * s + lg);
#pragma unroll
      for (int i = 0; i < T::kFragM; ++i) {
#pragma unroll
        for (int j = 0; j < T::kFragN; ++j) {
          if constexpr (kScaled) {
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                a[i], b[c][j], acc[i][j], FA, FB, 0, static_cast<int>((sa_w[i] >> sh) & 0xffu),
                0, static_cast<int>((sb_w[j] >> sh) & 0xffu));
          } else {
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[c][j], acc[i][j],
                                                                        FA, FB, 0, 0, 0, 0);
          }
        }
        if (!last) a[i] = frag_a(rb, i, s + 1);
      }
      if (!last) {
        interleave_hint<T>();
      } else {
        // The last sub-step's MFMAs are issued; while they run, wait for
        // step t+1 (data and scale words) and for every wave to finish
        // reading step t's slot, then read step t+1's first fragments (stale
        // and unused after the last step). The copies thus have the whole
        // step to land (8192 x 14336 x 4096: 0.553 -> 0.530 ms against waiting
        // before these MFMAs; the bf16 kernel's shorter MFMAs do not cover the
        // barrier this way and stay as they are).
        wait_step(t + 1);
        __syncthreads();
        rb = lds + nxt * T::kStage;
#pragma unroll
        for (int i = 0; i < T::kFragM; ++i) a[i] = frag_a(rb, i, 0);
#pragma unroll
        for (int j = 0; j < T::kFragN; ++j) b[n][j] = frag_b(rb, j, 0);
        // Its scale words too, so that its first MFMAs do not wait on them.
        read_scales(nxt);
      }
    }
    if constexpr (T::kSub % 2 == 1) {  // the next step's B fragments are in b[1]
#pragma unroll
      for (int j = 0; j < T::kFragN; ++j) b[0][j] = b[1][j];
    }
    cur = nxt;
  }

  // Writing C: as the bf16 kernel -- each wave stages its block through its
  // share of the idle LDS ring, then finishes row-contiguous groups of four
  // with the epilogue. Element v of a 32 x 32 accumulator sits at row
  // 8*(v/4) + 4*(lane/32) + v%4, column lane%32.
  {
    constexpr int kWaveLds = T::kLdsBytes / T::kWaves;
    constexpr int kPassFrags = kWaveLds / (32 * T::kWaveN * 4) < T::kFragM
                                   ? kWaveLds / (32 * T::kWaveN * 4) : T::kFragM;
    static_assert(kPassFrags >= 1 && T::kFragM % kPassFrags == 0, "epilogue staging");
    constexpr int kPassRows = 32 * kPassFrags;
    constexpr int kLanesPerRow = T::kWaveN / 4;
    constexpr int kRowsPerIter = 64 / kLanesPerRow;
    LDS_PTR(float) stage = (LDS_PTR(float))(lds + wave * kWaveLds);
    const int c4 = (lane % kLanesPerRow) * 4;
    const int col = n0 + wn * T::kWaveN + c4;
    const f32x4 bias4 = epi_bias4(col, N, epi);
    __syncthreads();  // every wave is done with the ring
#pragma unroll
    for (int i0 = 0; i0 < T::kFragM; i0 += kPassFrags) {
#pragma unroll
      for (int i = 0; i < kPassFrags; ++i)
#pragma unroll
        for (int j = 0; j < T::kFragN; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            stage[(i * 32 + (v >> 2) * 8 + lg * 4 + (v & 3)) * T::kWaveN + j * 32 + lr] =
                acc[i0 + i][j][v];
      __syncthreads();
#pragma unroll 4
      for (int r = lane / kLanesPerRow; r < kPassRows; r += kRowsPerIter) {
        const f32x4 v = *(LDS_PTR(const f32x4))(stage + r * T::kWaveN + c4);
        const int row = m0 + wm * T::kWaveM + i0 * 32 + r;
        if (row < M && col < N)
          epi_store4(C, static_cast<int64_t>(row) * N + col, col, N, v, bias4, epi);
      }
      __syncthreads();
    }
  }
}

template <class T, int FA, int FB, bool kScaled>
hipError_t launch_tile(const uint8_t* A, const uint8_t* B, const uint8_t* SA, const uint8_t* SB,
                       int scale_dw, void* C, int M, int N, int K, const Epilogue& e,
                       hipStream_t s) {
  static std::atomic<uint64_t> lds_ok{0};  // devices already opted in
  const void* kernel = reinterpret_cast<const void*>(mfma_fp8_kernel<T, FA, FB, kScaled>);
  hipError_t err = allow_lds(lds_ok, kernel, T::kLdsBytes);
  if (err != hipSuccess) return err;
  const int tiles_m = (M + T::BM - 1) / T::BM;
  const int tiles_n = (N + T::BN - 1) / T::BN;
  return launch(mfma_fp8_kernel<T, FA, FB, kScaled>, dim3(tiles_m * tiles_n), dim3(T::kThreads),
                T::kLdsBytes, s, A, B, SA, SB, scale_dw, C, M, N, K, tiles_m, tiles_n, e);
}

template <class T, int FA, int FB>
hipError_t launch_fmt(const uint8_t* A, const uint8_t* B, const uint8_t* SA, const uint8_t* SB,
                      int scale_dw, void* C, int M, int N, int K, const Epilogue& e,
                      hipStream_t s) {
  if (SA != nullptr)
    return launch_tile<T, FA, FB, true>(A, B, SA, SB, scale_dw, C, M, N, K, e, s);
  return launch_tile<T, FA, FB, false>(A, B, SA, SB, scale_dw, C, M, N, K, e, s);
}

template <class T>
hipError_t launch_cfg(const uint8_t* A, int fa, const uint8_t* B, int fb, const uint8_t* SA,
                      const uint8_t* SB, int scale_dw, void* C, int M, int N, int K,
                      const Epilogue& e, hipStream_t s) {
  if (fa == 0 && fb == 0) return launch_fmt<T, 0, 0>(A, B, SA, SB, scale_dw, C, M, N, K, e, s);
  if (fa == 0) return launch_fmt<T, 0, 1>(A, B, SA, SB, scale_dw, C, M, N, K, e, s);
  if (fb == 0) return launch_fmt<T, 1, 0>(A, B, SA, SB, scale_dw, C, M, N, K, e, s);
  return launch_fmt<T, 1, 1>(A, B, SA, SB, scale_dw, C, M, N, K, e, s);
}

}  // namespace

bool mfma_fp8_supports(int64_t M, int64_t N, int64_t K, int mis_a, int mis_b) {
  // 32-bit per-lane copy offsets: every row start of A and B below 4 GiB.
  return K % 32 == 0 && M * K < (int64_t{1} << 32) && N * K < (int64_t{1} << 32) &&
         mis_a == 0 && mis_b == 0;
}

hipError_t launch_mfma_fp8(const uint8_t* A, int a_fmt, const uint8_t* B, int b_fmt,
                           const uint8_t* a_scale, const uint8_t* b_scale, void* D, int M, int N,
                           int K, const Epilogue& e, hipStream_t s) {
  const int nkb = K / 32;
  const int scale_dw = a_scale != nullptr && nkb % 4 == 0 &&
                       reinterpret_cast<uintptr_t>(a_scale) % 4 == 0 &&
                       reinterpret_cast<uintptr_t>(b_scale) % 4 == 0;
  if (use_large_tiles(M, N, kLargeTileFillBf16))
    return launch_cfg<LargeTile>(A, a_fmt, B, b_fmt, a_scale, b_scale, scale_dw, D, M, N, K, e, s);
  return launch_cfg<SmallTile>(A, a_fmt, B, b_fmt, a_scale, b_scale, scale_dw, D, M, N, K, e, s);
}

}  // namespace tdm

// Attention forward on the gfx950 matrix cores: the FlashAttention scheme of
// the pages (CS336 Lecture 5 GPU notes, §6.2: tiling Q, K and V along the
// sequence, online softmax with a running row maximum m and normalizer l
// that rescale what was accumulated when a new block raises the maximum, and
// the three steps fused in one kernel so S and P never reach HBM; GPU/
// attention notes, "online softmax" and "why FlashAttention saves memory").
//
// Per (batch*head, 256-query block) one workgroup of eight waves; wave w owns
// queries q0 + 32w .. q0 + 32w + 31, as two groups of 16 (qg), and walks the
// keys in blocks of 64, on v_mfma_f32_16x16x32_bf16 (at the part's power
// limit a loop of these sustains 13% more FLOPs than one of 32x32x16 on
// random operands; this kernel: 955 -> 927 us, causal 550 -> 540 us):
//   1. S^T = K Q^T, keys as rows, in 16 x 16 tiles: A = 16 rows of the K
//      block (16-byte LDS reads), B = 16 queries, held in registers for the
//      whole kernel. Lane l then holds, for query 16*qg + l%16, keys
//      16*kt + 4*(l/16) + v of the block (kt, v = 0..3): a query's 64 scores
//      sit in four lanes, 16 each;
//   2. online softmax per query, in base 2 (scores times scale * log2 e):
//      block maximum over the lane's 16 values and lanes l^16, l^32,
//      m_new = max(m, block max), alpha = 2^(m - m_new), p = 2^(s - m_new),
//      l = l * alpha + sum p, O *= alpha (blocks without masked keys first
//      try the current m, with the scale folded into p's exponent, one FMA
//      per score, and fall back to the block maximum only when a sum shows
//      that some score passed m + 8);
//   3. O^T += V^T P^T over 32 keys at a time: the p values, rounded to bf16,
//      already sit where the MFMA's B operand wants them (element e of lane
//      l: key 16*(2pp + e/4) + 4*(l/16) + e%4); the A operand V^T is read
//      from the row-major V block with two ds_read_b64_tr_b16 that return
//      exactly those keys for d = 16*dt + l%16. Any key order works as long
//      as both operands share it.
// The waves form two groups, waves 0-3 and 4-7 (wave w runs on SIMD w % 4,
// so each SIMD holds one of each). Each block takes two phases separated by
// workgroup barriers: while one group issues the MFMAs of steps 3 (previous
// block) and 1 (this block), the other runs a softmax on the vector units,
// then they swap, so a SIMD's matrix core and vector unit work side by side
// (the FlashAttention-3 "ping-pong" arrangement). K and V blocks sit in a
// three-slot LDS ring (block t's K is read in phases 2t and 2t+1, its V in
// 2t+2 and 2t+3), filled by global_load_lds copies a block ahead. At the end
// O = O / l is stored in bf16 and lse = (m + log2 l) * ln 2 (the natural-log
// logsumexp of the scaled scores) in fp32.
//
// LDS rows are head_dim * 2 bytes; the swizzles (swz_k, swz_v) were each
// checked with a probe counting bank conflicts for the exact read pattern
// (with the swizzles of the earlier 32 x 32 layout, half of these reads
// conflicted); the kernel counts none.
//
// Ragged sizes: key rows past n_kv load row n_kv - 1 and are masked out
// (score -inf; their V rows are zeroed in LDS, so an infinite value in row
// n_kv - 1 cannot turn into NaN through a zero probability); query rows past
// n_q load row n_q - 1 and are not stored.
// Causal (key j > query i masked; n_q == n_kv): key blocks wholly above a
// wave's queries are skipped by that wave, and the query blocks run
// heaviest first (work_item).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lds_copy.h"
#include "tdm_internal.h"

namespace tdm {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8, kThreads = 64 * kWaves;
constexpr int kStages = 3;
constexpr int kBQ = 32 * kWaves;  // queries per workgroup
constexpr int kBKV = 64;          // keys per block

template <int D>
struct AttnCfg {
  static constexpr int kRow = D * 2;           // bytes per LDS row
  static constexpr int kChunks = kRow / 16;
  static constexpr int kBlock = kBKV * kRow;   // one K or V block
  static constexpr int kStage = 2 * kBlock;    // K block, then V block
  static constexpr int kLdsBytes = kStages * kStage;
  static constexpr int kRowsPerCopy = 1024 / kRow;
  static constexpr int kCopies = kBlock / 1024 / kWaves;  // per wave, per operand
  static constexpr int kKSteps = D / 32;       // MFMA k-steps of K Q^T
  static constexpr int kDTiles = D / 16;       // 16-row tiles of O^T
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  static_assert(kCopies * kWaves * 1024 == kBlock, "whole 1 KB copies");
};

// LDS swizzles (16-byte chunk c of row r at c ^ swz(r)), each measured with
// a probe counting SQ_LDS_BANK_CONFLICT for exactly the read pattern below.
// K rows are read 16 rows x 4 chunks per instruction (lane l: row l%16,
// chunk 4ks + l/16); V rows by transposing reads, 4 rows x 2 chunks per
// 16 lanes (rows 4(l/16) + 0..3). Both depend on the row modulo 8 only.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  if constexpr (D == 128)
    return 4 * (r & 3) + ((r >> 1) & 3);
  else
    return 5 * ((r >> 1) & 1) + 2 * ((r >> 2) & 1);
}
template <int D>
__device__ __forceinline__ int swz_v(int r) {
  if constexpr (D == 128)
    return ((r & 3) << 2) ^ (((r >> 1) & 1) << 1) ^ (((r >> 2) & 1) << 3);
  else
    return ((r & 1) << 2) ^ (((r >> 1) & 1) << 1) ^ (((r >> 2) & 1) << 2);
}

// Workgroup id -> (query block, head). Without the mask every workgroup does
// the same work; the query blocks of a head share its K and V, so they go to
// one XCD (4096-sequence attention: 6% faster than consecutive ids). With
// the causal mask query block b sees b+1 key blocks; consecutive ids are
// dealt round-robin to the 8 XCDs, so id -> block b = id mod n_qblocks would
// give XCD x blocks x, x+8, ... of every head (1.5x the work of XCD 7 at
// 32 blocks per head). Instead heads go in groups of 16 and, within a
// group, the heaviest blocks of all its heads come first: each XCD gets an
// even share of every weight, the short blocks fill the end, and the
// group's K and V stay warm in the caches.
__device__ __forceinline__ void work_item(int id, int n_qblocks, int n_heads, int causal,
                                          int& qb, int& head) {
  if (!causal) {
    // All query blocks of a head on one XCD (ids are dealt round-robin to
    // the 8 XCDs), so that XCD's L2 serves the head's K and V to all of
    // them; with a head count that is not a multiple of 8, heads in order.
    constexpr int kXcds = 8;
    if (n_heads % kXcds == 0) {
      const int xcd = id % kXcds, k = id / kXcds;
      head = (k / n_qblocks) * kXcds + xcd;
      qb = k % n_qblocks;
    } else {
      qb = id % n_qblocks;
      head = id / n_qblocks;
    }
    return;
  }
  constexpr int kGroup = 16;
  const int group = id / (kGroup * n_qblocks);
  const int in_group = id - group * kGroup * n_qblocks;
  const int heads = min(kGroup, n_heads - group * kGroup);  // last group may be short
  qb = n_qblocks - 1 - in_group / heads;
  head = group * kGroup + in_group % heads;
}

template <int D>
__global__ __launch_bounds__(kThreads, 1) void attention_fwd_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ lse, int n_q,
    int n_kv, int n_heads, float scale_log2, int causal) {
  using T = AttnCfg<D>;
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[];
  LDS_PTR(uint8_t) lds = (LDS_PTR(uint8_t))lds_raw;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lq = lane & 15, lg = lane >> 4;
  const int n_qblocks = (n_q + kBQ - 1) / kBQ;
  int qb, head;
  work_item(static_cast<int>(blockIdx.x), n_qblocks, n_heads, causal, qb, head);
  const int q0 = qb * kBQ;
  const int64_t bh = head;
  const uint16_t* Qh = Q + bh * n_q * D;
  const uint16_t* Kh = K + bh * n_kv * D;
  const uint16_t* Vh = V + bh * n_kv * D;

  // The wave's 32 queries form two groups of 16 (qg); lane l holds query
  // 16*qg + l%16 of each. Its Q operand for k-step ks: d = 32*ks + 8*(l/16)
  // + 0..7.
  const int qbase = q0 + 32 * wave + lq;  // + 16 qg
  bf16x8 qf[2][T::kKSteps];
#pragma unroll
  for (int qg = 0; qg < 2; ++qg) {
    const uint16_t* qrow = Qh + static_cast<int64_t>(min(qbase + 16 * qg, n_q - 1)) * D;
#pragma unroll
    for (int ks = 0; ks < T::kKSteps; ++ks)
      qf[qg][ks] =
          __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrow + 32 * ks + 8 * lg));
  }
  // Take delivery of Q here. Left to itself the compiler waits for these
  // loads at their first use inside the key loop, on every iteration, and
  // since memory operations complete in issue order that wait also holds
  // each block until the next block's K and V copies have landed.
#pragma unroll
  for (int qg = 0; qg < 2; ++qg)
#pragma unroll
    for (int ks = 0; ks < T::kKSteps; ++ks) asm volatile("" ::"v"(qf[qg][ks]));

  // Keys this workgroup visits: all, or (causal) up to its last query.
  const int kv_end = causal ? min(n_kv, q0 + kBQ) : n_kv;
  const int blocks = (kv_end + kBKV - 1) / kBKV;

  // Copy plan: copy j of this wave fills rows (wave + 8j) * kRowsPerCopy ..
  // of the block; lane L takes row +L/kChunks, LDS chunk L%kChunks.
  uint32_t off_k[T::kCopies], off_v[T::kCopies];
  const int crow = lane / T::kChunks, cslot = lane % T::kChunks;
#pragma unroll
  for (int j = 0; j < T::kCopies; ++j) {
    const int r = (wave + kWaves * j) * T::kRowsPerCopy + crow;
    off_k[j] = static_cast<uint32_t>(r * T::kRow + ((cslot ^ swz_k<D>(r)) << 4));
    off_v[j] = static_cast<uint32_t>(r * T::kRow + ((cslot ^ swz_v<D>(r)) << 4));
  }
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_offset(lds));
  // Rows past n_kv read row n_kv - 1 into their own (swizzled) LDS places;
  // their scores are masked.
  auto issue = [&](int t, int slot) {
    if (t >= blocks) return;
    const int kb0 = t * kBKV;
    const uint32_t stage = lds0 + slot * T::kStage;
    if (kb0 + kBKV <= n_kv) {  // every row in range
#pragma unroll
      for (int j = 0; j < T::kCopies; ++j) {
        dma16(Kh + static_cast<int64_t>(kb0) * D, off_k[j], stage + (wave + kWaves * j) * 1024);
        dma16(Vh + static_cast<int64_t>(kb0) * D, off_v[j],
              stage + T::kBlock + (wave + kWaves * j) * 1024);
      }
      return;
    }
#pragma unroll
    for (int j = 0; j < T::kCopies; ++j) {
      const int r = (wave + kWaves * j) * T::kRowsPerCopy + crow;
      const int over = kb0 + r - (n_kv - 1);
      const uint32_t back = over > 0 ? static_cast<uint32_t>(over * T::kRow) : 0u;
      dma16(Kh + static_cast<int64_t>(kb0) * D, off_k[j] - back, stage + (wave + kWaves * j) * 1024);
      dma16(Vh + static_cast<int64_t>(kb0) * D, off_v[j] - back,
            stage + T::kBlock + (wave + kWaves * j) * 1024);
    }
  };

  // Per-lane LDS offsets, fixed for the whole kernel. K read of k-step ks:
  // row l%16 of a 16-key tile, chunk 4ks + l/16. Transposing V reads of
  // d-tile dt: key rows 4*(l/16) + (l%16)/4 of a 16-key tile, columns
  // 16dt + 4*(l%4) .. +3; lane l receives, for its d = 16dt + l%16, the four
  // keys 4*(l/16) + 0..3. The swizzles see only the row modulo 8, so the
  // tiles' other rows add constant offsets.
  int koff[T::kKSteps], voff[T::kDTiles];
#pragma unroll
  for (int ks = 0; ks < T::kKSteps; ++ks)
    koff[ks] = lq * T::kRow + (((4 * ks + lg) ^ swz_k<D>(lq)) << 4);
  {
    const int r = 4 * lg + (lq >> 2);
#pragma unroll
    for (int dt = 0; dt < T::kDTiles; ++dt) {
      const int col = 16 * dt + 4 * (lq & 3);
      voff[dt] = r * T::kRow + (((col >> 3) ^ swz_v<D>(r)) << 4) + ((col & 7) << 1);
    }
  }

  f32x4 acc_o[2][T::kDTiles];
#pragma unroll
  for (int qg = 0; qg < 2; ++qg)
#pragma unroll
    for (int dt = 0; dt < T::kDTiles; ++dt)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc_o[qg][dt][v] = 0.f;
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};

  // Keys this wave needs: with the mask, blocks past its last query are
  // skipped (the workgroup still walks them for the copies and barriers).
  const int wave_blocks =
      causal ? min(blocks, (q0 + 32 * wave + 32 + kBKV - 1) / kBKV) : blocks;
  const int group = wave >> 2;  // 0: waves 0-3, 1: waves 4-7 (one of each per SIMD)
  constexpr float kSlack = 8.0f;
  // Scores of the block: s[qg][kt][v] = key 16*kt + 4*(lane/16) + v, query
  // 16*qg + lane%16 (a 16 x 16 accumulator, keys as rows).
  f32x4 s[2][4];
  // p of the last softmax phase in bf16, the B operand of O^T += V^T P^T for
  // the 32 keys of tiles 2pp and 2pp+1: element e = key 16*(2pp + e/4) +
  // 4*(lane/16) + e%4, the key order the V reads use.
  bf16x8 pop[2][2];

  // Matrix phase for block t: O^T += V^T P^T of block t-1, then S^T of block
  // t, at raised issue priority so the SIMD serves the MFMAs first.
  auto matrix = [&](int t) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
    if (t >= 1 && t <= wave_blocks) {
      LDS_PTR(const uint8_t) vblk = lds + ((t - 1) % kStages) * T::kStage + T::kBlock;
#pragma unroll
      for (int pp = 0; pp < 2; ++pp)
#pragma unroll
        for (int dt = 0; dt < T::kDTiles; ++dt) {
          LDS_PTR(const uint8_t) vw = vblk + 32 * pp * T::kRow + voff[dt];
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_PTR(s16x4))(vw));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_PTR(s16x4))(vw + 16 * T::kRow));
          const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
          const bf16x8 av = __builtin_bit_cast(bf16x8, u32x4{l2.x, l2.y, h2.x, h2.y});
#pragma unroll
          for (int qg = 0; qg < 2; ++qg)
            acc_o[qg][dt] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pop[qg][pp], acc_o[qg][dt], 0, 0, 0);
        }
      // V reads four fragments ahead of the MFMAs that use them.
      constexpr int kFrags = 2 * T::kDTiles;
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int g = 0; g < kFrags - 4; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    }
    if (t < wave_blocks) {
      LDS_PTR(const uint8_t) kblk = lds + (t % kStages) * T::kStage;
#pragma unroll
      for (int qg = 0; qg < 2; ++qg)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int v = 0; v < 4; ++v) s[qg][kt][v] = 0.f;
#pragma unroll
      for (int ks = 0; ks < T::kKSteps; ++ks)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const u32x4 a = *(LDS_PTR(const u32x4))(kblk + 16 * kt * T::kRow + koff[ks]);
#pragma unroll
          for (int qg = 0; qg < 2; ++qg)
            s[qg][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                               qf[qg][ks], s[qg][kt], 0, 0, 0);
        }
      // K reads eight ahead.
      constexpr int kReads = 4 * T::kKSteps;
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int g = 0; g < kReads - 8; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // Softmax phase for block t (online softmax in base 2), for both query
  // groups. A query's 64 scores sit in four lanes (l%16 equal), 16 each.
  auto softmax = [&](int t) __attribute__((always_inline)) {
    if (t < 0 || t >= wave_blocks) return;
    const int kb0 = t * kBKV;
    const bool masked = kb0 + kBKV > n_kv || (causal && kb0 + kBKV - 1 > q0 + 32 * wave);
    const bool general = !(scale_log2 >= 0.f) || masked;
    float psum[2] = {0.f, 0.f}, alpha[2] = {1.f, 1.f}, m_new[2] = {m_run[0], m_run[1]};
    auto exps = [&](int qg, float m_use, bool raw) __attribute__((always_inline)) {
      // Exponents, exponentials, then four partial sums: independent work
      // in each stage, so one wave alone on its SIMD keeps issuing.
      float p[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float x = s[qg][i >> 2][i & 3];
        p[i] = raw ? __builtin_fmaf(x, scale_log2, -m_use) : x - m_use;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) p[i] = __builtin_amdgcn_exp2f(p[i]);
      float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 16; ++i) part[i & 3] += p[i];
      psum[qg] = (part[0] + part[1]) + (part[2] + part[3]);
#pragma unroll
      for (int i = 0; i < 16; ++i) pop[qg][i >> 3][i & 7] = static_cast<__bf16>(p[i]);
    };
    auto rebase = [&](int qg, float bmax, bool raw) __attribute__((always_inline)) {
      bmax = fmaxf(bmax, __shfl_xor(bmax, 16));
      bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
      m_new[qg] = bmax > m_run[qg] + kSlack ? bmax : m_run[qg];
      const float m_use = m_new[qg] == -INFINITY ? 0.f : m_new[qg];  // all masked so far
      alpha[qg] = __builtin_amdgcn_exp2f(m_run[qg] - m_use);
      exps(qg, m_use, raw);
    };
    auto block_max = [&](int qg) __attribute__((always_inline)) {
      float bmax = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int v = 0; v < 4; ++v) bmax = fmaxf(bmax, s[qg][kt][v]);
      return bmax;
    };
    if (general) {
#pragma unroll
      for (int qg = 0; qg < 2; ++qg)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int v = 0; v < 4; ++v) s[qg][kt][v] *= scale_log2;
      if (masked) {
        // This lane's first key of the block, made here (an opaque value), so
        // the per-score key offsets are not kept in registers across the loop.
        int key0 = kb0 + 4 * lg;
        asm volatile("" : "+v"(key0));
#pragma unroll
        for (int qg = 0; qg < 2; ++qg) {
          const int lim = causal ? min(n_kv - 1, qbase + 16 * qg) : n_kv - 1;  // last visible key
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int v = 0; v < 4; ++v)
              s[qg][kt][v] = key0 + 16 * kt + v > lim ? -INFINITY : s[qg][kt][v];
        }
      }
#pragma unroll
      for (int qg = 0; qg < 2; ++qg) rebase(qg, block_max(qg), false);
    } else {
      exps(0, m_run[0], true);
      exps(1, m_run[1], true);
      if (__builtin_amdgcn_ballot_w64(!(psum[0] <= 256.f) || !(psum[1] <= 256.f)) != 0) {
#pragma unroll
        for (int qg = 0; qg < 2; ++qg) rebase(qg, block_max(qg) * scale_log2, true);
      }
    }
#pragma unroll
    for (int qg = 0; qg < 2; ++qg) {
      l_run[qg] = l_run[qg] * alpha[qg] + psum[qg];
      m_run[qg] = m_new[qg];
    }
    if (__builtin_amdgcn_ballot_w64(alpha[0] != 1.0f || alpha[1] != 1.0f) != 0) {
#pragma unroll
      for (int qg = 0; qg < 2; ++qg)
#pragma unroll
        for (int dt = 0; dt < T::kDTiles; ++dt)
#pragma unroll
          for (int v = 0; v < 4; ++v) acc_o[qg][dt][v] *= alpha[qg];
    }
  };

  // Two phases per block. Group 0 runs block t's matrix phase while group 1
  // runs the softmax of block t-1, then the roles swap, so each SIMD holds
  // one wave issuing MFMAs and one issuing vector work at any time. Block t
  // lives in slot t % 3: its K is read in phases 2t and 2t+1, its V in
  // phases 2t+2 and 2t+3, and block t+3's copy starts at phase 2t+4.
  issue(0, 0);
  auto phase_start = [&](int t) __attribute__((always_inline)) {
    wait_vm<0>();
    __syncthreads();  // block t landed; phase 2t begins
    issue(t + 1, (t + 1) % kStages);
    const int kb0 = t * kBKV;
    if (t < blocks && kb0 + kBKV > n_kv) {
      // Rows past n_kv hold copies of row n_kv - 1: zero their V rows (read
      // from phase 2t+2 on), so 0 * inf cannot make NaN.
      const int first = n_kv - kb0;
      LDS_PTR(uint8_t) vw = lds + (t % kStages) * T::kStage + T::kBlock;
      const u32x4 zero = {0u, 0u, 0u, 0u};
      for (int i = tid; i < (kBKV - first) * (T::kRow / 16); i += kThreads)
        *(LDS_PTR(u32x4))(vw + (first + i / (T::kRow / 16)) * T::kRow + (i % (T::kRow / 16)) * 16) = zero;
    }
  };
  // The two groups run the same barriers (two per block) in their own loops.
  if (group == 0) {
    for (int t = 0; t <= blocks; ++t) {
      phase_start(t);
      matrix(t);
      __syncthreads();  // phase 2t+1
      softmax(t);
    }
  } else {
    for (int t = 0; t <= blocks; ++t) {
      phase_start(t);
      softmax(t - 1);
      __syncthreads();  // phase 2t+1
      matrix(t);
    }
  }

  __builtin_amdgcn_s_setprio(0);
  // O = acc / l (bf16), lse = (m + log2 l) * ln 2. Lane l holds query
  // 16*qg + l%16 and d = 16*dt + 4*(l/16) + v: four consecutive d per
  // 8-byte store. A query's normalizer is the sum over its four lanes.
#pragma unroll
  for (int qg = 0; qg < 2; ++qg) {
    float l_all = l_run[qg] + __shfl_xor(l_run[qg], 16);
    l_all += __shfl_xor(l_all, 32);
    const int query = qbase + 16 * qg;
    if (query < n_q) {
      const float inv = 1.0f / l_all;
      uint16_t* orow = O + bh * n_q * D + static_cast<int64_t>(query) * D;
#pragma unroll
      for (int dt = 0; dt < T::kDTiles; ++dt) {
        bf16x4 ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = static_cast<__bf16>(acc_o[qg][dt][e] * inv);
        *reinterpret_cast<bf16x4*>(orow + 16 * dt + 4 * lg) = ov;
      }
      if (lse != nullptr && lg == 0)
        lse[bh * n_q + query] = (m_run[qg] + __log2f(l_all)) * 0.693147180559945309f;
    }
  }
}

template <int D>
hipError_t launch_d(const uint16_t* Q, const uint16_t* K, const uint16_t* V, uint16_t* O,
                    float* lse, int bh, int n_q, int n_kv, float scale, int causal,
                    hipStream_t s) {
  static std::atomic<uint64_t> lds_ok{0};
  hipError_t e = allow_lds(lds_ok, reinterpret_cast<const void*>(attention_fwd_kernel<D>),
                           AttnCfg<D>::kLdsBytes);
  if (e != hipSuccess) return e;
  const float scale_log2 = scale * 1.44269504088896341f;
  const dim3 grid(((n_q + kBQ - 1) / kBQ) * bh);
  return launch(attention_fwd_kernel<D>, grid, dim3(kThreads), AttnCfg<D>::kLdsBytes, s, Q, K, V,
                O, lse, n_q, n_kv, bh, scale_log2, causal);
}

}  // namespace

bool attention_supports(int64_t head_dim) { return head_dim == 64 || head_dim == 128; }

hipError_t launch_attention_fwd(const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                                uint16_t* O, float* lse, int bh, int n_q, int n_kv, int head_dim,
                                float scale, int causal, hipStream_t s) {
  if (head_dim == 64) return launch_d<64>(Q, K, V, O, lse, bh, n_q, n_kv, scale, causal, s);
  return launch_d<128>(Q, K, V, O, lse, bh, n_q, n_kv, scale, causal, s);
}

}  // namespace tdm

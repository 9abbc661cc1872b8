// Attention forward on the gfx950 matrix cores: the FlashAttention scheme of
// the pages (CS336 Lecture 5 GPU notes, §6.2: tiling Q, K and V along the
// sequence, online softmax with a running row maximum m and normalizer l
// that rescale what was accumulated when a new block raises the maximum, and
// the three steps fused in one kernel so S and P never reach HBM; GPU/
// attention notes, "online softmax" and "why FlashAttention saves memory").
//
// Per (batch*head, 256-query block) one workgroup of eight waves; wave w owns
// queries q0 + 32w .. q0 + 32w + 31 and walks the keys in blocks of 64:
//   1. S^T = K Q^T on v_mfma_f32_32x32x16_bf16, keys as rows: A = 32 rows of
//      the K block (16-byte LDS reads), B = the wave's queries, held in
//      registers for the whole kernel. Lane l then holds query l%32 and, of
//      each 32-key half, keys 8*(v/4) + 4*(l/32) + v%4 (v = 0..15);
//   2. online softmax per query, in base 2 (scores times scale * log2 e):
//      block maximum over the lane's 32 values and its partner lane l^32,
//      m_new = max(m, block max), alpha = 2^(m - m_new), p = 2^(s - m_new),
//      l = l * alpha + sum p, O *= alpha (blocks without masked keys first
//      try the current m, with the scale folded into p's exponent, one FMA
//      per score, and fall back to the block maximum only when a sum shows
//      that some score passed m + 8);
//   3. O^T += V^T P^T: the p values, rounded to bf16, already sit where the
//      MFMA's B operand wants them, for the key order of step 1 (within a
//      16-key window lane l holds keys 4*(l/32) + 0..3 and 8 + 4*(l/32) +
//      0..3); the A operand V^T is read from the row-major V block with two
//      ds_read_b64_tr_b16 that return exactly those keys for row d = l%32.
//      Any key order works as long as both operands share it.
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
// LDS rows are head_dim * 2 bytes. K: 16-byte chunk c of row r sits at
// c ^ f(r), f(r) = 2*(r % 8) + (r / 8) % 2 (d = 128) or (r >> 1) & 7
// (d = 64): the 16 rows one 16-byte read phase touches fall in 16
// different chunks, and so do rows r..r+7 read at chunks c and c+1. V:
// chunk c of row r at c ^ 4*(r % 4) (d = 128) or c ^ 4*((r / 2) % 2)
// (d = 64): the four rows and four chunks that 32 lanes of a transposing
// read touch land in 16 distinct chunks of the bank space (with
// c ^ 2*(r % 4), rows r and r+1 shared a chunk set: rocprof counted
// 6.7e7 bank-conflict cycles per call at sequence 4096, 32% of the LDS
// active cycles; now 0).
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
typedef float f32x16 __attribute__((ext_vector_type(16)));
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
  static constexpr int kKSteps = D / 16;       // MFMA k-steps of Q K^T
  static constexpr int kDBlocks = D / 32;      // 32-row blocks of O^T
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  static_assert(kCopies * kWaves * 1024 == kBlock, "whole 1 KB copies");
};

template <int D>
__device__ __forceinline__ int swz_k(int r) {
  if constexpr (D == 128)
    return ((r & 7) << 1) | ((r >> 3) & 1);
  else
    return (r >> 1) & 7;
}
template <int D>
__device__ __forceinline__ int swz_v(int r) {
  if constexpr (D == 128)
    return (r & 3) << 2;
  else
    return ((r >> 1) & 1) << 2;
}

typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;

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
  const int lr = lane & 31, lg = lane >> 5;
  const int n_qblocks = (n_q + kBQ - 1) / kBQ;
  int qb, head;
  work_item(static_cast<int>(blockIdx.x), n_qblocks, n_heads, causal, qb, head);
  const int q0 = qb * kBQ;
  const int64_t bh = head;
  const uint16_t* Qh = Q + bh * n_q * D;
  const uint16_t* Kh = K + bh * n_kv * D;
  const uint16_t* Vh = V + bh * n_kv * D;

  // This lane's query and its Q operand: d = 16*ks + 8*lg + 0..7.
  const int query = q0 + 32 * wave + lr;
  bf16x8 qf[T::kKSteps];
  {
    const uint16_t* qrow = Qh + static_cast<int64_t>(min(query, n_q - 1)) * D;
#pragma unroll
    for (int ks = 0; ks < T::kKSteps; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrow + 16 * ks + 8 * lg));
    // Take delivery of Q here. Left to itself the compiler waits for these
    // loads at their first use inside the key loop, on every iteration, and
    // since memory operations complete in issue order that wait also holds
    // each block until the next block's K and V copies have landed.
#pragma unroll
    for (int ks = 0; ks < T::kKSteps; ++ks) asm volatile("" ::"v"(qf[ks]));
  }

  // Keys this workgroup visits: all, or (causal) up to its last query.
  const int kv_end = causal ? min(n_kv, q0 + kBQ) : n_kv;
  const int blocks = (kv_end + kBKV - 1) / kBKV;

  // Copy plan: copy j of this wave fills rows (wave + 4j) * kRowsPerCopy ..
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

  // Per-lane LDS offsets, fixed for the whole kernel: the K reads of k-step
  // ks (row lr of a 32-row half; the other half is 32 rows further) and the
  // transposing V reads of d-block db (key rows 4*(G/2) + i/4 of a 16-key
  // window; the window and the +8 rows of the second read are further
  // rows). The swizzles see only the row modulo 16, so these offsets hold
  // for every half and window (computing them per read cost 4%).
  int koff[T::kKSteps], voff[T::kDBlocks];
#pragma unroll
  for (int ks = 0; ks < T::kKSteps; ++ks)
    koff[ks] = lr * T::kRow + (((2 * ks + lg) ^ swz_k<D>(lr)) << 4);
  {
    const int G = lane >> 4, i = lane & 15;
    const int r = 4 * (G >> 1) + (i >> 2);
#pragma unroll
    for (int db = 0; db < T::kDBlocks; ++db) {
      const int col = 32 * db + 16 * (G & 1) + 4 * (i & 3);
      voff[db] = r * T::kRow + (((col >> 3) ^ swz_v<D>(r)) << 4) + ((col & 7) << 1);
    }
  }

  f32x16 acc_o[T::kDBlocks];
#pragma unroll
  for (int db = 0; db < T::kDBlocks; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc_o[db][v] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // Keys this wave needs: with the mask, blocks past its last query are
  // skipped (the workgroup still walks them for the copies and barriers).
  const int wave_blocks =
      causal ? min(blocks, (q0 + 32 * wave + 32 + kBKV - 1) / kBKV) : blocks;
  const int group = wave >> 2;  // 0: waves 0-3, 1: waves 4-7 (one of each per SIMD)
  constexpr float kSlack = 8.0f;
  f32x16 s[2];
  bf16x8 pop[4];  // p of the last softmax phase in bf16, window w16 = keys 16*w16 ..

  // Matrix phase for block t: O^T += V^T P^T of block t-1, then S^T of block
  // t, at raised issue priority so the SIMD serves the MFMAs first.
  auto matrix = [&](int t) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
    if (t >= 1 && t <= wave_blocks) {
      LDS_PTR(const uint8_t) vblk = lds + ((t - 1) % kStages) * T::kStage + T::kBlock;
#pragma unroll
      for (int w16 = 0; w16 < 4; ++w16) {
#pragma unroll
        for (int db = 0; db < T::kDBlocks; ++db) {
          LDS_PTR(const uint8_t) vw = vblk + 16 * w16 * T::kRow + voff[db];
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_PTR(s16x4))(vw));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_PTR(s16x4))(vw + 8 * T::kRow));
          const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
          const u32x4 av = {l2.x, l2.y, h2.x, h2.y};
          acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), pop[w16],
                                                              acc_o[db], 0, 0, 0);
        }
      }
      // V reads eight ahead of the MFMAs that use them.
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int g = 0; g < 4 * T::kDBlocks - 4; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
    if (t < wave_blocks) {
      LDS_PTR(const uint8_t) kblk = lds + (t % kStages) * T::kStage;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int v = 0; v < 16; ++v) s[h][v] = 0.f;
      // The two halves' accumulator chains alternate.
#pragma unroll
      for (int ks = 0; ks < T::kKSteps; ++ks)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x4 a = *(LDS_PTR(const u32x4))(kblk + 32 * h * T::kRow + koff[ks]);
          s[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), qf[ks], s[h],
                                                         0, 0, 0);
        }
      // K reads eight ahead.
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int g = 0; g < 2 * T::kKSteps - 8; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // Softmax phase for block t (online softmax in base 2, as before).
  auto softmax = [&](int t) __attribute__((always_inline)) {
    if (t < 0 || t >= wave_blocks) return;
    const int kb0 = t * kBKV;
    const bool general =
        !(scale_log2 >= 0.f) || kb0 + kBKV > n_kv || (causal && kb0 + kBKV - 1 > q0 + 32 * wave);
    float psum = 0.f, alpha = 1.f, m_new = m_run;
    auto exps = [&](float m_use, bool raw) __attribute__((always_inline)) {
      // Exponents, exponentials, then four partial sums: independent work
      // in each stage, so one wave alone on its SIMD keeps issuing.
      float p[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const float x = s[i >> 4][i & 15];
        p[i] = raw ? __builtin_fmaf(x, scale_log2, -m_use) : x - m_use;
      }
#pragma unroll
      for (int i = 0; i < 32; ++i) p[i] = __builtin_amdgcn_exp2f(p[i]);
      float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 32; ++i) part[i & 3] += p[i];
      psum = (part[0] + part[1]) + (part[2] + part[3]);
#pragma unroll
      for (int i = 0; i < 32; ++i) pop[i >> 3][i & 7] = static_cast<__bf16>(p[i]);
    };
    auto rebase = [&](float bmax, bool raw) __attribute__((always_inline)) {
      bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
      m_new = bmax > m_run + kSlack ? bmax : m_run;
      const float m_use = m_new == -INFINITY ? 0.f : m_new;  // all masked so far
      alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      exps(m_use, raw);
    };
    if (general) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int v = 0; v < 16; ++v) s[h][v] *= scale_log2;
      if (kb0 + kBKV > n_kv || (causal && kb0 + kBKV - 1 > q0 + 32 * wave)) {
        const int lim = causal ? min(n_kv - 1, query) : n_kv - 1;  // last visible key
        // This lane's first key of the block, made here (an opaque value), so
        // the 32 per-score key offsets are not kept in registers across the
        // loop.
        int key0 = kb0 + 4 * lg;
        asm volatile("" : "+v"(key0));
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = key0 + 32 * h + 8 * (v >> 2) + (v & 3);
            s[h][v] = key > lim ? -INFINITY : s[h][v];
          }
      }
      float bmax = -INFINITY;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int v = 0; v < 16; ++v) bmax = fmaxf(bmax, s[h][v]);
      rebase(bmax, false);
    } else {
      exps(m_run, true);
      if (__builtin_amdgcn_ballot_w64(!(psum <= 256.f)) != 0) {
        float bmax = -INFINITY;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int v = 0; v < 16; ++v) bmax = fmaxf(bmax, s[h][v]);
        rebase(bmax * scale_log2, true);
      }
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
      for (int db = 0; db < T::kDBlocks; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc_o[db][v] *= alpha;
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
  // O = acc / l (bf16), lse = (m + log2 l) * ln 2. Lane l holds query lr,
  // d = 32*db + 8*(v/4) + 4*lg + v%4: four consecutive d per 8-byte store.
  l_run += __shfl_xor(l_run, 32);  // the row's two halves
  if (query < n_q) {
    const float inv = 1.0f / l_run;
    uint16_t* orow = O + bh * n_q * D + static_cast<int64_t>(query) * D;
#pragma unroll
    for (int db = 0; db < T::kDBlocks; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * db + 8 * q4 + 4 * lg;
        bf16x4 ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = static_cast<__bf16>(acc_o[db][4 * q4 + e] * inv);
        *reinterpret_cast<bf16x4*>(orow + d) = ov;
      }
    if (lse != nullptr && lg == 0)
      lse[bh * n_q + query] = (m_run + __log2f(l_run)) * 0.693147180559945309f;
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

// Small-M bf16 product (M <= 16): a bandwidth path.
//
// With a handful of rows in A the product does about 2*M FLOPs per byte of
// B, far below the ridge point, so its time is the time to stream B from HBM
// once (CS336 Lecture 5 GPU notes, §2.2 roofline; compute- vs memory-bound
// lesson, what to optimise when memory-bound: read every byte once, in large
// aligned coalesced blocks; LLM course ch. 15, §15.9 on decode-like steps).
//
// HBM streams well only when neighbouring lanes, waves and workgroups read
// long contiguous runs, so B is cut into blocks of 256 columns (512-byte row
// pieces) by a slice of K, sized so that at most 256 workgroups run (one per
// CU; fewer, longer slices measured faster than two per CU, and they halve
// the partial sums):
//   * a workgroup of 4 waves owns one block. Per step of 32 rows each wave
//     copies 8 rows of B and 4 rows of the matching 32 columns of A straight
//     into an LDS ring of kStages stages (global_load_lds, no registers),
//     kStages-1 steps ahead of the arithmetic. Nothing else in the loop
//     touches global memory, so the only waits are for copies that are
//     kStages-2 steps old;
//   * each wave then reads its 64 columns back with ds_read_b64_tr_b16,
//     which hands every lane four consecutive k of one column (the operand
//     layout of v_mfma_f32_16x16x32_bf16), and runs four MFMAs against the
//     staged rows of A;
//   * the workgroups of one column block each produce a partial 16 x 256
//     sum and write it to a workspace; a second, small kernel adds the
//     partials of each output in slice order and writes C, so the result is
//     bitwise reproducible. (Combining them inside the first kernel needs a
//     device-scope release by every workgroup, which writes back its XCD's
//     whole L2, or device-coherent stores, an arrival counter and
//     device-coherent loads by the last workgroup; both measured slower than
//     a second launch.) With a single slice the sums go straight to C,
//     finished by the epilogue in the first kernel.
//   * the workspace is static device memory of the library (no allocation
//     at call time): a table of kSlots buffers of 4 MB per device, one per
//     stream that calls this path, so calls on different streams never
//     share one and calls on one stream are ordered by the stream. A stream
//     that finds the table full runs the matrix-core kernel instead (same
//     result up to summation order; no workspace).
// A K that is not a multiple of 32 has its last step loaded through
// registers with every k beyond K set to zero. Rows of A at or beyond M
// are copied from row M-1; their products reach only rows of C that are not
// stored.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "tdm_internal.h"

namespace tdm {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

#define LDS_PTR(T) __attribute__((address_space(3))) T*

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBlockN = 256;                        // columns per workgroup
constexpr int kRowBytes = kBlockN * 2;              // 512
constexpr int kStepK = 32;                          // K rows per step
constexpr int kMaxM = 16;
constexpr int kStageB = kStepK * kRowBytes;         // 16 KB of B
constexpr int kRowA = kStepK * 2;                   // 64 bytes of one row of A
constexpr int kStageBytes = kStageB + kMaxM * kRowA;  // + 1 KB of A
constexpr int kStages = 3;                          // LDS ring: 51 KB
constexpr int kLdsBytes = kStages * kStageBytes;
constexpr int kTargetGroups = 256;                  // one per CU
constexpr int kCopiesB = kStepK * kRowBytes / 1024 / kWaves;  // 1-KB copies of B per wave per step
constexpr int kLanesPerRow = kRowBytes / 16;        // lanes of one copy that cover a row
constexpr int kColsPerWave = kBlockN / kWaves;
constexpr int kAcc = kColsPerWave / 16;             // 16 x 16 accumulators per wave
constexpr int kCopies = kCopiesB + 1;               // + one partial-wave copy of A
constexpr int kPer = kMaxM * kBlockN;               // floats per partial block

// Chunk swizzle of the staged rows of B: the four rows and two chunks that
// one 16-lane group of a transposed read touches land on distinct banks, and
// the group reading rows k+8.. in the same cycle lands on the other half.
__device__ __forceinline__ int swz(int k) {
  return ((k & 3) << 2) ^ (((k >> 1) & 1) << 1) ^ (((k >> 3) & 1) << 1);
}
// Chunk swizzle of the staged rows of A (64 bytes each, four per bank
// window): the 16 rows one read touches spread over every bank.
__device__ __forceinline__ int swz_a(int m) { return (m >> 2) & 3; }

__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_addr) {
  // global -> LDS, 16 bytes per active lane, lane l at lds_addr + 16*l,
  // marked non-temporal (streamed once). Inline assembly keeps the compiler
  // from stalling later LDS reads on it; the wait is explicit
  // (wait_copies_upto) before the barrier that publishes the stage. M0
  // carries the LDS address; nothing else here uses M0.
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt"
               :
               : "v"(gptr), "s"(lds_addr)
               : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_copies_upto() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ uint32_t lds_offset(LDS_PTR(const uint8_t) p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

// Copy step rows [k0, k0+32) x columns [n0, n0+kBlockN) of B and rows 0..15 x
// columns [k0, k0+32) of A into a stage. Wave w copies rows 8w..8w+7 of B,
// two rows per instruction, and 16/kWaves rows of A with its first lanes.
// Columns of B past N and rows of A past M are clamped.
__device__ __forceinline__ void copy_step(const uint16_t* __restrict__ A,
                                          const uint16_t* __restrict__ B, int M, int N, int K,
                                          int k0, int n0, int wave, int lane, uint32_t stage) {
#pragma unroll
  for (int j = 0; j < kCopiesB; ++j) {
    const int row = (wave * kCopiesB + j) * (64 / kLanesPerRow) + lane / kLanesPerRow;
    const int c = (lane % kLanesPerRow) ^ swz(row);
    const int gn = min(n0 + c * 8, N - 8);
    dma16(B + static_cast<int64_t>(k0 + row) * N + gn,
          stage + (wave * kCopiesB + j) * 1024);
  }
  constexpr int kRowsA = kMaxM / kWaves;  // rows of A per wave
  if (lane < 4 * kRowsA) {
    const int r = wave * kRowsA + (lane >> 2);
    const int m = min(r, M - 1);
    dma16(A + static_cast<int64_t>(m) * K + k0 + ((lane & 3) ^ swz_a(r)) * 8,
          stage + kStageB + wave * kRowsA * kRowA);
  }
}

// The same, through registers, with every k at or beyond K set to zero.
__device__ __forceinline__ void copy_step_masked(const uint16_t* __restrict__ A,
                                                 const uint16_t* __restrict__ B, int M, int N,
                                                 int K, int k0, int n0, int tid,
                                                 LDS_PTR(uint8_t) stage) {
  const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < kStageB / 16 / kThreads; ++i) {
    const int id = tid + kThreads * i;
    const int row = id / kLanesPerRow, c = id % kLanesPerRow;
    const int gk = k0 + row;
    const int gn = min(n0 + c * 8, N - 8);
    u32x4 v = zero;
    if (gk < K) v = *reinterpret_cast<const u32x4*>(B + static_cast<int64_t>(gk) * N + gn);
    *(LDS_PTR(u32x4))(stage + row * kRowBytes + ((c ^ swz(row)) << 4)) = v;
  }
  if (tid < kMaxM * 4) {  // A: 16 rows x 4 chunks of 8 k
    const int m = min(tid >> 2, M - 1), gk = k0 + ((tid & 3) ^ swz_a(tid >> 2)) * 8;
    u32x4 v = zero;
    if (gk < K) v = *reinterpret_cast<const u32x4*>(A + static_cast<int64_t>(m) * K + gk);
    *(LDS_PTR(u32x4))(stage + kStageB + tid * 16) = v;
  }
}

// Four consecutive k (k_base + 0..3) of column n_base + lane%16 (lane j of each
// 16-lane group receives element e from the address of lane 4e + j/4).
__device__ __forceinline__ s16x4 read_tr(LDS_PTR(const uint8_t) stage, int k_base, int n_base,
                                         int lane) {
  const int i = lane & 15;
  const int k = k_base + (i >> 2);
  const int col = n_base + 4 * (i & 3);
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (LDS_PTR(s16x4))(stage + k * kRowBytes + (((col >> 3) ^ swz(k)) << 4) + ((col & 7) << 1)));
}

__global__ __launch_bounds__(kThreads, 1) void skinny_bf16_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, void* C, int M, int N,
    int K, int slices, int slice_steps, float* __restrict__ partials, Epilogue epi) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[];
  LDS_PTR(uint8_t) lds = (LDS_PTR(uint8_t))lds_raw;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int block = blockIdx.x / slices;  // column block
  const int slice = blockIdx.x - block * slices;
  const int n0 = block * kBlockN;

  const int steps_total = (K + kStepK - 1) / kStepK;
  const int full_steps = K / kStepK;
  const int s_begin = min(steps_total, slice * slice_steps);
  const int s_end = min(steps_total, s_begin + slice_steps);
  const int nsteps = s_end - s_begin;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_offset(lds));

  auto issue = [&](int j) {  // step s_begin + j into stage j % kStages
    const int st = s_begin + j;
    if (j >= nsteps) return;
    const int stage = j % kStages;
    if (st < full_steps)
      copy_step(A, B, M, N, K, st * kStepK, n0, wave, lane, lds0 + stage * kStageBytes);
    else
      copy_step_masked(A, B, M, N, K, st * kStepK, n0, tid, lds + stage * kStageBytes);
  };

#pragma unroll
  for (int j = 0; j < kStages - 1; ++j) issue(j);

  f32x4 acc[kAcc];
#pragma unroll
  for (int q = 0; q < kAcc; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int g = lane >> 4;
  const int m = lane & 15;

  for (int j = 0; j < nsteps; ++j) {
    // Step j's copies (this wave's) are done once at most the copies of the
    // kStages-2 later steps are in flight; the barrier makes every wave's
    // copies visible and frees the stage step j-1 used.
    // (Only when all of those are copies; near a register-loaded tail step
    // wait for everything.)
    if (j + kStages - 2 < nsteps && s_begin + j + kStages - 2 < full_steps)
      wait_copies_upto<kCopies * (kStages - 2)>();
    else
      wait_copies_upto<0>();
    __syncthreads();
    issue(j + kStages - 1);

    LDS_PTR(const uint8_t) stage = lds + (j % kStages) * kStageBytes;
    // Lane (m, g) takes k = 8g..8g+7 of row m of A.
    const bf16x8 a = __builtin_bit_cast(
        bf16x8, *(LDS_PTR(const u32x4))(stage + kStageB + m * kRowA + ((g ^ swz_a(m)) << 4)));
#pragma unroll
    for (int q = 0; q < kAcc; ++q) {
      const int nb = wave * kColsPerWave + q * 16;
      const s16x4 lo = read_tr(stage, 8 * g, nb, lane);
      const s16x4 hi = read_tr(stage, 8 * g + 4, nb, lane);
      const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
      const u32x4 bw = {l2.x, l2.y, h2.x, h2.y};
      acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, bw),
                                                       acc[q], 0, 0, 0);
    }
  }

  // Element v of accumulator q: row 4*(lane/16) + v, column
  // kColsPerWave*wave + 16q + lane%16. Without a partial-sum buffer (one
  // slice) the sums are the outputs, finished by the epilogue here.
  if (partials == nullptr) {
#pragma unroll
    for (int q = 0; q < kAcc; ++q)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = 4 * g + v, col = n0 + wave * kColsPerWave + q * 16 + m;
        if (row < M && col < N)
          epi_store(C, static_cast<int64_t>(row) * N + col, col, acc[q][v], epi);
      }
    return;
  }

  // Partial sums: workspace[block][slice][16][kBlockN].
  float* mine = partials + (static_cast<int64_t>(block) * slices + slice) * (kMaxM * kBlockN);
#pragma unroll
  for (int q = 0; q < kAcc; ++q)
#pragma unroll
    for (int v = 0; v < 4; ++v)
      mine[(4 * g + v) * kBlockN + wave * kColsPerWave + q * 16 + m] = acc[q][v];
}

// C[row][col] = sum over slices (in slice order) of the partials, finished
// by the fused epilogue (an empty one stores the fp32 sum).
__global__ __launch_bounds__(256) void skinny_reduce_kernel(const float* __restrict__ partials,
                                                            void* C, int M, int N, int slices,
                                                            Epilogue epi) {
  constexpr int kGroups = kPer / 256;    // workgroups per column block
  const int block = blockIdx.x / kGroups;
  const int e = (blockIdx.x - block * kGroups) * 256 + threadIdx.x;
  const int row = e / kBlockN, col = block * kBlockN + (e - row * kBlockN);
  if (row >= M || col >= N) return;
  const float* p = partials + static_cast<int64_t>(block) * slices * kPer + e;
  float sum = 0.f;
  int s = 0;
  for (; s + 8 <= slices; s += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[(s + u) * kPer];
#pragma unroll
    for (int u = 0; u < 8; ++u) sum += v[u];
  }
  for (; s < slices; ++s) sum += p[s * kPer];
  epi_store(C, static_cast<int64_t>(row) * N + col, col, sum, epi);
}

// Workspace for the partial sums. A launch has at most kTargetGroups
// workgroups when it splits K (blocks * slices <= kTargetGroups), each
// writing one kPer-float partial block, so one buffer of kSlotFloats floats
// (4 MB) holds any call. The buffers are a static array of the library's
// code object, present on every device the library runs on from the first
// use until the process ends; nothing is allocated at call time.
constexpr int kSlots = 8;
constexpr size_t kSlotFloats = static_cast<size_t>(kTargetGroups) * kPer;
__device__ __align__(256) float g_partials[kSlots * kSlotFloats];

// The buffer of the allocation-free entry point (gemm_bf16_ex_noalloc): one
// 4 MB array per device, shared by every call of that entry point on the
// device, for callers that cannot allocate (graph capture, serving loops).
// Calls of that entry point that overlap on one device race on it. Nothing
// in it needs clearing: each workgroup writes its whole partial block before
// the reduction reads it, and the reduction reads only blocks of this call.
__device__ __align__(256) float scratch[kSlotFloats];

// Device address of `scratch`, per device, looked up once with that device
// current: the array's name is only a host-side stand-in for it.
struct ScratchTable {
  std::mutex mu;
  float* ptr[64] = {};
};
ScratchTable g_scratch;

hipError_t scratch_ptr(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch.mu);
  if (g_scratch.ptr[dev] == nullptr) {
    void* p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
    g_scratch.ptr[dev] = static_cast<float*>(p);
  }
  *out = g_scratch.ptr[dev];
  return hipSuccess;
}

// Per-device table: slot i belongs to the stream that first claimed it, for
// the rest of the process (a stream handle is only compared, never used).
// Calls on one stream are ordered by that stream, so its slot is never used
// by two launches at once.
constexpr int kMaxDevices = 64;
struct SlotTable {
  std::mutex mu;
  float* base = nullptr;  // device address of g_partials on this device
  int used = 0;
  hipStream_t owner[kSlots] = {};
};
SlotTable g_tables[kMaxDevices];

// The partial-sum buffer of stream s on the current device, or nullptr when
// all kSlots are owned by other streams.
hipError_t stream_slot(hipStream_t s, float** out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  SlotTable& t = g_tables[dev];
  std::lock_guard<std::mutex> lock(t.mu);
  if (t.base == nullptr) {
    // The array's name is a host-side stand-in; its address on this device
    // comes from the runtime.
    void* p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_partials))) != hipSuccess) return e;
    t.base = static_cast<float*>(p);
  }
  for (int i = 0; i < t.used; ++i)
    if (t.owner[i] == s) {
      *out = t.base + i * kSlotFloats;
      return hipSuccess;
    }
  if (t.used < kSlots) {
    t.owner[t.used] = s;
    *out = t.base + t.used * kSlotFloats;
    ++t.used;
  }
  return hipSuccess;
}

}  // namespace

bool skinny_bf16_supports(int64_t M, int64_t N, int64_t K, int mis_a,
                          int mis_b, int mis_c) {
  (void)mis_c;
  return M >= 1 && M <= kMaxM && N % 8 == 0 && K % 8 == 0 && K >= 8 && mis_a == 0 &&
         mis_b == 0;
}

namespace {

// Slices of K for a product with `blocks` column blocks: as many as keep
// the grid at one round of kTargetGroups workgroups, no empty ones.
void split(int N, int K, int* blocks, int* slices, int* slice_steps) {
  *blocks = (N + kBlockN - 1) / kBlockN;
  const int steps = (K + kStepK - 1) / kStepK;
  int sl = kTargetGroups / *blocks;  // rounded down: no second round of workgroups
  if (sl > steps) sl = steps;
  if (sl < 1) sl = 1;
  *slice_steps = (steps + sl - 1) / sl;
  *slices = (steps + *slice_steps - 1) / *slice_steps;
}

// shared_scratch: take the partial sums to `scratch` instead of the
// stream's buffer (the allocation-free entry point).
hipError_t launch_skinny(const uint16_t* A, const uint16_t* B, void* C, int M, int N, int K,
                         const Epilogue& epi, hipStream_t s, bool shared_scratch) {
  static std::atomic<uint64_t> lds_ok{0};  // devices already opted in
  hipError_t e = allow_lds(lds_ok, reinterpret_cast<const void*>(skinny_bf16_kernel), kLdsBytes);
  if (e != hipSuccess) return e;
  int blocks, slices, slice_steps;
  split(N, K, &blocks, &slices, &slice_steps);
  if (slices == 1)  // the sums are the outputs: no workspace
    return launch(skinny_bf16_kernel, dim3(blocks), dim3(kThreads), kLdsBytes, s, A, B, C, M,
                  N, K, slices, slice_steps, static_cast<float*>(nullptr), epi);
  float* partials = nullptr;
  if ((e = shared_scratch ? scratch_ptr(&partials) : stream_slot(s, &partials)) != hipSuccess)
    return e;
  // split() keeps blocks * slices <= kTargetGroups, so the partial blocks
  // always fit either buffer; the guard keeps a future split from writing
  // past one.
  if (static_cast<size_t>(blocks) * slices * kPer > kSlotFloats) return hipErrorInvalidValue;
  if (partials == nullptr) {  // every buffer belongs to another stream
    if (mfma_bf16_supports(M, N, K, 0, 0, 0))
      return launch_mfma_bf16_epi(A, B, false, false, C, M, N, K, epi, s);
    return launch_edge_bf16_epi(A, B, false, false, C, M, N, K, epi, s);
  }
  e = launch(skinny_bf16_kernel, dim3(blocks * slices), dim3(kThreads), kLdsBytes, s, A, B,
             static_cast<void*>(nullptr), M, N, K, slices, slice_steps, partials, epi);
  if (e != hipSuccess) return e;
  return launch(skinny_reduce_kernel, dim3(blocks * (kPer / 256)), dim3(256), 0, s, partials,
                C, M, N, slices, epi);
}

}  // namespace

hipError_t launch_skinny_bf16(const uint16_t* A, const uint16_t* B, float* C,
                              int M, int N, int K, hipStream_t s) {
  return launch_skinny(A, B, C, M, N, K, Epilogue{}, s, false);
}

hipError_t launch_skinny_bf16_epi(const uint16_t* A, const uint16_t* B, bool b_nk, void* D,
                                  int M, int N, int K, const Epilogue& e, hipStream_t s,
                                  bool shared_scratch) {
  if (b_nk) return launch_skinny_nk_bf16(A, B, D, M, N, K, e, s);  // gemm_skinny_nk_bf16.hip
  return launch_skinny(A, B, D, M, N, K, e, s, shared_scratch);
}

}  // namespace tdm

// Internal interface between the C ABI (tdm_api.hip) and the kernel files.
// Every launcher enqueues on `stream` and returns the status of its own
// launches (hipLaunchKernel's return value, not a sticky error left by some
// earlier call). Callers have validated sizes and pointers beforehand.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "epilogue.h"

#include <atomic>
#include <tuple>
#include <utility>

namespace tdm {

// Launch `kernel` and return the launch's status. The arguments are
// converted to the kernel's parameter types and passed by address.
template <typename... P, typename Tuple, size_t... I>
hipError_t launch_with(void (*kernel)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t s,
                       Tuple& args, std::index_sequence<I...>) {
  void* ptrs[] = {static_cast<void*>(&std::get<I>(args))...};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, lds, s);
}

template <typename... P, typename... A>
hipError_t launch(void (*kernel)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t s,
                  A... args) {
  static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
  std::tuple<P...> values(static_cast<P>(args)...);
  return launch_with(kernel, grid, block, lds, s, values, std::index_sequence_for<P...>{});
}

// Allow `kernel` more than the default 64 KB of dynamic LDS on the current
// device; done once per kernel and device (devices 0..63 are remembered;
// beyond that the attribute is set on every call).
inline hipError_t allow_lds(std::atomic<uint64_t>& done, const void* kernel, int bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t{1} << dev) : 0;
  if (bit != 0 && (done.load(std::memory_order_acquire) & bit) != 0) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit != 0) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

// Tile-size choice of the matrix-core kernels. A 256 x 256 tile moves half
// the bytes per FLOP of a 128 x 128 tile, but one workgroup per CU holds it,
// so a product with few of them leaves CUs idle in its last round. The large
// tile is taken when its rounds over the 256 CUs are at least `min_fill`
// full; below that the 128 x 128 tile (two per CU) balances better. The
// thresholds were set from timings of both tile sizes on square and
// rectangular products: the bandwidth-hungry bf16 kernel gains more from the
// large tile than the fp32 kernel, which is bound by matrix-core issue.
constexpr int kCUs = 256;
constexpr double kLargeTileFillBf16 = 0.70;
constexpr double kLargeTileFillF32 = 0.90;
inline bool use_large_tiles(int64_t M, int64_t N, double min_fill) {
  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  const int64_t rounds = (tiles + kCUs - 1) / kCUs;
  return static_cast<double>(tiles) >= min_fill * static_cast<double>(rounds * kCUs);
}

// --- shape requirements of each kernel family --------------------------
// Sizes are already known to be >= 1 and each matrix < 2^31 elements.

// 32x32 LDS-tiled kernel: any shape, element-aligned pointers.
inline bool edge_supports(int64_t, int64_t, int64_t) { return true; }

// fp32 register/LDS-tiled VALU kernel: 16-byte chunks along K and N.
bool valu_f32_supports(int64_t M, int64_t N, int64_t K, int mis_a, int mis_b,
                       int mis_c);

// fp32 MFMA kernel: 16-byte chunks along K, and along N (B stored K x N) or
// M (A stored K x M).
bool mfma_f32_supports(int64_t M, int64_t N, int64_t K, int mis_a, int mis_b,
                       int mis_c, bool b_nk = false, bool a_km = false);

// bf16 MFMA kernel: 16-byte chunks (8 elements) along K and N.
bool mfma_bf16_supports(int64_t M, int64_t N, int64_t K, int mis_a, int mis_b,
                        int mis_c);
// ... with B stored N x K (C = A * B^T): 16-byte chunks along K only.
// Attention forward (attention_fwd.hip): Q [bh][n_q][d], K and V
// [bh][n_kv][d], O [bh][n_q][d] bf16; lse [bh][n_q] fp32 or null; d 64 or 128.
bool attention_supports(int64_t head_dim);
hipError_t launch_attention_fwd(const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                                uint16_t* O, float* lse, int bh, int n_q, int n_kv, int head_dim,
                                float scale, int causal, hipStream_t s);

// FP8 product (gemm_mfma_fp8.hip): A M x K, B N x K, formats 0 = E4M3,
// 1 = E5M2; a_scale/b_scale both null (unscaled) or both block exponents.
bool mfma_fp8_supports(int64_t M, int64_t N, int64_t K, int mis_a, int mis_b);
hipError_t launch_mfma_fp8(const uint8_t* A, int a_fmt, const uint8_t* B, int b_fmt,
                           const uint8_t* a_scale, const uint8_t* b_scale, void* D, int M, int N,
                           int K, const Epilogue& e, hipStream_t s);
bool mfma_bf16_nk_supports(int64_t M, int64_t N, int64_t K, int mis_a, int mis_b,
                           int mis_c);
// ... with A stored K x M (C = A^T * op(B)): 16-byte chunks along M.
bool mfma_bf16_akm_supports(int64_t M, int64_t N, int64_t K, bool b_nk, int mis_a, int mis_b,
                            int mis_c);

// bf16 small-M streaming kernel.
bool skinny_bf16_supports(int64_t M, int64_t N, int64_t K, int mis_a,
                          int mis_b, int mis_c);
// ... with B stored N x K.
bool skinny_bf16_nk_supports(int64_t M, int64_t N, int64_t K, int mis_a, int mis_b,
                             int mis_c);

// --- launchers ----------------------------------------------------------
hipError_t launch_fill_zero_f32(float* C, int64_t count, hipStream_t s);

hipError_t launch_edge_f32(const float* A, const float* B, float* C, int M,
                           int N, int K, hipStream_t s);
// b_nk: B is stored N x K; a_km: A is stored K x M.
hipError_t launch_edge_f32_layout(const float* A, const float* B, bool b_nk, bool a_km, float* C,
                                  int M, int N, int K, hipStream_t s);
hipError_t launch_edge_bf16(const uint16_t* A, const uint16_t* B, float* C,
                            int M, int N, int K, hipStream_t s);

hipError_t launch_valu_f32(const float* A, const float* B, float* C, int M,
                           int N, int K, hipStream_t s);

hipError_t launch_mfma_f32(const float* A, const float* B, float* C, int M,
                           int N, int K, hipStream_t s);
hipError_t launch_mfma_f32_layout(const float* A, const float* B, bool b_nk, bool a_km, float* C,
                                  int M, int N, int K, hipStream_t s);

hipError_t launch_mfma_bf16(const uint16_t* A, const uint16_t* B, float* C,
                            int M, int N, int K, hipStream_t s);

hipError_t launch_skinny_bf16(const uint16_t* A, const uint16_t* B, float* C,
                              int M, int N, int K, hipStream_t s);

// The bf16 products with the fused epilogue of epilogue.h, written to D (fp32
// or bf16 as e.d_bf16 says). b_nk: B is stored N x K (op(B) = B^T); a_km: A
// is stored K x M (op(A) = A^T). K may be 0 on the edge kernel (D =
// epilogue(0)).
hipError_t launch_edge_bf16_epi(const uint16_t* A, const uint16_t* B, bool b_nk, bool a_km,
                                void* D, int M, int N, int K, const Epilogue& e, hipStream_t s);
hipError_t launch_mfma_bf16_epi(const uint16_t* A, const uint16_t* B, bool b_nk, bool a_km,
                                void* D, int M, int N, int K, const Epilogue& e, hipStream_t s);
// shared_scratch: the small-M K x N split-K partial sums go to the one
// static buffer of the allocation-free entry point instead of the stream's.
hipError_t launch_skinny_bf16_epi(const uint16_t* A, const uint16_t* B, bool b_nk, void* D,
                                  int M, int N, int K, const Epilogue& e, hipStream_t s,
                                  bool shared_scratch = false);
hipError_t launch_skinny_nk_bf16(const uint16_t* A, const uint16_t* B, void* D, int M, int N,
                                 int K, const Epilogue& e, hipStream_t s);

}  // namespace tdm

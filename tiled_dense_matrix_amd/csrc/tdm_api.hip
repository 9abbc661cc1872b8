// C ABI of libtdm.so: argument validation, path choice, cost model.
//
// The declarations and the contract (layouts, ownership, errors) are in
// include/tdm.h. Every check here runs on the host before any HIP call, so
// invalid calls are rejected identically with or without a GPU.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstring>

#include "tdm.h"
#include "tdm_internal.h"

namespace {

constexpr int64_t kMaxElems = int64_t{1} << 31;  // per matrix (32-bit indexing)

// MI355X figures used by the dispatcher (AMD's published peaks).
constexpr double kPeakMfmaBf16 = 2.5166e15;  // FLOP/s, dense
constexpr double kHbmBandwidth = 8.0e12;     // B/s

// The integer value of a C enum argument. A C caller may pass any int as an
// enum parameter, but C++ may not read an enum object whose value lies
// outside the enumeration's range, so every enum argument is range-checked
// through its bytes before it is read as the enum.
template <typename E>
int raw(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "C enums are int-sized");
  int v;
  std::memcpy(&v, &e, sizeof v);
  return v;
}
bool valid_kind(int k) { return k == TDM_KIND_F32 || k == TDM_KIND_BF16_F32ACC; }
bool valid_dtype(int d) { return d == TDM_DTYPE_F32 || d == TDM_DTYPE_BF16; }
bool valid_fp8(int f) { return f == TDM_FP8_E4M3 || f == TDM_FP8_E5M2; }

int misalign(const void* p) { return static_cast<int>(reinterpret_cast<uintptr_t>(p) & 15u); }

bool too_big(int64_t M, int64_t N, int64_t K) {
  auto over = [](int64_t a, int64_t b) {
    if (a == 0 || b == 0) return false;
    if (a > kMaxElems || b > kMaxElems) return true;
    return a > (kMaxElems - 1) / b;
  };
  return over(M, K) || over(K, N) || over(M, N);
}

// True when byte ranges [p, p+pb) and [q, q+qb) share an address.
bool overlaps(const void* p, uint64_t pb, const void* q, uint64_t qb) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
  return pb > 0 && qb > 0 && a < b + qb && b < a + pb;
}

tdm_status check_device() {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) return TDM_ERROR_NO_DEVICE;
  return TDM_SUCCESS;
}

// Shape/alignment admission of each path for one kind; b_nk: B is stored
// N x K, a_km: A is stored K x M (the vector-ALU kernel takes neither).
bool supports(tdm_kind kind, tdm_path path, int64_t M, int64_t N, int64_t K,
              int ma, int mb, int mc, bool b_nk = false, bool a_km = false) {
  const bool kind_ok =
      (path != TDM_PATH_VALU || (kind == TDM_KIND_F32 && !b_nk && !a_km)) &&
      (path != TDM_PATH_SKINNY || kind == TDM_KIND_BF16_F32ACC);
  if (!kind_ok) return false;
  if (M == 0 || N == 0 || K == 0) return true;  // nothing to run, or a zero fill
  switch (path) {
    case TDM_PATH_AUTO:
    case TDM_PATH_EDGE:
      return true;
    case TDM_PATH_VALU:
      return kind == TDM_KIND_F32 && tdm::valu_f32_supports(M, N, K, ma, mb, mc);
    case TDM_PATH_MFMA:
      if (kind == TDM_KIND_F32) return tdm::mfma_f32_supports(M, N, K, ma, mb, mc, b_nk, a_km);
      if (a_km) return tdm::mfma_bf16_akm_supports(M, N, K, b_nk, ma, mb, mc);
      return b_nk ? tdm::mfma_bf16_nk_supports(M, N, K, ma, mb, mc)
                  : tdm::mfma_bf16_supports(M, N, K, ma, mb, mc);
    case TDM_PATH_SKINNY:
      // the streaming kernels read A as M x K rows (M <= 16)
      if (kind != TDM_KIND_BF16_F32ACC || a_km) return false;
      return b_nk ? tdm::skinny_bf16_nk_supports(M, N, K, ma, mb, mc)
                  : tdm::skinny_bf16_supports(M, N, K, ma, mb, mc);
  }
  return false;
}

// Dispatcher: compare the product's intensity with the ridge point of the
// unit that would run it (CS336 Lecture 5 GPU notes, §2.2). Below the ridge a
// small-M bf16 product is memory-bound and goes to the streaming path; above
// it the compute paths are used.
tdm_path choose(tdm_kind kind, int64_t M, int64_t N, int64_t K, int ma, int mb, int mc,
                bool b_nk = false, bool a_km = false) {
  if (M <= 0 || N <= 0 || K <= 0) return TDM_PATH_EDGE;
  const double flops = 2.0 * M * N * K;
  const double in = kind == TDM_KIND_F32 ? 4.0 : 2.0;
  const double bytes = (double(M) * K + double(K) * N) * in + double(M) * N * 4.0;
  const double intensity = flops / bytes;
  if (kind == TDM_KIND_BF16_F32ACC) {
    const double ridge = kPeakMfmaBf16 / kHbmBandwidth;
    if (intensity < ridge && supports(kind, TDM_PATH_SKINNY, M, N, K, ma, mb, mc, b_nk, a_km))
      return TDM_PATH_SKINNY;
    if (supports(kind, TDM_PATH_MFMA, M, N, K, ma, mb, mc, b_nk, a_km)) return TDM_PATH_MFMA;
    return TDM_PATH_EDGE;
  }
  // fp32 has no streaming path; the choice is about filling the CUs. With
  // fewer than 16 tiles of 128 x 128 the 32 x 32 tiles of the edge kernel
  // spread further. Otherwise the matrix cores, which outran the vector ALUs
  // at every measured size; the VALU kernel takes what they cannot.
  const int64_t tiles128 = ((M + 127) / 128) * ((N + 127) / 128);
  if (tiles128 < 16) return TDM_PATH_EDGE;
  if (supports(kind, TDM_PATH_MFMA, M, N, K, ma, mb, mc, b_nk, a_km)) return TDM_PATH_MFMA;
  if (supports(kind, TDM_PATH_VALU, M, N, K, ma, mb, mc, b_nk, a_km)) return TDM_PATH_VALU;
  return TDM_PATH_EDGE;
}

tdm_status to_status(hipError_t e) { return e == hipSuccess ? TDM_SUCCESS : TDM_ERROR_LAUNCH; }

template <typename T>
tdm_status validate(const T* A, const T* B, const float* C, int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K < 0) return TDM_ERROR_INVALID_VALUE;
  if (M == 0 || N == 0) return TDM_SUCCESS;
  if (C == nullptr) return TDM_ERROR_INVALID_VALUE;
  if (K > 0 && (A == nullptr || B == nullptr)) return TDM_ERROR_INVALID_VALUE;
  if ((reinterpret_cast<uintptr_t>(C) % alignof(float)) != 0) return TDM_ERROR_INVALID_VALUE;
  if (K > 0 && ((reinterpret_cast<uintptr_t>(A) % alignof(T)) != 0 ||
                (reinterpret_cast<uintptr_t>(B) % alignof(T)) != 0))
    return TDM_ERROR_INVALID_VALUE;
  if (too_big(M, N, K)) return TDM_ERROR_NOT_SUPPORTED;
  if (K > 0) {  // C is written while A and B are read: it may share no byte with them
    const uint64_t c_bytes = uint64_t(M) * uint64_t(N) * sizeof(float);
    if (overlaps(C, c_bytes, A, uint64_t(M) * uint64_t(K) * sizeof(T)) ||
        overlaps(C, c_bytes, B, uint64_t(K) * uint64_t(N) * sizeof(T)))
      return TDM_ERROR_INVALID_VALUE;
  }
  return TDM_SUCCESS;
}

// layout: how A and B are stored (tdm_layout, checked by the caller).
tdm_status run_f32(const float* A, const float* B, int layout, float* C, int64_t M, int64_t N,
                   int64_t K, tdm_path path, void* stream) {
  tdm_status st = validate(A, B, C, M, N, K);
  if (st != TDM_SUCCESS || M == 0 || N == 0) return st;
  const bool b_nk = (layout & TDM_LAYOUT_NK) != 0, a_km = (layout & TDM_LAYOUT_KM_KN) != 0;
  const int ma = misalign(A), mb = misalign(B), mc = misalign(C);
  if (path != TDM_PATH_AUTO && !supports(TDM_KIND_F32, path, M, N, K, ma, mb, mc, b_nk, a_km))
    return TDM_ERROR_NOT_SUPPORTED;
  if ((st = check_device()) != TDM_SUCCESS) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (K == 0) return to_status(tdm::launch_fill_zero_f32(C, M * N, s));  // empty sum
  if (path == TDM_PATH_AUTO) path = choose(TDM_KIND_F32, M, N, K, ma, mb, mc, b_nk, a_km);
  const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
  switch (path) {
    case TDM_PATH_VALU: return to_status(tdm::launch_valu_f32(A, B, C, m, n, k, s));
    case TDM_PATH_MFMA:
      return to_status(tdm::launch_mfma_f32_layout(A, B, b_nk, a_km, C, m, n, k, s));
    default:
      if (!b_nk && !a_km) return to_status(tdm::launch_edge_f32(A, B, C, m, n, k, s));
      return to_status(tdm::launch_edge_f32_layout(A, B, b_nk, a_km, C, m, n, k, s));
  }
}

tdm_status run_bf16(const uint16_t* A, const uint16_t* B, float* C, int64_t M,
                    int64_t N, int64_t K, tdm_path path, void* stream) {
  tdm_status st = validate(A, B, C, M, N, K);
  if (st != TDM_SUCCESS || M == 0 || N == 0) return st;
  const int ma = misalign(A), mb = misalign(B), mc = misalign(C);
  if (path != TDM_PATH_AUTO && !supports(TDM_KIND_BF16_F32ACC, path, M, N, K, ma, mb, mc))
    return TDM_ERROR_NOT_SUPPORTED;
  if ((st = check_device()) != TDM_SUCCESS) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (K == 0) return to_status(tdm::launch_fill_zero_f32(C, M * N, s));  // empty sum
  if (path == TDM_PATH_AUTO) path = choose(TDM_KIND_BF16_F32ACC, M, N, K, ma, mb, mc);
  const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
  switch (path) {
    case TDM_PATH_MFMA: return to_status(tdm::launch_mfma_bf16(A, B, C, m, n, k, s));
    case TDM_PATH_SKINNY: return to_status(tdm::launch_skinny_bf16(A, B, C, m, n, k, s));
    default: return to_status(tdm::launch_edge_bf16(A, B, C, m, n, k, s));
  }
}

bool valid_path(int p) { return p >= TDM_PATH_AUTO && p <= TDM_PATH_SKINNY; }
bool valid_layout(int l) { return l >= TDM_LAYOUT_KN && l <= TDM_LAYOUT_KM_NK; }

// D = epilogue(op(A) * op(B)) for bf16 inputs (include/tdm.h).
tdm_status run_bf16_epi(const uint16_t* A, const uint16_t* B, tdm_layout layout, void* D,
                        tdm_dtype d_type, const void* bias, const void* residual, int gelu,
                        int64_t M, int64_t N, int64_t K, tdm_path path, void* stream,
                        bool shared_scratch = false) {
  if (d_type != TDM_DTYPE_F32 && d_type != TDM_DTYPE_BF16) return TDM_ERROR_INVALID_VALUE;
  if (!valid_layout(layout)) return TDM_ERROR_INVALID_VALUE;
  const bool b_nk = (layout & TDM_LAYOUT_NK) != 0, a_km = (layout & TDM_LAYOUT_KM_KN) != 0;
  const uint64_t dsize = d_type == TDM_DTYPE_BF16 ? 2 : 4;
  if (M < 0 || N < 0 || K < 0) return TDM_ERROR_INVALID_VALUE;
  if (M == 0 || N == 0) return TDM_SUCCESS;
  if (D == nullptr) return TDM_ERROR_INVALID_VALUE;
  if (K > 0 && (A == nullptr || B == nullptr)) return TDM_ERROR_INVALID_VALUE;
  auto aligned = [](const void* p, uint64_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; };
  if (!aligned(D, dsize) || !aligned(bias, dsize) || !aligned(residual, dsize))
    return TDM_ERROR_INVALID_VALUE;
  if (K > 0 && (!aligned(A, 2) || !aligned(B, 2))) return TDM_ERROR_INVALID_VALUE;
  if (too_big(M, N, K)) return TDM_ERROR_NOT_SUPPORTED;
  const uint64_t d_bytes = uint64_t(M) * uint64_t(N) * dsize;
  if (K > 0 && (overlaps(D, d_bytes, A, uint64_t(M) * uint64_t(K) * 2) ||
                overlaps(D, d_bytes, B, uint64_t(K) * uint64_t(N) * 2)))
    return TDM_ERROR_INVALID_VALUE;
  if (bias != nullptr && overlaps(D, d_bytes, bias, uint64_t(N) * dsize))
    return TDM_ERROR_INVALID_VALUE;
  if (residual != nullptr && residual != D && overlaps(D, d_bytes, residual, d_bytes))
    return TDM_ERROR_INVALID_VALUE;
  const int ma = misalign(A), mb = misalign(B);
  if (path != TDM_PATH_AUTO &&
      !supports(TDM_KIND_BF16_F32ACC, path, M, N, K, ma, mb, 0, b_nk, a_km))
    return TDM_ERROR_NOT_SUPPORTED;
  tdm_status st = check_device();
  if (st != TDM_SUCCESS) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  tdm::Epilogue e;
  e.bias = bias;
  e.residual = residual;
  e.gelu = gelu != 0;
  e.d_bf16 = d_type == TDM_DTYPE_BF16;
  const int m = static_cast<int>(M), n = static_cast<int>(N), k = static_cast<int>(K);
  if (K == 0) return to_status(tdm::launch_edge_bf16_epi(A, B, b_nk, a_km, D, m, n, 0, e, s));
  if (path == TDM_PATH_AUTO)
    path = choose(TDM_KIND_BF16_F32ACC, M, N, K, ma, mb, 0, b_nk, a_km);
  switch (path) {
    case TDM_PATH_MFMA:
      return to_status(tdm::launch_mfma_bf16_epi(A, B, b_nk, a_km, D, m, n, k, e, s));
    case TDM_PATH_SKINNY:
      return to_status(
          tdm::launch_skinny_bf16_epi(A, B, b_nk, D, m, n, k, e, s, shared_scratch));
    default: return to_status(tdm::launch_edge_bf16_epi(A, B, b_nk, a_km, D, m, n, k, e, s));
  }
}

tdm_status run_fp8(const uint8_t* A, tdm_fp8_format a_format, const uint8_t* a_scale,
                   const uint8_t* B, tdm_fp8_format b_format, const uint8_t* b_scale, void* D,
                   tdm_dtype d_type, const void* bias, const void* residual, int gelu, int64_t M,
                   int64_t N, int64_t K, void* stream) {
  auto valid_fmt = [](tdm_fp8_format f) { return f == TDM_FP8_E4M3 || f == TDM_FP8_E5M2; };
  if (!valid_fmt(a_format) || !valid_fmt(b_format)) return TDM_ERROR_INVALID_VALUE;
  if (d_type != TDM_DTYPE_F32 && d_type != TDM_DTYPE_BF16) return TDM_ERROR_INVALID_VALUE;
  if (M < 0 || N < 0 || K < 0) return TDM_ERROR_INVALID_VALUE;
  if ((a_scale == nullptr) != (b_scale == nullptr)) return TDM_ERROR_INVALID_VALUE;
  if (M == 0 || N == 0) return TDM_SUCCESS;
  if (D == nullptr) return TDM_ERROR_INVALID_VALUE;
  if (K > 0 && (A == nullptr || B == nullptr)) return TDM_ERROR_INVALID_VALUE;
  const uint64_t dsize = d_type == TDM_DTYPE_BF16 ? 2 : 4;
  auto aligned = [](const void* p, uint64_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; };
  if (!aligned(D, dsize) || !aligned(bias, dsize) || !aligned(residual, dsize))
    return TDM_ERROR_INVALID_VALUE;
  if (too_big(M, N, K)) return TDM_ERROR_NOT_SUPPORTED;
  const int ma = K > 0 ? misalign(A) : 0, mb = K > 0 ? misalign(B) : 0;
  if (!tdm::mfma_fp8_supports(M, N, K, ma, mb)) return TDM_ERROR_NOT_SUPPORTED;
  const uint64_t d_bytes = uint64_t(M) * uint64_t(N) * dsize;
  const uint64_t a_bytes = uint64_t(M) * uint64_t(K), b_bytes = uint64_t(N) * uint64_t(K);
  if (K > 0 && (overlaps(D, d_bytes, A, a_bytes) || overlaps(D, d_bytes, B, b_bytes)))
    return TDM_ERROR_INVALID_VALUE;
  if (K > 0 && a_scale != nullptr &&
      (overlaps(D, d_bytes, a_scale, a_bytes / 32) || overlaps(D, d_bytes, b_scale, b_bytes / 32)))
    return TDM_ERROR_INVALID_VALUE;
  if (bias != nullptr && overlaps(D, d_bytes, bias, uint64_t(N) * dsize))
    return TDM_ERROR_INVALID_VALUE;
  if (residual != nullptr && residual != D && overlaps(D, d_bytes, residual, d_bytes))
    return TDM_ERROR_INVALID_VALUE;
  tdm_status st = check_device();
  if (st != TDM_SUCCESS) return st;
  tdm::Epilogue e;
  e.bias = bias;
  e.residual = residual;
  e.gelu = gelu != 0;
  e.d_bf16 = d_type == TDM_DTYPE_BF16;
  const bool scaled = K > 0 && a_scale != nullptr;
  return to_status(tdm::launch_mfma_fp8(A, static_cast<int>(a_format), B,
                                        static_cast<int>(b_format), scaled ? a_scale : nullptr,
                                        scaled ? b_scale : nullptr, D, static_cast<int>(M),
                                        static_cast<int>(N), static_cast<int>(K), e,
                                        static_cast<hipStream_t>(stream)));
}

tdm_status run_attention(const uint16_t* Q, const uint16_t* K, const uint16_t* V, uint16_t* O,
                         float* lse, int64_t bh, int64_t n_q, int64_t n_kv, int64_t d,
                         float scale, int causal, void* stream) {
  if (bh < 0 || n_q < 0 || n_kv < 0 || d < 0) return TDM_ERROR_INVALID_VALUE;
  if (!(scale == scale) || scale - scale != 0.0f) return TDM_ERROR_INVALID_VALUE;  // NaN or inf
  if (causal != 0 && n_q != n_kv) return TDM_ERROR_INVALID_VALUE;
  if (bh == 0 || n_q == 0) return TDM_SUCCESS;
  if (n_kv == 0) return TDM_ERROR_INVALID_VALUE;
  if (Q == nullptr || K == nullptr || V == nullptr || O == nullptr) return TDM_ERROR_INVALID_VALUE;
  auto aligned = [](const void* p, uint64_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; };
  if (!aligned(O, 8) || !aligned(lse, 4)) return TDM_ERROR_INVALID_VALUE;
  if (!tdm::attention_supports(d)) return TDM_ERROR_NOT_SUPPORTED;
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16)) return TDM_ERROR_NOT_SUPPORTED;
  if (bh > 65535 || n_q >= (int64_t{1} << 22) || n_kv >= (int64_t{1} << 22))
    return TDM_ERROR_NOT_SUPPORTED;
  const uint64_t o_bytes = uint64_t(bh) * uint64_t(n_q) * uint64_t(d) * 2;
  const uint64_t kv_bytes = uint64_t(bh) * uint64_t(n_kv) * uint64_t(d) * 2;
  const uint64_t lse_bytes = uint64_t(bh) * uint64_t(n_q) * 4;
  if (overlaps(O, o_bytes, Q, o_bytes) || overlaps(O, o_bytes, K, kv_bytes) ||
      overlaps(O, o_bytes, V, kv_bytes) ||
      (lse != nullptr && overlaps(O, o_bytes, lse, lse_bytes)))
    return TDM_ERROR_INVALID_VALUE;
  // lse is written while other workgroups still read Q, K and V.
  if (lse != nullptr && (overlaps(lse, lse_bytes, Q, o_bytes) ||
                         overlaps(lse, lse_bytes, K, kv_bytes) ||
                         overlaps(lse, lse_bytes, V, kv_bytes)))
    return TDM_ERROR_INVALID_VALUE;
  tdm_status st = check_device();
  if (st != TDM_SUCCESS) return st;
  return to_status(tdm::launch_attention_fwd(Q, K, V, O, lse, static_cast<int>(bh),
                                             static_cast<int>(n_q), static_cast<int>(n_kv),
                                             static_cast<int>(d), scale, causal,
                                             static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

tdm_status attention_fwd(const uint16_t* Q, const uint16_t* K, const uint16_t* V, uint16_t* O,
                         float* lse, int64_t batch_heads, int64_t n_q, int64_t n_kv,
                         int64_t head_dim, float scale, int causal, void* stream) {
  return run_attention(Q, K, V, O, lse, batch_heads, n_q, n_kv, head_dim, scale, causal, stream);
}

tdm_status gemm_fp8(const uint8_t* A, tdm_fp8_format a_format, const uint8_t* a_scale,
                    const uint8_t* B, tdm_fp8_format b_format, const uint8_t* b_scale, void* D,
                    tdm_dtype d_type, const void* bias, const void* residual, int gelu, int64_t M,
                    int64_t N, int64_t K, void* stream) {
  if (!valid_fp8(raw(a_format)) || !valid_fp8(raw(b_format)) || !valid_dtype(raw(d_type)))
    return TDM_ERROR_INVALID_VALUE;
  return run_fp8(A, a_format, a_scale, B, b_format, b_scale, D, d_type, bias, residual, gelu, M,
                 N, K, stream);
}

int tdm_fp8_supports(int64_t M, int64_t N, int64_t K, int misalign_a, int misalign_b) {
  if (M < 0 || N < 0 || K < 0 || too_big(M, N, K)) return 0;
  return tdm::mfma_fp8_supports(M, N, K, misalign_a, misalign_b) ? 1 : 0;
}

tdm_status gemm_f32(const float* A, const float* B, float* C, int64_t M, int64_t N,
                    int64_t K, void* stream) {
  return run_f32(A, B, TDM_LAYOUT_KN, C, M, N, K, TDM_PATH_AUTO, stream);
}

tdm_status gemm_bf16_f32acc(const uint16_t* A, const uint16_t* B, float* C, int64_t M,
                            int64_t N, int64_t K, void* stream) {
  return run_bf16(A, B, C, M, N, K, TDM_PATH_AUTO, stream);
}

tdm_status tdm_gemm_f32_path(const float* A, const float* B, float* C, int64_t M,
                             int64_t N, int64_t K, tdm_path path, void* stream) {
  if (!valid_path(raw(path))) return TDM_ERROR_INVALID_VALUE;
  return run_f32(A, B, TDM_LAYOUT_KN, C, M, N, K, path, stream);
}

tdm_status gemm_f32_ex(const float* A, const float* B, tdm_layout layout, float* C, int64_t M,
                       int64_t N, int64_t K, void* stream) {
  if (!valid_layout(raw(layout))) return TDM_ERROR_INVALID_VALUE;
  return run_f32(A, B, raw(layout), C, M, N, K, TDM_PATH_AUTO, stream);
}

tdm_status tdm_gemm_f32_ex_path(const float* A, const float* B, tdm_layout layout, float* C,
                                int64_t M, int64_t N, int64_t K, tdm_path path, void* stream) {
  if (!valid_path(raw(path)) || !valid_layout(raw(layout))) return TDM_ERROR_INVALID_VALUE;
  return run_f32(A, B, raw(layout), C, M, N, K, path, stream);
}

tdm_status tdm_gemm_bf16_f32acc_path(const uint16_t* A, const uint16_t* B, float* C,
                                     int64_t M, int64_t N, int64_t K, tdm_path path,
                                     void* stream) {
  if (!valid_path(raw(path))) return TDM_ERROR_INVALID_VALUE;
  return run_bf16(A, B, C, M, N, K, path, stream);
}

tdm_status gemm_bf16_epilogue(const uint16_t* A, const uint16_t* B, void* D, tdm_dtype d_type,
                              const void* bias, const void* residual, int gelu, int64_t M,
                              int64_t N, int64_t K, void* stream) {
  if (!valid_dtype(raw(d_type))) return TDM_ERROR_INVALID_VALUE;
  return run_bf16_epi(A, B, TDM_LAYOUT_KN, D, d_type, bias, residual, gelu, M, N, K,
                      TDM_PATH_AUTO, stream);
}

tdm_status tdm_gemm_bf16_epilogue_path(const uint16_t* A, const uint16_t* B, void* D,
                                       tdm_dtype d_type, const void* bias, const void* residual,
                                       int gelu, int64_t M, int64_t N, int64_t K, tdm_path path,
                                       void* stream) {
  if (!valid_path(raw(path)) || !valid_dtype(raw(d_type))) return TDM_ERROR_INVALID_VALUE;
  return run_bf16_epi(A, B, TDM_LAYOUT_KN, D, d_type, bias, residual, gelu, M, N, K, path,
                      stream);
}

tdm_status gemm_bf16_ex(const uint16_t* A, const uint16_t* B, tdm_layout layout, void* D,
                        tdm_dtype d_type, const void* bias, const void* residual, int gelu,
                        int64_t M, int64_t N, int64_t K, void* stream) {
  if (!valid_layout(raw(layout)) || !valid_dtype(raw(d_type))) return TDM_ERROR_INVALID_VALUE;
  return run_bf16_epi(A, B, layout, D, d_type, bias, residual, gelu, M, N, K, TDM_PATH_AUTO,
                      stream);
}

tdm_status gemm_bf16_ex_noalloc(const uint16_t* A, const uint16_t* B, tdm_layout layout,
                                void* D, tdm_dtype d_type, const void* bias, const void* residual,
                                int gelu, int64_t M, int64_t N, int64_t K, void* stream) {
  if (!valid_layout(raw(layout)) || !valid_dtype(raw(d_type))) return TDM_ERROR_INVALID_VALUE;
  return run_bf16_epi(A, B, layout, D, d_type, bias, residual, gelu, M, N, K, TDM_PATH_AUTO,
                      stream, true);
}

tdm_status tdm_gemm_bf16_ex_path(const uint16_t* A, const uint16_t* B, tdm_layout layout,
                                 void* D, tdm_dtype d_type, const void* bias,
                                 const void* residual, int gelu, int64_t M, int64_t N,
                                 int64_t K, tdm_path path, void* stream) {
  if (!valid_path(raw(path)) || !valid_layout(raw(layout)) || !valid_dtype(raw(d_type)))
    return TDM_ERROR_INVALID_VALUE;
  return run_bf16_epi(A, B, layout, D, d_type, bias, residual, gelu, M, N, K, path, stream);
}

tdm_status gemm_roofline(tdm_kind kind, int64_t M, int64_t N, int64_t K, tdm_roofline* out) {
  if (out == nullptr || M < 0 || N < 0 || K < 0) return TDM_ERROR_INVALID_VALUE;
  if (!valid_kind(raw(kind))) return TDM_ERROR_INVALID_VALUE;
  double in_size;
  switch (kind) {
    case TDM_KIND_F32: in_size = 4.0; break;
    case TDM_KIND_BF16_F32ACC: in_size = 2.0; break;
    default: return TDM_ERROR_INVALID_VALUE;
  }
  const double m = double(M), n = double(N), k = double(K);
  out->flops = 2.0 * m * n * k;
  out->bytes = (m * k + k * n) * in_size + m * n * 4.0;
  out->intensity = out->bytes > 0.0 ? out->flops / out->bytes : 0.0;
  return TDM_SUCCESS;
}

const char* tdm_status_string(tdm_status s) {
  switch (raw(s)) {
    case TDM_SUCCESS: return "success";
    case TDM_ERROR_INVALID_VALUE: return "invalid value";
    case TDM_ERROR_NOT_SUPPORTED: return "not supported";
    case TDM_ERROR_NO_DEVICE: return "no HIP device";
    case TDM_ERROR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

int tdm_path_supports(tdm_kind kind, tdm_path path, int64_t M, int64_t N, int64_t K,
                      int misalign_a, int misalign_b, int misalign_c) {
  if (!valid_kind(raw(kind))) return 0;
  if (!valid_path(raw(path)) || M < 0 || N < 0 || K < 0 || too_big(M, N, K)) return 0;
  return supports(kind, path, M, N, K, misalign_a, misalign_b, misalign_c) ? 1 : 0;
}

tdm_path tdm_select_path(tdm_kind kind, int64_t M, int64_t N, int64_t K) {
  if (!valid_kind(raw(kind))) return TDM_PATH_EDGE;
  return choose(kind, M, N, K, 0, 0, 0);
}

int tdm_path_supports_ex(tdm_kind kind, tdm_layout layout, tdm_path path, int64_t M,
                         int64_t N, int64_t K, int misalign_a, int misalign_b, int misalign_c) {
  if (!valid_layout(raw(layout)) || !valid_kind(raw(kind))) return 0;
  if (!valid_path(raw(path)) || M < 0 || N < 0 || K < 0 || too_big(M, N, K)) return 0;
  return supports(kind, path, M, N, K, misalign_a, misalign_b, misalign_c,
                  (layout & TDM_LAYOUT_NK) != 0, (layout & TDM_LAYOUT_KM_KN) != 0) ? 1 : 0;
}

tdm_path tdm_select_path_ex(tdm_kind kind, tdm_layout layout, int64_t M, int64_t N,
                            int64_t K) {
  if (!valid_kind(raw(kind)) || !valid_layout(raw(layout))) return TDM_PATH_EDGE;
  return choose(kind, M, N, K, 0, 0, 0, (layout & TDM_LAYOUT_NK) != 0,
                (layout & TDM_LAYOUT_KM_KN) != 0);
}

const char* tdm_path_name(tdm_path p) {
  switch (raw(p)) {
    case TDM_PATH_AUTO: return "auto";
    case TDM_PATH_EDGE: return "edge";
    case TDM_PATH_VALU: return "valu";
    case TDM_PATH_MFMA: return "mfma";
    case TDM_PATH_SKINNY: return "skinny";
  }
  return "unknown";
}

int tdm_version(void) { return TDM_VERSION; }

}  // extern "C"

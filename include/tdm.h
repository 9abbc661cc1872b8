/*
 * tdm.h -- tiled dense matrix multiply for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libtdm.so. Plain pointers and sizes only.
 *
 * The operation is the dense matrix product C = A * B with
 *   C[i,j] = sum_{k < K} A[i,k] * B[k,j],   0 <= i < M, 0 <= j < N,
 * as defined in "09 计算受限还是访存受限" (compute- vs memory-bound lesson),
 * section on counting a matrix multiply, and in the CS336 Lecture 5 GPU
 * notes, §4.2 (C = AB for an M x K by K x N product).
 *
 * Layout contract (all GEMM entry points):
 *   - A is M x K, B is K x N, C is M x N, all row-major and dense: element
 *     (r, c) of an R x S matrix lives at base + r*S + c (CS336 Lecture 5 GPU
 *     notes, §4.1, on row-major storage). There are no leading dimensions;
 *     a strided or transposed view must be made contiguous by the caller.
 *   - A, B and C are DEVICE pointers on the current HIP device, owned by the
 *     caller. No call allocates memory or waits for the device. The small-M
 *     path (M <= 16, B K x N) splits K over workgroups and adds their
 *     partial sums in a second kernel; the partial sums live in static
 *     device memory of the library (8 buffers of 4 MB per device, present
 *     from its first use until the process ends). The first eight streams
 *     that run that path on a device each own one buffer, so calls on
 *     different streams never share one; on any further stream the call
 *     runs the matrix-core kernel instead (the same product, summed in
 *     another order).
 *   - A and B are read only. C is overwritten (there is no alpha/beta). C
 *     must not overlap A or B.
 *   - Element sizes: fp32 = 4 bytes; bf16 = 2 bytes passed as raw uint16_t
 *     bits (the upper half of an IEEE fp32 word, CS336 Lecture 5 GPU notes,
 *     §3.1). Pointers must be aligned to their element size.
 *
 * Execution: every GEMM call is asynchronous on `stream` (a hipStream_t;
 * NULL means the default stream) and returns once the work is enqueued.
 * Faults during execution surface at the caller's next synchronization.
 *
 * Errors: arguments are validated on the host before any HIP call.
 *   - NULL pointer (with M*N > 0 and, for A/B, K > 0), negative size, a
 *     misaligned pointer, or C's bytes overlapping A's or B's (with
 *     M*N*K > 0)                                        -> TDM_ERROR_INVALID_VALUE
 *   - a matrix with 2^31 or more elements, or a forced path that cannot run
 *     the given shape/alignment                         -> TDM_ERROR_NOT_SUPPORTED
 *   - no HIP device is visible                          -> TDM_ERROR_NO_DEVICE
 *   - a HIP call failed (kernel launch, the address of the small-M path's
 *     buffers or the kernels' LDS attribute)             -> TDM_ERROR_LAUNCH
 *   - M == 0 or N == 0: nothing to do, TDM_SUCCESS without any HIP call.
 *   - K == 0: C is filled with zeros (the empty sum), TDM_SUCCESS.
 *
 * Threading: the calls may be made from several host threads; work on one
 * stream is ordered as usual. The only mutable global state is the small-M
 * path's table of which stream owns which buffer (guarded by a mutex) and a
 * per-device record of the kernels' LDS attribute. A graph captured from a
 * stream keeps using that stream's buffer when replayed: do not replay it
 * concurrently with other small-M work on the stream it was captured from.
 */
#ifndef TDM_H
#define TDM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TDM_VERSION 1

/* Symbols of the C ABI are the only ones libtdm.so exports. */
#if defined(__GNUC__) || defined(__clang__)
#define TDM_API __attribute__((visibility("default")))
#else
#define TDM_API
#endif

typedef enum tdm_status {
  TDM_SUCCESS = 0,
  TDM_ERROR_INVALID_VALUE = 1,
  TDM_ERROR_NOT_SUPPORTED = 2,
  TDM_ERROR_NO_DEVICE = 3,
  TDM_ERROR_LAUNCH = 4
} tdm_status;

/* Which product a roofline query describes. */
typedef enum tdm_kind {
  TDM_KIND_F32 = 0,          /* fp32 in, fp32 accumulate, fp32 out         */
  TDM_KIND_BF16_F32ACC = 1   /* bf16 in, fp32 accumulate, fp32 out         */
} tdm_kind;

/* Kernel families behind the GEMM calls. */
typedef enum tdm_path {
  TDM_PATH_AUTO = 0,   /* let the dispatcher choose (what gemm_* do)        */
  TDM_PATH_EDGE = 1,   /* LDS-tiled kernels for any shape and alignment      */
  TDM_PATH_VALU = 2,   /* fp32 only: register- and LDS-tiled vector FMA      */
  TDM_PATH_MFMA = 3,   /* matrix cores: bf16 or fp32 in, fp32 accumulate     */
  TDM_PATH_SKINNY = 4  /* bf16 only, M <= 16: streams B once at HBM rate     */
} tdm_path;

/* Cost of one call with every matrix crossing HBM exactly once. */
typedef struct tdm_roofline {
  double flops;      /* 2*M*N*K                                             */
  double bytes;      /* (M*K + K*N)*in_size + M*N*4                         */
  double intensity;  /* flops / bytes (0 when bytes == 0)                   */
} tdm_roofline;

/* C = A * B in fp32: fp32 inputs, fp32 accumulation, fp32 output.
 * Definition: compute- vs memory-bound lesson, counting a matrix multiply. */
TDM_API tdm_status gemm_f32(const float* A, const float* B, float* C, int64_t M,
                    int64_t N, int64_t K, void* stream);

/* C = A * B with bf16 inputs (uint16_t bits), fp32 accumulation and fp32
 * output: the mixed-precision scheme of the CS336 Lecture 5 GPU notes, §3.2
 * (low-precision matrix products, fp32 accumulation). Each product of two
 * bf16 values is exact in fp32; only the sums round. */
TDM_API tdm_status gemm_bf16_f32acc(const uint16_t* A, const uint16_t* B, float* C,
                            int64_t M, int64_t N, int64_t K, void* stream);

/* Element type of an epilogue's output D, bias and residual. */
typedef enum tdm_dtype {
  TDM_DTYPE_F32 = 0,  /* 4-byte IEEE float                                   */
  TDM_DTYPE_BF16 = 1  /* bf16 as raw uint16_t bits                            */
} tdm_dtype;

/* D = epilogue(A * B): the bf16 product of gemm_bf16_f32acc, finished in
 * the kernel that computes it (fused: the fp32 sums never reach memory), as
 * in the operator-fusion section of the CS336 Lecture 5 GPU notes (§4.3) and
 * the GELU + residual example of LLM course ch. 15. Per output element, in
 * fp32:
 *   t = sum_k A[i,k] * B[k,j]                (as gemm_bf16_f32acc; 0 if K == 0)
 *   t = t + bias[j]                          if bias != NULL
 *   t = GELU(t) = t/2 * (1 + erf(t/sqrt(2))) if gelu != 0 (the exact form)
 *   t = t + residual[i,j]                    if residual != NULL
 *   D[i,j] = t, stored as d_type (bf16: rounded to nearest, ties to even)
 * D, bias (N elements) and residual (M x N, row-major) are device pointers
 * of element type d_type, aligned to it. residual may be D itself (an
 * in-place residual add); otherwise D may not overlap A, B, bias or
 * residual. Errors as for gemm_bf16_f32acc, plus TDM_ERROR_INVALID_VALUE for
 * an unknown d_type or a misaligned bias/residual. K == 0 is not a no-op:
 * D = epilogue(0). */
TDM_API tdm_status gemm_bf16_epilogue(const uint16_t* A, const uint16_t* B, void* D,
                                      tdm_dtype d_type, const void* bias, const void* residual,
                                      int gelu, int64_t M, int64_t N, int64_t K, void* stream);

/* Same, on a given path (TDM_PATH_EDGE, TDM_PATH_MFMA, TDM_PATH_SKINNY or
 * TDM_PATH_AUTO); TDM_ERROR_NOT_SUPPORTED where gemm_bf16_f32acc's path
 * would be. */
TDM_API tdm_status tdm_gemm_bf16_epilogue_path(const uint16_t* A, const uint16_t* B, void* D,
                                               tdm_dtype d_type, const void* bias,
                                               const void* residual, int gelu, int64_t M,
                                               int64_t N, int64_t K, tdm_path path,
                                               void* stream);

/* How A and B are stored (all row-major). Bit 0: B is N x K; bit 1: A is
 * K x M. */
typedef enum tdm_layout {
  TDM_LAYOUT_KN = 0,     /* A is M x K, B is K x N: C = A * B (every gemm_* call) */
  TDM_LAYOUT_NK = 1,     /* B is N x K -- a linear layer's weight, as a PyTorch
                            Linear stores it: C = A * B^T, i.e.
                            C[i,j] = sum_k A[i,k] * B[j,k]                        */
  TDM_LAYOUT_KM_KN = 2,  /* A is K x M -- the transpose of the operand, as
                            x = A.T @ B takes it: C = A^T * B, i.e.
                            C[i,j] = sum_k A[k,i] * B[k,j]                        */
  TDM_LAYOUT_KM_NK = 3   /* A is K x M and B is N x K: C = A^T * B^T, i.e.
                            C[i,j] = sum_k A[k,i] * B[j,k]                        */
} tdm_layout;

/* gemm_bf16_epilogue with A and B in any layout: D = epilogue(op(A) *
 * op(B)), op(A) = A^T when A is stored K x M, op(B) = B^T when B is stored
 * N x K (CS336 Lecture 5 GPU notes, review question 5 on x = A.T @ B and the
 * §4.1 warning on transposed views: a transposed operand is a different
 * memory layout, not a free view). M, N and K are the sizes of the product
 * C[M,N] = op(A)[M,K] * op(B)[K,N] whatever the layout. Everything else --
 * the epilogue, D, bias, residual, errors -- as gemm_bf16_epilogue;
 * TDM_ERROR_INVALID_VALUE for an unknown layout. With no bias, residual or
 * GELU and d_type TDM_DTYPE_F32 this is the plain product. The small-M
 * streaming path takes A as M x K only; an A stored K x M runs on the
 * matrix cores (M a multiple of 8, 16-byte aligned A) or the edge kernel. */
TDM_API tdm_status gemm_bf16_ex(const uint16_t* A, const uint16_t* B, tdm_layout layout,
                                void* D, tdm_dtype d_type, const void* bias,
                                const void* residual, int gelu, int64_t M, int64_t N, int64_t K,
                                void* stream);
TDM_API tdm_status tdm_gemm_bf16_ex_path(const uint16_t* A, const uint16_t* B,
                                         tdm_layout layout, void* D, tdm_dtype d_type,
                                         const void* bias, const void* residual, int gelu,
                                         int64_t M, int64_t N, int64_t K, tdm_path path,
                                         void* stream);

/* gemm_f32 with A and B in any layout: C = op(A) * op(B), op(A) = A^T when
 * A is stored K x M, op(B) = B^T when B is stored N x K (CS336 Lecture 5 GPU
 * notes, review question 5 on x = A.T @ B and the §4.1 warning on transposed
 * views: a transposed operand is a different memory layout, not a free
 * view). M, N and K are the sizes of the product C[M,N] = op(A)[M,K] *
 * op(B)[K,N] whatever the layout; C is M x N, row-major, overwritten.
 * Arguments, ownership, validation and errors as gemm_f32;
 * TDM_ERROR_INVALID_VALUE for an unknown layout. A transposed operand runs
 * on the fp32 matrix cores (K a multiple of 4, N a multiple of 4 when B is
 * K x N, M a multiple of 4 when A is K x M, 16-byte aligned A and B) or the
 * edge kernel; the vector-ALU kernel takes TDM_LAYOUT_KN only
 * (tdm_gemm_f32_ex_path with TDM_PATH_VALU and another layout:
 * TDM_ERROR_NOT_SUPPORTED). */
TDM_API tdm_status gemm_f32_ex(const float* A, const float* B, tdm_layout layout, float* C,
                               int64_t M, int64_t N, int64_t K, void* stream);
TDM_API tdm_status tdm_gemm_f32_ex_path(const float* A, const float* B, tdm_layout layout,
                                        float* C, int64_t M, int64_t N, int64_t K,
                                        tdm_path path, void* stream);

/* gemm_bf16_ex that allocates nothing and keeps no per-stream state, for
 * callers that cannot allocate device memory at call time: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Arguments, results and errors are those of gemm_bf16_ex, and so are the
 * kernels. The one difference: when the small-M path (M <= 16, B K x N)
 * splits K, its partial sums go to one static 4 MB device buffer of the
 * library per GPU (present from the first call on that GPU until the
 * process ends), shared by every call of this entry point on that GPU,
 * instead of the calling stream's own buffer. Calls of this entry point
 * that overlap in time on one GPU (several streams, or graph replays)
 * therefore race and give wrong results; calls ordered on one stream are
 * safe. No split needs more than the 4 MB (at most 256 workgroups write 16
 * x 256 fp32 sums each); the buffer needs no clearing between calls. */
TDM_API tdm_status gemm_bf16_ex_noalloc(const uint16_t* A, const uint16_t* B,
                                        tdm_layout layout, void* D, tdm_dtype d_type,
                                        const void* bias, const void* residual, int gelu,
                                        int64_t M, int64_t N, int64_t K, void* stream);

/* Host-only: tdm_path_supports / tdm_select_path for given layouts of A and
 * B (0 / TDM_PATH_EDGE for an unknown layout or kind). Layouts other than
 * TDM_LAYOUT_KN: bf16 on every path but the small-M one for an A stored
 * K x M; fp32 on the matrix cores and the edge kernel, never the vector
 * ALU. */
TDM_API int tdm_path_supports_ex(tdm_kind kind, tdm_layout layout, tdm_path path, int64_t M,
                                 int64_t N, int64_t K, int misalign_a, int misalign_b,
                                 int misalign_c);
TDM_API tdm_path tdm_select_path_ex(tdm_kind kind, tdm_layout layout, int64_t M, int64_t N,
                                    int64_t K);

/* FP8 element formats (CS336 Lecture 5 GPU notes, §3.1, table of
 * floating-point formats): 1 sign bit, then exponent and mantissa bits. */
typedef enum tdm_fp8_format {
  TDM_FP8_E4M3 = 0,  /* 4 exponent bits (bias 7), 3 mantissa bits, range +-448;
                        S.1111.111 is NaN, no infinities                      */
  TDM_FP8_E5M2 = 1   /* 5 exponent bits (bias 15), 2 mantissa bits, range
                        +-57344; IEEE-style infinities and NaNs               */
} tdm_fp8_format;

/* D = epilogue(A * B^T) for FP8 operands, with optional block scales: the
 * 8-bit formats of CS336 Lecture 5 GPU notes, §3.1 (E4M3 / E5M2, each
 * halving of the element width doubles the matrix-core peak) and the
 * fine-grained per-tile scaling that section says FP8 needs, taken here as
 * OCP Microscaling block scales along K. Per output element:
 *   t = sum_k (sa[i,k/32] * A[i,k]) * (sb[j,k/32] * B[j,k])   in fp32
 * then bias, GELU, residual and the store exactly as gemm_bf16_epilogue.
 *   A: M x K FP8 codes (uint8), row-major, format a_format;
 *   B: N x K FP8 codes, row-major -- the layout of a linear layer's weight,
 *      so C = A * B^T; format b_format;
 *   a_scale, b_scale: M x (K/32) and N x (K/32) bytes, row-major; byte e
 *      stands for the factor 2^(e-127) (e = 255: NaN) and applies to k in
 *      [32q, 32q + 32) of its row; both NULL for no scaling (factor 1);
 *   D, bias, residual: as gemm_bf16_epilogue (device, element type d_type).
 * All pointers are device pointers; the caller keeps ownership. Errors:
 * TDM_ERROR_INVALID_VALUE for a negative size, an unknown format or d_type,
 * a NULL operand (K > 0) or D, exactly one scale pointer NULL, a misaligned
 * D/bias/residual, or D overlapping an input (residual == D is allowed);
 * TDM_ERROR_NOT_SUPPORTED for K not a multiple of 32, A or B not 16-byte
 * aligned, or a matrix (A, B or D) of 2^31 elements or more. M == 0 or N ==
 * 0: nothing is done; K == 0: D = epilogue(0). */
TDM_API tdm_status gemm_fp8(const uint8_t* A, tdm_fp8_format a_format, const uint8_t* a_scale,
                            const uint8_t* B, tdm_fp8_format b_format, const uint8_t* b_scale,
                            void* D, tdm_dtype d_type, const void* bias, const void* residual,
                            int gelu, int64_t M, int64_t N, int64_t K, void* stream);

/* Host-only: 1 if gemm_fp8 runs this shape with A and B at these byte
 * offsets modulo 16, else 0. */
TDM_API int tdm_fp8_supports(int64_t M, int64_t N, int64_t K, int misalign_a, int misalign_b);

/* Attention forward: O = softmax(Q K^T * scale) V for every (batch, head),
 * computed the FlashAttention way (CS336 Lecture 5 GPU notes, §6.2: Q, K and
 * V tiled along the sequence, an online softmax keeping each row's running
 * maximum and normalizer, and the whole chain fused in one kernel, so the
 * n_q x n_kv scores never reach memory; GPU/attention notes, online
 * softmax). bf16 inputs and output, fp32 accumulation; the probabilities
 * are rounded to bf16 before they multiply V.
 *   Q: [batch_heads][n_q][head_dim], K and V: [batch_heads][n_kv][head_dim],
 *      O: [batch_heads][n_q][head_dim], all bf16 (uint16_t bits), row-major;
 *   lse: [batch_heads][n_q] fp32, the natural-log logsumexp of each row of
 *      scale * Q K^T over the visible keys (what a backward pass keeps), or
 *      NULL;
 *   scale: usually 1/sqrt(head_dim); causal != 0 masks key j > query i
 *      (requires n_q == n_kv).
 * Device pointers, owned by the caller. Errors: TDM_ERROR_INVALID_VALUE for a
 * negative size, n_kv == 0 with queries to compute, a NULL or misaligned
 * pointer (O 8-byte, lse 4-byte aligned), a non-finite scale, causal with n_q
 * != n_kv, O overlapping Q, K, V or lse, or lse overlapping Q, K or V;
 * TDM_ERROR_NOT_SUPPORTED for head_dim other than 64 or 128, Q, K or V not
 * 16-byte aligned, more than 65535 batch_heads, or a sequence of 2^22 rows or
 * more. batch_heads == 0 or n_q == 0: nothing is done. */
TDM_API tdm_status attention_fwd(const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                                 uint16_t* O, float* lse, int64_t batch_heads, int64_t n_q,
                                 int64_t n_kv, int64_t head_dim, float scale, int causal,
                                 void* stream);

/* Host-only cost query; touches no device. FLOPs = 2MNK (a multiply-add is
 * two operations) and bytes = reading A and B once and writing C once
 * (compute- vs memory-bound lesson, counting a matrix multiply; CS336
 * Lecture 5 GPU notes, §2.1). C is fp32 (4 bytes) for both kinds.
 * Errors: out == NULL, a negative size or an unknown kind ->
 * TDM_ERROR_INVALID_VALUE; products overflowing double are not checked. */
TDM_API tdm_status gemm_roofline(tdm_kind kind, int64_t M, int64_t N, int64_t K,
                         tdm_roofline* out);

/* Static, NUL-terminated description of a status code ("unknown status" for
 * values outside the enum). Never NULL. */
TDM_API const char* tdm_status_string(tdm_status s);

/* Same as gemm_f32 / gemm_bf16_f32acc, but run the given path. Returns
 * TDM_ERROR_NOT_SUPPORTED if that path cannot handle the dtype, shape or
 * alignment (see tdm_path_supports); TDM_PATH_AUTO behaves like gemm_*. */
TDM_API tdm_status tdm_gemm_f32_path(const float* A, const float* B, float* C,
                             int64_t M, int64_t N, int64_t K, tdm_path path,
                             void* stream);
TDM_API tdm_status tdm_gemm_bf16_f32acc_path(const uint16_t* A, const uint16_t* B,
                                     float* C, int64_t M, int64_t N, int64_t K,
                                     tdm_path path, void* stream);

/* Host-only: 1 if `path` can run this product with these pointer
 * alignments (pass the byte offsets of A, B and C modulo 16, or 0), else 0. */
TDM_API int tdm_path_supports(tdm_kind kind, tdm_path path, int64_t M, int64_t N,
                      int64_t K, int misalign_a, int misalign_b,
                      int misalign_c);

/* Host-only: the path gemm_* picks for this product (assuming 16-byte
 * aligned pointers). The choice compares the product's arithmetic intensity
 * with the ridge point of the target unit (CS336 Lecture 5 GPU notes, §2.2;
 * compute- vs memory-bound lesson, the quick test against the ridge). */
TDM_API tdm_path tdm_select_path(tdm_kind kind, int64_t M, int64_t N, int64_t K);

/* Static name of a path ("auto", "edge", "valu", "mfma", "skinny"). */
TDM_API const char* tdm_path_name(tdm_path p);

/* TDM_VERSION of the built library. */
TDM_API int tdm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TDM_H */

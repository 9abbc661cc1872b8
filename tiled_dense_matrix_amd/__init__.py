"""tiled_dense_matrix_amd -- tiled dense matrix multiply for AMD MI355X (gfx950).

The product C = A @ B runs in hand-written HIP kernels behind a C ABI
(include/tdm.h, built into libtdm.so). This package is the thin Python
binding over that ABI; the submodule ``inputs`` holds the seeded synthetic
input generator used by tests and the benchmark.
"""
from ._lib import (  # noqa: F401
    DType,
    Fp8Format,
    Kind,
    Layout,
    Path,
    Roofline,
    Status,
    TdmError,
    attention_fwd,
    gemm_bf16_epilogue,
    gemm_bf16_ex,
    gemm_bf16_ex_noalloc,
    gemm_bf16_f32acc,
    gemm_f32,
    gemm_f32_ex,
    gemm_fp8,
    gemm_roofline,
    load,
    path_name,
    status_string,
    tdm_gemm_bf16_epilogue_path,
    tdm_gemm_bf16_ex_path,
    tdm_gemm_bf16_f32acc_path,
    tdm_fp8_supports,
    tdm_gemm_f32_ex_path,
    tdm_gemm_f32_path,
    tdm_path_supports,
    tdm_path_supports_ex,
    tdm_select_path,
    tdm_select_path_ex,
    version,
)

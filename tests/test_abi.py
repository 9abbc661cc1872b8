"""Host-side checks of the C ABI (no GPU needed).

libtdm.so must load without a GPU, export every function include/tdm.h
declares, validate arguments before touching any device, and answer the
host-only queries (cost model, path choice) correctly.
"""
import ctypes
import os
import re

import pytest

import oracle
import tiled_dense_matrix_amd as tdm
from tiled_dense_matrix_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tdm.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"TDM_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)))


def test_header_declares_the_abi():
    names = declared_functions()
    for required in ("gemm_f32", "gemm_bf16_f32acc", "gemm_roofline", "tdm_status_string"):
        assert required in names
    assert set(names) == set(_lib.SIGNATURES), "binding and header disagree"


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_only_the_c_abi_is_exported():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert exported == set(declared_functions())


def test_version_and_strings():
    assert tdm.version() == 1
    assert tdm.status_string(0) == "success"
    assert tdm.status_string(1) == "invalid value"
    assert tdm.status_string(99) == "unknown status"
    assert [tdm.path_name(p) for p in range(5)] == ["auto", "edge", "valu", "mfma", "skinny"]
    assert tdm.path_name(42) == "unknown"


# ---------------------------------------------------------------------------
# Validation happens before any HIP call: these run identically without a GPU.
# ---------------------------------------------------------------------------

def skip_if_gpu():
    """Calls that pass validation launch kernels: with fake addresses they may
    only run where no GPU is visible (they then stop at the device check)."""
    try:
        import torch
    except ImportError:
        return
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: the call would launch on fake addresses")


# 64 KiB-aligned addresses that are never dereferenced, far enough apart that
# the fake A, B and C of these tests do not overlap (C may not overlap A or B).
FAKE = 0x10000
FAKE_B = 1 << 40
FAKE_C = 1 << 44


@pytest.mark.parametrize("fn", ["gemm_f32", "gemm_bf16_f32acc"])
def test_validation(fn):
    lib = tdm.load()
    f = getattr(lib, fn)
    S = tdm.Status
    assert f(FAKE, FAKE_B, FAKE_C, -1, 4, 4, None) == S.ERROR_INVALID_VALUE
    assert f(FAKE, FAKE_B, FAKE_C, 4, -1, 4, None) == S.ERROR_INVALID_VALUE
    assert f(FAKE, FAKE_B, FAKE_C, 4, 4, -1, None) == S.ERROR_INVALID_VALUE
    assert f(None, FAKE_B, FAKE_C, 4, 4, 4, None) == S.ERROR_INVALID_VALUE
    assert f(FAKE, None, FAKE_C, 4, 4, 4, None) == S.ERROR_INVALID_VALUE
    assert f(FAKE, FAKE_B, None, 4, 4, 4, None) == S.ERROR_INVALID_VALUE
    assert f(FAKE, FAKE_B, FAKE_C + 1, 4, 4, 4, None) == S.ERROR_INVALID_VALUE  # C misaligned
    assert f(FAKE + 1, FAKE_B, FAKE_C, 4, 4, 4, None) == S.ERROR_INVALID_VALUE  # A misaligned
    # Empty outputs are a no-op, with or without pointers and device.
    assert f(None, None, None, 0, 4, 4, None) == S.SUCCESS
    assert f(None, None, None, 4, 0, 4, None) == S.SUCCESS
    # 2^31 elements in one matrix is beyond 32-bit indexing.
    assert f(FAKE, FAKE_B, FAKE_C, 1 << 16, 1 << 15, 1, None) == S.ERROR_NOT_SUPPORTED
    assert f(FAKE, FAKE_B, FAKE_C, 1, 1 << 20, 1 << 11, None) == S.ERROR_NOT_SUPPORTED


@pytest.mark.parametrize("fn,esize", [("gemm_f32", 4), ("gemm_bf16_f32acc", 2)])
def test_output_overlapping_an_input_is_rejected(fn, esize):
    f = getattr(tdm.load(), fn)
    S = tdm.Status
    M = N = K = 64
    a_bytes, c_bytes = M * K * esize, M * N * 4
    # C starting inside A, A starting inside C, C == B, C ending on B's first byte
    assert f(FAKE, FAKE_B, FAKE + a_bytes - 16, M, N, K, None) == S.ERROR_INVALID_VALUE
    assert f(FAKE_C + 64, FAKE_B, FAKE_C, M, N, K, None) == S.ERROR_INVALID_VALUE
    assert f(FAKE, FAKE_B, FAKE_B, M, N, K, None) == S.ERROR_INVALID_VALUE
    assert f(FAKE, FAKE_B, FAKE_B - c_bytes + 4, M, N, K, None) == S.ERROR_INVALID_VALUE


@pytest.mark.parametrize("fn,esize", [("gemm_f32", 4), ("gemm_bf16_f32acc", 2)])
def test_adjacent_or_input_only_overlap_passes_validation(fn, esize):
    skip_if_gpu()
    f = getattr(tdm.load(), fn)
    S = tdm.Status
    M = N = K = 64
    a_bytes, c_bytes = M * K * esize, M * N * 4
    # Adjacent but disjoint is fine (without a GPU the call then stops at the
    # device check); A and B may overlap each other, both are only read; with
    # K == 0 nothing is read and only C matters.
    assert f(FAKE, FAKE_B, FAKE + a_bytes, M, N, K, None) == S.ERROR_NO_DEVICE
    assert f(FAKE, FAKE_B, FAKE_B - c_bytes, M, N, K, None) == S.ERROR_NO_DEVICE
    assert f(FAKE_B, FAKE_B, FAKE_C, M, N, K, None) == S.ERROR_NO_DEVICE
    assert f(FAKE_C, FAKE_C, FAKE_C, M, N, 0, None) == S.ERROR_NO_DEVICE


def test_validation_with_k_zero_needs_only_c():
    skip_if_gpu()
    lib = tdm.load()
    # K == 0: A and B may be NULL; without a GPU the call stops at the device check.
    assert lib.gemm_f32(None, None, FAKE, 3, 3, 0, None) == tdm.Status.ERROR_NO_DEVICE


def test_bad_path_and_unsupported_paths():
    lib = tdm.load()
    S, P = tdm.Status, tdm.Path
    assert lib.tdm_gemm_f32_path(FAKE, FAKE_B, FAKE_C, 4, 4, 4, 77, None) == S.ERROR_INVALID_VALUE
    # dtype/path mismatches are rejected before any device work
    assert lib.tdm_gemm_f32_path(FAKE, FAKE_B, FAKE_C, 64, 64, 62, P.MFMA, None) == S.ERROR_NOT_SUPPORTED
    assert lib.tdm_gemm_f32_path(FAKE, FAKE_B, FAKE_C, 16, 64, 64, P.SKINNY, None) == S.ERROR_NOT_SUPPORTED
    assert lib.tdm_gemm_bf16_f32acc_path(FAKE, FAKE_B, FAKE_C, 64, 64, 64, P.VALU, None) == S.ERROR_NOT_SUPPORTED
    # shape/alignment limits of the fast paths
    assert lib.tdm_gemm_bf16_f32acc_path(FAKE, FAKE_B, FAKE_C, 64, 64, 60, P.MFMA, None) == S.ERROR_NOT_SUPPORTED
    assert lib.tdm_gemm_bf16_f32acc_path(FAKE + 2, FAKE_B, FAKE_C, 64, 64, 64, P.MFMA, None) == S.ERROR_NOT_SUPPORTED
    assert lib.tdm_gemm_bf16_f32acc_path(FAKE, FAKE_B, FAKE_C, 17, 64, 64, P.SKINNY, None) == S.ERROR_NOT_SUPPORTED
    assert lib.tdm_gemm_f32_path(FAKE, FAKE_B, FAKE_C, 64, 66, 64, P.VALU, None) == S.ERROR_NOT_SUPPORTED


def test_no_device_is_reported_not_crashed():
    skip_if_gpu()
    lib = tdm.load()
    assert lib.gemm_f32(FAKE, FAKE_B, FAKE_C, 4, 4, 4, None) == tdm.Status.ERROR_NO_DEVICE
    assert lib.gemm_bf16_f32acc(FAKE, FAKE_B, FAKE_C, 4, 4, 4, None) == tdm.Status.ERROR_NO_DEVICE


# ---------------------------------------------------------------------------
# Cost model: the library's gemm_roofline against the oracle's definition and
# the pages' printed worked numbers.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K", [(4096, 4096, 4096), (256, 256, 256), (8192, 14336, 4096),
                                   (16, 8192, 8192), (1, 1, 1), (0, 5, 7), (3, 0, 0)])
def test_roofline_matches_oracle(M, N, K):
    for kind, in_bytes in ((tdm.Kind.F32, 4), (tdm.Kind.BF16_F32ACC, 2)):
        r = tdm.gemm_roofline(kind, M, N, K)
        flops, nbytes, ai = oracle.roofline(M, N, K, in_bytes, 4)
        assert r.flops == flops and r.bytes == nbytes
        assert r.intensity == pytest.approx(ai, rel=1e-15)


def test_roofline_pages_numbers():
    r = tdm.gemm_roofline(tdm.Kind.F32, 4096, 4096, 4096)
    # compute- vs memory-bound lesson, N = 4096 fp32 worked example
    assert r.flops == 137_438_953_472
    assert r.bytes == 201_326_592
    assert round(r.intensity) == 683


def test_roofline_errors():
    lib = tdm.load()
    out = _lib.Roofline()
    assert lib.gemm_roofline(0, 1, 1, 1, None) == tdm.Status.ERROR_INVALID_VALUE
    assert lib.gemm_roofline(0, -1, 1, 1, ctypes.byref(out)) == tdm.Status.ERROR_INVALID_VALUE
    assert lib.gemm_roofline(7, 1, 1, 1, ctypes.byref(out)) == tdm.Status.ERROR_INVALID_VALUE


def test_path_selection():
    K, P = tdm.Kind, tdm.Path
    assert tdm.tdm_select_path(K.BF16_F32ACC, 16, 8192, 8192) == P.SKINNY
    assert tdm.tdm_select_path(K.BF16_F32ACC, 4096, 4096, 4096) == P.MFMA
    assert tdm.tdm_select_path(K.BF16_F32ACC, 8192, 14336, 4096) == P.MFMA
    assert tdm.tdm_select_path(K.F32, 4096, 4096, 4096) == P.MFMA
    assert tdm.tdm_select_path(K.F32, 256, 256, 256) == P.EDGE   # 4 tiles of 128 x 128
    assert tdm.tdm_select_path(K.F32, 512, 512, 512) == P.MFMA   # 16 tiles
    assert tdm.tdm_select_path(K.F32, 512, 512, 510) == P.EDGE   # K % 4 != 0
    assert tdm.tdm_select_path(K.F32, 7, 5, 3) == P.EDGE
    assert tdm.tdm_select_path(K.BF16_F32ACC, 64, 64, 60) == P.EDGE  # K % 8 != 0


def test_path_supports():
    K, P = tdm.Kind, tdm.Path
    assert tdm.tdm_path_supports(K.BF16_F32ACC, P.MFMA, 300, 520, 136)
    assert not tdm.tdm_path_supports(K.BF16_F32ACC, P.MFMA, 300, 520, 136, misalign_a=2)
    assert tdm.tdm_path_supports(K.BF16_F32ACC, P.SKINNY, 16, 8192, 8192)
    assert not tdm.tdm_path_supports(K.BF16_F32ACC, P.SKINNY, 17, 8192, 8192)
    assert tdm.tdm_path_supports(K.F32, P.EDGE, 3, 5, 7, 1, 3, 5)
    assert not tdm.tdm_path_supports(K.F32, 9, 3, 5, 7)


def test_f32_mfma_copy_offset_limits():
    """The fp32 matrix-core kernel's per-lane copy offsets are 32-bit: K below
    2^22 (256 rows of A) and N below 2^25 (32 rows of B); beyond that the
    dispatcher takes the vector-ALU kernel."""
    K, P = tdm.Kind, tdm.Path
    assert tdm.tdm_path_supports(K.F32, P.MFMA, 256, 256, (1 << 22) - 4)
    assert not tdm.tdm_path_supports(K.F32, P.MFMA, 256, 256, 1 << 22)
    assert tdm.tdm_path_supports(K.F32, P.MFMA, 32, (1 << 25) - 4, 32)
    assert not tdm.tdm_path_supports(K.F32, P.MFMA, 32, 1 << 25, 32)
    # Valid matrices (under 2^31 elements) with K >= 2^22 have fewer than 16
    # tiles and go to the edge kernel anyway; a wide B can reach the limit.
    assert tdm.tdm_select_path(K.F32, 32, 1 << 25, 32) == P.VALU
    assert tdm.tdm_select_path(K.F32, 32, (1 << 25) - 4, 32) == P.MFMA


# ---------------------------------------------------------------------------
# The fused-epilogue entry points: validation before any HIP call.
# ---------------------------------------------------------------------------

FAKE_BIAS = 1 << 42
FAKE_RES = 1 << 43


def test_epilogue_validation():
    lib = tdm.load()
    f, fp = lib.gemm_bf16_epilogue, lib.tdm_gemm_bf16_epilogue_path
    S, P, D = tdm.Status, tdm.Path, tdm.DType
    M = N = K = 64
    assert f(FAKE, FAKE_B, FAKE_C, 7, None, None, 0, M, N, K, None) == S.ERROR_INVALID_VALUE
    assert f(FAKE, FAKE_B, None, D.BF16, None, None, 0, M, N, K, None) == S.ERROR_INVALID_VALUE
    assert f(FAKE, FAKE_B, FAKE_C + 2, D.F32, None, None, 0, M, N, K, None) == S.ERROR_INVALID_VALUE
    assert f(FAKE, FAKE_B, FAKE_C, D.BF16, FAKE_BIAS + 1, None, 1, M, N, K, None) == S.ERROR_INVALID_VALUE
    assert f(FAKE, FAKE_B, FAKE_C, D.F32, None, FAKE_RES + 2, 0, M, N, K, None) == S.ERROR_INVALID_VALUE
    assert f(None, FAKE_B, FAKE_C, D.BF16, None, None, 0, M, N, K, None) == S.ERROR_INVALID_VALUE
    # D may not overlap A, B or bias; residual must be D itself or disjoint from it
    assert f(FAKE, FAKE_B, FAKE + 64, D.BF16, None, None, 0, M, N, K, None) == S.ERROR_INVALID_VALUE
    assert f(FAKE, FAKE_B, FAKE_C, D.BF16, FAKE_C + 16, None, 0, M, N, K, None) == S.ERROR_INVALID_VALUE
    assert f(FAKE, FAKE_B, FAKE_C, D.BF16, None, FAKE_C + 2, 0, M, N, K, None) == S.ERROR_INVALID_VALUE
    # empty output: no-op; paths that cannot take bf16 or the shape
    assert f(None, None, None, D.F32, None, None, 1, 0, N, K, None) == S.SUCCESS
    assert fp(FAKE, FAKE_B, FAKE_C, D.BF16, None, None, 0, M, N, K, P.VALU, None) == S.ERROR_NOT_SUPPORTED
    assert fp(FAKE, FAKE_B, FAKE_C, D.BF16, None, None, 0, 17, N, K, P.SKINNY, None) == S.ERROR_NOT_SUPPORTED
    assert fp(FAKE, FAKE_B, FAKE_C, D.BF16, None, None, 0, M, N, K, 9, None) == S.ERROR_INVALID_VALUE


def test_layouts_of_a_and_b():
    """gemm_bf16_ex takes four layouts (bit 0: B stored N x K, bit 1: A
    stored K x M); another value is rejected. An A stored K x M runs on the
    matrix cores when M is a multiple of 8, never on the small-M streaming
    path, else on the edge kernel."""
    lib = tdm.load()
    S, P, D, L, K_ = tdm.Status, tdm.Path, tdm.DType, tdm.Layout, tdm.Kind.BF16_F32ACC
    f, fp = lib.gemm_bf16_ex, lib.tdm_gemm_bf16_ex_path
    for bad in (4, -1, 7):
        assert f(FAKE, FAKE_B, bad, FAKE_C, D.F32, None, None, 0, 64, 64, 64, None) == \
            S.ERROR_INVALID_VALUE
    assert fp(FAKE, FAKE_B, L.KM_KN, FAKE_C, D.F32, None, None, 0, 16, 1024, 2048, P.SKINNY,
              None) == S.ERROR_NOT_SUPPORTED
    assert fp(FAKE, FAKE_B, L.KM_KN, FAKE_C, D.F32, None, None, 0, 33, 64, 64, P.MFMA,
              None) == S.ERROR_NOT_SUPPORTED
    assert tdm.tdm_path_supports_ex(K_, L.KM_KN, P.MFMA, 256, 264, 520)
    assert tdm.tdm_path_supports_ex(K_, L.KM_NK, P.MFMA, 256, 257, 520)  # any N with B N x K
    assert not tdm.tdm_path_supports_ex(K_, L.KM_KN, P.MFMA, 256, 257, 520)
    assert not tdm.tdm_path_supports_ex(K_, L.KM_KN, P.MFMA, 33, 64, 64)
    assert not tdm.tdm_path_supports_ex(K_, L.KM_KN, P.SKINNY, 16, 1024, 2048)
    assert tdm.tdm_select_path_ex(K_, L.KM_KN, 16, 8192, 8192) == P.MFMA
    assert tdm.tdm_select_path_ex(K_, L.KM_NK, 8192, 8192, 8192) == P.MFMA
    assert tdm.tdm_select_path_ex(K_, L.KM_KN, 33, 65, 17) == P.EDGE
    assert tdm.tdm_select_path_ex(K_, L.KN, 16, 8192, 8192) == P.SKINNY


def test_f32_layouts():
    """gemm_f32_ex takes the four layouts (another value is rejected); a
    transposed operand runs on the fp32 matrix cores or the edge kernel,
    never on the vector-ALU kernel; the matrix cores want K, and N (B stored
    K x N) or M (A stored K x M), multiples of 4."""
    lib = tdm.load()
    S, P, L, F = tdm.Status, tdm.Path, tdm.Layout, tdm.Kind.F32
    f, fp = lib.gemm_f32_ex, lib.tdm_gemm_f32_ex_path
    for bad in (4, -1, 7):
        assert f(FAKE, FAKE_B, bad, FAKE_C, 64, 64, 64, None) == S.ERROR_INVALID_VALUE
        assert fp(FAKE, FAKE_B, bad, FAKE_C, 64, 64, 64, P.EDGE, None) == S.ERROR_INVALID_VALUE
    for layout in (L.NK, L.KM_KN, L.KM_NK):
        assert fp(FAKE, FAKE_B, layout, FAKE_C, 256, 256, 256, P.VALU, None) == \
            S.ERROR_NOT_SUPPORTED
        assert not tdm.tdm_path_supports_ex(F, layout, P.VALU, 4096, 4096, 4096)
        assert not tdm.tdm_path_supports_ex(F, layout, P.SKINNY, 16, 4096, 4096)
        assert tdm.tdm_path_supports_ex(F, layout, P.EDGE, 33, 65, 17)
        assert tdm.tdm_path_supports_ex(F, layout, P.MFMA, 256, 256, 256)
        assert tdm.tdm_select_path_ex(F, layout, 4096, 4096, 4096) == P.MFMA
        assert tdm.tdm_select_path_ex(F, layout, 64, 64, 64) == P.EDGE
        assert not tdm.tdm_path_supports_ex(F, layout, P.MFMA, 256, 256, 258)  # K % 4
    assert tdm.tdm_path_supports_ex(F, L.NK, P.MFMA, 256, 257, 256)      # any N, B N x K
    assert not tdm.tdm_path_supports_ex(F, L.KM_KN, P.MFMA, 256, 257, 256)
    assert tdm.tdm_path_supports_ex(F, L.NK, P.MFMA, 257, 256, 256)      # any M, A M x K
    assert not tdm.tdm_path_supports_ex(F, L.KM_NK, P.MFMA, 258, 256, 256)
    assert tdm.tdm_select_path_ex(F, L.KN, 4096, 4096, 4096) == P.MFMA
    # the plain product through the new entry point keeps gemm_f32's validation
    assert f(None, FAKE_B, L.KN, FAKE_C, 64, 64, 64, None) == S.ERROR_INVALID_VALUE
    assert f(FAKE, FAKE_B, L.NK, FAKE, 64, 64, 64, None) == S.ERROR_INVALID_VALUE  # C overlaps A


def test_epilogue_in_place_residual_and_k_zero_pass_validation():
    skip_if_gpu()
    f = tdm.load().gemm_bf16_epilogue
    S, D = tdm.Status, tdm.DType
    assert f(FAKE, FAKE_B, FAKE_C, D.BF16, FAKE_BIAS, FAKE_C, 1, 64, 64, 64, None) == S.ERROR_NO_DEVICE
    assert f(None, None, FAKE_C, D.F32, FAKE_BIAS, FAKE_RES, 1, 64, 64, 0, None) == S.ERROR_NO_DEVICE


def test_fp8_validation():
    """gemm_fp8 rejects bad arguments on the host: formats, d_type, sizes,
    null operands, one scale pointer alone, K not a multiple of 32,
    misaligned operands, overlapping outputs."""
    f = tdm.load().gemm_fp8
    S, D, F = tdm.Status, tdm.DType, tdm.Fp8Format
    E4, E5 = F.E4M3, F.E5M2
    M = N = K = 64
    ok = dict(A=FAKE, fa=E4, sa=None, B=FAKE_B, fb=E5, sb=None, D=FAKE_C, dt=D.BF16, bias=None,
              res=None, gelu=0, M=M, N=N, K=K)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["A"], a["fa"], a["sa"], a["B"], a["fb"], a["sb"], a["D"], a["dt"], a["bias"],
                 a["res"], a["gelu"], a["M"], a["N"], a["K"], None)

    assert call(fa=2) == S.ERROR_INVALID_VALUE
    assert call(fb=-1) == S.ERROR_INVALID_VALUE
    assert call(dt=5) == S.ERROR_INVALID_VALUE
    assert call(M=-1) == S.ERROR_INVALID_VALUE
    assert call(A=None) == S.ERROR_INVALID_VALUE
    assert call(D=None) == S.ERROR_INVALID_VALUE
    assert call(sa=FAKE_BIAS) == S.ERROR_INVALID_VALUE          # b_scale missing
    assert call(sb=FAKE_BIAS) == S.ERROR_INVALID_VALUE          # a_scale missing
    assert call(D=FAKE_C + 2, dt=D.F32) == S.ERROR_INVALID_VALUE
    assert call(D=FAKE + 32) == S.ERROR_INVALID_VALUE           # D overlaps A
    assert call(bias=FAKE_C + 64) == S.ERROR_INVALID_VALUE      # bias inside D
    assert call(sa=FAKE_C + 8, sb=FAKE_RES) == S.ERROR_INVALID_VALUE  # a scale inside D
    assert call(K=48) == S.ERROR_NOT_SUPPORTED                  # not a multiple of 32
    assert call(A=FAKE + 8) == S.ERROR_NOT_SUPPORTED            # A not 16-byte aligned
    assert call(M=1 << 20, K=1 << 12) == S.ERROR_NOT_SUPPORTED  # M*K = 2^32 bytes
    assert call(M=0) == S.SUCCESS and call(N=0, A=None, B=None) == S.SUCCESS
    assert tdm.tdm_fp8_supports(M, N, K) and tdm.tdm_fp8_supports(5, 7, 96)
    assert not tdm.tdm_fp8_supports(M, N, 40) and not tdm.tdm_fp8_supports(M, N, K, 8, 0)
    assert not tdm.tdm_fp8_supports((1 << 20) + 1, N, 4096)


def test_fp8_valid_calls_reach_the_device_check():
    skip_if_gpu()
    f = tdm.load().gemm_fp8
    S, D, F = tdm.Status, tdm.DType, tdm.Fp8Format
    assert f(FAKE, F.E4M3, None, FAKE_B, F.E4M3, None, FAKE_C, D.F32, None, None, 0, 64, 64, 64,
             None) == S.ERROR_NO_DEVICE
    assert f(FAKE, F.E5M2, FAKE_BIAS, FAKE_B, F.E4M3, FAKE_RES, FAKE_C, D.BF16, None, FAKE_C, 1,
             64, 64, 96, None) == S.ERROR_NO_DEVICE
    assert f(None, F.E4M3, None, None, F.E4M3, None, FAKE_C, D.BF16, FAKE_BIAS, None, 1, 8, 8, 0,
             None) == S.ERROR_NO_DEVICE


def test_attention_validation():
    """attention_fwd rejects bad arguments on the host."""
    f = tdm.load().attention_fwd
    S = tdm.Status
    nan, inf = float("nan"), float("inf")
    ok = dict(Q=FAKE, K=FAKE_B, V=FAKE_BIAS, O=FAKE_C, lse=None, bh=4, nq=128, nkv=128, d=128,
              scale=0.088, causal=0)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["Q"], a["K"], a["V"], a["O"], a["lse"], a["bh"], a["nq"], a["nkv"], a["d"],
                 a["scale"], a["causal"], None)

    assert call(bh=-1) == S.ERROR_INVALID_VALUE
    assert call(nkv=0) == S.ERROR_INVALID_VALUE
    assert call(Q=None) == S.ERROR_INVALID_VALUE and call(O=None) == S.ERROR_INVALID_VALUE
    assert call(O=FAKE_C + 4) == S.ERROR_INVALID_VALUE
    assert call(lse=FAKE_RES + 2) == S.ERROR_INVALID_VALUE
    assert call(scale=nan) == S.ERROR_INVALID_VALUE and call(scale=inf) == S.ERROR_INVALID_VALUE
    assert call(causal=1, nkv=64) == S.ERROR_INVALID_VALUE
    assert call(O=FAKE + 1024) == S.ERROR_INVALID_VALUE        # O overlaps Q
    assert call(lse=FAKE_C + 64) == S.ERROR_INVALID_VALUE      # lse inside O
    assert call(lse=FAKE + 256) == S.ERROR_INVALID_VALUE       # lse inside Q
    assert call(lse=FAKE_B + 1024) == S.ERROR_INVALID_VALUE    # lse inside K
    assert call(lse=FAKE_BIAS) == S.ERROR_INVALID_VALUE        # lse at V
    assert call(d=96) == S.ERROR_NOT_SUPPORTED
    assert call(K=FAKE_B + 8) == S.ERROR_NOT_SUPPORTED          # not 16-byte aligned
    assert call(bh=65536) == S.ERROR_NOT_SUPPORTED
    assert call(nq=1 << 22, nkv=1 << 22) == S.ERROR_NOT_SUPPORTED
    assert call(bh=0) == S.SUCCESS and call(nq=0, Q=None, O=None) == S.SUCCESS


def test_attention_valid_calls_reach_the_device_check():
    skip_if_gpu()
    f = tdm.load().attention_fwd
    S = tdm.Status
    assert f(FAKE, FAKE_B, FAKE_BIAS, FAKE_C, FAKE_RES, 2, 100, 100, 64, 0.125, 1, None) == S.ERROR_NO_DEVICE
    assert f(FAKE, FAKE_B, FAKE_BIAS, FAKE_C, None, 1, 7, 300, 128, -0.5, 0, None) == S.ERROR_NO_DEVICE

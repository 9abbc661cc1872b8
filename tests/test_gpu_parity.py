"""Parity of the HIP paths with the CPU oracle (needs an MI355X).

Every case calls the library through its C ABI (via the ctypes binding) on
seeded synthetic inputs and compares with the fp64 oracle:
  * normalized error max|C - R| / (max|A| max|B| K) within 1e-5 (fp32 inputs)
    or 4e-3 (bf16 inputs), and relative Frobenius error within 1e-5;
  * integer-valued inputs, where every partial sum is exact in fp32 under any
    summation order, must match bit for bit on every path;
  * the full workload sizes are compared element by element over the whole
    output in test_gpu_config_shapes.py.
"""
import numpy as np
import pytest

import oracle
import tiled_dense_matrix_amd as tdm
from tiled_dense_matrix_amd import inputs

from helpers import check_full, log, run, to_device

torch = pytest.importorskip("torch")

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

P = tdm.Path
KIND = {"f32": tdm.Kind.F32, "bf16": tdm.Kind.BF16_F32ACC}
ALL_PATHS = [P.AUTO, P.EDGE, P.VALU, P.MFMA, P.SKINNY]


def random_inputs(kind, M, N, K, seed):
    rng = np.random.default_rng(seed)
    if kind == "f32":
        return inputs.uniform_fp32(rng, (M, K)), inputs.uniform_fp32(rng, (K, N))
    return inputs.normal_bf16(rng, (M, K), 1.0), inputs.normal_bf16(rng, (K, N), 1.0)


def supported_paths(kind, M, N, K):
    return [p for p in ALL_PATHS if tdm.tdm_path_supports(KIND[kind], p, M, N, K)]


def gpu_product(kind, A, B, path=P.AUTO):
    C = run(kind, to_device(A), to_device(B), path)
    torch.cuda.synchronize()
    return C.cpu().numpy()


# ---------------------------------------------------------------------------
# The small workload, every path.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("path", [P.AUTO, P.EDGE, P.VALU, P.MFMA])
def test_f32_256_workload(path):
    log(f"case f32_256 path={path.name}")
    A, B = inputs.make_inputs("f32_256")
    check_full("f32", A, B, gpu_product("f32", A, B, path), f"f32_256/{path.name}")


@pytest.mark.parametrize("path", [P.AUTO, P.EDGE, P.MFMA])
def test_bf16_square_small(path):
    log(f"case bf16 512^3 path={path.name}")
    A, B = random_inputs("bf16", 512, 512, 512, 100)
    check_full("bf16", A, B, gpu_product("bf16", A, B, path), f"bf16_512/{path.name}")


@pytest.mark.parametrize("path", [P.AUTO, P.SKINNY, P.MFMA, P.EDGE])
def test_bf16_skinny_small(path):
    log(f"case bf16 16x1024x2048 path={path.name}")
    rng = np.random.default_rng(101)
    A = inputs.normal_bf16(rng, (16, 2048), 1.0)
    B = inputs.normal_bf16(rng, (2048, 1024), 0.02)
    check_full("bf16", A, B, gpu_product("bf16", A, B, path), f"skinny_small/{path.name}")


# ---------------------------------------------------------------------------
# Ragged shapes: partial tiles in M, N and K on every path that takes them.
# ---------------------------------------------------------------------------

RAGGED = [
    (1, 1, 1), (1, 8, 8), (5, 7, 3), (33, 65, 17), (64, 64, 64), (100, 200, 48),
    (255, 257, 264), (257, 255, 136), (300, 520, 136), (512, 512, 520), (129, 8, 4096),
    (16, 264, 4104), (7, 1000, 72), (16, 64, 32), (3, 72, 8), (513, 264, 200),
]


def _ragged_cases():
    for kind in ("f32", "bf16"):
        for shape in RAGGED:
            for p in supported_paths(kind, *shape):
                yield pytest.param(kind, shape, p, id=f"{kind}-{shape[0]}x{shape[1]}x{shape[2]}-{p.name}")


@pytest.mark.parametrize("kind,shape,path", list(_ragged_cases()))
def test_ragged(kind, shape, path):
    M, N, K = shape
    log(f"case ragged {kind} {shape} path={path.name}")
    A, B = random_inputs(kind, M, N, K, seed=M * 7 + N * 13 + K)
    check_full(kind, A, B, gpu_product(kind, A, B, path), f"{kind}/{shape}/{path.name}")


# Small fp32 products, which the edge path runs on 16 x 16 tiles with whole
# K panels in LDS (M and N up to 512, K up to 512, K and N multiples of 4,
# 16-byte aligned rows): ragged tiles, the largest K, K = 4.
SMALL_F32 = [(1, 4, 4), (17, 20, 4), (15, 16, 12), (256, 256, 256), (200, 100, 500),
             (511, 508, 512), (512, 512, 512)]


@pytest.mark.parametrize("shape", SMALL_F32, ids=[f"{m}x{n}x{k}" for m, n, k in SMALL_F32])
def test_small_f32_products(shape):
    M, N, K = shape
    log(f"case small f32 {shape}")
    A, B = random_inputs("f32", M, N, K, seed=M + 3 * N + 5 * K)
    check_full("f32", A, B, gpu_product("f32", A, B, P.EDGE), f"small f32 {shape}")
    rng = np.random.default_rng(M + N + K)
    A = inputs.small_int_matrix(rng, (M, K), kind="f32")
    B = inputs.small_int_matrix(rng, (K, N), kind="f32")
    assert np.array_equal(gpu_product("f32", A, B, P.EDGE).astype(np.float64), oracle.gemm(A, B))


# Shapes large enough that the matrix-core kernels take their 256 x 256 tiles
# (the last round of tiles over the 256 CUs is at least 70% full for bf16,
# 90% for fp32), with partial tiles in M, N and K.
LARGE_TILE_RAGGED = [("bf16", (3600, 3000, 200)), ("f32", (3900, 4000, 100))]


def _fill(M, N):
    tiles = -(-M // 256) * -(-N // 256)
    return tiles / (-(-tiles // 256) * 256)


@pytest.mark.parametrize("kind,shape", LARGE_TILE_RAGGED)
def test_large_tile_ragged(kind, shape):
    M, N, K = shape
    assert _fill(M, N) >= (0.7 if kind == "bf16" else 0.9)
    log(f"case large-tile ragged {kind} {shape}")
    A, B = random_inputs(kind, M, N, K, seed=M + N + K)
    check_full(kind, A, B, gpu_product(kind, A, B, P.MFMA), f"{kind}/{shape}/MFMA")
    rng = np.random.default_rng(17)
    A = inputs.small_int_matrix(rng, (M, K), kind=kind)
    B = inputs.small_int_matrix(rng, (K, N), kind=kind)
    assert np.array_equal(gpu_product(kind, A, B, P.MFMA).astype(np.float64), oracle.gemm(A, B))


@pytest.mark.parametrize("K", [32, 64, 96, 128, 160])
def test_large_tiles_with_few_k_steps(K):
    """bf16 256 x 256 tiles (3900 x 4000: one round, partial tiles) with
    K a multiple of 32 but fewer steps than, or about as many as, the four
    ring slots: the ping-pong schedule's tail, where later copies are not
    issued and every wait is for all copies. Integer inputs, bit for bit,
    and random inputs over the whole output."""
    M, N = 3900, 4000
    log(f"case large tiles few k steps bf16 {M}x{N}x{K}")
    rng = np.random.default_rng(K + 3)
    A = inputs.small_int_matrix(rng, (M, K), kind="bf16")
    B = inputs.small_int_matrix(rng, (K, N), kind="bf16")
    assert np.array_equal(gpu_product("bf16", A, B, P.MFMA).astype(np.float64), oracle.gemm(A, B))
    A, B = random_inputs("bf16", M, N, K, seed=K + 11)
    check_full("bf16", A, B, gpu_product("bf16", A, B, P.MFMA), f"bf16/{M}x{N}x{K}/MFMA")


@pytest.mark.parametrize("kind,shape,path", list(_ragged_cases()))
def test_integer_inputs_bit_exact(kind, shape, path):
    """Small integers: every partial sum is an exactly representable integer."""
    M, N, K = shape
    log(f"case integer {kind} {shape} path={path.name}")
    rng = np.random.default_rng(5 + M + N + K)
    A = inputs.small_int_matrix(rng, (M, K), kind=kind)
    B = inputs.small_int_matrix(rng, (K, N), kind=kind)
    C = gpu_product(kind, A, B, path)
    R = oracle.gemm(A, B)
    assert np.array_equal(C.astype(np.float64), R), (kind, shape, path.name)


# ---------------------------------------------------------------------------
# Closed forms and edge cases on the GPU.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kind,path", [("f32", P.VALU), ("f32", P.MFMA), ("f32", P.EDGE),
                                       ("bf16", P.MFMA), ("bf16", P.EDGE)])
def test_closed_forms(kind, path):
    log(f"case closed forms {kind} path={path.name}")
    M, N, K = 512, 768, 4096
    ones_a = np.ones((M, K), np.float32)
    ones_b = np.ones((K, N), np.float32)
    if kind == "bf16":
        ones_a, ones_b = inputs.fp32_to_bf16_bits(ones_a), inputs.fp32_to_bf16_bits(ones_b)
    C = gpu_product(kind, ones_a, ones_b, path)
    assert np.all(C == K)
    rng = np.random.default_rng(3)
    Bv = random_inputs(kind, 1, 256, 256, 9)[1]
    eye = np.eye(256, dtype=np.float32)
    if kind == "bf16":
        eye = inputs.fp32_to_bf16_bits(eye)
    C = gpu_product(kind, eye, Bv, path)
    assert np.array_equal(C.astype(np.float64), oracle.widen(Bv))
    del rng


def test_skinny_closed_forms():
    log("case closed forms skinny")
    ones_a = inputs.fp32_to_bf16_bits(np.ones((16, 8192), np.float32))
    ones_b = inputs.fp32_to_bf16_bits(np.ones((8192, 512), np.float32))
    assert np.all(gpu_product("bf16", ones_a, ones_b, P.SKINNY) == 8192)


@pytest.mark.parametrize("kind", ["f32", "bf16"])
def test_k_zero_and_empty(kind):
    log(f"case empty {kind}")
    dt = torch.float32 if kind == "f32" else torch.int16
    A = torch.empty((5, 0), dtype=dt, device="cuda")
    B = torch.empty((0, 7), dtype=dt, device="cuda")
    C = torch.full((5, 7), 3.0, device="cuda")
    run(kind, A, B, P.AUTO, C)
    torch.cuda.synchronize()
    assert torch.all(C == 0)
    E = run(kind, torch.empty((0, 4), dtype=dt, device="cuda"),
            torch.empty((4, 9), dtype=dt, device="cuda"))
    assert E.shape == (0, 9)


@pytest.mark.parametrize("kind,shape", [("f32", (1000, 1000, 1000)), ("bf16", (1024, 1024, 1024)),
                                        ("bf16", (16, 4096, 4096))])
def test_run_to_run_bitwise_determinism(kind, shape):
    M, N, K = shape
    log(f"case determinism {kind} {shape}")
    A, B = random_inputs(kind, M, N, K, 55)
    Ad, Bd = to_device(A), to_device(B)
    for p in supported_paths(kind, M, N, K):
        ref = run(kind, Ad, Bd, p).clone()
        for _ in range(100):
            assert torch.equal(run(kind, Ad, Bd, p), ref), p.name


def test_nondefault_stream():
    log("case stream")
    A, B = random_inputs("bf16", 512, 512, 512, 77)
    Ad, Bd = to_device(A), to_device(B)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        C = run("bf16", Ad, Bd, P.MFMA, stream=s)
    s.synchronize()
    check_full("bf16", A, B, C.cpu().numpy(), "stream")


def test_small_m_calls_on_two_streams_at_once():
    """The split-K partial sums live in a per-stream buffer: calls queued on
    two streams at the same time must not disturb each other."""
    log("case small-M two streams")
    rng = np.random.default_rng(79)
    ins = [(inputs.normal_bf16(rng, (16, 4096), 1.0), inputs.normal_bf16(rng, (4096, 2048), 0.02))
           for _ in range(2)]
    dev = [(to_device(A), to_device(B), torch.empty((16, 2048), device="cuda")) for A, B in ins]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for _ in range(20):
        for (Ad, Bd, Cd), s in zip(dev, streams):
            run("bf16", Ad, Bd, P.SKINNY, Cd, stream=s)
    torch.cuda.synchronize()
    for (A, B), (_, _, Cd) in zip(ins, dev):
        C = Cd.cpu().numpy()
        check_full("bf16", A, B, C, "two streams")
        assert np.array_equal(C, gpu_product("bf16", A, B, P.SKINNY))


def test_small_m_first_call_on_a_fresh_stream():
    """A stream's first small-M call needs no allocation and no device-wide
    wait: enqueued behind other work on that stream, it returns at once and
    the result is right."""
    log("case small-M fresh stream")
    A, B = random_inputs("bf16", 16, 2048, 4096, 81)
    Ad, Bd = to_device(A), to_device(B)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        C = run("bf16", Ad, Bd, P.SKINNY, stream=s)
    s.synchronize()
    check_full("bf16", A, B, C.cpu().numpy(), "fresh stream")


def test_small_m_calls_on_more_streams_than_workspace_slots():
    """34 streams: the first eight streams of the process that call the
    small-M path own a partial-sum buffer each; calls on the others run the
    matrix-core kernel. Every output equals one of the two paths' results
    bit for bit, and at least 26 of the 34 take the matrix-core kernel."""
    import ctypes
    log("case small-M 34 streams")
    hip = ctypes.CDLL("libamdhip64.so")
    A, B = random_inputs("bf16", 16, 1024, 2048, 80)
    Ad, Bd = to_device(A), to_device(B)
    ref = gpu_product("bf16", A, B, P.SKINNY)
    ref_mfma = gpu_product("bf16", A, B, P.MFMA)
    assert not np.array_equal(ref, ref_mfma)  # the two paths are told apart
    outs = [torch.empty((16, 1024), device="cuda") for _ in range(34)]
    handles = []
    try:
        for _ in range(34):
            h = ctypes.c_void_p()
            assert hip.hipStreamCreate(ctypes.byref(h)) == 0
            handles.append(h)
        torch.cuda.synchronize()
        for h, Cd in zip(handles, outs):
            run("bf16", Ad, Bd, P.SKINNY, Cd, stream=h.value)
        for h, Cd in zip(handles, outs):  # again, now with every buffer taken
            run("bf16", Ad, Bd, P.SKINNY, Cd, stream=h.value)
        torch.cuda.synchronize()
    finally:
        torch.cuda.synchronize()
        for h in handles:
            hip.hipStreamDestroy(h)
    took_mfma = 0
    for Cd in outs:
        C = Cd.cpu().numpy()
        assert np.array_equal(C, ref) or np.array_equal(C, ref_mfma)
        took_mfma += int(np.array_equal(C, ref_mfma))
    assert took_mfma >= 34 - 8
    check_full("bf16", A, B, ref_mfma, "fallback")


def test_misaligned_pointers():
    log("case misaligned")
    A, B = random_inputs("bf16", 64, 64, 64, 78)
    Araw = to_device(np.concatenate([np.zeros(1, np.uint16), A.ravel()]))
    Ad = Araw[1:].view(64, 64)  # 2-byte offset: not 16-byte aligned
    Bd = to_device(B)
    with pytest.raises(tdm.TdmError) as e:
        run("bf16", Ad, Bd, P.MFMA)
    assert e.value.status == tdm.Status.ERROR_NOT_SUPPORTED
    C = run("bf16", Ad, Bd, P.AUTO)
    torch.cuda.synchronize()
    check_full("bf16", A, B, C.cpu().numpy(), "misaligned")

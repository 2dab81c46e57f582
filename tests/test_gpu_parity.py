"""GPU parity: the HIP kernels against the CPU oracle, through the C interface.

Bar (stated here, applied element by element):
  * integer-valued inputs (every fp32 partial sum exact): bit-exact equality
    with the oracle's round-to-nearest-even result, for the none and bias
    epilogues, on every kernel family;
  * otherwise |C - ref64| <= rtol * (|ref64| + 1) with rtol = 1e-2 for fp16
    and 2e-2 for bf16 output, against the unrounded fp64 oracle, and every
    output finite (outputs start as NaN, so an unwritten element fails);
  * the GELU epilogue in isolation (accumulator = x exactly): within two
    output ulps + 1e-6 of the fp64 oracle.
The five workloads run at full size in the launch configuration the bench
times; the oracle checks all rows (256-cube, skinny) or the seeded sample of
64 rows (the other three).
"""
import numpy as np
import pytest

import oracle
import tiled_dense_gemm_tg_amd as tg
from tiled_dense_gemm_tg_amd import inputs as I
from gpu_util import check_exact, check_tolerance, log, run, to_bits, to_device

pytestmark = pytest.mark.gpu

EXPECTED_PATH = {
    "gemm_f16_256x256x256": tg.TG_PATH_TILED,
    "gemm_f16_4096x4096x4096": tg.TG_PATH_TILED,
    "gemm_bf16_4000x4093x4111_bias_gelu_tanh": tg.TG_PATH_TILED,
    "gemm_f16_skinny_16x11008x4096": tg.TG_PATH_SKINNY,
    "gemm_f16_8192x8192x8192_bias_gelu_tanh": tg.TG_PATH_TILED,
}


def test_one_hip_runtime_in_process():
    import torch
    torch.zeros(1, device="cuda")
    tg.load_library()
    maps = open("/proc/self/maps").read()
    hip = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(hip) == 1, hip
    assert any("libtg_gemm.so" in line for line in maps.splitlines())


@pytest.mark.parametrize("name", I.WORKLOAD_ORDER)
def test_workload_parity(name):
    w = I.WORKLOADS[name]
    log(f"[parity] {name}: generating inputs")
    ops = I.make_operands(w)
    log(f"[parity] {name}: GPU run, expected path {tg.PATH_NAMES[EXPECTED_PATH[name]]}")
    out = run(w.M, w.N, w.K, w.dtype, ops.A, ops.B, ops.bias, w.epilogue, expect_path=EXPECTED_PATH[name])
    got = to_bits(out)[ops.rows]
    log(f"[parity] {name}: oracle on {len(ops.rows)} rows")
    ref64, refq = oracle.gemm(w.M, w.N, w.K, w.dtype, ops.A, ops.B, ops.bias, w.epilogue, ops.rows)
    worst = check_tolerance(w.dtype, got, ref64, name)
    log(f"[parity] {name}: worst error ratio {worst:.4f}, exact-bits fraction {np.mean(got == refq):.4f}")


@pytest.mark.parametrize("name", I.WORKLOAD_ORDER)
def test_workload_small_integers_bit_exact(name):
    w = I.WORKLOADS[name]
    ops = I.make_small_int_operands(w)
    epi = I.EPI_BIAS if w.epilogue != I.EPI_NONE else I.EPI_NONE
    rows = ops.rows[:16] if w.M * w.N * w.K > 2 ** 33 else ops.rows
    log(f"[exact] {name}: GPU run")
    out = run(w.M, w.N, w.K, w.dtype, ops.A, ops.B, ops.bias, epi, expect_path=EXPECTED_PATH[name])
    _, refq = oracle.gemm(w.M, w.N, w.K, w.dtype, ops.A, ops.B, ops.bias, epi, rows)
    check_exact(to_bits(out)[rows], refq, name)


def _families(M, N, K):
    fams = [tg.TG_PATH_TILED_GENERIC, tg.TG_PATH_TILED]
    if M <= 64 and K % 8 == 0 and N % 4 == 0:
        fams.append(tg.TG_PATH_SKINNY)
    return fams


EDGE = [1, 2, 7, 8, 15, 16, 17, 31, 33, 63, 64, 65, 127, 129, 255, 257]


def _edge_cases(n, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = set()
    while len(cases) < n:
        cases.add(tuple(int(v) for v in rng.choice(EDGE, 3)))
    return sorted(cases)


@pytest.mark.parametrize("dtype", [I.F16, I.BF16])
def test_edge_shapes_every_family(dtype):
    cases = _edge_cases(40, 17 + dtype) + [(8, 64, 64), (16, 256, 512), (300, 520, 264), (513, 264, 1000)]
    for idx, (M, N, K) in enumerate(cases):
        epi = (I.EPI_NONE, I.EPI_BIAS, I.EPI_BIAS_GELU_TANH)[idx % 3]
        A = I.random_bits((M, K), ("uniform", -1.0, 1.0), dtype, 9000 + idx)
        B = I.random_bits((K, N), ("uniform", -1.0, 1.0), dtype, 9100 + idx)
        bias = I.random_bits((N,), ("uniform", -0.5, 0.5), dtype, 9200 + idx) if epi else None
        ref64, _ = oracle.gemm(M, N, K, dtype, A, B, bias, epi)
        Ai = I.small_int_bits((M, K), dtype, 9300 + idx)
        Bi = I.small_int_bits((K, N), dtype, 9400 + idx)
        bi = I.small_int_bits((N,), dtype, 9500 + idx) if epi else None
        epi_i = min(epi, I.EPI_BIAS)
        _, refq_i = oracle.gemm(M, N, K, dtype, Ai, Bi, bi if epi_i else None, epi_i)
        for fam in _families(M, N, K):
            what = f"{I.DTYPE_NAMES[dtype]} M={M} N={N} K={K} epi={epi} path={tg.PATH_NAMES[fam]}"
            log(f"[edge] {what}")
            out = run(M, N, K, dtype, A, B, bias, epi, path=fam)
            check_tolerance(dtype, to_bits(out), ref64, what)
            out = run(M, N, K, dtype, Ai, Bi, bi if epi_i else None, epi_i, path=fam)
            check_exact(to_bits(out), refq_i, what + " (integers)")


@pytest.mark.parametrize("dtype", [I.F16, I.BF16])
def test_skinny_every_row_count(dtype):
    N, K = 4 * 97, 8 * 75
    for M in range(1, 17):
        A = I.random_bits((M, K), ("normal", 0.0, 1.0), dtype, 800 + M)
        B = I.random_bits((K, N), ("normal", 0.0, 0.02), dtype, 850 + M)
        bias = I.random_bits((N,), ("normal", 0.0, 0.1), dtype, 870 + M)
        log(f"[skinny] {I.DTYPE_NAMES[dtype]} M={M}")
        ref64, _ = oracle.gemm(M, N, K, dtype, A, B, bias, I.EPI_BIAS_GELU_TANH)
        out = run(M, N, K, dtype, A, B, bias, I.EPI_BIAS_GELU_TANH, expect_path=tg.TG_PATH_SKINNY)
        check_tolerance(dtype, to_bits(out), ref64, f"skinny M={M}")


@pytest.mark.parametrize("dtype", [I.F16, I.BF16])
@pytest.mark.parametrize("K", [8 * 75, 2056])
def test_skinny_row_blocks_every_row_count(dtype, K):
    # 17 <= M <= 64: the skinny kernel carries 2, 3 or 4 blocks of 16 rows
    # per workgroup, all multiplying the same B vectors (4 blocks on 4 waves);
    # K = 600 gives every wave at most 5 steps (A loaded per step), K = 2056
    # 16 or 17 (A staged through LDS in chunks of 16 or 8 steps, the last
    # step ragged)
    N = 4 * 97
    for M in range(17, 65):
        A = I.random_bits((M, K), ("normal", 0.0, 1.0), dtype, 1800 + M)
        B = I.random_bits((K, N), ("normal", 0.0, 0.02), dtype, 1850 + M)
        bias = I.random_bits((N,), ("normal", 0.0, 0.1), dtype, 1870 + M)
        log(f"[skinny rows] {I.DTYPE_NAMES[dtype]} M={M} K={K}")
        ref64, _ = oracle.gemm(M, N, K, dtype, A, B, bias, I.EPI_BIAS_GELU_TANH)
        out = run(M, N, K, dtype, A, B, bias, I.EPI_BIAS_GELU_TANH, path=tg.TG_PATH_SKINNY)
        check_tolerance(dtype, to_bits(out), ref64, f"skinny M={M}")
        if M in (17, 32, 33, 48, 49, 64):
            Ai = I.small_int_bits((M, K), dtype, 1880 + M)
            Bi = I.small_int_bits((K, N), dtype, 1890 + M)
            bi = I.small_int_bits((N,), dtype, 1895 + M)
            _, refq = oracle.gemm(M, N, K, dtype, Ai, Bi, bi, I.EPI_BIAS)
            check_exact(to_bits(run(M, N, K, dtype, Ai, Bi, bi, I.EPI_BIAS, path=tg.TG_PATH_SKINNY)), refq,
                        f"skinny integers M={M}")


@pytest.mark.parametrize("M,N,K", [
    (48, 11008, 4096),    # three full row blocks at the decode width
    (40, 16384, 4096),    # three blocks, the last with 8 rows; 256 slabs
    (24, 68, 3336),       # one partial slab, ragged last step
    (45, 4100, 8200),     # partial slab, three blocks, 257 steps
    (64, 11008, 4096),    # four full blocks on four waves
    (57, 4100, 8200),     # four blocks, the last with 9 rows; partial slab
])
def test_skinny_row_blocks_full_size(M, N, K):
    dtype = I.F16
    A = I.random_bits((M, K), ("normal", 0.0, 1.0), dtype, 1900 + M)
    B = I.random_bits((K, N), ("normal", 0.0, 0.02), dtype, 1901 + M)
    bias = I.random_bits((N,), ("normal", 0.0, 0.1), dtype, 1902 + M)
    log(f"[skinny rows full] M={M} N={N} K={K}")
    ref64, _ = oracle.gemm(M, N, K, dtype, A, B, bias, I.EPI_BIAS_GELU_TANH)
    out = run(M, N, K, dtype, A, B, bias, I.EPI_BIAS_GELU_TANH, path=tg.TG_PATH_SKINNY)
    check_tolerance(dtype, to_bits(out), ref64, f"skinny rows M={M} N={N} K={K}")


@pytest.mark.parametrize("dtype", [I.F16, I.BF16])
@pytest.mark.parametrize("M,N,K", [
    (16, 4 * 97, 4096),   # 32 steps of 32 k per wave
    (5, 4 * 97, 2400),    # 75 steps: 18 or 19 per wave
    (1, 520, 4008),       # 126 steps, the last with 8 of its 32 k
    (11, 68, 3336),       # 105 steps: 26 or 27 per wave; one partial slab
    (7, 132, 2184),       # 69 steps: 17 or 18 per wave, the fewest that preload
    (16, 4 * 97, 8200),   # 257 steps: 64 or 65 per wave, A staged in chunks of 32 steps
    (3, 132, 5128),       # 161 steps: 40 or 41 per wave, the second chunk of 8 or 9 steps
])
def test_skinny_preloaded_A(dtype, M, N, K):
    # Shapes where every wave has more than 16 steps of 32 k, so the skinny
    # kernel stages its slice of A through LDS (whole, or in chunks of 32
    # steps) instead of loading A with every step of B.
    A = I.random_bits((M, K), ("normal", 0.0, 1.0), dtype, 900 + M)
    B = I.random_bits((K, N), ("normal", 0.0, 0.02), dtype, 901 + M)
    bias = I.random_bits((N,), ("normal", 0.0, 0.1), dtype, 902 + M)
    log(f"[skinny preload] {I.DTYPE_NAMES[dtype]} M={M} N={N} K={K}")
    ref64, _ = oracle.gemm(M, N, K, dtype, A, B, bias, I.EPI_BIAS_GELU_TANH)
    out = run(M, N, K, dtype, A, B, bias, I.EPI_BIAS_GELU_TANH, expect_path=tg.TG_PATH_SKINNY)
    check_tolerance(dtype, to_bits(out), ref64, f"skinny preload M={M} K={K}")
    Ai = I.small_int_bits((M, K), dtype, 903 + M)
    Bi = I.small_int_bits((K, N), dtype, 904 + M)
    _, refq = oracle.gemm(M, N, K, dtype, Ai, Bi)
    check_exact(to_bits(run(M, N, K, dtype, Ai, Bi, expect_path=tg.TG_PATH_SKINNY)), refq,
                f"skinny preload integers M={M} K={K}")


@pytest.mark.parametrize("dtype", [I.F16, I.BF16])
def test_identity_and_permutation_products(dtype):
    """MFMA operand/output layouts: one non-zero term per sum, so results are exact."""
    rng = np.random.Generator(np.random.PCG64(31))
    for M, K, N in [(300, 264, 200), (16, 64, 64), (257, 129, 65)]:
        A = I.random_bits((M, K), ("normal", 0.0, 2.0), dtype, 32)
        eye = I.values_bits(np.eye(K), dtype)
        perm = rng.permutation(K)
        P = np.zeros((K, K), dtype=np.float32)
        P[perm, np.arange(K)] = 1.0       # A @ P: column j of the result is column perm[j] of A
        for fam in _families(M, K, K):
            log(f"[layout] {I.DTYPE_NAMES[dtype]} M={M} K={K} path={tg.PATH_NAMES[fam]}")
            out = run(M, K, K, dtype, A, eye, path=fam)
            check_exact(to_bits(out), A, "A @ I")
            out = run(M, K, K, dtype, A, I.values_bits(P, dtype), path=fam)
            check_exact(to_bits(out), A[:, perm], "A @ P")
        B = I.random_bits((K, N), ("normal", 0.0, 2.0), dtype, 33)
        Q = np.zeros((M, K), dtype=np.float32)
        rows = rng.integers(0, K, M)
        Q[np.arange(M), rows] = 1.0       # Q @ B: row i of the result is row rows[i] of B
        for fam in _families(M, N, K):
            out = run(M, N, K, dtype, I.values_bits(Q, dtype), B, path=fam)
            check_exact(to_bits(out), B[rows], f"Q @ B path={tg.PATH_NAMES[fam]}")


@pytest.mark.parametrize("dtype", [I.F16, I.BF16])
def test_gelu_epilogue_tight(dtype):
    """Accumulator = x exactly (identity A); GELU(x + b) within 2 output ulps + 1e-6."""
    K = N = 256
    M = 256
    x = np.linspace(-4.0, 4.0, M * N).reshape(M, N)
    X = I.values_bits(x, dtype)
    eye = I.values_bits(np.eye(K), dtype)
    for with_bias in (False, True):
        b = I.random_bits((N,), ("uniform", -1.0, 1.0), dtype, 40) if with_bias else I.values_bits(np.zeros(N), dtype)
        ref64, _ = oracle.gemm(M, N, K, dtype, eye, X, b, I.EPI_BIAS_GELU_TANH)
        ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref64), 2.0 ** -14))) - (10 if dtype == I.F16 else 7))
        for fam in _families(M, N, K):
            log(f"[gelu] {I.DTYPE_NAMES[dtype]} bias={with_bias} path={tg.PATH_NAMES[fam]}")
            out = run(M, N, K, dtype, eye, X, b, I.EPI_BIAS_GELU_TANH, path=fam)
            got = oracle.decode(dtype, to_bits(out))
            err = np.abs(got - ref64)
            assert (err <= 2 * ulp + 1e-6).all(), float((err / (2 * ulp + 1e-6)).max())


@pytest.mark.parametrize("path", [tg.TG_PATH_TILED, tg.TG_PATH_TILED_GENERIC, tg.TG_PATH_SKINNY])
@pytest.mark.parametrize("epi", [I.EPI_NONE, I.EPI_BIAS, I.EPI_BIAS_GELU_TANH])
def test_empty_K_gives_epilogue_of_zero(path, epi):
    import torch
    N = 264
    bias = I.random_bits((N,), ("uniform", -2.0, 2.0), I.F16, 50) if epi else None
    for M in (16, 40, 64):   # one, three and four row blocks on the skinny path
        _, refq = oracle.gemm(M, N, 0, I.F16, None, None, bias, epi)
        log(f"[K=0] path={tg.PATH_NAMES[path]} M={M} epi={epi}")
        out = run(M, N, 0, I.F16, np.zeros(0, np.uint16), np.zeros(0, np.uint16), bias, epi, path=path)
        check_exact(to_bits(out), refq, f"K=0 M={M}")


@pytest.mark.parametrize("path,M,N,K", [
    (tg.TG_PATH_TILED, 300, 264, 200),
    (tg.TG_PATH_TILED_GENERIC, 301, 263, 201),
    (tg.TG_PATH_SKINNY, 13, 260, 200),
    (tg.TG_PATH_SKINNY, 37, 260, 200),
    (tg.TG_PATH_SKINNY, 61, 260, 200),
])
def test_guard_bands_untouched(path, M, N, K):
    """C sits inside a larger buffer; the bytes around it must survive."""
    import torch
    guard = 2048  # elements = 4 KiB on each side
    dtype = I.F16
    A = I.random_bits((M, K), ("uniform", -1.0, 1.0), dtype, 60)
    B = I.random_bits((K, N), ("uniform", -1.0, 1.0), dtype, 61)
    bias = I.random_bits((N,), ("uniform", -1.0, 1.0), dtype, 62)
    buf = torch.full((guard + M * N + guard,), 12345.0, dtype=torch.float16, device="cuda")
    out = buf[guard:guard + M * N].view(M, N)
    out.fill_(float("nan"))
    log(f"[guard] path={tg.PATH_NAMES[path]} M={M} N={N} K={K}")
    run(M, N, K, dtype, A, B, bias, I.EPI_BIAS_GELU_TANH, path=path, out=out)
    host = buf.cpu()
    assert (host[:guard] == 12345.0).all() and (host[guard + M * N:] == 12345.0).all()
    ref64, _ = oracle.gemm(M, N, K, dtype, A, B, bias, I.EPI_BIAS_GELU_TANH)
    check_tolerance(dtype, to_bits(out), ref64, "guarded")


def test_repeat_runs_are_bit_identical():
    w = I.WORKLOADS["gemm_f16_4096x4096x4096"]
    ops = I.make_operands(w)
    log("[repeat] 4096-cube twice")
    first = to_bits(run(w.M, w.N, w.K, w.dtype, ops.A, ops.B))
    second = to_bits(run(w.M, w.N, w.K, w.dtype, ops.A, ops.B))
    assert np.array_equal(first, second)
    w4 = I.WORKLOADS["gemm_f16_skinny_16x11008x4096"]
    ops4 = I.make_operands(w4)
    log("[repeat] skinny twice")
    first = to_bits(run(w4.M, w4.N, w4.K, w4.dtype, ops4.A, ops4.B))
    second = to_bits(run(w4.M, w4.N, w4.K, w4.dtype, ops4.A, ops4.B))
    assert np.array_equal(first, second)


def test_runs_on_a_non_default_stream():
    import torch
    M, N, K = 520, 264, 328
    A = I.random_bits((M, K), ("uniform", -1.0, 1.0), I.BF16, 70)
    B = I.random_bits((K, N), ("uniform", -1.0, 1.0), I.BF16, 71)
    ref64, _ = oracle.gemm(M, N, K, I.BF16, A, B)
    s = torch.cuda.Stream()
    log("[stream] side stream")
    with torch.cuda.stream(s):
        out = run(M, N, K, I.BF16, A, B, stream=s)
    s.synchronize()
    check_tolerance(I.BF16, to_bits(out), ref64, "side stream")


@pytest.mark.parametrize("dtype,M,N,K", [
    (I.F16, 2304, 8192, 200),    # 288 tiles, a multiple of the 8 XCDs
    (I.BF16, 4350, 4360, 96),    # 306 tiles, ragged in M and N
    (I.F16, 16384, 4096, 64),    # 1024 tiles, four per workgroup on 256 CUs
])
def test_persistent_grid_covers_every_tile(dtype, M, N, K):
    """More tiles than compute units: each workgroup of the vector kernel
    walks several tiles; every output must be written once, exactly."""
    A = I.small_int_bits((M, K), dtype, 80)
    B = I.small_int_bits((K, N), dtype, 81)
    bias = I.small_int_bits((N,), dtype, 82)
    log(f"[persistent] dtype={dtype} M={M} N={N} K={K}")
    out = run(M, N, K, dtype, A, B, bias, I.EPI_BIAS, expect_path=tg.TG_PATH_TILED)
    _, refq = oracle.gemm(M, N, K, dtype, A, B, bias, I.EPI_BIAS)
    check_exact(to_bits(out), refq, f"persistent {M}x{N}x{K}")


def _offset_tensor(bits, dtype, shape, offset):
    """A device tensor of `shape` starting `offset` elements into its buffer."""
    n = int(np.prod(shape))
    flat = to_device(np.concatenate([np.zeros(offset, np.uint16), np.ascontiguousarray(bits).reshape(-1)]), dtype)
    return flat[offset:offset + n].view(*shape)


@pytest.mark.parametrize("dtype", [I.F16, I.BF16])
@pytest.mark.parametrize("M,N,K,offsets", [
    (520, 264, 328, (1, 0, 0, 0)),    # A 2-byte aligned, shapes aligned
    (520, 264, 328, (0, 3, 0, 0)),    # B
    (520, 264, 328, (0, 0, 1, 1)),    # C and bias
    (300, 263, 201, (1, 1, 1, 1)),    # everything ragged and misaligned
])
def test_tiled_any_alignment(dtype, M, N, K, offsets):
    """The tiled family at 2-byte-aligned operands (unaligned direct loads,
    grouped 8-byte stores) against the oracle, bit-exact on integers."""
    import torch
    oa, ob, oc, obias = offsets
    for kind in ("random", "integers"):
        if kind == "random":
            A = I.random_bits((M, K), ("uniform", -1.0, 1.0), dtype, 400)
            B = I.random_bits((K, N), ("uniform", -1.0, 1.0), dtype, 401)
            bias = I.random_bits((N,), ("uniform", -0.5, 0.5), dtype, 402)
            epi = I.EPI_BIAS_GELU_TANH
        else:
            A = I.small_int_bits((M, K), dtype, 403)
            B = I.small_int_bits((K, N), dtype, 404)
            bias = I.small_int_bits((N,), dtype, 405)
            epi = I.EPI_BIAS
        ref64, refq = oracle.gemm(M, N, K, dtype, A, B, bias, epi)
        a = _offset_tensor(A, dtype, (M, K), oa)
        b = _offset_tensor(B, dtype, (K, N), ob)
        bb = _offset_tensor(bias, dtype, (N,), obias)
        c = _offset_tensor(np.full(M * N, 0x7E00, np.uint16), dtype, (M, N), oc)   # NaN-filled
        log(f"[align] dtype={dtype} {M}x{N}x{K} offsets={offsets} {kind}")
        st, p = tg.tg_gemm_plan(M, N, K, dtype, a.data_ptr(), b.data_ptr(), bb.data_ptr(), epi, c.data_ptr())
        assert st == tg.TG_OK and p == tg.TG_PATH_TILED
        tg.gemm(a, b, bb, {I.EPI_BIAS: "bias", I.EPI_BIAS_GELU_TANH: "bias_gelu_tanh"}[epi], out=c)
        torch.cuda.synchronize()
        if kind == "random":
            check_tolerance(dtype, to_bits(c), ref64, f"align {offsets}")
        else:
            check_exact(to_bits(c), refq, f"align {offsets}")


@pytest.mark.parametrize("path", [tg.TG_PATH_TILED, tg.TG_PATH_TILED_GENERIC])
@pytest.mark.parametrize("K", [37, 8, 33])
def test_k_tail_does_not_mix_rows(path, K):
    """Rows of A alternate between finite values and +inf at k = 0.  With K
    not a multiple of 8 the 16-byte chunk that crosses k = K of an even row
    also covers the first elements of the odd row after it; those must not
    enter the sum (inf * 0 would turn the even row into NaN)."""
    M, N = 64, 72
    dtype = I.F16
    A = I.random_bits((M, K), ("uniform", -1.0, 1.0), dtype, 410)
    inf = np.uint16(0x7C00)
    A = A.reshape(M, K).copy()
    A[1::2, 0] = inf
    B = I.random_bits((K, N), ("uniform", 0.5, 1.0), dtype, 411)    # positive: odd rows are +inf
    ref64, _ = oracle.gemm(M, N, K, dtype, A.reshape(-1), B)
    log(f"[k-tail] path={tg.PATH_NAMES[path]} K={K}")
    out = oracle.decode(dtype, to_bits(run(M, N, K, dtype, A.reshape(-1), B, path=path)))
    assert np.isposinf(out[1::2]).all()
    check_tolerance(dtype, to_bits(run(M, N, K, dtype, A.reshape(-1), B, path=path))[0::2], ref64[0::2],
                    "even rows")

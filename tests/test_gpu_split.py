"""GPU parity of split-K on the M <= 16 kernels, through tg_gemm_split (the
skinny kernel) and tg_gemm_w4_split (the 4-bit product).

Bar, as for every kernel family: bit-exact against the oracle on
integer-valued inputs (none and bias epilogues), |C - ref64| <= rtol (|ref64| + 1)
otherwise (rtol 1e-2 fp16, 2e-2 bf16), every output finite.  Split-K adds
its own properties: the same splits give bit-identical results on every
call, every completed call leaves the workspace counters at zero (so one
workspace serves call after call), and shapes off the skinny path leave the
workspace alone.
"""
import numpy as np
import pytest

import oracle
import tiled_dense_gemm_tg_amd as tg
from tiled_dense_gemm_tg_amd import inputs as I
from gpu_util import check_exact, check_tolerance, log, to_bits, to_device, torch_dtype

pytestmark = pytest.mark.gpu


def _split_run(M, N, K, dtype, A_bits, B_bits, bias_bits, epi, splits, ws=None):
    """tg_gemm_split on fresh NaN-filled C; returns (C, workspace)."""
    import torch
    A = to_device(A_bits.reshape(M, K), dtype) if M * K else torch.empty((M, K), dtype=torch_dtype(dtype), device="cuda")
    B = to_device(B_bits.reshape(K, N), dtype) if K * N else torch.empty((K, N), dtype=torch_dtype(dtype), device="cuda")
    bias = to_device(bias_bits, dtype) if bias_bits is not None else None
    C = torch.full((M, N), float("nan"), dtype=torch_dtype(dtype), device="cuda")
    if ws is None:
        ws = tg.split_workspace(M, N, K, splits)
    st = tg.tg_gemm_split(splits, M, N, K, dtype, A.data_ptr(), B.data_ptr(),
                          bias.data_ptr() if bias is not None else None, epi, C.data_ptr(),
                          ws.data_ptr() if ws is not None else None, ws.numel() if ws is not None else 0,
                          torch.cuda.current_stream().cuda_stream)
    assert st == tg.TG_OK, tg.tg_status_string(st)
    torch.cuda.synchronize()
    return C, ws


def _counters_zero(ws, N):
    if ws is None:
        return True
    slabs = (N + 63) // 64
    return int(ws[: 4 * slabs].count_nonzero()) == 0


CASES = [
    # M, N, K, splits: several slabs, ragged K (K % 32 != 0), more splits than
    # 32-k steps (empty splits), a single slab, odd split counts
    (16, 256, 4096, 2),
    (16, 256, 4096, 3),
    (16, 256, 4096, 8),
    (7, 1028, 1000, 5),
    (1, 64, 8, 4),
    (16, 4100, 2056, 64),
    (12, 520, 4104, 7),
    (5, 260, 8008, 2),      # 125 or 126 steps per split: the A slice staged through LDS
]


@pytest.mark.parametrize("dtype", [I.F16, I.BF16])
@pytest.mark.parametrize("M,N,K,splits", CASES)
def test_split_parity(dtype, M, N, K, splits):
    for epi in (I.EPI_NONE, I.EPI_BIAS_GELU_TANH):
        seed = 31000 + 97 * M + 13 * splits + epi + 5 * dtype
        A = I.random_bits((M, K), ("normal", 0.0, 1.0), dtype, seed)
        B = I.random_bits((K, N), ("normal", 0.0, 0.02), dtype, seed + 1)
        bias = I.random_bits((N,), ("normal", 0.0, 0.1), dtype, seed + 2) if epi else None
        what = f"{I.DTYPE_NAMES[dtype]} M={M} N={N} K={K} splits={splits} epi={epi}"
        log(f"[split] {what}")
        C, ws = _split_run(M, N, K, dtype, A, B, bias, epi, splits)
        ref64, _ = oracle.gemm(M, N, K, dtype, A, B, bias, epi)
        check_tolerance(dtype, to_bits(C), ref64, what)
        assert _counters_zero(ws, N), what


@pytest.mark.parametrize("dtype", [I.F16, I.BF16])
@pytest.mark.parametrize("M,N,K,splits", CASES)
def test_split_integers_bit_exact(dtype, M, N, K, splits):
    seed = 32000 + 97 * M + 13 * splits + 5 * dtype
    A = I.small_int_bits((M, K), dtype, seed)
    B = I.small_int_bits((K, N), dtype, seed + 1)
    bias = I.small_int_bits((N,), dtype, seed + 2)
    what = f"{I.DTYPE_NAMES[dtype]} M={M} N={N} K={K} splits={splits} (integers)"
    log(f"[split exact] {what}")
    C, _ = _split_run(M, N, K, dtype, A, B, bias, I.EPI_BIAS, splits)
    _, refq = oracle.gemm(M, N, K, dtype, A, B, bias, I.EPI_BIAS)
    check_exact(to_bits(C), refq, what)


def test_split_reuses_one_workspace_and_is_deterministic():
    """One workspace, sized for the largest call, through calls of several
    shapes and split counts: every call leaves the counters zero, and a
    repeated call is bit-identical."""
    import torch
    dtype = I.F16
    shapes = [(16, 4096, 2048, 4), (16, 1024, 4096, 8), (3, 4096, 2048, 4), (16, 4096, 2048, 4), (16, 256, 512, 2)]
    need = max(tg.tg_gemm_split_workspace_bytes(N, s) for (_, N, _, s) in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    first = {}
    for i, (M, N, K, splits) in enumerate(shapes):
        A = I.random_bits((M, K), ("normal", 0.0, 1.0), dtype, 33000 + i % 3)
        B = I.random_bits((K, N), ("normal", 0.0, 0.02), dtype, 33100 + i % 3)
        what = f"M={M} N={N} K={K} splits={splits} call {i}"
        log(f"[split reuse] {what}")
        C, _ = _split_run(M, N, K, dtype, A, B, None, I.EPI_NONE, splits, ws)
        assert _counters_zero(ws, 4096), what
        bits = to_bits(C)
        key = (M, N, K, splits)
        if key in first:
            assert np.array_equal(first[key], bits), what + ": not bit-identical to the first call"
        else:
            first[key] = bits
            ref64, _ = oracle.gemm(M, N, K, dtype, A, B, None, I.EPI_NONE)
            check_tolerance(dtype, bits, ref64, what)


def test_split_auto_matches_its_plan():
    """splits = 0 runs the count tg_gemm_split_plan reports for the device."""
    import torch
    dtype = I.F16
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for M, N, K in [(16, 4096, 11008), (16, 11008, 4096), (4, 2048, 8192), (16, 11008, 11008)]:
        st, splits, nbytes = tg.tg_gemm_split_plan(M, N, K, cus)
        assert st == tg.TG_OK
        A = I.random_bits((M, K), ("normal", 0.0, 1.0), dtype, 34000 + N)
        B = I.random_bits((K, N), ("normal", 0.0, 0.02), dtype, 34001 + N)
        log(f"[split auto] M={M} N={N} K={K}: plan {splits} splits, {nbytes} bytes")
        C_auto, _ = _split_run(M, N, K, dtype, A, B, None, I.EPI_NONE, 0)
        C_plan, _ = _split_run(M, N, K, dtype, A, B, None, I.EPI_NONE, splits)
        if (M, N, K) == (16, 11008, 11008):
            assert splits == tg.TG_SPLIT_STREAM_K
        assert torch.equal(C_auto.view(torch.int16), C_plan.view(torch.int16))
        rows = np.arange(M)[:: max(1, M // 4)]
        ref64, _ = oracle.gemm(M, N, K, dtype, A, B, None, I.EPI_NONE, rows)
        check_tolerance(dtype, to_bits(C_auto)[rows], ref64, f"auto M={M} N={N} K={K}")


def test_split_off_the_skinny_path_leaves_workspace_alone():
    """Split-K is for M <= 16 only: with more rows tg_gemm_split runs as
    tg_gemm (unsplit) and never touches the workspace (filled with a pattern
    it would change)."""
    import torch
    dtype = I.BF16
    M, N, K = 40, 520, 264
    A = I.random_bits((M, K), ("uniform", -1.0, 1.0), dtype, 35000)
    B = I.random_bits((K, N), ("uniform", -1.0, 1.0), dtype, 35001)
    ws = torch.full((tg.tg_gemm_split_workspace_bytes(N, 4),), 0x5A, dtype=torch.uint8, device="cuda")
    C, _ = _split_run(M, N, K, dtype, A, B, None, I.EPI_NONE, 4, ws)
    assert int((ws != 0x5A).sum()) == 0
    ref64, _ = oracle.gemm(M, N, K, dtype, A, B, None, I.EPI_NONE)
    check_tolerance(dtype, to_bits(C), ref64, "M=40 through tg_gemm_split")


@pytest.mark.parametrize("M,N,K", [(16, 11008, 4096), (16, 4096, 11008)])
def test_split_decode_shapes_full_size(M, N, K):
    """The decode shapes at full size with the library's split count and with
    2 and 8 splits, every row against the oracle."""
    dtype = I.F16
    A = I.random_bits((M, K), ("normal", 0.0, 1.0), dtype, 36000 + N)
    B = I.random_bits((K, N), ("normal", 0.0, 0.02), dtype, 36001 + N)
    ref64, _ = oracle.gemm(M, N, K, dtype, A, B, None, I.EPI_NONE)
    for splits in (0, 2, 8, tg.TG_SPLIT_STREAM_K):
        what = f"M={M} N={N} K={K} splits={splits}"
        log(f"[split full] {what}")
        C, ws = _split_run(M, N, K, dtype, A, B, None, I.EPI_NONE, splits)
        check_tolerance(dtype, to_bits(C), ref64, what)
        assert _counters_zero(ws, N), what


# ------------------------------------------------------------ stream-K

SK = tg.TG_SPLIT_STREAM_K

SK_CASES = [
    # M, N, K: the decode shape (172 slabs on the CUs: 86 steps per workgroup,
    # parts of one or two slabs each); ragged N and K with a few steps per
    # workgroup; one step in all (one workgroup); 16-step slabs under
    # 18-19-step ranges (workgroups that finish a whole slab between two
    # shared ones); few slabs (fewer workgroups than CUs)
    (16, 11008, 4096),
    (7, 1028, 1000),
    (1, 64, 8),
    (16, 19200, 512),
    (12, 520, 4104),
    (5, 8256, 8008),
]


@pytest.mark.parametrize("dtype", [I.F16, I.BF16])
@pytest.mark.parametrize("M,N,K", SK_CASES)
def test_streamk_parity(dtype, M, N, K):
    rows = np.arange(M) if N * K <= 4096 * 4096 else np.arange(M)[:: max(1, M // 4)]
    for epi in (I.EPI_NONE, I.EPI_BIAS_GELU_TANH):
        seed = 38000 + 97 * M + epi + 5 * dtype + N % 1000
        A = I.random_bits((M, K), ("normal", 0.0, 1.0), dtype, seed)
        B = I.random_bits((K, N), ("normal", 0.0, 0.02), dtype, seed + 1)
        bias = I.random_bits((N,), ("normal", 0.0, 0.1), dtype, seed + 2) if epi else None
        what = f"stream-K {I.DTYPE_NAMES[dtype]} M={M} N={N} K={K} epi={epi}"
        log(f"[stream-K] {what}")
        C, ws = _split_run(M, N, K, dtype, A, B, bias, epi, SK)
        ref64, _ = oracle.gemm(M, N, K, dtype, A, B, bias, epi, rows)
        check_tolerance(dtype, to_bits(C)[rows], ref64, what)
        assert np.isfinite(C.float().cpu().numpy()).all(), what
        assert _counters_zero(ws, N), what


@pytest.mark.parametrize("dtype", [I.F16, I.BF16])
@pytest.mark.parametrize("M,N,K", SK_CASES[1:])
def test_streamk_integers_bit_exact(dtype, M, N, K):
    seed = 39000 + 97 * M + 5 * dtype + N % 1000
    A = I.small_int_bits((M, K), dtype, seed)
    B = I.small_int_bits((K, N), dtype, seed + 1)
    bias = I.small_int_bits((N,), dtype, seed + 2)
    what = f"stream-K {I.DTYPE_NAMES[dtype]} M={M} N={N} K={K} (integers)"
    log(f"[stream-K exact] {what}")
    C, _ = _split_run(M, N, K, dtype, A, B, bias, I.EPI_BIAS, SK)
    _, refq = oracle.gemm(M, N, K, dtype, A, B, bias, I.EPI_BIAS)
    check_exact(to_bits(C), refq, what)


def test_streamk_reuses_one_workspace_and_is_deterministic():
    """One workspace through stream-K calls of several shapes, even splits
    between them: the call's counters end at zero and a repeated
    call is bit-identical (the parts of a slab are added in K order,
    whichever workgroup comes last)."""
    import torch
    dtype = I.F16
    shapes = [(16, 11008, 4096, SK), (16, 4096, 2048, 4), (16, 11008, 4096, SK), (3, 19200, 512, SK),
              (16, 11008, 4096, SK)]
    need = max(tg.tg_gemm_split_workspace_bytes(N, s) for (_, N, _, s) in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    first = {}
    for i, (M, N, K, splits) in enumerate(shapes):
        A = I.random_bits((M, K), ("normal", 0.0, 1.0), dtype, 40000 + N)
        B = I.random_bits((K, N), ("normal", 0.0, 0.02), dtype, 40100 + N)
        what = f"M={M} N={N} K={K} splits={splits} call {i}"
        log(f"[stream-K reuse] {what}")
        C, _ = _split_run(M, N, K, dtype, A, B, None, I.EPI_NONE, splits, ws)
        assert _counters_zero(ws, N), what     # the counters of this call's slabs
        bits = to_bits(C)
        key = (M, N, K, splits)
        if key in first:
            assert np.array_equal(first[key], bits), what + ": not bit-identical to the first call"
        else:
            first[key] = bits
            rows = np.arange(M)[:: max(1, M // 4)]
            ref64, _ = oracle.gemm(M, N, K, dtype, A, B, None, I.EPI_NONE, rows)
            check_tolerance(dtype, bits[rows], ref64, what)


# ------------------------------------------------------------ 4-bit weights

W4_EPI = {I.EPI_NONE: "none", I.EPI_BIAS: "bias", I.EPI_BIAS_GELU_TANH: "bias_gelu_tanh"}


def _w4_split_run(M, N, K, G, dtype, A, Q, S, bias, epi, splits, ws=None):
    import torch
    q = torch.from_numpy(np.ascontiguousarray(Q)).cuda()
    packed = tg.w4_pack(q)
    a = to_device(A.reshape(M, K), dtype)
    s = to_device(S.reshape(-1), dtype)
    b = to_device(bias, dtype) if bias is not None else None
    out = torch.full((M, N), float("nan"), dtype=a.dtype, device="cuda")
    if ws is None:
        ws = tg.w4_split_workspace(M, N, K, G, splits)
    tg.gemm_w4(a, packed, s, G, N, b, W4_EPI[epi], out=out, splits=splits, workspace=ws)
    torch.cuda.synchronize()
    return to_bits(out), ws


W4_CASES = [
    # M, N, K, G, splits: the narrow decode shape, several row blocks, ragged N
    # (element-wise scales), more splits than scale groups, 32-k groups
    (16, 4096, 4096, 128, 4),
    (16, 256, 2048, 64, 3),
    (40, 300, 1024, 128, 2),
    (9, 1001, 512, 32, 5),
    (3, 128, 256, 128, 4),
    (16, 512, 8192, 256, 8),
    (11, 320, 8192, 128, 2),   # 4 groups of 4 steps per wave: A staged through LDS
]


@pytest.mark.parametrize("dtype", [I.F16, I.BF16])
@pytest.mark.parametrize("M,N,K,G,splits", W4_CASES)
def test_w4_split_parity(dtype, M, N, K, G, splits):
    epi = I.EPI_BIAS_GELU_TANH if (M + splits) % 2 else I.EPI_NONE
    seed = 37000 + M + 7 * splits + G + 3 * dtype
    A = I.random_bits((M, K), ("normal", 0.0, 1.0), dtype, seed)
    Q = I.w4_weights(K, N, seed + 1)
    S = I.random_bits((K // G, N), ("uniform", 0.001, 0.01), dtype, seed + 2)
    bias = I.random_bits((N,), ("uniform", -0.5, 0.5), dtype, seed + 3) if epi else None
    what = f"w4 {I.DTYPE_NAMES[dtype]} M={M} N={N} K={K} G={G} splits={splits} epi={epi}"
    log(f"[w4 split] {what}")
    got, ws = _w4_split_run(M, N, K, G, dtype, A, Q, S, bias, epi, splits)
    ref64, _ = oracle.gemm_w4(M, N, K, dtype, A, Q, S, G, bias, epi)
    check_tolerance(dtype, got, ref64, what)
    blocks = ((N + 63) // 64) * ((M + 15) // 16)
    assert ws is None or int(ws[: 4 * blocks].count_nonzero()) == 0, what


@pytest.mark.parametrize("M,N,K,G,splits", W4_CASES)
def test_w4_split_integers_bit_exact(M, N, K, G, splits):
    dtype = I.F16
    seed = 38000 + M + 7 * splits + G
    rng = np.random.Generator(np.random.PCG64(seed))
    A = I.small_int_bits((M, K), dtype, seed + 1)
    Q = I.w4_weights(K, N, seed + 2)
    S = I.values_bits(2.0 ** rng.integers(-3, 2, size=(K // G, N)), dtype)
    bias = I.small_int_bits((N,), dtype, seed + 3)
    what = f"w4 integers M={M} N={N} K={K} G={G} splits={splits}"
    log(f"[w4 split exact] {what}")
    got, _ = _w4_split_run(M, N, K, G, dtype, A, Q, S, bias, I.EPI_BIAS, splits)
    _, refq = oracle.gemm_w4(M, N, K, dtype, A, Q, S, G, bias, I.EPI_BIAS)
    check_exact(got, refq, what)


def test_w4_split_auto_and_repeat():
    """splits = 0 matches the plan's count bit for bit, and one workspace
    serves repeated calls (counters back at zero each time)."""
    import torch
    dtype = I.F16
    M, N, K, G = 16, 4096, 11008 // 128 * 128, 128
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    st, splits, nbytes = tg.tg_gemm_w4_split_plan(M, N, K, G, cus)
    assert st == tg.TG_OK
    A = I.random_bits((M, K), ("normal", 0.0, 1.0), dtype, 39000)
    Q = I.w4_weights(K, N, 39001)
    S = I.random_bits((K // G, N), ("uniform", 0.001, 0.01), dtype, 39002)
    ws = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    log(f"[w4 split auto] plan {splits} splits")
    first, _ = _w4_split_run(M, N, K, G, dtype, A, Q, S, None, I.EPI_NONE, 0, ws)
    for _ in range(2):
        again, _ = _w4_split_run(M, N, K, G, dtype, A, Q, S, None, I.EPI_NONE, splits, ws)
        assert np.array_equal(first, again)
        assert int(ws[:256].count_nonzero()) == 0
    ref64, _ = oracle.gemm_w4(M, N, K, dtype, A, Q, S, G, None, I.EPI_NONE)
    check_tolerance(dtype, first, ref64, "w4 split auto")

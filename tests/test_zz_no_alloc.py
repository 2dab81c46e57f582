"""GPU test of tg_gemm_split_static, the split-K entry point that allocates
nothing: its workspace is the library's static per-GPU scratch array.

Its output must equal tg_gemm_split's with the same splits (same kernels,
same split order: bit-identical) and meet the oracle's bar, on two calls in a
row through the same scratch, the second with a smaller input (fewer slabs,
more splits, so the second call's counters sit where the first call's did and
its partial blocks overwrite the first call's).  Inputs are seeded normal
values at the decode shape's distributions.
"""
import numpy as np
import pytest

import oracle
import tiled_dense_gemm_tg_amd as tg
from tiled_dense_gemm_tg_amd import inputs as I
from gpu_util import check_exact, check_tolerance, log, to_bits, to_device, torch_dtype

pytestmark = pytest.mark.gpu


def _operands(M, N, K, dtype, epi, seed):
    A = I.random_bits((M, K), ("normal", 0.0, 1.0), dtype, seed)
    B = I.random_bits((K, N), ("normal", 0.0, 0.02), dtype, seed + 1)
    bias = I.random_bits((N,), ("normal", 0.0, 0.1), dtype, seed + 2) if epi else None
    return A, B, bias


def _both(M, N, K, dtype, epi, splits, seed):
    """(static-scratch C bits, caller-workspace C bits, oracle ref64)."""
    import torch
    A_bits, B_bits, bias_bits = _operands(M, N, K, dtype, epi, seed)
    A = to_device(A_bits.reshape(M, K), dtype)
    B = to_device(B_bits.reshape(K, N), dtype)
    bias = to_device(bias_bits, dtype) if bias_bits is not None else None
    bp = bias.data_ptr() if bias is not None else None
    s = torch.cuda.current_stream().cuda_stream
    C_static = torch.full((M, N), float("nan"), dtype=torch_dtype(dtype), device="cuda")
    st = tg.tg_gemm_split_static(splits, M, N, K, dtype, A.data_ptr(), B.data_ptr(), bp, epi,
                                 C_static.data_ptr(), s)
    assert st == tg.TG_OK, tg.tg_status_string(st)
    torch.cuda.synchronize()
    ws = tg.split_workspace(M, N, K, splits)
    C_ws = torch.full((M, N), float("nan"), dtype=torch_dtype(dtype), device="cuda")
    st = tg.tg_gemm_split(splits, M, N, K, dtype, A.data_ptr(), B.data_ptr(), bp, epi, C_ws.data_ptr(),
                          ws.data_ptr() if ws is not None else None, ws.numel() if ws is not None else 0, s)
    assert st == tg.TG_OK, tg.tg_status_string(st)
    torch.cuda.synchronize()
    ref64, _ = oracle.gemm(M, N, K, dtype, A_bits, B_bits, bias_bits, epi)
    return to_bits(C_static), to_bits(C_ws), ref64


@pytest.mark.parametrize("dtype", [I.F16, I.BF16])
def test_static_split_matches_workspace_split_twice(dtype):
    calls = [
        # M, N, K, splits: 64 slabs x 4 splits, then 16 slabs x 8 splits
        (16, 4096, 4096, 4),
        (9, 1000, 2056, 8),
    ]
    for i, (M, N, K, splits) in enumerate(calls):
        for epi in (I.EPI_NONE, I.EPI_BIAS_GELU_TANH):
            what = f"static split {I.DTYPE_NAMES[dtype]} M={M} N={N} K={K} splits={splits} epi={epi} call {i}"
            log(f"[no-alloc] {what}")
            got, want, ref64 = _both(M, N, K, dtype, epi, splits, 52000 + 100 * i + 10 * dtype + epi)
            check_exact(got, want, what)
            check_tolerance(dtype, got, ref64, what)


@pytest.mark.parametrize("dtype", [I.F16, I.BF16])
def test_static_streamk_matches_workspace_streamk_twice(dtype):
    calls = [
        # M, N, K: 172 slabs over the CUs (427 partial blocks), then 17 slabs
        # (a smaller input whose partials overwrite the first call's)
        (16, 11008, 4096),
        (7, 1028, 1000),
    ]
    for i, (M, N, K) in enumerate(calls):
        for epi in (I.EPI_NONE, I.EPI_BIAS_GELU_TANH):
            what = f"static stream-K {I.DTYPE_NAMES[dtype]} M={M} N={N} K={K} epi={epi} call {i}"
            log(f"[no-alloc] {what}")
            got, want, ref64 = _both(M, N, K, dtype, epi, tg.TG_SPLIT_STREAM_K, 54000 + 100 * i + 10 * dtype + epi)
            check_exact(got, want, what)
            check_tolerance(dtype, got, ref64, what)


def test_static_split_library_choice_and_unsplit_shapes():
    # splits = 0 takes the plan's count; M > 16 and off-skinny shapes run as
    # tg_gemm and give its result.
    for M, N, K in ((16, 4096, 4096), (16, 11008, 4096), (40, 1024, 512), (300, 263, 201)):
        dtype, epi = I.F16, I.EPI_BIAS_GELU_TANH
        what = f"static split auto M={M} N={N} K={K}"
        log(f"[no-alloc] {what}")
        got, want, ref64 = _both(M, N, K, dtype, epi, 0, 53000 + M)
        check_exact(got, want, what)
        check_tolerance(dtype, got, ref64, what)

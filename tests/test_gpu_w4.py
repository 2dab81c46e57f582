"""GPU parity of the weight-only 4-bit product (tg_w4_pack + tg_gemm_w4)
against the oracle's gemm_w4, through the C interface.

Bar: the fused bar of the 16-bit product, |C - ref64| <= rtol (|ref64| + 1)
(rtol 1e-2 fp16, 2e-2 bf16) against the unrounded fp64 oracle, all outputs
finite; bit-exact with integer activations and power-of-two scales, where
every partial sum is exact in fp32.
"""
import numpy as np
import pytest

import oracle
import tiled_dense_gemm_tg_amd as tg
from tiled_dense_gemm_tg_amd import inputs as I
from gpu_util import check_exact, check_tolerance, log, to_bits, to_device

pytestmark = pytest.mark.gpu

EPI_NAME = {I.EPI_NONE: "none", I.EPI_BIAS: "bias", I.EPI_BIAS_GELU_TANH: "bias_gelu_tanh"}


def _run(M, N, K, G, dtype, A, Q, S, bias, epi):
    import torch
    q = torch.from_numpy(np.ascontiguousarray(Q)).cuda()
    packed = tg.w4_pack(q)
    a = to_device(A.reshape(M, K), dtype) if M * K else torch.empty((M, K), dtype=torch.float16, device="cuda")
    s = to_device(S.reshape(-1), dtype)
    b = to_device(bias, dtype) if bias is not None else None
    out = torch.full((M, N), float("nan"), dtype=a.dtype, device="cuda")
    tg.gemm_w4(a, packed, s, G, N, b, EPI_NAME[epi], out=out)
    torch.cuda.synchronize()
    return to_bits(out)


@pytest.mark.parametrize("dtype,M,N,K,G,epi", [
    (I.F16, 16, 11008, 4096, 128, I.EPI_NONE),           # the decode shape
    (I.BF16, 16, 11008, 4096, 128, I.EPI_BIAS_GELU_TANH),
    (I.F16, 1, 64, 32, 32, I.EPI_BIAS),
    (I.F16, 13, 1000, 256, 64, I.EPI_BIAS_GELU_TANH),    # ragged N, M < 16
    (I.BF16, 40, 300, 512, 256, I.EPI_BIAS),             # several 16-row blocks
    (I.F16, 7, 72, 96, 32, I.EPI_NONE),                  # fewer groups than waves
    (I.F16, 9, 1001, 256, 64, I.EPI_BIAS),               # N % 4 != 0: scales read element by element
    (I.BF16, 16, 70, 128, 32, I.EPI_BIAS_GELU_TANH),
    # A staged through LDS (every wave's groups span 9..16 steps of 32 k)
    (I.F16, 5, 388, 3584, 128, I.EPI_BIAS_GELU_TANH),   # 3 or 4 groups per wave, ragged N, M < 16
    (I.BF16, 20, 264, 4096, 64, I.EPI_BIAS),            # two 16-row blocks, the second partial
    (I.F16, 16, 388, 4096, 256, I.EPI_NONE),            # two 256-k groups per wave
])
def test_w4_matches_oracle(dtype, M, N, K, G, epi):
    A = I.random_bits((M, K), ("normal", 0.0, 1.0), dtype, 500 + M)
    Q = I.w4_weights(K, N, 501 + M)
    S = I.random_bits((K // G, N), ("uniform", 0.001, 0.01), dtype, 502 + M)
    bias = I.random_bits((N,), ("uniform", -0.5, 0.5), dtype, 503 + M) if epi else None
    ref64, _ = oracle.gemm_w4(M, N, K, dtype, A, Q, S, G, bias, epi)
    log(f"[w4] dtype={dtype} M={M} N={N} K={K} G={G} epi={epi}")
    check_tolerance(dtype, _run(M, N, K, G, dtype, A, Q, S, bias, epi), ref64, "w4")


@pytest.mark.parametrize("dtype", [I.F16, I.BF16])
@pytest.mark.parametrize("G", [32, 64, 128, 256])
def test_w4_integers_bit_exact(dtype, G):
    M, N, K = 16, 200, 512
    rng = np.random.Generator(np.random.PCG64(510 + G))
    A = I.small_int_bits((M, K), dtype, 511 + G)
    Q = I.w4_weights(K, N, 512 + G)
    S = I.values_bits(2.0 ** rng.integers(-3, 2, size=(K // G, N)), dtype)
    bias = I.small_int_bits((N,), dtype, 513 + G)
    _, refq = oracle.gemm_w4(M, N, K, dtype, A, Q, S, G, bias, I.EPI_BIAS)
    log(f"[w4 exact] dtype={dtype} G={G}")
    check_exact(_run(M, N, K, G, dtype, A, Q, S, bias, I.EPI_BIAS), refq, "w4 integers")


def test_w4_empty_K_gives_epilogue_of_zero():
    import torch
    M, N = 5, 70
    bias = I.random_bits((N,), ("uniform", -2.0, 2.0), I.F16, 520)
    _, refq = oracle.gemm_w4(M, N, 0, I.F16, None, None, None, 32, bias, I.EPI_BIAS_GELU_TANH)
    b = to_device(bias, I.F16)
    out = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    log("[w4 K=0]")
    st = tg.tg_gemm_w4(M, N, 0, I.F16, None, None, None, 32, b.data_ptr(), I.EPI_BIAS_GELU_TANH, out.data_ptr(),
                       torch.cuda.current_stream().cuda_stream)
    assert st == tg.TG_OK
    torch.cuda.synchronize()
    check_exact(to_bits(out), refq, "w4 K=0")


@pytest.mark.parametrize("dtype", [I.F16, I.BF16])
def test_w4_scales_at_any_alignment(dtype):
    """Scales starting 2 bytes past an 8-byte boundary (N % 4 == 0) take the
    element-by-element scale loads; integer operands, exact."""
    import torch
    M, N, K, G = 16, 264, 256, 64
    rng = np.random.Generator(np.random.PCG64(530))
    A = I.small_int_bits((M, K), dtype, 531)
    Q = I.w4_weights(K, N, 532)
    S = I.values_bits(2.0 ** rng.integers(-3, 2, size=(K // G, N)), dtype)
    _, refq = oracle.gemm_w4(M, N, K, dtype, A, Q, S, G)
    packed = tg.w4_pack(torch.from_numpy(np.ascontiguousarray(Q)).cuda())
    a = to_device(A.reshape(M, K), dtype)
    flat = to_device(np.concatenate([np.zeros(1, np.uint16), S.reshape(-1)]), dtype)
    s = flat[1:].view(K // G, N)
    assert s.data_ptr() % 8 != 0
    out = torch.full((M, N), float("nan"), dtype=a.dtype, device="cuda")
    log(f"[w4 scales 2-byte aligned] dtype={dtype}")
    tg.gemm_w4(a, packed, s, G, N, out=out)
    torch.cuda.synchronize()
    check_exact(to_bits(out), refq, "w4 misaligned scales")

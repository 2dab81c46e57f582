"""GPU parity of the unfused epilogue: the elementwise passes and the
three-launch product, through the C interface, against the CPU oracle.

Bar:
  * bias add: x + b is produced by the oracle as the product of an identity
    matrix with X plus the bias (every sum exact), so the result must be the
    oracle's rounded value, within one output ulp (the kernel adds in fp32 and
    rounds once more; bit-exact on small integers);
  * GELU: within two output ulps + 1e-6 of the oracle's fp64 GELU of the
    same 16-bit input, as for the fused epilogue;
  * the unfused product: the fused bar, |C - ref64| <= rtol (|ref64| + 1),
    against the oracle's fused fp64 result, and bit-exact with integer inputs
    and the bias epilogue (every intermediate is then exact).
"""
import numpy as np
import pytest

import oracle
import tiled_dense_gemm_tg_amd as tg
from tiled_dense_gemm_tg_amd import inputs as I
from gpu_util import check_exact, check_tolerance, log, run, to_bits, to_device

pytestmark = pytest.mark.gpu


def _ulp(dtype, v):
    frac_bits = 10 if dtype == I.F16 else 7
    min_exp = -14 if dtype == I.F16 else -126
    return 2.0 ** (np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** min_exp))) - frac_bits)


def _elementwise(op, X_bits, dtype, bias_bits=None, in_place=False, offset=0):
    """Runs tg_elementwise on a device copy of X (optionally at an element
    offset into a larger buffer, which breaks 16-byte alignment)."""
    import torch
    M, N = X_bits.shape
    flat = to_device(np.concatenate([np.zeros(offset, np.uint16), X_bits.reshape(-1)]), dtype)
    X = flat[offset:].view(M, N)
    bias = to_device(bias_bits, dtype) if bias_bits is not None else None
    out = X if in_place else torch.full((M, N), float("nan"), dtype=X.dtype, device="cuda")
    tg.elementwise(op, X, bias, out=out)
    torch.cuda.synchronize()
    return to_bits(out)


@pytest.mark.parametrize("dtype", [I.F16, I.BF16])
@pytest.mark.parametrize("M,N,offset", [(64, 4096, 0), (37, 4099, 0), (40, 1024, 1), (1, 8, 0)])
def test_bias_add_matches_oracle(dtype, M, N, offset):
    X = I.random_bits((M, N), ("normal", 0.0, 3.0), dtype, 300 + M)
    b = I.random_bits((N,), ("uniform", -2.0, 2.0), dtype, 301 + M)
    eye = I.values_bits(np.eye(M), dtype)
    ref64, refq = oracle.gemm(M, N, M, dtype, eye, X, b, I.EPI_BIAS)
    log(f"[ew bias] dtype={dtype} M={M} N={N} offset={offset}")
    got_bits = _elementwise("bias_add", X, dtype, b, offset=offset)
    got = oracle.decode(dtype, got_bits)
    assert np.isfinite(got).all()
    err = np.abs(got - oracle.decode(dtype, refq))
    assert (err <= _ulp(dtype, ref64)).all(), float((err / _ulp(dtype, ref64)).max())


@pytest.mark.parametrize("dtype", [I.F16, I.BF16])
def test_bias_add_small_integers_exact_and_in_place(dtype):
    M, N = 48, 2048
    X = I.small_int_bits((M, N), dtype, 310, -50, 50)
    b = I.small_int_bits((N,), dtype, 311, -50, 50)
    eye = I.values_bits(np.eye(M), dtype)
    _, refq = oracle.gemm(M, N, M, dtype, eye, X, b, I.EPI_BIAS)
    log(f"[ew bias exact] dtype={dtype}")
    check_exact(_elementwise("bias_add", X, dtype, b), refq, "bias add")
    check_exact(_elementwise("bias_add", X, dtype, b, in_place=True), refq, "bias add in place")


@pytest.mark.parametrize("dtype", [I.F16, I.BF16])
@pytest.mark.parametrize("N,offset", [(4096, 0), (4093, 0), (512, 3)])
def test_gelu_pass_within_two_ulps(dtype, N, offset):
    M = 64
    x = np.linspace(-6.0, 6.0, M * N).reshape(M, N)
    X = I.values_bits(x, dtype)
    ref64 = oracle.gelu_tanh(oracle.decode(dtype, X))
    log(f"[ew gelu] dtype={dtype} N={N} offset={offset}")
    got = oracle.decode(dtype, _elementwise("gelu_tanh", X, dtype, offset=offset))
    err = np.abs(got - ref64)
    bar = 2 * _ulp(dtype, ref64) + 1e-6
    assert (err <= bar).all(), float((err / bar).max())


@pytest.mark.parametrize("dtype,M,N,K,epi", [
    (I.F16, 256, 256, 256, I.EPI_BIAS_GELU_TANH),
    (I.BF16, 300, 263, 201, I.EPI_BIAS_GELU_TANH),
    (I.F16, 16, 1024, 512, I.EPI_BIAS_GELU_TANH),
    (I.F16, 520, 264, 328, I.EPI_BIAS),
])
def test_unfused_product_meets_the_fused_bar(dtype, M, N, K, epi):
    A = I.random_bits((M, K), ("uniform", -1.0, 1.0), dtype, 320)
    B = I.random_bits((K, N), ("uniform", -1.0, 1.0), dtype, 321)
    bias = I.random_bits((N,), ("uniform", -0.5, 0.5), dtype, 322)
    ref64, _ = oracle.gemm(M, N, K, dtype, A, B, bias, epi)
    log(f"[unfused] dtype={dtype} M={M} N={N} K={K} epi={epi}")
    import torch
    a, b, bb = to_device(A.reshape(M, K), dtype), to_device(B.reshape(K, N), dtype), to_device(bias, dtype)
    out = torch.full((M, N), float("nan"), dtype=a.dtype, device="cuda")
    tg.gemm(a, b, bb, {I.EPI_BIAS: "bias", I.EPI_BIAS_GELU_TANH: "bias_gelu_tanh"}[epi], out=out, unfused=True)
    torch.cuda.synchronize()
    check_tolerance(dtype, to_bits(out), ref64, "unfused")


def test_unfused_small_integers_bit_exact():
    import torch
    M, N, K = 300, 264, 200
    dtype = I.F16
    A = I.small_int_bits((M, K), dtype, 330)
    B = I.small_int_bits((K, N), dtype, 331)
    bias = I.small_int_bits((N,), dtype, 332)
    _, refq = oracle.gemm(M, N, K, dtype, A, B, bias, I.EPI_BIAS)
    log("[unfused exact]")
    a, b, bb = to_device(A.reshape(M, K), dtype), to_device(B.reshape(K, N), dtype), to_device(bias, dtype)
    out = tg.gemm(a, b, bb, "bias", unfused=True)
    torch.cuda.synchronize()
    check_exact(to_bits(out), refq, "unfused bias")

"""Helpers for the GPU parity tests: move 16-bit patterns to the device, run
the C interface on them, and compare with the oracle to the required bar."""
from __future__ import annotations

import sys

import numpy as np

import oracle
import tiled_dense_gemm_tg_amd as tg
from tiled_dense_gemm_tg_amd import inputs as I

# Tolerance on the unrounded fp64 oracle: |C - ref| <= RTOL * (|ref| + 1).
RTOL = {I.F16: 1e-2, I.BF16: 2e-2}


def log(msg: str) -> None:
    """Name the case on stdout before each GPU step (flushed)."""
    print(msg, flush=True)
    sys.stdout.flush()


def torch_dtype(dtype):
    import torch
    return torch.float16 if dtype == I.F16 else torch.bfloat16


def to_device(bits: np.ndarray, dtype, device="cuda"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy())
    return t.view(torch_dtype(dtype)).to(device)


def to_bits(t) -> np.ndarray:
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def run(M, N, K, dtype, A_bits, B_bits, bias_bits=None, epilogue=I.EPI_NONE, path=tg.TG_PATH_AUTO,
        out=None, stream=None, expect_path=None, tiles=tg.TG_TILES_AUTO, group_m=0):
    """Runs one GEMM through the C interface (tg_gemm_path, or tg_gemm_tiled
    when a tile configuration is given); returns the output tensor."""
    import torch
    dev = "cuda"
    A = to_device(A_bits.reshape(M, K), dtype) if M * K else torch.empty((M, K), dtype=torch_dtype(dtype), device=dev)
    B = to_device(B_bits.reshape(K, N), dtype) if K * N else torch.empty((K, N), dtype=torch_dtype(dtype), device=dev)
    bias = to_device(bias_bits, dtype) if bias_bits is not None else None
    if out is None:
        out = torch.full((M, N), float("nan"), dtype=torch_dtype(dtype), device=dev)
    if expect_path is not None:
        st, p = tg.tg_gemm_plan(M, N, K, dtype, A.data_ptr(), B.data_ptr(),
                                bias.data_ptr() if bias is not None else None, epilogue, out.data_ptr())
        assert st == tg.TG_OK and p == expect_path, (st, tg.PATH_NAMES.get(p))
    epi_name = {I.EPI_NONE: "none", I.EPI_BIAS: "bias", I.EPI_BIAS_GELU_TANH: "bias_gelu_tanh"}[epilogue]
    tg.gemm(A, B, bias, epi_name, out=out, path=path, stream=stream, tiles=tiles, group_m=group_m)
    torch.cuda.synchronize()
    return out


def check_tolerance(dtype, got_bits: np.ndarray, ref64: np.ndarray, what: str = ""):
    got = oracle.decode(dtype, got_bits)
    assert np.isfinite(got).all(), f"{what}: non-finite outputs at {np.argwhere(~np.isfinite(got))[:5].tolist()}"
    ratio = np.abs(got - ref64) / (RTOL[dtype] * (np.abs(ref64) + 1.0))
    worst = float(ratio.max()) if ratio.size else 0.0
    assert worst <= 1.0, f"{what}: max |C-ref|/(rtol(|ref|+1)) = {worst:.3f} at {np.unravel_index(ratio.argmax(), ratio.shape)}"
    return worst


def check_exact(got_bits: np.ndarray, refq: np.ndarray, what: str = ""):
    bad = np.argwhere(got_bits != refq)
    assert bad.size == 0, f"{what}: {len(bad)} mismatching elements, first {bad[:5].tolist()}"

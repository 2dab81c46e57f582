"""MI355X-native tiled half-precision GEMM (gfx950), behind a C-ABI library.

Thin ctypes binding of ``libtg_gemm.so`` (include/tg_gemm.h).  Functions with
the C names take raw integers (device pointers, a hipStream_t handle) and
return the C status; :func:`gemm` is a convenience over torch tensors that
passes their device pointers and torch's current stream.  Every step of the
computation runs in the HIP kernels; this module only marshals arguments.
If the library has not been built this module raises instead of falling back
to anything else.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

from .inputs import BF16, EPI_BIAS, EPI_BIAS_GELU_TANH, EPI_NONE, F16  # noqa: F401

PKG = os.path.dirname(os.path.abspath(__file__))
# TG_GEMM_LIBRARY lets the sanitizer test load an instrumented build of the
# same sources.
LIBRARY = os.environ.get("TG_GEMM_LIBRARY") or os.path.join(PKG, "libtg_gemm.so")

TG_OK = 0
TG_ERR_INVALID_ARG = 1
TG_ERR_UNSUPPORTED = 2
TG_ERR_LAUNCH = 3

TG_PATH_AUTO = 0
TG_PATH_TILED = 1
TG_PATH_TILED_GENERIC = 2
TG_PATH_SKINNY = 3
TG_PATH_NONE = 4
PATH_NAMES = {TG_PATH_AUTO: "auto", TG_PATH_TILED: "tiled", TG_PATH_TILED_GENERIC: "tiled_generic",
              TG_PATH_SKINNY: "skinny", TG_PATH_NONE: "none"}

TG_EW_BIAS_ADD = 0
TG_EW_GELU_TANH = 1

TG_SPLIT_STREAM_K = -1   # tg_gemm_split: stream-K division of all slabs' 32-k steps over the CUs

TG_TILES_AUTO = 0
TG_TILES_256x256 = 1
TG_TILES_256x128 = 2
TG_TILES_128x256 = 3
TG_TILES_128x128 = 4
TG_TILES_256x256_K64 = 5
TG_TILES_256x128_K64 = 6
TG_TILES_128x256_K64 = 7
TG_TILES_128x128_K64 = 8
TG_TILES_256x256_W8 = 9
TILES_NAMES = {TG_TILES_AUTO: "auto", TG_TILES_256x256: "256x256", TG_TILES_256x128: "256x128",
               TG_TILES_128x256: "128x256", TG_TILES_128x128: "128x128",
               TG_TILES_256x256_K64: "256x256_k64", TG_TILES_256x128_K64: "256x128_k64",
               TG_TILES_128x256_K64: "128x256_k64", TG_TILES_128x128_K64: "128x128_k64",
               TG_TILES_256x256_W8: "256x256_w8"}
# (BM, BN, BK, stages, waves) of each configuration
TILES_AXES = {TG_TILES_256x256: (256, 256, 32, 4, 4), TG_TILES_256x128: (256, 128, 32, 4, 4),
              TG_TILES_128x256: (128, 256, 32, 4, 4), TG_TILES_128x128: (128, 128, 32, 4, 4),
              TG_TILES_256x256_K64: (256, 256, 64, 2, 4), TG_TILES_256x128_K64: (256, 128, 64, 3, 4),
              TG_TILES_128x256_K64: (128, 256, 64, 3, 4), TG_TILES_128x128_K64: (128, 128, 64, 2, 4),
              TG_TILES_256x256_W8: (256, 256, 32, 4, 8)}

EXPORTED = ("tg_gemm", "tg_gemm_path", "tg_gemm_plan", "tg_gemm_tiled", "tg_gemm_tiled_grouped", "tg_gemm_tiles_plan",
            "tg_gemm_split",
            "tg_gemm_split_workspace_bytes", "tg_gemm_split_plan", "tg_gemm_split_static", "tg_elementwise", "tg_gemm_unfused",
            "tg_w4_packed_bytes", "tg_w4_pack", "tg_gemm_w4", "tg_gemm_w4_split", "tg_gemm_w4_split_workspace_bytes",
            "tg_gemm_w4_split_plan", "tg_attention_fwd", "tg_status_string", "tg_version")

_lib = None


class TgError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {tg_status_string(status)} ({status})")
        self.status = status


def load_library():
    """Load libtg_gemm.so (after torch, so both share one HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY):
        raise RuntimeError(f"{LIBRARY} is not built; run `python -m tiled_dense_gemm_tg_amd.build` "
                           "(or __graft_entry__.build()) first")
    try:
        import torch  # noqa: F401  -- loads the HIP runtime the library must share
    except ImportError:
        pass
    lib = ctypes.CDLL(LIBRARY)
    i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.tg_gemm.argtypes = [i64, i64, i64, ci, vp, vp, vp, ci, vp, vp]
    lib.tg_gemm.restype = ci
    lib.tg_gemm_path.argtypes = [ci, i64, i64, i64, ci, vp, vp, vp, ci, vp, vp]
    lib.tg_gemm_path.restype = ci
    lib.tg_gemm_plan.argtypes = [i64, i64, i64, ci, vp, vp, vp, ci, vp, ctypes.POINTER(ci)]
    lib.tg_gemm_plan.restype = ci
    lib.tg_gemm_tiled.argtypes = [ci, i64, i64, i64, ci, vp, vp, vp, ci, vp, vp]
    lib.tg_gemm_tiled.restype = ci
    lib.tg_gemm_tiled_grouped.argtypes = [ci, ci, i64, i64, i64, ci, vp, vp, vp, ci, vp, vp]
    lib.tg_gemm_tiled_grouped.restype = ci
    lib.tg_gemm_tiles_plan.argtypes = [i64, i64, i64, ci, ctypes.POINTER(ci)]
    lib.tg_gemm_tiles_plan.restype = ci
    lib.tg_gemm_split.argtypes = [ci, i64, i64, i64, ci, vp, vp, vp, ci, vp, vp, i64, vp]
    lib.tg_gemm_split.restype = ci
    lib.tg_gemm_split_static.argtypes = [ci, i64, i64, i64, ci, vp, vp, vp, ci, vp, vp]
    lib.tg_gemm_split_static.restype = ci
    lib.tg_gemm_split_workspace_bytes.argtypes = [i64, ci]
    lib.tg_gemm_split_workspace_bytes.restype = i64
    lib.tg_gemm_split_plan.argtypes = [i64, i64, i64, ci, ctypes.POINTER(ci), ctypes.POINTER(i64)]
    lib.tg_gemm_split_plan.restype = ci
    lib.tg_elementwise.argtypes = [ci, i64, i64, ci, vp, vp, vp, vp]
    lib.tg_elementwise.restype = ci
    lib.tg_gemm_unfused.argtypes = [i64, i64, i64, ci, vp, vp, vp, ci, vp, vp]
    lib.tg_gemm_unfused.restype = ci
    lib.tg_w4_packed_bytes.argtypes = [i64, i64]
    lib.tg_w4_packed_bytes.restype = i64
    lib.tg_w4_pack.argtypes = [i64, i64, vp, vp, vp]
    lib.tg_w4_pack.restype = ci
    lib.tg_gemm_w4.argtypes = [i64, i64, i64, ci, vp, vp, vp, i64, vp, ci, vp, vp]
    lib.tg_gemm_w4.restype = ci
    lib.tg_gemm_w4_split.argtypes = [ci, i64, i64, i64, ci, vp, vp, vp, i64, vp, ci, vp, vp, i64, vp]
    lib.tg_gemm_w4_split.restype = ci
    lib.tg_gemm_w4_split_workspace_bytes.argtypes = [i64, i64, ci]
    lib.tg_gemm_w4_split_workspace_bytes.restype = i64
    lib.tg_gemm_w4_split_plan.argtypes = [i64, i64, i64, i64, ci, ctypes.POINTER(ci), ctypes.POINTER(i64)]
    lib.tg_gemm_w4_split_plan.restype = ci
    lib.tg_attention_fwd.argtypes = [i64, i64, i64, i64, i64, ci, vp, vp, vp, ci, ctypes.c_float, vp, vp]
    lib.tg_attention_fwd.restype = ci
    lib.tg_status_string.argtypes = [ci]
    lib.tg_status_string.restype = ctypes.c_char_p
    lib.tg_version.argtypes = []
    lib.tg_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def tg_gemm(M, N, K, dtype, A, B, bias, epilogue, C, stream) -> int:
    """C-ABI tg_gemm: pointers and stream are integers (0 / None for NULL)."""
    return load_library().tg_gemm(M, N, K, dtype, A, B, bias, epilogue, C, stream)


def tg_gemm_path(path, M, N, K, dtype, A, B, bias, epilogue, C, stream) -> int:
    return load_library().tg_gemm_path(path, M, N, K, dtype, A, B, bias, epilogue, C, stream)


def tg_gemm_plan(M, N, K, dtype, A, B, bias, epilogue, C):
    """Returns (status, path) without touching the GPU."""
    out = ctypes.c_int(-1)
    st = load_library().tg_gemm_plan(M, N, K, dtype, A, B, bias, epilogue, C, ctypes.byref(out))
    return st, out.value


def tg_gemm_tiled(tiles, M, N, K, dtype, A, B, bias, epilogue, C, stream) -> int:
    return load_library().tg_gemm_tiled(tiles, M, N, K, dtype, A, B, bias, epilogue, C, stream)


def tg_gemm_tiled_grouped(tiles, group_m, M, N, K, dtype, A, B, bias, epilogue, C, stream) -> int:
    return load_library().tg_gemm_tiled_grouped(tiles, group_m, M, N, K, dtype, A, B, bias, epilogue, C, stream)


def tg_gemm_tiles_plan(M, N, K, num_cu=0):
    """Returns (status, tile configuration TG_TILES_AUTO would use)."""
    out = ctypes.c_int(-1)
    st = load_library().tg_gemm_tiles_plan(M, N, K, num_cu, ctypes.byref(out))
    return st, out.value


def tg_gemm_split(splits, M, N, K, dtype, A, B, bias, epilogue, C, workspace, workspace_bytes, stream) -> int:
    return load_library().tg_gemm_split(splits, M, N, K, dtype, A, B, bias, epilogue, C, workspace,
                                        workspace_bytes, stream)


def tg_gemm_split_static(splits, M, N, K, dtype, A, B, bias, epilogue, C, stream) -> int:
    """tg_gemm_split with the library's static workspace (no allocation)."""
    return load_library().tg_gemm_split_static(splits, M, N, K, dtype, A, B, bias, epilogue, C, stream)


def tg_gemm_split_workspace_bytes(N, splits) -> int:
    return load_library().tg_gemm_split_workspace_bytes(N, splits)


def tg_gemm_split_plan(M, N, K, num_cu=0):
    """Returns (status, splits, workspace bytes) that tg_gemm_split(0, ...) uses."""
    splits, nbytes = ctypes.c_int(-1), ctypes.c_int64(-1)
    st = load_library().tg_gemm_split_plan(M, N, K, num_cu, ctypes.byref(splits), ctypes.byref(nbytes))
    return st, splits.value, nbytes.value


def split_workspace(M, N, K, splits=0, device=None):
    """A zero-filled workspace (uint8 torch tensor) for tg_gemm_split with
    `splits` (0: the mode the library chooses on `device`; TG_SPLIT_STREAM_K:
    enough for stream-K on any device), or None when that needs none."""
    import torch
    device = torch.device("cuda" if device is None else device)
    if splits == 0:
        cus = torch.cuda.get_device_properties(device).multi_processor_count
        st, _, nbytes = tg_gemm_split_plan(M, N, K, cus)
        if st != TG_OK:
            raise TgError(st, "tg_gemm_split_plan")
    else:
        nbytes = tg_gemm_split_workspace_bytes(N, splits)
        if nbytes < 0:
            raise TgError(TG_ERR_INVALID_ARG, "tg_gemm_split_workspace_bytes")
    return torch.zeros(nbytes, dtype=torch.uint8, device=device) if nbytes > 0 else None


def tg_elementwise(op, M, N, dtype, bias, X, Y, stream) -> int:
    return load_library().tg_elementwise(op, M, N, dtype, bias, X, Y, stream)


def tg_gemm_unfused(M, N, K, dtype, A, B, bias, epilogue, C, stream) -> int:
    return load_library().tg_gemm_unfused(M, N, K, dtype, A, B, bias, epilogue, C, stream)


def tg_w4_packed_bytes(K, N) -> int:
    return load_library().tg_w4_packed_bytes(K, N)


def tg_w4_pack(K, N, q, packed, stream) -> int:
    return load_library().tg_w4_pack(K, N, q, packed, stream)


def tg_gemm_w4(M, N, K, dtype, A, packed, scales, group, bias, epilogue, C, stream) -> int:
    return load_library().tg_gemm_w4(M, N, K, dtype, A, packed, scales, group, bias, epilogue, C, stream)


def tg_gemm_w4_split(splits, M, N, K, dtype, A, packed, scales, group, bias, epilogue, C, workspace,
                     workspace_bytes, stream) -> int:
    return load_library().tg_gemm_w4_split(splits, M, N, K, dtype, A, packed, scales, group, bias, epilogue, C,
                                           workspace, workspace_bytes, stream)


def tg_gemm_w4_split_workspace_bytes(M, N, splits) -> int:
    return load_library().tg_gemm_w4_split_workspace_bytes(M, N, splits)


def tg_gemm_w4_split_plan(M, N, K, group, num_cu=0):
    """Returns (status, splits, workspace bytes) that tg_gemm_w4_split(0, ...) uses."""
    splits, nbytes = ctypes.c_int(-1), ctypes.c_int64(-1)
    st = load_library().tg_gemm_w4_split_plan(M, N, K, group, num_cu, ctypes.byref(splits), ctypes.byref(nbytes))
    return st, splits.value, nbytes.value


def w4_split_workspace(M, N, K, group, splits=0, device=None):
    """A zero-filled workspace (uint8 torch tensor) for tg_gemm_w4_split with
    `splits` (0: the count the library chooses on `device`), or None when
    that needs none."""
    import torch
    device = torch.device("cuda" if device is None else device)
    if splits == 0:
        cus = torch.cuda.get_device_properties(device).multi_processor_count
        st, _, nbytes = tg_gemm_w4_split_plan(M, N, K, group, cus)
        if st != TG_OK:
            raise TgError(st, "tg_gemm_w4_split_plan")
    else:
        nbytes = tg_gemm_w4_split_workspace_bytes(M, N, splits)
        if nbytes < 0:
            raise TgError(TG_ERR_INVALID_ARG, "tg_gemm_w4_split_workspace_bytes")
    return torch.zeros(nbytes, dtype=torch.uint8, device=device) if nbytes > 0 else None


def tg_attention_fwd(batch, Sq, Sk, heads, head_dim, dtype, Q, K, V, causal, scale, O, stream) -> int:
    return load_library().tg_attention_fwd(batch, Sq, Sk, heads, head_dim, dtype, Q, K, V, causal, scale, O, stream)


def tg_status_string(status: int) -> str:
    return load_library().tg_status_string(status).decode()


def tg_version() -> str:
    return load_library().tg_version().decode()


_EPI = {"none": EPI_NONE, "bias": EPI_BIAS, "bias_gelu_tanh": EPI_BIAS_GELU_TANH, "gelu": EPI_BIAS_GELU_TANH}


def gemm(A, B, bias=None, epilogue: str = "none", out=None, path: int = TG_PATH_AUTO, stream=None,
         unfused: bool = False, tiles: int = TG_TILES_AUTO, splits=None, workspace=None, group_m: int = 0):
    """epilogue(A @ B [+ bias]) on torch device tensors (fp16 or bf16, row-major).

    Returns ``out`` (allocated when not given).  Runs on ``stream`` or torch's
    current stream; asynchronous like any torch op.  ``unfused=True`` calls
    tg_gemm_unfused (the product, then the epilogue steps as separate passes;
    ``path`` must then be TG_PATH_AUTO).  A ``tiles`` configuration other than
    TG_TILES_AUTO calls tg_gemm_tiled (the tiled family with that tile size;
    ``path`` must then be TG_PATH_AUTO or TG_PATH_TILED); ``group_m`` > 0 sets
    the tile rows per raster group of that call (tg_gemm_tiled_grouped).
    ``splits`` (0 for
    the library's choice, 2..64 even splits, TG_SPLIT_STREAM_K for stream-K
    over the CUs) calls tg_gemm_split with ``workspace`` (a
    zero-filled uint8 GPU tensor from :func:`split_workspace`, allocated here
    when not given; reuse one per stream to skip that); ``path`` must then be
    TG_PATH_AUTO.
    """
    import torch
    if A.dtype not in (torch.float16, torch.bfloat16):
        raise TypeError("A must be float16 or bfloat16")
    if B.dtype != A.dtype or (bias is not None and bias.dtype != A.dtype):
        raise TypeError("A, B and bias must share one dtype")
    if A.dim() != 2 or B.dim() != 2 or A.shape[1] != B.shape[0]:
        raise ValueError(f"shapes {tuple(A.shape)} @ {tuple(B.shape)} do not chain")
    for name, t in (("A", A), ("B", B), ("bias", bias), ("out", out)):
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    M, K = A.shape
    N = B.shape[1]
    epi = _EPI[epilogue]
    if (epi == EPI_NONE) != (bias is None):
        raise ValueError("bias must be given exactly when the epilogue uses it")
    if bias is not None and bias.numel() != N:
        raise ValueError("bias must have N entries")
    if out is None:
        out = torch.empty((M, N), dtype=A.dtype, device=A.device)
    elif out.shape != (M, N) or out.dtype != A.dtype:
        raise ValueError("out has the wrong shape or dtype")
    dtype = F16 if A.dtype == torch.float16 else BF16
    s = (stream if stream is not None else torch.cuda.current_stream(A.device)).cuda_stream
    if (tiles != TG_TILES_AUTO or group_m) and (unfused or path not in (TG_PATH_AUTO, TG_PATH_TILED)):
        raise ValueError("a tile configuration applies to the tiled family only")
    if splits is not None and (unfused or path != TG_PATH_AUTO or tiles != TG_TILES_AUTO):
        raise ValueError("split-K goes with the library's own choice of kernel")
    if workspace is not None and splits is None:
        raise ValueError("a workspace goes with split-K (splits)")
    if splits is not None:
        if workspace is None:
            workspace = split_workspace(M, N, K, splits, A.device)
        elif workspace.dtype != torch.uint8 or not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous uint8 GPU tensor")
        st = tg_gemm_split(splits, M, N, K, dtype, A.data_ptr(), B.data_ptr(),
                           bias.data_ptr() if bias is not None else None, epi, out.data_ptr(),
                           workspace.data_ptr() if workspace is not None else None,
                           workspace.numel() if workspace is not None else 0, s)
        if st != TG_OK:
            raise TgError(st, "tg_gemm_split")
        return out
    if unfused:
        if path != TG_PATH_AUTO:
            raise ValueError("the unfused form chooses its own kernel family")
        st = tg_gemm_unfused(M, N, K, dtype, A.data_ptr(), B.data_ptr(),
                             bias.data_ptr() if bias is not None else None, epi, out.data_ptr(), s)
    elif tiles != TG_TILES_AUTO or group_m:
        st = tg_gemm_tiled_grouped(tiles, group_m, M, N, K, dtype, A.data_ptr(), B.data_ptr(),
                                   bias.data_ptr() if bias is not None else None, epi, out.data_ptr(), s)
    else:
        st = tg_gemm_path(path, M, N, K, dtype, A.data_ptr(), B.data_ptr(),
                          bias.data_ptr() if bias is not None else None, epi, out.data_ptr(), s)
    if st != TG_OK:
        raise TgError(st, "tg_gemm_unfused" if unfused else "tg_gemm")
    return out


_EW = {"bias_add": TG_EW_BIAS_ADD, "gelu_tanh": TG_EW_GELU_TANH}


def elementwise(op: str, X, bias=None, out=None, stream=None):
    """One elementwise epilogue step over a 2-D torch device tensor: ``op`` is
    "bias_add" (X + bias[n], bias of N entries) or "gelu_tanh".  ``out`` may
    be X itself (in place); allocated when not given."""
    import torch
    if X.dtype not in (torch.float16, torch.bfloat16) or X.dim() != 2:
        raise TypeError("X must be a 2-D float16 or bfloat16 tensor")
    ew = _EW[op]
    if (ew == TG_EW_BIAS_ADD) != (bias is not None):
        raise ValueError("bias must be given exactly for bias_add")
    M, N = X.shape
    if bias is not None and (bias.numel() != N or bias.dtype != X.dtype):
        raise ValueError("bias must have N entries of X's dtype")
    if out is None:
        out = torch.empty_like(X)
    elif out.shape != X.shape or out.dtype != X.dtype:
        raise ValueError("out has the wrong shape or dtype")
    for name, t in (("X", X), ("bias", bias), ("out", out)):
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    dtype = F16 if X.dtype == torch.float16 else BF16
    s = (stream if stream is not None else torch.cuda.current_stream(X.device)).cuda_stream
    st = tg_elementwise(ew, M, N, dtype, bias.data_ptr() if bias is not None else None, X.data_ptr(),
                        out.data_ptr(), s)
    if st != TG_OK:
        raise TgError(st, "tg_elementwise")
    return out


def w4_pack(q, stream=None):
    """Packs 4-bit weights ``q`` (a (K, N) uint8 GPU tensor, values 0..15)
    into the layout :func:`gemm_w4` reads; returns a new uint8 tensor."""
    import torch
    if q.dtype != torch.uint8 or q.dim() != 2 or not q.is_cuda or not q.is_contiguous():
        raise TypeError("q must be a contiguous 2-D uint8 GPU tensor")
    K, N = q.shape
    nbytes = tg_w4_packed_bytes(K, N)
    if nbytes < 0:
        raise ValueError("K must be a multiple of 32")
    packed = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    s = (stream if stream is not None else torch.cuda.current_stream(q.device)).cuda_stream
    st = tg_w4_pack(K, N, q.data_ptr(), packed.data_ptr(), s)
    if st != TG_OK:
        raise TgError(st, "tg_w4_pack")
    return packed


def gemm_w4(A, packed, scales, group: int, N: int, bias=None, epilogue: str = "none", out=None, stream=None,
            splits=None, workspace=None):
    """epilogue(A @ W [+ bias]) with W[k, n] = (q[k, n] - 8) * scales[k // group, n]
    and q packed by :func:`w4_pack`; A (M, K) and scales (K // group, N) share
    one 16-bit dtype.  ``splits`` (0 for the library's choice) calls
    tg_gemm_w4_split with ``workspace`` (from :func:`w4_split_workspace`,
    allocated here when not given)."""
    import torch
    if A.dtype not in (torch.float16, torch.bfloat16) or A.dim() != 2:
        raise TypeError("A must be a 2-D float16 or bfloat16 tensor")
    M, K = A.shape
    if scales.dtype != A.dtype or scales.numel() != (K // group) * N:
        raise ValueError("scales must be (K // group, N) of A's dtype")
    epi = _EPI[epilogue]
    if (epi == EPI_NONE) != (bias is None):
        raise ValueError("bias must be given exactly when the epilogue uses it")
    if out is None:
        out = torch.empty((M, N), dtype=A.dtype, device=A.device)
    for name, t in (("A", A), ("packed", packed), ("scales", scales), ("bias", bias), ("out", out)):
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    dtype = F16 if A.dtype == torch.float16 else BF16
    s = (stream if stream is not None else torch.cuda.current_stream(A.device)).cuda_stream
    if workspace is not None and splits is None:
        raise ValueError("a workspace goes with split-K (splits)")
    if splits is not None:
        if workspace is None:
            workspace = w4_split_workspace(M, N, K, group, splits, A.device)
        elif workspace.dtype != torch.uint8 or not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous uint8 GPU tensor")
        st = tg_gemm_w4_split(splits, M, N, K, dtype, A.data_ptr(), packed.data_ptr(), scales.data_ptr(), group,
                              bias.data_ptr() if bias is not None else None, epi, out.data_ptr(),
                              workspace.data_ptr() if workspace is not None else None,
                              workspace.numel() if workspace is not None else 0, s)
        if st != TG_OK:
            raise TgError(st, "tg_gemm_w4_split")
        return out
    st = tg_gemm_w4(M, N, K, dtype, A.data_ptr(), packed.data_ptr(), scales.data_ptr(), group,
                    bias.data_ptr() if bias is not None else None, epi, out.data_ptr(), s)
    if st != TG_OK:
        raise TgError(st, "tg_gemm_w4")
    return out


def attention(Q, K, V, causal: bool = False, scale: float = 0.0, out=None, stream=None):
    """softmax(scale Q K^T) V over BSHD tensors: Q (batch, Sq, heads, 128),
    K and V (batch, Sk, heads, 128), one 16-bit dtype; ``scale`` 0 means
    1/sqrt(128).  Returns ``out`` (allocated like Q when not given)."""
    import torch
    if Q.dtype not in (torch.float16, torch.bfloat16) or Q.dim() != 4:
        raise TypeError("Q must be a 4-D float16 or bfloat16 tensor (batch, seq, heads, dim)")
    Bn, Sq, H, Dh = Q.shape
    if K.shape != V.shape or K.dim() != 4 or K.shape[0] != Bn or K.shape[2] != H or K.shape[3] != Dh:
        raise ValueError("K and V must be (batch, Sk, heads, dim) matching Q")
    if K.dtype != Q.dtype or V.dtype != Q.dtype:
        raise TypeError("Q, K and V must share one dtype")
    if out is None:
        out = torch.empty_like(Q)
    for name, t in (("Q", Q), ("K", K), ("V", V), ("out", out)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    dtype = F16 if Q.dtype == torch.float16 else BF16
    s = (stream if stream is not None else torch.cuda.current_stream(Q.device)).cuda_stream
    st = tg_attention_fwd(Bn, Sq, K.shape[1], H, Dh, dtype, Q.data_ptr(), K.data_ptr(), V.data_ptr(),
                          1 if causal else 0, float(scale), out.data_ptr(), s)
    if st != TG_OK:
        raise TgError(st, "tg_attention_fwd")
    return out

"""CPU oracle for the tiled half-precision GEMM (test infrastructure only).

Only ``tests/``, the smoke check and the bench's CPU-baseline leg may import
this package.  It wraps ``libtg_oracle.so`` (plain C + OpenMP, built from
``tg_oracle.c`` beside this file with gcc) through ctypes.  It shares no code
with the GEMM library: its own 16-bit decoder/encoder, fp64 accumulation in
ascending k and an fp64 GELU(tanh) epilogue, written from the definition of
the matrix product on the first TileLang page (section 2) and the
GELU(MatMul + Bias) epilogue on the fourth (part 3, "Epilogue fusion").

All pins of this oracle (what checks it against something other than itself)
live in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "tg_oracle.c")
# TG_ORACLE_LIBRARY lets the mutation tests load a deliberately broken copy.
LIBRARY = os.environ.get("TG_ORACLE_LIBRARY") or os.path.join(HERE, "libtg_oracle.so")

# The oracle's own numbering of formats and epilogues.
F16 = 0
BF16 = 1
EPI_NONE = 0
EPI_BIAS = 1
EPI_BIAS_GELU_TANH = 2

_lib = None


def build(force: bool = True) -> str:
    """Compile libtg_oracle.so with gcc (plain C11, OpenMP, no fast-math)."""
    if force or not os.path.exists(LIBRARY):
        tmp = LIBRARY + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, SOURCE, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIBRARY)
    return LIBRARY


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            build(force=True)
        lib = ctypes.CDLL(LIBRARY)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        f64p = ctypes.POINTER(ctypes.c_double)
        i64p = ctypes.POINTER(ctypes.c_int64)
        i64 = ctypes.c_int64
        lib.tg_oracle_decode.argtypes = [ctypes.c_int, u16p, f64p, i64]
        lib.tg_oracle_encode.argtypes = [ctypes.c_int, f64p, u16p, i64]
        lib.tg_oracle_gelu_tanh.argtypes = [f64p, f64p, i64]
        lib.tg_oracle_max_threads.argtypes = []
        lib.tg_oracle_gemm.argtypes = [i64, i64, i64, ctypes.c_int, u16p, u16p, u16p, ctypes.c_int,
                                       i64p, i64, f64p, u16p]
        u8p = ctypes.POINTER(ctypes.c_uint8)
        lib.tg_oracle_gemm_w4.argtypes = [i64, i64, i64, ctypes.c_int, u16p, u8p, u16p, i64, u16p, ctypes.c_int,
                                          i64p, i64, f64p, u16p]
        lib.tg_oracle_attention.argtypes = [i64, i64, i64, i64, i64, ctypes.c_int, u16p, u16p, u16p, ctypes.c_int,
                                            ctypes.c_double, i64p, i64, f64p, u16p]
        for f in (lib.tg_oracle_decode, lib.tg_oracle_encode, lib.tg_oracle_gelu_tanh,
                  lib.tg_oracle_max_threads, lib.tg_oracle_gemm, lib.tg_oracle_gemm_w4, lib.tg_oracle_attention):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray], ctype):
    if a is None:
        return ctypes.cast(None, ctypes.POINTER(ctype))
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"expected uint16 bit patterns, got {a.dtype}")
    return a


def decode(dtype: int, bits) -> np.ndarray:
    bits = _u16(bits)
    out = np.empty(bits.shape, dtype=np.float64)
    rc = _load().tg_oracle_decode(dtype, _ptr(bits, ctypes.c_uint16), _ptr(out, ctypes.c_double), bits.size)
    if rc != 0:
        raise ValueError(f"tg_oracle_decode failed ({rc})")
    return out


def encode(dtype: int, values) -> np.ndarray:
    v = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    rc = _load().tg_oracle_encode(dtype, _ptr(v, ctypes.c_double), _ptr(out, ctypes.c_uint16), v.size)
    if rc != 0:
        raise ValueError(f"tg_oracle_encode failed ({rc})")
    return out


def gelu_tanh(x) -> np.ndarray:
    v = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.float64)
    rc = _load().tg_oracle_gelu_tanh(_ptr(v, ctypes.c_double), _ptr(out, ctypes.c_double), v.size)
    if rc != 0:
        raise ValueError(f"tg_oracle_gelu_tanh failed ({rc})")
    return out


def max_threads() -> int:
    return int(_load().tg_oracle_max_threads())


def gemm(M: int, N: int, K: int, dtype: int, A, B, bias=None, epilogue: int = EPI_NONE,
         rows=None) -> Tuple[np.ndarray, np.ndarray]:
    """Rows ``rows`` (default: all) of epilogue(A @ B [+ bias]).

    A: (M, K) and B: (K, N) uint16 bit patterns, bias: (N,) or None.
    Returns (ref64, refq): the fp64 result and its RNE-rounded 16-bit bits,
    both of shape (len(rows), N).
    """
    A = _u16(A) if K > 0 and M > 0 else (None if A is None else _u16(A))
    B = _u16(B) if K > 0 and N > 0 else (None if B is None else _u16(B))
    if A is not None and A.size != M * K:
        raise ValueError("A has the wrong size")
    if B is not None and B.size != K * N:
        raise ValueError("B has the wrong size")
    bias_a = None
    if bias is not None:
        bias_a = _u16(bias)
        if bias_a.size != N:
            raise ValueError("bias has the wrong size")
    if rows is None:
        rows_a = None
        nrows = M
    else:
        rows_a = np.ascontiguousarray(rows, dtype=np.int64)
        nrows = rows_a.size
    out64 = np.empty((nrows, N), dtype=np.float64)
    outq = np.empty((nrows, N), dtype=np.uint16)
    rc = _load().tg_oracle_gemm(M, N, K, dtype, _ptr(A, ctypes.c_uint16), _ptr(B, ctypes.c_uint16),
                                _ptr(bias_a, ctypes.c_uint16), epilogue, _ptr(rows_a, ctypes.c_int64),
                                nrows, _ptr(out64, ctypes.c_double), _ptr(outq, ctypes.c_uint16))
    if rc != 0:
        raise ValueError(f"tg_oracle_gemm failed ({rc})")
    return out64, outq


def gemm_w4(M: int, N: int, K: int, dtype: int, A, Q, scales, group: int, bias=None,
            epilogue: int = EPI_NONE, rows=None) -> Tuple[np.ndarray, np.ndarray]:
    """Rows ``rows`` (default: all) of epilogue(A @ W [+ bias]) with the
    weights W[k, n] = (Q[k, n] - 8) * scales[k // group, n].

    A: (M, K) uint16 bit patterns; Q: (K, N) uint8 values 0..15 (one per
    byte, unpacked); scales: (K // group, N) uint16 bit patterns; bias: (N,)
    or None.  Returns (ref64, refq) as :func:`gemm`.
    """
    A = None if A is None else _u16(A)
    Q = None if Q is None else np.ascontiguousarray(Q, dtype=np.uint8)
    S = None if scales is None else _u16(scales)
    if K > 0 and M > 0 and (A is None or A.size != M * K):
        raise ValueError("A has the wrong size")
    if K > 0 and N > 0 and (Q is None or Q.size != K * N):
        raise ValueError("Q has the wrong size")
    if K > 0 and N > 0 and (S is None or group <= 0 or S.size != (K // group) * N):
        raise ValueError("scales have the wrong size")
    bias_a = None
    if bias is not None:
        bias_a = _u16(bias)
        if bias_a.size != N:
            raise ValueError("bias has the wrong size")
    if rows is None:
        rows_a, nrows = None, M
    else:
        rows_a = np.ascontiguousarray(rows, dtype=np.int64)
        nrows = rows_a.size
    out64 = np.empty((nrows, N), dtype=np.float64)
    outq = np.empty((nrows, N), dtype=np.uint16)
    rc = _load().tg_oracle_gemm_w4(M, N, K, dtype, _ptr(A, ctypes.c_uint16), _ptr(Q, ctypes.c_uint8),
                                   _ptr(S, ctypes.c_uint16), group, _ptr(bias_a, ctypes.c_uint16), epilogue,
                                   _ptr(rows_a, ctypes.c_int64), nrows, _ptr(out64, ctypes.c_double),
                                   _ptr(outq, ctypes.c_uint16))
    if rc != 0:
        raise ValueError(f"tg_oracle_gemm_w4 failed ({rc})")
    return out64, outq


def attention(Bn: int, Sq: int, Sk: int, H: int, D: int, dtype: int, Q, K, V, causal: bool = False,
              scale: Optional[float] = None, queries=None) -> Tuple[np.ndarray, np.ndarray]:
    """softmax(scale * Q K^T) V for the queries ``queries`` (an (n, 3) array of
    (batch, position, head); default: all, in (b, i, h) order), BSHD layout:
    Q (Bn, Sq, H, D), K and V (Bn, Sk, H, D) uint16 bit patterns.  ``scale``
    defaults to 1/sqrt(D); ``causal`` (Sq == Sk) lets query i see keys 0..i.
    Returns (ref64, refq), each (n, D)."""
    Qa = _u16(Q)
    Ka = None if K is None else _u16(K)
    Va = None if V is None else _u16(V)
    if Qa.size != Bn * Sq * H * D:
        raise ValueError("Q has the wrong size")
    if Sk > 0 and (Ka is None or Va is None or Ka.size != Bn * Sk * H * D or Va.size != Bn * Sk * H * D):
        raise ValueError("K or V has the wrong size")
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    if queries is None:
        b, i, h = np.meshgrid(np.arange(Bn), np.arange(Sq), np.arange(H), indexing="ij")
        queries = np.stack([b.ravel(), i.ravel(), h.ravel()], axis=1)
    qa = np.ascontiguousarray(queries, dtype=np.int64).reshape(-1, 3)
    nq = qa.shape[0]
    out64 = np.empty((nq, D), dtype=np.float64)
    outq = np.empty((nq, D), dtype=np.uint16)
    rc = _load().tg_oracle_attention(Bn, Sq, Sk, H, D, dtype, _ptr(Qa, ctypes.c_uint16), _ptr(Ka, ctypes.c_uint16),
                                     _ptr(Va, ctypes.c_uint16), 1 if causal else 0, float(scale),
                                     _ptr(qa, ctypes.c_int64), nq, _ptr(out64, ctypes.c_double),
                                     _ptr(outq, ctypes.c_uint16))
    if rc != 0:
        raise ValueError(f"tg_oracle_attention failed ({rc})")
    return out64, outq

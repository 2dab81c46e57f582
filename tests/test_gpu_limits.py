"""GPU parity at the kernels' size limits, through the C interface.

The direct-load tiled kernel addresses A and B with 32-bit byte offsets into
buffers that start 4 KiB before each operand and take every operand padded
to whole tiles below 2 GiB less 64 KiB; beyond that the register-gathered
kernel takes over, up to 2^31 - 64 elements per operand (byte offsets near
2^32).  These tests run both just below and just above that limit, in A and
in B, and check sampled rows and columns that include the last ones (the
largest offsets) bit-exactly against the oracle.

Operands are integer-valued (a hash of the row and column, values -2..2, so
every fp32 partial sum is exact and a row or column read from the wrong
place shows as a mismatch) and are generated on the device; the oracle gets
the sampled rows of A and columns of B only.
"""
import numpy as np
import pytest

import oracle
import tiled_dense_gemm_tg_amd as tg
from tiled_dense_gemm_tg_amd import inputs as I
from gpu_util import check_exact, log, to_bits

pytestmark = pytest.mark.gpu


def _hashed(rows, cols, salt):
    """(rows x cols) fp16 device tensor of small integers from a hash of (row, col)."""
    import torch
    r = torch.arange(rows, device="cuda", dtype=torch.int64)[:, None]
    out = torch.empty((rows, cols), dtype=torch.float16, device="cuda")
    step = max(1, (1 << 27) // cols)       # rows per chunk: bounded temporaries
    c = torch.arange(cols, device="cuda", dtype=torch.int64)[None, :]
    for r0 in range(0, rows, step):
        rr = r[r0:r0 + step]
        v = ((rr * 2654435761 + c * 40503 + salt * 97) >> 11) % 5 - 2
        out[r0:r0 + step] = v.to(torch.float16)
    return out


def _sample(n, count, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    idx = rng.choice(n, size=min(count, n), replace=False)
    return np.unique(np.concatenate([idx, [0, n - 2, n - 1]])).astype(np.int64)


@pytest.mark.parametrize("M,N,K,path", [
    (130808, 256, 8192, tg.TG_PATH_TILED),           # A padded just below 2 GiB - 64 KiB
    (130812, 256, 8192, tg.TG_PATH_TILED_GENERIC),   # A just above: 2.14 GB, offsets past 2^31
    (256, 129792, 8192, tg.TG_PATH_TILED),           # B padded just below the limit
    (256, 129800, 8192, tg.TG_PATH_TILED_GENERIC),   # B just above
], ids=lambda v: str(v))
def test_largest_operands(M, N, K, path):
    import torch
    dtype = I.F16
    log(f"[limits] {M}x{N}x{K}: generating operands on the device")
    A = _hashed(M, K, 1)
    B = _hashed(K, N, 2)
    bias = _hashed(1, N, 3).reshape(N)
    C = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    st, p = tg.tg_gemm_plan(M, N, K, dtype, A.data_ptr(), B.data_ptr(), bias.data_ptr(), I.EPI_BIAS, C.data_ptr())
    assert st == tg.TG_OK and p == path, (st, tg.PATH_NAMES.get(p))
    log(f"[limits] {M}x{N}x{K}: GPU run on path {tg.PATH_NAMES[p]}")
    tg.gemm(A, B, bias, "bias", out=C)
    torch.cuda.synchronize()
    rows = _sample(M, 24, 31 + M)
    cols = _sample(N, 192, 37 + N)
    a_rows = to_bits(A[torch.from_numpy(rows).cuda()])
    b_cols = to_bits(B[:, torch.from_numpy(cols).cuda()])
    bias_cols = to_bits(bias[torch.from_numpy(cols).cuda()])
    got = to_bits(C[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()])
    del A, B, C
    torch.cuda.empty_cache()
    log(f"[limits] {M}x{N}x{K}: oracle on {len(rows)} rows x {len(cols)} columns")
    _, refq = oracle.gemm(len(rows), len(cols), K, dtype, a_rows.reshape(-1), b_cols.reshape(-1), bias_cols,
                          I.EPI_BIAS)
    check_exact(got, refq.reshape(len(rows), len(cols)), f"{M}x{N}x{K}")


@pytest.mark.parametrize("Bn,S,H,causal", [
    (1, 767, 8192, False),    # Q, K, V and O 1.6 GB each: padded just below the 2 GiB limit
    (2, 767, 4096, True),
], ids=lambda v: str(v))
def test_attention_largest_tensors(Bn, S, H, causal):
    """Attention with the largest tensors the kernel takes (token stride 2 MB
    or 1 MB): sampled queries of sampled heads against the oracle."""
    import torch
    from gpu_util import check_tolerance
    D = 128
    dtype = I.F16
    log(f"[limits] attention B={Bn} S={S} H={H} causal={causal}: generating inputs on the device")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(41 + H)
    q = torch.randn((Bn, S, H, D), generator=gen, device="cuda").half()
    k = torch.randn((Bn, S, H, D), generator=gen, device="cuda").half()
    v = torch.randn((Bn, S, H, D), generator=gen, device="cuda").half()
    o = torch.full_like(q, float("nan"))
    log(f"[limits] attention B={Bn} S={S} H={H}: GPU run")
    tg.attention(q, k, v, causal=causal, out=o)
    torch.cuda.synchronize()
    rng = np.random.Generator(np.random.PCG64(43))
    heads = np.unique(np.concatenate([rng.choice(H, 4, replace=False), [0, H - 1]]))
    for b in (0, Bn - 1):
        for h in heads:
            qs = np.unique(np.concatenate([rng.choice(S, 12, replace=False), [0, S - 1]]))
            qh, kh, vh = (to_bits(x[b, :, int(h)]) for x in (q, k, v))     # (S, D) of this batch and head
            triples = np.stack([np.zeros_like(qs), qs, np.zeros_like(qs)], axis=1)
            ref64, _ = oracle.attention(1, S, S, 1, D, dtype, qh.reshape(-1), kh.reshape(-1), vh.reshape(-1),
                                        causal=causal, queries=triples)
            got = to_bits(o[b, torch.from_numpy(qs).cuda(), int(h)])
            check_tolerance(dtype, got, ref64, f"attention b={b} h={h}")


def test_skinny_largest_weight():
    """The decode-shaped kernel with B of 2^31 - 65536 elements (4.3 GB,
    byte offsets up to 2^32 - 2^17): sampled columns, every row, exact."""
    import torch
    M, N, K = 16, 262136, 8192
    dtype = I.F16
    log(f"[limits] skinny {M}x{N}x{K}: generating operands on the device")
    A = _hashed(M, K, 4)
    B = _hashed(K, N, 5)
    C = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    st, p = tg.tg_gemm_plan(M, N, K, dtype, A.data_ptr(), B.data_ptr(), None, I.EPI_NONE, C.data_ptr())
    assert st == tg.TG_OK and p == tg.TG_PATH_SKINNY, (st, tg.PATH_NAMES.get(p))
    log(f"[limits] skinny {M}x{N}x{K}: GPU run")
    tg.gemm(A, B, out=C)
    torch.cuda.synchronize()
    cols = torch.from_numpy(_sample(N, 256, 47)).cuda()
    b_cols = to_bits(B[:, cols])
    got = to_bits(C[:, cols])
    a_bits = to_bits(A)
    del B, C
    torch.cuda.empty_cache()
    _, refq = oracle.gemm(M, len(cols), K, dtype, a_bits.reshape(-1), b_cols.reshape(-1))
    check_exact(got, refq.reshape(M, len(cols)), "skinny at the limit")


def test_w4_largest_weight():
    """The 4-bit product with 2^31 - 2^20 weight codes (2.1 GB unpacked, 1.07 GB
    packed) and power-of-two scales: sampled columns, every row, exact."""
    import torch
    M, N, K, G = 16, 131008, 16384, 128
    dtype = I.F16
    log(f"[limits] w4 {M}x{N}x{K}: generating operands on the device")
    A = _hashed(M, K, 6)
    r = torch.arange(K, device="cuda", dtype=torch.int64)[:, None]
    q = torch.empty((K, N), dtype=torch.uint8, device="cuda")
    c = torch.arange(N, device="cuda", dtype=torch.int64)[None, :]
    step = (1 << 27) // N
    for r0 in range(0, K, step):
        q[r0:r0 + step] = (((r[r0:r0 + step] * 2246822519 + c * 3266489917) >> 9) % 16).to(torch.uint8)
    e = (torch.arange(K // G, device="cuda")[:, None] * 3 + torch.arange(N, device="cuda")[None, :]) % 4
    scales = torch.pow(2.0, -e.to(torch.float32)).half()      # 1, 1/2, 1/4, 1/8: exact products
    packed = tg.w4_pack(q)
    log(f"[limits] w4 {M}x{N}x{K}: GPU run")
    C = tg.gemm_w4(A, packed, scales, G, N)
    torch.cuda.synchronize()
    cols = torch.from_numpy(_sample(N, 256, 53)).cuda()
    q_cols = q[:, cols].cpu().numpy()
    s_cols = to_bits(scales[:, cols])
    got = to_bits(C[:, cols])
    a_bits = to_bits(A)
    del q, packed, C
    torch.cuda.empty_cache()
    _, refq = oracle.gemm_w4(M, len(cols), K, dtype, a_bits.reshape(-1), q_cols, s_cols, G)
    check_exact(got, refq.reshape(M, len(cols)), "w4 at the limit")

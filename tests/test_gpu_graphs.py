"""The library's calls inside a captured HIP graph (torch.cuda.CUDAGraph).

Every entry point only enqueues kernels on the caller's stream (no
allocation, no memset, no host synchronisation), so a graph captured from
them must replay to the same bits as the eager calls.  The graph holds a
tiled product with the fused epilogue (tile configuration chosen by the
library), a decode-shaped product, the 4-bit product and the attention
forward; it is replayed several times, with eager work and host
synchronisation between replays and the outputs poisoned before each, and
every replay is compared with the eager results bit for bit (and the eager
results with the oracle).
"""
import numpy as np
import pytest

import oracle
import tiled_dense_gemm_tg_amd as tg
from tiled_dense_gemm_tg_amd import inputs as I
from gpu_util import check_tolerance, log, to_bits, to_device

pytestmark = pytest.mark.gpu


def test_replays_match_eager_calls():
    import torch
    dt = I.BF16
    M, N, K = 520, 264, 328
    A = to_device(I.random_bits((M, K), ("uniform", -1.0, 1.0), dt, 14000).reshape(M, K), dt)
    B = to_device(I.random_bits((K, N), ("uniform", -1.0, 1.0), dt, 14001).reshape(K, N), dt)
    bias = to_device(I.random_bits((N,), ("uniform", -0.5, 0.5), dt, 14002), dt)
    Ms, Ns, Ks = 16, 1024, 512
    As = to_device(I.random_bits((Ms, Ks), ("normal", 0.0, 1.0), dt, 14003).reshape(Ms, Ks), dt)
    Bs = to_device(I.random_bits((Ks, Ns), ("normal", 0.0, 0.02), dt, 14004).reshape(Ks, Ns), dt)
    q = torch.from_numpy(I.w4_weights(Ks, Ns, 14005)).cuda()
    packed = tg.w4_pack(q)
    scales = to_device(I.random_bits((Ks // 128, Ns), ("uniform", 0.001, 0.01), dt, 14006).reshape(Ks // 128, Ns), dt)
    Bn, S, H, D = 1, 300, 2, 128
    Q, Kt, V = (to_device(I.random_bits((Bn, S, H, D), ("normal", 0.0, 1.0), dt, 14007 + i).reshape(Bn, S, H, D), dt)
                for i in range(3))
    C1 = torch.empty((M, N), dtype=A.dtype, device="cuda")
    C2 = torch.empty((Ms, Ns), dtype=A.dtype, device="cuda")
    C3 = torch.empty((Ms, Ns), dtype=A.dtype, device="cuda")
    O = torch.empty_like(Q)

    def calls():
        tg.gemm(A, B, bias, "bias_gelu_tanh", out=C1)
        tg.gemm(As, Bs, out=C2)
        tg.gemm_w4(As, packed, scales, 128, Ns, out=C3)
        tg.attention(Q, Kt, V, causal=True, out=O)

    log("[graph] eager calls")
    calls()
    torch.cuda.synchronize()
    eager = [to_bits(t) for t in (C1, C2, C3, O)]
    ref64, _ = oracle.gemm(M, N, K, dt, to_bits(A).reshape(-1), to_bits(B).reshape(-1), to_bits(bias),
                           I.EPI_BIAS_GELU_TANH)
    check_tolerance(dt, eager[0], ref64, "eager tiled")

    log("[graph] capture")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g):
            calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        for t in (C1, C2, C3, O):
            t.fill_(float("nan"))
        # unrelated eager work between replays
        torch.matmul(A.float(), B.float()).sum().item()
        log(f"[graph] replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        for name, t, e in zip(("tiled", "skinny", "w4", "attention"), (C1, C2, C3, O), eager):
            assert np.array_equal(to_bits(t), e), f"replay {rep}: {name} differs from the eager call"


def test_static_split_replays_match_eager_calls():
    """The allocation-free split-K entry point (tg_gemm_split_static) is for
    callers under graph capture: after one eager call on the device (which
    looks its scratch array up and zeroes the counters, outside capture),
    even splits and stream-K captured into one graph replay to the eager
    bits, every replay leaving the counters zero for the next."""
    import torch
    dt = I.F16
    shapes = [(16, 4096, 2048, 4), (7, 2048, 4104, tg.TG_SPLIT_STREAM_K), (16, 11008, 1024, 0)]
    ops = []
    for i, (M, N, K, splits) in enumerate(shapes):
        A = to_device(I.random_bits((M, K), ("normal", 0.0, 1.0), dt, 14100 + i).reshape(M, K), dt)
        B = to_device(I.random_bits((K, N), ("normal", 0.0, 0.02), dt, 14110 + i).reshape(K, N), dt)
        bias = to_device(I.random_bits((N,), ("normal", 0.0, 0.1), dt, 14120 + i), dt)
        C = torch.empty((M, N), dtype=A.dtype, device="cuda")
        ops.append((M, N, K, splits, A, B, bias, C))

    def calls():
        stream = torch.cuda.current_stream().cuda_stream   # the capture stream inside torch.cuda.graph
        for M, N, K, splits, A, B, bias, C in ops:
            st = tg.tg_gemm_split_static(splits, M, N, K, dt, A.data_ptr(), B.data_ptr(), bias.data_ptr(),
                                         I.EPI_BIAS_GELU_TANH, C.data_ptr(), stream)
            assert st == tg.TG_OK, tg.tg_status_string(st)

    log("[graph static] eager calls")
    calls()
    torch.cuda.synchronize()
    eager = [to_bits(op[7]) for op in ops]
    for (M, N, K, splits, A, B, bias, C), e in zip(ops, eager):
        rows = np.arange(M)
        ref64, _ = oracle.gemm(M, N, K, dt, to_bits(A).reshape(-1), to_bits(B).reshape(-1), to_bits(bias),
                               I.EPI_BIAS_GELU_TANH, rows)
        check_tolerance(dt, e, ref64, f"eager static split M={M} N={N} K={K} splits={splits}")

    log("[graph static] capture")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g):
            calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        for op in ops:
            op[7].fill_(float("nan"))
        ops[0][4].float().sum().item()   # unrelated eager work between replays
        log(f"[graph static] replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        for (M, N, K, splits, *_rest), e in zip(ops, eager):
            assert np.array_equal(to_bits(_rest[-1]), e), \
                f"replay {rep}: M={M} N={N} K={K} splits={splits} differs from the eager call"
    # eager calls after the replays still see zero counters
    calls()
    torch.cuda.synchronize()
    for op, e in zip(ops, eager):
        assert np.array_equal(to_bits(op[7]), e), "eager call after the replays"

"""GPU parity of every tile configuration of the tiled family (tg_gemm_tiled)
against the oracle, through the C interface, to the same bar as the other
parity tests: bit-exact on integer-valued inputs, |C - ref64| <= rtol
(|ref64| + 1) otherwise (rtol 1e-2 fp16, 2e-2 bf16), every output written.

Each configuration is its own instance of the direct-load kernel (its own
load mapping, fragment reads, LDS layout, last-slice fix-ups and staged
store), so each gets the edge-shape sweep, 2-byte-aligned operands, the K
tail, more tiles than its persistent grid has workgroups, guard bands around
C, exact layout probes, and a full-size shape on sampled rows.
"""
import numpy as np
import pytest

import oracle
import tiled_dense_gemm_tg_amd as tg
from tiled_dense_gemm_tg_amd import inputs as I
from gpu_util import check_exact, check_tolerance, log, run, to_bits, to_device

pytestmark = pytest.mark.gpu

CONFIGS = sorted(tg.TILES_AXES)
TILE_SHAPE = {cfg: axes[:2] for cfg, axes in tg.TILES_AXES.items()}
EDGE = [1, 2, 7, 8, 15, 16, 17, 31, 33, 63, 64, 65, 127, 129, 255, 257]
EPI_NAMES = {I.EPI_NONE: "none", I.EPI_BIAS: "bias", I.EPI_BIAS_GELU_TANH: "bias_gelu_tanh"}


def _name(cfg):
    return tg.TILES_NAMES[cfg]


def _edge_cases(n, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = set()
    while len(cases) < n:
        cases.add(tuple(int(v) for v in rng.choice(EDGE, 3)))
    return sorted(cases)


@pytest.mark.parametrize("cfg", CONFIGS, ids=_name)
@pytest.mark.parametrize("dtype", [I.F16, I.BF16])
def test_edge_shapes(cfg, dtype):
    cases = _edge_cases(24, 40 + 3 * cfg + dtype) + [(300, 520, 264), (513, 264, 1000), (129, 385, 41)]
    for idx, (M, N, K) in enumerate(cases):
        epi = (I.EPI_NONE, I.EPI_BIAS, I.EPI_BIAS_GELU_TANH)[idx % 3]
        A = I.random_bits((M, K), ("uniform", -1.0, 1.0), dtype, 12000 + idx)
        B = I.random_bits((K, N), ("uniform", -1.0, 1.0), dtype, 12100 + idx)
        bias = I.random_bits((N,), ("uniform", -0.5, 0.5), dtype, 12200 + idx) if epi else None
        ref64, _ = oracle.gemm(M, N, K, dtype, A, B, bias, epi)
        what = f"tiles={_name(cfg)} {I.DTYPE_NAMES[dtype]} M={M} N={N} K={K} epi={epi}"
        log(f"[tiles-edge] {what}")
        check_tolerance(dtype, to_bits(run(M, N, K, dtype, A, B, bias, epi, tiles=cfg)), ref64, what)
        Ai = I.small_int_bits((M, K), dtype, 12300 + idx)
        Bi = I.small_int_bits((K, N), dtype, 12400 + idx)
        bi = I.small_int_bits((N,), dtype, 12500 + idx)
        _, refq = oracle.gemm(M, N, K, dtype, Ai, Bi, bi, I.EPI_BIAS)
        check_exact(to_bits(run(M, N, K, dtype, Ai, Bi, bi, I.EPI_BIAS, tiles=cfg)), refq, what + " (integers)")


def _offset_tensor(bits, dtype, shape, offset):
    n = int(np.prod(shape))
    flat = to_device(np.concatenate([np.zeros(offset, np.uint16), np.ascontiguousarray(bits).reshape(-1)]), dtype)
    return flat[offset:offset + n].view(*shape)


@pytest.mark.parametrize("cfg", CONFIGS, ids=_name)
@pytest.mark.parametrize("M,N,K,offsets", [
    (520, 264, 328, (1, 3, 1, 1)),    # aligned shapes, 2-byte-aligned operands
    (300, 263, 201, (1, 1, 1, 1)),    # everything ragged and misaligned
])
def test_any_alignment(cfg, M, N, K, offsets):
    import torch
    dtype = I.BF16
    oa, ob, oc, obias = offsets
    for kind in ("random", "integers"):
        if kind == "random":
            A = I.random_bits((M, K), ("uniform", -1.0, 1.0), dtype, 13000)
            B = I.random_bits((K, N), ("uniform", -1.0, 1.0), dtype, 13001)
            bias = I.random_bits((N,), ("uniform", -0.5, 0.5), dtype, 13002)
            epi = I.EPI_BIAS_GELU_TANH
        else:
            A = I.small_int_bits((M, K), dtype, 13003)
            B = I.small_int_bits((K, N), dtype, 13004)
            bias = I.small_int_bits((N,), dtype, 13005)
            epi = I.EPI_BIAS
        ref64, refq = oracle.gemm(M, N, K, dtype, A, B, bias, epi)
        a = _offset_tensor(A, dtype, (M, K), oa)
        b = _offset_tensor(B, dtype, (K, N), ob)
        bb = _offset_tensor(bias, dtype, (N,), obias)
        c = _offset_tensor(np.full(M * N, 0x7FC0, np.uint16), dtype, (M, N), oc)   # NaN-filled
        log(f"[tiles-align] tiles={_name(cfg)} {M}x{N}x{K} offsets={offsets} {kind}")
        tg.gemm(a, b, bb, EPI_NAMES[epi], out=c, tiles=cfg)
        torch.cuda.synchronize()
        if kind == "random":
            check_tolerance(dtype, to_bits(c), ref64, f"align {offsets}")
        else:
            check_exact(to_bits(c), refq, f"align {offsets}")


@pytest.mark.parametrize("cfg", CONFIGS, ids=_name)
@pytest.mark.parametrize("K", [37, 8, 33, 71, 100])
def test_k_tail_does_not_mix_rows(cfg, K):
    """Odd rows of A hold +inf at k = 0; with K % 8 != 0 the chunk crossing
    k = K of an even row also covers the odd row's first elements, which
    must not enter the even row's sum."""
    M, N = 136, 200
    dtype = I.F16
    A = I.random_bits((M, K), ("uniform", -1.0, 1.0), dtype, 13100).reshape(M, K).copy()
    A[1::2, 0] = np.uint16(0x7C00)
    B = I.random_bits((K, N), ("uniform", 0.5, 1.0), dtype, 13101)
    ref64, _ = oracle.gemm(M, N, K, dtype, A.reshape(-1), B)
    log(f"[tiles-k-tail] tiles={_name(cfg)} K={K}")
    got = to_bits(run(M, N, K, dtype, A.reshape(-1), B, tiles=cfg))
    assert np.isposinf(oracle.decode(dtype, got)[1::2]).all()
    check_tolerance(dtype, got[0::2], ref64[0::2], "even rows")


@pytest.mark.parametrize("cfg,M,N,K", [
    (tg.TG_TILES_256x128, 2304, 4224, 64),   # 297 tiles: more than one per CU
    (tg.TG_TILES_128x256, 4224, 2304, 72),
    (tg.TG_TILES_128x128, 3000, 3100, 40),   # 600 tiles: more than two per CU, ragged
    (tg.TG_TILES_128x128, 4096, 4096, 24),   # 1024 tiles, a multiple of the 8 XCDs
    (tg.TG_TILES_256x256, 4352, 4352, 48),   # 289 tiles
    (tg.TG_TILES_256x256_K64, 4352, 4352, 136),
    (tg.TG_TILES_256x128_K64, 2304, 4224, 200),
    (tg.TG_TILES_128x256_K64, 4224, 2304, 72),
    (tg.TG_TILES_128x128_K64, 3000, 3100, 130),
    (tg.TG_TILES_256x256_W8, 4352, 4352, 72),
], ids=lambda v: str(v))
def test_persistent_grid_covers_every_tile(cfg, M, N, K):
    dtype = I.F16
    A = I.small_int_bits((M, K), dtype, 13200)
    B = I.small_int_bits((K, N), dtype, 13201)
    bias = I.small_int_bits((N,), dtype, 13202)
    log(f"[tiles-persistent] tiles={_name(cfg)} {M}x{N}x{K}")
    out = run(M, N, K, dtype, A, B, bias, I.EPI_BIAS, tiles=cfg)
    _, refq = oracle.gemm(M, N, K, dtype, A, B, bias, I.EPI_BIAS)
    check_exact(to_bits(out), refq, f"persistent {M}x{N}x{K}")


@pytest.mark.parametrize("cfg", CONFIGS, ids=_name)
def test_identity_and_permutation(cfg):
    dtype = I.F16
    rng = np.random.Generator(np.random.PCG64(13300))
    M, K = 300, 264
    A = I.random_bits((M, K), ("normal", 0.0, 2.0), dtype, 13301)
    perm = rng.permutation(K)
    P = np.zeros((K, K))
    P[perm, np.arange(K)] = 1.0
    log(f"[tiles-layout] tiles={_name(cfg)}")
    check_exact(to_bits(run(M, K, K, dtype, A, I.values_bits(np.eye(K), dtype), tiles=cfg)), A, "A @ I")
    check_exact(to_bits(run(M, K, K, dtype, A, I.values_bits(P, dtype), tiles=cfg)), A.reshape(M, K)[:, perm],
                "A @ P")


@pytest.mark.parametrize("cfg", CONFIGS, ids=_name)
def test_guard_bands_untouched(cfg):
    import torch
    M, N, K = 301, 263, 201
    guard = 2048
    dtype = I.F16
    A = I.random_bits((M, K), ("uniform", -1.0, 1.0), dtype, 13400)
    B = I.random_bits((K, N), ("uniform", -1.0, 1.0), dtype, 13401)
    bias = I.random_bits((N,), ("uniform", -1.0, 1.0), dtype, 13402)
    buf = torch.full((guard + M * N + guard,), 12345.0, dtype=torch.float16, device="cuda")
    out = buf[guard:guard + M * N].view(M, N)
    out.fill_(float("nan"))
    log(f"[tiles-guard] tiles={_name(cfg)}")
    run(M, N, K, dtype, A, B, bias, I.EPI_BIAS_GELU_TANH, out=out, tiles=cfg)
    host = buf.cpu()
    assert (host[:guard] == 12345.0).all() and (host[guard + M * N:] == 12345.0).all()
    ref64, _ = oracle.gemm(M, N, K, dtype, A, B, bias, I.EPI_BIAS_GELU_TANH)
    check_tolerance(dtype, to_bits(out), ref64, "guarded")


@pytest.mark.parametrize("cfg", CONFIGS, ids=_name)
@pytest.mark.parametrize("name", list(I.TILE_WORKLOADS))
def test_sweep_shapes_on_sampled_rows(cfg, name):
    """The mid-size shapes the tile choice is for, at full size, every
    configuration, on the workload's seeded row sample."""
    w = I.TILE_WORKLOADS[name]
    ops = I.make_operands(w)
    log(f"[tiles-full] {name} tiles={_name(cfg)}")
    got = to_bits(run(w.M, w.N, w.K, w.dtype, ops.A, ops.B, ops.bias, w.epilogue, tiles=cfg))[ops.rows]
    ref64, _ = oracle.gemm(w.M, w.N, w.K, w.dtype, ops.A, ops.B, ops.bias, w.epilogue, ops.rows)
    check_tolerance(w.dtype, got, ref64, f"{name} tiles={_name(cfg)}")


@pytest.mark.parametrize("M,N,K", [(2048, 2048, 2048), (512, 11008, 4096), (4096, 4096, 512), (300, 263, 201)])
def test_automatic_choice_is_the_planned_configuration(M, N, K):
    """tg_gemm (TG_TILES_AUTO) and tg_gemm_tiled with the configuration
    tg_gemm_tiles_plan names run the same kernel instance: bit-identical."""
    import torch
    dtype = I.F16
    A = I.random_bits((M, K), ("normal", 0.0, 0.1), dtype, 13500)
    B = I.random_bits((K, N), ("normal", 0.0, 0.1), dtype, 13501)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    st, cfg = tg.tg_gemm_tiles_plan(M, N, K, cus)
    assert st == tg.TG_OK and cfg in CONFIGS
    log(f"[tiles-auto] {M}x{N}x{K}: {_name(cfg)} on {cus} CUs")
    auto = to_bits(run(M, N, K, dtype, A, B, expect_path=tg.TG_PATH_TILED))
    explicit = to_bits(run(M, N, K, dtype, A, B, tiles=cfg))
    assert np.array_equal(auto, explicit)


@pytest.mark.parametrize("cfg", CONFIGS, ids=_name)
@pytest.mark.parametrize("epi", [I.EPI_NONE, I.EPI_BIAS, I.EPI_BIAS_GELU_TANH])
def test_empty_K_gives_epilogue_of_zero(cfg, epi):
    M, N = 300, 264
    bias = I.random_bits((N,), ("uniform", -2.0, 2.0), I.F16, 13600) if epi else None
    _, refq = oracle.gemm(M, N, 0, I.F16, None, None, bias, epi)
    log(f"[tiles-K=0] tiles={_name(cfg)} epi={epi}")
    out = run(M, N, 0, I.F16, np.zeros(0, np.uint16), np.zeros(0, np.uint16), bias, epi, tiles=cfg)
    check_exact(to_bits(out), refq, "K=0")


@pytest.mark.parametrize("cfg", CONFIGS, ids=_name)
def test_every_pipeline_depth(cfg):
    """K from one slice to two turns of the stage ring past the first
    requests, exact and ragged, so every prologue, steady (unrolled over the
    ring, and its remainders of 0 .. S-1 slices), last-request and tail step
    of the pipeline runs (integers: exact)."""
    dtype = I.BF16
    M, N = 136, 264
    bk, stages = tg.TILES_AXES[cfg][2], tg.TILES_AXES[cfg][3]
    for n in range(1, 2 * stages + 6):
        for K in (n * bk, n * bk - 5):
            A = I.small_int_bits((M, K), dtype, 13700 + K)
            B = I.small_int_bits((K, N), dtype, 13800 + K)
            bias = I.small_int_bits((N,), dtype, 13900 + K)
            _, refq = oracle.gemm(M, N, K, dtype, A, B, bias, I.EPI_BIAS)
            log(f"[tiles-depth] tiles={_name(cfg)} K={K}")
            check_exact(to_bits(run(M, N, K, dtype, A, B, bias, I.EPI_BIAS, tiles=cfg)), refq, f"K={K}")


def _odd_n_shapes(cfg):
    bn, bk = TILE_SHAPE[cfg][1], tg.TILES_AXES[cfg][2]
    ns = [1, 3, bn - 1, bn + 1, 2 * bn + 1, 2 * bn + 5, 2 * bn + 7, 2 * bn + 9]
    ks = [1, 2, bk, 3 * bk, 3 * bk - 2, 3 * bk - 1, 5 * bk + 6]
    return [(ns[i % len(ns)], ks[i % len(ks)]) for i in range(len(ns) * len(ks))][::3]


@pytest.mark.parametrize("cfg", CONFIGS, ids=_name)
def test_odd_n_every_chunk_of_the_last_row(cfg):
    """N odd (every other k-row of B starts 2 bytes past a 4-byte boundary):
    widths that end in every position of a tile and one element past it,
    with K even and odd (B's last row, whose chunk crossing N is rewritten
    from element loads, odd or even) and exact or ragged in k; integers:
    exact."""
    dtype = I.F16
    M = 72
    for idx, (N, K) in enumerate(_odd_n_shapes(cfg)):
        A = I.small_int_bits((M, K), dtype, 14200 + idx)
        B = I.small_int_bits((K, N), dtype, 14300 + idx)
        bias = I.small_int_bits((N,), dtype, 14400 + idx)
        _, refq = oracle.gemm(M, N, K, dtype, A, B, bias, I.EPI_BIAS)
        what = f"tiles={_name(cfg)} M={M} N={N} K={K}"
        log(f"[tiles-odd-n] {what}")
        check_exact(to_bits(run(M, N, K, dtype, A, B, bias, I.EPI_BIAS, tiles=cfg)), refq, what)


@pytest.mark.parametrize("cfg", CONFIGS, ids=_name)
@pytest.mark.parametrize("K", [96, 95, 70])
def test_odd_n_does_not_mix_columns(cfg, K):
    """N odd: the last column of every tile holds +inf in every row of B, so
    exactly those columns of C are infinite; a chunk put one column off
    would move an infinity into a neighbour."""
    bn = TILE_SHAPE[cfg][1]
    M, N = 136, 3 * bn + 17
    dtype = I.BF16
    A = I.random_bits((M, K), ("uniform", 0.5, 1.0), dtype, 14500)
    B = I.random_bits((K, N), ("uniform", -1.0, 1.0), dtype, 14501).reshape(K, N).copy()
    inf_cols = np.arange(bn - 1, N, bn)
    B[:, inf_cols] = np.uint16(0x7F80)
    ref64, _ = oracle.gemm(M, N, K, dtype, A, B.reshape(-1))
    log(f"[tiles-odd-n-inf] tiles={_name(cfg)} K={K}")
    bits = to_bits(run(M, N, K, dtype, A, B.reshape(-1), tiles=cfg)).reshape(M, N)
    got = oracle.decode(dtype, bits)
    assert np.isposinf(got[:, inf_cols]).all()
    finite = np.setdiff1d(np.arange(N), inf_cols)
    check_tolerance(dtype, np.ascontiguousarray(bits[:, finite]).reshape(-1),
                    ref64.reshape(M, N)[:, finite].reshape(-1), "finite columns")


@pytest.mark.parametrize("group_m", [1, 2, 3, 8, 64])
def test_raster_group_changes_nothing_but_the_order(group_m):
    """tg_gemm_tiled_grouped: every group size covers every tile once
    (integers: exact), also groups taller than the tile rows and sizes that
    do not divide them, on a persistent grid with several tiles per CU."""
    dtype = I.F16
    M, N, K = 2600, 3000, 40
    A = I.small_int_bits((M, K), dtype, 14000)
    B = I.small_int_bits((K, N), dtype, 14001)
    bias = I.small_int_bits((N,), dtype, 14002)
    _, refq = oracle.gemm(M, N, K, dtype, A, B, bias, I.EPI_BIAS)
    for cfg in (tg.TG_TILES_256x256, tg.TG_TILES_128x128):
        log(f"[tiles-group] tiles={_name(cfg)} group_m={group_m}")
        got = to_bits(run(M, N, K, dtype, A, B, bias, I.EPI_BIAS, tiles=cfg, group_m=group_m))
        check_exact(got, refq, f"group_m={group_m} tiles={_name(cfg)}")

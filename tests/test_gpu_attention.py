"""GPU parity of the attention forward kernel (tg_attention_fwd) against the
oracle's attention, through the C interface.

Bar: |O - ref64| <= rtol (|ref64| + 1) elementwise against the unrounded fp64
oracle (rtol 1e-2 fp16, 2e-2 bf16, as for the product), every output finite;
exact where the softmax weights are exact (a single visible key, one
dominant key, uniform weights over a power-of-two number of keys with
integer values).  The large shapes are checked on seeded query samples.
"""
import numpy as np
import pytest

import oracle
import tiled_dense_gemm_tg_amd as tg
from tiled_dense_gemm_tg_amd import inputs as I
from gpu_util import check_exact, check_tolerance, log, to_bits, to_device

pytestmark = pytest.mark.gpu
D = 128


def _run(Bn, Sq, Sk, H, dtype, Q, K, V, causal, scale=0.0):
    import torch
    q = to_device(Q.reshape(Bn, Sq, H, D), dtype)
    k = to_device(K.reshape(Bn, Sk, H, D), dtype) if Sk else torch.empty((Bn, 0, H, D), dtype=q.dtype, device="cuda")
    v = to_device(V.reshape(Bn, Sk, H, D), dtype) if Sk else torch.empty((Bn, 0, H, D), dtype=q.dtype, device="cuda")
    out = torch.full((Bn, Sq, H, D), float("nan"), dtype=q.dtype, device="cuda")
    tg.attention(q, k, v, causal=causal, scale=scale, out=out)
    torch.cuda.synchronize()
    return to_bits(out).reshape(Bn * Sq * H, D)


def _sample(Bn, Sq, H, n, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    idx = rng.choice(Bn * Sq * H, size=min(n, Bn * Sq * H), replace=False)
    idx = np.unique(np.concatenate([idx, [0, Bn * Sq * H - 1]]))
    b, rem = np.divmod(idx, Sq * H)
    i, h = np.divmod(rem, H)
    return idx, np.stack([b, i, h], axis=1)


@pytest.mark.parametrize("dtype,Bn,Sq,Sk,H,causal", [
    (I.F16, 1, 256, 256, 2, False),
    (I.F16, 1, 256, 256, 2, True),
    (I.BF16, 2, 300, 200, 3, False),      # ragged query and key blocks
    (I.BF16, 1, 520, 520, 2, True),       # causal over three query blocks
    (I.F16, 1, 1, 1, 1, False),
    (I.F16, 1, 5, 777, 2, False),
    (I.F16, 1, 4096, 4096, 32, True),     # the measured shape, sampled queries
    (I.BF16, 1, 4096, 4096, 32, False),
    (I.BF16, 2, 700, 700, 3, True),       # causal, ragged last query and key blocks, two batches
    (I.F16, 1, 257, 257, 2, True),        # one query past a query block
    (I.F16, 1, 1000, 130, 4, False),      # many query blocks over a short, ragged key range
    (I.F16, 1, 8192, 8192, 8, True),      # the longer sequence the notes quote, sampled queries
])
def test_attention_matches_oracle(dtype, Bn, Sq, Sk, H, causal):
    Q = I.random_bits((Bn, Sq, H, D), ("normal", 0.0, 1.0), dtype, 700 + Sq)
    K = I.random_bits((Bn, Sk, H, D), ("normal", 0.0, 1.0), dtype, 701 + Sk)
    V = I.random_bits((Bn, Sk, H, D), ("normal", 0.0, 1.0), dtype, 702 + Sk)
    idx, qs = _sample(Bn, Sq, H, 96, 703)
    ref64, _ = oracle.attention(Bn, Sq, Sk, H, D, dtype, Q, K, V, causal=causal, queries=qs)
    log(f"[attn] dtype={dtype} B={Bn} Sq={Sq} Sk={Sk} H={H} causal={causal}")
    got = _run(Bn, Sq, Sk, H, dtype, Q, K, V, causal)
    check_tolerance(dtype, got[idx], ref64, "attention")


@pytest.mark.parametrize("dtype,causal", [(I.F16, False), (I.BF16, True)])
def test_attention_large_scores(dtype, causal):
    """Q and K drawn 4x wider, so scores spread over hundreds (in log2
    units) and the reference maximum of the online softmax moves many times
    (every move rescales the partial output and sum)."""
    Bn, Sq, Sk, H = 1, 600, 600 if causal else 900, 2
    Q = I.random_bits((Bn, Sq, H, D), ("normal", 0.0, 4.0), dtype, 720)
    K = I.random_bits((Bn, Sk, H, D), ("normal", 0.0, 4.0), dtype, 721)
    V = I.random_bits((Bn, Sk, H, D), ("normal", 0.0, 1.0), dtype, 722)
    idx, qs = _sample(Bn, Sq, H, 96, 723)
    ref64, _ = oracle.attention(Bn, Sq, Sk, H, D, dtype, Q, K, V, causal=causal, queries=qs)
    log(f"[attn-large] dtype={dtype} causal={causal}")
    got = _run(Bn, Sq, Sk, H, dtype, Q, K, V, causal)
    check_tolerance(dtype, got[idx], ref64, "attention, large scores")


@pytest.mark.parametrize("dtype", [I.F16, I.BF16])
def test_attention_exact_weights(dtype):
    """K = 0 gives uniform weights: with 128 keys of integer values the mean is
    exact; causal row 0 sees only key 0; a dominant key selects its value."""
    Bn, S, H = 1, 128, 2
    Q = I.random_bits((Bn, S, H, D), ("normal", 0.0, 1.0), dtype, 710)
    K = I.values_bits(np.zeros((Bn, S, H, D)), dtype)
    V = I.small_int_bits((Bn, S, H, D), dtype, 711, -8, 8)
    _, refq = oracle.attention(Bn, S, S, H, D, dtype, Q, K, V)
    log(f"[attn exact] uniform dtype={dtype}")
    check_exact(_run(Bn, S, S, H, dtype, Q, K, V, False), refq, "uniform")
    K2 = I.random_bits((Bn, S, H, D), ("normal", 0.0, 1.0), dtype, 712)
    _, refc = oracle.attention(Bn, S, S, H, D, dtype, Q, K2, V, causal=True, queries=[(0, 0, 0), (0, 0, 1)])
    got = _run(Bn, S, S, H, dtype, Q, K2, V, True)
    check_exact(got[[0, 1]], refc, "causal row 0")
    # one dominant key per head: score 64 above all others (weights e^-64)
    Qd = np.zeros((Bn, 1, H, D))
    Qd[..., 0] = 1.0
    Kd = np.zeros((Bn, S, H, D))
    Kd[0, 37, 0, 0] = 64.0
    Kd[0, 101, 1, 0] = 64.0
    Qb, Kb = I.values_bits(Qd, dtype), I.values_bits(Kd, dtype)
    _, refd = oracle.attention(Bn, 1, S, H, D, dtype, Qb, Kb, V, scale=1.0)
    got = _run(Bn, 1, S, H, dtype, Qb, Kb, V, False, scale=1.0)
    # Where V is 0 the result is only the e^-64 weights times the other values,
    # about 1e-26: fp16 weights of e^-64 are 0 (result +0), bf16 ones keep 8
    # bits, so those entries agree to 1e-20; every other entry is V exactly.
    g, r = oracle.decode(dtype, got), oracle.decode(dtype, refd)
    big = np.abs(r) >= 1e-3
    assert np.array_equal(g[big], r[big]) and (np.abs(g[~big] - r[~big]) <= 1e-20).all(), "dominant key"


def test_attention_empty_keys_give_zero():
    import torch
    q = torch.randn(1, 3, 2, D, device="cuda").half()
    k = torch.empty(1, 0, 2, D, device="cuda").half()
    out = torch.full_like(q, float("nan"))
    log("[attn] Sk = 0")
    tg.attention(q, k, k, out=out)
    torch.cuda.synchronize()
    assert (out == 0).all()

"""Pins for the oracle's 16-bit codec (decode to double, round-to-nearest-even encode).

The oracle's decoder and encoder are written from the IEEE binary16 and
bfloat16 format definitions; here they are checked against independent
library conversions (numpy's float16, torch's bfloat16) over every bit
pattern, and against a brute-force nearest-value search over the full table
of representable values.
"""
import numpy as np
import pytest
import torch

import oracle

ALL = np.arange(65536, dtype=np.uint16)


def _numpy_f16(bits):
    return bits.view(np.float16).astype(np.float64)


def _torch_bf16(bits):
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()


def _same(a, b):
    return ((a == b) & (np.signbit(a) == np.signbit(b))) | (np.isnan(a) & np.isnan(b))


@pytest.mark.parametrize("dtype,ref", [(oracle.F16, _numpy_f16), (oracle.BF16, _torch_bf16)])
def test_decode_every_pattern(dtype, ref):
    d = oracle.decode(dtype, ALL)
    assert _same(d, ref(ALL)).all()


@pytest.mark.parametrize("dtype", [oracle.F16, oracle.BF16])
def test_encode_roundtrips_every_finite_pattern(dtype):
    d = oracle.decode(dtype, ALL)
    keep = ~np.isnan(d)
    back = oracle.encode(dtype, d[keep])
    assert np.array_equal(back, ALL[keep])


@pytest.mark.parametrize("dtype", [oracle.F16, oracle.BF16])
def test_encode_nan_is_nan(dtype):
    q = oracle.encode(dtype, np.array([np.nan, -np.nan]))
    assert np.isnan(oracle.decode(dtype, q)).all()


def _table(dtype):
    """Sorted non-negative finite values and their patterns, decoded by the library."""
    ref = _numpy_f16 if dtype == oracle.F16 else _torch_bf16
    pos = ALL[ALL < 0x8000]
    vals = ref(pos)
    fin = np.isfinite(vals)
    vals, pos = vals[fin], pos[fin]
    order = np.argsort(vals, kind="stable")
    vals, pos = vals[order], pos[order]
    # +0 only (drop nothing else; all positive patterns are distinct values)
    return vals, pos


def _brute_force_round(dtype, x):
    """Nearest representable value by search; ties to the even pattern; overflow past
    the midpoint between the largest finite value and the next power of two -> inf."""
    vals, pats = _table(dtype)
    top = 2.0 ** 16 if dtype == oracle.F16 else 2.0 ** 128
    inf_pat = 0x7C00 if dtype == oracle.F16 else 0x7F80
    a = np.abs(x)
    idx = np.searchsorted(vals, a, side="right") - 1
    lo = vals[idx]
    lo_p = pats[idx].astype(np.int64)
    has_hi = idx + 1 < len(vals)
    hi = np.where(has_hi, vals[np.minimum(idx + 1, len(vals) - 1)], top)
    hi_p = np.where(has_hi, pats[np.minimum(idx + 1, len(vals) - 1)], inf_pat).astype(np.int64)
    d_lo = a - lo          # exact: lo <= a <= hi are adjacent (Sterbenz)
    d_hi = hi - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi_p % 2 == 0))
    p = np.where(pick_hi, hi_p, lo_p)
    p = np.where(a >= top, inf_pat, p)
    p = p | np.where(np.signbit(x), 0x8000, 0)
    return p.astype(np.uint16)


def _probe_values(dtype, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    vals, _ = _table(dtype)
    lo_e, hi_e = (-26, 17) if dtype == oracle.F16 else (-136, 128.5)
    wide = np.exp2(rng.uniform(lo_e, hi_e, 40000)) * rng.choice([-1.0, 1.0], 40000)
    # exact midpoints between neighbours (ties), and one double-ulp either side of them
    i = rng.integers(0, len(vals) - 1, 20000)
    mid = (vals[i] + vals[i + 1]) / 2
    near = np.concatenate([mid, np.nextafter(mid, 0), np.nextafter(mid, np.inf)])
    near = near * rng.choice([-1.0, 1.0], near.size)
    edges = np.array([0.0, -0.0, vals[-1], -vals[-1], vals[1], vals[1] / 2, vals[1] / 2 * 1.0000001,
                      (vals[-1] + (2.0 ** 16 if dtype == oracle.F16 else 2.0 ** 128)) / 2])
    return np.concatenate([wide, near, edges])


@pytest.mark.parametrize("dtype", [oracle.F16, oracle.BF16])
def test_encode_matches_brute_force_nearest_even(dtype):
    x = _probe_values(dtype, 7 + dtype)
    got = oracle.encode(dtype, x)
    want = _brute_force_round(dtype, x)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(x[i], hex(got[i]), hex(want[i])) for i in bad[:5]]


def test_encode_f16_matches_numpy_cast():
    x = _probe_values(oracle.F16, 11)
    got = oracle.encode(oracle.F16, x)
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)


def test_encode_bf16_matches_torch_on_float32_values():
    # torch rounds float32 -> bfloat16 to nearest even; restrict to float32-exact inputs
    with np.errstate(over="ignore"):
        x = _probe_values(oracle.BF16, 13).astype(np.float32)
    x = x[np.isfinite(x)].astype(np.float64)
    got = oracle.encode(oracle.BF16, x)
    want = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)


def test_encode_overflow_and_subnormal_boundaries_f16():
    e = oracle.encode
    assert e(oracle.F16, [65504.0])[0] == 0x7BFF
    assert e(oracle.F16, [65519.99])[0] == 0x7BFF
    assert e(oracle.F16, [65520.0])[0] == 0x7C00          # tie with 2^16 goes to even -> inf
    assert e(oracle.F16, [-1e9])[0] == 0xFC00
    assert e(oracle.F16, [2.0 ** -24])[0] == 0x0001
    assert e(oracle.F16, [2.0 ** -25])[0] == 0x0000       # tie with 0 goes to even (0)
    assert e(oracle.F16, [1.5 * 2.0 ** -24])[0] == 0x0002  # tie between 1 and 2 ulps -> 2
    assert e(oracle.F16, [2.0 ** -14 - 2.0 ** -26])[0] == 0x0400  # rounds up to the smallest normal

"""The chain's scores divide by the temperature as c * RN64(1/T) rounded once
to fp32 (one fp64 multiply instead of an fp32 division).  That is the IEEE
fp32 quotient for every fp32 c and T > 0: the fp64 product is within 2^-52
of c/T relatively, while a quotient of two fp32 numbers never comes within
2^-51 of its magnitude of an fp32 rounding midpoint.  Checked here on
random bit patterns and on every significand at several exponents against
numpy's fp32 division (CPU only)."""

import numpy as np


def _check(c, T):
    with np.errstate(all="ignore"):
        ref = c / T
        dev = (c.astype(np.float64) * (1.0 / T.astype(np.float64))).astype(np.float32)
    same = (ref.view(np.uint32) == dev.view(np.uint32)) | (np.isnan(ref) & np.isnan(dev))
    return int((~same).sum())


def test_random_bit_patterns():
    rng = np.random.default_rng(20261202)
    bad = n = 0
    for _ in range(4):
        c = rng.integers(0, 2**32, size=4_000_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
        T = rng.integers(0, 2**31, size=4_000_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
        ok = np.isfinite(c) & np.isfinite(T) & (T > 0)
        bad += _check(c[ok], T[ok])
        n += int(ok.sum())
    assert n > 10**7 and bad == 0


def test_every_significand_at_sampled_temperatures():
    sig = np.arange(2**23, dtype=np.uint32)
    for Tv in (0.7, 1.5, 0.3, 1e-30, 1e30, 1.17549435e-38, 1e-45, np.inf):
        T = np.full(sig.size, Tv, dtype=np.float32)
        for e in (0, 1, 127, 200, 254):
            c = ((np.uint32(e) << np.uint32(23)) | sig).view(np.float32)
            assert _check(c, T) == 0 and _check(-c, T) == 0, (Tv, e)


def test_special_values():
    c = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1.0, -3.5], dtype=np.float32)
    for Tv in (0.7, np.inf, 1e-45):
        assert _check(c, np.full(c.size, Tv, dtype=np.float32)) == 0

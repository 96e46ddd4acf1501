"""Pins for the oracle's E4M3 decode and encode.

The pages fix the format only as "E4M3 (4-bit exponent and 3-bit mantissa)"
used on all tensors (jp-study.kr page, the passage that sets aside the
hybrid E4M3/E5M2 format of prior work for E4M3 everywhere).  The oracle reads it as
OCP E4M3FN with round-to-nearest-even and saturation at 448; these tests pin
that reading with closed forms, a brute-force nearest-value search written
here, and PyTorch's own float8_e4m3fn cast.
"""
import concurrent.futures as cf
from fractions import Fraction

import numpy as np
import pytest
import torch


def _all_codes():
    return np.arange(256, dtype=np.uint8)


def test_decode_closed_forms(oracle):
    d = oracle.e4m3_decode(_all_codes())
    nan = np.isnan(d)
    assert np.flatnonzero(nan).tolist() == [0x7F, 0xFF]
    assert d[0x00] == 0.0 and not np.signbit(d[0x00])
    assert d[0x80] == 0.0 and np.signbit(d[0x80])
    # named values from the bit layout s eeee mmm, bias 7
    assert d[0x7E] == 448.0            # 1.75 * 2^8, largest finite
    assert d[0x01] == 2.0 ** -9        # smallest subnormal
    assert d[0x07] == 7 * 2.0 ** -9    # largest subnormal
    assert d[0x08] == 2.0 ** -6        # smallest normal
    assert d[0x38] == 1.0
    assert d[0x40] == 2.0
    assert d[0x3C] == 1.5
    assert d[0x77] == 240.0            # 1.875 * 2^7
    pos = d[:0x7F]
    assert np.all(np.diff(pos) > 0), "positive codes must be strictly increasing"
    assert np.count_nonzero(pos > 0) == 126
    assert np.array_equal(d[0x80:0xFF], -pos)


def test_decode_matches_torch_float8(oracle):
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    ref = ref.to(torch.float64).numpy()
    d = oracle.e4m3_decode(_all_codes())
    both_nan = np.isnan(ref) & np.isnan(d)
    assert np.array_equal(np.isnan(ref), np.isnan(d))
    assert np.array_equal(ref[~both_nan], d[~both_nan])
    assert np.array_equal(np.signbit(ref[~both_nan]), np.signbit(d[~both_nan]))


def test_encode_roundtrip_all_codes(oracle):
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = oracle.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(vals), codes)


def test_encode_midpoints_tie_to_even(oracle):
    pos = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    for c in range(0x7E):
        mid = np.float32((pos[c] + pos[c + 1]) / 2)   # exact in fp32 (<= 5 bits)
        assert float(mid) == (pos[c] + pos[c + 1]) / 2
        even = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_encode(np.array([mid]))[0] == even, hex(c)
        assert oracle.e4m3_encode(np.array([-mid]))[0] == even | 0x80
        below = np.nextafter(mid, np.float32(0))
        above = np.nextafter(mid, np.float32(np.inf))
        assert oracle.e4m3_encode(np.array([below]))[0] == c
        assert oracle.e4m3_encode(np.array([above]))[0] == c + 1


def test_encode_saturation_and_specials(oracle):
    f = np.float32
    big = [f(448), np.nextafter(f(448), f(np.inf)), f(448 * (1 + 2 ** -23)), f(463.9), f(464),
           f(470), f(1e30), f(np.inf), f(np.finfo(np.float32).max)]
    assert np.all(oracle.e4m3_encode(np.array(big)) == 0x7E)
    assert np.all(oracle.e4m3_encode(-np.array(big)) == 0xFE)
    nan = oracle.e4m3_encode(np.array([np.nan, -np.nan], dtype=np.float32))
    assert nan[0] == 0x7F and nan[1] == 0xFF
    # below half of the smallest subnormal -> signed zero
    tiny = np.array([2.0 ** -11, 2.0 ** -10, 1e-30, 1e-45, 0.0], dtype=np.float32)
    assert np.all(oracle.e4m3_encode(tiny) == 0x00)
    assert np.all(oracle.e4m3_encode(-tiny) == 0x80)
    # just above half of the smallest subnormal -> smallest subnormal
    assert oracle.e4m3_encode(np.array([np.nextafter(f(2.0 ** -10), f(1))]))[0] == 0x01
    assert oracle.e4m3_encode(np.array([f(1.5 * 2.0 ** -9)]))[0] == 0x02   # tie -> even


def _brute_force_nearest(v: np.ndarray) -> np.ndarray:
    """Nearest E4M3 magnitude by exhaustive search over all 127 finite
    non-negative values (built from the bit layout here, not the oracle), ties
    to the even code, saturating at 448, sign kept.  Distances in fp64 are
    exact for |v| >= 2^-12 (both operands are multiples of 2^-36 and below
    2^9); smaller magnitudes are all nearer to zero than to 2^-9."""
    mags = []
    for c in range(0x7F):
        e, m = c >> 3, c & 7
        mags.append(m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    mags = np.array(mags)
    a = np.abs(v.astype(np.float64))
    out = np.empty(v.shape, dtype=np.uint8)
    chunk = 1 << 16
    for i in range(0, v.size, chunk):
        aa = np.minimum(a[i:i + chunk], 448.0)
        dist = np.abs(aa[:, None] - mags[None, :])
        best = dist.min(axis=1, keepdims=True)
        cand = dist == best
        # among equally near codes prefer the even one
        even = cand & (np.arange(0x7F)[None, :] % 2 == 0)
        pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
        out[i:i + chunk] = pick
    out[np.signbit(v)] |= 0x80
    return out


def test_encode_matches_brute_force(oracle):
    rng = np.random.default_rng(7)
    parts = [
        rng.uniform(-470, 470, 200_000),
        rng.uniform(-0.05, 0.05, 200_000),
        rng.standard_normal(200_000) * 30,
        np.ldexp(rng.uniform(1, 2, 200_000), rng.integers(-14, 9, 200_000)),
    ]
    v = np.concatenate(parts).astype(np.float32)
    v = v[np.abs(v) >= 2.0 ** -12]
    assert np.array_equal(oracle.e4m3_encode(v), _brute_force_nearest(v))


def test_encode_matches_brute_force_exact_rationals(oracle):
    """Exact rational distances (no floating point at all) on fp32 values that
    sit at and around every midpoint, including the subnormal range."""
    def exact(c):
        e, m = c >> 3, c & 7
        return Fraction(m, 512) if e == 0 else Fraction(8 + m, 8) * Fraction(2) ** (e - 7)

    pos = [exact(c) for c in range(0x7F)]
    vals = []
    for c in range(0x7E):
        mid = float((pos[c] + pos[c + 1]) / 2)
        f = np.float32(mid)
        for _ in range(3):
            f = np.nextafter(f, np.float32(0))
        for _ in range(7):
            vals.append(f)
            f = np.nextafter(f, np.float32(np.inf))
    vals = np.array(vals, dtype=np.float32)
    got = oracle.e4m3_encode(vals)
    for v, g in zip(vals, got):
        a = Fraction(float(v))
        best = min(range(0x7F), key=lambda c: (abs(a - pos[c]), c % 2))
        assert g == best, (float(v), hex(g), hex(best))


def _torch_cast(v: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(v).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_encode_matches_torch_all_patterns_below_464(oracle):
    """Every FP32 bit pattern with |v| < 464 (about 2.28e9 values, both signs).

    PyTorch's CPU cast is round-to-nearest-even and sign-preserving; it does
    not saturate, but below 464 it rounds into [0, 448] like the saturating
    encoder, so the two must agree bit for bit on this range."""
    limit = int(np.array([464.0], dtype=np.float32).view(np.uint32)[0])  # first pattern >= 464
    chunk = 1 << 25
    starts = list(range(0, limit, chunk))

    def check(start):
        stop = min(limit, start + chunk)
        bits = np.arange(start, stop, dtype=np.uint32)
        for sign in (0, 0x80000000):
            v = (bits | np.uint32(sign)).view(np.float32)
            got = oracle.e4m3_encode(v)
            ref = _torch_cast(v)
            if not np.array_equal(got, ref):
                bad = np.flatnonzero(got != ref)[0]
                return (float(v[bad]), int(got[bad]), int(ref[bad]))
        return None

    workers = min(8, len(__import__("os").sched_getaffinity(0)))
    torch.set_num_threads(1)
    try:
        with cf.ThreadPoolExecutor(workers) as ex:
            for res in ex.map(check, starts):
                assert res is None, res
    finally:
        torch.set_num_threads(workers)

"""Pins for the oracle's number formats: code tables, round trips, every
rounding tie, brute-force nearest-value search and torch's own casts."""
import os

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    rows = []
    for line in open(os.path.join(GOLDEN, name)):
        if line.startswith("#") or not line.strip():
            continue
        a, b = line.split()
        rows.append((a, float(b)))
    return rows


def test_e4m3_landmarks():
    for hexcode, val in _golden("e4m3_landmarks.txt"):
        c = int(hexcode, 16)
        got = F.e4m3_decode(np.array([c], np.uint8))[0]
        assert got == val and np.signbit(got) == np.signbit(val)


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = F.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.nanmax(ours) == 448.0


def test_e4m3_round_trip():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = F.e4m3_decode(codes).astype(np.float32)
    vals[codes == 0x80] = np.float32(-0.0)
    assert np.array_equal(F.e4m3_encode(vals), codes)


def _positive_grid():
    codes = np.arange(0, 0x7F, dtype=np.uint8)
    return codes, F.e4m3_decode(codes)


def test_e4m3_ties_to_even_at_every_midpoint():
    codes, vals = _positive_grid()
    for i in range(len(vals) - 1):
        lo, hi = vals[i], vals[i + 1]
        mid = np.float32((lo + hi) / 2)           # exact in float32
        assert float(mid) == (lo + hi) / 2
        even = codes[i] if codes[i] % 2 == 0 else codes[i + 1]
        assert F.e4m3_encode(np.array([mid]))[0] == even
        below = np.nextafter(mid, np.float32(0))
        above = np.nextafter(mid, np.float32(1e9))
        assert F.e4m3_encode(np.array([below]))[0] == codes[i]
        assert F.e4m3_encode(np.array([above]))[0] == codes[i + 1]
        # negative side mirrors with the sign bit
        assert F.e4m3_encode(np.array([-mid]))[0] == (even | 0x80)


def test_e4m3_saturation_and_specials():
    x = np.array([448.0, 449.0, 464.0, 465.0, 480.0, 1e6, np.inf, -np.inf, -1e30, 0.0, -0.0,
                  1e-40, -1e-40], np.float32)
    want = [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x00, 0x80, 0x00, 0x80]
    assert list(F.e4m3_encode(x)) == want
    assert F.e4m3_encode(np.array([np.nan], np.float32))[0] & 0x7F == 0x7F


def _torch_e4m3(x):
    xc = np.clip(x, -448.0, 448.0).astype(np.float32)
    return torch.from_numpy(xc).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_all_bf16_patterns_match_torch():
    bits = np.arange(65536, dtype=np.uint32) << 16
    x = bits.view(np.float32)
    x = x[~np.isnan(x)]
    assert np.array_equal(F.e4m3_encode(x), _torch_e4m3(x))


def test_e4m3_random_fp32_match_torch():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2**32, size=4_000_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    # plus values concentrated in the representable range
    y = (rng.standard_normal(4_000_000) * np.exp2(rng.uniform(-12, 10, 4_000_000))).astype(np.float32)
    for a in (x, y):
        assert np.array_equal(F.e4m3_encode(a), _torch_e4m3(a))


def test_e4m3_exhaustive_subnormal_boundary_binades():
    # every float32 in [2^-11, 2^-5): the subnormal/normal transition
    lo = np.float32(2.0 ** -11).view(np.uint32)
    hi = np.float32(2.0 ** -5).view(np.uint32)
    x = np.arange(lo, hi, dtype=np.uint32).view(np.float32)
    assert np.array_equal(F.e4m3_encode(x), _torch_e4m3(x))
    assert np.array_equal(F.e4m3_encode(-x), _torch_e4m3(-x))


def test_e2m1_table_and_round_trip():
    table = _golden("e2m1_values.txt")
    codes = np.array([int(c) for c, _ in table])
    vals = np.array([v for _, v in table])
    assert np.array_equal(F.e2m1_decode(codes), vals)
    assert np.array_equal(F.e2m1_decode(codes | 8), -vals)
    assert F.e2m1_decode(np.arange(16)).max() == F.E2M1_MAX == 6.0
    assert np.array_equal(F.e2m1_encode(vals.astype(np.float32)), codes)
    neg = F.e2m1_encode((-vals).astype(np.float32))
    assert np.array_equal(neg, codes | 8)         # -0 -> 0x8 too


def test_e2m1_ties_to_even_code():
    x = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    want_vals = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]
    got = F.e2m1_decode(F.e2m1_encode(x))
    assert list(got) == want_vals
    assert list(F.e2m1_decode(F.e2m1_encode(-x))) == [-v for v in want_vals]


def test_e2m1_brute_force_nearest():
    grid = F.e2m1_decode(np.arange(8))
    rng = np.random.default_rng(3)
    x = (rng.uniform(-8, 8, 200_000)).astype(np.float32)
    got = F.e2m1_decode(F.e2m1_encode(x))
    ax = np.minimum(np.abs(x).astype(np.float64), 6.0)
    dist = np.abs(ax[:, None] - grid[None, :])
    best = dist.min(axis=1)
    assert np.allclose(np.abs(np.abs(got) - ax), best, rtol=0, atol=0)
    assert np.all(np.sign(got[got != 0]) == np.sign(x[got != 0]))
    sat = np.array([6.0, 6.5, 7.0, 8.0, 1e9, np.inf], np.float32)
    assert np.all(F.e2m1_decode(F.e2m1_encode(sat)) == 6.0)


def test_e2m1_pack_low_nibble_first():
    codes = np.array([[1, 2, 3, 4]], np.uint8)
    packed = F.e2m1_pack(codes)
    assert list(packed[0]) == [0x21, 0x43]
    assert np.array_equal(F.e2m1_unpack(packed), codes)


def test_e8m0_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = F.e8m0_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).double().numpy()
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    assert np.array_equal(ours[:255], ref[:255])


def test_unbiased_exponent_against_frexp():
    rng = np.random.default_rng(5)
    bits = rng.integers(1, 0x7F800000, size=200_000, dtype=np.int64).astype(np.uint32)
    x = bits.view(np.float32)
    mant, ex = np.frexp(x.astype(np.float64))
    assert np.array_equal(F.f32_unbiased_exponent(x), ex - 1)
    sub = np.array([1, 2, 3, 0x400000, 0x7FFFFF], np.uint32).view(np.float32)
    assert list(F.f32_unbiased_exponent(sub)) == [-149, -148, -148, -127, -127]

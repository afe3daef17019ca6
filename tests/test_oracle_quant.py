"""Pins for the oracle's quantizers: closed forms, error bounds, the axis each
scale belongs to, and torch casts of the scaled values."""
import numpy as np
import torch

from oracle import formats as F
from oracle import quant as Q


def _torch_codes(xs):
    xc = np.clip(xs, -448, 448).astype(np.float32)
    return torch.from_numpy(xc).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_fp8_block_basic_closed_forms():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((2, 3, 200, 64)).astype(np.float32)
    codes, s = Q.fp8_block_quantize(x, 64)
    assert s.shape == (2, 3, 4)
    for b in range(4):
        xb = x[..., b * 64:(b + 1) * 64, :]
        amax = np.abs(xb).max(axis=(-2, -1))
        assert np.array_equal(s[..., b], (np.float32(448.0) / amax).astype(np.float32))
        # the amax element encodes to +-448
        cb = codes[..., b * 64:(b + 1) * 64, :].reshape(2, 3, -1)
        flat = xb.reshape(2, 3, -1)
        at = np.abs(flat).argmax(axis=-1)
        got = np.take_along_axis(cb, at[..., None], -1)[..., 0]
        assert np.all((got & 0x7F) == 0x7E)
        # codes are the torch cast of fl32(x * s)
        assert np.array_equal(cb, _torch_codes(flat * s[..., b][..., None]))
    # partial last block (tokens 192..199) uses its own amax
    amax_last = np.abs(x[..., 192:, :]).max(axis=(-2, -1))
    assert np.array_equal(s[..., 3], (np.float32(448) / amax_last).astype(np.float32))


def test_fp8_block_error_bound():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((4, 256, 32)) * np.exp2(rng.uniform(-8, 8, (4, 256, 1)))).astype(np.float32)
    codes, s = Q.fp8_block_quantize(x, 64)
    xh = Q.fp8_block_dequantize(codes, s, 64)
    sr = np.repeat(s.astype(np.float64), 64, axis=-1)[..., :, None]
    y = np.abs(x.astype(np.float64)) * sr
    err = np.abs(xh - x)
    normal = y >= 2.0 ** -6
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(x[normal]) * (1 + 1e-6))
    assert np.all(err[~normal] * sr[..., 0:1].repeat(32, -1)[~normal] <= 2.0 ** -10 * (1 + 1e-6))


def test_fp8_block_powers_of_two_exact_and_idempotent():
    rng = np.random.default_rng(2)
    ex = rng.integers(-6, 6, (128, 16))
    x = (np.ldexp(1.0, ex) * rng.choice([-1, 1], (128, 16))).astype(np.float32)
    codes, s = Q.fp8_block_quantize(x, 64)
    assert np.array_equal(Q.fp8_block_dequantize(codes, s, 64), x.astype(np.float64))
    y = rng.standard_normal((128, 16)).astype(np.float32)
    c1, s1 = Q.fp8_block_quantize(y, 64)
    yh = Q.fp8_block_dequantize(c1, s1, 64).astype(np.float32)
    c2, s2 = Q.fp8_block_quantize(yh, 64)
    assert np.array_equal(s1, s2) and np.array_equal(c1, c2)


def test_fp8_block_scale_belongs_to_its_block():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1, 256, 16)).astype(np.float32)
    c0, s0 = Q.fp8_block_quantize(x, 64)
    x2 = x.copy()
    x2[:, 64:128] *= 2
    c1, s1 = Q.fp8_block_quantize(x2, 64)
    assert np.array_equal(c0, c1)
    assert s1[0, 1] == s0[0, 1] / 2
    assert np.array_equal(np.delete(s1, 1, axis=1), np.delete(s0, 1, axis=1))


def test_fp8_zero_block():
    x = np.zeros((128, 8), np.float32)
    x[64:] = 1.0
    codes, s = Q.fp8_block_quantize(x, 64)
    assert s[0] == 1.0 and np.all(codes[:64] == 0)
    assert s[1] == 448.0 and np.all(codes[64:] == 0x7E)


def test_fp8_channel_scale_belongs_to_its_channel():
    rng = np.random.default_rng(4)
    v = rng.standard_normal((2, 300, 32)).astype(np.float32)
    c0, s0 = Q.fp8_channel_quantize(v)
    assert s0.shape == (2, 32)
    assert np.array_equal(s0, (np.float32(448) / np.abs(v).max(axis=-2)).astype(np.float32))
    v2 = v.copy()
    v2[..., 5] *= 4
    c1, s1 = Q.fp8_channel_quantize(v2)
    assert np.array_equal(c0, c1)
    assert np.all(s1[:, 5] == s0[:, 5] / 4)
    assert np.array_equal(c0, _torch_codes(v * s0[:, None, :]))
    vh = Q.fp8_channel_dequantize(c0, s0)
    assert np.all(np.abs(vh - v) <= 2.0 ** -4 * np.abs(v) + 2.0 ** -10 / s0[:, None, :])


def test_mxfp4_scale_rule_and_bounds():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((64, 128)) * np.exp2(rng.uniform(-20, 20, (64, 4)).repeat(32, -1))).astype(np.float32)
    codes, e8 = Q.mxfp4_quantize(x)
    assert codes.shape == x.shape and e8.shape == (64, 4)
    e = e8.astype(np.int64) - 127
    amax = np.abs(x).reshape(64, 4, 32).max(-1)
    ratio = amax / np.ldexp(1.0, e)
    assert np.all((ratio >= 4) & (ratio < 8))
    xh = Q.mxfp4_dequantize(codes, e8)
    grid = F.e2m1_decode(np.arange(8))
    y = np.abs(x.reshape(64, 4, 32).astype(np.float64)) / np.ldexp(1.0, e)[..., None]
    yc = np.minimum(y, 6.0)
    best = np.abs(yc[..., None] - grid).min(-1)
    got = np.abs(xh.reshape(64, 4, 32)) / np.ldexp(1.0, e)[..., None]
    assert np.allclose(np.abs(got - yc), best, atol=0, rtol=0)


def test_mxfp4_constant_zero_and_clipped_groups():
    x = np.zeros((3, 64), np.float32)
    x[0, :32] = 1.0          # -> e = -2, y = 4, exact
    x[0, 32:] = 1.5          # -> y = 6, exact
    x[1, :32] = 1.75         # -> y = 7, clips to 6 * 2^-2 = 1.5
    codes, e8 = Q.mxfp4_quantize(x)
    xh = Q.mxfp4_dequantize(codes, e8)
    assert np.all(xh[0] == x[0])
    assert np.all(xh[1, :32] == 1.5)
    assert e8[2, 0] == 0 and e8[2, 1] == 0 and np.all(codes[2] == 0)
    assert e8[1, 1] == 0
    assert e8[0, 0] == 125 and e8[0, 1] == 125


def test_mxfp4_tiny_and_subnormal_groups():
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = np.float32(2.0 ** -130)  # subnormal amax -> clamped exponent
    x[0, 1] = -np.float32(2.0 ** -131)
    codes, e8 = Q.mxfp4_quantize(x)
    assert e8[0, 0] == 0              # e = -127
    xh = Q.mxfp4_dequantize(codes, e8)
    # y = 2^-130 * 2^127 = 1/8 -> 0 ; keep sign of zero on the negative element
    assert xh[0, 0] == 0 and codes[0, 1] == 0x8


def test_mxfp4_token_scale_belongs_to_its_channel_and_group():
    """V for FP4 P.V: one E8M0 scale per channel and per 32 consecutive
    tokens.  A single nonzero value at (token 37, channel 5) sets only the
    scale of (group 1, channel 5): 3.0 -> e = floor(log2 3) - 2 = -1, code
    3.0 / 2^-1 = 6 (E2M1 code 7)."""
    v = np.zeros((96, 8), np.float32)
    v[37, 5] = 3.0
    codes, e8 = Q.mxfp4_token_quantize(v)
    assert e8.shape == (3, 8) and codes.shape == (96, 8)
    want = np.zeros((3, 8), np.uint8)        # all-zero groups: e = -127, code 0
    want[1, 5] = 127 - 1
    assert np.array_equal(e8, want)
    assert codes[37, 5] == 7 and np.count_nonzero(codes) == 1
    deq = Q.mxfp4_token_dequantize(codes, e8)
    assert deq[37, 5] == 3.0 and np.count_nonzero(deq) == 1


def test_mxfp4_token_bounds():
    """Per (32-token group, channel): amax / 2^e in [4, 8), and every element
    lands on the nearest E2M1 point of its group's grid after clipping at 6."""
    rng = np.random.default_rng(12)
    v = (rng.standard_normal((128, 16)) * np.exp(rng.standard_normal((1, 16)))).astype(np.float32)
    codes, e8 = Q.mxfp4_token_quantize(v)
    e = e8.astype(np.int64) - 127                               # [4, 16]
    a = np.abs(v.astype(np.float64)).reshape(4, 32, 16)
    ratio = a.max(axis=1) / np.ldexp(1.0, e)
    assert np.all((ratio >= 4) & (ratio < 8))
    y = np.minimum(a / np.ldexp(1.0, e)[:, None, :], 6.0)
    grid = F.e2m1_decode(np.arange(8))
    best = np.abs(y[..., None] - grid).min(-1)
    got = np.abs(Q.mxfp4_token_dequantize(codes, e8)).reshape(4, 32, 16) / np.ldexp(1.0, e)[:, None, :]
    assert np.array_equal(np.abs(got - y), best)


def test_mxfp4_token_partial_group():
    """N = 40 tokens: the second group holds tokens 32..39 only, and its scale
    comes from them alone (amax 0.75 -> e = floor(log2 0.75) - 2 = -3)."""
    v = np.zeros((40, 2), np.float32)
    v[:32, 0] = 4.0                       # group 0: e = 0
    v[35, 0] = 0.75
    v[39, 1] = -0.5                       # group 1, channel 1: e = -3, code -4 (0xE)
    codes, e8 = Q.mxfp4_token_quantize(v)
    assert e8.shape == (2, 2) and codes.shape == (40, 2)
    assert e8[0, 0] == 127 and e8[1, 0] == 127 - 3 and e8[1, 1] == 127 - 3
    deq = Q.mxfp4_token_dequantize(codes, e8)
    assert deq[35, 0] == 0.75 and deq[39, 1] == -0.5 and np.all(deq[:32, 0] == 4.0)

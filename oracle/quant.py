"""Quantizers of the staged precision recipe (test infrastructure).

[FPS §2.1] block FP8 quantisation: X_hat = dequantize(FP8_convert(X * s_g)) / s_g
           with one scale s_g per block.
[FPS §3.1, staged quantisation strategy]
           Q and K: FP8 per block, each block with its own scale;
           V: FP8 per channel;
           P: FP8 per tensor with the fixed scale 1/448 (see attention.py).
[FP4G §1, micro-scaling] divide a block by a scale kept at higher precision,
           round to E2M1; dequantised value = code * scale.  The MX variant
           keeps one E8M0 (power-of-two) scale per 32 elements.
[FV §1, FP4 attention] both products in FP4: for the P.V product V is
           quantised to MXFP4 along the token axis (the reduction axis of
           P.V): one E8M0 scale per channel and per 32 consecutive tokens.

Readings where the pages leave a step open (listed with reasons in the design
notes of the repository):
  * s_g = fl32(448 / amax) over the block (IEEE float32 division); s_g = 1 when
    amax == 0 or the quotient is not finite.  The scale multiplies before the
    conversion and divides after it.
  * a Q/K "block" is `blk` consecutive tokens x all d channels of one
    (batch, head); the last block may be partial and uses its own tokens.
  * V "channel" granularity: one scale per (batch, head, channel) over all
    tokens.
  * MXFP4 shared exponent: e = floor(log2 amax) - 2 (E2M1's largest exponent is
    2), clamped to [-127, 127]; e = -127 for an all-zero group; the E8M0 code is
    e + 127; element codes are E2M1(x * 2^-e) with saturation at 6.
All arrays have the token axis second to last and channels last.
"""
import numpy as np

from .formats import (e4m3_encode, e4m3_decode, e2m1_encode, e2m1_decode,
                      f32_unbiased_exponent)

FP8_QMAX = np.float32(448.0)


def fp8_scale_from_amax(amax):
    """s = fl32(448 / amax); 1 where amax is 0 or the quotient is not finite."""
    amax = np.asarray(amax, dtype=np.float32)
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        s = (FP8_QMAX / amax).astype(np.float32)
    bad = (amax == 0) | ~np.isfinite(s)
    return np.where(bad, np.float32(1.0), s).astype(np.float32)


def fp8_block_quantize(x, blk):
    """Per-block FP8: returns (codes uint8 same shape as x, scales float32
    [..., ceil(N/blk)])."""
    x = np.asarray(x, dtype=np.float32)
    n = x.shape[-2]
    nb = -(-n // blk)
    codes = np.empty(x.shape, dtype=np.uint8)
    scales = np.empty(x.shape[:-2] + (nb,), dtype=np.float32)
    for b in range(nb):
        xb = x[..., b * blk:(b + 1) * blk, :]
        amax = np.abs(xb).max(axis=(-2, -1))
        s = fp8_scale_from_amax(amax)
        scales[..., b] = s
        codes[..., b * blk:(b + 1) * blk, :] = e4m3_encode(xb * s[..., None, None])
    return codes, scales


def fp8_block_dequantize(codes, scales, blk):
    n = codes.shape[-2]
    s = np.repeat(scales.astype(np.float64), blk, axis=-1)[..., :n]
    return e4m3_decode(codes) / s[..., :, None]


def fp8_channel_quantize(v):
    """Per-channel FP8: returns (codes uint8 same shape, scales float32 [..., d])."""
    v = np.asarray(v, dtype=np.float32)
    amax = np.abs(v).max(axis=-2)
    s = fp8_scale_from_amax(amax)
    codes = e4m3_encode(v * s[..., None, :])
    return codes, s


def fp8_channel_dequantize(codes, scales):
    return e4m3_decode(codes) / scales.astype(np.float64)[..., None, :]


def mxfp4_quantize(x, group=32):
    """MXFP4 along the last axis: returns (codes uint8 4-bit, one per element;
    e8m0 uint8 [..., d/group])."""
    x = np.asarray(x, dtype=np.float32)
    d = x.shape[-1]
    assert d % group == 0
    g = x.reshape(x.shape[:-1] + (d // group, group))
    amax = np.abs(g).max(axis=-1)
    e = np.clip(f32_unbiased_exponent(amax) - 2, -127, 127)
    e = np.where(amax == 0, -127, e)
    # x * 2^-e is exact in float64; converting to float32 rounds only values
    # far below E2M1's smallest step, which encode to (signed) zero either way.
    scaled = (g.astype(np.float64) * np.ldexp(1.0, -e)[..., None]).astype(np.float32)
    codes = e2m1_encode(scaled).reshape(x.shape)
    return codes, (e + 127).astype(np.uint8)


def mxfp4_dequantize(codes, e8m0, group=32):
    d = codes.shape[-1]
    vals = e2m1_decode(codes).reshape(codes.shape[:-1] + (d // group, group))
    scale = np.ldexp(1.0, e8m0.astype(np.int64) - 127)
    return (vals * scale[..., None]).reshape(codes.shape)


def mxfp4_token_quantize(v, group=32):
    """MXFP4 along the token axis (second to last): one E8M0 scale per
    channel and per `group` consecutive tokens; a last partial group counts
    only its tokens (as zero-padded token slots would).  Returns (codes uint8
    4-bit, same shape as v; e8m0 uint8 [..., ceil(N/group), d])."""
    v = np.asarray(v, dtype=np.float32)
    n = v.shape[-2]
    npad = -(-n // group) * group
    pad = np.zeros(v.shape[:-2] + (npad - n, v.shape[-1]), np.float32)
    vt = np.swapaxes(np.concatenate([v, pad], axis=-2), -1, -2)
    codes, e8 = mxfp4_quantize(vt, group)
    return np.swapaxes(codes, -1, -2)[..., :n, :], np.swapaxes(e8, -1, -2)


def mxfp4_token_dequantize(codes, e8m0, group=32):
    n = codes.shape[-2]
    sc = np.ldexp(1.0, e8m0.astype(np.int64) - 127)
    return e2m1_decode(codes) * np.repeat(sc, group, axis=-2)[..., :n, :]

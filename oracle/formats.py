"""Number formats, written from their bit definitions (test infrastructure).

FP8 E4M3 [FPS §2.1 names E4M3/E5M2; the fixed P scale 1/448 of §3.1 fixes the
variant with maximum 448, i.e. the OCP "fn" encoding]:
    1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities; the only NaN
    patterns are S.1111.111 (0x7F, 0xFF); largest finite 0x7E = 448;
    subnormals m/8 * 2^-6 (step 2^-9).
FP4 E2M1 [FP4G §1]: 1 sign, 2 exponent (bias 1), 1 mantissa bit; magnitudes
    {0, 0.5, 1, 1.5, 2, 3, 4, 6}; largest 6.
E8M0 [FP4G §1, the higher-precision block scale of micro-scaling]: an unsigned
    8-bit biased exponent, value 2^(c-127); 0xFF is NaN.

Encoders round to nearest, ties to even (on the code's last bit), saturate at
the largest finite magnitude and keep the sign of zero.  They work on the
IEEE-754 binary32 bit pattern with integer operations so that no host
floating-point rounding mode is involved.
"""
import numpy as np

E4M3_MAX = 448.0
E2M1_MAX = 6.0


def _f32_bits(x):
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    return x.view(np.uint32)


# ---------------------------------------------------------------- E4M3 (fn)
def e4m3_decode(codes):
    """Exact value of each E4M3 code as float64 (NaN for 0x7F/0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = (1.0 + m / 8.0) * np.ldexp(1.0, e - 7)
    sub = (m / 8.0) * 2.0 ** -6
    val = sign * np.where(e == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def e4m3_encode(x):
    """float32 -> E4M3 code: round-to-nearest-even, saturate to +-448,
    subnormals kept, -0 -> 0x80, NaN -> 0x7F|sign."""
    bits = _f32_bits(x).astype(np.int64)
    sign = (bits >> 31) & 1
    a = bits & 0x7FFFFFFF                      # |x| bit pattern
    is_nan = a > 0x7F800000
    e32 = a >> 23                              # biased binary32 exponent
    m32 = a & 0x7FFFFF
    # normal E4M3 range |x| >= 2^-6  <=>  e32 >= 127 - 6
    # Re-bias the exponent to E4M3 (bias 7) keeping all 23 fraction bits, then
    # round away the low 20 bits to nearest-even; a carry propagates into the
    # exponent by itself.
    rebased = ((e32 - 127 + 7) << 23) | m32
    lsb = (rebased >> 20) & 1
    rounded = (rebased + 0x7FFFF + lsb) >> 20
    normal_code = np.minimum(rounded, 0x7E)    # saturate (0x7F would be NaN)
    # subnormal range |x| < 2^-6: value = k * 2^-9, k = rint(|x| * 2^9)
    # (scaling by a power of two is exact; np.rint rounds half to even).
    ax = np.abs(np.asarray(x, dtype=np.float32)).astype(np.float64)
    ax = np.where(e32 >= 127 - 6, 0.0, ax)     # only the subnormal range is used
    k = np.rint(ax * 512.0).astype(np.int64)   # in [0, 8]; 8 == code 0x08 = 2^-6
    code = np.where(e32 >= 127 - 6, normal_code, k)
    code = np.where(a >= 0x7F800000, 0x7E, code)   # +-inf saturates
    code = code | (sign << 7)
    code = np.where(is_nan, 0x7F | (sign << 7), code)
    return code.astype(np.uint8)


# ---------------------------------------------------------------- E2M1
def e2m1_decode(codes):
    """Exact value of each 4-bit E2M1 code (low 4 bits of the input)."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    sign = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = c & 0x1
    normal = (1.0 + m / 2.0) * np.ldexp(1.0, e - 1)
    sub = m * 0.5
    return sign * np.where(e == 0, sub, normal)


def e2m1_encode(x):
    """float32 -> 4-bit E2M1 code: round-to-nearest-even, saturate to +-6,
    -0 -> 0x8 (NaN inputs are outside the contract and map to +-6)."""
    bits = _f32_bits(x).astype(np.int64)
    sign = (bits >> 31) & 1
    a = bits & 0x7FFFFFFF
    e32 = a >> 23
    m32 = a & 0x7FFFFF
    # normal range |x| >= 1 (E2M1 bias 1): keep 1 fraction bit, drop 22
    rebased = ((e32 - 127 + 1) << 23) | m32
    lsb = (rebased >> 22) & 1
    rounded = (rebased + 0x1FFFFF + lsb) >> 22
    normal_code = np.minimum(rounded, 0x7)
    ax = np.abs(np.asarray(x, dtype=np.float32)).astype(np.float64)
    ax = np.where(e32 >= 127, 0.0, ax)         # only the subnormal range is used
    k = np.rint(ax * 2.0).astype(np.int64)     # subnormal step 0.5; 2 == code 2 = 1.0
    code = np.where(e32 >= 127, normal_code, k)
    code = np.where(a >= 0x7F800000, 0x7, code)
    return (code | (sign << 3)).astype(np.uint8)


def e2m1_pack(codes):
    """Pack 4-bit codes two per byte along the last axis: element 2k in the low
    nibble, element 2k+1 in the high nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    assert c.shape[-1] % 2 == 0
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def e2m1_unpack(packed):
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


# ---------------------------------------------------------------- E8M0
def e8m0_decode(codes):
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    return np.where(c == 255, np.nan, np.ldexp(1.0, c - 127))


def f32_unbiased_exponent(x):
    """floor(log2|x|) for finite nonzero float32 x, from the bit pattern
    (subnormals included: their exponent comes from the leading set bit)."""
    a = _f32_bits(x).astype(np.int64) & 0x7FFFFFFF
    e32 = a >> 23
    m32 = a & 0x7FFFFF
    # for subnormals the value is m32 * 2^-149; floor(log2) = bitlen(m32)-1-149
    bitlen = np.zeros_like(m32)
    t = m32.copy()
    for _ in range(23):
        nz = t > 0
        bitlen += nz
        t >>= 1
    return np.where(e32 > 0, e32 - 127, bitlen - 1 - 149)

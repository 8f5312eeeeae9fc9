"""Exact decoders from storage codes to float64 (oracle; test infrastructure only).

Every decoded value is exactly representable in float64, so nothing here
rounds.
"""
import numpy as np


def decode_f32(a):
    """float32 array -> float64 (exact)."""
    a = np.asarray(a)
    if a.dtype != np.float32:
        raise TypeError("decode_f32 expects float32, got %s" % a.dtype)
    return a.astype(np.float64)


def decode_bf16(bits):
    """bfloat16 codes (uint16 array) -> float64.

    A bfloat16 is the upper half of an IEEE binary32 word, so widening the
    code by 16 zero bits yields the binary32 value exactly.
    """
    bits = np.asarray(bits)
    if bits.dtype != np.uint16:
        raise TypeError("decode_bf16 expects uint16 codes, got %s" % bits.dtype)
    with np.errstate(invalid="ignore"):
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def decode_e4m3fn(codes):
    """OCP 8-bit float E4M3 ("fn": finite + NaN, no infinities) -> float64.

    Written from the format definition in the OCP 8-bit floating point
    specification: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
    exponent field 0 encodes subnormals m/8 * 2^-6; the single pattern
    S.1111.111 is NaN; the largest finite magnitude is 1.75 * 2^8 = 448.
    """
    c = np.asarray(codes)
    if c.dtype != np.uint8:
        raise TypeError("decode_e4m3fn expects uint8 codes, got %s" % c.dtype)
    c = c.astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = c & 0x7
    normal = np.ldexp(1.0 + man / 8.0, exp - 7)
    subnormal = np.ldexp(man / 8.0, -6)
    mag = np.where(exp == 0, subnormal, normal)
    mag = np.where((exp == 0xF) & (man == 0x7), np.nan, mag)
    return sign * mag


def encode_e4m3fn(x):
    """float32 values -> OCP E4M3FN codes: round to nearest, ties to even,
    finite values beyond +-448 saturate to +-448 ("satfinite"), NaN -> 0x7F.

    Written from the format definition (see decode_e4m3fn).  The codes 0x00 ..
    0x7E enumerate the non-negative finite values in increasing order, so the
    nearest magnitude is found by bisection over that table; on a tie the code
    whose mantissa LSB is 0 wins, and for these codes the mantissa LSB is the
    code's own LSB.  The sign bit is copied, so a negative input that rounds to
    zero gives 0x80.
    """
    x = np.asarray(x, dtype=np.float32)
    table = decode_e4m3fn(np.arange(0x7F, dtype=np.uint8))  # 0 .. 448, strictly increasing
    a = np.minimum(np.abs(x).astype(np.float64), 448.0)
    hi = np.clip(np.searchsorted(table, a, side="left"), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_lo = a - table[lo]
    d_hi = table[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo).astype(np.uint8)
    code = code | (np.signbit(x).astype(np.uint8) << np.uint8(7))
    return np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)

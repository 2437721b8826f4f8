"""Storage-format decoding and encoding for the oracle (test infrastructure only).

bf16 is the upper half of an IEEE binary32; OCP FP8 E4M3FN has 1 sign bit, 4
exponent bits (bias 7) and 3 mantissa bits, no infinities, and the all-ones
exponent+mantissa pattern as NaN (largest finite value 448).  Both decoders are
written from those definitions by bit manipulation; the e4m3 encoder picks the
nearest finite value from the decoded code table.
"""
import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP E4M3FN codes (uint8) -> float64, exactly.  NaN codes decode to NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.ldexp(1.0, (e - 7).astype(np.int64))
    subnormal = (m / 8.0) * np.ldexp(1.0, -6)
    v = np.where(e == 0, subnormal, normal) * sign
    return np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, v)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bits with a single round-to-nearest-even to 8 significant bits.

    Finite, normal-range inputs only (|x| in [2^-126, 2^128)) plus exact zeros,
    which is all the oracle rounds.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                       # x = m * 2^e, 0.5 <= |m| < 1
    r = np.rint(m * 256.0) / 256.0           # 8 significant bits, ties to even
    y = np.ldexp(r, e).astype(np.float32)    # exact: 8 bits fit in binary32
    return (y.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# the 127 non-negative finite e4m3 values, ascending with their codes 0x00..0x7E
_E4M3_POS = None


def f64_to_e4m3_codes(x: np.ndarray) -> np.ndarray:
    """float64 -> OCP E4M3FN codes: the nearest finite e4m3 value, ties to the even code
    (even mantissa), magnitudes above 448 saturated to 448.  -0.0 encodes as 0x80."""
    global _E4M3_POS
    if _E4M3_POS is None:
        _E4M3_POS = e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
    x = np.asarray(x, dtype=np.float64)
    assert np.isfinite(x).all()
    a = np.minimum(np.abs(x), _E4M3_POS[-1])
    hi = np.clip(np.searchsorted(_E4M3_POS, a, side="left"), 0, 0x7E)   # first value >= a
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - _E4M3_POS[lo], _E4M3_POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(x), code | np.uint8(0x80), code).astype(np.uint8)


# ----------------------------------------------------------------------------- MXFP4
# OCP Microscaling (MX) v1.0: an MXFP4 block is 32 FP4 E2M1 elements sharing one E8M0
# scale.  E2M1 has 1 sign bit, 2 exponent bits (bias 1) and 1 mantissa bit, no
# infinities or NaN; its magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6.  E8M0 is an unsigned
# power of two 2^(c - 127), with code 0xFF as NaN.  Packing (a reading; the format fixes
# the element encoding, not the byte layout): element 2i sits in the low nibble of byte i
# and element 2i+1 in the high nibble.

MX_BLOCK = 32


def e2m1_to_f64(codes: np.ndarray) -> np.ndarray:
    """FP4 E2M1 codes (the low 4 bits of each uint8) -> float64, exactly."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64) & 0xF
    sign = np.where((c >> 3) & 1, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = (c & 0x1).astype(np.float64)
    normal = (1.0 + m / 2.0) * np.ldexp(1.0, (e - 1).astype(np.int64))
    subnormal = m / 2.0                       # m * 2^(1 - bias) * 2^-1
    return np.where(e == 0, subnormal, normal) * sign


def e8m0_to_f64(codes: np.ndarray) -> np.ndarray:
    """E8M0 scale codes (uint8) -> float64 2^(c - 127); 0xFF decodes to NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    return np.where(c == 0xFF, np.nan, np.ldexp(1.0, c - 127))


def unpack_fp4(packed: np.ndarray) -> np.ndarray:
    """[..., n] bytes -> [..., 2n] E2M1 codes, element 2i from the low nibble of byte i."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def mxfp4_to_f64(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP4 rows -> float64 [..., D]: packed [..., D/2] bytes, scales [..., D/32] E8M0.

    Element d is e2m1(code d) * 2^(scale[d // 32] - 127), exact in float64.
    """
    vals = e2m1_to_f64(unpack_fp4(packed))
    s = e8m0_to_f64(scales)
    assert vals.shape[-1] == MX_BLOCK * s.shape[-1], (vals.shape, s.shape)
    return vals * np.repeat(s, MX_BLOCK, axis=-1)

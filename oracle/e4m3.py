"""OCP 8-bit floating point E4M3 ("E4M3FN") codec, written from the format
definition in the OCP 8-bit Floating Point Specification (OFP8), rev. 1.0:
1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0
encodes subnormals m/8 * 2^-6; S.1111.111 is NaN; there are no infinities, so
the largest finite magnitude is 1.75 * 2^8 = 448.  Conversion rounds to the
nearest representable value, ties to the even mantissa, and saturates to +-448
(the "saturating" conversion mode of the specification).

Used by the oracle's low-precision tier: the low tier of the method runs a tile
in reduced precision (HierPAS: progressively reduced precision; APT:
dual-precision execution; the kernel's fp8 MFMA consumes exactly these codes).
TEST INFRASTRUCTURE ONLY.
"""
import numpy as np

MAX = 448.0
NAN_CODE = 0x7F


def _decode_scalar(c: int) -> float:
    s = -1.0 if c & 0x80 else 1.0
    e = (c >> 3) & 0xF
    m = c & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


DECODE = np.array([_decode_scalar(c) for c in range(256)], dtype=np.float64)
# non-negative finite codes 0x00..0x7E in increasing value order
_POS = DECODE[:0x7F].copy()


def decode(codes: np.ndarray) -> np.ndarray:
    """uint8 codes -> float64 values."""
    return DECODE[np.asarray(codes, dtype=np.uint8)]


def encode(x) -> np.ndarray:
    """Round float values (taken exactly as given, e.g. float32) to E4M3 codes:
    nearest, ties to even mantissa, saturating to +-448; NaN -> 0x7F.
    The sign bit is kept for values that round to zero (-tiny -> 0x80)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    hi = np.searchsorted(_POS, a, side="left")           # first code with value >= a
    hi = np.clip(hi, 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    dlo = a - _POS[lo]
    dhi = _POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0) & (hi != lo))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= MAX, 0x7E, code)
    out = code.astype(np.uint8)
    out = np.where(np.signbit(x), out | 0x80, out).astype(np.uint8)
    out = np.where(np.isnan(x), NAN_CODE, out).astype(np.uint8)
    return out

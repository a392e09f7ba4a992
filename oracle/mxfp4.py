"""OCP MXFP4 codec, written from the OCP Microscaling Formats (MX)
Specification v1.0: a block of 32 elements shares one E8M0 scale X = 2^e
(8-bit biased exponent, bias 127, no mantissa); each element is FP4 E2M1:
1 sign bit, 2 exponent bits with bias 1, 1 mantissa bit, so the magnitudes are
0, 0.5 (the one subnormal), 1, 1.5, 2, 3, 4, 6 and there is no infinity or NaN.
The shared exponent of a block is floor(log2(max |x|)) - 2, 2 being the
exponent of E2M1's largest normal (6 = 1.5 * 2^2); elements are x / X rounded
to the nearest E2M1 value, ties to the even mantissa, magnitudes beyond 6
clamped to 6.

Used by the oracle's skim tier: Triage's skim tier runs a tile in a 4-bit
microscaled format ("Triage" abstract: skimming a tile in 4-bit floating
point); MXFP4 is the 4-bit block-scaled format the gfx950 matrix cores take.
TEST INFRASTRUCTURE ONLY.
"""
import numpy as np

BLOCK = 32
E_MIN, E_MAX = -127, 127          # E8M0 exponent range (byte 0xFF is NaN, never produced)
EMAX_ELEM = 2                     # exponent of E2M1's largest normal
# magnitude of code c (c = 2 * exponent field + mantissa bit), c = 0..7
GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def decode(codes: np.ndarray) -> np.ndarray:
    """4-bit codes (0..15, bit 3 the sign) -> float64 values."""
    c = np.asarray(codes, dtype=np.int64)
    v = GRID[c & 7]
    return np.where(c & 8, -v, v)


def encode(y) -> np.ndarray:
    """Round values (taken exactly as given) to E2M1 codes: the nearest grid
    magnitude, ties to the even code (the even mantissa), magnitudes >= 6
    clamped to 6.  The sign bit is set for every negative input, also where
    the magnitude rounds to zero."""
    y = np.asarray(y, dtype=np.float64)
    a = np.minimum(np.abs(y), GRID[-1])
    dist = np.abs(a[..., None] - GRID)                       # [..., 8]
    best = dist.min(axis=-1, keepdims=True)
    tied = dist == best
    # among the nearest grid points prefer an even code (at most two are tied,
    # and two neighbouring codes differ in their last bit)
    even_pick = np.where(tied & (np.arange(8) % 2 == 0), 1, 0)
    code = np.where(even_pick.any(axis=-1), even_pick.argmax(axis=-1), tied.argmax(axis=-1))
    return (code | np.where(y < 0, 8, 0)).astype(np.uint8)


def block_exponents(x: np.ndarray) -> np.ndarray:
    """Shared exponent e of every block of 32 consecutive elements along the
    last axis of x (whose length is a multiple of 32): floor(log2(amax)) - 2,
    clamped to the E8M0 range; -127 for an all-zero block."""
    x = np.asarray(x, dtype=np.float64)
    blocks = x.reshape(*x.shape[:-1], x.shape[-1] // BLOCK, BLOCK)
    amax = np.abs(blocks).max(axis=-1)
    _, ex = np.frexp(amax)                                   # amax = f * 2^ex, f in [0.5, 1)
    e = np.where(amax > 0, ex.astype(np.int64) - 1 - EMAX_ELEM, E_MIN)
    return np.clip(e, E_MIN, E_MAX)


def quantise(x: np.ndarray):
    """MXFP4 quantisation of x along its last axis.  Returns (codes uint8 of
    the same shape, one 4-bit code per element; scale bytes uint8 [..., d/32],
    the E8M0 encoding e + 127; dequantised values float64, code value * 2^e)."""
    x = np.asarray(x, dtype=np.float64)
    e = block_exponents(x)
    ee = np.repeat(e, BLOCK, axis=-1)
    codes = encode(np.ldexp(x, -ee))
    deq = np.ldexp(decode(codes), ee)
    return codes, (e + 127).astype(np.uint8), deq


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Two codes per byte along the last axis: element 2m in the low nibble of
    byte m, element 2m + 1 in the high nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)

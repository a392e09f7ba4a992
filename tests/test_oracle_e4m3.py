"""Pins of the oracle's E4M3 codec against the OCP OFP8 format definition (P6)."""
import os
import struct

import numpy as np
import pytest

from oracle import e4m3

GOLD = os.path.join(os.path.dirname(__file__), "golden", "e4m3_ocp_values.txt")


def _bitwise_rne_e4m3(x: float) -> int:
    """Independent encoder working on the float32 bit pattern (integer rounding),
    written from the format definition: bias 7, 3 mantissa bits, subnormals below 2^-6,
    saturate at 448, NaN -> 0x7F."""
    (u,) = struct.unpack("<I", struct.pack("<f", x))
    sign = 0x80 if u >> 31 else 0
    exp = (u >> 23) & 0xFF
    man = u & 0x7FFFFF
    if exp == 0xFF:
        return 0x7F if man else sign | 0x7E
    if exp == 0:
        return sign  # float32 subnormals are far below 2^-10 -> zero
    e = exp - 127
    full = man | 0x800000                     # 24-bit significand, value = full * 2^(e-23)
    if e >= -6:
        shift = 20                            # keep 3 mantissa bits
        q = full >> shift
        rem = full & ((1 << shift) - 1)
        half = 1 << (shift - 1)
        if rem > half or (rem == half and (q & 1)):
            q += 1
        ee = e
        if q == 16:                           # mantissa overflow -> next binade
            q = 8
            ee += 1
        code_e = ee + 7
        if code_e > 15 or (code_e == 15 and (q - 8) == 7):
            return sign | 0x7E
        return sign | (code_e << 3) | (q - 8)
    # subnormal target: value = m * 2^-9, m = full * 2^(e-23+9)
    shift = 23 - 9 - e                        # >= 21
    if shift > 40:
        return sign
    q = full >> shift
    rem = full & ((1 << shift) - 1)
    half = 1 << (shift - 1)
    if rem > half or (rem == half and (q & 1)):
        q += 1
    if q == 8:
        return sign | 0x08                    # rounds up to the min normal
    return sign | q


def test_golden_values_from_spec():
    for line in open(GOLD):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        code, val = line.split()
        got = e4m3.decode(np.array([int(code, 16)], dtype=np.uint8))[0]
        if val == "nan":
            assert np.isnan(got)
        else:
            assert got == float(val), (code, got, val)
            if val == "-0":
                assert np.signbit(got)


def test_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = e4m3.decode(codes)
    assert np.all(e4m3.encode(vals.astype(np.float32)) == codes)


def test_monotone_and_count():
    pos = e4m3.decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)
    assert pos[-1] == 448.0 and pos[1] == 2.0 ** -9


def test_midpoints_round_to_even():
    pos = e4m3.decode(np.arange(0x7F, dtype=np.uint8))
    for c in range(0x7E):
        mid = np.float32(0.5 * (pos[c] + pos[c + 1]))
        assert float(mid) == 0.5 * (pos[c] + pos[c + 1])   # exactly representable in fp32
        want = c if c % 2 == 0 else c + 1
        assert e4m3.encode(mid) == want
        assert e4m3.encode(-mid) == (want | 0x80)
        assert e4m3.encode(np.nextafter(mid, np.float32(0))) == c
        assert e4m3.encode(np.nextafter(mid, np.float32(1e9))) == c + 1


def test_saturation_nan_and_zero():
    assert e4m3.encode(np.float32(448.0)) == 0x7E
    assert e4m3.encode(np.float32(463.99)) == 0x7E
    assert e4m3.encode(np.float32(1e30)) == 0x7E
    assert e4m3.encode(np.float32(-1e30)) == 0xFE
    assert e4m3.encode(np.float32(np.nan)) == 0x7F
    assert e4m3.encode(np.float32(0.0)) == 0x00
    assert e4m3.encode(np.float32(-0.0)) == 0x80
    assert e4m3.encode(np.float32(2.0 ** -10)) == 0x00        # tie between 0 and 2^-9 -> even (0)
    assert e4m3.encode(np.float32(2.0 ** -10 * 1.0001)) == 0x01


def test_against_independent_bitwise_encoder():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(40000).astype(np.float32) * 50,
        (rng.standard_normal(20000) * 1e-2).astype(np.float32),
        rng.uniform(-480, 480, 20000).astype(np.float32),
        (2.0 ** rng.uniform(-12, 9, 20000) * rng.choice([-1, 1], 20000)).astype(np.float32),
    ])
    got = e4m3.encode(x)
    ref = np.array([_bitwise_rne_e4m3(float(v)) for v in x], dtype=np.uint8)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(ref[i])) for i in bad[:5]]

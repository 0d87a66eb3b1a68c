"""Pins of the oracle's E4M3 codec against the OCP 8-bit FP definition.

The decoder is pinned by spot codes from the format definition and by
structural facts (count of distinct values, monotonicity); the encoder by an
exhaustive brute-force nearest-value search over every finite code, for every
one of the 65,536 bf16 bit patterns.
"""

import numpy as np
import pytest

from oracle import e4m3_decode, e4m3_encode, bf16_bits_to_f64

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def test_spot_codes():
    spots = {0x00: 0.0, 0x38: 1.0, 0x40: 2.0, 0x7E: 448.0, 0x08: 2.0 ** -6,
             0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x77: 240.0, 0x3C: 1.5,
             0xB8: -1.0, 0xC4: -3.0, 0x78: 256.0, 0x4A: 5.0}
    for c, v in spots.items():
        assert e4m3_decode(np.uint8(c)) == v, hex(c)
    assert np.isnan(e4m3_decode(np.uint8(0x7F)))
    assert np.isnan(e4m3_decode(np.uint8(0xFF)))
    z = e4m3_decode(np.uint8(0x80))
    assert z == 0.0 and np.signbit(z)


def test_all_codes_structure():
    v = e4m3_decode(np.arange(256, dtype=np.uint8))
    finite = v[np.isfinite(v)]
    assert finite.size == 254
    assert np.unique(finite).size == 253  # +0 and -0 are one value
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)  # codes 0x00..0x7E increase strictly
    assert pos.max() == 448.0
    assert np.array_equal(v[0x80:0xFF], -v[:0x7F])


def test_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(e4m3_encode(e4m3_decode(codes)), codes)


def _brute_force_encode(x):
    """Nearest finite code with the sign of x; ties -> even mantissa; clamp."""
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    vals = e4m3_decode(codes.astype(np.uint8))
    out = np.empty(x.shape, dtype=np.uint8)
    for i, xi in enumerate(x):
        neg = np.signbit(xi)
        sel = codes[(codes >> 7) == (1 if neg else 0)]
        sv = vals[(codes >> 7) == (1 if neg else 0)]
        xc = min(max(xi, -448.0), 448.0)
        d = np.abs(sv - xc)
        best = np.flatnonzero(d == d.min())
        if best.size > 1:
            best = best[(sel[best] & 1) == 0]
        assert best.size == 1
        out[i] = sel[best[0]]
    return out


def test_encode_matches_brute_force_all_bf16():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = bf16_bits_to_f64(bits)
    x = x[np.isfinite(x)]
    got = e4m3_encode(x)
    # brute force in chunks through a value->code cache (many bf16 share a code)
    want = _brute_force_encode(x)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, (x[bad[:5]], got[bad[:5]], want[bad[:5]])


def test_encode_ties_to_even():
    # 1 + 1/16 lies halfway between 1.0 (M=0) and 1.125 (M=1): goes to M=0
    assert e4m3_encode(np.array([1.0625]))[0] == 0x38
    # 1.1875 halfway between 1.125 (M=1) and 1.25 (M=2): goes to M=2
    assert e4m3_encode(np.array([1.1875]))[0] == 0x3A
    # subnormal tie: 1.5 * 2^-9 between M=1 and M=2 -> M=2
    assert e4m3_encode(np.array([1.5 * 2.0 ** -9]))[0] == 0x02
    # half of the smallest subnormal rounds to (signed) zero
    assert e4m3_encode(np.array([2.0 ** -10]))[0] == 0x00
    assert e4m3_encode(np.array([-(2.0 ** -10)]))[0] == 0x80
    # saturation
    assert e4m3_encode(np.array([1e6]))[0] == 0x7E
    assert e4m3_encode(np.array([-1e6]))[0] == 0xFE
    # 464 is halfway between 448 and the unrepresentable 480: stays 448
    assert e4m3_encode(np.array([464.0]))[0] == 0x7E

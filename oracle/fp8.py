"""FP8 E4M3 codec and bf16 decoding, float64, for the oracle (test infrastructure only).

The pages ask for low-precision scoring inputs ([P5] "Index Selection Path",
first bullet) and name FP8 as the low-precision compute format ([P1] section 5;
[P4] "Breaking Down the Model Architecture", item 2) without fixing the FP8
variant.  The oracle uses the E4M3 variant of the OCP 8-bit floating point
specification (OFP8, 2023): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
bits, no infinities, a single NaN mantissa pattern (S.1111.111), largest
finite magnitude 448, subnormal spacing 2**-9.
"""

import numpy as np

E4M3_MAX = 448.0
E4M3_SUBNORMAL_STEP = 2.0 ** -9
E4M3_MIN_NORMAL = 2.0 ** -6


def e4m3_decode(codes):
    """Value (float64) of each E4M3 code (uint8 array).

    sign = bit 7, E = bits 6..3, M = bits 2..0;
    E == 0: (-1)^sign * M * 2^-9 (subnormal, including +-0);
    E == 15 and M == 7: NaN;
    otherwise: (-1)^sign * (1 + M/8) * 2^(E-7).
    """
    c = np.asarray(codes).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(
        e == 0,
        m * E4M3_SUBNORMAL_STEP,
        (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)),
    )
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def e4m3_encode(x):
    """E4M3 code (uint8) of each finite float64 in ``x``.

    Round to nearest; a value exactly halfway between two representable
    magnitudes goes to the one with an even mantissa field (code bit 0 clear).
    Magnitudes above 448 saturate to 448.  The sign bit is copied from ``x``
    (so -0.0, and negative values that round to zero, give code 0x80).
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("e4m3_encode: inputs must be finite")
    neg = np.signbit(x)
    a = np.minimum(np.abs(x), E4M3_MAX)
    # spacing of the grid that ``a`` falls in: 2^-9 below the smallest normal,
    # otherwise 2^(floor(log2 a) - 3) (three mantissa bits).
    _, ex = np.frexp(a)  # a = f * 2^ex with f in [0.5, 1); floor(log2 a) = ex - 1
    step = np.where(a < E4M3_MIN_NORMAL, E4M3_SUBNORMAL_STEP,
                    np.exp2((ex - 1 - 3).astype(np.float64)))
    n = np.rint(a / step)  # a/step is exact (power-of-two step); rint: ties to even
    v = np.minimum(n * step, E4M3_MAX)
    # code of the rounded magnitude v
    sub = v < E4M3_MIN_NORMAL
    _, ev = np.frexp(np.where(sub, 1.0, v))
    exp_field = np.where(sub, 0, ev - 1 + 7)
    mant_field = np.where(
        sub,
        np.rint(v / E4M3_SUBNORMAL_STEP),
        np.rint(v / np.exp2((ev - 1).astype(np.float64)) * 8.0) - 8.0,
    ).astype(np.int64)
    code = (exp_field.astype(np.int64) << 3) | mant_field
    code = code | np.where(neg, 0x80, 0)
    return code.astype(np.uint8)


def bf16_bits_to_f64(bits):
    """Value (float64) of bfloat16 numbers given as their uint16 bit patterns."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)

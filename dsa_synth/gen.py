"""Seeded, counter-based synthetic inputs (host side).

This module only makes input data.  It holds none of the method's arithmetic
(no scoring, selection or attention), and it is the one piece of code that
both the HIP path (through ``bench.py``/tests) and the oracle consume.

Every random number is a pure function of (seed, tag, element index), so any
element of any tensor can be regenerated on demand -- on the host here, or on
the device by ``fill.hip`` which implements the same definition:

  h(seed, tag, i) = mix64(base + (i + 1) * 0x9E3779B97F4A7C15)
  base           = mix64((seed << 8) | tag)
  mix64(z)       : z ^= z >> 30; z *= 0xBF58476D1CE4E5B9;
                   z ^= z >> 27; z *= 0x94D049BB133111EB; z ^= z >> 31
(the SplitMix64 output function of Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014), all arithmetic mod 2^64.

Normal variates come from a 65,536-entry table of standard-normal quantiles,
T[i] = Phi^-1((i + 0.5) / 65536) (scipy's ndtri), indexed by 16 bits of a hash.
Element e of a "bf16 normal" tensor uses 16-bit lane (e & 3) of h(seed, tag,
e >> 2) as the table index and the bf16 rounding (nearest-even) of T as value.
Uniform variates: U = ((h >> 40) + 0.5) * 2^-24.
"""

import numpy as np
from scipy.special import ndtri

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
MUL1 = np.uint64(0xBF58476D1CE4E5B9)
MUL2 = np.uint64(0x94D049BB133111EB)

TAG_Q = 1
TAG_K = 2
TAG_V = 3
TAG_QIDX = 4
TAG_IDXKEY = 5
TAG_W = 6
TAG_TABLE = 7
TAG_LENS = 8
TAG_PLANT = 9


def mix64(z):
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * MUL1
        z = (z ^ (z >> np.uint64(27))) * MUL2
    return z ^ (z >> np.uint64(31))


def stream_base(seed, tag):
    return mix64(np.array([(int(seed) << 8) | int(tag)], dtype=np.uint64))[0]


def hash_at(seed, tag, idx):
    """64-bit hash of element counters ``idx`` (uint64 array) of stream (seed, tag)."""
    base = stream_base(seed, tag)
    idx = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return mix64(base + (idx + np.uint64(1)) * GOLDEN)


_TABLES = {}


def normal_table_f64():
    if "f64" not in _TABLES:
        i = np.arange(65536, dtype=np.float64)
        _TABLES["f64"] = ndtri((i + 0.5) / 65536.0)
    return _TABLES["f64"]


def f32_to_bf16_bits(x):
    """bf16 bit pattern (uint16) of float32 values, round to nearest even."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits):
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def normal_table_bf16():
    """uint16 [65536]: bf16 bits of the normal quantile table (uploaded to the device filler)."""
    if "bf16" not in _TABLES:
        _TABLES["bf16"] = f32_to_bf16_bits(normal_table_f64().astype(np.float32))
    return _TABLES["bf16"]


def normal_table_f32():
    if "f32" not in _TABLES:
        _TABLES["f32"] = normal_table_f64().astype(np.float32)
    return _TABLES["f32"]


def _lane_index(seed, tag, elems):
    elems = np.asarray(elems, dtype=np.uint64)
    h = hash_at(seed, tag, elems >> np.uint64(2))
    lane = (elems & np.uint64(3)) * np.uint64(16)
    return ((h >> lane) & np.uint64(0xFFFF)).astype(np.int64)


def _range_index(seed, tag, offset, n):
    """Table indices of the contiguous elements [offset, offset + n)."""
    g0 = offset // 4
    g1 = (offset + n + 3) // 4
    h = hash_at(seed, tag, np.arange(g0, g1, dtype=np.uint64))
    lanes = h.view(np.uint16)  # little endian: lane k = bits 16k..16k+15
    start = offset - 4 * g0
    return lanes[start: start + n]


def bf16_normal_bits(seed, tag, elems):
    """bf16 bits of standard-normal elements at flat indices ``elems``."""
    return normal_table_bf16()[_lane_index(seed, tag, elems)]


def bf16_normal_tensor(seed, tag, shape, offset=0):
    n = int(np.prod(shape))
    return normal_table_bf16()[_range_index(seed, tag, int(offset), n)].reshape(shape)


def f32_normal_tensor(seed, tag, shape, offset=0):
    n = int(np.prod(shape))
    return normal_table_f32()[_range_index(seed, tag, int(offset), n)].reshape(shape)


def uniform_tensor(seed, tag, shape, offset=0):
    """float64 uniform in (0, 1), one hash per element."""
    n = int(np.prod(shape))
    h = hash_at(seed, tag, np.arange(offset, offset + n, dtype=np.uint64))
    return (((h >> np.uint64(40)).astype(np.float64) + 0.5) * 2.0 ** -24).reshape(shape)


def permutation(seed, tag, n):
    """A seeded permutation of range(n): argsort of n hashes (stable)."""
    h = hash_at(seed, tag, np.arange(n, dtype=np.uint64))
    return np.argsort(h, kind="stable").astype(np.int64)

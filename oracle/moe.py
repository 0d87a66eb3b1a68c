"""MXFP4 expert weights and the grouped FP8 expert GEMM, for the oracle
(test infrastructure only).

What the pages fix:
  * expert weights are stored in MXFP4: fixed blocks of 4-bit floating-point
    elements sharing one block-level scale ([P1] "Day-0 Adaptation for Massive
    LLMs...", sections 2 and 5; [P5] "Day-0 Readiness...", "MXFP4 Expert
    Weights");
  * the weights of the experts a batch is routed to are unpacked to FP8
    online into a reused FP8 workspace, and the expert matmuls run in FP8 on
    that workspace with the block scales ([P1] section 5(2) and its
    schematic; [P2] "Day-0 Adaptation for Trillion-Parameter LLMs...",
    sections 3.1-3.2; [P3] "Day-0 Adaptation for Trillion-Parameter
    Models...", section 5);
  * the unpacked layout must be the matmul's input layout, and the block
    scales must be matched to the FP8 range ([P1] section 5(3)).

Formats: the OCP Microscaling Formats (MX) specification v1.0 (2023), which
"MXFP4" names:
  * E2M1 element: sign bit 3, exponent bits 2-1 (bias 1), mantissa bit 0;
    exponent 0 is subnormal: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6;
  * E8M0 scale: value 2^(s - 127), s = 255 is NaN;
  * a block is 32 consecutive elements sharing one scale;
  * MXFP8 with E4M3 elements (emax 8): shared exponent floor(log2 max|x|) - 8,
    elements E4M3(x / 2^shared), saturating at +-448.

Readings (the pages are silent here):
  * W_e is [N, K] (outputs x inputs) and is blocked along K; two E2M1 codes
    per byte, element 2i in bits 3-0 and element 2i + 1 in bits 7-4;
  * the FP8 workspace holds the E4M3 code of every E2M1 element (exact: each
    E2M1 value is an E4M3 value) and the E8M0 scales unchanged, so no scale is
    folded into the FP8 elements and nothing can overflow the FP8 range;
  * activations reach the FP8 matmul as MXFP8 (E4M3 elements, one E8M0 scale
    per 32 along K), computed from bf16 by the rule above; a block of zeros
    gets scale code 0;
  * the grouped matmul computes, for every routed (token t, slot j) with
    expert e = route[t, j] >= 0, out[t, j, :] = xq[t, :] . W_e^T (dequantized
    operands, float64 here); slots with route -1 are zero.  Gating and the
    combine over slots belong to the caller.
"""

import numpy as np

from .fp8 import e4m3_decode, e4m3_encode, E4M3_MAX

MX_BLOCK = 32
E4M3_EMAX = 8


def e2m1_decode(codes):
    """Value (float64) of each E2M1 code (integers 0..15)."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where((c >> 3) & 1, -1.0, 1.0)
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, (1.0 + 0.5 * m) * np.exp2((e - 1).astype(np.float64)))
    return sign * mag


def e8m0_decode(s):
    """Value (float64) of each E8M0 scale code: 2^(s - 127), NaN for 255."""
    s = np.asarray(s).astype(np.int64)
    return np.where(s == 255, np.nan, np.exp2((s - 127).astype(np.float64)))


def unpack_fp4(packed, k):
    """E2M1 codes [..., k] from packed bytes [..., k / 2] (element 2i in the low nibble)."""
    p = np.asarray(packed).astype(np.uint8)
    codes = np.empty(p.shape[:-1] + (k,), dtype=np.uint8)
    codes[..., 0::2] = p & 0x0F
    codes[..., 1::2] = p >> 4
    return codes


def mxfp4_dequant(packed, scales):
    """Values (float64) [..., K] of MXFP4 data: packed codes [..., K/2], E8M0 scales [..., K/32]."""
    s = np.asarray(scales)
    k = s.shape[-1] * MX_BLOCK
    v = e2m1_decode(unpack_fp4(packed, k))
    return v * np.repeat(e8m0_decode(s), MX_BLOCK, axis=-1)


def mxfp4_to_fp8(packed, scales):
    """The FP8 workspace form of MXFP4 data: (E4M3 codes [..., K], E8M0 scales [..., K/32]).
    Each E4M3 code has the value of its E2M1 element; the scales are unchanged."""
    s = np.asarray(scales).astype(np.uint8)
    codes = unpack_fp4(packed, s.shape[-1] * MX_BLOCK)
    return e4m3_encode(e2m1_decode(codes)), s.copy()


def mx_quantize_e4m3(x):
    """MXFP8 (E4M3 elements) of x [..., K] (K a multiple of 32): (codes uint8 [..., K],
    E8M0 scale codes uint8 [..., K/32]).  Per block: amax = max |x|; shared exponent
    floor(log2 amax) - 8 (clamped to [-127, 127]; scale code 0 for an all-zero
    block); elements E4M3(x / 2^shared), round to nearest even, saturating at 448."""
    x = np.asarray(x, dtype=np.float64)
    k = x.shape[-1]
    if k % MX_BLOCK:
        raise ValueError("mx_quantize_e4m3: K must be a multiple of 32")
    blocks = x.reshape(x.shape[:-1] + (k // MX_BLOCK, MX_BLOCK))
    amax = np.max(np.abs(blocks), axis=-1)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))      # amax = f 2^ex, f in [0.5, 1)
    shared = np.clip(ex - 1 - E4M3_EMAX, -127, 127)      # floor(log2 amax) - emax
    s = np.where(amax > 0, shared + 127, 0).astype(np.int64)
    y = blocks / np.exp2((s - 127).astype(np.float64))[..., None]   # exact: power of two
    codes = e4m3_encode(np.clip(y, -E4M3_MAX, E4M3_MAX))
    return codes.reshape(x.shape), s.astype(np.uint8)


def mx_dequant_e4m3(codes, scales):
    """Values (float64) of MXFP8 data (E4M3 codes [..., K], E8M0 scales [..., K/32])."""
    v = e4m3_decode(codes)
    return v * np.repeat(e8m0_decode(scales), MX_BLOCK, axis=-1)


def grouped_gemm(x_codes, x_scales, w_packed, w_scales, route):
    """out[t, j, n] = sum_k xq[t, k] * W[route[t, j], n, k] (float64), zero where
    route[t, j] < 0.  x: MXFP8 [T, K] (codes, scales); W: MXFP4 [E, N, K/2] packed
    codes and [E, N, K/32] scales; route: int [T, slots]."""
    xq = mx_dequant_e4m3(x_codes, x_scales)
    route = np.asarray(route)
    t_n, slots = route.shape
    n = np.asarray(w_scales).shape[1]
    out = np.zeros((t_n, slots, n), dtype=np.float64)
    for e in np.unique(route[route >= 0]):
        w = mxfp4_dequant(w_packed[e], w_scales[e])       # [N, K]
        tt, jj = np.nonzero(route == e)
        out[tt, jj] = xq[tt] @ w.T
    return out


def grouped_gemm_abs(x_codes, x_scales, w_packed, w_scales, route):
    """sum_k |xq[t, k] * W[e, n, k]|: the scale of each output's rounding error."""
    xq = np.abs(mx_dequant_e4m3(x_codes, x_scales))
    route = np.asarray(route)
    t_n, slots = route.shape
    n = np.asarray(w_scales).shape[1]
    out = np.zeros((t_n, slots, n), dtype=np.float64)
    for e in np.unique(route[route >= 0]):
        w = np.abs(mxfp4_dequant(w_packed[e], w_scales[e]))
        tt, jj = np.nonzero(route == e)
        out[tt, jj] = xq[tt] @ w.T
    return out

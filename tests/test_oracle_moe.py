"""Pins of the MXFP4 / MXFP8 oracle (oracle/moe.py).

E2M1: the value table of the MX specification (tests/golden/mx_formats.json).
E8M0: PyTorch's float8_e8m0fnu decoding, an independent decoder, for every
code.  E2M1 -> E4M3 and the MXFP8 elements: PyTorch's float8_e4m3fn encoder on
the same values.  MXFP8 scales: hand-worked blocks, the spec's range property
(the block maximum lands in [256, 448] after scaling), saturation, zero
blocks.  Grouped matmul: a scalar brute force that reads the nibbles and scales
itself, on tiny inputs, plus exact scaling and routing invariants."""

import json
import os

import numpy as np
import pytest

from oracle import e4m3_decode
from oracle.moe import (e2m1_decode, e8m0_decode, unpack_fp4, mxfp4_dequant, mxfp4_to_fp8,
                        mx_quantize_e4m3, mx_dequant_e4m3, grouped_gemm, grouped_gemm_abs)

torch = pytest.importorskip("torch")
GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "mx_formats.json")))


def test_e2m1_matches_the_spec_table():
    v = e2m1_decode(np.arange(16))
    want = np.array(GOLD["e2m1_values_by_code"])
    assert np.array_equal(v, want)
    assert np.array_equal(np.signbit(v), np.signbit(want))  # code 8 is -0


def test_e8m0_matches_torch_decoder():
    codes = np.arange(255, dtype=np.uint8)
    t = torch.from_numpy(codes.copy()).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(e8m0_decode(codes), t)
    assert np.isnan(e8m0_decode(np.array([GOLD["e8m0_nan_code"]])))[0]
    assert e8m0_decode(np.array([GOLD["e8m0_bias"]]))[0] == 1.0


def test_fp4_packing_low_nibble_first():
    packed = np.array([[0x21, 0xF8, 0x07]], dtype=np.uint8)
    assert unpack_fp4(packed, 6).tolist() == [[1, 2, 8, 15, 7, 0]]


def test_fp8_workspace_is_exact_and_matches_torch_encoder():
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 256, size=(5, 64), dtype=np.uint8)  # 128 E2M1 elements per row
    scales = rng.integers(100, 150, size=(5, 4), dtype=np.uint8)
    e4, s = mxfp4_to_fp8(codes, scales)
    assert np.array_equal(s, scales)
    vals = e2m1_decode(unpack_fp4(codes, 128))
    assert np.array_equal(e4m3_decode(e4), vals)                      # exact
    t = torch.from_numpy(vals.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4, t)
    # the workspace form dequantizes to the MXFP4 values
    assert np.array_equal(np.repeat(e8m0_decode(s), 32, -1) * e4m3_decode(e4),
                          mxfp4_dequant(codes, scales))


def test_mxfp8_hand_example():
    x = np.zeros(32)
    x[:4] = [3.0, 1.0, -0.5, 0.1]
    codes, s = mx_quantize_e4m3(x)
    # amax 3: floor(log2 3) = 1, shared exponent 1 - 8 = -7, scale code 120
    assert s.tolist() == [120]
    # elements x * 2^7: 384 = 1.5 * 2^8, 128 = 2^7, -64 = -2^6, 12.8 -> 13 (spacing 1 in [8, 16))
    assert e4m3_decode(codes[:4]).tolist() == [384.0, 128.0, -64.0, 13.0]
    assert not codes[4:].any()


def test_mxfp8_matches_torch_encoder_and_range():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((40, 256)) * 10.0 ** rng.uniform(-4, 4, size=(40, 1))).astype(np.float32)
    x[3, :32] = 0.0                      # a zero block
    x[4, 32:64] = 448.0 * 2.0 ** -3      # amax exactly a power-of-two multiple of 448
    codes, s = mx_quantize_e4m3(x)
    assert s[3, 0] == 0 and not codes[3, :32].any()
    scale = np.repeat(e8m0_decode(s), 32, -1)
    y = np.clip(x / scale, -448, 448)
    t = torch.from_numpy(y.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    nz = np.repeat(s != 0, 32, -1)
    assert np.array_equal(codes[nz], t[nz])
    # block maxima scale into [256, 512), saturating at 448
    blocks = np.abs(x).reshape(40, 8, 32).max(-1)
    m = blocks > 0
    r = blocks[m] / e8m0_decode(s)[m]
    assert np.all((r >= 256) & (r < 512))
    dq = mx_dequant_e4m3(codes, s)
    bmax = np.abs(dq).reshape(40, 8, 32).max(-1)
    assert np.all(bmax[m] / e8m0_decode(s)[m] <= 448)


def _brute(x_codes, x_scales, w_packed, w_scales, route, k):
    """Scalar loops: nibbles, E2M1 table, scales read element by element.
    Returns (sum_k xv * w, sum_k |xv * w|) per (token, slot, column)."""
    table = GOLD["e2m1_values_by_code"]
    t_n, slots = route.shape
    n = w_scales.shape[1]
    out = np.zeros((t_n, slots, n))
    mag = np.zeros((t_n, slots, n))
    for t in range(t_n):
        for j in range(slots):
            e = int(route[t, j])
            if e < 0:
                continue
            for c in range(n):
                acc = 0.0
                acc_abs = 0.0
                for i in range(k):
                    byte = int(w_packed[e, c, i // 2])
                    nib = (byte >> 4) if i % 2 else (byte & 15)
                    w = table[nib] * 2.0 ** (int(w_scales[e, c, i // 32]) - 127)
                    xv = float(e4m3_decode(np.array([x_codes[t, i]]))[0]) * \
                        2.0 ** (int(x_scales[t, i // 32]) - 127)
                    acc += xv * w
                    acc_abs += abs(xv * w)
                out[t, j, c] = acc
                mag[t, j, c] = acc_abs
    return out, mag


def _moe_case(seed, t_n=3, slots=2, e_n=3, n=4, k=64):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((t_n, k))
    xc, xs = mx_quantize_e4m3(x)
    wp = rng.integers(0, 256, size=(e_n, n, k // 2), dtype=np.uint8)
    ws = rng.integers(118, 136, size=(e_n, n, k // 32), dtype=np.uint8)
    route = rng.integers(-1, e_n, size=(t_n, slots))
    return xc, xs, wp, ws, route


def test_grouped_gemm_brute_force():
    for seed in range(3):
        xc, xs, wp, ws, route = _moe_case(seed)
        got = grouped_gemm(xc, xs, wp, ws, route)
        want, _ = _brute(xc, xs, wp, ws, route, 64)
        assert np.allclose(got, want, rtol=1e-12, atol=1e-12)
        assert not got[route < 0].any()


def test_grouped_gemm_abs_brute_force():
    """The error scale of the matmul's parity bar, sum_k |xq w|, against the
    scalar loops: activation and weight block scales each enter it once."""
    for seed in range(3):
        xc, xs, wp, ws, route = _moe_case(seed)
        # activation blocks with different scales, so a dropped scale shows
        xs = xs.copy()
        xs[:, 1] = np.clip(xs[:, 1].astype(np.int64) + 3, 1, 254).astype(np.uint8)
        got = grouped_gemm_abs(xc, xs, wp, ws, route)
        _, want = _brute(xc, xs, wp, ws, route, 64)
        assert np.allclose(got, want, rtol=1e-12, atol=1e-300)
        assert not got[route < 0].any()


def test_grouped_gemm_invariants():
    xc, xs, wp, ws, route = _moe_case(7, t_n=5, slots=3, e_n=4, n=6, k=96)
    base = grouped_gemm(xc, xs, wp, ws, route)
    # doubling every scale of expert 2 doubles its outputs exactly, nothing else
    ws2 = ws.copy()
    ws2[2] += 1
    out2 = grouped_gemm(xc, xs, wp, ws2, route)
    assert np.array_equal(out2[route == 2], 2 * base[route == 2])
    assert np.array_equal(out2[route != 2], base[route != 2])
    # relabelling experts (weights and routes together) changes nothing
    perm = np.array([3, 0, 2, 1])
    inv = np.argsort(perm)
    r2 = np.where(route >= 0, inv[np.maximum(route, 0)], -1)
    assert np.array_equal(grouped_gemm(xc, xs, wp[perm], ws[perm], r2), base)
    # the absolute-value sum bounds the result
    assert np.all(np.abs(base) <= grouped_gemm_abs(xc, xs, wp, ws, route) * (1 + 1e-12))

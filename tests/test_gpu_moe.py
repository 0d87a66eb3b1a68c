"""GPU parity of the MXFP4 expert path (dsa_mx_quantize, dsa_mxfp4_to_fp8,
dsa_moe_grouped_gemm) against the oracle (oracle/moe.py).

Quantization and the FP8 unpack are bit-exact.  The matmul's products are
exact (E4M3 x E4M3 or E4M3 x E2M1, times powers of two) but the matrix unit
sums them with its own internal precision: measured within 1.4e-4 of
sum_k |xq w| on random operands, so the bar is |gpu - oracle| <= 2^-9 *
sum_k |xq[t, k] w[n, k]| per output (oracle.moe.grouped_gemm_abs)."""

import sys

import numpy as np
import pytest

from oracle.moe import (mx_quantize_e4m3, mxfp4_to_fp8, grouped_gemm, grouped_gemm_abs,
                        mxfp4_dequant, mx_dequant_e4m3)

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
TOL = 2.0 ** -9


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dynamic_sparse_attention_paged_amd as m
    m._lib.load()
    return m


def _bf16(rng, shape, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)   # truncate to bf16 bits


def _bf16_to_f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return (t.view(dtype) if dtype is not None else t).cuda()


def _experts(rng, e, n, k, lo=118, hi=131):
    return (rng.integers(0, 256, size=(e, n, k // 2), dtype=np.uint8),
            rng.integers(lo, hi, size=(e, n, k // 32), dtype=np.uint8))


def test_mx_quantize_bit_exact(dsa):
    rng = np.random.default_rng(31)
    rows, k = 70, 384
    x = _bf16(rng, (rows, k), 1.0)
    x[1] = _bf16(rng, (k,), 1e-38)                         # bf16 subnormals and tiny normals
    x[2] = _bf16(rng, (k,), 1e30)
    x[3, :32] = 0                                          # a zero block
    x[3, 32:64] = 0x8000                                   # a block of -0
    x[4] = (np.float32(448.0 * 4).view(np.uint32) >> 16)   # every element the block max
    x[5, :32] = _bf16(rng, (32,), 3.0)
    x[5, 0] = np.float32(-3.0).view(np.uint32) >> 16
    codes, scales = dsa.mx_quantize(_dev(x.view(np.int16), torch.bfloat16))
    torch.cuda.synchronize()
    want_c, want_s = mx_quantize_e4m3(_bf16_to_f32(x).astype(np.float64))
    got_c, got_s = codes.cpu().numpy(), scales.cpu().numpy()
    assert np.array_equal(got_s, want_s), np.argwhere(got_s != want_s)[:5]
    bad = np.argwhere(got_c != want_c)
    assert bad.size == 0, f"codes differ at {bad[:5].tolist()}: {got_c[tuple(bad[0])]:#x} vs " \
                          f"{want_c[tuple(bad[0])]:#x}"


def test_mxfp4_to_fp8_bit_exact(dsa):
    rng = np.random.default_rng(32)
    wp, ws = _experts(rng, 5, 48, 256)
    experts = np.array([3, 0, 4], np.int32)
    w = dsa.MxExperts(_dev(wp), _dev(ws))
    codes, scales = dsa.mxfp4_to_fp8(w, _dev(experts))
    torch.cuda.synchronize()
    want_c, want_s = mxfp4_to_fp8(wp[experts], ws[experts])
    assert np.array_equal(codes.cpu().numpy(), want_c)
    assert np.array_equal(scales.cpu().numpy(), want_s)


def _gemm_case(seed, e, n, k, t, slots, frac_unrouted=0.1, skew=None):
    rng = np.random.default_rng(seed)
    wp, ws = _experts(rng, e, n, k)
    x = _bf16(rng, (t, k))
    if skew is None:
        route = rng.integers(0, e, size=(t, slots)).astype(np.int32)
    else:  # most pairs on one expert (several row tiles), some experts never used
        route = np.where(rng.random((t, slots)) < skew, 0,
                         rng.integers(1, max(2, e // 2), size=(t, slots))).astype(np.int32)
    route[rng.random((t, slots)) < frac_unrouted] = -1
    return wp, ws, x, route


def _check_gemm(dsa, wp, ws, x, route, label):
    w = dsa.MxExperts(_dev(wp), _dev(ws))
    xc, xs = dsa.mx_quantize(_dev(x.view(np.int16), torch.bfloat16))
    rt = _dev(route)
    outs = {}
    for mode, name in ((dsa._lib.MOE_FP4_DIRECT, "fp4"), (dsa._lib.MOE_FP8_WORKSPACE, "fp8")):
        outs[name] = dsa.moe_grouped_gemm(w, xc, xs, rt, mode=mode)
    torch.cuda.synchronize()
    xc_h, xs_h = xc.cpu().numpy(), xs.cpu().numpy()
    ref = grouped_gemm(xc_h, xs_h, wp, ws, route)
    bound = TOL * grouped_gemm_abs(xc_h, xs_h, wp, ws, route)
    for name, o in outs.items():
        got = o.cpu().numpy().astype(np.float64)
        err = np.abs(got - ref)
        worst = (err / np.maximum(bound / TOL, 1e-300)).max()
        assert np.all(err <= bound), f"{label} {name}: error over the bar at " \
                                     f"{np.argwhere(err > bound)[:3].tolist()}"
        assert not got[route < 0].any()
        _say(f"{label} {name}: worst |err| / sum|xq w| = {worst:.2e}")
    return outs


@pytest.mark.parametrize("e,n,k,t,slots", [(6, 320, 384, 37, 3),    # ragged: n, pairs
                                           (4, 256, 256, 64, 2),
                                           (9, 64, 128, 5, 8),
                                           (4, 320, 512, 300, 2),   # 150 pairs per expert: 128-row tiles
                                           (4, 256, 2048, 400, 2),  # tall tiles, 16-step K: scale groups
                                           (6, 128, 1024, 40, 4),   # short tiles, K 1024: scale groups
                                           (8, 64, 128, 1500, 3),   # pairs over several grouping chunks
                                           (2100, 64, 128, 300, 2)])  # more experts than the LDS table
def test_grouped_gemm_matches_oracle(dsa, e, n, k, t, slots):
    wp, ws, x, route = _gemm_case(40 + e, e, n, k, t, slots)
    _check_gemm(dsa, wp, ws, x, route, f"E{e} N{n} K{k} T{t} S{slots}")


def test_grouped_gemm_skewed_routing_and_determinism(dsa):
    """One expert takes most pairs (several 32-pair row tiles), several take
    none; two runs agree bit for bit."""
    wp, ws, x, route = _gemm_case(50, 12, 192, 256, 90, 2, frac_unrouted=0.05, skew=0.6)
    outs = _check_gemm(dsa, wp, ws, x, route, "skewed")
    w = dsa.MxExperts(_dev(wp), _dev(ws))
    xc, xs = dsa.mx_quantize(_dev(x.view(np.int16), torch.bfloat16))
    again = dsa.moe_grouped_gemm(w, xc, xs, _dev(route))
    torch.cuda.synchronize()
    assert torch.equal(again, outs["fp4"])


def test_grouped_gemm_sampled_at_size(dsa):
    """E 16, N 1024, K 2048, 128 tokens x 4 slots: sampled columns against the
    oracle, computed for those columns only."""
    rng = np.random.default_rng(60)
    e, n, k, t, slots = 16, 1024, 2048, 128, 4
    wp, ws = _experts(rng, e, n, k)
    x = _bf16(rng, (t, k))
    route = rng.integers(0, e, size=(t, slots)).astype(np.int32)
    w = dsa.MxExperts(_dev(wp), _dev(ws))
    xc, xs = dsa.mx_quantize(_dev(x.view(np.int16), torch.bfloat16))
    out4 = dsa.moe_grouped_gemm(w, xc, xs, _dev(route), mode=dsa._lib.MOE_FP4_DIRECT)
    out8 = dsa.moe_grouped_gemm(w, xc, xs, _dev(route), mode=dsa._lib.MOE_FP8_WORKSPACE)
    torch.cuda.synchronize()
    xq = mx_dequant_e4m3(xc.cpu().numpy(), xs.cpu().numpy())
    cols = np.array([0, 1, 255, 256, 511, 700, 1023])
    for name, o in (("fp4", out4), ("fp8", out8)):
        got = o.cpu().numpy()
        for ex in range(e):
            wv = mxfp4_dequant(wp[ex, cols], ws[ex, cols])        # [cols, K]
            tt, jj = np.nonzero(route == ex)
            ref = xq[tt] @ wv.T
            bound = TOL * (np.abs(xq[tt]) @ np.abs(wv).T)
            assert np.all(np.abs(got[tt, jj][:, cols] - ref) <= bound), (name, ex)

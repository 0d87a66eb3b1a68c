"""Pins of the oracle's write path (oracle/write.py).

quantize_coarse_key: a hand example worked from the E4M3 definition, the zero
vector, PyTorch's own float8_e4m3fn conversion (an independent encoder) on
the scaled values, the largest entry landing on +-448, and the error bound of
round-to-nearest.  kv_write: tokens written through the block table read back
through it, and nothing else changes."""

import numpy as np
import pytest

from oracle import e4m3_decode
from oracle.write import kv_write, quantize_coarse_key

torch = pytest.importorskip("torch")


def test_hand_examples_coarse_key():
    # x = (1, -2, 0.5): max 2, ks = 2/448, y = (224, -448, 112)
    codes, ks = quantize_coarse_key([1.0, -2.0, 0.5])
    assert ks == np.float32(2.0 / 448.0)
    assert codes.tolist() == [0x76, 0xFE, 0x6E]  # 1.75*2^7, -1.75*2^8, 1.75*2^6
    # x = (448, 3, -0.25): ks = 1, y = x; 3 = 1.5*2^1 -> 0x44; -0.25 = -2^-2 -> 0xA8
    codes, ks = quantize_coarse_key([448.0, 3.0, -0.25])
    assert ks == np.float32(1.0) and codes.tolist() == [0x7E, 0x44, 0xA8]
    # ties to even with ks = 1 (spacing 2 in [16, 32)): 17 lies between 16
    # (0x58, mantissa 0) and 18 (0x59): even -> 16; 19 between 18 and 20
    # (0x5A, mantissa 2): even -> 20
    codes, _ = quantize_coarse_key([448.0, 17.0, 19.0])
    assert codes.tolist() == [0x7E, 0x58, 0x5A]


def test_zero_vector():
    codes, ks = quantize_coarse_key(np.zeros(64, np.float32))
    assert ks == np.float32(1.0 / 448.0) and not codes.any()


def _torch_codes(y):
    return torch.from_numpy(np.asarray(y, np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def test_codes_match_torch_float8_conversion():
    rng = np.random.default_rng(5)
    for trial in range(400):
        dim = 64 if trial % 2 else 128
        scale = 10.0 ** rng.uniform(-6, 6)
        x = (rng.standard_normal(dim) * scale).astype(np.float32)
        if trial % 7 == 0:
            x[rng.integers(dim)] = 0.0
        codes, ks = quantize_coarse_key(x)
        y = np.clip((x / ks).astype(np.float32), -448.0, 448.0)
        assert np.array_equal(codes, _torch_codes(y)), trial


def test_largest_entry_and_error_bound():
    rng = np.random.default_rng(6)
    for trial in range(200):
        x = (rng.standard_normal(128) * 10.0 ** rng.uniform(-3, 3)).astype(np.float32)
        codes, ks = quantize_coarse_key(x)
        v = e4m3_decode(codes)
        i = int(np.argmax(np.abs(x)))
        assert abs(v[i]) == 448.0 and np.sign(v[i]) == np.sign(x[i])
        # ks approximates max|x| / 448 to float32 precision
        assert abs(float(ks) * 448.0 / float(np.abs(x).max()) - 1.0) < 1e-6
        # round to nearest: within half a step of the E4M3 grid at |y|
        y = x.astype(np.float64) / float(ks)
        e = np.floor(np.log2(np.maximum(np.abs(y), 2.0 ** -6)))
        half_step = np.exp2(e - 3) / 2
        assert np.all(np.abs(v - y) <= half_step * (1 + 1e-6) + 1e-9), trial


def test_kv_write_round_trip():
    rng = np.random.default_rng(7)
    P, bs, H, d = 12, 64, 2, 8
    k_pool = rng.integers(0, 1 << 16, size=(P, bs, H, d), dtype=np.uint16)
    v_pool = rng.integers(0, 1 << 16, size=(P, bs, H, d), dtype=np.uint16)
    table = np.array([[3, 7, 1, 0], [9, 4, 11, 2]], dtype=np.int32)
    seq_lens = np.array([200, 130], dtype=np.int32)
    tok_seq = np.array([0, 0, 1, 1, 0], dtype=np.int32)
    tok_pos = np.array([0, 199, 64, 129, 77], dtype=np.int32)
    k_new = rng.integers(0, 1 << 16, size=(5, H, d), dtype=np.uint16)
    v_new = rng.integers(0, 1 << 16, size=(5, H, d), dtype=np.uint16)
    k2, v2 = kv_write(k_pool, v_pool, table, seq_lens, tok_seq, tok_pos, k_new, v_new, bs)
    touched = set()
    for i in range(5):
        p, t = table[tok_seq[i]][tok_pos[i] // bs], tok_pos[i] % bs
        assert np.array_equal(k2[p, t], k_new[i]) and np.array_equal(v2[p, t], v_new[i])
        touched.add((p, t))
    for p in range(P):
        for t in range(bs):
            if (p, t) not in touched:
                assert np.array_equal(k2[p, t], k_pool[p, t]) and np.array_equal(v2[p, t], v_pool[p, t])
    # decode default: query i of sequence i at seq_lens[i] - 1
    k3, _ = kv_write(k_pool, v_pool, table, seq_lens, None, None, k_new[:2], v_new[:2], bs)
    assert np.array_equal(k3[table[0][199 // bs], 199 % bs], k_new[0])
    assert np.array_equal(k3[table[1][129 // bs], 129 % bs], k_new[1])


def test_kv_write_round_trip_large_blocks():
    rng = np.random.default_rng(8)
    for bs in (128, 512):
        P, H, d = 5, 1, 4
        k_pool = rng.integers(0, 1 << 16, size=(P, bs, H, d), dtype=np.uint16)
        table = np.array([[4, 0, 2], [1, 3, -1]], dtype=np.int32)
        seq_lens = np.array([2 * bs + 3, bs + 1], dtype=np.int32)
        tok_seq = np.array([0, 0, 1, 1], dtype=np.int32)
        tok_pos = np.array([bs - 1, 2 * bs + 2, bs, 0], dtype=np.int32)
        k_new = rng.integers(0, 1 << 16, size=(4, H, d), dtype=np.uint16)
        k2, _ = kv_write(k_pool, k_pool, table, seq_lens, tok_seq, tok_pos, k_new, k_new, bs)
        want = k_pool.copy()
        want[4, bs - 1], want[2, 2], want[3, 0], want[1, 0] = k_new
        assert np.array_equal(k2, want)

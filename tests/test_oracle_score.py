"""Pins of the oracle's query quantization and index scoring.

* q scale: closed form (smallest power of two that brings max|q| under 448)
  and the invariant max|q|/scale in (224, 448];
* scores: exact integer recomputation (int64 counts of 2^-18), the
  identity-activation closed form, and the hand examples H1-H3.
"""

import numpy as np
import pytest

from oracle import (e4m3_decode, e4m3_encode, quantize_q_idx, index_scores,
                    bf16_bits_to_f64)
from oracle.pipeline import score_query


def _rand_bf16(rng, shape, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    bits = (x.view(np.uint32) + 0x7FFF + ((x.view(np.uint32) >> 16) & 1)) >> 16
    return bf16_bits_to_f64(bits.astype(np.uint16))


def test_q_scale_closed_form_and_invariant():
    rng = np.random.default_rng(1)
    for scale in (1e-3, 0.1, 1.0, 37.0, 1e4):
        q = _rand_bf16(rng, (64, 8, 128), scale)
        codes, sq = quantize_q_idx(q)
        # scale is a power of two
        m, e = np.frexp(sq)
        assert np.all(m == 0.5)
        amax = np.abs(q).max(axis=-1)
        assert np.all(amax <= 448.0 * sq)
        assert np.all(amax > 448.0 * sq / 2)  # the next smaller power fails
        r = amax / sq
        assert np.all((r > 224.0) & (r <= 448.0))
        # after round-to-nearest the largest code value lies in [224, 448]
        cmax = np.abs(e4m3_decode(codes)).max(axis=-1)
        assert np.all((cmax >= 224.0) & (cmax <= 448.0))
        # codes are the RNE encoding of q/scale (division exact)
        assert np.array_equal(codes, e4m3_encode(q / sq[..., None]))


def test_q_scale_zero_and_exact_powers():
    codes, sq = quantize_q_idx(np.zeros((2, 4)))
    assert np.all(sq == 1.0) and np.all(codes == 0)
    # amax = 448 exactly: scale 1, code 0x7E
    codes, sq = quantize_q_idx(np.array([[448.0, -1.0]]))
    assert sq[0] == 1.0 and codes[0, 0] == 0x7E and codes[0, 1] == 0xB8
    # amax = 449: needs scale 2
    codes, sq = quantize_q_idx(np.array([[449.0, 0.0]]))
    assert sq[0] == 2.0


def test_scores_exact_integer_recomputation():
    rng = np.random.default_rng(2)
    for d_i in (64, 128):
        qc = rng.integers(0, 256, size=(8, d_i)).astype(np.uint8)
        kc = rng.integers(0, 256, size=(300, d_i)).astype(np.uint8)
        qc[(qc & 0x7F) == 0x7F] = 0x7E  # no NaN codes
        kc[(kc & 0x7F) == 0x7F] = 0x7E
        # integer value in units of 2^-9, from the bit fields directly
        def units(c):
            c = c.astype(np.int64)
            e, m = (c >> 3) & 15, c & 7
            mag = np.where(e == 0, m, (8 + m) << np.maximum(e - 1, 0))
            return np.where(c >> 7, -mag, mag)
        d_int = units(qc) @ units(kc).T  # int64, exact
        sq = np.exp2(rng.integers(-12, 4, size=8).astype(np.float64))
        ks = rng.uniform(0.001, 0.01, size=300)
        w = rng.uniform(0, 1, size=8)
        got = index_scores(qc, sq, w, kc, ks)
        want = np.zeros(300)
        for h in range(8):
            t = (sq[h] * ks) * (d_int[h].astype(np.float64) * 2.0 ** -18)
            want = want + w[h] * np.where(t > 0, t, 0.0)
        assert np.array_equal(got, want)
        assert np.all(np.abs(d_int) < 2 ** 43)


def test_identity_activation_closed_form():
    rng = np.random.default_rng(3)
    qc = rng.integers(0, 0x7E, size=(4, 64)).astype(np.uint8)
    kc = rng.integers(0, 0x7E, size=(50, 64)).astype(np.uint8)
    sq = np.exp2(rng.integers(-10, 0, size=4).astype(np.float64))
    ks = rng.uniform(0.001, 0.01, size=50)
    w = rng.uniform(0, 1, size=4)
    got = index_scores(qc, sq, w, kc, ks, activation="identity")
    qsum = (w * sq) @ e4m3_decode(qc)  # [64]
    want = ks * (e4m3_decode(kc) @ qsum)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=0)


def test_hand_examples_scores(golden):
    h1 = golden["H1"]
    codes, sq = quantize_q_idx(np.array(h1["q_idx"]))
    assert codes.tolist() == h1["q_codes"] and sq.tolist() == h1["q_scale"]
    kcodes = e4m3_encode(np.array(h1["key_values"]))
    assert kcodes.tolist() == h1["key_codes"]
    cand, s, loc = score_query(np.array(h1["q_idx"]), h1["w"], [0, 1], h1["pos"],
                               h1["seq_len"], 2, kcodes, np.ones(2))
    assert cand.tolist() == [0, 1] and loc == 1 and s.tolist() == h1["scores"]

    h2 = golden["H2"]
    kcodes = e4m3_encode(np.array(h2["key_values"]))
    assert kcodes.tolist() == h2["key_codes"]
    for act in ("relu", "identity"):
        _, s, _ = score_query(np.array(h2["q_idx"]), h2["w"], [0, 1, 2], h2["pos"],
                              h2["seq_len"], 2, kcodes, np.ones(3), activation=act)
        assert s.tolist() == h2[act]["scores"]

    h3 = golden["H3"]
    kcodes = e4m3_encode(np.array(h3["key_values"]))
    assert kcodes.tolist() == h3["key_codes"]
    _, s, _ = score_query(np.array(h3["q_idx"]), h3["w"], [0, 1, 2], h3["pos"],
                          h3["seq_len"], 2, kcodes, np.ones(3))
    assert s.tolist() == h3["scores"]

    h4 = golden["H4"]
    kcodes = e4m3_encode(np.array(h1["key_values"]))
    cand, s, loc = score_query(np.array(h1["q_idx"]), h1["w"], [0, 1], h4["pos"],
                               h4["seq_len"], 2, kcodes, np.ones(2))
    assert cand.tolist() == [0, 1] and loc == 1 and s.tolist() == h4["scores"]


def test_scores_use_the_block_table():
    # the physical key row of logical block j is table[j]
    kcodes = e4m3_encode(np.array([[1.0, 0.0], [5.0, 0.0], [2.0, 0.0]]))
    _, s, _ = score_query(np.array([[1.0, 0.0]]), [1.0], [2, 0, 1], 5, 6, 2,
                          kcodes, np.ones(3))
    assert s.tolist() == [2.0, 1.0, 5.0]

"""The seeded input generator: published SplitMix64 outputs, determinism,
random access, moments and the shapes of the benchmark-shaped workloads."""

import numpy as np

from dsa_synth import gen, workload


def test_splitmix64_published_outputs():
    # SplitMix64 with state 1234567: the first five outputs of the reference
    # generator (Steele, Lea, Flood 2014; Vigna's public test vectors).
    x = np.uint64(1234567) + np.arange(1, 6, dtype=np.uint64) * gen.GOLDEN
    want = [6457827717110365317, 3203168211198807973, 9817491932198370423,
            4593380528125082431, 16408922859458223821]
    assert gen.mix64(x).tolist() == want


def test_random_access_matches_ranges():
    full = gen.bf16_normal_tensor(7, gen.TAG_K, (1000,))
    for off, n in ((0, 10), (3, 17), (996, 4), (5, 1)):
        assert np.array_equal(gen.bf16_normal_tensor(7, gen.TAG_K, (n,), offset=off),
                              full[off: off + n])
    e = np.array([0, 1, 2, 3, 4, 999], dtype=np.uint64)
    assert np.array_equal(gen.bf16_normal_bits(7, gen.TAG_K, e), full[e.astype(np.int64)])


def test_moments_and_tables():
    x = gen.bf16_bits_to_f32(gen.bf16_normal_tensor(3, gen.TAG_Q, (1 << 20,))).astype(np.float64)
    assert abs(x.mean()) < 5e-3 and abs(x.var() - 1.0) < 1e-2
    u = gen.uniform_tensor(3, gen.TAG_W, (1 << 18,))
    assert u.min() > 0 and u.max() < 1 and abs(u.mean() - 0.5) < 5e-3
    t = gen.normal_table_f64()
    assert np.all(np.diff(t) > 0) and abs(t[32767] + t[32768]) < 1e-12


def test_streams_differ_and_are_deterministic():
    a = gen.bf16_normal_tensor(11, gen.TAG_K, (4096,))
    b = gen.bf16_normal_tensor(11, gen.TAG_V, (4096,))
    c = gen.bf16_normal_tensor(11, gen.TAG_K, (4096,))
    assert np.array_equal(a, c) and not np.array_equal(a, b)


def test_workload_shapes():
    w = workload.tiny_decode()
    assert w.block_table.shape == (1, 64) and sorted(w.block_table[0]) == list(range(64))
    assert w.q_bits.shape == (1, 8, 128) and w.q_idx_bits.shape == (1, 4, 64)
    assert w.idx_keys.shape == (64, 64) and np.all((w.idx_keys & 0x7F) != 0x7F)
    s = workload.small_decode()
    assert s.block_table.shape[0] == 5
    used = np.concatenate([s.block_table[i, : -(-int(L) // 64)] for i, L in enumerate(s.seq_lens)])
    assert np.unique(used).size == used.size and used.max() < s.num_blocks
    p = workload.small_prefill()
    assert p.q_pos[-1] == p.seq_lens[0] - 1 and not p.decode


def test_multi_prefill_queries():
    for inter in (False, True):
        w = workload.multi_prefill(interleave=inter)
        assert w.num_queries == 280 and not w.decode
        assert (w.q_pos < w.seq_lens[w.q_seq]).all() and (w.q_pos >= 0).all()
        for s, c in enumerate((120, 90, 70)):
            pos = np.sort(w.q_pos[w.q_seq == s])
            assert np.array_equal(pos, np.arange(w.seq_lens[s] - c, w.seq_lens[s]))
        nb = -(-w.seq_lens // 64)
        used = np.concatenate([w.block_table[s, :nb[s]] for s in range(3)])
        assert np.unique(used).size == used.size and used.max() < w.num_blocks
    w = workload.multi_prefill(interleave=True)
    assert list(w.q_seq[:6]) == [0, 1, 2, 0, 1, 2]

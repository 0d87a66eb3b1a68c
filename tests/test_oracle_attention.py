"""Pins of the oracle's sparse attention, dense attention and partial merge.

* hand examples H1 and H4 (closed forms);
* Top-K covering every block reproduces dense causal attention (the
  full-vs-sparse relation), and dense attention matches torch's
  scaled_dot_product_attention in float64 on the CPU (a library routine);
* V == 1 gives out == 1 (softmax weights sum to one);
* block size 1 with K = 1 gives the current token's V row;
* permuting the physical pool together with the block table changes nothing;
* merging the partials of a split token set equals the one-pass result.
"""

import numpy as np
import torch

from oracle import (sparse_attention, dense_attention, attention_partial,
                    merge_partials, e4m3_encode)
from oracle.dsa import _gather_tokens
from oracle.pipeline import run_query


def _paged(rng, nb, bs, hkv, d, extra=3):
    """A random paged cache: pool of nb+extra blocks, random table."""
    P = nb + extra
    K = rng.standard_normal((P, bs, hkv, d))
    V = rng.standard_normal((P, bs, hkv, d))
    table = rng.permutation(P)[:nb]
    return K, V, table


def test_hand_examples_attention(golden):
    h1 = golden["H1"]
    K = np.array(h1["k_tokens"]).reshape(2, 2, 1, 2)
    V = np.array(h1["v_tokens"]).reshape(2, 2, 1, 2)
    kcodes = e4m3_encode(np.array(h1["key_values"]))
    for c in h1["cases"]:
        r = run_query(np.array(h1["q"]), np.array(h1["q_idx"]), h1["w"], [0, 1],
                      h1["pos"], h1["seq_len"], 2, kcodes, np.ones(2), c["top_k"],
                      lambda p: K[p], lambda p: V[p], 1.0, 1)
        assert r["idx"].tolist() == c["idx"] and r["cnt"] == c["cnt"]
        np.testing.assert_allclose(r["out"], c["out"], rtol=0, atol=1e-14)
        np.testing.assert_allclose(r["lse"], c["lse"], rtol=0, atol=1e-14)
    h4 = golden["H4"]
    for c in h4["cases"]:
        r = run_query(np.array(h1["q"]), np.array(h1["q_idx"]), h1["w"], [0, 1],
                      h4["pos"], h4["seq_len"], 2, kcodes, np.ones(2), c["top_k"],
                      lambda p: K[p], lambda p: V[p], 1.0, 1)
        assert r["idx"].tolist() == c["idx"] and r["cnt"] == c["cnt"]
        np.testing.assert_allclose(r["out"], c["out"], rtol=0, atol=1e-14)
        np.testing.assert_allclose(r["lse"], c["lse"], rtol=0, atol=1e-14)


def test_all_blocks_equals_dense_and_torch():
    rng = np.random.default_rng(5)
    for bs, nb, hq, hkv in ((4, 5, 4, 2), (8, 3, 6, 3), (1, 7, 2, 1), (4, 6, 8, 1)):
        d = 8
        K, V, table = _paged(rng, nb, bs, hkv, d)
        for L in (nb * bs, nb * bs - 1, (nb - 1) * bs + 1):
            for pos in (L - 1, max(0, L - bs - 1)):
                q = rng.standard_normal((hq, d))
                ids = list(range(pos // bs + 1))
                o_s, l_s = sparse_attention(q, ids, table, pos, L, bs,
                                            lambda p: K[p], lambda p: V[p], 0.3, hkv)
                o_d, l_d = dense_attention(q, table, pos, L, bs,
                                           lambda p: K[p], lambda p: V[p], 0.3, hkv)
                np.testing.assert_allclose(o_s, o_d, rtol=0, atol=1e-12)
                np.testing.assert_allclose(l_s, l_d, rtol=0, atol=1e-12)
                # library routine: torch SDPA in float64 over the linear tokens
                toks = [table[a // bs] * bs + a % bs for a in range(pos + 1)]
                Kf = K.reshape(-1, hkv, d)[toks]  # [T, hkv, d]
                Vf = V.reshape(-1, hkv, d)[toks]
                g = (np.arange(hq) * hkv) // hq
                qt = torch.from_numpy(q)[:, None, :]  # [hq, 1, d]
                kt = torch.from_numpy(np.ascontiguousarray(Kf[:, g, :].transpose(1, 0, 2)))
                vt = torch.from_numpy(np.ascontiguousarray(Vf[:, g, :].transpose(1, 0, 2)))
                ref = torch.nn.functional.scaled_dot_product_attention(
                    qt, kt, vt, scale=0.3)[:, 0, :].numpy()
                np.testing.assert_allclose(o_d, ref, rtol=0, atol=1e-12)


def test_v_one_gives_one():
    rng = np.random.default_rng(6)
    K, V, table = _paged(rng, 6, 4, 2, 8)
    V[:] = 1.0
    q = rng.standard_normal((4, 8)) * 3
    o, _ = sparse_attention(q, [1, 3, 5], table, 23, 24, 4,
                            lambda p: K[p], lambda p: V[p], 1.0, 2)
    np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-14)


def test_block_size_one_top1_is_current_v():
    rng = np.random.default_rng(7)
    K, V, table = _paged(rng, 9, 1, 2, 8)
    q = rng.standard_normal((4, 8))
    for pos in range(9):
        o, lse = sparse_attention(q, [pos], table, pos, 9, 1,
                                  lambda p: K[p], lambda p: V[p], 0.5, 2)
        for h in range(4):
            g = (h * 2) // 4
            np.testing.assert_array_equal(o[h], V[table[pos], 0, g])
            assert lse[h] == 0.5 * (K[table[pos], 0, g] @ q[h])


def test_pool_permutation_invariance():
    rng = np.random.default_rng(8)
    K, V, table = _paged(rng, 7, 4, 2, 8, extra=5)
    perm = rng.permutation(K.shape[0])  # new physical id of old block p: perm[p]
    K2 = np.empty_like(K)
    V2 = np.empty_like(V)
    K2[perm] = K
    V2[perm] = V
    table2 = perm[table]
    q = rng.standard_normal((4, 8))
    a = sparse_attention(q, [0, 2, 6], table, 26, 27, 4, lambda p: K[p], lambda p: V[p], 0.7, 2)
    b = sparse_attention(q, [0, 2, 6], table2, 26, 27, 4, lambda p: K2[p], lambda p: V2[p], 0.7, 2)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_merge_identity():
    rng = np.random.default_rng(9)
    K, V, table = _paged(rng, 8, 4, 2, 8)
    q = rng.standard_normal((4, 8)) * 2
    sel = [0, 2, 3, 5, 7]
    o1, l1 = sparse_attention(q, sel, table, 31, 32, 4, lambda p: K[p], lambda p: V[p], 0.4, 2)
    parts = []
    for chunk in ([0, 2], [3], [5, 7]):
        Kc, Vc, _ = _gather_tokens(chunk, table, 31, 32, 4, lambda p: K[p], lambda p: V[p])
        parts.append(attention_partial(q, Kc, Vc, 0.4, 2))
    o2, l2 = merge_partials(parts)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-13)

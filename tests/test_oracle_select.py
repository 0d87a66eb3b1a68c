"""Pins of the oracle's Top-K block selection.

Brute force on thousands of tiny random cases (including integer-valued
scores that force ties): a block other than the local one is kept iff fewer
than K-1 other candidates beat it in the order (score desc, id asc).  This is
a counting rule, not a sort, so it checks the oracle's sort independently.
Invariants and the hand examples H2/H3 are checked too.
"""

import numpy as np

from oracle import select_blocks


def _brute(cand, scores, local, k):
    keep = [local]
    for j, s in zip(cand, scores):
        if j == local:
            continue
        better = sum(1 for j2, s2 in zip(cand, scores)
                     if j2 != local and j2 != j and (s2 > s or (s2 == s and j2 < j)))
        if better < k - 1:
            keep.append(j)
    keep = sorted(keep)
    return keep


def test_select_brute_force_random():
    rng = np.random.default_rng(4)
    for trial in range(3000):
        n = int(rng.integers(1, 12))
        k = int(rng.integers(1, 14))
        cand = np.arange(n)
        if trial % 2:
            scores = rng.integers(0, 3, size=n).astype(np.float32)  # many ties
        else:
            scores = rng.standard_normal(n).astype(np.float32)
        local = n - 1
        idx, cnt = select_blocks(cand, scores, local, k)
        want = _brute(cand.tolist(), scores.tolist(), local, k)
        assert cnt == len(want) == min(k, n)
        assert idx[:cnt].tolist() == want
        assert np.all(idx[cnt:] == -1) and idx.size == k
        # invariants
        assert local in idx[:cnt]
        assert np.all(np.diff(idx[:cnt]) > 0)
        unselected = [j for j in range(n) if j not in idx[:cnt]]
        sel_other = [j for j in idx[:cnt] if j != local]
        for u in unselected:
            for s in sel_other:
                assert (scores[s] > scores[u]) or (scores[s] == scores[u] and s < u)


def test_select_negative_zero_equals_zero():
    cand = np.arange(3)
    idx, _ = select_blocks(cand, np.array([-0.0, 0.0, 1.0], np.float32), 2, 2)
    assert idx.tolist() == [0, 2]
    idx, _ = select_blocks(cand, np.array([0.0, -0.0, 1.0], np.float32), 2, 2)
    assert idx.tolist() == [0, 2]


def test_hand_examples_select(golden):
    h2 = golden["H2"]
    for act in ("relu", "identity"):
        c = h2[act]
        idx, cnt = select_blocks(np.arange(3), np.array(c["scores"]), 2, c["top_k"])
        assert idx.tolist() == c["idx"] and cnt == c["cnt"]
    h3 = golden["H3"]
    for c in h3["cases"]:
        idx, cnt = select_blocks(np.arange(3), np.array(h3["scores"]), 2, c["top_k"])
        assert idx.tolist() == c["idx"] and cnt == c["cnt"]
    h1 = golden["H1"]
    for c in h1["cases"]:
        idx, cnt = select_blocks(np.arange(2), np.array(h1["scores"]), 1, c["top_k"])
        assert idx.tolist() == c["idx"] and cnt == c["cnt"]


def test_visible_blocks_are_the_causal_prefix():
    from oracle import visible_blocks, local_block
    for bs in (1, 2, 64):
        for L in range(1, 3 * bs + 2):
            for pos in range(L):
                v = visible_blocks(pos, L, bs).tolist()
                # exactly the blocks holding at least one token at or before pos
                want = sorted({a // bs for a in range(pos + 1)})
                assert v == want
                assert v[-1] == local_block(pos, bs)
    # the larger block sizes, on lengths and positions around block edges
    for bs in (128, 256, 512):
        for L in (1, bs - 1, bs, bs + 1, 3 * bs - 5, 4 * bs):
            for pos in sorted({0, bs - 1, bs, 2 * bs - 1, 2 * bs + 7, L - 1} & set(range(L))):
                v = visible_blocks(pos, L, bs).tolist()
                assert v == sorted({a // bs for a in range(pos + 1)})
                assert v[-1] == local_block(pos, bs)

"""Scoring + selection of many queries in one launch (index_topk_fp8.hip):
approximate FP8 matrix-core scores with an error bound, exact int8 digit
scores for the blocks the bound leaves undecided.  The selection must be the
exact one: equal, for every query, to the oracle's and to the stage-wise path
(dsa_index_score, whose scores are the oracle's bit for bit, then
dsa_topk_blocks).  Cases cover indexer heads 1-16, key dims 64 and 128, block
sizes 64-512, K from 1 past the context, ragged query counts, several
sequences per workgroup (grouped and interleaved), all-equal keys (every
block undecided: the exact path decides all), zero and negative head
weights."""

import sys

import numpy as np
import pytest

from dsa_synth import workload
from tests import parity

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


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


def _with(base, **fields):
    import copy
    v = copy.copy(base)
    for k, val in fields.items():
        setattr(v, k, val)
    return v


def _check(dsa, w, label, oracle_all=True, sample=None):
    kv, qs = parity.to_device(w)
    K = w.top_k
    bi, bc = dsa.index_topk(kv, qs, K)            # the FP8 + exact-rescoring kernel
    scores = dsa.index_score(kv, qs)              # exact scores (int8 digits)
    ri, rc = dsa.topk_blocks(scores, kv, qs, K)   # exact selection
    torch.cuda.synchronize()
    bi, bc, ri, rc = bi.cpu().numpy(), bc.cpu().numpy(), ri.cpu().numpy(), rc.cpu().numpy()
    bad = np.flatnonzero((bi != ri).any(axis=1) | (bc != rc))
    assert bad.size == 0, f"{label}: {bad.size} queries differ from the exact path, first {bad[:5]}"
    qis = range(w.num_queries) if oracle_all else (sample or [])
    for qi in qis:
        r = parity.oracle_select(w, int(qi))
        assert np.array_equal(bi[qi], r["idx"]) and int(bc[qi]) == r["cnt"], \
            f"{label} q{qi}: {bi[qi][:8]}.. vs oracle {r['idx'][:8]}.."
    _say(f"{label}: {w.num_queries} queries equal the exact path; "
         f"{len(qis)} checked against the oracle")
    del kv, qs, scores
    torch.cuda.empty_cache()


CASES = [
    dict(seed=4001, L=64 * 700 + 13, count=300, hi=8, di=128, top_k=16),
    dict(seed=4002, L=64 * 520, count=256, hi=4, di=64, top_k=8),
    dict(seed=4003, L=64 * 2048, count=264, hi=8, di=128, top_k=64),    # 2048 blocks, the limit
    dict(seed=4004, L=64 * 900 - 1, count=333, hi=1, di=128, top_k=32),
    dict(seed=4005, L=64 * 400 + 7, count=259, hi=3, di=64, top_k=5),
    dict(seed=4006, L=64 * 1200, count=270, hi=16, di=128, top_k=100),
    dict(seed=4007, L=64 * 300, count=256, hi=12, di=64, top_k=2),
    dict(seed=4008, L=64 * 640 + 1, count=280, hi=8, di=128, top_k=1),
    dict(seed=4009, L=64 * 50, count=300, hi=8, di=128, top_k=3000),    # K past the context
    dict(seed=4010, L=64 * 1500, count=257, hi=8, di=128, top_k=700),
]


@pytest.mark.parametrize("case", CASES, ids=[str(c["seed"]) for c in CASES])
def test_fp8_selection_matches_exact(dsa, case):
    w = workload.small_prefill(**case)
    _check(dsa, w, f"fp8 index_topk {case}", oracle_all=case["L"] <= 64 * 700 + 13)
    if case["L"] > 64 * 700 + 13:
        _check(dsa, w, f"fp8 index_topk {case} (oracle sample)", oracle_all=False,
               sample=[0, 1, 7, 8, 100, w.num_queries - 1])


@pytest.mark.parametrize("bs", [128, 256, 512])
def test_fp8_selection_block_sizes(dsa, bs):
    w = workload.small_prefill(seed=4020 + bs, L=bs * 200 + 33, count=260, hi=8, di=128,
                               top_k=12, bs=bs)
    _check(dsa, w, f"fp8 index_topk bs={bs}")


@pytest.mark.parametrize("interleave", [False, True])
def test_fp8_selection_several_sequences(dsa, interleave):
    """Queries of three sequences in one batch: a workgroup of 8 queries holds
    one or several sequences (interleaved: all three), scored once per
    sequence."""
    w = workload.multi_prefill(seed=4030 + int(interleave), lens=(64 * 300 + 7, 64 * 120,
                                                                  64 * 210 - 1),
                               counts=(120, 90, 70), interleave=interleave, top_k=10)
    _check(dsa, w, f"fp8 index_topk multi-sequence interleave={interleave}")


def test_fp8_selection_all_keys_equal(dsa):
    """Every coarse key and scale equal: all candidates tie, every one is
    undecided by the bound (more than 1024 a query: the rescoring runs in
    rounds), and the lowest ids win."""
    w = workload.small_prefill(seed=4040, L=64 * 1500, count=256, hi=8, di=128, top_k=40)
    keys = np.repeat(w.idx_keys[:1], w.idx_keys.shape[0], axis=0)
    w = _with(w, idx_keys=keys, idx_scale=np.full_like(w.idx_scale, w.idx_scale[0]))
    _check(dsa, w, "fp8 index_topk all keys equal", oracle_all=False, sample=[0, 5, 255])


def test_fp8_selection_zero_and_negative_weights(dsa):
    """Head weights of both signs, and queries whose weights are all zero
    (every score 0: the exact path breaks the ties toward the lowest ids)."""
    w = workload.small_prefill(seed=4050, L=64 * 800 + 3, count=272, hi=8, di=128, top_k=20)
    ww = w.w.copy()
    ww[:, 1::2] *= -1.0
    ww[5] = 0.0
    ww[200] = 0.0
    w = _with(w, w=ww.astype(np.float32))
    _check(dsa, w, "fp8 index_topk signed / zero weights", oracle_all=False,
           sample=[0, 5, 6, 200, 271])


def test_fp8_selection_zero_query_rows(dsa):
    """Indexer query rows that are all zero for some heads (scale exponent 0,
    every product zero)."""
    w = workload.small_prefill(seed=4060, L=64 * 600, count=264, hi=8, di=128, top_k=9)
    qb = w.q_idx_bits.copy()
    qb[3, :, :] = 0
    qb[10, 2, :] = 0
    qb[11, :5, :] = 0
    w = _with(w, q_idx_bits=qb)
    _check(dsa, w, "fp8 index_topk zero query rows", oracle_all=False, sample=[3, 10, 11, 12])


def _e4m3_codes(x):
    """E4M3 codes (uint8) of x by torch's float8_e4m3fn conversion."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def _bf16_bits(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def test_fp8_selection_outlier_operands(dsa):
    """Keys and query rows made mostly of small values with a few large ones
    in random dims (the FP8 matrix unit's truncation errors are then largest
    against the products that survive), and pairs of blocks with identical
    keys and scales (exact ties that the bound must leave undecided): the
    selection still equals the exact one for every query."""
    w = workload.small_prefill(seed=4070, L=64 * 1100 + 5, count=264, hi=8, di=128, top_k=24)
    rng = np.random.default_rng(4071)
    P, dI = w.idx_keys.shape
    kx = rng.standard_normal((P, dI)) * 0.05
    hit = rng.random((P, dI)) < 0.04
    kx = np.where(hit, rng.standard_normal((P, dI)) * 3.0, kx)
    kx = kx * (448.0 / np.maximum(np.abs(kx).max(axis=1, keepdims=True), 1e-30))
    keys = _e4m3_codes(kx)
    ks = (rng.uniform(0.5, 2.0, P) / 448.0).astype(np.float32)
    twin = rng.random(P) < 0.1  # block p takes block p - 1's key and scale
    for p in np.flatnonzero(twin[1:]) + 1:
        keys[p] = keys[p - 1]
        ks[p] = ks[p - 1]
    nq, hi = w.q_idx_bits.shape[0], w.q_idx_bits.shape[1]
    qx = rng.standard_normal((nq, hi, dI)) * 0.1
    qhit = rng.random((nq, hi, dI)) < 0.05
    qx = np.where(qhit, rng.standard_normal((nq, hi, dI)) * 4.0, qx)
    w = _with(w, idx_keys=keys, idx_scale=ks, q_idx_bits=_bf16_bits(qx))
    _check(dsa, w, "fp8 index_topk outlier operands", oracle_all=False,
           sample=[0, 1, 63, 64, 131, 263])

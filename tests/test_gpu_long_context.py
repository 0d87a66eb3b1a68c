"""The long-context decode path of dsa_sparse_decode_fused (two launches):
chunk scoring on the int8 matrix cores with a candidate list per 256-block
chunk (index_cand_scores, index_score.hip), then attention whose workgroups
merge their query's lists themselves (the list-maxima filter, or two levels
when too many candidates survive it) and whose last split per (query, KV head)
merges the split partials in the same launch (sparse_attn_split, attn.hip).

Every case is checked query by query against the oracle (indices exact,
attention at the stated bar), and the selection against the stage-wise path
(dsa_index_topk).  Cases: K = 2, 32 and 128 (K = 1 and 129 take other paths,
checked the same way), queries whose context holds fewer than K blocks next
to long ones (their later chunks lie wholly past their position), indexer
heads 1-16 with key dims 64 and 128, block sizes 128 and 512, a batch wide
enough for one split per (query, KV head) (no split counters), all candidates
tied (the two-level merge), more than 64 lists a query (no list-maxima
filter), and two query sets alternating through one workspace (the split
counters are zeroed by each call's scoring launch; a stale hand-off would show
as the other set's result)."""

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


def _run(dsa, kv, qs, w, workspace=None):
    nq, K = w.num_queries, w.top_k
    bi = torch.full((nq, K), -7, dtype=torch.int32, device="cuda")
    bc = torch.full((nq,), -7, dtype=torch.int32, device="cuda")
    out, lse, _, _ = dsa.decode_fused(kv, qs, K, w.softmax_scale, block_idx=bi, block_cnt=bc,
                                      workspace=workspace)
    torch.cuda.synchronize()
    return bi.cpu().numpy(), bc.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy()


def _check(dsa, w, label, qis=None, kv=None, qs=None, res=None):
    if kv is None:
        kv, qs = parity.to_device(w)
    idx, cnt, out, lse = res if res is not None else _run(dsa, kv, qs, w)
    si, sc = dsa.index_topk(kv, qs, w.top_k)
    torch.cuda.synchronize()
    assert np.array_equal(si.cpu().numpy(), idx) and np.array_equal(sc.cpu().numpy(), cnt), \
        f"{label}: selection differs from the stage-wise path"
    assert np.isfinite(out).all() and np.isfinite(lse).all(), f"{label}: non-finite output"
    qis = range(w.num_queries) if qis is None else qis
    worst = 0.0
    for qi in qis:
        r = parity.oracle_query(w, int(qi))
        assert np.array_equal(idx[qi], r["idx"]) and int(cnt[qi]) == r["cnt"], \
            f"{label} q{qi}: indices {idx[qi][:8]}.. cnt {cnt[qi]} vs {r['idx'][:8]}.. {r['cnt']}"
        good, a, rel = parity.attn_ok(out[qi], r["out"])
        assert good, f"{label} q{qi}: attention max-abs {a:.3e} max-rel {rel:.3e}"
        la, _ = parity.attn_errors(lse[qi], r["lse"])
        assert la <= 1e-3, f"{label} q{qi}: lse {la:.3e}"
        worst = max(worst, a)
    _say(f"{label}: {len(qis)} queries equal the oracle's selection, worst max-abs {worst:.2e}")


@pytest.mark.parametrize("top_k", [1, 2, 32, 128, 129])
def test_long_context_top_k(dsa, top_k):
    # 3072 blocks: twelve 256-block chunks, whose lists fit the score
    # workspace up to K = 128
    w = workload.small_decode(seed=2400 + top_k, lens=(64 * 2300 + 17, 64 * 2049, 64 * 3072 - 5),
                              hq=16, hkv=2, hi=8, di=128, top_k=top_k)
    _check(dsa, w, f"long-context K={top_k}")


def test_long_context_short_queries_in_a_long_batch(dsa):
    """Contexts of 1, 20 and 40 blocks (at or below K - 1 = 31) beside long
    ones: the short queries' lists are empty past their first chunk and their
    selection is every block they have."""
    w = workload.small_decode(seed=2420, lens=(64 * 2600, 1, 64 * 20 - 3, 64 * 2200 + 1, 64 * 40,
                                               64 * 300 + 5),
                              hq=16, hkv=2, hi=8, di=128, top_k=32)
    _check(dsa, w, "long-context short queries")


@pytest.mark.parametrize("hi,di", [(1, 128), (3, 64), (4, 64), (16, 128), (12, 64)])
def test_long_context_indexer_shapes(dsa, hi, di):
    w = workload.small_decode(seed=2430 + hi + di, lens=(64 * 2100 + 9, 64 * 2500 - 1),
                              hq=8, hkv=1, hi=hi, di=di, top_k=20)
    _check(dsa, w, f"long-context hi={hi} di={di}")


@pytest.mark.parametrize("bs", [128, 512])
def test_long_context_block_sizes(dsa, bs):
    w = workload.small_decode(seed=2450 + bs, lens=(bs * 2100 - 100, bs * 2300 + 3),
                              hq=16, hkv=2, hi=4, di=64, top_k=12, bs=bs)
    _check(dsa, w, f"long-context bs={bs}")


def test_long_context_one_split_per_head(dsa):
    """32 queries x 8 KV heads = 256 (query, head) units: one split each, no
    partials (outputs written by the attention workgroups themselves)."""
    w = workload.shared_pool_decode()
    _check(dsa, w, "long-context one split per head", qis=[0, 1, 13, 30, 31])


def test_long_context_alternating_query_sets(dsa):
    """Two query sets over one cache, alternating through one workspace for
    six launches; each launch must give its own set's result."""
    wa = workload.small_decode(seed=2470, lens=(64 * 2400 + 3, 64 * 2100, 64 * 2900 - 7, 64 * 2048),
                               hq=16, hkv=2, hi=8, di=128, top_k=16)
    wb = workload.with_query_seed(wa, 99)
    kv, qa = parity.to_device(wa)
    _, qb = parity.to_device(wb)
    from dynamic_sparse_attention_paged_amd import _lib
    ws = dsa.make_workspace(_lib.OP_DECODE_FUSED, kv, qa, wa.top_k)
    first = {}
    for i in range(6):
        w, qs = (wa, qa) if i % 2 == 0 else (wb, qb)
        res = _run(dsa, kv, qs, w, workspace=ws)
        key = i % 2
        if key not in first:
            first[key] = res
            _check(dsa, w, f"alternating set {key}", kv=kv, qs=qs, res=res)
        else:
            for a, b in zip(res, first[key]):
                assert np.array_equal(a, b), f"launch {i}: set {key} result changed"
    assert not np.array_equal(first[0][0], first[1][0]), "the two sets select the same blocks"
    _say("alternating query sets: six launches, each equal to its set's checked result")


def _with(base, **fields):
    import copy
    v = copy.copy(base)
    for k, val in fields.items():
        setattr(v, k, val)
    return v


def test_long_context_all_keys_equal(dsa):
    """Every coarse key and scale equal: all candidates tie, the list maxima
    filter keeps every one of 18 x 31 candidates (past the one-wave bound:
    the two-level merge), and the lowest ids win."""
    w = workload.small_decode(seed=2480, lens=(64 * 4500 + 3, 64 * 4200), hq=16, hkv=2, hi=8,
                              di=128, top_k=32)
    keys = np.repeat(w.idx_keys[:1], w.idx_keys.shape[0], axis=0)
    w = _with(w, idx_keys=keys, idx_scale=np.full_like(w.idx_scale, w.idx_scale[0]))
    _check(dsa, w, "long-context all keys equal")


@pytest.mark.parametrize("top_k", [8, 20])
def test_long_context_more_than_64_lists(dsa, top_k):
    """67 chunks a query (no list-maxima filter): 67 x 7 candidates (one
    wave) and 67 x 19 (two levels)."""
    w = workload.small_decode(seed=2490 + top_k, lens=(64 * 17000 - 9, 64 * 16500), hq=8, hkv=1,
                              hi=4, di=64, top_k=top_k)
    _check(dsa, w, f"long-context 67 lists K={top_k}")

"""GPU parity at the five benchmark-shaped workloads, in the launch
configuration bench.py times (fused decode; index_score -> topk -> prefill
attention for the chunked prefill), on queries the oracle can check one by
one.  Also exercises every Top-K variant: one wave for up to 128, 512 and 2048
candidates, the two-level selection for longer lists, and the LDS radix for
long lists with a large K."""

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


def _check(w, qis, idx, cnt, out, lse, label):
    worst = (0.0, 0.0)
    swaps = 0
    for qi in qis:
        r = parity.oracle_query(w, int(qi))
        ok, nsw = parity.check_indices(idx[qi], cnt[qi], r, w.top_k)
        assert ok, f"{label} q{qi}: indices {idx[qi][:8]}.. cnt {cnt[qi]} vs {r['idx'][:8]}.. {r['cnt']}"
        swaps += nsw
        ref = r if nsw == 0 else parity.oracle_query(w, int(qi), sel_override=idx[qi][:cnt[qi]])
        good, a, rel = parity.attn_ok(out[qi], ref["out"])
        assert good, f"{label} q{qi}: attention max-abs {a:.3e} max-rel {rel:.3e}"
        la, _ = parity.attn_errors(lse[qi], ref["lse"])
        assert la <= 1e-3, f"{label} q{qi}: lse {la:.3e}"
        worst = (max(worst[0], a), max(worst[1], rel))
    _say(f"{label}: {len(qis)} queries ok, {swaps} near-tie swaps, worst max-abs {worst[0]:.2e} "
         f"max-rel {worst[1]:.2e}")


def _fused(dsa, w, kv_layout=0):
    kv, qs = parity.to_device(w, kv_layout=kv_layout)
    nq, K = w.num_queries, w.top_k
    bi = torch.empty(nq, K, dtype=torch.int32, device="cuda")
    bc = torch.empty(nq, dtype=torch.int32, device="cuda")
    out, lse, _, _ = dsa.decode_fused(kv, qs, K, w.softmax_scale, block_idx=bi, block_cnt=bc)
    torch.cuda.synchronize()
    res = bi.cpu().numpy(), bc.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy()
    del kv, qs, out, lse, bi, bc
    torch.cuda.empty_cache()
    return res


@pytest.mark.parametrize("lens,top_k", [((64 * 1500 - 3, 64 * 700, 64 * 513 + 1), 40),
                                         ((64 * 2500, 64 * 2049 - 1, 64 * 5000 + 7), 24),
                                         ((64 * 3000 + 9, 64 * 2100), 200),
                                         ((64 * 17000, 64 * 900), 33)])
def test_topk_variants_long_lists(dsa, lens, top_k):
    w = workload.small_decode(seed=2201 + len(lens) + top_k, lens=lens, hq=16, hkv=2, hi=8,
                              top_k=top_k)
    _say(f"long lists {lens} K={top_k}")
    idx, cnt, out, lse = _fused(dsa, w)
    _check(w, range(w.num_queries), idx, cnt, out, lse, "long lists")
    # scoring + selection alone (dsa_index_topk): the same lists
    kv, qs = parity.to_device(w)
    bi, bc = dsa.index_topk(kv, qs, top_k)
    torch.cuda.synchronize()
    assert np.array_equal(bi.cpu().numpy(), idx) and np.array_equal(bc.cpu().numpy(), cnt)


@pytest.mark.parametrize("kv_layout", [0, 1], ids=["token_major", "head_major"])
def test_batched_decode_full(dsa, kv_layout):
    w = workload.batched_decode()
    _say(f"batched decode 32 x 32768, all queries, kv_layout {kv_layout}")
    idx, cnt, out, lse = _fused(dsa, w, kv_layout)
    _check(w, range(w.num_queries), idx, cnt, out, lse, "batched_decode")
    # the fused step's attention kernel alone, as bench.py times it for its
    # roofline: scores from dsa_index_score, selection inside the attention
    kv, qs = parity.to_device(w, kv_layout=kv_layout)
    scores = dsa.index_score(kv, qs)
    bi = torch.empty(w.num_queries, w.top_k, dtype=torch.int32, device="cuda")
    bc = torch.empty(w.num_queries, dtype=torch.int32, device="cuda")
    o2, l2, _, _ = dsa.sparse_attn_decode_topk(kv, qs, scores, w.top_k, w.softmax_scale,
                                               block_idx=bi, block_cnt=bc)
    torch.cuda.synchronize()
    assert np.array_equal(bi.cpu().numpy(), idx) and np.array_equal(bc.cpu().numpy(), cnt)
    # the same kernel as the fused step's, on the same selection: the same bits
    assert np.array_equal(o2.cpu().numpy(), out) and np.array_equal(l2.cpu().numpy(), lse)
    del kv, qs, scores, o2, l2
    torch.cuda.empty_cache()


@pytest.mark.parametrize("kv_layout", [0, 1], ids=["token_major", "head_major"])
def test_million_decode_full(dsa, kv_layout):
    w = workload.million_decode()
    _say(f"million-token decode 4 x 1048576, all queries, kv_layout {kv_layout}")
    idx, cnt, out, lse = _fused(dsa, w, kv_layout)
    _check(w, range(w.num_queries), idx, cnt, out, lse, "million_decode")


@pytest.mark.parametrize("kv_layout", [0, 1], ids=["token_major", "head_major"])
def test_ragged_decode_sampled(dsa, kv_layout):
    w = workload.ragged_decode()
    _say(f"ragged decode 128 seqs, pool {w.num_blocks} blocks, 16 sampled queries, "
         f"kv_layout {kv_layout}")
    idx, cnt, out, lse = _fused(dsa, w, kv_layout)
    order = np.argsort(w.seq_lens)
    qis = sorted(set(order[:4].tolist() + order[-4:].tolist() + list(range(0, 128, 16))))
    _check(w, qis, idx, cnt, out, lse, "ragged_decode")
    # the scores (eight 16-block tiles a wave at this size): the oracle's, bit for bit
    kv, qs = parity.to_device(w, kv_layout=kv_layout)
    sh = dsa.index_score(kv, qs).cpu().numpy()
    del kv, qs
    torch.cuda.empty_cache()
    for qi in [int(order[0]), int(order[-1]), 37]:
        r = parity.oracle_query(w, qi)
        assert parity.check_scores_exact(sh[qi], r, w.block_table.shape[1]).size == 0, f"q{qi}"


# tile edges (queries 63/64/65, 127/128), the first and last queries, the
# middle of the chunk, and a stride through the rest
PREFILL_SAMPLE = [0, 1, 63, 64, 65, 127, 128, 4095, 4096, 8190, 8191] + list(range(700, 8192, 1013))


@pytest.mark.parametrize("kv_layout", [0, 1], ids=["token_major", "head_major"])
def test_chunked_prefill_sampled(dsa, kv_layout):
    """The full 8192-query chunk through both prefill paths, as bench.py times
    them: index_score -> topk -> the per-query prefill kernel, and the one-call
    block-inverted prefill (dsa_sparse_prefill_fused: ~256 queries per pool
    tile list, a 17 GB partial-state region, byte offsets past 2^31).  Sampled
    queries against the oracle, each computed on its own."""
    w = workload.chunked_prefill()
    _say(f"chunked prefill 8192 queries, {len(PREFILL_SAMPLE)} sampled, kv_layout {kv_layout}")
    kv, qs = parity.to_device(w, kv_layout=kv_layout)
    K = w.top_k
    scores = dsa.index_score(kv, qs)
    idx, cnt = dsa.topk_blocks(scores, kv, qs, K)
    out, lse = dsa.sparse_attn_prefill(kv, qs, idx, cnt, K, w.softmax_scale)
    torch.cuda.synchronize()
    sh = scores.cpu().numpy()
    idx_h, cnt_h, out_h, lse_h = idx.cpu().numpy(), cnt.cpu().numpy(), out.cpu().numpy(), \
        lse.cpu().numpy()
    del scores, out, lse
    bi = torch.empty_like(idx)
    bc = torch.empty_like(cnt)
    fo, fl, _, _ = dsa.prefill_fused(kv, qs, K, w.softmax_scale, block_idx=bi, block_cnt=bc)
    torch.cuda.synchronize()
    bi_h, bc_h, fo_h, fl_h = bi.cpu().numpy(), bc.cpu().numpy(), fo.cpu().numpy(), fl.cpu().numpy()
    del kv, qs, idx, cnt, bi, bc, fo, fl
    torch.cuda.empty_cache()
    # the one-call prefill selects exactly what the stage-wise path selects, for every query
    assert np.array_equal(bi_h, idx_h) and np.array_equal(bc_h, cnt_h)
    _check(w, PREFILL_SAMPLE, idx_h, cnt_h, out_h, lse_h, "chunked_prefill per-query")
    _check(w, PREFILL_SAMPLE, bi_h, bc_h, fo_h, fl_h, "chunked_prefill fused (block-inverted)")
    # the scores themselves are the oracle's float64 score rounded to fp32, bit for bit
    for qi in PREFILL_SAMPLE[:6]:
        r = parity.oracle_query(w, qi)
        assert parity.check_scores_exact(sh[qi], r, w.block_table.shape[1]).size == 0

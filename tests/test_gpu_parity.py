"""GPU parity: the HIP library against the float64 oracle on seeded inputs.

Each stage is checked in isolation (scoring on its own; Top-K fed the
oracle's scores; attention fed the oracle's indices) and end to end.
Scores must equal the oracle's float64 score rounded to fp32 bit for bit;
indices must be identical (swaps only among oracle scores within 1e-6
relative); attention within 2e-3 max-abs and 1e-2 max-rel (|oracle| >= 0.2).
"""

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
    m._lib.load()  # must be the HIP library; raises if not built
    return m


SMALL_DECODE_CASES = [
    dict(seed=2001),  # ragged lens incl. 1 and 64 tokens, Hq 16 / Hkv 2, HI 4 x 128, K 8
    dict(seed=2002, hq=8, hkv=1, hi=4, di=64, top_k=8, lens=(4096, 64 * 9 + 3, 130)),
    dict(seed=2003, hq=64, hkv=8, hi=8, di=128, top_k=32, lens=(64 * 70, 64 * 33 - 5, 64 * 31)),
    dict(seed=2004, hq=4, hkv=4, hi=1, di=128, top_k=1, lens=(700, 64, 1)),
    dict(seed=2005, hq=32, hkv=2, hi=16, di=64, top_k=200, lens=(64 * 150 + 1, 64 * 199)),
    dict(seed=2006, hq=12, hkv=3, hi=3, di=128, top_k=5, lens=(64 * 40 - 1, 64 * 6)),
]


def _run_all_stages(dsa, w, label, kv_layout=0):
    kv, qs = parity.to_device(w, kv_layout=kv_layout)
    maxb = w.block_table.shape[1]
    K = w.top_k
    scores = dsa.index_score(kv, qs)
    idx, cnt = dsa.topk_blocks(scores, kv, qs, K)
    out, lse = dsa.sparse_attn_decode(kv, qs, idx, cnt, K, w.softmax_scale) if w.decode else \
        dsa.sparse_attn_prefill(kv, qs, idx, cnt, K, w.softmax_scale)
    torch.cuda.synchronize()
    scores_h = scores.cpu().numpy()
    idx_h, cnt_h = idx.cpu().numpy(), cnt.cpu().numpy()
    out_h, lse_h = out.cpu().numpy(), lse.cpu().numpy()

    # stage-isolated runs: Top-K on the oracle's scores, attention on the oracle's indices
    refs = [parity.oracle_query(w, qi) for qi in range(w.num_queries)]
    ref_scores = np.full((w.num_queries, maxb), -np.inf, dtype=np.float32)
    ref_idx = np.stack([r["idx"] for r in refs]).astype(np.int32)
    ref_cnt = np.array([r["cnt"] for r in refs], dtype=np.int32)
    for qi, r in enumerate(refs):
        ref_scores[qi, r["cand"]] = r["scores"].astype(np.float32)
    idx2, cnt2 = dsa.topk_blocks(torch.from_numpy(ref_scores).cuda(), kv, qs, K)
    ri, rc = torch.from_numpy(ref_idx).cuda(), torch.from_numpy(ref_cnt).cuda()
    out2, lse2 = dsa.sparse_attn_decode(kv, qs, ri, rc, K, w.softmax_scale) if w.decode else \
        dsa.sparse_attn_prefill(kv, qs, ri, rc, K, w.softmax_scale)
    # decode attention that selects from the scores itself: on the library's
    # scores (the selection bit for bit the Top-K kernel's) and on the oracle's
    # (the oracle's selection); only the count is asked for in the second call
    fused_sel = w.decode and maxb <= 2048 and K <= 2048
    if fused_sel:
        bi3 = torch.empty_like(idx)
        bc3 = torch.empty_like(cnt)
        out3, lse3, _, _ = dsa.sparse_attn_decode_topk(kv, qs, scores, K, w.softmax_scale,
                                                       block_idx=bi3, block_cnt=bc3)
        bc4 = torch.empty_like(cnt)
        out4, lse4, _, _ = dsa.sparse_attn_decode_topk(kv, qs, torch.from_numpy(ref_scores).cuda(),
                                                       K, w.softmax_scale, block_cnt=bc4)
    torch.cuda.synchronize()
    if fused_sel:
        assert np.array_equal(bi3.cpu().numpy(), idx_h) and np.array_equal(bc3.cpu().numpy(), cnt_h), \
            f"{label}: selection inside attention differs from the Top-K kernel's"
        assert np.array_equal(bc4.cpu().numpy(), ref_cnt)
        extra = [(out3, lse3), (out4, lse4)]
    else:
        extra = []

    worst = (0.0, 0.0)
    for qi, r in enumerate(refs):
        bad = parity.check_scores_exact(scores_h[qi], r, maxb)
        assert bad.size == 0, f"{label} q{qi}: scores differ at {bad[:8]}"
        assert np.array_equal(idx2[qi].cpu().numpy(), r["idx"]), f"{label} q{qi}: topk(oracle scores)"
        assert int(cnt2[qi]) == r["cnt"]
        ok, _ = parity.check_indices(idx_h[qi], cnt_h[qi], r, K)
        assert ok, f"{label} q{qi}: idx {idx_h[qi]} cnt {cnt_h[qi]} vs {r['idx']} {r['cnt']}"
        for o, l in [(out_h[qi], lse_h[qi]), (out2[qi].cpu().numpy(), lse2[qi].cpu().numpy())] + \
                [(o_[qi].cpu().numpy(), l_[qi].cpu().numpy()) for o_, l_ in extra]:
            good, a, rel = parity.attn_ok(o, r["out"])
            assert good, f"{label} q{qi}: attention max-abs {a:.3e} max-rel {rel:.3e}"
            la, _ = parity.attn_errors(l, r["lse"])
            assert la <= 1e-3, f"{label} q{qi}: lse max-abs {la:.3e}"
            worst = (max(worst[0], a), max(worst[1], rel))
    _say(f"{label}: {w.num_queries} queries ok; worst attention max-abs {worst[0]:.2e} "
         f"max-rel {worst[1]:.2e}")
    return kv, qs, refs


@pytest.mark.parametrize("kv_layout", [0, 1], ids=["token_major", "head_major"])
@pytest.mark.parametrize("case", SMALL_DECODE_CASES, ids=[str(c["seed"]) for c in SMALL_DECODE_CASES])
def test_small_decode_stages(dsa, case, kv_layout):
    w = workload.small_decode(**case)
    _say(f"small_decode {case} kv_layout {kv_layout}")
    kv, qs, refs = _run_all_stages(dsa, w, f"small_decode[{case['seed']}]", kv_layout)
    # fused entry point: same results
    K = w.top_k
    bi = torch.empty(w.num_queries, K, dtype=torch.int32, device="cuda")
    bc = torch.empty(w.num_queries, dtype=torch.int32, device="cuda")
    out, lse, _, _ = dsa.decode_fused(kv, qs, K, w.softmax_scale, block_idx=bi, block_cnt=bc)
    bi2, bc2 = dsa.index_topk(kv, qs, K)
    torch.cuda.synchronize()
    for qi, r in enumerate(refs):
        assert np.array_equal(bi[qi].cpu().numpy(), r["idx"]) and int(bc[qi]) == r["cnt"]
        assert np.array_equal(bi2[qi].cpu().numpy(), r["idx"]) and int(bc2[qi]) == r["cnt"]
        good, a, rel = parity.attn_ok(out[qi].cpu().numpy(), r["out"])
        assert good, f"fused q{qi}: {a:.3e} {rel:.3e}"


def _tiny_sweep():
    cases = []
    for nb in (1, 2, 3, 7, 64, 65):
        for k in sorted({1, nb - 1, nb, nb + 3}):
            if k >= 1:
                cases.append((nb, k))
    return cases


@pytest.mark.parametrize("nb,top_k", _tiny_sweep(), ids=[f"nb{n}-K{k}" for n, k in _tiny_sweep()])
def test_tiny_sweep_stages(dsa, nb, top_k):
    """Every stage in isolation and the fused entry points, for sequences of
    nb blocks (full, a ragged last block, and one token into the last block)
    and K below, at and above the number of visible blocks."""
    lens = sorted({nb * 64, max(1, nb * 64 - 5), (nb - 1) * 64 + 1})
    w = workload.small_decode(seed=2500 + 7 * nb + top_k, lens=tuple(lens), hq=16, hkv=2, hi=4,
                              di=128, top_k=top_k)
    kv, qs, refs = _run_all_stages(dsa, w, f"sweep nb={nb} K={top_k}")
    bi = torch.empty(w.num_queries, top_k, dtype=torch.int32, device="cuda")
    bc = torch.empty(w.num_queries, dtype=torch.int32, device="cuda")
    out, lse, _, _ = dsa.decode_fused(kv, qs, top_k, w.softmax_scale, block_idx=bi, block_cnt=bc)
    bi2, bc2 = dsa.index_topk(kv, qs, top_k)
    torch.cuda.synchronize()
    for qi, r in enumerate(refs):
        assert np.array_equal(bi[qi].cpu().numpy(), r["idx"]) and int(bc[qi]) == r["cnt"]
        assert np.array_equal(bi2[qi].cpu().numpy(), r["idx"]) and int(bc2[qi]) == r["cnt"]
        good, a, rel = parity.attn_ok(out[qi].cpu().numpy(), r["out"])
        assert good, f"fused q{qi}: {a:.3e} {rel:.3e}"


@pytest.mark.parametrize("seed,count,L,top_k", [(2101, 200, 64 * 20 - 5, 6),
                                                (2102, 130, 64 * 3 + 1, 2),
                                                (2103, 257, 64 * 40, 64)])
@pytest.mark.parametrize("kv_layout", [0, 1], ids=["token_major", "head_major"])
def test_small_prefill_stages(dsa, seed, count, L, top_k, kv_layout):
    w = workload.small_prefill(seed=seed, count=count, L=L, top_k=top_k)
    _say(f"small_prefill seed={seed} count={count} L={L} K={top_k} kv_layout {kv_layout}")
    _run_all_stages(dsa, w, f"small_prefill[{seed}]", kv_layout)


# Batches of 256+ prefill queries of one sequence are scored on the int8
# matrix cores: HI 4 / 8 x dI 64 / 128, several 512-block column ranges, a
# ragged tail of queries and of blocks.
MANY_QUERY_PREFILL_CASES = [
    dict(seed=2111, L=64 * 700 + 13, count=300, hi=8, di=64, top_k=16),
    dict(seed=2112, L=64 * 520, count=256, hi=4, di=64, top_k=8),
    dict(seed=2113, L=64 * 300 - 9, count=333, hi=8, di=128, top_k=24),
]


@pytest.mark.parametrize("case", MANY_QUERY_PREFILL_CASES,
                         ids=[str(c["seed"]) for c in MANY_QUERY_PREFILL_CASES])
def test_many_query_prefill_stages(dsa, case):
    w = workload.small_prefill(**case)
    _say(f"many-query prefill {case}")
    _run_all_stages(dsa, w, f"prefill[{case['seed']}]")


@pytest.mark.parametrize("interleave", [False, True])
def test_multi_sequence_prefill_stages(dsa, interleave):
    # neighbouring queries of different sequences share waves of the scorer
    w = workload.multi_prefill(interleave=interleave)
    _say(f"multi-sequence prefill interleave={interleave} ({w.num_queries} queries)")
    _run_all_stages(dsa, w, f"multi_prefill[{interleave}]")


def _with(base, **fields):
    import copy
    v = copy.copy(base)
    for k, val in fields.items():
        setattr(v, k, val)
    return v


@pytest.mark.parametrize("lens,top_k", [((64 * 40 - 3, 64 * 9), 8),          # fused short-context path
                                         ((64 * 700, 64 * 300 + 5), 16),     # selection inside attention
                                         ((64 * 2600, 64 * 2100), 24)])      # separate Top-K kernel
def test_ties_all_equal_scores(dsa, lens, top_k):
    # every coarse key and scale equal: all visible blocks tie, so the lowest
    # ids win (and the local block)
    w = workload.small_decode(seed=2301, lens=lens, hq=16, hkv=2, hi=8, di=128, top_k=top_k)
    keys = np.repeat(w.idx_keys[:1], w.idx_keys.shape[0], axis=0)
    w = _with(w, idx_keys=keys, idx_scale=np.full_like(w.idx_scale, w.idx_scale[0]))
    _say(f"ties: lens {lens} K={top_k}")
    kv, qs, refs = _run_all_stages(dsa, w, "ties")
    for r in refs:
        n = r["cnt"]
        loc = int(r["idx"][n - 1])
        assert list(r["idx"][:n - 1]) == list(range(min(n - 1, loc)))  # oracle: lowest ids
    out, lse, bi, bc = dsa.decode_fused(kv, qs, top_k, w.softmax_scale,
                                        block_idx=torch.empty(w.num_queries, top_k, dtype=torch.int32,
                                                              device="cuda"),
                                        block_cnt=torch.empty(w.num_queries, dtype=torch.int32,
                                                              device="cuda"))
    torch.cuda.synchronize()
    for qi, r in enumerate(refs):
        assert np.array_equal(bi[qi].cpu().numpy(), r["idx"]) and int(bc[qi]) == r["cnt"]


def test_negative_head_weights(dsa):
    # w of any sign: scores can be negative (ReLU is per head, before the weights)
    w = workload.small_decode(seed=2302, lens=(64 * 300 + 17, 64 * 33), hq=16, hkv=2, hi=8,
                              di=128, top_k=12)
    ww = w.w.copy()
    ww[:, ::2] *= -1.0
    w = _with(w, w=ww)
    _say("negative head weights")
    _run_all_stages(dsa, w, "negative_w")


@pytest.mark.parametrize("lens,top_k", [((64 * 2048, 64 * 2400 - 7, 64 * 100), 2048),
                                         ((64 * 2048 - 5, 64 * 1000), 2048),  # in-attention selection
                                         ((64 * 2048, 64 * 1500 + 3, 64 * 90), 4096),
                                         ((64 * 4200 + 1, 64 * 300), 4096)])
def test_large_top_k(dsa, lens, top_k):
    # large K up to 4096 (the largest accepted): padding below K visible blocks
    # (every path, including the fused ones), a full selection above it
    w = workload.small_decode(seed=2303, lens=lens, hq=8, hkv=1, hi=4, di=64, top_k=top_k)
    _say(f"K = {top_k}, lens {lens}")
    kv, qs, refs = _run_all_stages(dsa, w, "large_top_k")
    nq = w.num_queries
    bi = torch.empty(nq, top_k, dtype=torch.int32, device="cuda")
    bc = torch.empty(nq, dtype=torch.int32, device="cuda")
    out, lse, _, _ = dsa.decode_fused(kv, qs, top_k, w.softmax_scale, block_idx=bi, block_cnt=bc)
    bi2, bc2 = dsa.index_topk(kv, qs, top_k)
    torch.cuda.synchronize()
    for qi, r in enumerate(refs):
        assert np.array_equal(bi[qi].cpu().numpy(), r["idx"]) and int(bc[qi]) == r["cnt"]
        assert np.array_equal(bi2[qi].cpu().numpy(), r["idx"]) and int(bc2[qi]) == r["cnt"]
        good, a, rel = parity.attn_ok(out[qi].cpu().numpy(), r["out"])
        assert good, f"fused q{qi}: {a:.3e} {rel:.3e}"


def test_tiny_decode_config(dsa):
    w = workload.tiny_decode()
    _say("tiny_decode (1 x 4096, K 8)")
    kv, qs, refs = _run_all_stages(dsa, w, "tiny_decode")
    out, lse, _, _ = dsa.decode_fused(kv, qs, w.top_k, w.softmax_scale)
    torch.cuda.synchronize()
    good, a, rel = parity.attn_ok(out[0].cpu().numpy(), refs[0]["out"])
    assert good


def test_device_filler_matches_host_generator(dsa):
    from dsa_synth import gen
    w = workload.small_decode(seed=2001)
    kv, _ = parity.to_device(w)
    k = kv.k_cache.view(torch.int16).cpu().numpy().view(np.uint16)
    v = kv.v_cache.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(k, w.pool_bits(gen.TAG_K))
    assert np.array_equal(v, w.pool_bits(gen.TAG_V))


def test_dense_equivalence_when_k_covers_everything(dsa):
    """Top-K >= visible blocks: the sparse result is dense causal attention."""
    from oracle import dense_attention, bf16_bits_to_f64
    w = workload.small_decode(seed=2011, lens=(64 * 12 - 7, 64 * 5, 33), top_k=16)
    kv, qs = parity.to_device(w)
    out, lse, _, _ = dsa.decode_fused(kv, qs, w.top_k, w.softmax_scale)
    torch.cuda.synchronize()
    for qi in range(w.num_queries):
        s, pos, L = int(w.q_seq[qi]), int(w.q_pos[qi]), int(w.seq_lens[qi])
        ref, _ = dense_attention(bf16_bits_to_f64(w.q_bits[qi]), w.block_table[s], pos, L, 64,
                                 lambda p: bf16_bits_to_f64(w.k_block_bits(p)),
                                 lambda p: bf16_bits_to_f64(w.v_block_bits(p)),
                                 w.softmax_scale, w.num_kv_heads)
        good, a, rel = parity.attn_ok(out[qi].cpu().numpy(), ref)
        assert good, (qi, a, rel)


def test_v_one_gives_one(dsa):
    """Softmax weights sum to one: with V == 1 every output is 1."""
    w = workload.small_decode(seed=2012)
    kv, qs = parity.to_device(w)
    kv.v_cache.fill_(1.0)
    out, _, _, _ = dsa.decode_fused(kv, qs, w.top_k, w.softmax_scale)
    torch.cuda.synchronize()
    assert torch.max(torch.abs(out - 1.0)).item() <= 1e-5


def test_run_to_run_bit_determinism(dsa):
    w = workload.small_decode(seed=2013, hq=64, hkv=8, hi=8, top_k=32,
                              lens=(64 * 300, 64 * 280 + 9, 64 * 77))
    kv, qs = parity.to_device(w)
    a = dsa.decode_fused(kv, qs, w.top_k, w.softmax_scale)[0].clone()
    b = dsa.decode_fused(kv, qs, w.top_k, w.softmax_scale)[0].clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def _random_decode_case(seed):
    rng = np.random.default_rng(seed)
    hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    hi = int(rng.integers(1, 17))
    di = int(rng.choice([64, 128]))
    nseq = int(rng.integers(1, 6))
    # each sequence short, medium or long (ragged tails), independently
    ranges = [(1, 64 * 40), (64 * 200, 64 * 2100), (64 * 2000, 64 * 5000)]
    lens = tuple(int(rng.integers(*ranges[int(rng.integers(0, 3))])) for _ in range(nseq))
    kind = int(rng.integers(0, 5))
    top_k = [1, int(rng.integers(2, 9)), int(rng.integers(9, 65)), int(rng.integers(65, 300)),
             int(rng.integers(300, 700))][kind]
    return dict(seed=3000 + seed, lens=lens, hq=hkv * G, hkv=hkv, hi=hi, di=di, top_k=top_k)


@pytest.mark.parametrize("seed", list(range(10)))
def test_random_decode_configs(dsa, seed):
    case = _random_decode_case(seed)
    w = workload.small_decode(**case)
    _say(f"random decode {case}")
    kv, qs, refs = _run_all_stages(dsa, w, f"random[{seed}]")
    K, nq = w.top_k, w.num_queries
    bi = torch.empty(nq, K, dtype=torch.int32, device="cuda")
    bc = torch.empty(nq, dtype=torch.int32, device="cuda")
    out, lse, _, _ = dsa.decode_fused(kv, qs, K, w.softmax_scale, block_idx=bi, block_cnt=bc)
    bi2, bc2 = dsa.index_topk(kv, qs, K)
    torch.cuda.synchronize()
    for qi, r in enumerate(refs):
        assert np.array_equal(bi[qi].cpu().numpy(), r["idx"]) and int(bc[qi]) == r["cnt"]
        assert np.array_equal(bi2[qi].cpu().numpy(), r["idx"]) and int(bc2[qi]) == r["cnt"]
        good, a, rel = parity.attn_ok(out[qi].cpu().numpy(), r["out"])
        assert good, f"fused q{qi}: {a:.3e} {rel:.3e}"


@pytest.mark.parametrize("nq,hkv,top_k", [(40, 8, 16),   # 320 (query, KV head) workgroups
                                           (24, 8, 32),   # 192 pairs x 2 splits: 384 workgroups
                                           (3, 2, 9)])    # 6 pairs x 3 splits, in-attention scoring
def test_fused_decode_short_context_paths(dsa, nq, hkv, top_k):
    """Short contexts (<= 256 blocks) through the fused entry point: with at
    most one workgroup per CU the attention workgroups score and select their
    blocks themselves; with more, one workgroup per query scores and selects
    first.  Both must give the oracle's indices and attention."""
    rng = np.random.default_rng(nq * 7 + hkv)
    lens = tuple(int(x) for x in rng.integers(1, 64 * 256 + 1, size=nq))
    w = workload.small_decode(seed=2300 + nq, lens=lens, hq=8 * hkv, hkv=hkv, hi=8, di=128,
                              top_k=top_k)
    _say(f"fused short contexts nq={nq} hkv={hkv} K={top_k} maxb={w.block_table.shape[1]}")
    kv, qs = parity.to_device(w)
    bi = torch.empty(nq, top_k, dtype=torch.int32, device="cuda")
    bc = torch.empty(nq, dtype=torch.int32, device="cuda")
    out, lse, _, _ = dsa.decode_fused(kv, qs, top_k, w.softmax_scale, block_idx=bi, block_cnt=bc)
    torch.cuda.synchronize()
    for qi in range(nq):
        r = parity.oracle_query(w, qi)
        assert np.array_equal(bi[qi].cpu().numpy(), r["idx"]) and int(bc[qi]) == r["cnt"], \
            f"q{qi}: {bi[qi].cpu().numpy()[:8]} vs {r['idx'][:8]}"
        good, a, rel = parity.attn_ok(out[qi].cpu().numpy(), r["out"])
        assert good, f"q{qi}: attention {a:.3e} {rel:.3e}"
        la, _ = parity.attn_errors(lse[qi].cpu().numpy(), r["lse"])
        assert la <= 1e-3, f"q{qi}: lse {la:.3e}"


@pytest.mark.parametrize("seed", list(range(4)))
def test_random_prefill_configs(dsa, seed):
    rng = np.random.default_rng(100 + seed)
    hkv = int(rng.choice([1, 2, 8]))
    G = int(rng.choice([1, 4, 8]))
    hi = int(rng.choice([3, 4, 8, 16])) if seed % 2 else int(rng.choice([4, 8]))
    di = int(rng.choice([64, 128]))
    L = int(rng.integers(64 * 50, 64 * 900))
    count = int(rng.integers(256, 400)) if seed % 2 == 0 else int(rng.integers(20, 300))
    top_k = int(rng.choice([1, int(rng.integers(2, 20)), int(rng.integers(20, 120))]))
    w = workload.small_prefill(seed=3100 + seed, L=L, count=count, hq=hkv * G, hkv=hkv, hi=hi,
                               di=di, top_k=top_k)
    _say(f"random prefill L={L} count={count} hq={hkv * G} hkv={hkv} hi={hi} di={di} K={top_k}")
    _run_all_stages(dsa, w, f"random_prefill[{seed}]")


# ---------------------------------------------------------------------------
# blocks of 128, 256 and 512 tokens: every kernel takes the block size at run
# time; attention walks a selected block as 64-token tiles
# ---------------------------------------------------------------------------
BLOCK_SIZES = [128, 256, 512]


@pytest.mark.parametrize("bs", BLOCK_SIZES)
def test_block_size_decode_stages(dsa, bs):
    """Stages and the fused entry (in-attention scoring: short contexts, one
    round of workgroups) on ragged lengths that end mid-tile and mid-block."""
    lens = (bs * 7 - 17, bs * 30, bs * 3 - 1, 1, bs, 65)
    w = workload.small_decode(seed=2700 + bs, lens=lens, hq=16, hkv=2, hi=4, di=128, top_k=5,
                              bs=bs)
    _say(f"block size {bs}: decode stages")
    kv, qs, refs = _run_all_stages(dsa, w, f"decode_bs{bs}")
    K = w.top_k
    bi = torch.empty(w.num_queries, K, dtype=torch.int32, device="cuda")
    bc = torch.empty(w.num_queries, dtype=torch.int32, device="cuda")
    out, _, _, _ = dsa.decode_fused(kv, qs, K, w.softmax_scale, block_idx=bi, block_cnt=bc)
    bi2, bc2 = dsa.index_topk(kv, qs, K)
    torch.cuda.synchronize()
    for qi, r in enumerate(refs):
        assert np.array_equal(bi[qi].cpu().numpy(), r["idx"]) and int(bc[qi]) == r["cnt"]
        assert np.array_equal(bi2[qi].cpu().numpy(), r["idx"]) and int(bc2[qi]) == r["cnt"]
        good, a, rel = parity.attn_ok(out[qi].cpu().numpy(), r["out"])
        assert good, f"fused bs{bs} q{qi}: {a:.3e} {rel:.3e}"


@pytest.mark.parametrize("bs", BLOCK_SIZES)
@pytest.mark.parametrize("nq,hkv,top_k,nb", [
    (40, 8, 6, 200),   # 320 workgroups: fused scoring + selection, then attention
    (2, 2, 16, 200),   # 4 (query, KV head) pairs, each split over its 64-token tiles
    (3, 2, 4, 600),    # past 256 blocks: scoring, then selection inside attention
])
def test_block_size_fused_paths(dsa, bs, nq, hkv, top_k, nb):
    rng = np.random.default_rng(bs + nq)
    lens = tuple(int(x) for x in rng.integers(1, bs * nb, size=nq))
    w = workload.small_decode(seed=2710 + bs + nq, lens=lens, hq=8 * hkv, hkv=hkv, hi=8, di=64,
                              top_k=top_k, bs=bs)
    _say(f"block size {bs}: fused nq={nq} hkv={hkv} K={top_k} maxb={w.block_table.shape[1]}")
    kv, qs = parity.to_device(w)
    bi = torch.empty(nq, top_k, dtype=torch.int32, device="cuda")
    bc = torch.empty(nq, dtype=torch.int32, device="cuda")
    out, lse, _, _ = dsa.decode_fused(kv, qs, top_k, w.softmax_scale, block_idx=bi, block_cnt=bc)
    torch.cuda.synchronize()
    for qi in range(nq):
        r = parity.oracle_query(w, qi)
        assert np.array_equal(bi[qi].cpu().numpy(), r["idx"]) and int(bc[qi]) == r["cnt"]
        good, a, rel = parity.attn_ok(out[qi].cpu().numpy(), r["out"])
        assert good, f"bs{bs} q{qi}: attention {a:.3e} {rel:.3e}"
        la, _ = parity.attn_errors(lse[qi].cpu().numpy(), r["lse"])
        assert la <= 1e-3, f"bs{bs} q{qi}: lse {la:.3e}"


@pytest.mark.parametrize("bs", BLOCK_SIZES)
def test_block_size_prefill_stages(dsa, bs):
    """A prefill chunk of 96 queries (vector scorer) and one of 256 (int8
    matrix-core scorer), both ending inside a block."""
    w = workload.small_prefill(seed=2720 + bs, L=bs * 12 - 5, count=96, top_k=4, bs=bs)
    _say(f"block size {bs}: prefill 96")
    _run_all_stages(dsa, w, f"prefill_bs{bs}")
    w = workload.small_prefill(seed=2730 + bs, L=bs * 9 + 70, count=256, hi=8, di=64, top_k=3,
                               bs=bs)
    _say(f"block size {bs}: prefill 256")
    _run_all_stages(dsa, w, f"prefill256_bs{bs}")


def test_block_size_long_context_candidates(dsa):
    """2100 blocks of 512 tokens (1.07M tokens): the candidate-list path of
    the fused entry and of index_topk."""
    bs, top_k = 512, 6
    lens = (bs * 2100 - 100, bs * 1500 + 3)
    w = workload.small_decode(seed=2740, lens=lens, hq=8, hkv=1, hi=4, di=64, top_k=top_k,
                              bs=bs, extra=2)
    _say(f"block size {bs}: long context maxb={w.block_table.shape[1]}")
    kv, qs = parity.to_device(w)
    bi = torch.empty(2, top_k, dtype=torch.int32, device="cuda")
    bc = torch.empty(2, dtype=torch.int32, device="cuda")
    out, _, _, _ = dsa.decode_fused(kv, qs, top_k, w.softmax_scale, block_idx=bi, block_cnt=bc)
    bi2, bc2 = dsa.index_topk(kv, qs, top_k)
    torch.cuda.synchronize()
    for qi in range(2):
        r = parity.oracle_query(w, qi)
        assert np.array_equal(bi[qi].cpu().numpy(), r["idx"]) and int(bc[qi]) == r["cnt"]
        assert np.array_equal(bi2[qi].cpu().numpy(), r["idx"]) and int(bc2[qi]) == r["cnt"]
        good, a, rel = parity.attn_ok(out[qi].cpu().numpy(), r["out"])
        assert good, f"long bs{bs} q{qi}: {a:.3e} {rel:.3e}"

"""The fused decode captured in a HIP graph: every replay, with eager work and
synchronizations between replays, equals the eager result bit for bit."""

import numpy as np
import pytest

from dsa_synth import workload
from tests import parity

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def test_fused_decode_graph_replays_match_eager():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dynamic_sparse_attention_paged_amd as dsa
    # short contexts (scoring inside attention), mid-length (selection inside
    # attention, split partials), long (per-workgroup candidates and a merge)
    for seed, kw in ((2301, {}), (2302, dict(hq=64, hkv=8, hi=8, top_k=32,
                                            lens=(64 * 300, 64 * 90 + 5, 64 * 2))),
                     (2303, dict(hq=16, hkv=2, hi=8, top_k=16,
                                 lens=(64 * 2600, 64 * 2100 + 3)))):
        w = workload.small_decode(seed=seed, **kw)
        kv, qs = parity.to_device(w)
        other = workload.with_query_seed(w, seed + 50)
        _, qs2 = parity.to_device(other)
        K, nq = w.top_k, w.num_queries
        ws = dsa.make_workspace(dsa._lib.OP_DECODE_FUSED, kv, qs, K)
        out = torch.empty(nq, w.num_q_heads, 128, dtype=torch.float32, device="cuda")
        lse = torch.empty(nq, w.num_q_heads, dtype=torch.float32, device="cuda")
        bi = torch.empty(nq, K, dtype=torch.int32, device="cuda")
        bc = torch.empty(nq, dtype=torch.int32, device="cuda")
        dsa.decode_fused(kv, qs, K, w.softmax_scale, out=out, lse=lse, block_idx=bi,
                         block_cnt=bc, workspace=ws)
        torch.cuda.synchronize()
        ref = [t.clone() for t in (out, lse, bi, bc)]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            dsa.decode_fused(kv, qs, K, w.softmax_scale, out=out, lse=lse, block_idx=bi,
                             block_cnt=bc, workspace=ws)
        for rep in range(4):
            # eager work on other inputs with the same buffers, then a replay
            dsa.decode_fused(kv, qs2, K, w.softmax_scale, out=out, lse=lse, block_idx=bi,
                             block_cnt=bc, workspace=ws)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for a, b in zip((out, lse, bi, bc), ref):
                assert torch.equal(a.view(torch.int32), b.view(torch.int32)), (seed, rep)


def test_calls_on_a_side_stream_match_the_default_stream():
    """Every entry point enqueues on the stream it is given (torch's current
    stream in the binding): the same calls on a side stream give the same bits."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dynamic_sparse_attention_paged_amd as dsa
    w = workload.small_decode(seed=2304, hq=32, hkv=4, hi=8, top_k=12,
                              lens=(64 * 700 + 9, 64 * 40, 64 * 3))
    kv, qs = parity.to_device(w)
    K = w.top_k

    def run():
        sc = dsa.index_score(kv, qs)
        i, c = dsa.topk_blocks(sc, kv, qs, K)
        o, l = dsa.sparse_attn_decode(kv, qs, i, c, K, w.softmax_scale)
        fo, fl, _, _ = dsa.decode_fused(kv, qs, K, w.softmax_scale)
        return sc, i, c, o, l, fo, fl

    ref = run()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        got = run()
    side.synchronize()
    for a, b in zip(got, ref):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_fused_workspace_reused_across_shapes():
    """One workspace serves fused calls of different sizes, split counts and
    paths in any order: each call equals the same call on a fresh workspace."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dynamic_sparse_attention_paged_amd as dsa
    cases = [workload.small_decode(seed=2305, hq=64, hkv=8, hi=8, top_k=32,
                                   lens=(64 * 60, 64 * 33 - 5, 64 * 31)),          # scoring in attention
             workload.small_decode(seed=2306, hq=16, hkv=2, hi=8, top_k=16,
                                   lens=(64 * 2600, 64 * 2100 + 3)),               # candidate lists
             workload.small_decode(seed=2307, hq=32, hkv=4, hi=4, top_k=24,
                                   lens=(64 * 700, 64 * 300 + 1, 64 * 5, 64 * 900))]  # selection
    dev = [parity.to_device(w) for w in cases]
    fresh = []
    for w, (kv, qs) in zip(cases, dev):
        out, lse, _, _ = dsa.decode_fused(kv, qs, w.top_k, w.softmax_scale)
        fresh.append((out.clone(), lse.clone()))
    size = max(dsa.workspace_size(dsa._lib.OP_DECODE_FUSED, kv, qs, w.top_k)
               for w, (kv, qs) in zip(cases, dev))
    ws = torch.zeros(size, dtype=torch.uint8, device="cuda")
    for rnd in range(3):
        for k in ((0, 1, 2), (2, 0, 1), (1, 2, 0))[rnd]:
            w, (kv, qs) = cases[k], dev[k]
            out, lse, _, _ = dsa.decode_fused(kv, qs, w.top_k, w.softmax_scale, workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int32), fresh[k][0].view(torch.int32)), (rnd, k)
            assert torch.equal(lse.view(torch.int32), fresh[k][1].view(torch.int32)), (rnd, k)


def test_fused_prefill_graph_replays_match_eager():
    """The block-inverted prefill (its CSR counters are cleared by a kernel,
    not a memset) replays bit for bit, with eager calls on other queries
    between the replays."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dynamic_sparse_attention_paged_amd as dsa
    w = workload.small_prefill(seed=2880, L=64 * 30 + 7, count=120, hq=16, hkv=2, hi=4, top_k=8)
    kv, qs = parity.to_device(w)
    _, qs2 = parity.to_device(workload.with_query_seed(w, 2881))
    K, nq = w.top_k, w.num_queries
    ws = dsa.make_workspace(dsa._lib.OP_PREFILL_FUSED, kv, qs, K)
    out = torch.empty(nq, w.num_q_heads, 128, dtype=torch.float32, device="cuda")
    lse = torch.empty(nq, w.num_q_heads, dtype=torch.float32, device="cuda")
    bi = torch.empty(nq, K, dtype=torch.int32, device="cuda")
    bc = torch.empty(nq, dtype=torch.int32, device="cuda")

    def call(q):
        dsa.prefill_fused(kv, q, K, w.softmax_scale, out=out, lse=lse, block_idx=bi,
                          block_cnt=bc, workspace=ws)
    call(qs)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, lse, bi, bc)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(qs)
    for rep in range(4):
        call(qs2)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((out, lse, bi, bc), ref):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), rep


def test_moe_grouped_gemm_graph_replays_match_eager():
    """The MXFP4 grouped matmul in both modes (pair grouping, expert slots and,
    for the FP8 mode, the unpack, all inside the graph) replays bit for bit."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import numpy as np
    import dynamic_sparse_attention_paged_amd as dsa
    rng = np.random.default_rng(2890)
    e, n, k, t, slots = 8, 256, 256, 40, 3
    w = dsa.MxExperts(torch.from_numpy(rng.integers(0, 256, (e, n, k // 2), dtype=np.uint8)).cuda(),
                      torch.from_numpy(rng.integers(118, 131, (e, n, k // 32), dtype=np.uint8)).cuda())
    x = torch.randn(t, k, device="cuda").to(torch.bfloat16)
    xc, xs = dsa.mx_quantize(x)
    route = torch.from_numpy(rng.integers(-1, e, (t, slots)).astype(np.int32)).cuda()
    route2 = torch.from_numpy(rng.integers(0, e, (t, slots)).astype(np.int32)).cuda()
    for mode in (dsa._lib.MOE_FP4_DIRECT, dsa._lib.MOE_FP8_WORKSPACE):
        ws = dsa._workspace(dsa.moe_workspace_size(w, t, slots, mode), route.device)
        out = torch.empty(t, slots, n, dtype=torch.float32, device="cuda")
        dsa.moe_grouped_gemm(w, xc, xs, route, mode=mode, out=out, workspace=ws)
        torch.cuda.synchronize()
        ref = out.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            dsa.moe_grouped_gemm(w, xc, xs, route, mode=mode, out=out, workspace=ws)
        for rep in range(4):
            dsa.moe_grouped_gemm(w, xc, xs, route2, mode=mode, out=out, workspace=ws)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref), (mode, rep)


def test_fused_decode_on_any_workspace_contents():
    """The fused decode needs no particular workspace contents: on a workspace
    of random bytes, eager calls and graph replays equal the stage-wise path
    (scores, Top-K, attention) bit for bit, and the selection equals the
    oracle's.  Shapes: 32 sequences x 8 KV heads of 260 blocks (one split,
    selection inside attention) and 4 x 4 (six splits, merged by a second
    launch)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dynamic_sparse_attention_paged_amd as dsa
    cases = [workload.small_decode(seed=2311, hq=64, hkv=8, hi=8, top_k=32,
                                   lens=tuple(64 * 260 - 37 * (s % 5) for s in range(32))),
             workload.small_decode(seed=2312, hq=32, hkv=4, hi=4, top_k=24,
                                   lens=(64 * 700, 64 * 300 + 1, 64 * 5, 64 * 900))]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(2313)
    for w in cases:
        kv, qs = parity.to_device(w)
        K, nq = w.top_k, w.num_queries
        sc = dsa.index_score(kv, qs)
        ri, rc = dsa.topk_blocks(sc, kv, qs, K)
        ro, rl = dsa.sparse_attn_decode(kv, qs, ri, rc, K, w.softmax_scale)
        torch.cuda.synchronize()
        ref = (ro.clone(), rl.clone(), ri.clone(), rc.clone())
        for qi in (0, nq - 1):
            r = parity.oracle_select(w, qi)
            assert np.array_equal(ri[qi].cpu().numpy(), r["idx"]), (w.name, qi)
        nbytes = dsa.workspace_size(dsa._lib.OP_DECODE_FUSED, kv, qs, K)
        ws = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=gen)
        out = torch.empty(nq, w.num_q_heads, 128, dtype=torch.float32, device="cuda")
        lse = torch.empty(nq, w.num_q_heads, dtype=torch.float32, device="cuda")
        bi = torch.empty(nq, K, dtype=torch.int32, device="cuda")
        bc = torch.empty(nq, dtype=torch.int32, device="cuda")

        def check(label):
            for a, b in zip((out, lse, bi, bc), ref):
                assert torch.equal(a.view(torch.int32), b.view(torch.int32)), (w.name, label)

        for rep in range(3):
            dsa.decode_fused(kv, qs, K, w.softmax_scale, out=out, lse=lse, block_idx=bi,
                             block_cnt=bc, workspace=ws)
            torch.cuda.synchronize()
            check(f"eager {rep}")
        ws.random_(0, 256, generator=gen)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            dsa.decode_fused(kv, qs, K, w.softmax_scale, out=out, lse=lse, block_idx=bi,
                             block_cnt=bc, workspace=ws)
        for rep in range(3):
            out.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            check(f"replay {rep}")
        del kv, qs, ws, g
        torch.cuda.empty_cache()

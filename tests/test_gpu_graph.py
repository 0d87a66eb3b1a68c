"""The fused decode captured in a HIP graph: every replay, with eager work and
synchronizations between replays, equals the eager result bit for bit."""

import pytest

from dsa_synth import workload
from tests import parity

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def test_fused_decode_graph_replays_match_eager():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dynamic_sparse_attention_paged_amd as dsa
    for seed, kw in ((2301, {}), (2302, dict(hq=64, hkv=8, hi=8, top_k=32,
                                            lens=(64 * 300, 64 * 90 + 5, 64 * 2)))):
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

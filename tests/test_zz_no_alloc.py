"""The fused decode entry point that allocates nothing
(dsa_sparse_decode_fused_noalloc, scratch in the library's per-GPU array)
against the one that takes a workspace (dsa_sparse_decode_fused): two calls
in a row, the second smaller, bit for bit equal outputs, lse and selections,
through the scoring paths the fused decode takes (short context: scoring in
the attention kernel; mid-length: selection in the attention kernel with
split partials; long context: candidate lists merged by attention).  The
selections are also checked against the oracle."""

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


def _both(dsa, w):
    kv, qs = parity.to_device(w)
    nq, K = w.num_queries, w.top_k
    outs = []
    for fn in (dsa.decode_fused, dsa.decode_fused_noalloc):
        bi = torch.full((nq, K), -7, dtype=torch.int32, device="cuda")
        bc = torch.full((nq,), -7, dtype=torch.int32, device="cuda")
        out, lse, _, _ = fn(kv, qs, K, w.softmax_scale, block_idx=bi, block_cnt=bc)
        torch.cuda.synchronize()
        outs.append((out.cpu(), lse.cpu(), bi.cpu(), bc.cpu()))
    (o1, l1, i1, c1), (o2, l2, i2, c2) = outs
    assert torch.equal(o1, o2) and torch.equal(l1, l2), f"{w.name}: out/lse differ"
    assert torch.equal(i1, i2) and torch.equal(c1, c2), f"{w.name}: selections differ"
    for qi in range(nq):
        r = parity.oracle_select(w, qi)
        assert np.array_equal(i2[qi].numpy(), r["idx"]) and int(c2[qi]) == r["cnt"]
    return o2


@pytest.mark.parametrize("case", [
    # scoring inside attention (short context), then a smaller call
    (dict(seed=4101, lens=(64 * 200 + 5, 64 * 90, 64 * 130 - 1), hq=16, hkv=2, hi=8, top_k=12),
     dict(seed=4102, lens=(64 * 40, 64 * 7 + 3), hq=16, hkv=2, hi=8, top_k=5)),
    # selection inside attention with split partials (mid length), then smaller
    (dict(seed=4103, lens=(64 * 1500 + 9, 64 * 900), hq=64, hkv=8, hi=8, top_k=32),
     dict(seed=4104, lens=(64 * 600,), hq=64, hkv=8, hi=8, top_k=16)),
    # long contexts: per-workgroup candidates merged by attention, then smaller
    (dict(seed=4105, lens=(64 * 9000, 64 * 4100 + 1), hq=16, hkv=2, hi=8, top_k=24),
     dict(seed=4106, lens=(64 * 3000,), hq=16, hkv=2, hi=8, top_k=8)),
], ids=["scored_in_attention", "selected_in_attention", "candidate_lists"])
def test_noalloc_matches_workspace_entry(dsa, case):
    big, small = case
    w1 = workload.small_decode(**big)
    w2 = workload.small_decode(**small)
    _both(dsa, w1)
    _both(dsa, w2)  # the second call is smaller: stale scratch from the first must not leak
    _say(f"noalloc == workspace entry: {w1.name} then {w2.name}")


def test_noalloc_rejects_too_much_scratch(dsa):
    """A decode whose scratch exceeds the library's array is refused before any
    launch, with the size in the message."""
    w = workload.small_decode(seed=4107, lens=(64 * 2,), hq=16, hkv=2, hi=8, top_k=2)
    kv, qs = parity.to_device(w)
    big = dsa.PagedKV(kv.k_cache, kv.v_cache, kv.idx_keys, kv.idx_scale,
                      torch.zeros((4096, 8192), dtype=torch.int32, device="cuda"),
                      torch.full((4096,), 128, dtype=torch.int32, device="cuda"))
    q = dsa.Queries(torch.zeros((4096, 16, 128), dtype=torch.bfloat16, device="cuda"),
                    torch.zeros((4096, 8, 128), dtype=torch.bfloat16, device="cuda"),
                    torch.zeros((4096, 8), dtype=torch.float32, device="cuda"))
    with pytest.raises(dsa.DSAError, match="scratch"):
        dsa.decode_fused_noalloc(big, q, 8, 0.1)

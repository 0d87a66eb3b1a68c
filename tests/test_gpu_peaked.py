"""Peaked softmax: attention queries scaled by 16 and 64, so the logits of one
query head spread over hundreds of units and the softmax weights are nearly
one-hot.  This is the regime where the kernels' base-2 online softmax (running
maximum, rescaling by 2^(m_old - m_new)), the split of each weight into a bf16
high part and a bf16 residual before the P V product, and the merges of wave,
workgroup and per-pick partial states could lose accuracy.  Every output is
compared element by element with the oracle (float64) at the usual bar, for
the decode paths (fused, stage-wise with split partials) and both prefill
paths (per-query kernel, block-inverted fused prefill)."""

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


def _check_all(w, idx, cnt, out, lse, label):
    worst = (0.0, 0.0, 0.0)
    spread = 0.0
    for qi in range(w.num_queries):
        r = parity.oracle_query(w, qi)
        ok, nsw = parity.check_indices(idx[qi], cnt[qi], r, w.top_k)
        assert ok, f"{label} q{qi}: indices differ"
        if nsw:
            r = parity.oracle_query(w, qi, sel_override=idx[qi][:cnt[qi]])
        good, a, rel = parity.attn_ok(out[qi], r["out"])
        assert good, f"{label} q{qi}: attention max-abs {a:.3e} max-rel {rel:.3e}"
        la, _ = parity.attn_errors(lse[qi], r["lse"])
        assert la <= 1e-3, f"{label} q{qi}: lse max-abs {la:.3e}"
        worst = (max(worst[0], a), max(worst[1], rel), max(worst[2], la))
        spread = max(spread, float(np.max(r["lse"])))
    _say(f"{label}: {w.num_queries} queries ok; largest lse {spread:.1f}; worst max-abs "
         f"{worst[0]:.2e} max-rel {worst[1]:.2e} lse {worst[2]:.2e}")


@pytest.mark.parametrize("log2_factor", [4, 6], ids=["qx16", "qx64"])
@pytest.mark.parametrize("kv_layout", [0, 1], ids=["token_major", "head_major"])
def test_peaked_decode(dsa, log2_factor, kv_layout):
    """Fused decode and stage-wise decode (split partials + merge kernel)."""
    w = workload.with_q_scale(workload.small_decode(seed=2301, top_k=8), log2_factor)
    kv, qs = parity.to_device(w, kv_layout=kv_layout)
    K = w.top_k
    bi = torch.empty(w.num_queries, K, dtype=torch.int32, device="cuda")
    bc = torch.empty(w.num_queries, dtype=torch.int32, device="cuda")
    out, lse, _, _ = dsa.decode_fused(kv, qs, K, w.softmax_scale, block_idx=bi, block_cnt=bc)
    torch.cuda.synchronize()
    idx, cnt = bi.cpu().numpy(), bc.cpu().numpy()
    _check_all(w, idx, cnt, out.cpu().numpy(), lse.cpu().numpy(), f"{w.name} fused")
    o2, l2 = dsa.sparse_attn_decode(kv, qs, bi, bc, K, w.softmax_scale)
    torch.cuda.synchronize()
    _check_all(w, idx, cnt, o2.cpu().numpy(), l2.cpu().numpy(), f"{w.name} stage-wise")


@pytest.mark.parametrize("log2_factor", [4, 6], ids=["qx16", "qx64"])
@pytest.mark.parametrize("kv_layout", [0, 1], ids=["token_major", "head_major"])
def test_peaked_prefill(dsa, log2_factor, kv_layout):
    """Per-query prefill kernel and the block-inverted fused prefill."""
    w = workload.with_q_scale(workload.small_prefill(seed=2311, L=64 * 14 - 9, count=120,
                                                     top_k=5), log2_factor)
    kv, qs = parity.to_device(w, kv_layout=kv_layout)
    K = w.top_k
    bi = torch.empty(w.num_queries, K, dtype=torch.int32, device="cuda")
    bc = torch.empty(w.num_queries, dtype=torch.int32, device="cuda")
    out, lse, _, _ = dsa.prefill_fused(kv, qs, K, w.softmax_scale, block_idx=bi, block_cnt=bc)
    torch.cuda.synchronize()
    idx, cnt = bi.cpu().numpy(), bc.cpu().numpy()
    _check_all(w, idx, cnt, out.cpu().numpy(), lse.cpu().numpy(), f"{w.name} fused prefill")
    o2, l2 = dsa.sparse_attn_prefill(kv, qs, bi, bc, K, w.softmax_scale)
    torch.cuda.synchronize()
    _check_all(w, idx, cnt, o2.cpu().numpy(), l2.cpu().numpy(), f"{w.name} per-query prefill")

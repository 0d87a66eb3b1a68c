"""dsa_check_inputs on the GPU: a valid workload passes, and each planted
violation of the device-side contract raises exactly its flag.  Only the
check kernel sees the planted data (it dereferences none of it); no compute
kernel is run on invalid input."""

import sys

import numpy as np
import pytest

from dsa_synth import workload

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


def _views(dsa, w, table=None, seq_lens=None, q_seq=None, q_pos=None):
    def dev(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()
    table = w.block_table if table is None else table
    seq_lens = w.seq_lens if seq_lens is None else seq_lens
    kv = dsa.PagedKV(None, None, dev(w.idx_keys), None, dev(table.astype(np.int32)),
                     dev(seq_lens.astype(np.int32)))
    q_idx = torch.from_numpy(w.q_idx_bits.view(np.int16)).view(torch.bfloat16).cuda()
    qs = dsa.Queries(None, q_idx, None, dev(q_seq), dev(q_pos))  # q_idx only sizes the batch
    return kv, qs


def test_check_decode_contract(dsa):
    w = workload.small_decode(seed=2401, lens=(64 * 9 + 5, 64 * 3, 1, 64 * 12), top_k=4)
    _say("check: decode contract")
    assert dsa.check_inputs(*_views(dsa, w)) == []
    nb = -(-w.seq_lens // 64)
    t = w.block_table.copy()
    t[0, nb[0] - 1] = w.num_blocks  # a block holding tokens names no pool block
    assert dsa.check_inputs(*_views(dsa, w, table=t)) == ["table"]
    t = w.block_table.copy()
    t[1, nb[1]:] = -7  # entries past the sequence's tokens are free
    assert dsa.check_inputs(*_views(dsa, w, table=t)) == []
    L = w.seq_lens.copy()
    L[2] = 0
    assert dsa.check_inputs(*_views(dsa, w, seq_lens=L)) == ["q_pos", "seq_len"]
    L = w.seq_lens.copy()
    L[3] = w.block_table.shape[1] * 64 + 1
    assert dsa.check_inputs(*_views(dsa, w, seq_lens=L)) == ["seq_len"]


def test_check_prefill_positions(dsa):
    w = workload.small_prefill(seed=2402, L=64 * 10 + 3, count=50, top_k=4)
    _say("check: prefill positions")
    assert dsa.check_inputs(*_views(dsa, w, q_seq=w.q_seq, q_pos=w.q_pos)) == []
    s = w.q_seq.copy()
    s[7] = w.num_seqs
    assert dsa.check_inputs(*_views(dsa, w, q_seq=s, q_pos=w.q_pos)) == ["q_seq"]
    p = w.q_pos.copy()
    p[3] = w.seq_lens[0]
    assert dsa.check_inputs(*_views(dsa, w, q_seq=w.q_seq, q_pos=p)) == ["q_pos"]
    p[3] = -1
    assert dsa.check_inputs(*_views(dsa, w, q_seq=w.q_seq, q_pos=p)) == ["q_pos"]


def test_check_block_lists(dsa):
    w = workload.small_decode(seed=2403, lens=(64 * 20, 64 * 9 + 1, 64 * 2), top_k=5)
    _say("check: block lists")
    kv, qs = _views(dsa, w)
    K = w.top_k
    # valid lists: what dsa_topk_blocks produces (local block last, -1 padding)
    idx = np.full((3, K), -1, dtype=np.int32)
    idx[0] = [0, 3, 7, 11, 19]
    idx[1, :4] = [1, 2, 4, 9]
    idx[2, :2] = [0, 1]
    cnt = np.array([5, 4, 2], dtype=np.int32)

    def run(i, c):
        return dsa.check_inputs(kv, qs, torch.from_numpy(i).cuda(), torch.from_numpy(c).cuda(), K)
    assert run(idx, cnt) == []
    bad = []
    x = idx.copy(); x[0, [1, 2]] = x[0, [2, 1]]; bad.append((x, cnt))       # not ascending
    x = idx.copy(); x[1, 3] = 8; bad.append((x, cnt))                        # local block missing
    x = idx.copy(); x[2, 0] = 2; x[2, 1] = 3; bad.append((x, cnt))           # id past the local block
    x = idx.copy(); x[1, 4] = 0; bad.append((x, cnt))                        # padding not -1
    x = idx.copy(); x[0, 1] = x[0, 0]; bad.append((x, cnt))                  # repeated id
    c = cnt.copy(); c[2] = 0; bad.append((idx, c))                           # empty selection
    c = cnt.copy(); c[0] = K + 1; bad.append((idx, c))                       # count above top_k
    for i, (x, c) in enumerate(bad):
        assert run(x, c) == ["block_list"], f"case {i}"

"""Block sizes 128 / 256 / 512 on the write path and the device-data check:
the same oracle comparisons as at 64 tokens per block."""

import numpy as np
import pytest

from oracle.write import kv_write

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dynamic_sparse_attention_paged_amd as m
    m._lib.load()
    return m


def _dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return (t.view(dtype) if dtype is not None else t).cuda()


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("bs", [128, 256, 512])
def test_kv_write_large_blocks(dsa, bs):
    rng = np.random.default_rng(bs)
    P, H = 9, 2
    table = np.array([[3, 7, 1, 0], [8, 4, 2, -1]], dtype=np.int32)
    seq_lens = np.array([3 * bs + 5, 2 * bs + 1], dtype=np.int32)
    k_pool = rng.integers(0, 1 << 16, size=(P, bs, H, 128), dtype=np.uint16)
    v_pool = rng.integers(0, 1 << 16, size=(P, bs, H, 128), dtype=np.uint16)
    tok_seq = np.array([0, 0, 0, 1, 1, 1, 1], np.int32)
    tok_pos = np.array([0, bs - 1, 3 * bs + 4, bs, 2 * bs, 3 * bs, 2 * bs + 5], np.int32)
    ok = [0, 1, 2, 3, 4, 6]   # position 3 bs of sequence 1 falls on table entry -1: skipped
    n = tok_seq.size
    k_new = rng.integers(0, 1 << 16, size=(n, H, 128), dtype=np.uint16)
    v_new = rng.integers(0, 1 << 16, size=(n, H, 128), dtype=np.uint16)
    kd = _dev(k_pool.view(np.int16), torch.bfloat16)
    vd = _dev(v_pool.view(np.int16), torch.bfloat16)
    kv = dsa.PagedKV(kd, vd, None, None, _dev(table), _dev(seq_lens))
    dsa.kv_write(kv, _dev(k_new.view(np.int16), torch.bfloat16),
                 _dev(v_new.view(np.int16), torch.bfloat16), _dev(tok_seq), _dev(tok_pos))
    torch.cuda.synchronize()
    want_k, want_v = kv_write(k_pool, v_pool, table, seq_lens, tok_seq[ok], tok_pos[ok],
                              k_new[ok], v_new[ok], bs)
    assert np.array_equal(_bits(kd), want_k) and np.array_equal(_bits(vd), want_v)


@pytest.mark.parametrize("bs", [128, 512])
def test_check_inputs_large_blocks(dsa, bs):
    table = np.array([[2, 0, 1], [3, -1, -1]], dtype=np.int32)
    lens = np.array([2 * bs + 1, bs], dtype=np.int32)
    kv = dsa.PagedKV(None, None, _dev(np.zeros((4, 64), np.uint8)), None, _dev(table),
                     _dev(lens), block_size=bs)
    q_pos = np.array([2 * bs, bs - 1], np.int32)
    qs = dsa.Queries(None, None, None, _dev(np.array([0, 1], np.int32)), _dev(q_pos))
    idx = _dev(np.array([[0, 2], [0, -1]], np.int32))
    cnt = _dev(np.array([2, 1], np.int32))
    assert dsa.check_inputs(kv, qs, idx, cnt, 2) == []
    # 2 bs + 1 tokens fit three blocks of bs; one more block's worth does not
    # fit the table row; position 2 bs lies in block 2, so block 1 alone is
    # not the local block
    bad_lens = _dev(np.array([3 * bs + 1, bs], np.int32))
    kv2 = dsa.PagedKV(None, None, kv.idx_keys, None, kv.block_table, bad_lens, block_size=bs)
    assert dsa.check_inputs(kv2, qs, idx, cnt, 2) == ["seq_len"]
    idx_bad = _dev(np.array([[0, 1], [0, -1]], np.int32))
    assert dsa.check_inputs(kv, qs, idx_bad, cnt, 2) == ["block_list"]

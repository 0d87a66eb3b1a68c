"""GPU parity of the paged write path (dsa_kv_write, dsa_index_key_write)
against the oracle (oracle/write.py), bit for bit, and a rebuild of a whole
synthetic cache through the write path that the attention tests read."""

import sys

import numpy as np
import pytest

from dsa_synth import gen, workload
from oracle.write import kv_write, quantize_coarse_key
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


def _dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return (t.view(dtype) if dtype is not None else t).cuda()


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def test_kv_write_matches_oracle(dsa):
    rng = np.random.default_rng(11)
    P, H = 20, 2
    table = np.array([[3, 7, 1, 0, 12], [9, 4, 11, 2, -1], [5, 6, 8, 10, 13]], dtype=np.int32)
    seq_lens = np.array([300, 250, 64 * 5], dtype=np.int32)
    k_pool = rng.integers(0, 1 << 16, size=(P, 64, H, 128), dtype=np.uint16)
    v_pool = rng.integers(0, 1 << 16, size=(P, 64, H, 128), dtype=np.uint16)
    cases = [
        (None, None, 3),  # decode: the newest token of each sequence
        (np.array([0, 0, 1, 1, 2, 2, 0], np.int32), np.array([0, 63, 64, 249, 128, 319, 200], np.int32), 7),
    ]
    for tok_seq, tok_pos, n in cases:
        kd, vd = _dev(k_pool.view(np.int16), torch.bfloat16), _dev(v_pool.view(np.int16), torch.bfloat16)
        kv = dsa.PagedKV(kd, vd, None, None, _dev(table), _dev(seq_lens))
        k_new = rng.integers(0, 1 << 16, size=(n, H, 128), dtype=np.uint16)
        v_new = rng.integers(0, 1 << 16, size=(n, H, 128), dtype=np.uint16)
        dsa.kv_write(kv, _dev(k_new.view(np.int16), torch.bfloat16),
                     _dev(v_new.view(np.int16), torch.bfloat16),
                     None if tok_seq is None else _dev(tok_seq),
                     None if tok_pos is None else _dev(tok_pos))
        torch.cuda.synchronize()
        want_k, want_v = kv_write(k_pool, v_pool, table, seq_lens, tok_seq, tok_pos, k_new, v_new, 64)
        assert np.array_equal(_bits(kd), want_k) and np.array_equal(_bits(vd), want_v), n
    # targets outside the table row or the pool are skipped
    kd, vd = _dev(k_pool.view(np.int16), torch.bfloat16), _dev(v_pool.view(np.int16), torch.bfloat16)
    kv = dsa.PagedKV(kd, vd, None, None, _dev(table), _dev(seq_lens))
    tok_seq = np.array([1, 0, 2, 5, 0], np.int32)          # block -1; ok; past the row; no sequence; ok
    tok_pos = np.array([300, 5, 64 * 5, 0, 70], np.int32)
    k_new = rng.integers(0, 1 << 16, size=(5, H, 128), dtype=np.uint16)
    dsa.kv_write(kv, _dev(k_new.view(np.int16), torch.bfloat16), _dev(k_new.view(np.int16), torch.bfloat16),
                 _dev(tok_seq), _dev(tok_pos))
    torch.cuda.synchronize()
    ok = [1, 4]
    want_k, _ = kv_write(k_pool, v_pool, table, seq_lens, tok_seq[ok], tok_pos[ok], k_new[ok],
                         k_new[ok], 64)
    assert np.array_equal(_bits(kd), want_k)


@pytest.mark.parametrize("bs", [64, 256])
def test_kv_write_head_major_matches_oracle(dsa, bs):
    """The same writes into a head-major pool ([P, Hkv, bs, 128]) land where
    the oracle's token-major result, transposed, puts them."""
    rng = np.random.default_rng(12 + bs)
    P, H = 9, 3
    table = np.array([[3, 7, 1], [0, 4, 8], [5, 6, 2]], dtype=np.int32)
    seq_lens = np.array([bs * 2 + 5, bs * 3, 17], dtype=np.int32)
    k_pool = rng.integers(0, 1 << 16, size=(P, bs, H, 128), dtype=np.uint16)
    v_pool = rng.integers(0, 1 << 16, size=(P, bs, H, 128), dtype=np.uint16)
    hm = lambda a: np.ascontiguousarray(a.transpose(0, 2, 1, 3))
    for tok_seq, tok_pos, n in ((None, None, 3),
                                (np.array([0, 1, 1, 2, 0], np.int32),
                                 np.array([0, bs - 1, bs * 3 - 1, 16, bs + 3], np.int32), 5)):
        kd = _dev(hm(k_pool).view(np.int16), torch.bfloat16)
        vd = _dev(hm(v_pool).view(np.int16), torch.bfloat16)
        kv = dsa.PagedKV(kd, vd, None, None, _dev(table), _dev(seq_lens),
                         kv_layout=dsa.KV_HEAD_MAJOR)
        assert kv.tokens_per_block == bs and kv.kv_heads == H
        k_new = rng.integers(0, 1 << 16, size=(n, H, 128), dtype=np.uint16)
        v_new = rng.integers(0, 1 << 16, size=(n, H, 128), dtype=np.uint16)
        dsa.kv_write(kv, _dev(k_new.view(np.int16), torch.bfloat16),
                     _dev(v_new.view(np.int16), torch.bfloat16),
                     None if tok_seq is None else _dev(tok_seq),
                     None if tok_pos is None else _dev(tok_pos))
        torch.cuda.synchronize()
        want_k, want_v = kv_write(k_pool, v_pool, table, seq_lens, tok_seq, tok_pos, k_new, v_new, bs)
        assert np.array_equal(_bits(kd), hm(want_k)) and np.array_equal(_bits(vd), hm(want_v)), n


@pytest.mark.parametrize("di", [64, 128])
def test_index_key_write_matches_oracle(dsa, di):
    rng = np.random.default_rng(12 + di)
    P = 300
    keys = rng.integers(0, 256, size=(P, di), dtype=np.uint8)
    scale = rng.random(P, dtype=np.float32)
    n = 200
    x = (rng.standard_normal((n, di)) * (10.0 ** rng.uniform(-5, 5, size=(n, 1)))).astype(np.float32)
    x[0] = 0.0                                           # zero vector
    x[1] = rng.integers(-224, 224, size=di) + 0.5        # with 448 below: ks = 1, many halves
    x[1, 0] = 448.0
    x[2] = np.where(rng.random(di) < 0.5, 17.0, 19.0)    # ties to even after scaling
    x[2, 3] = -448.0
    x[3] = -0.0
    ids = rng.permutation(P)[:n].astype(np.int32)
    ids[5] = P + 3                                       # outside the pool: skipped
    ids[6] = -1
    kd, sd = _dev(keys), _dev(scale)
    kv = dsa.PagedKV(None, None, kd, sd, _dev(np.zeros((1, 1), np.int32)), _dev(np.ones(1, np.int32)))
    dsa.index_key_write(kv, _dev(ids), _dev(x))
    torch.cuda.synchronize()
    got_k, got_s = kd.cpu().numpy(), sd.cpu().numpy()
    want_k, want_s = keys.copy(), scale.copy()
    for i in range(n):
        if 0 <= ids[i] < P:
            want_k[ids[i]], want_s[ids[i]] = quantize_coarse_key(x[i])
    bad = np.argwhere(got_k != want_k)
    assert bad.size == 0, f"codes differ at {bad[:5].tolist()}"
    assert np.array_equal(got_s.view(np.uint32), want_s.view(np.uint32))


def test_write_path_rebuilds_the_synthetic_cache(dsa):
    """Writing every token's K/V and every block's coarse key (the generator's
    float keys) through the library reproduces the cache the attention tests
    use: K/V rows and the generator's E4M3 codes (PyTorch's conversion) alike."""
    w = workload.small_decode(seed=2601, lens=(64 * 9 + 5, 64 * 3, 1, 64 * 12), hq=16, hkv=2,
                              hi=4, di=128, top_k=4)
    _say(f"rebuild {w.name}: pool {w.num_blocks} blocks")
    ref_kv, _ = parity.to_device(w)
    shape = (w.num_blocks, 64, w.num_kv_heads, 128)
    kd = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    vd = torch.zeros_like(kd)
    keys = torch.zeros((w.num_blocks, w.idx_dim), dtype=torch.uint8, device="cuda")
    scale = torch.zeros(w.num_blocks, dtype=torch.float32, device="cuda")
    kv = dsa.PagedKV(kd, vd, keys, scale, ref_kv.block_table, ref_kv.seq_lens)
    tok_seq, tok_pos, k_rows, v_rows = [], [], [], []
    for s, L in enumerate(w.seq_lens):
        for pos in range(int(L)):
            p = int(w.block_table[s][pos // 64])
            tok_seq.append(s)
            tok_pos.append(pos)
            k_rows.append(w.k_block_bits(p)[pos % 64])
            v_rows.append(w.v_block_bits(p)[pos % 64])
    k_new = np.stack(k_rows).astype(np.uint16)
    v_new = np.stack(v_rows).astype(np.uint16)
    dsa.kv_write(kv, _dev(k_new.view(np.int16), torch.bfloat16), _dev(v_new.view(np.int16), torch.bfloat16),
                 _dev(np.array(tok_seq, np.int32)), _dev(np.array(tok_pos, np.int32)))
    coarse = gen.f32_normal_tensor(w.seed, gen.TAG_IDXKEY, (w.num_blocks, w.idx_dim)).astype(np.float32)
    dsa.index_key_write(kv, _dev(np.arange(w.num_blocks, dtype=np.int32)), _dev(coarse))
    torch.cuda.synchronize()
    got_k, got_v = _bits(kd), _bits(vd)
    ref_k, ref_v = _bits(ref_kv.k_cache), _bits(ref_kv.v_cache)
    for s, pos in zip(tok_seq, tok_pos):
        p, t = int(w.block_table[s][pos // 64]), pos % 64
        assert np.array_equal(got_k[p, t], ref_k[p, t]) and np.array_equal(got_v[p, t], ref_v[p, t])
    assert np.array_equal(keys.cpu().numpy(), w.idx_keys)
    assert np.array_equal(scale.cpu().numpy().view(np.uint32), w.idx_scale.view(np.uint32))

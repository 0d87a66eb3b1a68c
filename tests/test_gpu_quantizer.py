"""GPU sweep of the query quantizer against the oracle's E4M3 encoder.

Every finite bf16 value x with |x| <= 448 goes through the library's scoring
kernels once.  A query row holds 448 in dimension 0, so its power-of-two
scale is 1, and test values in the other dimensions.  Each block's coarse key
is +1 or -1 in a single dimension, with scale 1 and weight 1, so

    S[q, j] = max(0, +-value(E4M3(x)))    exactly,

and the returned fp32 scores must equal the oracle's encode-then-decode of
every x, bit for bit (ties to even, subnormals, the 448 edge, signed zero
through the ReLU).  The decode layout runs the float64 scorer; the
many-query layout (sequence and position given, 256+ queries, 4 indexer
heads) runs the int8 matrix-core scorer.
"""

import sys

import numpy as np
import pytest

from oracle import e4m3_decode, e4m3_encode, bf16_bits_to_f64

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

BF16_448 = 0x43E0  # bf16 bits of 448.0


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


def _sweep_values():
    mags = np.arange(0, BF16_448 + 1, dtype=np.uint32)  # +0 .. 448, every bf16 in between
    return np.concatenate([mags, mags | 0x8000]).astype(np.uint16)


@pytest.mark.parametrize("layout,di", [("decode", 64), ("decode", 128),
                                       ("many_query", 64), ("many_query", 128)])
def test_quantizer_sweep_all_bf16(dsa, layout, di):
    vals = _sweep_values()
    per_row = di - 1
    nq = -(-vals.size // per_row)
    padded = np.zeros(nq * per_row, dtype=np.uint16)
    padded[:vals.size] = vals
    hi = 1 if layout == "decode" else 4
    q_idx = np.zeros((nq, hi, di), dtype=np.uint16)
    q_idx[:, 0, 0] = BF16_448
    q_idx[:, 0, 1:] = padded.reshape(nq, per_row)
    w = np.zeros((nq, hi), dtype=np.float32)
    w[:, 0] = 1.0
    # blocks 0 .. di-2: +1 in dim j+1; blocks di-1 .. 2di-3: -1 in dim j-di+2; then the local block
    nb = 2 * per_row + 1
    keys = np.zeros((nb, di), dtype=np.uint8)
    for j in range(per_row):
        keys[j, j + 1] = 0x38
        keys[per_row + j, j + 1] = 0xB8
    scale = np.ones(nb, dtype=np.float32)
    L = nb * 64
    if layout == "decode":
        seq_lens = np.full(nq, L, dtype=np.int32)
        table = np.tile(np.arange(nb, dtype=np.int32), (nq, 1))
        q_seq = q_pos = None
    else:
        assert nq >= 256
        seq_lens = np.array([L], dtype=np.int32)
        table = np.arange(nb, dtype=np.int32)[None, :]
        q_seq = np.zeros(nq, dtype=np.int32)
        q_pos = np.full(nq, L - 1, dtype=np.int32)
    _say(f"quantizer sweep {layout} dI={di}: {vals.size} values in {nq} queries x {nb} blocks")

    def dev(a, dtype=None):
        if a is None:
            return None
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t.view(dtype) if dtype is not None else t).cuda()

    kv = dsa.PagedKV(None, None, dev(keys), dev(scale), dev(table), dev(seq_lens))
    qs = dsa.Queries(None, dev(q_idx.view(np.int16), torch.bfloat16), dev(w), dev(q_seq),
                     dev(q_pos))
    scores = dsa.index_score(kv, qs).cpu().numpy()

    x = bf16_bits_to_f64(padded)
    qv = e4m3_decode(e4m3_encode(x)).reshape(nq, per_row)
    want = np.zeros((nq, nb), dtype=np.float32)
    # the ReLU gives +0 for every non-positive product (never -0)
    want[:, :per_row] = np.where(qv > 0.0, qv, 0.0).astype(np.float32)
    want[:, per_row:2 * per_row] = np.where(-qv > 0.0, -qv, 0.0).astype(np.float32)
    got = scores.view(np.uint32)
    bad = np.argwhere(got != want.view(np.uint32))
    if bad.size:
        q, j = bad[0]
        d = j % per_row + 1
        _say(f"first mismatch: query {q} block {j} value bits {q_idx[q, 0, d]:#06x} "
             f"got {scores[q, j]!r} want {want[q, j]!r}")
    assert bad.size == 0, f"{len(bad)} scores differ from the oracle's encode/decode"

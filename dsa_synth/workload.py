"""Synthetic workloads shaped like the pages' long-context decode / prefill cases.

Only input data lives here (shapes, seeded values, block tables, lengths);
none of the method's arithmetic.  Five named workloads mirror the five
benchmark configurations (tiny decode, batched decode, ragged decode,
chunked prefill, million-token decode); the small ones are for parity tests.

Recipe (all from ``gen.py``'s counter-based streams, seed = 1000 + number):
  * Q, K, V, q_idx: standard normal rounded to bf16;
  * w: uniform (0, 1) per (query, indexer head), float32;
  * coarse indexer keys: a float32 normal vector per block, with per-block
    scale ks = max|k| / 448 and E4M3 codes of k / ks (PyTorch's float8_e4m3fn
    conversion); the ragged workload first adds 2 * u_s to 5% of each
    sequence's blocks, u_s the unit vector along sum_h w[s,h] q_idx[s,h,:];
  * block tables: seeded permutations of the pool (interleaved across
    sequences for the batched workload, one shared pool cut in order for the
    ragged one);
  * ragged lengths: nb_s = 128 + floor(U * 1921) blocks, L_s = 64 nb_s.
"""

from dataclasses import dataclass, field
import math

import numpy as np

from . import gen


@dataclass
class Workload:
    name: str
    seed: int
    block_size: int
    num_kv_heads: int
    head_dim: int
    num_q_heads: int
    idx_heads: int
    idx_dim: int
    top_k: int
    num_blocks: int
    seq_lens: np.ndarray          # int32 [B]
    block_table: np.ndarray       # int32 [B, max_blocks]
    q_seq: np.ndarray             # int32 [Nq]
    q_pos: np.ndarray             # int32 [Nq]
    decode: bool                  # True: query i belongs to sequence i at L_i - 1
    q_bits: np.ndarray            # uint16 (bf16) [Nq, Hq, d]
    q_idx_bits: np.ndarray        # uint16 (bf16) [Nq, HI, dI]
    w: np.ndarray                 # float32 [Nq, HI]
    idx_keys: np.ndarray          # uint8 [P, dI]
    idx_scale: np.ndarray         # float32 [P]
    softmax_scale: float = float(np.float32(1.0 / math.sqrt(128.0)))
    meta: dict = field(default_factory=dict)

    @property
    def num_queries(self):
        return int(self.q_pos.shape[0])

    @property
    def num_seqs(self):
        return int(self.seq_lens.shape[0])

    @property
    def pool_elems(self):
        return self.num_blocks * self.block_size * self.num_kv_heads * self.head_dim

    def _block_shape(self):
        return (self.block_size, self.num_kv_heads, self.head_dim)

    def k_block_bits(self, p):
        n = self.block_size * self.num_kv_heads * self.head_dim
        return gen.bf16_normal_tensor(self.seed, gen.TAG_K, self._block_shape(), offset=p * n)

    def v_block_bits(self, p):
        n = self.block_size * self.num_kv_heads * self.head_dim
        return gen.bf16_normal_tensor(self.seed, gen.TAG_V, self._block_shape(), offset=p * n)

    def pool_bits(self, tag):
        """Whole K (tag 2) or V (tag 3) pool as bf16 bits; small workloads only."""
        if self.pool_elems > (1 << 28):
            raise MemoryError("pool too large to build on the host; use the device filler")
        return gen.bf16_normal_tensor(self.seed, tag, (self.num_blocks,) + self._block_shape())


def _coarse_keys(seed, num_blocks, idx_dim, plant=None):
    """E4M3 codes + float32 scale of one coarse key per physical block."""
    import torch

    k = gen.f32_normal_tensor(seed, gen.TAG_IDXKEY, (num_blocks, idx_dim)).astype(np.float32)
    if plant is not None:
        rows, vecs = plant
        k[rows] = (k[rows].astype(np.float64) + vecs).astype(np.float32)
    amax = np.abs(k).max(axis=1)
    amax = np.where(amax == 0, np.float32(1.0), amax).astype(np.float32)
    ks = (amax / np.float32(448.0)).astype(np.float32)
    x = np.clip(k / ks[:, None], -448.0, 448.0).astype(np.float32)
    codes = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    return codes, ks


def _queries(seed, nq, hq, d, hi, di):
    q = gen.bf16_normal_tensor(seed, gen.TAG_Q, (nq, hq, d))
    qi = gen.bf16_normal_tensor(seed, gen.TAG_QIDX, (nq, hi, di))
    w = gen.uniform_tensor(seed, gen.TAG_W, (nq, hi)).astype(np.float32)
    return q, qi, w


def build(name, seed, seq_lens, table, num_blocks, hq, hkv, hi, di, top_k,
          prefill=None, plant_frac=0.0, bs=64, d=128, meta=None):
    """Assemble a workload.

    seq_lens: tokens per sequence; table: int [B, max_blocks] physical ids;
    prefill: None for decode (one query per sequence at L-1), else
    (seq, first_pos, count) for a chunk of consecutive query positions, or a
    list of such chunks (their queries concatenated in order), or a pair of
    int arrays (q_seq, q_pos) giving every query's sequence and position.
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    table = np.asarray(table, dtype=np.int32)
    if prefill is None:
        q_seq = np.arange(seq_lens.size, dtype=np.int32)
        q_pos = (seq_lens - 1).astype(np.int32)
    elif isinstance(prefill, tuple) and len(prefill) == 2:
        q_seq = np.asarray(prefill[0], dtype=np.int32)
        q_pos = np.asarray(prefill[1], dtype=np.int32)
    else:
        chunks = [prefill] if isinstance(prefill, tuple) else list(prefill)
        q_seq = np.concatenate([np.full(c, s, dtype=np.int32) for s, _, c in chunks])
        q_pos = np.concatenate([np.arange(f, f + c, dtype=np.int32) for _, f, c in chunks])
    nq = q_pos.size
    q, qi, w = _queries(seed, nq, hq, d, hi, di)
    plant = None
    if plant_frac > 0:
        rows, vecs = [], []
        qif = gen.bf16_bits_to_f32(qi).astype(np.float64)
        for s in range(seq_lens.size):
            # decode workloads only: query s belongs to sequence s
            u = (w[s].astype(np.float64)[:, None] * qif[s]).sum(axis=0)
            u /= np.linalg.norm(u)
            nb = -(-int(seq_lens[s]) // bs)
            m = int(round(plant_frac * nb))
            h = gen.hash_at(seed, gen.TAG_PLANT,
                            np.arange(nb, dtype=np.uint64) + np.uint64(s << 24))
            js = np.argsort(h, kind="stable")[:m]
            for j in js:
                rows.append(int(table[s, j]))
                vecs.append(2.0 * u)
        plant = (np.asarray(rows, dtype=np.int64), np.asarray(vecs))
    keys, ks = _coarse_keys(seed, num_blocks, di, plant)
    return Workload(name=name, seed=seed, block_size=bs, num_kv_heads=hkv, head_dim=d,
                    num_q_heads=hq, idx_heads=hi, idx_dim=di, top_k=top_k,
                    num_blocks=num_blocks, seq_lens=seq_lens, block_table=table,
                    q_seq=q_seq, q_pos=q_pos, decode=prefill is None, q_bits=q,
                    q_idx_bits=qi, w=w, idx_keys=keys, idx_scale=ks, meta=meta or {})


# ---------------------------------------------------------------------------
# the five benchmark-shaped workloads
# ---------------------------------------------------------------------------
def tiny_decode():
    seed = 1001
    perm = gen.permutation(seed, gen.TAG_TABLE, 64)
    return build("tiny_decode_1x4096_k8", seed, [4096], perm[None, :], 64,
                 hq=8, hkv=1, hi=4, di=64, top_k=8)


def batched_decode():
    seed = 1002
    B, nb = 32, 512
    perm = gen.permutation(seed, gen.TAG_TABLE, B * nb)
    j = np.arange(nb)
    table = np.stack([perm[j * B + s] for s in range(B)])
    return build("batched_decode_32x32768_k32", seed, [nb * 64] * B, table, B * nb,
                 hq=64, hkv=8, hi=8, di=128, top_k=32)


def batched_decode_blocks(bs):
    """The batched decode shape (32 sequences of 32768 tokens) with blocks of
    bs tokens and top_k = 2048 / bs, so that every query attends the same
    2048 tokens' worth of blocks at any block size."""
    seed = 1002
    B, nb = 32, 32768 // bs
    perm = gen.permutation(seed, gen.TAG_TABLE, B * nb)
    j = np.arange(nb)
    table = np.stack([perm[j * B + s] for s in range(B)])
    return build(f"batched_decode_32x32768_bs{bs}_k{2048 // bs}", seed, [32768] * B, table,
                 B * nb, hq=64, hkv=8, hi=8, di=128, top_k=2048 // bs, bs=bs)


def ragged_decode():
    seed = 1003
    B = 128
    u = gen.uniform_tensor(seed, gen.TAG_LENS, (B,))
    nbs = (128 + np.floor(u * 1921)).astype(np.int64)
    P = int(nbs.sum())
    perm = gen.permutation(seed, gen.TAG_TABLE, P)
    table = np.zeros((B, int(nbs.max())), dtype=np.int64)
    off = 0
    for s in range(B):
        table[s, : nbs[s]] = perm[off: off + nbs[s]]
        off += nbs[s]
    return build("ragged_decode_128xU[8k,128k]_k64", seed, (nbs * 64).tolist(), table, P,
                 hq=64, hkv=8, hi=8, di=128, top_k=64, plant_frac=0.05)


def chunked_prefill():
    seed = 1004
    nb = 2048
    perm = gen.permutation(seed, gen.TAG_TABLE, nb)
    return build("chunked_prefill_8192q_at_122880_ctx131072_k64", seed, [nb * 64],
                 perm[None, :], nb, hq=64, hkv=8, hi=8, di=128, top_k=64,
                 prefill=(0, 122880, 8192))


def million_decode():
    seed = 1005
    B, nb = 4, 16384
    perm = gen.permutation(seed, gen.TAG_TABLE, B * nb)
    table = perm.reshape(B, nb)
    return build("million_decode_4x1048576_k32", seed, [nb * 64] * B, table, B * nb,
                 hq=64, hkv=8, hi=8, di=128, top_k=32)


NAMED = {
    1: tiny_decode,
    2: batched_decode,
    3: ragged_decode,
    4: chunked_prefill,
    5: million_decode,
}


# ---------------------------------------------------------------------------
# small workloads for parity tests
# ---------------------------------------------------------------------------
def small_decode(seed=2001, lens=(64 * 7 - 17, 64 * 65, 64 * 130 - 63, 64, 1),
                 hq=16, hkv=2, hi=4, di=128, top_k=8, extra=5, bs=64):
    """Ragged decode over a shared permuted pool with a few unused blocks."""
    nbs = [-(-L // bs) for L in lens]
    P = sum(nbs) + extra
    perm = gen.permutation(seed, gen.TAG_TABLE, P)
    table = np.zeros((len(lens), max(nbs)), dtype=np.int64)
    off = 0
    for s, nb in enumerate(nbs):
        table[s, :nb] = perm[off: off + nb]
        off += nb
    name = f"small_decode_s{seed}" + ("" if bs == 64 else f"_bs{bs}")
    return build(name, seed, list(lens), table, P, hq=hq, hkv=hkv, hi=hi, di=di,
                 top_k=top_k, bs=bs)


def shared_pool_decode(seed=2301, n_seqs=32, L=64 * 2100 + 5, pool_blocks=2300, hq=64, hkv=8,
                       hi=8, di=128, top_k=32):
    """Decode of n_seqs long sequences whose block tables all map into one
    pool of pool_blocks blocks, each sequence through a permutation of its own
    (blocks shared between sequences, as with a common prefix): a wide batch
    without a pool per sequence."""
    nb = -(-L // 64)
    assert nb <= pool_blocks
    table = np.zeros((n_seqs, nb), dtype=np.int64)
    for s in range(n_seqs):
        table[s] = gen.permutation(seed + 7 * s, gen.TAG_TABLE, pool_blocks)[:nb]
    return build(f"shared_pool_decode_s{seed}", seed, [L] * n_seqs, table, pool_blocks, hq=hq,
                 hkv=hkv, hi=hi, di=di, top_k=top_k)


def small_prefill(seed=2101, L=64 * 20 - 5, count=200, hq=16, hkv=2, hi=4, di=128,
                  top_k=6, extra=3, bs=64):
    nb = -(-L // bs)
    P = nb + extra
    perm = gen.permutation(seed, gen.TAG_TABLE, P)
    name = f"small_prefill_s{seed}" + ("" if bs == 64 else f"_bs{bs}")
    return build(name, seed, [L], perm[None, :nb], P, hq=hq, hkv=hkv, hi=hi, di=di,
                 top_k=top_k, prefill=(0, L - count, count), bs=bs)


def multi_prefill(seed=2121, lens=(64 * 30 + 7, 64 * 12, 64 * 21 - 1), counts=(120, 90, 70),
                  interleave=False, hq=16, hkv=2, hi=8, di=128, top_k=8):
    """Prefill chunks of several sequences in one batch: the last counts[s]
    positions of sequence s, concatenated, or with ``interleave`` taken
    round-robin across the sequences (so neighbouring queries differ in
    sequence)."""
    lens = [int(x) for x in lens]
    nbs = [-(-L // 64) for L in lens]
    maxb = max(nbs)
    P = sum(nbs) + 5
    perm = gen.permutation(seed, gen.TAG_TABLE, P)
    table = np.zeros((len(lens), maxb), dtype=np.int32)
    o = 0
    for s, nb in enumerate(nbs):
        table[s, :nb] = perm[o:o + nb]
        o += nb
    per = [np.arange(L - c, L, dtype=np.int32) for L, c in zip(lens, counts)]
    if interleave:
        qs, qp = [], []
        for i in range(max(counts)):
            for s, pos in enumerate(per):
                if i < len(pos):
                    qs.append(s)
                    qp.append(int(pos[i]))
        pre = (np.asarray(qs), np.asarray(qp))
    else:
        pre = [(s, L - c, c) for s, (L, c) in enumerate(zip(lens, counts))]
    return build(f"multi_prefill_s{seed}", seed, lens, table, P, hq=hq, hkv=hkv, hi=hi, di=di,
                 top_k=top_k, prefill=pre)


def with_query_seed(w, qseed):
    """A copy of ``w`` whose queries (q, q_idx, w) come from stream seed ``qseed``;
    the cache, keys and tables are shared.  Used to rotate distinct query batches
    over one cache so that consecutive steps select different blocks."""
    import copy
    q, qi, ww = _queries(qseed, w.num_queries, w.num_q_heads, w.head_dim, w.idx_heads,
                         w.idx_dim)
    v = copy.copy(w)
    v.q_bits, v.q_idx_bits, v.w = q, qi, ww
    v.meta = dict(w.meta, query_seed=qseed)
    return v


def with_q_scale(w, log2_factor):
    """A copy of ``w`` whose attention queries are multiplied by 2^log2_factor
    (exact in bf16 for these magnitudes).  Large factors make the softmax
    peaked: the logits spread over hundreds of units and the weights become
    nearly one-hot."""
    import copy
    f = gen.bf16_bits_to_f32(w.q_bits).astype(np.float32) * np.float32(2.0 ** log2_factor)
    assert np.all(np.isfinite(f))
    v = copy.copy(w)
    v.q_bits = gen.f32_to_bf16_bits(f)
    assert np.array_equal(gen.bf16_bits_to_f32(v.q_bits), f), "scaling must be exact"
    v.name = f"{w.name}_qx{2 ** log2_factor}"
    v.meta = dict(w.meta, q_log2_scale=log2_factor)
    return v

"""Float64 oracle of the dynamic-sparse-attention hot path (test infrastructure only).

One query at a time, in the order the pages give the method: score the coarse
per-block keys, keep the Top-K blocks, attend exactly over the selected blocks
([P1] section 4(3), the decode schematic: select, gather, sparse attention;
[P3] section 4.1, scoring followed by top-k).  Source tags [P1]..[P5] are
listed in ``oracle/__init__.py``.

Shapes (one layer):
  block table row  int   [max_blocks]        logical block j -> physical block p
  k_block(p), v_block(p) -> float64 [block_size, num_kv_heads, head_dim]
  key codes        uint8 [num_blocks, idx_dim] (E4M3), key scale float [num_blocks]
  q                float64 [num_q_heads, head_dim]
  q_idx            float64 [idx_heads, idx_dim], w float [idx_heads]
"""

import numpy as np

from .fp8 import e4m3_decode, e4m3_encode, E4M3_MAX


# ---------------------------------------------------------------------------
# a2: query-side quantization of the indexer query
# ---------------------------------------------------------------------------
def quantize_q_idx(q_idx):
    """FP8 codes and power-of-two scales of the indexer query.

    The pages want low-precision scoring inputs ([P5] "Index Selection Path")
    but do not say how the query is brought to FP8.  Reading taken: one scale
    per (query, indexer head), the smallest power of two 2^e with
    max_d |q_idx| <= 448 * 2^e, then q8 = E4M3(q_idx / 2^e) rounded to nearest
    even.  A power-of-two scale keeps the division exact.

    q_idx: float64 [..., idx_heads, idx_dim] -> (codes uint8 same shape,
    scale float64 [..., idx_heads]).
    """
    q = np.asarray(q_idx, dtype=np.float64)
    amax = np.max(np.abs(q), axis=-1)
    f, ex = np.frexp(amax)  # amax = f * 2^ex, f in [0.5, 1)
    # 448 = 0.875 * 2^9, so 2^(ex-9) suffices iff f <= 0.875; otherwise 2^(ex-8).
    e = np.where(f <= 0.875, ex - 9, ex - 8)
    e = np.where(amax == 0.0, 0, e)
    scale = np.exp2(e.astype(np.float64))
    codes = e4m3_encode(q / scale[..., None])
    return codes, scale


# ---------------------------------------------------------------------------
# a1 / causality
# ---------------------------------------------------------------------------
def local_block(pos, block_size):
    """Logical block holding the query's own position."""
    return int(pos) // int(block_size)


def visible_blocks(pos, seq_len, block_size):
    """Logical blocks a query at absolute position ``pos`` may select.

    A block is a candidate iff it exists (j < ceil(L / block_size)) and its
    first token is not after the query (j * block_size <= pos): causal block
    masking of the indexer.  The query's own block is always a candidate.
    """
    nb = -(-int(seq_len) // int(block_size))
    j = np.arange(nb, dtype=np.int64)
    return j[j * int(block_size) <= int(pos)]


# ---------------------------------------------------------------------------
# a3: indexer scoring
# ---------------------------------------------------------------------------
def index_scores(q_codes, q_scale, w, key_codes, key_scale, activation="relu"):
    """Index score of each candidate block for one query.

    The pages give the score only as an inner product between the query and
    the compressed / coarse block representation at low precision ([P1]
    section 4(1); [P5] "Index Selection Path"), for a model of the DSA class
    ([P2] section 1).  Reading taken (the DSA-class indexer form): per
    indexer head h an FP8 inner product, scaled back by the query and key
    scales, a ReLU, then a weighted sum over heads in ascending h:

        D[h, j] = sum_d val(q8[h, d]) * val(k8[j, d])          (exact in f64)
        S[j]    = sum_h w[h] * max(0, (sq[h] * ks[j]) * D[h, j])

    Every E4M3 value is an integer multiple of 2^-9 below 2^9, so each product
    is a multiple of 2^-18 below 2^18 and every partial sum of at most 128
    such products needs fewer than 53 bits: D is exact in float64 whatever
    the summation order.  ``activation="identity"`` drops the ReLU (used only
    by a closed-form test).

    q_codes uint8 [H, dI], q_scale float [H], w float [H],
    key_codes uint8 [n, dI], key_scale float [n] -> float64 [n].
    """
    qv = e4m3_decode(q_codes)  # [H, dI]
    kv = e4m3_decode(key_codes)  # [n, dI]
    d = qv @ kv.T  # [H, n]
    t = (np.asarray(q_scale, np.float64)[:, None] *
         np.asarray(key_scale, np.float64)[None, :]) * d
    if activation == "relu":
        t = np.where(t > 0.0, t, 0.0)  # ReLU emitting +0
    elif activation != "identity":
        raise ValueError(activation)
    w = np.asarray(w, np.float64)
    s = np.zeros(kv.shape[0], dtype=np.float64)
    for h in range(qv.shape[0]):
        s = s + w[h] * t[h]
    return s


# ---------------------------------------------------------------------------
# a4: Top-K selection
# ---------------------------------------------------------------------------
def select_blocks(cand, scores, local, top_k):
    """Top-K block selection for one query.

    The pages: keep the Top-K relevant blocks and output their block indices
    ([P1] section 4(1)); the order of the selected indices must match what the
    downstream gather expects ([P5] "Index Selection Path", second bullet);
    ragged selections are padded ([P1] section 4(1), third bullet).
    Readings taken: the query's own (local) block is always kept and counts
    towards K; the other K-1 are the candidates with the largest score, equal
    scores going to the lower logical block id; the result is emitted in
    ascending logical block id, padded with -1 to length K, with the number
    of valid entries returned beside it.  If there are at most K candidates
    all of them are kept.

    cand: logical ids (int array), scores: same length (any float dtype; the
    comparison is done in that dtype), local: the local block id (in cand).
    Returns (idx int32 [top_k], count int).
    """
    cand = np.asarray(cand, dtype=np.int64)
    scores = np.asarray(scores)
    if top_k < 1:
        raise ValueError("top_k must be >= 1")
    if local not in set(cand.tolist()):
        raise ValueError("local block must be a candidate")
    if cand.size <= top_k:
        sel = np.sort(cand)
    else:
        others = [(j, s) for j, s in zip(cand.tolist(), scores.tolist()) if j != local]
        # sort by (score descending, id ascending)
        others.sort(key=lambda js: (-js[1], js[0]))
        keep = [j for j, _ in others[: top_k - 1]] + [int(local)]
        sel = np.sort(np.asarray(keep, dtype=np.int64))
    out = np.full(top_k, -1, dtype=np.int32)
    out[: sel.size] = sel
    return out, int(sel.size)


# ---------------------------------------------------------------------------
# a5..a7: attention over the gathered blocks
# ---------------------------------------------------------------------------
def _gather_tokens(block_ids, table_row, pos, seq_len, block_size, k_block, v_block):
    """K/V rows of the selected blocks, in ascending logical position.

    A token (j, t) takes part iff its position j*bs + t is <= pos (causality
    inside the local block) and < seq_len (a ragged last block).
    Returns K [T, Hkv, d], V [T, Hkv, d] float64 and the absolute positions.
    """
    ks, vs, ps = [], [], []
    for j in sorted(int(b) for b in block_ids if int(b) >= 0):
        p = int(table_row[j])
        kb = np.asarray(k_block(p), dtype=np.float64)
        vb = np.asarray(v_block(p), dtype=np.float64)
        for t in range(block_size):
            a = j * block_size + t
            if a <= pos and a < seq_len:
                ks.append(kb[t])
                vs.append(vb[t])
                ps.append(a)
    return np.asarray(ks), np.asarray(vs), np.asarray(ps, dtype=np.int64)


def attention_partial(q, K, V, softmax_scale, num_kv_heads):
    """Softmax statistics of one query over a set of tokens.

    For each query head h with its KV head g = floor(h * Hkv / Hq) (heads
    grouped contiguously):
        x_t = scale * <q_h, K_t,g>,  m = max_t x_t,  l = sum_t exp(x_t - m),
        o   = sum_t exp(x_t - m) V_t,g / l.
    Returns (m [Hq], l [Hq], o [Hq, d]).
    """
    q = np.asarray(q, dtype=np.float64)
    hq = q.shape[0]
    m = np.empty(hq)
    l = np.empty(hq)
    o = np.empty_like(q)
    for h in range(hq):
        g = (h * num_kv_heads) // hq
        x = float(softmax_scale) * (K[:, g, :] @ q[h])
        m[h] = x.max()
        p = np.exp(x - m[h])
        l[h] = p.sum()
        o[h] = (p @ V[:, g, :]) / l[h]
    return m, l, o


def merge_partials(parts):
    """Combine softmax partials (m_i, l_i, o_i) over disjoint token sets.

        m = max_i m_i,  l = sum_i l_i e^(m_i - m),
        o = sum_i l_i e^(m_i - m) o_i / l,  lse = m + ln l.
    Returns (o, lse).
    """
    ms = np.stack([p[0] for p in parts])
    m = ms.max(axis=0)
    wts = [p[1] * np.exp(p[0] - m) for p in parts]
    l = np.sum(wts, axis=0)
    o = sum(wt[:, None] * p[2] for wt, p in zip(wts, parts)) / l[:, None]
    return o, m + np.log(l)


def sparse_attention(q, block_ids, table_row, pos, seq_len, block_size,
                     k_block, v_block, softmax_scale, num_kv_heads):
    """Exact attention of one query over the tokens of its selected blocks.

    Sparse attention computes only the index-selected pairs and is otherwise
    the full-attention formula ([P4] full-vs-sparse table, decode row);
    blocks are read whole through the block table ([P5] "KV Cache Layout").
    Returns (out [Hq, d], lse [Hq]).
    """
    K, V, _ = _gather_tokens(block_ids, table_row, pos, seq_len, block_size,
                             k_block, v_block)
    m, l, o = attention_partial(q, K, V, softmax_scale, num_kv_heads)
    return o, m + np.log(l)


def dense_attention(q, table_row, pos, seq_len, block_size, k_block, v_block,
                    softmax_scale, num_kv_heads):
    """Full causal attention of one query: every token 0..pos, walked one
    token at a time in logical order through the block table.  A separate
    code path from ``sparse_attention``, used by the invariants."""
    q = np.asarray(q, dtype=np.float64)
    hq = q.shape[0]
    Ks, Vs = [], []
    for a in range(0, min(int(pos) + 1, int(seq_len))):
        p = int(table_row[a // block_size])
        Ks.append(np.asarray(k_block(p), np.float64)[a % block_size])
        Vs.append(np.asarray(v_block(p), np.float64)[a % block_size])
    K = np.asarray(Ks)
    V = np.asarray(Vs)
    out = np.empty_like(q)
    lse = np.empty(hq)
    for h in range(hq):
        g = (h * num_kv_heads) // hq
        x = float(softmax_scale) * (K[:, g, :] @ q[h])
        mx = x.max()
        e = np.exp(x - mx)
        out[h] = (e @ V[:, g, :]) / e.sum()
        lse[h] = mx + np.log(e.sum())
    return out, lse

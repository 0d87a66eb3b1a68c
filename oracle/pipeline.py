"""One query through the whole oracle path (test infrastructure only).

Order of the steps follows the decode schematic of [P1] section 4(3)
(select blocks, gather them, sparse attention) with the selection itself
split as in [P3] section 4.1 (lightweight scoring, then top-k).
"""

import numpy as np

from .dsa import (quantize_q_idx, visible_blocks, local_block, index_scores,
                  select_blocks, sparse_attention)


def score_query(q_idx, w, table_row, pos, seq_len, block_size, key_codes,
                key_scale, activation="relu"):
    """Scores of every visible logical block of one query.

    Returns (cand int64 [n], scores float64 [n], local int).  The table walk
    maps each visible logical block j to its physical block table_row[j]
    whose coarse key row is read ([P5] "KV Cache Layout").
    """
    q8, sq = quantize_q_idx(q_idx)
    cand = visible_blocks(pos, seq_len, block_size)
    phys = np.asarray(table_row, dtype=np.int64)[cand]
    s = index_scores(q8, sq, w, np.asarray(key_codes)[phys],
                     np.asarray(key_scale)[phys], activation=activation)
    return cand, s, local_block(pos, block_size)


def run_query(q, q_idx, w, table_row, pos, seq_len, block_size, key_codes,
              key_scale, top_k, k_block, v_block, softmax_scale, num_kv_heads,
              decision_dtype=np.float32):
    """Score, select and attend for one query.

    The Top-K decision is taken on the scores rounded to ``decision_dtype``:
    the pages fix no precision for the score, and the library stores scores
    as float32, so the oracle decides in float32 too (with the same
    lower-id-wins rule on equal values).

    Returns a dict with cand, scores (float64), scores_dec, idx, cnt, out, lse.
    """
    cand, s, loc = score_query(q_idx, w, table_row, pos, seq_len, block_size,
                               key_codes, key_scale)
    s_dec = s.astype(decision_dtype)
    idx, cnt = select_blocks(cand, s_dec, loc, top_k)
    out, lse = sparse_attention(q, idx[:cnt], table_row, pos, seq_len,
                                block_size, k_block, v_block, softmax_scale,
                                num_kv_heads)
    return dict(cand=cand, scores=s, scores_dec=s_dec, idx=idx, cnt=cnt,
                out=out, lse=lse, local=loc)

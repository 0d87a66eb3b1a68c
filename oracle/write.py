"""The paged write path, for the oracle (test infrastructure only).

[P5] "Day-0 Readiness for Trillion-Parameter Models...", "KV Cache Layout":
a layer's cache is [block][token][head][dim] reached through a block table;
prefill writes a chunk's tokens into their blocks in batch, decode appends
the newest token.  [P1] "Day-0 Adaptation for Massive LLMs...", section 4(2):
each block also carries a compressed index representation, kept apart from
the fine-grained KV.  How that representation is derived from the block is
not given by the pages; here it is an input vector per block (for instance a
projection of the block's keys) that is stored at low precision: E4M3 codes
with one float32 scale per block.
"""

import numpy as np

from .fp8 import e4m3_encode, E4M3_MAX


def kv_write(k_pool, v_pool, table, seq_lens, tok_seq, tok_pos, k_new, v_new, block_size):
    """Copies of the pools with token i's K/V rows written to block
    table[s][pos // block_size], row pos % block_size (s = tok_seq[i], pos =
    tok_pos[i]; tok_seq None: s = i; tok_pos None: pos = seq_lens[s] - 1).
    Rows are copied bit for bit (any dtype)."""
    k_out, v_out = np.array(k_pool, copy=True), np.array(v_pool, copy=True)
    n = np.asarray(k_new).shape[0]
    for i in range(n):
        s = i if tok_seq is None else int(tok_seq[i])
        pos = int(seq_lens[s]) - 1 if tok_pos is None else int(tok_pos[i])
        p = int(table[s][pos // block_size])
        k_out[p, pos % block_size] = k_new[i]
        v_out[p, pos % block_size] = v_new[i]
    return k_out, v_out


def quantize_coarse_key(x):
    """E4M3 codes and float32 scale of one block's coarse key x (float32 [dI]).

    ks = max_d |x[d]| / 448 (with 1 in place of a zero maximum), computed in
    float32; y[d] = x[d] / ks in float32, clamped to [-448, 448]; code[d] =
    E4M3(y[d]) rounding to nearest even.  So the code of the largest entry is
    +-448 and the key value ks * value(code) approximates x.
    """
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0.0)
    if amax == 0:
        amax = np.float32(1.0)
    ks = np.float32(amax / np.float32(E4M3_MAX))     # float32 division, rounded once
    y = (x / ks).astype(np.float32)                   # float32 division, rounded once
    y = np.clip(y, -E4M3_MAX, E4M3_MAX)
    return e4m3_encode(y.astype(np.float64)), ks

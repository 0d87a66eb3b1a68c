"""CPU oracle for query-driven dynamic sparse attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The HIP library never uses it, and it shares no code with the HIP
library: it is a plain, slow, float64 NumPy restatement of what the method
computes, written so that each step can be checked against the sources by eye.

Sources (the pages the method is taken from):

  [P1] "Day-0 Adaptation for Massive LLMs: Overcoming Sparse Attention and
       MXFP4 Expert Weights", https://intl.cloud.baidu.com/en/article/9584108
  [P2] "Day-0 Adaptation for Trillion-Parameter LLMs: Sparse Attention and
       MXFP4 Inference Optimization",
       https://intl.cloud.baidu.com/en/article/9577114
  [P3] "Day-0 Adaptation for Trillion-Parameter Models: Engineering Practices
       and Technical Breakdown", https://intl.cloud.baidu.com/en/article/9581058
  [P4] "Day-0 Adaptation for Large Language Models: From Architecture Analysis
       to Inference Serving", https://intl.cloud.baidu.com/en/article/9584606
  [P5] "Day-0 Readiness for Trillion-Parameter Models: Engineering Sparse
       Attention and Expert Weight Compression",
       https://intl.cloud.baidu.com/en/article/9576887

What the pages fix, and what the oracle follows:
  * each query scores a compressed / coarse representation of every earlier
    KV block at low precision, keeps the Top-K blocks and runs exact attention
    on those blocks only ([P1] section 4(1) "Index Selection"; [P3] section 4
    and 4.1; [P5] "Index Selection Path");
  * the KV cache is organised as fixed-size blocks reached through a block
    table, [block][token_in_block][head][dim] ([P5] "KV Cache Layout");
  * sparse attention is full attention restricted to the index-selected pairs
    ([P4] "Deep Integration of Sparse Attention and Vision Computation", the
    full-vs-sparse table).
  * the write path: tokens' K/V rows go to their blocks through the table,
    and each block's coarse key is stored as E4M3 codes with a per-block
    float32 scale ([P5] "KV Cache Layout"; [P1] section 4(2)); write.py.
  * the MXFP4 expert path: MXFP4 weights unpacked to an FP8 workspace, and
    the grouped expert matmul in FP8 with block scales ([P1] section 5; [P2]
    sections 3.1-3.2; [P5] "MXFP4 Expert Weights"); moe.py.

Where the pages are silent the oracle takes the plainest reading; each reading
is named in the function that uses it.  Parity pins: every function in this
package is pinned by a ``-m "not gpu"`` test in ``tests/test_oracle_*.py``
against something other than itself (brute force, closed forms, hand-worked
examples, invariants).  No function here is "parity unpinned".
"""

from .fp8 import e4m3_decode, e4m3_encode, bf16_bits_to_f64, E4M3_MAX
from .dsa import (
    quantize_q_idx,
    visible_blocks,
    local_block,
    index_scores,
    select_blocks,
    sparse_attention,
    dense_attention,
    merge_partials,
    attention_partial,
)
from .write import kv_write, quantize_coarse_key

__all__ = [
    "e4m3_decode",
    "e4m3_encode",
    "bf16_bits_to_f64",
    "E4M3_MAX",
    "quantize_q_idx",
    "kv_write",
    "quantize_coarse_key",
    "visible_blocks",
    "local_block",
    "index_scores",
    "select_blocks",
    "sparse_attention",
    "dense_attention",
    "merge_partials",
    "attention_partial",
]

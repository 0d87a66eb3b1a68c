/*
 * dsa.h -- C ABI of the MI355X (gfx950) dynamic sparse attention library.
 *
 * Query-driven dynamic sparse attention over a paged (block-managed) KV cache:
 * every query scores one coarse FP8 key per KV block, keeps the Top-K blocks
 * and runs exact softmax attention over the gathered K/V of those blocks only.
 *
 * Sources (the operations below restate what these pages describe):
 *   [P1] "Day-0 Adaptation for Massive LLMs: Overcoming Sparse Attention and
 *        MXFP4 Expert Weights" (intl.cloud.baidu.com/en/article/9584108)
 *   [P3] "Day-0 Adaptation for Trillion-Parameter Models: Engineering
 *        Practices and Technical Breakdown" (.../article/9581058)
 *   [P4] "Day-0 Adaptation for Large Language Models: From Architecture
 *        Analysis to Inference Serving" (.../article/9584606)
 *   [P5] "Day-0 Readiness for Trillion-Parameter Models: Engineering Sparse
 *        Attention and Expert Weight Compression" (.../article/9576887)
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers, row-major, owned by the caller.
 *     The library never allocates, frees, copies host<->device or
 *     synchronizes; it only enqueues kernels on `stream` (NULL = the default
 *     stream).  Results are valid once the stream reaches them.
 *   - Arguments are validated on the host before anything is enqueued; an
 *     invalid call returns a negative dsa_status and enqueues nothing.
 *     dsa_last_error() then holds a thread-local message.  A failed launch
 *     returns DSA_ERR_HIP with the HIP error text in dsa_last_error().
 *   - Device data (table entries, lengths, positions) is trusted: block
 *     table entries of visible blocks must lie in [0, num_blocks),
 *     seq_lens[s] <= max_blocks_per_seq * block_size, q_pos < seq_lens[q_seq],
 *     and all floating inputs must be finite.  Violations are undefined.
 *   - Entry points keep no state between calls and are thread-safe; calls
 *     sharing a workspace buffer must be ordered on one stream.  The one
 *     exception is dsa_sparse_decode_fused_noalloc, whose scratch lives in the
 *     library (see its declaration).
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_ABI_VERSION 2

typedef enum {
  DSA_OK = 0,
  DSA_ERR_NULL = -1,        /* a required pointer is NULL                        */
  DSA_ERR_SHAPE = -2,       /* sizes inconsistent or out of range                */
  DSA_ERR_UNSUPPORTED = -3, /* a size the library has no kernel for             */
  DSA_ERR_ALIGN = -4,       /* a pointer is not aligned as documented            */
  DSA_ERR_WORKSPACE = -5,   /* workspace NULL or smaller than dsa_workspace_size */
  DSA_ERR_HIP = -6          /* the HIP runtime reported an error                 */
} dsa_status;

/*
 * One layer of the paged KV cache ([P5] "KV Cache Layout":
 * [block_id][token_in_block][head][dim], reached through a block table that
 * maps each sequence's logical block j to a physical block), together with
 * the coarse per-block index keys used for block selection ([P1] section
 * 4(2): compressed index blocks kept apart from the fine-grained KV blocks).
 *
 * Block size: selection works at the granularity of the cache's pages ([P1]
 * section 4(2): index granularity aligned with page granularity; [P3] section
 * 4.2: blocks aligned to the hardware tile); the pages recommend tuning it,
 * starting from 256 or 512 tokens ([P2] section 2.1, note).  Any of 64, 128,
 * 256, 512 is accepted at run time; max_blocks_per_seq * block_size and
 * num_blocks * block_size / 64 must stay below 2^31 (DSA_ERR_UNSUPPORTED).
 *
 * Order inside a physical block (kv_layout): DSA_KV_TOKEN_MAJOR is the
 * pages' [token_in_block][head][dim] order, where one head's 256 B row of a
 * token sits num_kv_heads * 256 B from the next token's; DSA_KV_HEAD_MAJOR
 * stores [head][token_in_block][dim], so each (block, head) is one
 * contiguous block_size * 256 B run.  Both hold the same values, and every
 * entry point that reads or writes k_cache / v_cache takes either; any other
 * value is DSA_ERR_UNSUPPORTED there.
 */
typedef enum { DSA_KV_TOKEN_MAJOR = 0, DSA_KV_HEAD_MAJOR = 1 } dsa_kv_layout;

typedef struct {
  const void* k_cache;         /* bf16 [num_blocks, block_size, num_kv_heads, head_dim] (token-major)
                                  or [num_blocks, num_kv_heads, block_size, head_dim] (head-major),
                                  16 B aligned                                                         */
  const void* v_cache;         /* bf16, same shape and layout as k_cache, 16 B aligned                */
  const uint8_t* idx_keys;     /* E4M3 (OCP, bias 7, max 448) codes [num_blocks, idx_dim], 16 B aligned */
  const float* idx_scale;      /* fp32 [num_blocks], > 0: key value = scale * E4M3 value              */
  const int32_t* block_table;  /* int32 [num_seqs, max_blocks_per_seq]: logical -> physical block    */
  const int32_t* seq_lens;     /* int32 [num_seqs]: tokens in the cache, current token included      */
  int32_t num_blocks;          /* physical blocks in the pool, >= 1                                  */
  int32_t block_size;          /* tokens per block: 64, 128, 256 or 512 (see below)                  */
  int32_t num_kv_heads;        /* >= 1                                                               */
  int32_t head_dim;            /* 128: the one head size the kernels support                         */
  int32_t idx_dim;             /* coarse key length: 64 or 128                                       */
  int32_t num_seqs;            /* >= 1                                                               */
  int32_t max_blocks_per_seq;  /* row length of block_table, >= 1                                    */
  int32_t kv_layout;           /* dsa_kv_layout of k_cache and v_cache                               */
} dsa_paged_kv;

/*
 * A batch of queries.  Decode: q_seq == NULL means query i belongs to
 * sequence i (num_queries <= num_seqs); q_pos == NULL means each query sits
 * at the last cached position, seq_lens[s] - 1 (its own K/V already written).
 * Chunked prefill: q_seq and q_pos give the sequence and absolute position
 * of every query; the chunk's K/V must already be in the cache.
 */
typedef struct {
  int32_t num_queries;         /* 0 <= Nq <= 65535 (0: every call is a no-op)                       */
  int32_t num_q_heads;         /* Hq, a multiple of num_kv_heads, Hq / Hkv <= 16                     */
  int32_t idx_heads;           /* indexer heads HI, 1..16                                            */
  const int32_t* q_seq;        /* int32 [Nq] or NULL                                                 */
  const int32_t* q_pos;        /* int32 [Nq] or NULL                                                 */
  const void* q;               /* bf16 [Nq, Hq, head_dim], 16 B aligned                              */
  const void* q_idx;           /* bf16 [Nq, HI, idx_dim], 16 B aligned                               */
  const float* w_idx;          /* fp32 [Nq, HI]: per-query, per-indexer-head weights                 */
} dsa_queries;

/*
 * Index scoring ([P1] section 4(1) "Index Selection": score the compressed
 * representation of every earlier KV block against the query; [P3] section
 * 4.1 "lightweight scoring"; [P5] "Index Selection Path": low-precision
 * inputs).  For query q of sequence s at position pos, and each logical block
 * j with j * block_size <= pos (causal block mask), p = block_table[s][j]:
 *
 *   sq[h]   = smallest power of two with max_d |q_idx[q,h,d]| <= 448 sq[h]
 *   q8[h,:] = E4M3(q_idx[q,h,:] / sq[h]), round to nearest even
 *   D[h]    = sum_d q8[h,d] * idx_keys[p,d]          (exact)
 *   S[q,j]  = sum_h w_idx[q,h] * max(0, (sq[h] * idx_scale[p]) * D[h])
 *
 * evaluated in float64 in that order and rounded once to fp32.  Columns j of
 * invisible blocks (j * block_size > pos, or j >= max_blocks_per_seq) are -inf.
 *
 * scores: fp32 [num_queries, max_blocks_per_seq], 4 B aligned, written whole.
 * Needs idx_keys, idx_scale, block_table, seq_lens, q_idx, w_idx.
 */
dsa_status dsa_index_score(const dsa_paged_kv* kv, const dsa_queries* qs, float* scores,
                           hipStream_t stream);

/*
 * Top-K block selection ([P1] section 4(1): Top-K relevant blocks, no full
 * sort; [P5] "Index Selection Path": index order must match the downstream
 * gather; padding for ragged selections, [P1] section 4(1)).  For each query
 * the local block l = pos / block_size is always kept; the other top_k - 1
 * are the visible blocks j < l with the largest scores[q, j], equal scores
 * going to the lower j (-0.0 == +0.0).  Output in ascending logical block id
 * (so l is last), padded with -1 to top_k; block_cnt[q] = min(top_k, l + 1).
 *
 * scores: fp32 [Nq, max_blocks_per_seq] as written by dsa_index_score.
 * block_idx: int32 [Nq, top_k]; block_cnt: int32 [Nq].  1 <= top_k <= 4096.
 * Needs block_table (unused), seq_lens, and q_pos/q_seq if given.
 */
dsa_status dsa_topk_blocks(const float* scores, const dsa_paged_kv* kv, const dsa_queries* qs,
                           int32_t top_k, int32_t* block_idx, int32_t* block_cnt,
                           hipStream_t stream);

/*
 * Sparse attention of decode queries over their selected blocks ([P1]
 * section 4(3): gather the selected blocks, then sparse attention; [P4]
 * full-vs-sparse table: only index-selected pairs).  For each query head h
 * with KV head g = h / (Hq / Hkv), over the tokens t of the selected logical
 * blocks block_idx[q, 0 .. block_cnt[q]) whose position j*bs + t is <= pos
 * and < seq_len:
 *
 *   x_t = softmax_scale * <q[q,h,:], K[p_j, t, g, :]>
 *   out[q,h,:] = sum_t e^(x_t - m) V[p_j, t, g, :] / sum_t e^(x_t - m),
 *   lse[q,h]   = m + ln sum_t e^(x_t - m)                 (m = max_t x_t)
 *
 * The selected blocks are split across workgroups and the partial softmax
 * states are merged in a final pass.  block_idx entries must be visible
 * logical ids or -1 beyond block_cnt; the local block must be among them.
 * out: fp32 [Nq, Hq, head_dim]; lse: fp32 [Nq, Hq] or NULL.
 * workspace: device buffer of at least dsa_workspace_size(DSA_OP_ATTN_DECODE)
 * bytes, 256 B aligned (may be NULL when that size is 0); it holds the
 * split partials.  Calls that share a workspace must not overlap in time.
 */
dsa_status dsa_sparse_attn_decode(const dsa_paged_kv* kv, const dsa_queries* qs,
                                  const int32_t* block_idx, const int32_t* block_cnt,
                                  int32_t top_k, float softmax_scale, float* out, float* lse,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Decode attention with the Top-K selection fused in ([P3] "Day-0
 * Adaptation for Trillion-Parameter Models...", section 4.1: Top-K fused with
 * the operators before and after it; [P5] "Day-0 Readiness...",
 * "Differentiated Adaptation of Prefill and Decode": selection, gather and
 * attention fused in decode).  scores: fp32 [num_queries,
 * max_blocks_per_seq] as dsa_index_score writes them (only a query's visible
 * blocks 0 .. pos / block_size - 1 are read), 4 B aligned.  Every attention
 * workgroup selects its query's blocks from that row with dsa_topk_blocks's
 * rule, into on-chip memory, and attends them: the selection is the one
 * dsa_topk_blocks returns and the outputs are those of dsa_sparse_attn_decode
 * on it (within the decode tolerance); out and lse (nullable) as there.
 * block_idx_out / block_cnt_out (nullable, each on its own) receive the
 * selection.  Limits:
 * max_blocks_per_seq <= 2048 and top_k <= 2048 (DSA_ERR_UNSUPPORTED).
 * workspace: at least dsa_workspace_size(DSA_OP_ATTN_DECODE) bytes, 256 B
 * aligned (may be NULL when that size is 0).
 */
dsa_status dsa_sparse_attn_decode_topk(const dsa_paged_kv* kv, const dsa_queries* qs,
                                       const float* scores, int32_t top_k, float softmax_scale,
                                       float* out, float* lse, int32_t* block_idx_out,
                                       int32_t* block_cnt_out, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream);

/*
 * Sparse attention of a chunk of prefill queries ([P3] section 4.3 and [P5]
 * "Differentiated Adaptation of Prefill and Decode": the prefill path is
 * compute-bound and batches many queries).  Same result as
 * dsa_sparse_attn_decode; q_seq and q_pos are required.  No workspace.
 */
dsa_status dsa_sparse_attn_prefill(const dsa_paged_kv* kv, const dsa_queries* qs,
                                   const int32_t* block_idx, const int32_t* block_cnt,
                                   int32_t top_k, float softmax_scale, float* out, float* lse,
                                   hipStream_t stream);

/*
 * One-call decode ([P5] "Differentiated Adaptation of Prefill and Decode":
 * fuse index selection, gather and attention in decode): dsa_index_score,
 * dsa_topk_blocks and dsa_sparse_attn_decode in one entry point with the
 * same results.  block_idx_out / block_cnt_out (nullable, each on its
 * own) receive the selection.  workspace: at least dsa_workspace_size(DSA_OP_DECODE_FUSED)
 * bytes, 256 B aligned.
 */
dsa_status dsa_sparse_decode_fused(const dsa_paged_kv* kv, const dsa_queries* qs, int32_t top_k,
                                   float softmax_scale, float* out, float* lse,
                                   int32_t* block_idx_out, int32_t* block_cnt_out,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * dsa_sparse_decode_fused without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, serving loops
 * that must not call hipMalloc, harnesses that forbid it.  The same results
 * as dsa_sparse_decode_fused.  Its scratch (split partials, scores or
 * candidate lists, the selection) is one array of DSA_NOALLOC_SCRATCH_BYTES
 * in the library's device memory, one per GPU, held until the process ends;
 * a call needing more (dsa_workspace_size(DSA_OP_DECODE_FUSED) larger than
 * that) returns DSA_ERR_UNSUPPORTED before anything is enqueued.  Every call
 * on a GPU uses that GPU's array: calls that overlap in time on one GPU (on
 * different streams, or from different threads) race and must not be made.
 * The first call on a device looks up the array's address there (a host
 * query); nothing is ever allocated, freed, copied or cleared.
 */
#define DSA_NOALLOC_SCRATCH_BYTES (16 * 1024 * 1024)
dsa_status dsa_sparse_decode_fused_noalloc(const dsa_paged_kv* kv, const dsa_queries* qs,
                                           int32_t top_k, float softmax_scale, float* out,
                                           float* lse, int32_t* block_idx_out,
                                           int32_t* block_cnt_out, hipStream_t stream);

/*
 * One-call chunked prefill ([P1] section 4(3): prefill is compute-intensive,
 * and scoring, block selection and attention can run as one pipeline; [P3]
 * section 4.3: selection fused with the attention inside blocks; [P5]
 * "Differentiated Adaptation of Prefill and Decode": batch the prefill's
 * selection).  The selection is that of dsa_index_topk; the attention is that
 * of dsa_sparse_attn_prefill (same formula and tolerance, a different
 * summation order), computed block-inverted: the selection is transposed into
 * per-pool-tile lists of (query, pick), each 64-token tile of K/V is read once
 * per KV head for all the queries that picked it, and one partial softmax
 * state per (query, pick, head) is merged per query in pick order (results do
 * not depend on scheduling).  q_seq and q_pos are required; out: fp32
 * [Nq, Hq, 128], 8 B aligned; lse (nullable) fp32 [Nq, Hq].  block_idx_out /
 * block_cnt_out (nullable, together) receive the selection.  workspace: at
 * least dsa_workspace_size(DSA_OP_PREFILL_FUSED) bytes, 256 B aligned; it
 * grows as Nq * top_k * (block_size / 64) * Hq * 520 B (the partial states:
 * 17.4 GB for 8192 queries, K 64, 64 query heads, 64-token blocks).
 */
dsa_status dsa_sparse_prefill_fused(const dsa_paged_kv* kv, const dsa_queries* qs, int32_t top_k,
                                    float softmax_scale, float* out, float* lse,
                                    int32_t* block_idx_out, int32_t* block_cnt_out,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Scoring and selection in one entry point ([P3] section 4.1: top-k fused
 * with the scoring before it to avoid materialising intermediate tensors).
 * Same block_idx / block_cnt as dsa_index_score followed by dsa_topk_blocks.
 * workspace: at least dsa_workspace_size(DSA_OP_INDEX_TOPK) bytes.
 */
dsa_status dsa_index_topk(const dsa_paged_kv* kv, const dsa_queries* qs, int32_t top_k,
                          int32_t* block_idx, int32_t* block_cnt, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/*
 * Paged write path ([P5] "KV Cache Layout": prefill writes a chunk's tokens
 * into their blocks in batch, decode appends the newest token, through the
 * same block table the reads use).  Token i's K and V rows (bf16 [Hkv, 128]
 * each, k_new / v_new: bf16 [n_tokens, Hkv, 128], 16 B aligned) are copied to
 * block block_table[s][pos / block_size], row pos % block_size of
 * kv->k_cache / kv->v_cache, which this call writes (the const qualifiers of
 * dsa_paged_kv describe the other calls).  s = tok_seq[i] (NULL: s = i, which
 * needs n_tokens <= num_seqs); pos = tok_pos[i] (NULL: seq_lens[s] - 1, the
 * newest token of a decode step).  Block allocation and the table entries
 * themselves are the caller's.  A token whose target falls outside the table
 * row or the pool is skipped (nothing is written for it); rows of tokens that
 * share a target are written in no particular order.  Needs k_cache, v_cache,
 * block_table, seq_lens.
 */
dsa_status dsa_kv_write(const dsa_paged_kv* kv, int32_t n_tokens, const int32_t* tok_seq,
                        const int32_t* tok_pos, const void* k_new, const void* v_new,
                        hipStream_t stream);

/*
 * Coarse index keys at low precision ([P1] section 4(2): a compressed
 * representation per block, kept apart from the fine-grained KV; [P5] "Index
 * Selection Path": low-precision scoring inputs).  How the representation is
 * derived from a block is left open by the pages; it is given here as one
 * float vector per block (coarse: fp32 [n_blocks, idx_dim], 4 B aligned) and
 * stored for physical block p = block_ids[i] as
 *   ks = max_d |x[d]| / 448 (1 / 448 for a zero vector),
 *   idx_keys[p][d] = E4M3(clamp(x[d] / ks, -448, 448)), round to nearest even,
 *   idx_scale[p] = ks,
 * every division in float32, rounded once; this call writes kv->idx_keys and
 * kv->idx_scale.  Ids outside [0, num_blocks) are skipped.  The result is
 * exactly what dsa_index_score expects (key value = idx_scale * E4M3 value).
 */
dsa_status dsa_index_key_write(const dsa_paged_kv* kv, int32_t n_blocks, const int32_t* block_ids,
                               const float* coarse, hipStream_t stream);

/*
 * Device-data check.  The entry points above trust the device-side contract
 * (conventions at the top of this file); this one checks it and is meant for
 * debugging and for callers that receive tables or block lists from
 * elsewhere.  It reads block_table, seq_lens, q_seq / q_pos when given, and
 * block_idx / block_cnt when given, all within their declared shapes, and
 * dereferences none of their values, so it is safe on any data.  It enqueues
 * two small kernels on `stream`; once the stream reaches them, *flags (a
 * device uint32, 4 B aligned) holds the OR of the DSA_CHECK_* bits of every
 * violation found, 0 if none:
 *   DSA_CHECK_SEQ_LEN    seq_lens[s] < 1 or > max_blocks_per_seq * block_size
 *   DSA_CHECK_TABLE      a block holding tokens (j * block_size < seq_lens[s])
 *                        has a table entry outside [0, num_blocks)
 *   DSA_CHECK_Q_SEQ      q_seq[i] outside [0, num_seqs)
 *   DSA_CHECK_Q_POS      the query position is outside [0, seq_lens[s])
 *   DSA_CHECK_BLOCK_LIST a selection (as dsa_sparse_attn_decode / _prefill
 *                        take it) breaks the rule of dsa_topk_blocks ([P1]
 *                        section 4(1)): block_cnt[i] in 1..top_k, ids
 *                        ascending and visible (j * block_size <= pos),
 *                        the last one the local block pos / block_size,
 *                        then -1 up to top_k
 * block_idx / block_cnt: NULL to skip the list check (then top_k is unused),
 * else int32 [Nq, top_k] / [Nq] with 1 <= top_k <= 4096.  Only block_table,
 * seq_lens (and the queries' q_seq / q_pos) are required of kv / qs; no
 * K/V, index keys or query vectors are read.
 */
enum {
  DSA_CHECK_SEQ_LEN = 1,
  DSA_CHECK_TABLE = 2,
  DSA_CHECK_Q_SEQ = 4,
  DSA_CHECK_Q_POS = 8,
  DSA_CHECK_BLOCK_LIST = 16
};
dsa_status dsa_check_inputs(const dsa_paged_kv* kv, const dsa_queries* qs,
                            const int32_t* block_idx, const int32_t* block_cnt, int32_t top_k,
                            uint32_t* flags, hipStream_t stream);

/*
 * MXFP4 expert weights of one MoE layer ([P1] "Day-0 Adaptation for Massive
 * LLMs...", section 5; [P5] "Day-0 Readiness...", "MXFP4 Expert Weights"):
 * expert e's weight W_e [n, k] (outputs x inputs) in MXFP4 along k (OCP MX
 * specification v1.0): E2M1 codes, two per byte, element 2i in bits 3-0;
 * one E8M0 scale (value 2^(s - 127)) per 32 consecutive elements.
 */
typedef struct {
  const uint8_t* w_fp4;    /* [num_experts, n, k / 2], 16 B aligned                               */
  const uint8_t* w_scale;  /* [num_experts, n, k / 32]                                             */
  int32_t num_experts;     /* >= 1                                                                 */
  int32_t n;               /* >= 1                                                                 */
  int32_t k;               /* a multiple of 128; n * k < 2^31                                      */
} dsa_mx_experts;

/*
 * Activations to MXFP8 ([P1] section 5(2): the expert matmuls run in FP8):
 * per 32-element block of each row of x (bf16 [rows, k], k a multiple of 32,
 * 16 B aligned), shared = floor(log2 max|x|) - 8 clamped to [-127, 127],
 * scales[block] = shared + 127 (0 for a block of zeros), codes = E4M3(x /
 * 2^shared) (OCP E4M3, round to nearest even, clamped to +-448).  codes: uint8
 * [rows, k], 16 B aligned; scales: uint8 [rows, k / 32].
 */
dsa_status dsa_mx_quantize(const void* x, int32_t rows, int32_t k, uint8_t* codes, uint8_t* scales,
                           hipStream_t stream);

/*
 * The online conversion ([P1] section 5(2) and its schematic; [P2] "Day-0
 * Adaptation for Trillion-Parameter LLMs...", section 3.1): the weights of
 * experts[0 .. n_experts) (device int32, each in [0, num_experts)) unpacked
 * into workspace slots 0 .. n_experts-1: ws_codes uint8 [n_experts, n, k]
 * holds the E4M3 code of every E2M1 element (exact), ws_scales uint8
 * [n_experts, n, k / 32] the E8M0 scales unchanged, so the block scales stay
 * apart from the FP8 elements and nothing leaves the FP8 range ([P1] section
 * 5(3)).  The layout is the grouped matmul's FP8 input layout.
 */
dsa_status dsa_mxfp4_to_fp8(const dsa_mx_experts* w, const int32_t* experts, int32_t n_experts,
                            uint8_t* ws_codes, uint8_t* ws_scales, hipStream_t stream);

/*
 * The grouped expert matmul ([P1] section 5(2): grouped FP8 matmul with block
 * scales; [P5] "MXFP4 Expert Weights": only the routed experts are
 * converted).  For each (token t, slot j) with e = route[t, j] in [0,
 * num_experts): out[t, j, :] = xq[t, :] . W_e^T, where xq is the MXFP8 row
 * (x_codes uint8 [tokens, k], 16 B aligned; x_scales uint8 [tokens, k / 32],
 * 4 B aligned, from dsa_mx_quantize) and W_e the MXFP4 weights; rows of other slots are
 * zero.  out: fp32 [tokens, slots, n].  Computed on the scaled matrix cores
 * (E8M0 block scales applied in hardware; the products are exact, the sums
 * are the matrix unit's, within 2^-9 of sum |xq w| per output).  mode:
 *   DSA_MOE_FP8_WORKSPACE  the pages' path: the routed experts are unpacked
 *                          to FP8 into the workspace, then multiplied;
 *   DSA_MOE_FP4_DIRECT     the FP4 weights feed the matrix cores directly
 *                          (same values; no FP8 copy).
 * workspace: at least dsa_moe_workspace_size bytes, 256 B aligned (with
 * DSA_MOE_FP8_WORKSPACE it holds min(num_experts, tokens * slots) expert
 * slots of n * k + n * k / 32 bytes).  route: int32 [tokens, slots].
 * Limits (DSA_ERR_UNSUPPORTED beyond them): tokens * slots <= 2^30, n * k <
 * 2^31, and fewer than 2^24 (row tile, column block) work items.  Output rows are
 * independent of the order pairs are grouped in, so results are bit-exact
 * from run to run.
 */
enum { DSA_MOE_FP8_WORKSPACE = 0, DSA_MOE_FP4_DIRECT = 1 };
dsa_status dsa_moe_workspace_size(const dsa_mx_experts* w, int32_t tokens, int32_t slots,
                                  int32_t mode, size_t* bytes);
dsa_status dsa_moe_grouped_gemm(const dsa_mx_experts* w, const uint8_t* x_codes,
                                const uint8_t* x_scales, int32_t tokens, const int32_t* route,
                                int32_t slots, int32_t mode, float* out, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

/* Workspace sizes.  op: one of the DSA_OP_* values. */
enum { DSA_OP_ATTN_DECODE = 1, DSA_OP_DECODE_FUSED = 2, DSA_OP_INDEX_TOPK = 3,
       DSA_OP_PREFILL_FUSED = 4 };
dsa_status dsa_workspace_size(int op, const dsa_paged_kv* kv, const dsa_queries* qs,
                              int32_t top_k, size_t* bytes);

const char* dsa_status_str(dsa_status s);
const char* dsa_last_error(void); /* thread-local; "" after a successful call */
int dsa_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* DSA_H */

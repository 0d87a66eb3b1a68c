// Internal interface between the C-ABI layer (dsa_api.cpp) and the gfx950
// kernels.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

constexpr int kBlockSize = 64;   // tokens per attention tile (a KV block is 1, 2, 4 or 8 tiles)
constexpr int kHeadDim = 128;    // attention head dim
constexpr int kMaxGroup = 16;    // max query heads per KV head
constexpr int kMaxIdxHeads = 16;
constexpr int kMaxTopK = 4096;

struct KvView {
  const uint16_t* k;        // bf16 [P, block size, Hkv, 128] or [P, Hkv, block size, 128]
  const uint16_t* v;
  const uint8_t* idx_keys;  // [P, dI]
  const float* idx_scale;   // [P]
  const int32_t* table;     // [B, maxb]
  const int32_t* seq_lens;  // [B]
  int num_blocks, num_kv_heads, idx_dim, num_seqs, maxb;
  int bs_shift;             // log2(tokens per block): 6, 7, 8 or 9
  int head_major;           // 0: [P, bs, Hkv, 128]; 1: [P, Hkv, bs, 128]
};

// Elements between consecutive tokens of one KV head.
__host__ __device__ inline size_t kv_tok_stride(const KvView& kv) {
  return kv.head_major ? (size_t)kHeadDim : (size_t)kv.num_kv_heads * kHeadDim;
}

// Element offset of token 0 of 64-token pool tile `tile` (physical block
// tile >> (bs_shift - 6), tile within it tile & (2^(bs_shift - 6) - 1)), KV head g.
__host__ __device__ inline size_t kv_tile_base(const KvView& kv, int tile, int g) {
  if (!kv.head_major) return ((size_t)tile * 64 * kv.num_kv_heads + g) * kHeadDim;
  const int ts = kv.bs_shift - 6;
  const size_t blk = (size_t)(tile >> ts), t = (size_t)(tile & ((1 << ts) - 1));
  return ((((blk * kv.num_kv_heads + g) << kv.bs_shift) + t * 64) * kHeadDim);
}

struct QView {
  int nq, hq, hi;
  const int32_t* q_seq;     // nullable: query i -> sequence i
  const int32_t* q_pos;     // nullable: seq_lens[s] - 1
  const uint16_t* q;        // bf16 [Nq, Hq, 128]
  const uint16_t* q_idx;    // bf16 [Nq, HI, dI]
  const float* w;           // [Nq, HI]
};

// Per-query (sequence, position, local block) resolution shared by kernels.
__host__ __device__ inline int query_seq(const QView& q, int i) { return q.q_seq ? q.q_seq[i] : i; }

hipError_t launch_index_score(const KvView& kv, const QView& q, float* scores, hipStream_t s);
// Exact scoring of many queries on the int8 matrix cores (same results).
bool index_score_mfma_supported(const KvView& kv, const QView& q);
hipError_t launch_index_score_mfma(const KvView& kv, const QView& q, float* scores, hipStream_t s);
// Scoring that keeps only each workgroup's Top-K candidates (in the score
// workspace), then one merging wave per query: the same indices as
// launch_index_score followed by launch_topk, for long lists and small K.
bool index_cand_topk_supported(const KvView& kv, const QView& q, int top_k);
hipError_t launch_index_cand_topk(const KvView& kv, const QView& q, int top_k, float* ws,
                                  int32_t* idx, int32_t* cnt, hipStream_t s);
// Only the scoring kernel of launch_index_cand_topk: the candidate lists in ws;
// when done is given, it also zeroes the split counters (attn_done_bytes)
// of the launch_sparse_attn_cand that follows.
hipError_t launch_index_cand_scores(const KvView& kv, const QView& q, int top_k, float* ws,
                                    uint32_t* done, hipStream_t s);
// Scoring and Top-K of one query per workgroup, scores kept on chip (same
// results as launch_index_score followed by launch_topk).
bool index_topk_fused_supported(const KvView& kv, const QView& q);
hipError_t launch_index_topk_fused(const KvView& kv, const QView& q, int top_k, int32_t* idx,
                                   int32_t* cnt, hipStream_t s);
hipError_t launch_topk(const float* scores, const KvView& kv, const QView& q, int top_k,
                       int32_t* idx, int32_t* cnt, hipStream_t s);
// Scoring and Top-K of many queries (a prefill chunk) in one launch:
// approximate scores on the FP8 matrix cores with an error bound, exact
// scores only for the blocks the bound leaves undecided (the same indices as
// launch_index_score followed by launch_topk), for sequences of at most 2048
// blocks.
bool index_topk_fp8_supported(const KvView& kv, const QView& q);
hipError_t launch_index_topk_fp8(const KvView& kv, const QView& q, int top_k, int32_t* idx,
                                 int32_t* cnt, hipStream_t s);

// Split-K sparse attention.  num_splits == 1 writes out/lse directly;
// otherwise partial softmax states go to `partials` and a merge kernel follows
// on the same stream.
struct AttnPlan {
  int waves;   // waves per workgroup (4 or 8)
  int splits;  // workgroups per (query, KV head)
  bool stream; // K/V read with the non-temporal cache policy (decode)
};
// Compute units of the current device (hipDeviceAttributeMultiprocessorCount,
// cached per device; 256 when no device can be queried).
int device_cu_count();
// tiles: 64-token tiles per query (top_k * block_size / 64)
AttnPlan attn_plan(int nq, int hkv, int tiles, bool prefill);
size_t attn_partials_bytes(int nq, int hq, int splits);
hipError_t launch_sparse_attn(const KvView& kv, const QView& q, const int32_t* idx,
                              const int32_t* cnt, int top_k, float scale, float* out, float* lse,
                              float* partials, AttnPlan plan, hipStream_t s);
// Decode attention that first selects each query's blocks from its scores
// (scores as written by launch_index_score; the same selection as
// launch_topk), for sequences of at most 2048 blocks and top_k <= 2048.
// idx_out / cnt_out may be null.
bool attn_select_supported(const KvView& kv, const QView& q, int top_k, const AttnPlan& plan);
hipError_t launch_sparse_attn_select(const KvView& kv, const QView& q, const float* scores,
                                     int top_k, float scale, float* out, float* lse,
                                     float* partials, AttnPlan plan, int32_t* idx_out,
                                     int32_t* cnt_out, hipStream_t s);
// Decode attention that first scores (exactly, on chip) and selects each
// query's blocks itself: the same scores, selection and attention as
// launch_index_score, launch_topk and launch_sparse_attn, in one launch, for
// sequences of at most 256 blocks and grids of at most one workgroup per CU.
// idx_out / cnt_out may be null.
bool attn_score_supported(const KvView& kv, const QView& q, int top_k, const AttnPlan& plan);
hipError_t launch_sparse_attn_score(const KvView& kv, const QView& q, int top_k, float scale,
                                    float* out, float* lse, float* partials, AttnPlan plan,
                                    int32_t* idx_out, int32_t* cnt_out, hipStream_t s);
// Decode attention that first merges each query's candidate lists (as left
// by launch_index_cand_scores in ws) into its selection, the same as
// launch_index_cand_topk's; for the lists launch_index_cand_topk takes.
// done (attn_done_bytes, zeroed by launch_index_cand_scores given the same
// pointer): the split partials are merged inside this launch when
// attn_fused_merge holds; nullptr: by a merging launch after it.
bool attn_cand_supported(const KvView& kv, const QView& q, int top_k, const AttnPlan& plan);
size_t attn_done_bytes(int nq, int hkv);
bool attn_fused_merge(const QView& q, int hkv, const AttnPlan& plan);
hipError_t launch_sparse_attn_cand(const KvView& kv, const QView& q, float* ws, int top_k,
                                   float scale, float* out, float* lse, float* partials,
                                   AttnPlan plan, int32_t* idx_out, int32_t* cnt_out,
                                   uint32_t* done, hipStream_t s);

// Paged write path (write.hip): token K/V rows into their blocks; per-block
// coarse keys quantized to E4M3 with scale max|x| / 448.
hipError_t launch_kv_write(const KvView& kv, int n, const int32_t* tok_seq, const int32_t* tok_pos,
                           const void* k_new, const void* v_new, void* k_out, void* v_out,
                           hipStream_t s);
hipError_t launch_index_key_write(const KvView& kv, int n, const int32_t* blk, const float* x,
                                  uint8_t* keys_out, float* scale_out, hipStream_t s);

// Device-data check (check.hip): zeroes *flags, then ORs in the
// DSA_CHECK_* bits of every violation.
hipError_t launch_check_inputs(const KvView& kv, const QView& q, const int32_t* block_idx,
                               const int32_t* block_cnt, int top_k, uint32_t* flags,
                               hipStream_t s);

// Block-inverted prefill attention (prefill_inv.hip): the selection becomes a
// CSR list "pool tile -> (query, pick)", one workgroup per (tile, KV head)
// attends all of a tile's queries, and a merge combines each query's partial
// states: o[128] (512 B rows, whole cache lines) and {m, l}, per (query, head,
// pick).
struct InvLayout {
  int items_max;      // item slots per query: top_k * tiles per block
  long pool_tiles;    // num_blocks * tiles per block
  long tile_slots;    // grid rows of the attention kernel
  long entries_max;   // nq * items_max: (query, pick) slots
  size_t n_items, count, offset, cursor, tiles, n_tiles, entries, part_o, part_ml, total;  // bytes
};
InvLayout inv_layout(const KvView& kv, int nq, int hq, int top_k, size_t base);
bool prefill_inv_supported(const KvView& kv, const QView& q);
hipError_t launch_prefill_inv(const KvView& kv, const QView& q, const int32_t* idx,
                              const int32_t* cnt, int top_k, float scale, float* out, float* lse,
                              char* ws, const InvLayout& layout, hipStream_t s);

// MXFP4 expert weights (moe.hip): MXFP8 activations, the online MXFP4 -> FP8
// conversion, and the grouped expert matmul on the scaled matrix cores.
struct MxExperts {
  const uint8_t* fp4;    // [E][N][K/2] E2M1 codes, element 2i in the low nibble
  const uint8_t* scale;  // [E][N][K/32] E8M0
  int num_experts, n, k;
};
struct MoeLayout {
  int bm;  // pairs per row tile: 32, or 128 when the experts average many pairs
  int max_tiles, max_active;
  size_t active, slot, n_active, ws_codes, ws_scales;                      // bytes
  size_t count, cursor, list, tile_e, tile_p0, tile_p1, n_tiles, total;  // bytes
};
hipError_t launch_mx_quant_act(const uint16_t* x, int t, int k, uint8_t* codes, uint8_t* scales,
                               hipStream_t s);
hipError_t launch_mxfp4_unpack(const MxExperts& w, const int32_t* experts, int n_active,
                               uint8_t* ws_codes, uint8_t* ws_scales, hipStream_t s);
MoeLayout moe_layout(const MxExperts& w, int pairs, bool fp8_workspace, size_t base);
hipError_t launch_moe_gemm(const MxExperts& w, bool fp8_workspace, const uint8_t* a_codes,
                           const uint8_t* a_scales, int t, const int32_t* route, int slots,
                           float* out, char* ws, const MoeLayout& layout, hipStream_t s);

}  // namespace dsa

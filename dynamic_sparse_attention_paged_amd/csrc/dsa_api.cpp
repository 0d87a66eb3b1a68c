// C-ABI entry points: host-side validation, workspace layout, dispatch.
// Every check runs before anything is enqueued, so an invalid call has no
// side effects and needs no GPU.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/dsa.h"
#include "dsa_internal.h"

namespace {

thread_local char g_err[512] = "";

dsa_status fail(dsa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

dsa_status ok() {
  g_err[0] = '\0';
  return DSA_OK;
}

dsa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool block_size_ok(int bs) { return bs == 64 || bs == 128 || bs == 256 || bs == 512; }

int log2_block(int bs) { return bs == 512 ? 9 : bs == 256 ? 8 : bs == 128 ? 7 : 6; }

// 64-token attention tiles in top_k blocks
int tiles_of(const dsa_paged_kv* kv, int top_k) { return top_k << (log2_block(kv->block_size) - 6); }

// Token positions and 64-token tile ids of the pool are 32-bit in the kernels.
dsa_status check_extent(const dsa_paged_kv* kv) {
  if (kv->kv_layout != DSA_KV_TOKEN_MAJOR && kv->kv_layout != DSA_KV_HEAD_MAJOR)
    return fail(DSA_ERR_UNSUPPORTED, "kv_layout %d: supported 0 (token-major), 1 (head-major)",
                kv->kv_layout);
  if ((long long)kv->max_blocks_per_seq * kv->block_size > INT32_MAX ||
      (long long)kv->num_blocks * kv->block_size > INT32_MAX * 64LL)
    return fail(DSA_ERR_UNSUPPORTED, "max_blocks_per_seq * block_size (or the pool's 64-token tiles) "
                                     "exceed 2^31 - 1");
  return DSA_OK;
}

enum Need : unsigned {
  kNeedIndex = 1u,  // idx_keys, idx_scale, q_idx, w_idx
  kNeedAttn = 2u,   // k_cache, v_cache, q
};

dsa_status check_common(const dsa_paged_kv* kv, const dsa_queries* qs, unsigned need) {
  if (!kv || !qs) return fail(DSA_ERR_NULL, "kv and qs must not be NULL");
  if (qs->num_queries < 0) return fail(DSA_ERR_SHAPE, "num_queries < 0");
  if (qs->num_queries > 65535)
    return fail(DSA_ERR_UNSUPPORTED, "num_queries %d: at most 65535 per call (one grid row per query)",
                qs->num_queries);
  if (!block_size_ok(kv->block_size))
    return fail(DSA_ERR_UNSUPPORTED, "block_size %d: supported 64, 128, 256, 512", kv->block_size);
  if (kv->head_dim != dsa::kHeadDim)
    return fail(DSA_ERR_UNSUPPORTED, "head_dim %d: the library supports 128 only", kv->head_dim);
  if (kv->num_blocks < 1 || kv->num_seqs < 1 || kv->max_blocks_per_seq < 1 ||
      kv->num_kv_heads < 1)
    return fail(DSA_ERR_SHAPE, "num_blocks, num_seqs, max_blocks_per_seq, num_kv_heads must be >= 1");
  if (check_extent(kv) != DSA_OK) return DSA_ERR_UNSUPPORTED;
  if (!kv->block_table || !kv->seq_lens) return fail(DSA_ERR_NULL, "block_table/seq_lens NULL");
  if (!qs->q_seq && qs->num_queries > kv->num_seqs)
    return fail(DSA_ERR_SHAPE, "decode batch (q_seq NULL) needs num_queries <= num_seqs");
  if (need & kNeedIndex) {
    if (kv->idx_dim != 64 && kv->idx_dim != 128)
      return fail(DSA_ERR_UNSUPPORTED, "idx_dim %d: supported 64, 128", kv->idx_dim);
    if (qs->idx_heads < 1 || qs->idx_heads > dsa::kMaxIdxHeads)
      return fail(DSA_ERR_UNSUPPORTED, "idx_heads %d: supported 1..16", qs->idx_heads);
    if (!kv->idx_keys || !kv->idx_scale || !qs->q_idx || !qs->w_idx)
      return fail(DSA_ERR_NULL, "idx_keys/idx_scale/q_idx/w_idx NULL");
    if (!aligned(kv->idx_keys, 16) || !aligned(qs->q_idx, 16) || !aligned(kv->idx_scale, 4) ||
        !aligned(qs->w_idx, 4))
      return fail(DSA_ERR_ALIGN, "idx_keys/q_idx need 16 B, idx_scale/w_idx 4 B alignment");
  }
  if (need & kNeedAttn) {
    if (qs->num_q_heads < 1 || qs->num_q_heads % kv->num_kv_heads != 0)
      return fail(DSA_ERR_SHAPE, "num_q_heads %d must be a positive multiple of num_kv_heads %d",
                  qs->num_q_heads, kv->num_kv_heads);
    if (qs->num_q_heads / kv->num_kv_heads > dsa::kMaxGroup)
      return fail(DSA_ERR_UNSUPPORTED, "more than 16 query heads per KV head");
    if (!kv->k_cache || !kv->v_cache || !qs->q) return fail(DSA_ERR_NULL, "k_cache/v_cache/q NULL");
    if (!aligned(kv->k_cache, 16) || !aligned(kv->v_cache, 16) || !aligned(qs->q, 16))
      return fail(DSA_ERR_ALIGN, "k_cache/v_cache/q need 16 B alignment");
  }
  return DSA_OK;
}

dsa_status check_topk(int32_t top_k) {
  if (top_k < 1 || top_k > dsa::kMaxTopK) return fail(DSA_ERR_SHAPE, "top_k %d not in 1..4096", top_k);
  return DSA_OK;
}

dsa::KvView kv_view(const dsa_paged_kv* kv) {
  dsa::KvView v;
  v.k = static_cast<const uint16_t*>(kv->k_cache);
  v.v = static_cast<const uint16_t*>(kv->v_cache);
  v.idx_keys = kv->idx_keys;
  v.idx_scale = kv->idx_scale;
  v.table = kv->block_table;
  v.seq_lens = kv->seq_lens;
  v.num_blocks = kv->num_blocks;
  v.num_kv_heads = kv->num_kv_heads;
  v.idx_dim = kv->idx_dim;
  v.num_seqs = kv->num_seqs;
  v.maxb = kv->max_blocks_per_seq;
  v.bs_shift = log2_block(kv->block_size);
  v.head_major = kv->kv_layout == DSA_KV_HEAD_MAJOR;
  return v;
}

dsa::QView q_view(const dsa_queries* qs) {
  dsa::QView v;
  v.nq = qs->num_queries;
  v.hq = qs->num_q_heads;
  v.hi = qs->idx_heads;
  v.q_seq = qs->q_seq;
  v.q_pos = qs->q_pos;
  v.q = static_cast<const uint16_t*>(qs->q);
  v.q_idx = static_cast<const uint16_t*>(qs->q_idx);
  v.w = qs->w_idx;
  return v;
}

size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

// Attention workspace: split partials.
struct AttnLayout {
  size_t partials, total;
  dsa::AttnPlan plan;
};

AttnLayout attn_layout(const dsa_paged_kv* kv, const dsa_queries* qs, int top_k, size_t base) {
  AttnLayout a;
  a.plan = dsa::attn_plan(qs->num_queries, kv->num_kv_heads, tiles_of(kv, top_k), false);
  a.partials = base;
  a.total = align_up(a.partials + dsa::attn_partials_bytes(qs->num_queries, qs->num_q_heads,
                                                           a.plan.splits));
  if (a.plan.splits <= 1) a.total = base;
  return a;
}

// Fused-decode workspace: attention layout | scores | idx | cnt.
// Scoring and Top-K selection into (idx, cnt), the cheapest route for the
// shape; scores: nq * max_blocks_per_seq floats of scratch.
dsa_status select_blocks(const dsa::KvView& kvv, const dsa::QView& qv, int top_k, int32_t* idx,
                         int32_t* cnt, float* scores, hipStream_t stream, const char* who) {
  char what[96];
  if (dsa::index_topk_fp8_supported(kvv, qv)) {
    snprintf(what, sizeof what, "%s: fp8 index_topk launch", who);
    return hip_status(dsa::launch_index_topk_fp8(kvv, qv, top_k, idx, cnt, stream), what);
  }
  if (dsa::index_topk_fused_supported(kvv, qv)) {
    snprintf(what, sizeof what, "%s: index_topk fused launch", who);
    return hip_status(dsa::launch_index_topk_fused(kvv, qv, top_k, idx, cnt, stream), what);
  }
  if (dsa::index_cand_topk_supported(kvv, qv, top_k)) {
    snprintf(what, sizeof what, "%s: candidate launch", who);
    return hip_status(dsa::launch_index_cand_topk(kvv, qv, top_k, scores, idx, cnt, stream), what);
  }
  hipError_t e = dsa::launch_index_score(kvv, qv, scores, stream);
  if (e != hipSuccess) {
    snprintf(what, sizeof what, "%s: score launch", who);
    return hip_status(e, what);
  }
  snprintf(what, sizeof what, "%s: topk launch", who);
  return hip_status(dsa::launch_topk(scores, kvv, qv, top_k, idx, cnt, stream), what);
}

// Fused prefill workspace: scores, the selection, then the block-inverted
// attention's CSR lists and partial states.
struct PrefillLayout {
  size_t scores, idx, cnt, total;
  dsa::InvLayout inv;
};
PrefillLayout prefill_layout(const dsa_paged_kv* kv, const dsa_queries* qs, int top_k) {
  PrefillLayout f;
  const size_t nq = (size_t)qs->num_queries;
  f.scores = 0;
  f.idx = align_up(nq * kv->max_blocks_per_seq * sizeof(float));
  f.cnt = align_up(f.idx + nq * top_k * sizeof(int32_t));
  f.inv = dsa::inv_layout(kv_view(kv), qs->num_queries, qs->num_q_heads, top_k,
                          align_up(f.cnt + nq * sizeof(int32_t)));
  f.total = f.inv.total;
  return f;
}

struct FusedLayout {
  AttnLayout attn;
  size_t scores, idx, cnt, sync, total;
};

FusedLayout fused_layout(const dsa_paged_kv* kv, const dsa_queries* qs, int top_k) {
  FusedLayout f;
  const size_t nq = (size_t)qs->num_queries;
  f.attn = attn_layout(kv, qs, top_k, 0);
  f.scores = align_up(f.attn.total);
  f.idx = align_up(f.scores + nq * kv->max_blocks_per_seq * sizeof(float));
  f.cnt = align_up(f.idx + nq * top_k * sizeof(int32_t));
  f.sync = align_up(f.cnt + nq * sizeof(int32_t));
  // split counters of the long-context path's attention launch
  f.total = align_up(f.sync + dsa::attn_done_bytes(qs->num_queries, kv->num_kv_heads));
  return f;
}

// Arguments of the fused decode, checked on the host (no GPU call).
dsa_status check_decode_fused(const dsa_paged_kv* kv, const dsa_queries* qs, int32_t top_k,
                              float* out, int32_t* block_idx_out, int32_t* block_cnt_out) {
  dsa_status st = check_common(kv, qs, kNeedAttn | kNeedIndex);
  if (st != DSA_OK) return st;
  if ((st = check_topk(top_k)) != DSA_OK) return st;
  if (!out) return fail(DSA_ERR_NULL, "out NULL");
  if (!aligned(out, 4)) return fail(DSA_ERR_ALIGN, "out needs 4 B alignment");
  if ((block_idx_out && !aligned(block_idx_out, 4)) || (block_cnt_out && !aligned(block_cnt_out, 4)))
    return fail(DSA_ERR_ALIGN, "block_idx_out/block_cnt_out need 4 B alignment");
  return DSA_OK;
}

// The fused decode on a checked call and a workspace of f.total bytes.
dsa_status decode_fused_on(const dsa_paged_kv* kv, const dsa_queries* qs, int32_t top_k,
                           float softmax_scale, float* out, float* lse, int32_t* block_idx_out,
                           int32_t* block_cnt_out, const FusedLayout& f, char* ws,
                           hipStream_t stream) {
  float* scores = reinterpret_cast<float*>(ws + f.scores);
  int32_t* idx = block_idx_out ? block_idx_out : reinterpret_cast<int32_t*>(ws + f.idx);
  int32_t* cnt = block_cnt_out ? block_cnt_out : reinterpret_cast<int32_t*>(ws + f.cnt);
  const dsa::KvView kvv = kv_view(kv);
  const dsa::QView qv = q_view(qs);
  const bool split = f.attn.plan.splits > 1;
  float* partials = split ? reinterpret_cast<float*>(ws + f.attn.partials) : nullptr;
  hipError_t e;
  if (dsa::attn_score_supported(kvv, qv, top_k, f.attn.plan)) {
    // short contexts, small grids: every attention workgroup scores and
    // selects its query's blocks itself, in one launch
    e = dsa::launch_sparse_attn_score(kvv, qv, top_k, softmax_scale, out, lse, partials,
                                      f.attn.plan, block_idx_out, block_cnt_out, stream);
    return hip_status(e, "fused: score + select + attention launch");
  }
  if (dsa::index_topk_fused_supported(kvv, qv)) {
    // short contexts: scoring and selection in one kernel
    e = dsa::launch_index_topk_fused(kvv, qv, top_k, idx, cnt, stream);
    if (e != hipSuccess) return hip_status(e, "fused: index_topk launch");
  } else if (dsa::index_cand_topk_supported(kvv, qv, top_k)) {
    // long contexts, small K: per-chunk candidates, merged by the attention
    // workgroups themselves (which also merge their splits), or else by a
    // merging kernel first
    if (dsa::attn_cand_supported(kvv, qv, top_k, f.attn.plan)) {
      uint32_t* done = reinterpret_cast<uint32_t*>(ws + f.sync);
      e = dsa::launch_index_cand_scores(kvv, qv, top_k, scores, done, stream);
      if (e != hipSuccess) return hip_status(e, "fused: candidate scoring launch");
      e = dsa::launch_sparse_attn_cand(kvv, qv, scores, top_k, softmax_scale, out, lse, partials,
                                       f.attn.plan, block_idx_out, block_cnt_out, done, stream);
      return hip_status(e, "fused: candidate merge + attention launch");
    }
    e = dsa::launch_index_cand_topk(kvv, qv, top_k, scores, idx, cnt, stream);
    if (e != hipSuccess) return hip_status(e, "fused: index_cand_topk launch");
  } else {
    e = dsa::launch_index_score(kvv, qv, scores, stream);
    if (e != hipSuccess) return hip_status(e, "fused: index_score launch");
    if (dsa::attn_select_supported(kvv, qv, top_k, f.attn.plan)) {
      // the attention workgroups select their query's blocks themselves
      e = dsa::launch_sparse_attn_select(kvv, qv, scores, top_k, softmax_scale, out, lse, partials,
                                         f.attn.plan, block_idx_out, block_cnt_out, stream);
      return hip_status(e, "fused: select + attention launch");
    }
    e = dsa::launch_topk(scores, kvv, qv, top_k, idx, cnt, stream);
    if (e != hipSuccess) return hip_status(e, "fused: topk launch");
  }
  e = dsa::launch_sparse_attn(kvv, qv, idx, cnt, top_k, softmax_scale, out, lse, partials,
                              f.attn.plan, stream);
  return hip_status(e, "fused: attention launch");
}

// Scratch of dsa_sparse_decode_fused_noalloc: one array per GPU, held until
// the process ends.  Host code never passes the array's name to a kernel (on
// the host it is a stand-in, not a device address): it uses the address
// hipGetSymbolAddress returns for the current device, resolved once per
// device and kept.
static __device__ __align__(256) char scratch[DSA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

dsa_status scratch_of_current_device(char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(DSA_ERR_UNSUPPORTED, "noalloc: device %d beyond the %d this library tracks", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "noalloc: hipGetSymbolAddress(scratch)");
    if (!p) return fail(DSA_ERR_HIP, "noalloc: scratch has no device address");
    g_scratch_ptr[dev] = static_cast<char*>(p);
  }
  *out = g_scratch_ptr[dev];
  return DSA_OK;
}

}  // namespace

extern "C" {

int dsa_abi_version(void) { return DSA_ABI_VERSION; }

const char* dsa_last_error(void) { return g_err; }

const char* dsa_status_str(dsa_status s) {
  switch (s) {
    case DSA_OK: return "ok";
    case DSA_ERR_NULL: return "null pointer";
    case DSA_ERR_SHAPE: return "bad shape";
    case DSA_ERR_UNSUPPORTED: return "unsupported size";
    case DSA_ERR_ALIGN: return "misaligned pointer";
    case DSA_ERR_WORKSPACE: return "workspace too small";
    case DSA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

dsa_status dsa_workspace_size(int op, const dsa_paged_kv* kv, const dsa_queries* qs,
                              int32_t top_k, size_t* bytes) {
  if (!bytes) return fail(DSA_ERR_NULL, "bytes NULL");
  *bytes = 0;
  dsa_status st;
  switch (op) {
    case DSA_OP_ATTN_DECODE: {
      if ((st = check_common(kv, qs, kNeedAttn)) != DSA_OK) return st;
      if ((st = check_topk(top_k)) != DSA_OK) return st;
      *bytes = attn_layout(kv, qs, top_k, 0).total;
      return ok();
    }
    case DSA_OP_DECODE_FUSED: {
      if ((st = check_common(kv, qs, kNeedAttn | kNeedIndex)) != DSA_OK) return st;
      if ((st = check_topk(top_k)) != DSA_OK) return st;
      *bytes = fused_layout(kv, qs, top_k).total;
      return ok();
    }
    case DSA_OP_PREFILL_FUSED: {
      if ((st = check_common(kv, qs, kNeedAttn | kNeedIndex)) != DSA_OK) return st;
      if ((st = check_topk(top_k)) != DSA_OK) return st;
      *bytes = prefill_layout(kv, qs, top_k).total;
      return ok();
    }
    case DSA_OP_INDEX_TOPK: {
      if ((st = check_common(kv, qs, kNeedIndex)) != DSA_OK) return st;
      if ((st = check_topk(top_k)) != DSA_OK) return st;
      *bytes = align_up((size_t)qs->num_queries * kv->max_blocks_per_seq * sizeof(float));
      return ok();
    }
  }
  return fail(DSA_ERR_SHAPE, "unknown op %d", op);
}

dsa_status dsa_index_score(const dsa_paged_kv* kv, const dsa_queries* qs, float* scores,
                           hipStream_t stream) {
  dsa_status st = check_common(kv, qs, kNeedIndex);
  if (st != DSA_OK) return st;
  if (!scores) return fail(DSA_ERR_NULL, "scores NULL");
  if (!aligned(scores, 4)) return fail(DSA_ERR_ALIGN, "scores needs 4 B alignment");
  if (qs->num_queries == 0) return ok();
  return hip_status(dsa::launch_index_score(kv_view(kv), q_view(qs), scores, stream),
                    "index_score launch");
}

dsa_status dsa_topk_blocks(const float* scores, const dsa_paged_kv* kv, const dsa_queries* qs,
                           int32_t top_k, int32_t* block_idx, int32_t* block_cnt,
                           hipStream_t stream) {
  dsa_status st = check_common(kv, qs, 0);
  if (st != DSA_OK) return st;
  if ((st = check_topk(top_k)) != DSA_OK) return st;
  if (!scores || !block_idx || !block_cnt) return fail(DSA_ERR_NULL, "scores/block_idx/block_cnt NULL");
  if (!aligned(scores, 4) || !aligned(block_idx, 4) || !aligned(block_cnt, 4))
    return fail(DSA_ERR_ALIGN, "scores/block_idx/block_cnt need 4 B alignment");
  if (qs->num_queries == 0) return ok();
  return hip_status(dsa::launch_topk(scores, kv_view(kv), q_view(qs), top_k, block_idx, block_cnt,
                                     stream),
                    "topk launch");
}

static dsa_status attn_common(const dsa_paged_kv* kv, const dsa_queries* qs,
                              const int32_t* block_idx, const int32_t* block_cnt, int32_t top_k,
                              float* out) {
  dsa_status st = check_common(kv, qs, kNeedAttn);
  if (st != DSA_OK) return st;
  if ((st = check_topk(top_k)) != DSA_OK) return st;
  if (!block_idx || !block_cnt || !out) return fail(DSA_ERR_NULL, "block_idx/block_cnt/out NULL");
  if (!aligned(block_idx, 4) || !aligned(block_cnt, 4) || !aligned(out, 4))
    return fail(DSA_ERR_ALIGN, "block_idx/block_cnt/out need 4 B alignment");
  return DSA_OK;
}

dsa_status dsa_sparse_attn_decode(const dsa_paged_kv* kv, const dsa_queries* qs,
                                  const int32_t* block_idx, const int32_t* block_cnt,
                                  int32_t top_k, float softmax_scale, float* out, float* lse,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  dsa_status st = attn_common(kv, qs, block_idx, block_cnt, top_k, out);
  if (st != DSA_OK) return st;
  const AttnLayout a = attn_layout(kv, qs, top_k, 0);
  const size_t need = a.total;
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "workspace %zu B < required %zu B", workspace_bytes, need);
  if (need > 0 && !aligned(workspace, 256)) return fail(DSA_ERR_ALIGN, "workspace needs 256 B alignment");
  if (qs->num_queries == 0) return ok();
  char* ws = static_cast<char*>(workspace);
  return hip_status(
      dsa::launch_sparse_attn(kv_view(kv), q_view(qs), block_idx, block_cnt, top_k,
                              softmax_scale, out, lse,
                              a.plan.splits > 1 ? reinterpret_cast<float*>(ws + a.partials)
                                                : nullptr,
                              a.plan, stream),
      "sparse_attn_decode launch");
}

dsa_status dsa_sparse_attn_decode_topk(const dsa_paged_kv* kv, const dsa_queries* qs,
                                       const float* scores, int32_t top_k, float softmax_scale,
                                       float* out, float* lse, int32_t* block_idx_out,
                                       int32_t* block_cnt_out, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
  dsa_status st = check_common(kv, qs, kNeedAttn);
  if (st != DSA_OK) return st;
  if ((st = check_topk(top_k)) != DSA_OK) return st;
  if (!scores || !out) return fail(DSA_ERR_NULL, "scores/out NULL");
  if (!aligned(scores, 4) || !aligned(out, 4) || (lse && !aligned(lse, 4)) ||
      (block_idx_out && !aligned(block_idx_out, 4)) || (block_cnt_out && !aligned(block_cnt_out, 4)))
    return fail(DSA_ERR_ALIGN, "scores/out/lse/block_idx_out/block_cnt_out need 4 B alignment");
  if (kv->max_blocks_per_seq > 2048 || top_k > 2048)
    return fail(DSA_ERR_UNSUPPORTED, "selection inside attention: at most 2048 blocks per "
                "sequence and top_k <= 2048 (got %d, %d)", kv->max_blocks_per_seq, top_k);
  const AttnLayout a = attn_layout(kv, qs, top_k, 0);
  const size_t need = a.total;
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "workspace %zu B < required %zu B", workspace_bytes, need);
  if (need > 0 && !aligned(workspace, 256)) return fail(DSA_ERR_ALIGN, "workspace needs 256 B alignment");
  if (qs->num_queries == 0) return ok();
  // the selecting kernel runs four waves a workgroup; the eight-wave plan of a
  // short list (one split, no partials) becomes the four-wave one
  dsa::AttnPlan plan = a.plan;
  if (plan.waves != 4) {
    plan.waves = 4;
    plan.splits = 1;
  }
  char* ws = static_cast<char*>(workspace);
  return hip_status(
      dsa::launch_sparse_attn_select(kv_view(kv), q_view(qs), scores, top_k, softmax_scale, out,
                                     lse, plan.splits > 1 ? reinterpret_cast<float*>(ws + a.partials)
                                                          : nullptr,
                                     plan, block_idx_out, block_cnt_out, stream),
      "sparse_attn_decode_topk launch");
}

dsa_status dsa_sparse_attn_prefill(const dsa_paged_kv* kv, const dsa_queries* qs,
                                   const int32_t* block_idx, const int32_t* block_cnt,
                                   int32_t top_k, float softmax_scale, float* out, float* lse,
                                   hipStream_t stream) {
  dsa_status st = attn_common(kv, qs, block_idx, block_cnt, top_k, out);
  if (st != DSA_OK) return st;
  if (!qs->q_seq || !qs->q_pos) return fail(DSA_ERR_NULL, "prefill needs q_seq and q_pos");
  if (qs->num_queries == 0) return ok();
  return hip_status(dsa::launch_sparse_attn(kv_view(kv), q_view(qs), block_idx, block_cnt, top_k,
                                            softmax_scale, out, lse, nullptr,
                                            dsa::attn_plan(qs->num_queries, kv->num_kv_heads,
                                                           tiles_of(kv, top_k), true),
                                            stream),
                    "sparse_attn_prefill launch");
}

dsa_status dsa_sparse_decode_fused(const dsa_paged_kv* kv, const dsa_queries* qs, int32_t top_k,
                                   float softmax_scale, float* out, float* lse,
                                   int32_t* block_idx_out, int32_t* block_cnt_out,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  dsa_status st = check_decode_fused(kv, qs, top_k, out, block_idx_out, block_cnt_out);
  if (st != DSA_OK) return st;
  const FusedLayout f = fused_layout(kv, qs, top_k);
  if (!workspace || workspace_bytes < f.total)
    return fail(DSA_ERR_WORKSPACE, "workspace %zu B < required %zu B", workspace_bytes, f.total);
  if (!aligned(workspace, 256)) return fail(DSA_ERR_ALIGN, "workspace needs 256 B alignment");
  if (qs->num_queries == 0) return ok();
  return decode_fused_on(kv, qs, top_k, softmax_scale, out, lse, block_idx_out, block_cnt_out, f,
                         static_cast<char*>(workspace), stream);
}

dsa_status dsa_sparse_decode_fused_noalloc(const dsa_paged_kv* kv, const dsa_queries* qs,
                                           int32_t top_k, float softmax_scale, float* out,
                                           float* lse, int32_t* block_idx_out,
                                           int32_t* block_cnt_out, hipStream_t stream) {
  dsa_status st = check_decode_fused(kv, qs, top_k, out, block_idx_out, block_cnt_out);
  if (st != DSA_OK) return st;
  const FusedLayout f = fused_layout(kv, qs, top_k);
  if (f.total > (size_t)DSA_NOALLOC_SCRATCH_BYTES)
    return fail(DSA_ERR_UNSUPPORTED,
                "the call needs %zu B of scratch, more than the %d B this entry point holds; "
                "use dsa_sparse_decode_fused with a workspace",
                f.total, DSA_NOALLOC_SCRATCH_BYTES);
  if (qs->num_queries == 0) return ok();
  char* ws = nullptr;
  if ((st = scratch_of_current_device(&ws)) != DSA_OK) return st;
  return decode_fused_on(kv, qs, top_k, softmax_scale, out, lse, block_idx_out, block_cnt_out, f,
                         ws, stream);
}

dsa_status dsa_index_topk(const dsa_paged_kv* kv, const dsa_queries* qs, int32_t top_k,
                          int32_t* block_idx, int32_t* block_cnt, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  dsa_status st = check_common(kv, qs, kNeedIndex);
  if (st != DSA_OK) return st;
  if ((st = check_topk(top_k)) != DSA_OK) return st;
  if (!block_idx || !block_cnt) return fail(DSA_ERR_NULL, "block_idx/block_cnt NULL");
  if (!aligned(block_idx, 4) || !aligned(block_cnt, 4))
    return fail(DSA_ERR_ALIGN, "block_idx/block_cnt need 4 B alignment");
  const size_t need = align_up((size_t)qs->num_queries * kv->max_blocks_per_seq * sizeof(float));
  if (!workspace || workspace_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "workspace %zu B < required %zu B", workspace_bytes, need);
  if (!aligned(workspace, 256)) return fail(DSA_ERR_ALIGN, "workspace needs 256 B alignment");
  if (qs->num_queries == 0) return ok();
  return select_blocks(kv_view(kv), q_view(qs), top_k, block_idx, block_cnt,
                       static_cast<float*>(workspace), stream, "index_topk");
}

dsa_status dsa_sparse_prefill_fused(const dsa_paged_kv* kv, const dsa_queries* qs, int32_t top_k,
                                    float softmax_scale, float* out, float* lse,
                                    int32_t* block_idx_out, int32_t* block_cnt_out,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  dsa_status st = check_common(kv, qs, kNeedAttn | kNeedIndex);
  if (st != DSA_OK) return st;
  if ((st = check_topk(top_k)) != DSA_OK) return st;
  if (!qs->q_seq || !qs->q_pos) return fail(DSA_ERR_NULL, "prefill needs q_seq and q_pos");
  if (!out) return fail(DSA_ERR_NULL, "out NULL");
  if (!aligned(out, 8) || (lse && !aligned(lse, 4)))
    return fail(DSA_ERR_ALIGN, "out needs 8 B alignment, lse 4 B");
  if ((block_idx_out && !aligned(block_idx_out, 4)) || (block_cnt_out && !aligned(block_cnt_out, 4)))
    return fail(DSA_ERR_ALIGN, "block_idx_out/block_cnt_out need 4 B alignment");
  if ((block_idx_out == nullptr) != (block_cnt_out == nullptr))
    return fail(DSA_ERR_NULL, "block_idx_out and block_cnt_out go together");
  const PrefillLayout f = prefill_layout(kv, qs, top_k);
  if (!workspace || workspace_bytes < f.total)
    return fail(DSA_ERR_WORKSPACE, "workspace %zu B < required %zu B", workspace_bytes, f.total);
  if (!aligned(workspace, 256)) return fail(DSA_ERR_ALIGN, "workspace needs 256 B alignment");
  if (qs->num_queries == 0) return ok();
  char* ws = static_cast<char*>(workspace);
  int32_t* idx = block_idx_out ? block_idx_out : reinterpret_cast<int32_t*>(ws + f.idx);
  int32_t* cnt = block_cnt_out ? block_cnt_out : reinterpret_cast<int32_t*>(ws + f.cnt);
  const dsa::KvView kvv = kv_view(kv);
  const dsa::QView qv = q_view(qs);
  st = select_blocks(kvv, qv, top_k, idx, cnt, reinterpret_cast<float*>(ws + f.scores), stream,
                     "prefill_fused");
  if (st != DSA_OK) return st;
  return hip_status(dsa::launch_prefill_inv(kvv, qv, idx, cnt, top_k, softmax_scale, out, lse, ws,
                                            f.inv, stream),
                    "prefill_fused: block-inverted attention launch");
}

dsa_status dsa_kv_write(const dsa_paged_kv* kv, int32_t n_tokens, const int32_t* tok_seq,
                        const int32_t* tok_pos, const void* k_new, const void* v_new,
                        hipStream_t stream) {
  if (!kv) return fail(DSA_ERR_NULL, "kv must not be NULL");
  if (n_tokens < 0) return fail(DSA_ERR_SHAPE, "n_tokens < 0");
  if (!block_size_ok(kv->block_size))
    return fail(DSA_ERR_UNSUPPORTED, "block_size %d: supported 64, 128, 256, 512", kv->block_size);
  if (kv->head_dim != dsa::kHeadDim)
    return fail(DSA_ERR_UNSUPPORTED, "head_dim %d: the library supports 128 only", kv->head_dim);
  if (kv->num_blocks < 1 || kv->num_seqs < 1 || kv->max_blocks_per_seq < 1 ||
      kv->num_kv_heads < 1)
    return fail(DSA_ERR_SHAPE, "num_blocks, num_seqs, max_blocks_per_seq, num_kv_heads must be >= 1");
  if (check_extent(kv) != DSA_OK) return DSA_ERR_UNSUPPORTED;
  if (!kv->k_cache || !kv->v_cache || !kv->block_table || !kv->seq_lens)
    return fail(DSA_ERR_NULL, "k_cache/v_cache/block_table/seq_lens NULL");
  if (n_tokens > 0 && (!k_new || !v_new)) return fail(DSA_ERR_NULL, "k_new/v_new NULL");
  if (!aligned(kv->k_cache, 16) || !aligned(kv->v_cache, 16) || !aligned(k_new, 16) ||
      !aligned(v_new, 16))
    return fail(DSA_ERR_ALIGN, "k_cache/v_cache/k_new/v_new need 16 B alignment");
  if (!tok_seq && n_tokens > kv->num_seqs)
    return fail(DSA_ERR_SHAPE, "tok_seq NULL needs n_tokens <= num_seqs");
  if (n_tokens == 0) return ok();
  const dsa::KvView kvv = kv_view(kv);
  return hip_status(dsa::launch_kv_write(kvv, n_tokens, tok_seq, tok_pos, k_new, v_new,
                                         const_cast<void*>(kv->k_cache),
                                         const_cast<void*>(kv->v_cache), stream),
                    "kv_write launch");
}

dsa_status dsa_index_key_write(const dsa_paged_kv* kv, int32_t n_blocks, const int32_t* block_ids,
                               const float* coarse, hipStream_t stream) {
  if (!kv) return fail(DSA_ERR_NULL, "kv must not be NULL");
  if (n_blocks < 0) return fail(DSA_ERR_SHAPE, "n_blocks < 0");
  if (kv->num_blocks < 1) return fail(DSA_ERR_SHAPE, "num_blocks must be >= 1");
  if (kv->idx_dim != 64 && kv->idx_dim != 128)
    return fail(DSA_ERR_UNSUPPORTED, "idx_dim %d: supported 64, 128", kv->idx_dim);
  if (!kv->idx_keys || !kv->idx_scale) return fail(DSA_ERR_NULL, "idx_keys/idx_scale NULL");
  if (n_blocks > 0 && (!block_ids || !coarse)) return fail(DSA_ERR_NULL, "block_ids/coarse NULL");
  if (!aligned(block_ids, 4) || !aligned(coarse, 4) || !aligned(kv->idx_scale, 4))
    return fail(DSA_ERR_ALIGN, "block_ids/coarse/idx_scale need 4 B alignment");
  if (n_blocks == 0) return ok();
  const dsa::KvView kvv = kv_view(kv);
  return hip_status(dsa::launch_index_key_write(kvv, n_blocks, block_ids, coarse,
                                                const_cast<uint8_t*>(kv->idx_keys),
                                                const_cast<float*>(kv->idx_scale), stream),
                    "index_key_write launch");
}

// ---------------------------------------------------------------------------
// MXFP4 expert weights
// ---------------------------------------------------------------------------
namespace {
dsa_status check_experts(const dsa_mx_experts* w) {
  if (!w) return fail(DSA_ERR_NULL, "experts must not be NULL");
  if (!w->w_fp4 || !w->w_scale) return fail(DSA_ERR_NULL, "w_fp4/w_scale NULL");
  if (w->num_experts < 1 || w->n < 1 || w->k < 128)
    return fail(DSA_ERR_SHAPE, "num_experts, n >= 1 and k >= 128 required");
  if (w->k % 128) return fail(DSA_ERR_UNSUPPORTED, "k %d: a multiple of 128 required", w->k);
  if ((long long)w->num_experts * w->n * (w->k / 2) > (1LL << 46) ||
      (long long)w->n * w->k >= (1LL << 31))
    return fail(DSA_ERR_UNSUPPORTED, "weights too large (n * k must stay below 2^31)");
  if (!aligned(w->w_fp4, 16)) return fail(DSA_ERR_ALIGN, "w_fp4 needs 16 B alignment");
  return DSA_OK;
}
dsa::MxExperts mx_view(const dsa_mx_experts* w) {
  dsa::MxExperts m;
  m.fp4 = w->w_fp4;
  m.scale = w->w_scale;
  m.num_experts = w->num_experts;
  m.n = w->n;
  m.k = w->k;
  return m;
}
}  // namespace

dsa_status dsa_mx_quantize(const void* x, int32_t rows, int32_t k, uint8_t* codes, uint8_t* scales,
                           hipStream_t stream) {
  if (rows < 0 || k < 0) return fail(DSA_ERR_SHAPE, "rows, k >= 0 required");
  if (k % 32) return fail(DSA_ERR_UNSUPPORTED, "k %d: a multiple of 32 required", k);
  if (rows == 0 || k == 0) return ok();
  if (!x || !codes || !scales) return fail(DSA_ERR_NULL, "x/codes/scales NULL");
  if (!aligned(x, 16) || !aligned(codes, 16)) return fail(DSA_ERR_ALIGN, "x/codes need 16 B alignment");
  return hip_status(dsa::launch_mx_quant_act(static_cast<const uint16_t*>(x), rows, k, codes, scales,
                                             stream),
                    "mx_quantize launch");
}

dsa_status dsa_mxfp4_to_fp8(const dsa_mx_experts* w, const int32_t* experts, int32_t n_experts,
                            uint8_t* ws_codes, uint8_t* ws_scales, hipStream_t stream) {
  dsa_status st = check_experts(w);
  if (st != DSA_OK) return st;
  if (n_experts < 0) return fail(DSA_ERR_SHAPE, "n_experts < 0");
  if (n_experts == 0) return ok();
  if (!experts || !ws_codes || !ws_scales) return fail(DSA_ERR_NULL, "experts/ws_codes/ws_scales NULL");
  if (!aligned(ws_codes, 16)) return fail(DSA_ERR_ALIGN, "ws_codes needs 16 B alignment");
  return hip_status(dsa::launch_mxfp4_unpack(mx_view(w), experts, n_experts, ws_codes, ws_scales,
                                             stream),
                    "mxfp4_to_fp8 launch");
}

dsa_status dsa_moe_workspace_size(const dsa_mx_experts* w, int32_t tokens, int32_t slots,
                                  int32_t mode, size_t* bytes) {
  if (!bytes) return fail(DSA_ERR_NULL, "bytes NULL");
  *bytes = 0;
  dsa_status st = check_experts(w);
  if (st != DSA_OK) return st;
  if (tokens < 0 || slots < 1) return fail(DSA_ERR_SHAPE, "tokens >= 0, slots >= 1 required");
  if ((long long)tokens * slots > (1LL << 30)) return fail(DSA_ERR_UNSUPPORTED, "too many pairs");
  if (mode != DSA_MOE_FP8_WORKSPACE && mode != DSA_MOE_FP4_DIRECT)
    return fail(DSA_ERR_SHAPE, "unknown mode %d", mode);
  const dsa::MoeLayout L = dsa::moe_layout(mx_view(w), tokens * slots, mode == DSA_MOE_FP8_WORKSPACE, 0);
  // one workgroup per (row tile, column block of 128 or more): the grid must stay
  // below 2^24 workgroups
  if ((long long)L.max_tiles * ((w->n + 127) / 128) >= (1LL << 24))
    return fail(DSA_ERR_UNSUPPORTED, "too many pairs x columns for one launch");
  *bytes = L.total;
  return ok();
}

dsa_status dsa_moe_grouped_gemm(const dsa_mx_experts* w, const uint8_t* x_codes,
                                const uint8_t* x_scales, int32_t tokens, const int32_t* route,
                                int32_t slots, int32_t mode, float* out, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  size_t need = 0;
  dsa_status st = dsa_moe_workspace_size(w, tokens, slots, mode, &need);
  if (st != DSA_OK) return st;
  if (tokens == 0) return ok();
  if (!x_codes || !x_scales || !route || !out) return fail(DSA_ERR_NULL, "x_codes/x_scales/route/out NULL");
  if (!aligned(x_codes, 16) || !aligned(x_scales, 4) || !aligned(route, 4) || !aligned(out, 4))
    return fail(DSA_ERR_ALIGN, "x_codes 16 B; x_scales, route and out 4 B alignment required");
  if (!workspace || workspace_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "workspace %zu B < required %zu B", workspace_bytes, need);
  if (!aligned(workspace, 256)) return fail(DSA_ERR_ALIGN, "workspace needs 256 B alignment");
  const dsa::MxExperts m = mx_view(w);
  const bool fp8 = mode == DSA_MOE_FP8_WORKSPACE;
  return hip_status(dsa::launch_moe_gemm(m, fp8, x_codes, x_scales, tokens, route, slots, out,
                                         static_cast<char*>(workspace),
                                         dsa::moe_layout(m, tokens * slots, fp8, 0), stream),
                    "moe_grouped_gemm launch");
}

dsa_status dsa_check_inputs(const dsa_paged_kv* kv, const dsa_queries* qs,
                            const int32_t* block_idx, const int32_t* block_cnt, int32_t top_k,
                            uint32_t* flags, hipStream_t stream) {
  if (!kv || !qs || !flags) return fail(DSA_ERR_NULL, "kv, qs and flags must not be NULL");
  if (!aligned(flags, 4)) return fail(DSA_ERR_ALIGN, "flags needs 4 B alignment");
  if (qs->num_queries < 0) return fail(DSA_ERR_SHAPE, "num_queries < 0");
  if (!block_size_ok(kv->block_size))
    return fail(DSA_ERR_UNSUPPORTED, "block_size %d: supported 64, 128, 256, 512", kv->block_size);
  if (kv->num_blocks < 1 || kv->num_seqs < 1 || kv->max_blocks_per_seq < 1)
    return fail(DSA_ERR_SHAPE, "num_blocks, num_seqs, max_blocks_per_seq must be >= 1");
  if (check_extent(kv) != DSA_OK) return DSA_ERR_UNSUPPORTED;
  if (!kv->block_table || !kv->seq_lens) return fail(DSA_ERR_NULL, "block_table/seq_lens NULL");
  if (!qs->q_seq && qs->num_queries > kv->num_seqs)
    return fail(DSA_ERR_SHAPE, "decode batch (q_seq NULL) needs num_queries <= num_seqs");
  if ((block_idx == nullptr) != (block_cnt == nullptr))
    return fail(DSA_ERR_NULL, "block_idx and block_cnt go together");
  if (block_idx) {
    dsa_status st = check_topk(top_k);
    if (st != DSA_OK) return st;
    if (!aligned(block_idx, 4) || !aligned(block_cnt, 4))
      return fail(DSA_ERR_ALIGN, "block_idx/block_cnt need 4 B alignment");
  }
  dsa::KvView kvv = kv_view(kv);
  dsa::QView qv = q_view(qs);
  return hip_status(dsa::launch_check_inputs(kvv, qv, block_idx, block_cnt, top_k, flags, stream),
                    "check_inputs launch");
}

}  // extern "C"

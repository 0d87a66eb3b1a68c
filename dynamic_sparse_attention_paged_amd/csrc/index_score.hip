// Indexer scoring: one coarse FP8 key per KV block, scored against the query.
//
// What is computed ([P1] "Day-0 Adaptation for Massive LLMs...", section
// 4(1) "Index Selection"; [P5] "Day-0 Readiness for Trillion-Parameter
// Models...", "Index Selection Path": a lightweight inner product with
// low-precision inputs), for query q and visible logical block j with
// physical block p = table[s][j]:
//
//   sq[h] = 2^e[h], the smallest power of two with max|q_idx[h,:]| <= 448 sq[h]
//   q8[h,:] = E4M3(q_idx[h,:] / sq[h])              (round to nearest even)
//   D[h] = sum_d q8[h,d] k8[p,d]                     (exact)
//   S = sum_{h ascending} w[h] * max(0, (sq[h] * ks[p]) * D[h])   in float64,
//   stored rounded to fp32.
//
// Exactness: every E4M3 value is a multiple of 2^-9 below 2^9, so products
// are multiples of 2^-18 below 2^18 and any partial sum of <= 128 of them
// fits in 43 bits; float64 FMA accumulation is therefore exact in any order.
// The gfx950 FP8 MFMA does not accumulate exactly (it aligns products to the
// largest one and drops low bits), so it cannot reproduce these scores.
//
// Mapping: four lanes per logical block, each owning a quarter of the key
// row (16 or 32 B, read with 16 B loads), and one or four blocks per lane.
// The query's decoded FP8 values live in LDS as float64 [dI][HP]; a read
// serves the 16 lanes of a quarter with one broadcast address and, with four
// blocks per lane, four blocks' FMAs.
#include <hip/hip_runtime.h>
#include <math.h>

#include "dsa_internal.h"
#include "score_common.h"
#include "cand_common.h"
#include "score_i8_lds.h"
#include "select_common.h"

namespace dsa {
namespace {

constexpr int kScoreThreads = 256;

constexpr int kMergeWaves = 16;

// One workgroup per query: the local block plus the need best of the
// workgroups' candidate lists (cand_common.h); the same rule as topk.hip.
__global__ __launch_bounds__(64 * kMergeWaves) void topk_merge_candidates(
    float* __restrict__ ws, KvView kv, QView Q, int top_k, int nwg, int32_t* __restrict__ out_idx,
    int32_t* __restrict__ out_cnt) {
  __shared__ uint32_t ck[kMergeMaxCand], k2[kMergeMaxCand];
  __shared__ int32_t cj[kMergeMaxCand], j2[kMergeMaxCand], pos[kMergeMaxCand];
  __shared__ int off[kMergeMaxCand + 1];
  __shared__ int n2[kMergeWaves];
  __shared__ uint4 hist4[kMergeWaves * 64];
  __shared__ int rc[kCandScratchExtraWords];
  const int tid = threadIdx.x, lane = tid & 63;
  const int qi = blockIdx.x;
  const int s = query_seq(Q, qi);
  const int len = kv.seq_lens[s];
  const int pos_q = Q.q_pos ? Q.q_pos[qi] : len - 1;
  const int local = pos_q >> kv.bs_shift;
  const int need = top_k - 1;
  int32_t* out = out_idx + (size_t)qi * top_k;
  if (local <= need) {  // uniform over the workgroup
    for (int i = tid; i < top_k; i += 64 * kMergeWaves) out[i] = i <= local ? i : -1;
    if (tid == 0) out_cnt[qi] = local + 1;
    return;
  }
  if (need == 0) {
    if (tid == 0) {
      out[0] = local;
      out_cnt[qi] = 1;
    }
    return;
  }
  const CandScratch S{ck, cj, off, k2, j2, pos, n2, hist4, rc};
  const int c = merge_candidate_lists<kMergeWaves>(ws, nwg, need, qi, S, out);
  if (tid >= 64) return;
  if (lane == 0) {
    out[c] = local;  // c == need: the lists hold at least need candidates below local
    out_cnt[qi] = c + 1;
  }
  for (int i = c + 1 + lane; i < top_k; i += 64) out[i] = -1;
}

// Lanes: 4 per block (dims DI/4 each); a lane holds NB blocks (16 apart), so a
// wave covers 16 NB blocks and a workgroup 64 NB (score_chunk).  Blocks past
// the local block score -inf.
template <int DI, int HP, int NB>
__global__ __launch_bounds__(kScoreThreads) void index_score_exact(KvView kv, QView Q,
                                                                   float* __restrict__ scores) {
  __shared__ double qv[DI * HP];
  __shared__ double sq[HP], wq[HP];
  __shared__ int expo[HP];
  const int qi = blockIdx.y, chunk = blockIdx.x;
  float S[NB];
  bool visible[NB];
  int local;
  const bool any = score_chunk<DI, HP, NB>(kv, Q, qi, chunk, qv, sq, wq, expo, S, visible, local);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j0 = chunk * 64 * NB + wave * 16 * NB + (lane & 15);
  float* row = scores + (size_t)qi * kv.maxb;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int j = j0 + 16 * b;
    if ((lane >> 4) == 0 && j < kv.maxb) row[j] = (any && visible[b]) ? S[b] : -INFINITY;
  }
}

// grid (ceil(maxb / 64 kT), Nq), block 256: the rows of index_score_exact,
// bit for bit, from the int8 matrix cores (score_chunk_i8: 18 int8 products
// per 16 blocks instead of 256 float64 FMAs a lane).  Blocks past the local
// block score -inf.
template <int DI, int HP, int kT>
__global__ __launch_bounds__(256) void index_score_i8_rows(KvView kv, QView Q,
                                                           float* __restrict__ scores) {
  __shared__ uint32_t lut[256];
  __shared__ double wsq[16];
  __shared__ float scw[64 * kT];
  const int qi = blockIdx.y, chunk = blockIdx.x;
  int local;
  const bool any = score_chunk_i8<DI, HP, kT>(kv, Q, qi, chunk, lut, wsq, scw, local);
  if (any) __syncthreads();  // uniform: the scores are visible to every wave
  float* row = scores + (size_t)qi * kv.maxb;
  for (int e = threadIdx.x; e < 64 * kT; e += 256) {
    const int j = chunk * 64 * kT + e;
    if (j < kv.maxb) row[j] = (any && j <= local) ? scw[e] : -INFINITY;
  }
}

// grid (nwg, Nq), block 256: chunk `blockIdx.x` of query blockIdx.y scored on
// the int8 matrix cores (score_chunk_i8: the same scores as above, bit for
// bit), then its candidate list (chunk_candidates_lds; layout in
// cand_common.h).  The chunk-0 workgroup of each query also zeroes that
// query's split counters of the attention launch that follows (done:
// nq x hkv counters, one per 256-byte line; nullptr when none follows).
template <int DI, int HP>
__global__ __launch_bounds__(256) void index_cand_scores(KvView kv, QView Q, float* __restrict__ ws,
                                                         int need, uint32_t* __restrict__ done) {
  __shared__ uint32_t lut[256];
  __shared__ double wsq[16];
  __shared__ float scw[256];
  __shared__ uint4 hist4[64];
  const int qi = blockIdx.y, chunk = blockIdx.x;
  if (done && chunk == 0 && (int)threadIdx.x < kv.num_kv_heads)
    done[((size_t)qi * kv.num_kv_heads + threadIdx.x) * kDoneLineWords] = 0u;
  int local;
  const bool any = score_chunk_i8<DI, HP>(kv, Q, qi, chunk, lut, wsq, scw, local);
  if (any) __syncthreads();  // uniform: the scores are visible to wave 0
  chunk_candidates_lds<4>(any, local, scw, hist4, ws, gridDim.x, need, qi, chunk);
}

template <int DI, int HP>
hipError_t launch_t(const KvView& kv, const QView& Q, float* scores, hipStream_t st) {
  // Small jobs: one block per lane quarter, many workgroups.  Large jobs (more
  // than ~256 CUs x 256 blocks): four blocks per lane quarter, so every query
  // value read from LDS feeds four blocks.
  const long pairs = (long)Q.nq * kv.maxb;
  if (pairs >= 256L * 256) {
    dim3 grid((kv.maxb + 255) / 256, Q.nq);
    hipLaunchKernelGGL((index_score_exact<DI, HP, 4>), grid, dim3(kScoreThreads), 0, st, kv, Q,
                       scores);
  } else {
    dim3 grid((kv.maxb + 63) / 64, Q.nq);
    hipLaunchKernelGGL((index_score_exact<DI, HP, 1>), grid, dim3(kScoreThreads), 0, st, kv, Q,
                       scores);
  }
  return hipGetLastError();
}

template <int DI, int HP>
hipError_t launch_cand_t(const KvView& kv, const QView& Q, int need, float* ws, uint32_t* done,
                         hipStream_t st) {
  dim3 grid((kv.maxb + kCandBlocks - 1) / kCandBlocks, Q.nq);
  hipLaunchKernelGGL((index_cand_scores<DI, HP>), grid, dim3(256), 0, st, kv, Q, ws, need, done);
  return hipGetLastError();
}

template <int DI>
hipError_t launch_cand_di(const KvView& kv, const QView& Q, int need, float* ws, uint32_t* done,
                          hipStream_t st) {
  if (Q.hi <= 4) return launch_cand_t<DI, 4>(kv, Q, need, ws, done, st);
  if (Q.hi <= 8) return launch_cand_t<DI, 8>(kv, Q, need, ws, done, st);
  return launch_cand_t<DI, 16>(kv, Q, need, ws, done, st);
}

template <int DI, int HP>
hipError_t launch_i8_rows_t(const KvView& kv, const QView& Q, float* scores, hipStream_t st) {
  // One 16-block tile a wave (64 blocks a workgroup) while that grid fits a
  // few workgroups per CU; larger jobs (many long sequences) take eight tiles
  // a wave, so that each workgroup's query set-up (its rows quantized into
  // digit planes) serves 512 blocks (measured on 128 sequences of up to 2048
  // blocks: 22 us with one tile a wave, the decode step 6-8 us shorter).
  const long wg1 = (long)((kv.maxb + 63) / 64) * Q.nq;
  if (wg1 > 4L * device_cu_count()) {
    dim3 grid((kv.maxb + 511) / 512, Q.nq);
    hipLaunchKernelGGL((index_score_i8_rows<DI, HP, 8>), grid, dim3(256), 0, st, kv, Q, scores);
  } else {
    dim3 grid((kv.maxb + 63) / 64, Q.nq);
    hipLaunchKernelGGL((index_score_i8_rows<DI, HP, 1>), grid, dim3(256), 0, st, kv, Q, scores);
  }
  return hipGetLastError();
}

template <int DI>
hipError_t launch_di(const KvView& kv, const QView& Q, float* scores, hipStream_t st) {
  if (Q.hi <= 1) return launch_t<DI, 1>(kv, Q, scores, st);
  if (Q.hi <= 2) return launch_t<DI, 2>(kv, Q, scores, st);
  // four or more heads: the int8 matrix cores
  if (Q.hi <= 4) return launch_i8_rows_t<DI, 4>(kv, Q, scores, st);
  if (Q.hi <= 8) return launch_i8_rows_t<DI, 8>(kv, Q, scores, st);
  return launch_i8_rows_t<DI, 16>(kv, Q, scores, st);
}

}  // namespace

bool index_cand_topk_supported(const KvView& kv, const QView& Q, int top_k) {
  // long candidate lists (past what a selecting attention workgroup holds),
  // few queries, and the candidate lists fit the score workspace and one
  // merging wave
  const int need = top_k - 1;
  const int nwg = (kv.maxb + kCandBlocks - 1) / kCandBlocks;
  return kv.maxb > 2048 && need >= 1 && !index_score_mfma_supported(kv, Q) &&
         (long)nwg * need <= kMergeMaxCand && cand_query_words(nwg, need) <= (size_t)kv.maxb;
}

hipError_t launch_index_cand_scores(const KvView& kv, const QView& Q, int top_k, float* ws,
                                    uint32_t* done, hipStream_t st) {
  const int need = top_k - 1;
  return kv.idx_dim == 64 ? launch_cand_di<64>(kv, Q, need, ws, done, st)
                          : launch_cand_di<128>(kv, Q, need, ws, done, st);
}

hipError_t launch_index_cand_topk(const KvView& kv, const QView& Q, int top_k, float* ws,
                                  int32_t* idx, int32_t* cnt, hipStream_t st) {
  const int nwg = (kv.maxb + kCandBlocks - 1) / kCandBlocks;
  hipError_t e = launch_index_cand_scores(kv, Q, top_k, ws, nullptr, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_merge_candidates, dim3(Q.nq), dim3(64 * kMergeWaves), 0, st, ws, kv, Q,
                     top_k, nwg, idx, cnt);
  return hipGetLastError();
}

hipError_t launch_index_score(const KvView& kv, const QView& Q, float* scores, hipStream_t st) {
  // many queries at once: the same scores from the int8 matrix cores
  if (index_score_mfma_supported(kv, Q)) return launch_index_score_mfma(kv, Q, scores, st);
  if (kv.idx_dim == 64) return launch_di<64>(kv, Q, scores, st);
  return launch_di<128>(kv, Q, scores, st);
}

}  // namespace dsa

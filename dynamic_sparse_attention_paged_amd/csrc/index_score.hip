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
  const CandScratch S{ck, cj, off, k2, j2, pos, n2, hist4};
  const int c = merge_candidate_lists<kMergeWaves>(ws, nwg, need, qi, S, out);
  if (tid >= 64) return;
  if (lane == 0) {
    out[c] = local;  // c == need: the lists hold at least need candidates below local
    out_cnt[qi] = c + 1;
  }
  for (int i = c + 1 + lane; i < top_k; i += 64) out[i] = -1;
}

// Lanes: 4 per block (dims DI/4 each); a lane holds NB blocks (16 apart), so a
// wave covers 16 NB blocks and a workgroup 64 NB.
//
// kCand: instead of the score row, the workgroup writes its Top-K
// candidates: the need best of its blocks below the local block (equal
// scores to the lower id), as order-preserving keys and ids in increasing id
// order, with their count (layout: cand_layout below).
template <int DI, int HP, int NB, bool kCand>
__global__ __launch_bounds__(kScoreThreads) void index_score_exact(KvView kv, QView Q,
                                                                   float* __restrict__ scores,
                                                                   int need) {
  __shared__ double qv[DI * HP];
  __shared__ float scw[kCand ? 64 * NB : 1];
  __shared__ uint4 hist4[kCand ? 64 : 1];
  __shared__ double sq[HP], wq[HP];
  __shared__ int expo[HP];
  constexpr int kBlocksPerWg = 64 * NB;

  const int qi = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int gq = lane >> 4;
  const int j0 = blockIdx.x * kBlocksPerWg + wave * 16 * NB + (lane & 15);
  const int s = query_seq(Q, qi);
  float* row = scores + (size_t)qi * kv.maxb;

  // Block-table entries, key quarters and scales are requested first, before
  // the query position is known (physical ids clamped into the pool, so the
  // speculative reads stay in bounds), so that the table -> key chain
  // overlaps the position read and the query prologue.
  KeyQuarter<DI> kq[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int j = min(j0 + 16 * b, kv.maxb - 1);
    kq[b].p = min(max(kv.table[(size_t)s * kv.maxb + j], 0), kv.num_blocks - 1);
    const uint4* krow =
        reinterpret_cast<const uint4*>(kv.idx_keys + (size_t)kq[b].p * DI + gq * (DI / 4));
#pragma unroll
    for (int i = 0; i < DI / 64; ++i) kq[b].w[i] = krow[i];
    kq[b].ks = gq == 0 ? kv.idx_scale[kq[b].p] : 0.f;
  }
  const int len = kv.seq_lens[s];
  const int pos = Q.q_pos ? Q.q_pos[qi] : len - 1;
  const int local = pos >> kv.bs_shift;

  // Workgroups whose blocks are all invisible only write -inf (or no candidates).
  if (blockIdx.x * kBlocksPerWg > local) {
    if (kCand) {
      if (threadIdx.x == 0) cand_count(scores, gridDim.x, need, qi)[blockIdx.x] = 0;
      return;
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int j = j0 + 16 * b;
      if (gq == 0 && j < kv.maxb) row[j] = -INFINITY;
    }
    return;
  }
  // invisible blocks score zero key words (their result is replaced by -inf)
  bool visible[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int j = j0 + 16 * b;
    visible[b] = j <= local && j < kv.maxb;
    if (!visible[b]) {
#pragma unroll
      for (int i = 0; i < DI / 64; ++i) kq[b].w[i] = make_uint4(0u, 0u, 0u, 0u);
      kq[b].ks = 0.f;
    }
  }
  load_query<DI, HP>(Q, qi, qv, sq, wq, expo);
  float S[NB];
  score_quarters<DI, HP, NB>(kq, gq, qv, sq, wq, S);
  if (!kCand) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int j = j0 + 16 * b;
      if (gq == 0 && j < kv.maxb) row[j] = visible[b] ? S[b] : -INFINITY;
    }
    return;
  }
  // ---- candidates of this workgroup: blocks jbase + o, o < c (below local)
  if (gq == 0) {
#pragma unroll
    for (int b = 0; b < NB; ++b) scw[wave * 16 * NB + (lane & 15) + 16 * b] = S[b];
  }
  __syncthreads();
  if (wave != 0) return;
  const int jbase = blockIdx.x * kBlocksPerWg;
  const int c = min(max(local - jbase, 0), kBlocksPerWg);
  int32_t* cnt_out = cand_count(scores, gridDim.x, need, qi);
  uint32_t* keys_out = cand_keys(scores, gridDim.x, need, qi) + (size_t)blockIdx.x * need;
  int32_t* ids_out = cand_ids(scores, gridDim.x, need, qi) + (size_t)blockIdx.x * need;
  uint32_t k[NB], valid = 0u;
#pragma unroll
  for (int m = 0; m < NB; ++m) {
    const int o = lane * NB + m;
    k[m] = order_key(scw[o]);
    valid |= (o < c) ? (1u << m) : 0u;
  }
  if (c <= need) {  // all of them
#pragma unroll
    for (int m = 0; m < NB; ++m) {
      const int o = lane * NB + m;
      if (o < c) {
        keys_out[o] = k[m];
        ids_out[o] = jbase + o;
      }
    }
    if (lane == 0) cnt_out[blockIdx.x] = c;
    return;
  }
  uint32_t T, take_eq, o;
  wave_select<NB>(k, valid, (uint32_t)need, hist4, T, take_eq);
  const uint32_t keep = wave_keep<NB>(k, valid, T, take_eq, &o);
#pragma unroll
  for (int m = 0; m < NB; ++m)
    if (((keep >> m) & 1u) && o < (uint32_t)need) {
      keys_out[o] = k[m];
      ids_out[o] = jbase + lane * NB + m;
      ++o;
    }
  if (lane == 0) cnt_out[blockIdx.x] = need;
}

template <int DI, int HP>
hipError_t launch_t(const KvView& kv, const QView& Q, float* scores, hipStream_t st) {
  // Small jobs: one block per lane quarter, many workgroups.  Large jobs (more
  // than ~256 CUs x 256 blocks): four blocks per lane quarter, so every query
  // value read from LDS feeds four blocks.
  const long pairs = (long)Q.nq * kv.maxb;
  if (pairs >= 256L * 256) {
    dim3 grid((kv.maxb + 255) / 256, Q.nq);
    hipLaunchKernelGGL((index_score_exact<DI, HP, 4, false>), grid, dim3(kScoreThreads), 0, st, kv,
                       Q, scores, 0);
  } else {
    dim3 grid((kv.maxb + 63) / 64, Q.nq);
    hipLaunchKernelGGL((index_score_exact<DI, HP, 1, false>), grid, dim3(kScoreThreads), 0, st, kv,
                       Q, scores, 0);
  }
  return hipGetLastError();
}

template <int DI, int HP>
hipError_t launch_cand_t(const KvView& kv, const QView& Q, int need, float* ws, hipStream_t st) {
  static_assert(64 * 4 == kCandBlocks, "NB = 4: one list per 256-block workgroup");
  dim3 grid((kv.maxb + kCandBlocks - 1) / kCandBlocks, Q.nq);
  hipLaunchKernelGGL((index_score_exact<DI, HP, 4, true>), grid, dim3(kScoreThreads), 0, st, kv, Q,
                     ws, need);
  return hipGetLastError();
}

template <int DI>
hipError_t launch_cand_di(const KvView& kv, const QView& Q, int need, float* ws, hipStream_t st) {
  if (Q.hi <= 1) return launch_cand_t<DI, 1>(kv, Q, need, ws, st);
  if (Q.hi <= 2) return launch_cand_t<DI, 2>(kv, Q, need, ws, st);
  if (Q.hi <= 4) return launch_cand_t<DI, 4>(kv, Q, need, ws, st);
  if (Q.hi <= 8) return launch_cand_t<DI, 8>(kv, Q, need, ws, st);
  return launch_cand_t<DI, 16>(kv, Q, need, ws, st);
}

template <int DI>
hipError_t launch_di(const KvView& kv, const QView& Q, float* scores, hipStream_t st) {
  if (Q.hi <= 1) return launch_t<DI, 1>(kv, Q, scores, st);
  if (Q.hi <= 2) return launch_t<DI, 2>(kv, Q, scores, st);
  if (Q.hi <= 4) return launch_t<DI, 4>(kv, Q, scores, st);
  if (Q.hi <= 8) return launch_t<DI, 8>(kv, Q, scores, st);
  return launch_t<DI, 16>(kv, Q, scores, st);
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
                                    hipStream_t st) {
  const int need = top_k - 1;
  return kv.idx_dim == 64 ? launch_cand_di<64>(kv, Q, need, ws, st)
                          : launch_cand_di<128>(kv, Q, need, ws, st);
}

hipError_t launch_index_cand_topk(const KvView& kv, const QView& Q, int top_k, float* ws,
                                  int32_t* idx, int32_t* cnt, hipStream_t st) {
  const int nwg = (kv.maxb + kCandBlocks - 1) / kCandBlocks;
  hipError_t e = launch_index_cand_scores(kv, Q, top_k, ws, st);
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

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

namespace dsa {
namespace {

constexpr int kScoreThreads = 256;

// Lanes: 4 per block (dims DI/4 each); a lane holds NB blocks (16 apart), so a
// wave covers 16 NB blocks and a workgroup 64 NB.
template <int DI, int HP, int NB>
__global__ __launch_bounds__(kScoreThreads) void index_score_exact(KvView kv, QView Q,
                                                                   float* __restrict__ scores) {
  __shared__ double qv[DI * HP];
  __shared__ double sq[HP], wq[HP];
  __shared__ uint32_t amax_bits[HP];
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
  const int local = pos / kBlockSize;

  // Workgroups whose blocks are all invisible only write -inf.
  if (blockIdx.x * kBlocksPerWg > local) {
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
  load_query<DI, HP>(Q, qi, qv, sq, wq, amax_bits, expo);
  float S[NB];
  score_quarters<DI, HP, NB>(kq, gq, qv, sq, wq, S);
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int j = j0 + 16 * b;
    if (gq == 0 && j < kv.maxb) row[j] = visible[b] ? S[b] : -INFINITY;
  }
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

template <int DI>
hipError_t launch_di(const KvView& kv, const QView& Q, float* scores, hipStream_t st) {
  if (Q.hi <= 1) return launch_t<DI, 1>(kv, Q, scores, st);
  if (Q.hi <= 2) return launch_t<DI, 2>(kv, Q, scores, st);
  if (Q.hi <= 4) return launch_t<DI, 4>(kv, Q, scores, st);
  if (Q.hi <= 8) return launch_t<DI, 8>(kv, Q, scores, st);
  return launch_t<DI, 16>(kv, Q, scores, st);
}

}  // namespace

hipError_t launch_index_score(const KvView& kv, const QView& Q, float* scores, hipStream_t st) {
  // many queries at once: the same scores from the int8 matrix cores
  if (index_score_mfma_supported(kv, Q)) return launch_index_score_mfma(kv, Q, scores, st);
  if (kv.idx_dim == 64) return launch_di<64>(kv, Q, scores, st);
  return launch_di<128>(kv, Q, scores, st);
}

}  // namespace dsa

// Indexer scoring and Top-K selection of one query in one workgroup, for
// decode batches whose sequences have at most kFusedMaxBlocks blocks (short
// contexts: one CU scores all of a query's blocks faster than a separate
// scoring launch, a score round trip through memory and a selection launch;
// longer contexts spread the scoring over many workgroups instead).
//
// What is computed is exactly what index_score.hip followed by topk.hip
// compute ([P1] "Day-0 Adaptation for Massive LLMs...", section 4(1) "Index
// Selection"; [P5] "Day-0 Readiness for Trillion-Parameter Models...",
// "Index Selection Path": a lightweight low-precision inner product per
// block, then the Top-K blocks with the local block always kept, ids in
// increasing order):
//   S[j] = sum_{h ascending} w[h] * max(0, (sq[h] * ks[p]) * D[h, j])  (float64,
//   stored as fp32), D exact; then the local block plus the K - 1 best other
//   visible blocks, equal scores going to the lower id.
// The scores never leave LDS.  D is formed on the int8 matrix cores from
// base-128 digit planes (digit_mfma.h): rows of the MFMA tiles are the
// query's indexer heads, columns 16 blocks, k the key dims; the five int32
// digit sums are combined by Horner's rule and the epilogue follows the
// oracle's float64 order, head by head.
#include <hip/hip_runtime.h>
#include <math.h>

#include "dsa_internal.h"
#include "score_i8_lds.h"

namespace dsa {
namespace {

constexpr int kFusedWaves = 8;
constexpr int kFusedMaxBlocks = 256;  // visible blocks per query held in LDS
constexpr int kSelM = kFusedMaxBlocks / 64;

// grid (Nq), block 512.  HP (4, 8 or 16) >= HI rows per tile; rows >= HI
// are zero and weigh zero.
template <int DI, int HP>
__global__ __launch_bounds__(64 * kFusedWaves) void index_topk_i8(KvView kv, QView Q, int top_k,
                                                                  int32_t* __restrict__ out_idx,
                                                                  int32_t* __restrict__ out_cnt) {
  constexpr int KC = DI / 64;
  __shared__ uint32_t lut[256];
  __shared__ float sc[kFusedMaxBlocks];
  __shared__ int tab[kFusedMaxBlocks];  // the sequence's block-table row
  __shared__ double wsq[16];
  __shared__ uint4 hist4[64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qi = blockIdx.x;
  const int s = query_seq(Q, qi);

  QueryRows<DI> qr;
  qr.fetch(Q, qi, lane);
  const int len = kv.seq_lens[s];
  const int pos = Q.q_pos ? Q.q_pos[qi] : len - 1;
  const int local = pos >> kv.bs_shift;  // visible blocks: 0 .. local
  for (int c = tid; c < 256; c += 64 * kFusedWaves) lut[c] = digits_of_code((uint32_t)c);
  for (int j = tid; j <= local; j += 64 * kFusedWaves) tab[j] = kv.table[(size_t)s * kv.maxb + j];
  __syncthreads();
  i32x4 qa[KC][3];
  qr.build(lut, lane, wave == 0, wsq, qa);
  __syncthreads();

  // local < kFusedMaxBlocks (host check)
  score_tiles_i8<DI, HP, kFusedWaves>(kv, qa, wave, lane, local, lut, tab, wsq, sc);
  __syncthreads();

  // ---- Top-K on one wave, keys from LDS
  if (wave != 0) return;
  int32_t* out = out_idx + (size_t)qi * top_k;
  const int c = local <= 64 * 2 ? select_lds_blocks<2>(sc, local, top_k, hist4, out)
                                : select_lds_blocks<kSelM>(sc, local, top_k, hist4, out);
  if (lane == 0) out_cnt[qi] = c;
}

template <int DI>
hipError_t launch_di(const KvView& kv, const QView& Q, int top_k, int32_t* idx, int32_t* cnt,
                     hipStream_t st) {
  const dim3 grid(Q.nq), block(64 * kFusedWaves);
  if (Q.hi <= 4) {
    hipLaunchKernelGGL((index_topk_i8<DI, 4>), grid, block, 0, st, kv, Q, top_k, idx, cnt);
  } else if (Q.hi <= 8) {
    hipLaunchKernelGGL((index_topk_i8<DI, 8>), grid, block, 0, st, kv, Q, top_k, idx, cnt);
  } else {
    hipLaunchKernelGGL((index_topk_i8<DI, 16>), grid, block, 0, st, kv, Q, top_k, idx, cnt);
  }
  return hipGetLastError();
}

}  // namespace

bool index_topk_fused_supported(const KvView& kv, const QView& Q) {
  // every query's blocks fit the LDS score array (short contexts); few enough
  // queries that the many-query scorer would not be chosen
  return kv.maxb <= kFusedMaxBlocks && Q.nq >= 1 && !index_score_mfma_supported(kv, Q) &&
         (kv.idx_dim == 64 || kv.idx_dim == 128) && Q.hi >= 1 && Q.hi <= 16;
}

hipError_t launch_index_topk_fused(const KvView& kv, const QView& Q, int top_k, int32_t* idx,
                                   int32_t* cnt, hipStream_t st) {
  return kv.idx_dim == 64 ? launch_di<64>(kv, Q, top_k, idx, cnt, st)
                          : launch_di<128>(kv, Q, top_k, idx, cnt, st);
}

}  // namespace dsa

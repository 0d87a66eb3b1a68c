// Per-workgroup Top-K candidate lists for long contexts, and their merge.
//
// The scoring kernel (index_score.hip, kCand) gives each workgroup of
// kCandBlocks consecutive blocks one list: the need = K - 1 best of its
// blocks below the local block (equal scores to the lower id), as
// order-preserving keys and ids in increasing id order.  Every block of the
// query's final Top-K is among its workgroup's need best, so merging the
// lists with the same rule gives the same selection as selecting from all
// scores ([P1] "Day-0 Adaptation for Massive LLMs...", section 4(1) "Index
// Selection": Top-K without a full sort; [P5] "Day-0 Readiness for
// Trillion-Parameter Models...", "Index Selection Path": ids in gather order).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "select_common.h"

namespace dsa {

constexpr int kCandBlocks = 256;      // blocks per scoring workgroup (one list)
constexpr int kMergeMaxCand = 2048;   // candidates a query's lists may hold in total

// Lists in the score workspace, per query q: int32 counts [nwg], uint32 keys
// [nwg][need], int32 ids [nwg][need].
__host__ __device__ inline size_t cand_query_words(int nwg, int need) {
  return (size_t)nwg * (1 + 2 * (size_t)need);
}
__device__ inline int32_t* cand_count(float* ws, int nwg, int need, int q) {
  return reinterpret_cast<int32_t*>(ws) + (size_t)q * cand_query_words(nwg, need);
}
__device__ inline uint32_t* cand_keys(float* ws, int nwg, int need, int q) {
  return reinterpret_cast<uint32_t*>(cand_count(ws, nwg, need, q) + nwg);
}
__device__ inline int32_t* cand_ids(float* ws, int nwg, int need, int q) {
  return reinterpret_cast<int32_t*>(cand_keys(ws, nwg, need, q) + (size_t)nwg * need);
}

// One wave keeps the need best of the n candidates keys[0 .. n) (n <= 64 M),
// equal keys going to the earlier position, and writes their positions (in
// increasing order) to out_pos[0 .. min(n, need)); returns that count.
template <int M>
__device__ __forceinline__ int wave_keep_best(const uint32_t* keys, int n, int need,
                                              uint4* hist4, int32_t* out_pos) {
  const int lane = threadIdx.x & 63;
  if (n <= need) {
    for (int i = lane; i < n; i += 64) out_pos[i] = i;
    return n;
  }
  uint32_t k[M], valid = 0u;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int p = lane * M + m;
    k[m] = p < n ? keys[p] : 0u;
    valid |= (p < n) ? (1u << m) : 0u;
  }
  uint32_t T, take_eq, o;
  wave_select<M>(k, valid, (uint32_t)need, hist4, T, take_eq);
  const uint32_t keep = wave_keep<M>(k, valid, T, take_eq, &o);
#pragma unroll
  for (int m = 0; m < M; ++m)
    if (((keep >> m) & 1u) && o < (uint32_t)need) out_pos[o++] = lane * M + m;
  return need;
}

// LDS scratch of merge_candidate_lists (kMergeMaxCand entries each unless noted).
struct CandScratch {
  uint32_t* ck;   // compacted keys
  int32_t* cj;    // compacted ids
  int* off;       // list offsets, kMergeMaxCand + 1
  uint32_t* k2;   // survivors of the first level
  int32_t* j2;
  int32_t* pos;   // positions kept by the waves
  int* n2;        // kWaves
  uint4* hist4;   // 64 per wave
};

// The need best of query q's candidate lists, by the kWaves waves of the
// calling workgroup (every thread calls it; requires need >= 1, and that the
// lists hold at least need candidates, as they do whenever the local block
// has need blocks before it).  Two levels: each wave keeps the need best of a
// contiguous slice of the concatenated lists, then wave 0 keeps the need best
// of the survivors, concatenated in wave order (so still in id order).  A
// candidate outside its slice's need best has need better ones before it and
// cannot be among the final need.  Wave 0 writes the ids, ascending, to
// out[0 .. need) (LDS or global) and returns need; the other waves return 0
// after the last barrier they share.
template <int kWaves>
__device__ int merge_candidate_lists(float* ws, int nwg, int need, int q, const CandScratch& S,
                                     int32_t* out) {
  constexpr int kSlice = kMergeMaxCand / kWaves;  // candidates per first-level wave
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t* counts = cand_count(ws, nwg, need, q);
  const uint32_t* keys = cand_keys(ws, nwg, need, q);
  const int32_t* ids = cand_ids(ws, nwg, need, q);
  if (wave == 0) {  // list offsets, 64 lists at a time
    int total = 0;
    for (int w0 = 0; w0 < nwg; w0 += 64) {
      const int w = w0 + lane;
      const int cw = w < nwg ? counts[w] : 0;
      const uint32_t incl = wave_incl_scan((uint32_t)cw);
      if (w < nwg) S.off[w] = total + (int)incl - cw;
      total += __builtin_amdgcn_readlane((int)incl, 63);
    }
    if (lane == 0) S.off[nwg] = total;
  }
  __syncthreads();
  const int total = S.off[nwg];  // <= nwg need <= kMergeMaxCand
  for (int i = tid; i < nwg * need; i += 64 * kWaves) {
    const int w = i / need, r = i - w * need;
    const int o = S.off[w];
    if (o + r < S.off[w + 1]) {
      S.ck[o + r] = keys[i];
      S.cj[o + r] = ids[i];
    }
  }
  __syncthreads();
  const int slice = (total + kWaves - 1) / kWaves;  // <= kSlice
  {
    const int lo = min(total, wave * slice), hi = min(total, lo + slice);
    const int c = wave_keep_best<kSlice / 64>(S.ck + lo, hi - lo, need, S.hist4 + 64 * wave,
                                              S.pos + kSlice * wave);
    if (lane == 0) S.n2[wave] = c;
  }
  __syncthreads();
  if (wave != 0) return 0;
  int base = 0;
  for (int v = 0; v < kWaves; ++v) {
    const int c = S.n2[v];
    const int lo = min(total, v * slice);
    for (int i = lane; i < c; i += 64) {
      S.k2[base + i] = S.ck[lo + S.pos[kSlice * v + i]];
      S.j2[base + i] = S.cj[lo + S.pos[kSlice * v + i]];
    }
    base += c;
  }
  // one wave: its LDS writes are visible to its later reads; the first-level
  // positions are consumed, so S.pos takes the final ones
  int c;
  if (base <= 64 * 2) {
    c = wave_keep_best<2>(S.k2, base, need, S.hist4, S.pos);
  } else if (base <= 64 * 8) {
    c = wave_keep_best<8>(S.k2, base, need, S.hist4, S.pos);
  } else {
    c = wave_keep_best<32>(S.k2, base, need, S.hist4, S.pos);
  }
  for (int i = lane; i < c; i += 64) out[i] = S.j2[S.pos[i]];
  return c;
}

}  // namespace dsa

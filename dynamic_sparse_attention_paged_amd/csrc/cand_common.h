// Per-workgroup Top-K candidate lists for long contexts, and their merge.
//
// The scoring kernel (index_score.hip, index_cand_scores) gives each chunk of
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

// Stores and loads between the workgroups of one launch (split partials
// merged by the last split to finish): agent-scope atomic accesses, which
// gfx950 performs coherently across its XCDs' L2 caches; plain accesses
// otherwise.
template <bool kCoh, typename T>
__device__ __forceinline__ void st_maybe_coh(T* p, T v) {
  if (kCoh)
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = v;
}
template <bool kCoh, typename T>
__device__ __forceinline__ T ld_maybe_coh(const T* p) {
  if (kCoh) return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return *p;
}

// Split counters of the candidate path's attention launch: one per (query,
// KV head), each in a 256-byte line of its own (word 0), so that the atomics
// on one do not queue behind those on another.
constexpr int kDoneLineWords = 64;

// Lists in the score workspace, per query q: int32 counts [nwg], uint32 list
// maxima [nwg] (the best key of each list, 0 for an empty one), uint32 keys
// [nwg][need], int32 ids [nwg][need].
__host__ __device__ inline size_t cand_query_words(int nwg, int need) {
  return (size_t)nwg * (2 + 2 * (size_t)need);
}
__device__ inline int32_t* cand_count(float* ws, int nwg, int need, int q) {
  return reinterpret_cast<int32_t*>(ws) + (size_t)q * cand_query_words(nwg, need);
}
__device__ inline uint32_t* cand_max(float* ws, int nwg, int need, int q) {
  return reinterpret_cast<uint32_t*>(cand_count(ws, nwg, need, q) + nwg);
}
__device__ inline uint32_t* cand_keys(float* ws, int nwg, int need, int q) {
  return cand_max(ws, nwg, need, q) + nwg;
}
__device__ inline int32_t* cand_ids(float* ws, int nwg, int need, int q) {
  return reinterpret_cast<int32_t*>(cand_keys(ws, nwg, need, q) + (size_t)nwg * need);
}

// The list of chunk `chunk` of query q (blocks chunk 64 NB .. + 64 NB): the
// need best of the chunk's blocks strictly below the local block, equal
// scores to the lower id, in increasing id order, from the chunk's scores in
// LDS (scw[o]: block chunk 64 NB + o), written by wave 0, with the list's
// best key (hist4: 64 entries of LDS).  any == false (uniform): no
// block of the chunk is visible, the list is empty.  Every thread calls it,
// after the scores are visible to wave 0.
template <int NB>
__device__ void chunk_candidates_lds(bool any, int local, const float* scw, uint4* hist4,
                                     float* ws, int nwg, int need, int q, int chunk) {
  constexpr int kBlocks = 64 * NB;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int32_t* cnt_out = cand_count(ws, nwg, need, q);
  uint32_t* max_out = cand_max(ws, nwg, need, q);
  if (!any) {
    if (threadIdx.x == 0) {
      cnt_out[chunk] = 0;
      max_out[chunk] = 0u;
    }
    return;
  }
  if (wave != 0) return;
  const int jbase = chunk * kBlocks;
  const int c = min(max(local - jbase, 0), kBlocks);
  uint32_t* keys_out = cand_keys(ws, nwg, need, q) + (size_t)chunk * need;
  int32_t* ids_out = cand_ids(ws, nwg, need, q) + (size_t)chunk * need;
  uint32_t k[NB], valid = 0u, kmax = 0u;
#pragma unroll
  for (int m = 0; m < NB; ++m) {
    const int o = lane * NB + m;
    k[m] = order_key(scw[o]);
    valid |= (o < c) ? (1u << m) : 0u;
    kmax = (o < c) ? max(kmax, k[m]) : kmax;
  }
  // the list's best key (kept in either case below)
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, off, 64));
  if (lane == 0) max_out[chunk] = kmax;
  if (c <= need) {  // all of them
#pragma unroll
    for (int m = 0; m < NB; ++m) {
      const int o = lane * NB + m;
      if (o < c) {
        keys_out[o] = k[m];
        ids_out[o] = jbase + o;
      }
    }
    if (lane == 0) cnt_out[chunk] = c;
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
  if (lane == 0) cnt_out[chunk] = need;
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
    wave_lds_fence();  // the caller's lanes read other lanes' positions
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
  wave_lds_fence();  // the caller's lanes read other lanes' positions
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
  int* rc;        // kMergeMaxCand / 64 + 1 survivor counts (the last: the threshold)
};
constexpr int kCandScratchExtraWords = kMergeMaxCand / 64 + 1;  // rc

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
  const uint32_t* maxes = cand_max(ws, nwg, need, q);
  const uint32_t* keys = cand_keys(ws, nwg, need, q);
  const int32_t* ids = cand_ids(ws, nwg, need, q);
  // Every list entry (kPer per thread, nwg need <= kMergeMaxCand) is
  // requested at once, together with the counts; entries past a list's
  // count are read but not kept (the region is the lists').
  constexpr int kPer = kMergeMaxCand / (64 * kWaves);
  const int nall = nwg * need;
  uint32_t kk[kPer];
  int32_t jj[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = tid + 64 * kWaves * u;
    if (i < nall) {
      kk[u] = keys[i];
      jj[u] = ids[i];
    }
  }
  // Pre-filter (up to 64 lists): if at least need lists have a maximum >= T0
  // (T0: the need-th largest list maximum), a candidate below T0 has need
  // strictly better ones and cannot be selected; the survivors, >= T0, are
  // at least need and hold the selection.
  const bool filter = nwg <= 64;  // uniform
  int* const thr = S.rc + kMergeMaxCand / 64;
  if (wave == 0) {  // list offsets, 64 lists at a time; the threshold
    int total = 0, lc = 0;
    uint32_t lm = 0u;
    for (int w0 = 0; w0 < nwg; w0 += 64) {
      const int w = w0 + lane;
      const int cw = w < nwg ? counts[w] : 0;
      if (filter) {  // one pass of this loop
        lm = w < nwg ? maxes[w] : 0u;
        lc = cw;
      }
      const uint32_t incl = wave_incl_scan((uint32_t)cw);
      if (w < nwg) S.off[w] = total + (int)incl - cw;
      total += __builtin_amdgcn_readlane((int)incl, 63);
    }
    if (lane == 0) S.off[nwg] = total;
    uint32_t T0 = 0u;
    if (filter) {
      // lane w: list w's maximum; T0 = the largest maximum that at least
      // need maxima reach (counted across the lanes, no LDS)
      const bool has = lane < nwg && lc > 0;
      const uint64_t hm = __ballot(has);
      if (__builtin_popcountll(hm) > need) {
        int ge = 0;
#pragma unroll
        for (int j = 0; j < 64; ++j) {
          const uint32_t xj = (uint32_t)__builtin_amdgcn_readlane((int)lm, j);
          ge += (((hm >> j) & 1u) && xj >= lm) ? 1 : 0;
        }
        uint32_t cand = (has && ge >= need) ? lm : 0u;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1)
          cand = max(cand, (uint32_t)__shfl_xor((int)cand, off, 64));
        T0 = cand;
      }
    }
    if (lane == 0) *thr = (int)T0;
  }
  __syncthreads();
  const int total = S.off[nwg];  // <= nwg need <= kMergeMaxCand
  bool vld[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = tid + 64 * kWaves * u;
    vld[u] = false;
    if (i < nall) {
      const int w = i / need, r = i - w * need;
      vld[u] = S.off[w] + r < S.off[w + 1];
    }
  }
  const uint32_t T0 = (uint32_t)*thr;
  // survivors in candidate order: round u holds candidates 64 kWaves u +
  // tid, so the order is round, then wave, then lane
  uint32_t surv = 0u;
#pragma unroll
  for (int u = 0; u < kPer; ++u) surv |= (vld[u] && kk[u] >= T0) ? (1u << u) : 0u;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int cu = __builtin_popcountll(__ballot((surv >> u) & 1u));
    if (lane == 0) S.rc[u * kWaves + wave] = cu;
  }
  __syncthreads();
  // every round's per-wave counts at once: this thread's output offset in
  // each round, and the total
  int first[kPer];
  int nsurv = 0;
  {
    int rcv[kPer * kWaves];
#pragma unroll
    for (int v = 0; v < kPer * kWaves; ++v) rcv[v] = S.rc[v];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      first[u] = nsurv;
#pragma unroll
      for (int v = 0; v < kWaves; ++v) {
        first[u] += v < wave ? rcv[u * kWaves + v] : 0;
        nsurv += rcv[u * kWaves + v];
      }
    }
  }
  if (nsurv <= 64 * 8) {  // uniform: one wave selects from the survivors
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const uint64_t b = __ballot((surv >> u) & 1u);
      if ((surv >> u) & 1u) {
        const int at = first[u] + (int)__builtin_amdgcn_mbcnt_hi(
                                      (uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
        S.ck[at] = kk[u];
        S.cj[at] = jj[u];
      }
    }
    __syncthreads();
    if (wave != 0) return 0;
    const int c = nsurv <= 64 * 2 ? wave_keep_best<2>(S.ck, nsurv, need, S.hist4, S.pos)
                                  : wave_keep_best<8>(S.ck, nsurv, need, S.hist4, S.pos);
    for (int i = lane; i < c; i += 64) out[i] = S.cj[S.pos[i]];
    return c;
  }
  // many survivors (near-equal scores): every candidate, two levels
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = tid + 64 * kWaves * u;
    if (vld[u]) {
      const int w = i / need, r = i - w * need;
      S.ck[S.off[w] + r] = kk[u];
      S.cj[S.off[w] + r] = jj[u];
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
  wave_lds_fence();  // the survivors, written across the lanes, are read across them
  // the first-level positions are consumed, so S.pos takes the final ones
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

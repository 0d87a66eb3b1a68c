// Device helpers for Top-K block selection (one wave, keys in registers).
//
// Rule implemented ([P1] "Day-0 Adaptation for Massive LLMs...", section
// 4(1); [P5] "Day-0 Readiness for Trillion-Parameter Models...", "Index
// Selection Path"): keep the `need` largest keys, equal keys going to the
// earlier candidate position; emit kept positions in increasing order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

// Order-preserving uint32 image of an fp32 score (-0.0 and +0.0 map alike).
__device__ __forceinline__ uint32_t order_key(float f) {
  if (f == 0.0f) f = 0.0f;
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// A hand-off of LDS data between the lanes of one wave: a fence at
// wavefront scope.  The hardware completes a wave's LDS operations in order
// (the fence emits at most a wait), but without it the compiler may move or
// forward LDS accesses across the hand-off whenever it can assume that no
// other lane writes the memory (seen: a histogram read sunk into the lanes
// that had added to it, the other lanes reading back their own zeros).
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
}

// Inclusive prefix sum across the 64 lanes of a wave with DPP: Hillis-Steele
// within each 16-lane row (row_shr 1, 2, 4, 8), then the row totals are
// carried forward (row_bcast:15 into rows 1 and 3, row_bcast:31 into rows 2
// and 3).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true);   // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// Radix selection within one wave.  Lane l holds keys k[0..M) of candidate
// positions l*M + m; bit m of `valid` marks real candidates.  Requires
// need < number of valid keys.  Up to four 8-bit MSB-first passes over a
// wave-private 256-bin LDS histogram `hist4` (64 x uint4; one wave: its LDS
// operations complete in order, and wave_lds_fence orders them for the
// compiler).  Returns the key T
// of the need-th largest candidate and how many keys equal to T are kept.
template <int M>
__device__ __forceinline__ void wave_select(const uint32_t (&k)[M], uint32_t valid, uint32_t need,
                                            uint4* hist4, uint32_t& T_out, uint32_t& take_eq) {
  const int lane = threadIdx.x & 63;
  uint32_t* hist = reinterpret_cast<uint32_t*>(hist4);
  // Bits above the highest bit in which the largest and smallest valid keys
  // differ are common to every key, hence to T; the 8-bit windows start just
  // below them (a window over shared bits would send every key to one
  // histogram bin).
  uint32_t hi = 0u, lo = 0xFFFFFFFFu;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    if ((valid >> m) & 1u) {
      hi = max(hi, k[m]);
      lo = min(lo, k[m]);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    hi = max(hi, (uint32_t)__shfl_xor((int)hi, off, 64));
    lo = min(lo, (uint32_t)__shfl_xor((int)lo, off, 64));
  }
  const uint32_t diff = hi ^ lo;
  if (diff == 0u) {  // every valid key is equal
    T_out = hi;
    take_eq = need;
    return;
  }
  const int top = 31 - __builtin_clz(diff);
  uint32_t mask = top == 31 ? 0u : ~((2u << top) - 1u);
  uint32_t T = hi & mask, remaining = need;
  for (int shift = top - 7; shift > -8; shift -= 8) {
    // window bits [max(shift, 0), shift + 8)
    const int sh = shift < 0 ? 0 : shift;
    const int width = shift < 0 ? 8 + shift : 8;
    const uint32_t wmask = ((1u << width) - 1u) << sh;
    hist4[lane] = make_uint4(0u, 0u, 0u, 0u);
    wave_lds_fence();
#pragma unroll
    for (int m = 0; m < M; ++m)
      if (((valid >> m) & 1u) && (k[m] & mask) == T)
        atomicAdd(&hist[(k[m] & wmask) >> sh], 1u);
    wave_lds_fence();
    const uint4 h = hist4[lane];
    const uint32_t mine = h.x + h.y + h.z + h.w;
    const uint32_t incl = wave_incl_scan(mine);
    const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    const uint32_t above = total - incl;  // keys in digits above this lane's four
    // the digit holding the remaining-th largest key lies in the lane where
    // above < remaining <= above + mine; find it among the lane's four digits
    uint32_t c = above;
    int d = 3;
    const uint32_t hs[4] = {h.x, h.y, h.z, h.w};
    for (; d > 0; --d) {
      if (c + hs[d] >= remaining) break;
      c += hs[d];
    }
    const bool hit = above < remaining && remaining <= above + mine;
    const int L = __builtin_ffsll((long long)__ballot(hit)) - 1;
    const int dig = __builtin_amdgcn_readlane(4 * lane + d, L);
    const uint32_t cut = (uint32_t)__builtin_amdgcn_readlane((int)c, L);
    const uint32_t in_bucket = (uint32_t)__builtin_amdgcn_readlane((int)hs[d], L);
    T |= (uint32_t)dig << sh;
    remaining -= cut;
    mask |= wmask;
    if (in_bucket == remaining) {
      // The whole digit bucket is kept: every key with this prefix is at
      // least T (low bits zero), keys above it exceed T, keys below are
      // under it.  Keep all keys equal to T.
      T_out = T;
      take_eq = 0xFFFFFFFFu;
      return;
    }
  }
  T_out = T;
  take_eq = remaining;
}

// After wave_select: position (in increasing candidate order) of this lane's
// first kept key, and the keep mask of its slots.  Keys > T are kept; of the
// keys == T, the first take_eq in candidate order.
template <int M>
__device__ __forceinline__ uint32_t wave_keep(const uint32_t (&k)[M], uint32_t valid, uint32_t T,
                                              uint32_t take_eq, uint32_t* first_out) {
  uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    if ((valid >> m) & 1u) {
      n_gt += k[m] > T;
      n_eq += k[m] == T;
    }
  }
  const uint32_t eq_before = wave_incl_scan(n_eq) - n_eq;
  const uint32_t eq_take = eq_before >= take_eq ? 0u : min(n_eq, take_eq - eq_before);
  const uint32_t mine = n_gt + eq_take;
  *first_out = wave_incl_scan(mine) - mine;
  uint32_t keep = 0u, eq_seen = 0;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    if ((valid >> m) & 1u) {
      bool kp = k[m] > T;
      if (k[m] == T) {
        kp = eq_seen < eq_take;
        ++eq_seen;
      }
      keep |= kp ? (1u << m) : 0u;
    }
  }
  return keep;
}

// One wave selects a query's blocks: the local block plus the need =
// top_k - 1 best of candidates 0 .. local - 1 (fp32 scores row[0 .. local)),
// equal scores going to the lower id; ids in increasing order to out[0 ..
// cnt) (the local block last) and -1 up to top_k.  out may point to global
// memory or LDS.  Requires local <= 64 M when more than need candidates
// exist.  Returns cnt.
template <int M>
__device__ __forceinline__ int select_query_blocks(const float* row, int maxb, int local,
                                                   int top_k, uint4* hist4, int32_t* out) {
  const int lane = threadIdx.x & 63;
  // clamped (in-row) loads, all in flight at once; candidates past n masked
  float v[M];
#pragma unroll
  for (int m = 0; m < M; ++m) v[m] = row[min(lane * M + m, maxb - 1)];
  const int n = local;
  const int need = top_k - 1;
  if (n <= need) {
    for (int i = lane; i < top_k; i += 64) out[i] = i <= local ? i : -1;
    return local + 1;
  }
  if (need == 0) {  // K = 1: the local block alone
    if (lane == 0) out[0] = local;
    return 1;
  }
  uint32_t k[M], valid = 0u;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    k[m] = order_key(v[m]);
    valid |= (lane * M + m < n) ? (1u << m) : 0u;
  }
  uint32_t T, take_eq, o;
  wave_select<M>(k, valid, (uint32_t)need, hist4, T, take_eq);
  const uint32_t keep = wave_keep<M>(k, valid, T, take_eq, &o);
#pragma unroll
  for (int m = 0; m < M; ++m)
    if (((keep >> m) & 1u) && o < (uint32_t)need) out[o++] = lane * M + m;
  if (lane == 0) out[need] = local;  // largest visible id: last in ascending order
  return top_k;
}

// LDS slot of candidate j's score when a query's scores are kept in LDS:
// XOR-swizzled within each group of 32, so that one lane's reads of M
// consecutive scores and the wave's reads of a row hit distinct banks.
__device__ __forceinline__ int sc_slot(int j) { return j ^ ((j >> 5) & 31); }

// select_query_blocks with the scores in LDS (slot sc_slot(j) of candidate
// j): the same rule, output and return value.  Requires local <= 64 M when
// more than top_k - 1 candidates exist.
template <int M>
__device__ __forceinline__ int select_lds_blocks(const float* sc, int local, int top_k,
                                                 uint4* hist4, int32_t* out) {
  const int lane = threadIdx.x & 63;
  const int n = local;
  const int need = top_k - 1;
  if (n <= need) {
    for (int i = lane; i < top_k; i += 64) out[i] = i <= local ? i : -1;
    return local + 1;
  }
  if (need == 0) {
    if (lane == 0) out[0] = local;
    return 1;
  }
  uint32_t k[M], valid = 0u;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int c = lane * M + m;
    k[m] = c < n ? order_key(sc[sc_slot(c)]) : 0u;
    valid |= (c < n) ? (1u << m) : 0u;
  }
  uint32_t T, take_eq, o;
  wave_select<M>(k, valid, (uint32_t)need, hist4, T, take_eq);
  const uint32_t keep = wave_keep<M>(k, valid, T, take_eq, &o);
#pragma unroll
  for (int m = 0; m < M; ++m)
    if (((keep >> m) & 1u) && o < (uint32_t)need) out[o++] = lane * M + m;
  if (lane == 0) out[need] = local;
  return top_k;
}

}  // namespace dsa

// Per-query Top-K block selection by LDS radix select.
//
// What is selected ([P1] "Day-0 Adaptation for Massive LLMs...", section
// 4(1): Top-K relevant blocks, block-wise reduction and partial selection
// rather than a full sort, padding for ragged batches; [P5] "Day-0 Readiness
// for Trillion-Parameter Models...", "Index Selection Path": the selected
// indices are ordered the way the gather consumes them):
//   - the local block l = pos / block_size is always kept;
//   - of the candidates j < l the K-1 with the largest score are kept,
//     equal scores going to the lower j (and -0.0 == +0.0);
//   - output in ascending j (so l is last), -1 padded, count = min(K, l+1).
//
// Method: scores become order-preserving uint32 keys and the key T of the
// (K-1)-th largest candidate is found by four 8-bit MSB-first radix passes
// over an LDS histogram -- one wave per query with the keys in registers for
// up to 2048 candidates, a 1024-thread workgroup per query for longer lists.  Every key > T is kept and, of the keys
// == T, the lowest-j ones up to the remaining count.  Compaction over
// contiguous j ranges with a prefix sum yields the ascending output order
// without any sort.
#include <hip/hip_runtime.h>

#include "dsa_internal.h"
#include "select_common.h"

namespace dsa {
namespace {

constexpr int kTopkLdsKeys = 16384;  // candidates cached in LDS (64 KiB)

// Exclusive prefix sum over the workgroup (wave scans + one cross-wave step).
// Returns this thread's prefix; *total receives the workgroup sum.
template <int kThreads>
__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* wave_tot, uint32_t* total) {
  constexpr int kWaves = kThreads / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t x = wave_incl_scan(v);
  if (lane == 63) wave_tot[wave] = x;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t t = wave_tot[w];
    before += w < wave ? t : 0u;
    tot += t;
  }
  __syncthreads();  // wave_tot may be reused by the next scan
  *total = tot;
  return before + x - v;
}

template <int kThreads, bool kKeysInLds>
__global__ __launch_bounds__(kThreads) void topk_radix(const float* __restrict__ scores,
                                                       KvView kv, QView Q, int top_k,
                                                       int32_t* __restrict__ out_idx,
                                                       int32_t* __restrict__ out_cnt) {
  __shared__ uint32_t keys[kKeysInLds ? kTopkLdsKeys : 1];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wave_tot[kThreads / 64];
  __shared__ uint32_t sel_prefix, sel_remaining;

  const int tid = threadIdx.x;
  const int qi = blockIdx.x;
  const int s = query_seq(Q, qi);
  const int len = kv.seq_lens[s];
  const int pos = Q.q_pos ? Q.q_pos[qi] : len - 1;
  const int local = pos >> kv.bs_shift;
  const int n = local;              // candidates 0..local-1 (the local block is forced)
  const int need = top_k - 1;       // how many candidates to keep
  const float* row = scores + (size_t)qi * kv.maxb;
  int32_t* out = out_idx + (size_t)qi * top_k;

  if (n <= need) {  // everything visible is kept
    for (int i = tid; i < top_k; i += kThreads) out[i] = i <= local ? i : -1;
    if (tid == 0) out_cnt[qi] = local + 1;
    return;
  }
  if (need == 0) {  // K = 1: the local block alone
    if (tid == 0) {
      out[0] = local;
      out_cnt[qi] = 1;
    }
    return;
  }
  if (kKeysInLds) {
    // eight loads in flight per thread (clamped in-row indices, masked stores)
    for (int base = 0; base < n; base += 8 * kThreads) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = row[min(base + u * kThreads + tid, kv.maxb - 1)];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = base + u * kThreads + tid;
        if (j < n) keys[j] = order_key(v[u]);
      }
    }
  }
  if (tid == 0) {
    sel_prefix = 0u;
    sel_remaining = (uint32_t)need;
  }
  uint32_t mask = 0u;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int b = tid; b < 256; b += kThreads) hist[b] = 0u;
    __syncthreads();
    const uint32_t prefix = sel_prefix;
    for (int j = tid; j < n; j += kThreads) {
      const uint32_t k = kKeysInLds ? keys[j] : order_key(row[j]);
      if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 0xFFu], 1u);
    }
    __syncthreads();
    // Find the digit where the count of larger-or-equal keys reaches `remaining`.
    // Wave 0: lane l owns digits 4l..4l+3; suffix sums from the top digit down.
    if (tid < 64) {
      const uint32_t remaining = sel_remaining;
      const uint32_t h0 = hist[4 * tid], h1 = hist[4 * tid + 1], h2 = hist[4 * tid + 2],
                     h3 = hist[4 * tid + 3];
      const uint32_t mine = h0 + h1 + h2 + h3;
      const uint32_t incl = wave_incl_scan(mine);
      const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
      const uint32_t suf = total - incl + mine;  // inclusive suffix sum over lanes tid..63
      const uint32_t above = suf - mine;         // keys in digits > 4 tid + 3
      if (above < remaining && remaining <= suf) {
        uint32_t c = above;
        int d = 3;
        const uint32_t hs[4] = {h0, h1, h2, h3};
        for (; d > 0; --d) {
          if (c + hs[d] >= remaining) break;
          c += hs[d];
        }
        sel_prefix = prefix | ((uint32_t)(4 * tid + d) << shift);
        sel_remaining = remaining - c;
      }
    }
    mask |= 0xFFu << shift;
    __syncthreads();
  }
  const uint32_t T = sel_prefix;
  const uint32_t take_eq = sel_remaining;  // keys == T to keep, lowest j first

  // Ascending compaction over contiguous ranges.
  const int chunk = (n + kThreads - 1) / kThreads;
  const int j0 = min(n, tid * chunk), j1 = min(n, j0 + chunk);
  uint32_t n_gt = 0, n_eq = 0;
  for (int j = j0; j < j1; ++j) {
    const uint32_t k = kKeysInLds ? keys[j] : order_key(row[j]);
    n_gt += k > T;
    n_eq += k == T;
  }
  uint32_t total;
  const uint32_t eq_before = block_exclusive_scan<kThreads>(n_eq, wave_tot, &total);
  const uint32_t eq_take_here = eq_before >= take_eq ? 0u : min(n_eq, take_eq - eq_before);
  const uint32_t out_before = block_exclusive_scan<kThreads>(n_gt + eq_take_here, wave_tot, &total);
  uint32_t o = out_before, eq_seen = 0;
  for (int j = j0; j < j1; ++j) {
    const uint32_t k = kKeysInLds ? keys[j] : order_key(row[j]);
    bool keep = k > T;
    if (k == T) {
      keep = eq_seen < eq_take_here;
      ++eq_seen;
    }
    if (keep && o < (uint32_t)need) out[o++] = j;
  }
  if (tid == 0) {
    out[need] = local;  // largest visible id: last in ascending order
    out_cnt[qi] = top_k;
  }
}

// Single-wave selection for up to 64 * M candidates, keys in registers.
// Lane l owns candidates [l M, l M + M).
template <int M>
__global__ __launch_bounds__(64) void topk_wave(const float* __restrict__ scores, KvView kv,
                                                QView Q, int top_k, int32_t* __restrict__ out_idx,
                                                int32_t* __restrict__ out_cnt) {
  __shared__ uint4 hist4[64];
  const int lane = threadIdx.x;
  const int qi = blockIdx.x;
  const int s = query_seq(Q, qi);
  const float* row = scores + (size_t)qi * kv.maxb;
  const int len = kv.seq_lens[s];
  const int pos = Q.q_pos ? Q.q_pos[qi] : len - 1;
  const int c = select_query_blocks<M>(row, kv.maxb, pos >> kv.bs_shift, top_k, hist4,
                                       out_idx + (size_t)qi * top_k);
  if (lane == 0) out_cnt[qi] = c;
}

// Two-level selection for long candidate lists (up to 16 * 64 * M, with
// K - 1 <= kTreeMaxNeed): each of the 16 waves selects the K-1 best of its
// contiguous range into LDS (in increasing position), then wave 0 selects
// the K-1 best of those candidates, which are already in increasing order.
constexpr int kTreeWaves = 16;
constexpr int kTreeMaxNeed = 128;

template <int M>
__global__ __launch_bounds__(64 * kTreeWaves) void topk_tree(
    const float* __restrict__ scores, KvView kv, QView Q, int top_k,
    int32_t* __restrict__ out_idx, int32_t* __restrict__ out_cnt) {
  constexpr int M2 = kTreeWaves * kTreeMaxNeed / 64;  // second-level slots per lane
  __shared__ uint4 hist4[kTreeWaves][64];
  __shared__ uint32_t ck[kTreeWaves * kTreeMaxNeed];
  __shared__ int32_t cj[kTreeWaves * kTreeMaxNeed];
  __shared__ uint32_t wcnt[kTreeWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int qi = blockIdx.x;
  const int s = query_seq(Q, qi);
  const int len = kv.seq_lens[s];
  const int pos = Q.q_pos ? Q.q_pos[qi] : len - 1;
  const int local = pos >> kv.bs_shift;
  const int n = local;
  const int need = top_k - 1;
  const float* row = scores + (size_t)qi * kv.maxb;
  int32_t* out = out_idx + (size_t)qi * top_k;
  if (n <= need) {
    for (int i = threadIdx.x; i < top_k; i += 64 * kTreeWaves) out[i] = i <= local ? i : -1;
    if (threadIdx.x == 0) out_cnt[qi] = local + 1;
    return;
  }
  if (need == 0) {  // K = 1: the local block alone
    if (threadIdx.x == 0) {
      out[0] = local;
      out_cnt[qi] = 1;
    }
    return;
  }
  // level 1: wave w owns positions [w R, w R + R), R = 64 M
  {
    const int base = wave * 64 * M + lane * M;
    float v[M];
#pragma unroll
    for (int m = 0; m < M; ++m) v[m] = row[min(base + m, kv.maxb - 1)];
    uint32_t k[M], valid = 0u;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      k[m] = order_key(v[m]);
      valid |= (base + m < n) ? (1u << m) : 0u;
    }
    const int nw = min(max(n - wave * 64 * M, 0), 64 * M);
    uint32_t keep, o;
    if (nw <= need) {  // keep the whole range
      keep = valid;
      const uint32_t c = (uint32_t)__builtin_popcount(valid);
      o = wave_incl_scan(c) - c;
    } else {
      uint32_t T, take_eq;
      wave_select<M>(k, valid, (uint32_t)need, hist4[wave], T, take_eq);
      keep = wave_keep<M>(k, valid, T, take_eq, &o);
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
      if (((keep >> m) & 1u) && o < (uint32_t)need) {
        ck[wave * kTreeMaxNeed + o] = k[m];
        cj[wave * kTreeMaxNeed + o] = base + m;
        ++o;
      }
    }
    if (lane == 0) wcnt[wave] = (uint32_t)min(nw, need);
  }
  __syncthreads();
  if (wave != 0) return;
  // level 2: candidate c = w * need + i (i < wcnt[w]) in increasing position
  uint32_t k2[M2], valid2 = 0u;
#pragma unroll
  for (int m = 0; m < M2; ++m) {
    const int c = lane * M2 + m;
    const int w = c / kTreeMaxNeed, i = c % kTreeMaxNeed;
    const bool ok = w < kTreeWaves && i < need && (uint32_t)i < wcnt[min(w, kTreeWaves - 1)];
    k2[m] = ok ? ck[c] : 0u;
    valid2 |= ok ? (1u << m) : 0u;
  }
  uint32_t T, take_eq, o;
  wave_select<M2>(k2, valid2, (uint32_t)need, hist4[0], T, take_eq);
  const uint32_t keep = wave_keep<M2>(k2, valid2, T, take_eq, &o);
#pragma unroll
  for (int m = 0; m < M2; ++m)
    if (((keep >> m) & 1u) && o < (uint32_t)need) out[o++] = cj[lane * M2 + m];
  if (lane == 0) {
    out[need] = local;
    out_cnt[qi] = top_k;
  }
}

template <int kThreads>
hipError_t launch_t(const float* scores, const KvView& kv, const QView& Q, int top_k,
                    int32_t* idx, int32_t* cnt, hipStream_t st) {
  const int nmax = kv.maxb - 1;  // candidates per query at most
  if (nmax <= kTopkLdsKeys) {
    hipLaunchKernelGGL((topk_radix<kThreads, true>), dim3(Q.nq), dim3(kThreads), 0, st, scores,
                       kv, Q, top_k, idx, cnt);
  } else {
    hipLaunchKernelGGL((topk_radix<kThreads, false>), dim3(Q.nq), dim3(kThreads), 0, st, scores,
                       kv, Q, top_k, idx, cnt);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_topk(const float* scores, const KvView& kv, const QView& Q, int top_k,
                       int32_t* idx, int32_t* cnt, hipStream_t st) {
  const int nmax = kv.maxb - 1;  // candidates per query at most
  const dim3 g(Q.nq);
  if (nmax <= 64 * 2) {
    hipLaunchKernelGGL(topk_wave<2>, g, dim3(64), 0, st, scores, kv, Q, top_k, idx, cnt);
  } else if (nmax <= 64 * 8) {
    hipLaunchKernelGGL(topk_wave<8>, g, dim3(64), 0, st, scores, kv, Q, top_k, idx, cnt);
  } else if (nmax <= 64 * 32) {
    hipLaunchKernelGGL(topk_wave<32>, g, dim3(64), 0, st, scores, kv, Q, top_k, idx, cnt);
  } else if (nmax <= kTreeWaves * 64 * 16 && top_k - 1 <= kTreeMaxNeed) {
    hipLaunchKernelGGL(topk_tree<16>, g, dim3(64 * kTreeWaves), 0, st, scores, kv, Q, top_k, idx,
                       cnt);
  } else {
    // long lists with large K: 8-bit radix passes over an LDS histogram
    return launch_t<1024>(scores, kv, Q, top_k, idx, cnt, st);
  }
  return hipGetLastError();
}

}  // namespace dsa

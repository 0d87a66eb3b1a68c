// Per-query Top-K block selection by LDS radix select.
//
// What is selected ([P1] "Day-0 Adaptation for Massive LLMs...", section
// 4(1): Top-K relevant blocks, block-wise reduction and partial selection
// rather than a full sort, padding for ragged batches; [P5] "Day-0 Readiness
// for Trillion-Parameter Models...", "Index Selection Path": the selected
// indices are ordered the way the gather consumes them):
//   - the local block l = pos / 64 is always kept;
//   - of the candidates j < l the K-1 with the largest score are kept,
//     equal scores going to the lower j (and -0.0 == +0.0);
//   - output in ascending j (so l is last), -1 padded, count = min(K, l+1).
//
// Method: scores become order-preserving uint32 keys; four 8-bit MSB-first
// histogram passes find the key T of the (K-1)-th largest candidate; every
// key > T is kept and, of the keys == T, the lowest-j ones up to the
// remaining count.  The ascending compaction is a workgroup prefix sum over
// contiguous j ranges, which yields the output order without any sort.
#include <hip/hip_runtime.h>

#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kTopkThreads = 256;
constexpr int kTopkLdsKeys = 15360;  // candidates cached in LDS (60 KiB, + ~2 KiB static)

__device__ __forceinline__ uint32_t order_key(float f) {
  if (f == 0.0f) f = 0.0f;  // -0.0 and +0.0 compare equal
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum over the workgroup; returns this thread's prefix and
// the total in *total.  `buf` holds kTopkThreads uint32 of LDS.
__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* buf, uint32_t* total) {
  const int tid = threadIdx.x;
  buf[tid] = v;
  __syncthreads();
  for (int off = 1; off < kTopkThreads; off <<= 1) {
    const uint32_t add = tid >= off ? buf[tid - off] : 0u;
    __syncthreads();
    buf[tid] += add;
    __syncthreads();
  }
  const uint32_t incl = buf[tid];
  *total = buf[kTopkThreads - 1];
  __syncthreads();
  return incl - v;
}

template <bool kKeysInLds>
__global__ __launch_bounds__(kTopkThreads) void topk_radix(const float* __restrict__ scores,
                                                           KvView kv, QView Q, int top_k,
                                                           int32_t* __restrict__ out_idx,
                                                           int32_t* __restrict__ out_cnt) {
  extern __shared__ uint32_t keys[];  // kTopkLdsKeys when kKeysInLds
  __shared__ uint32_t hist[256];
  __shared__ uint32_t scan_buf[kTopkThreads];
  __shared__ uint32_t sel_prefix, sel_remaining;

  const int tid = threadIdx.x;
  const int qi = blockIdx.x;
  const int s = query_seq(Q, qi);
  const int len = kv.seq_lens[s];
  const int pos = Q.q_pos ? Q.q_pos[qi] : len - 1;
  const int local = pos / kBlockSize;
  const int n = local;              // candidates 0..local-1 (the local block is forced)
  const int need = top_k - 1;       // how many candidates to keep
  const float* row = scores + (size_t)qi * kv.maxb;
  int32_t* out = out_idx + (size_t)qi * top_k;

  if (n <= need) {  // everything visible is kept
    for (int i = tid; i < top_k; i += kTopkThreads) out[i] = i <= local ? i : -1;
    if (tid == 0) out_cnt[qi] = local + 1;
    return;
  }
  if (kKeysInLds) {
    for (int j = tid; j < n; j += kTopkThreads) keys[j] = order_key(row[j]);
  }
  if (tid == 0) { sel_prefix = 0u; sel_remaining = (uint32_t)need; }
  uint32_t mask = 0u;
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[tid] = 0u;  // kTopkThreads == 256 bins
    __syncthreads();
    const uint32_t prefix = sel_prefix;
    for (int j = tid; j < n; j += kTopkThreads) {
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
      // inclusive suffix sum over lanes tid..63
      uint32_t suf = mine;
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_down(suf, off, 64);
        if (tid + off < 64) suf += o;
      }
      const uint32_t above = suf - mine;  // keys in digits > 4 tid + 3
      if (above < remaining && remaining <= suf) {
        // crossing inside this lane's four digits, scanning from the top
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
  const int chunk = (n + kTopkThreads - 1) / kTopkThreads;
  const int j0 = min(n, tid * chunk), j1 = min(n, j0 + chunk);
  uint32_t n_gt = 0, n_eq = 0;
  for (int j = j0; j < j1; ++j) {
    const uint32_t k = kKeysInLds ? keys[j] : order_key(row[j]);
    n_gt += k > T;
    n_eq += k == T;
  }
  uint32_t total;
  const uint32_t eq_before = block_exclusive_scan(n_eq, scan_buf, &total);
  const uint32_t eq_take_here =
      eq_before >= take_eq ? 0u : min(n_eq, take_eq - eq_before);
  const uint32_t out_before = block_exclusive_scan(n_gt + eq_take_here, scan_buf, &total);
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

}  // namespace

hipError_t launch_topk(const float* scores, const KvView& kv, const QView& Q, int top_k,
                       int32_t* idx, int32_t* cnt, hipStream_t st) {
  if (kv.maxb - 1 <= kTopkLdsKeys) {
    hipLaunchKernelGGL(topk_radix<true>, dim3(Q.nq), dim3(kTopkThreads),
                       (size_t)(kv.maxb - 1) * sizeof(uint32_t), st, scores, kv, Q, top_k, idx,
                       cnt);
  } else {
    hipLaunchKernelGGL(topk_radix<false>, dim3(Q.nq), dim3(kTopkThreads), 0, st, scores, kv, Q,
                       top_k, idx, cnt);
  }
  return hipGetLastError();
}

}  // namespace dsa

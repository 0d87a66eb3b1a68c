// Check of the device-side input contract (block tables, lengths, query
// positions and, optionally, caller-supplied block lists).  The compute
// kernels trust these values; this kernel reads them, and only them, within
// their declared shapes and dereferences none of them, so it is safe to run
// on any data.  Violations are ORed into one flag word.
//
// Visibility and the block-list rules restate the selection contract ([P1]
// "Day-0 Adaptation for Massive LLMs...", section 4(1) "Index Selection":
// Top-K blocks, padded for ragged batches; [P5] "Day-0 Readiness for
// Trillion-Parameter Models...", "Index Selection Path" and "KV Cache
// Layout": ids in gather order, one table row per sequence): a query at
// position pos sees logical blocks j with j * block_size <= pos; a list holds cnt
// ascending visible ids ending with the local block pos / block_size, then -1.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsa.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

__global__ void zero_flags(uint32_t* flags) { *flags = 0u; }

// One thread per item: items [0, B * maxb) are table entries, then Nq
// queries (sequence, position, and the block list when given).
__global__ __launch_bounds__(256) void check_inputs(KvView kv, QView Q,
                                                    const int32_t* __restrict__ block_idx,
                                                    const int32_t* __restrict__ block_cnt,
                                                    int top_k, uint32_t* flags) {
  const long n_tab = (long)kv.num_seqs * kv.maxb;
  const long n_items = n_tab + Q.nq;
  const long stride = (long)gridDim.x * blockDim.x;
  uint32_t f = 0u;
  for (long it = (long)blockIdx.x * blockDim.x + threadIdx.x; it < n_items; it += stride) {
    if (it < n_tab) {
      const int s = (int)(it / kv.maxb), j = (int)(it % kv.maxb);
      const int len = kv.seq_lens[s];
      if (j == 0 && (len < 1 || (long)len > ((long)kv.maxb << kv.bs_shift))) f |= DSA_CHECK_SEQ_LEN;
      // entries of blocks that hold tokens must name pool blocks
      if (((long)j << kv.bs_shift) < (long)len) {
        const int p = kv.table[it];
        if (p < 0 || p >= kv.num_blocks) f |= DSA_CHECK_TABLE;
      }
      continue;
    }
    const int qi = (int)(it - n_tab);
    const int s = Q.q_seq ? Q.q_seq[qi] : qi;
    if (s < 0 || s >= kv.num_seqs) {
      f |= DSA_CHECK_Q_SEQ;
      continue;
    }
    const int len = kv.seq_lens[s];
    const int pos = Q.q_pos ? Q.q_pos[qi] : len - 1;
    if (pos < 0 || pos >= len) {
      f |= DSA_CHECK_Q_POS;
      continue;
    }
    if (block_idx) {
      const int local = pos >> kv.bs_shift;
      const int c = block_cnt[qi];
      if (c < 1 || c > top_k) {
        f |= DSA_CHECK_BLOCK_LIST;
        continue;
      }
      const int32_t* row = block_idx + (size_t)qi * top_k;
      int prev = -1;
      for (int i = 0; i < c; ++i) {
        const int j = row[i];
        if (j <= prev || j > local) f |= DSA_CHECK_BLOCK_LIST;  // ascending, visible
        prev = j;
      }
      if (prev != local) f |= DSA_CHECK_BLOCK_LIST;  // the local block ends the list
      for (int i = c; i < top_k; ++i)
        if (row[i] != -1) f |= DSA_CHECK_BLOCK_LIST;
    }
  }
  // one atomic per wave
  uint32_t wf = f;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) wf |= (uint32_t)__shfl_xor((int)wf, off, 64);
  if ((threadIdx.x & 63) == 0 && wf != 0u) atomicOr(flags, wf);
}

}  // namespace

hipError_t launch_check_inputs(const KvView& kv, const QView& Q, const int32_t* block_idx,
                               const int32_t* block_cnt, int top_k, uint32_t* flags,
                               hipStream_t st) {
  hipLaunchKernelGGL(zero_flags, dim3(1), dim3(1), 0, st, flags);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long items = (long)kv.num_seqs * kv.maxb + Q.nq;
  long wgs = (items + 255) / 256;
  if (wgs > 4096) wgs = 4096;
  if (wgs < 1) wgs = 1;
  hipLaunchKernelGGL(check_inputs, dim3((unsigned)wgs), dim3(256), 0, st, kv, Q, block_idx,
                     block_cnt, top_k, flags);
  return hipGetLastError();
}

}  // namespace dsa

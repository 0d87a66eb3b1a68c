// The paged write path: new tokens' K/V rows into their blocks, and the
// per-block coarse index keys at low precision.
//
// [P5] "Day-0 Readiness for Trillion-Parameter Models...", "KV Cache Layout":
// the cache is [block][token][head][dim] behind a block table; prefill writes
// a chunk's tokens in batch, decode appends the newest token.  [P1] "Day-0
// Adaptation for Massive LLMs...", section 4(2): every block carries a
// compressed index representation, kept apart from the fine-grained KV.  The
// pages do not say how that representation is derived from the block, so it
// is an input vector per block here, stored as E4M3 codes with one float32
// scale:
//   ks = max_d |x[d]| / 448 (1 / 448 for a zero vector),  y = x / ks (float32,
//   each division rounded once), code = E4M3(clamp(y, -448, 448)) to nearest even.
//
// Both kernels write only inside the pool and the table: a token or block whose
// target lies outside them is skipped.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kWriteThreads = 256;

// One thread per 16 B of a token's K or V row (num_kv_heads * 128 bf16); the
// chunk c of head c / 16 lands at its place in either block order.
__global__ __launch_bounds__(kWriteThreads) void kv_write_rows(
    KvView kv, int n, const int32_t* __restrict__ tok_seq, const int32_t* __restrict__ tok_pos,
    const uint4* __restrict__ k_new, const uint4* __restrict__ v_new, uint4* __restrict__ k_out,
    uint4* __restrict__ v_out) {
  const int chunks = kv.num_kv_heads * (kHeadDim / 8);
  const long total = 2L * n * chunks;
  const long stride = (long)gridDim.x * kWriteThreads;
  for (long it = (long)blockIdx.x * kWriteThreads + threadIdx.x; it < total; it += stride) {
    const bool is_v = it >= (long)n * chunks;
    const long e = is_v ? it - (long)n * chunks : it;
    const int i = (int)(e / chunks), c = (int)(e - (long)i * chunks);
    const int s = tok_seq ? tok_seq[i] : i;
    if (s < 0 || s >= kv.num_seqs) continue;
    const int pos = tok_pos ? tok_pos[i] : kv.seq_lens[s] - 1;
    if (pos < 0 || (pos >> kv.bs_shift) >= kv.maxb) continue;
    const int p = kv.table[(size_t)s * kv.maxb + (pos >> kv.bs_shift)];
    if (p < 0 || p >= kv.num_blocks) continue;
    const size_t t = (size_t)(pos & ((1 << kv.bs_shift) - 1));
    const size_t dst =
        kv.head_major
            ? ((((size_t)p * kv.num_kv_heads + c / 16) << kv.bs_shift) + t) * 16 + (c & 15)
            : (((size_t)p << kv.bs_shift) + t) * chunks + c;
    const uint4 val = (is_v ? v_new : k_new)[(size_t)i * chunks + c];
    (is_v ? v_out : k_out)[dst] = val;
  }
}

// One wave per block; lane l holds dims l and l + 64.
template <int DI>
__global__ __launch_bounds__(kWriteThreads) void index_key_rows(KvView kv, int n,
                                                                const int32_t* __restrict__ blk,
                                                                const float* __restrict__ x,
                                                                uint8_t* __restrict__ keys_out,
                                                                float* __restrict__ scale_out) {
  constexpr int kPer = DI / 64;
  const int lane = threadIdx.x & 63;
  const int b = blockIdx.x * (kWriteThreads / 64) + (threadIdx.x >> 6);
  if (b >= n) return;
  const int p = blk[b];
  if (p < 0 || p >= kv.num_blocks) return;
  float v[kPer];
  float a = 0.f;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    v[u] = x[(size_t)b * DI + lane + 64 * u];
    a = fmaxf(a, fabsf(v[u]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
  if (a == 0.f) a = 1.f;
  const float ks = a / 448.0f;  // IEEE division, rounded once
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const float y = fminf(fmaxf(v[u] / ks, -448.0f), 448.0f);
    // v_cvt_pk_fp8_f32: E4M3, round to nearest even
    const uint32_t code = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y, 0.0f, 0, false) & 0xFFu;
    keys_out[(size_t)p * DI + lane + 64 * u] = (uint8_t)code;
  }
  if (lane == 0) scale_out[p] = ks;
}

}  // namespace

hipError_t launch_kv_write(const KvView& kv, int n, const int32_t* tok_seq, const int32_t* tok_pos,
                           const void* k_new, const void* v_new, void* k_out, void* v_out,
                           hipStream_t st) {
  const long total = 2L * n * kv.num_kv_heads * (kHeadDim / 8);
  long wgs = (total + kWriteThreads - 1) / kWriteThreads;
  if (wgs > 8192) wgs = 8192;
  hipLaunchKernelGGL(kv_write_rows, dim3((unsigned)wgs), dim3(kWriteThreads), 0, st, kv, n,
                     tok_seq, tok_pos, static_cast<const uint4*>(k_new),
                     static_cast<const uint4*>(v_new), static_cast<uint4*>(k_out),
                     static_cast<uint4*>(v_out));
  return hipGetLastError();
}

hipError_t launch_index_key_write(const KvView& kv, int n, const int32_t* blk, const float* x,
                                  uint8_t* keys_out, float* scale_out, hipStream_t st) {
  const dim3 grid((n + kWriteThreads / 64 - 1) / (kWriteThreads / 64)), block(kWriteThreads);
  if (kv.idx_dim == 64) {
    hipLaunchKernelGGL(index_key_rows<64>, grid, block, 0, st, kv, n, blk, x, keys_out, scale_out);
  } else {
    hipLaunchKernelGGL(index_key_rows<128>, grid, block, 0, st, kv, n, blk, x, keys_out, scale_out);
  }
  return hipGetLastError();
}

}  // namespace dsa

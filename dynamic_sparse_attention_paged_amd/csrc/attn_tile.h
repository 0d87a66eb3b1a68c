// One 64-token tile of attention for one wave: the building blocks shared by
// the per-query kernel (attn.hip) and the block-inverted prefill kernel
// (prefill_inv.hip).
//
// With the 16 MFMA columns holding 16 (query, head) columns:
//   S^T[64 tok x 16] = K[64 x 128] . Q^T        16 x mfma 16x16x32 bf16
//   softmax per column (column = lane % 16 in every tile), base 2
//   O^T[128 x 16] += V^T[128 x 64] . P^T[64 x 16]  32 x mfma (P = hi + lo bf16)
// K is an MFMA operand read straight from memory (8 consecutive dims per
// lane); V is read 8 tokens per lane, so it is staged in LDS, in an
// XOR-swizzled layout read back with the gfx950 transpose read.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace dsa {
namespace tile {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) short i16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x4 mfma_bf16(i16x8 a, i16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

struct WaveState {
  float m;      // running max (base-2 logits) of the lane's head
  float l;      // running sum of 2^(x - m)
  f32x4 o[8];   // O^T tiles: o[dt][i] = O[head = lane%16][d = 16 dt + 4 (lane/16) + i]
};

typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

// V tile of one block and KV head in LDS: 64 token rows of 256 B, no padding.
// The 16 B chunk c (dims 8c .. 8c+7) of token row t sits in chunk slot
// c ^ (2 (t & 3)), which makes the transposed reads below bank-conflict free.
// Loaded straight from global memory into LDS (16 B per lane, lane l of a
// load landing at LDS offset 16 l), so V takes no registers.
//
// kNT: non-temporal loads (the nt cache policy), for data read once per
// call, as in decode, where the gather streams every selected block once and
// nothing is reused; plain loads where the same blocks serve many queries
// (prefill).  A streaming-read probe of the whole chip reads ~7.0 TB/s with
// nt loads against ~6.2 TB/s with plain ones.
constexpr int kCpolNT = 2;  // the cache-policy operand's nt bit (gfx950)

template <bool kNT = false>
__device__ __forceinline__ void dma_v(const uint16_t* __restrict__ vbase, size_t tok_stride,
                                      uint32_t lane_off, uint16_t* vs) {
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    // uniform part (rows 4u ..) in scalar registers, lane part loop-invariant
    const char* rows = reinterpret_cast<const char*>(vbase + (size_t)(4 * u) * tok_stride);
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint16_t*>(rows + lane_off),
                                     (lds_void_t*)(vs + 512 * u), 16, 0, kNT ? kCpolNT : 0);
  }
}

// Byte offset of lane l's 16 B of a V row group: token row l / 16 of the
// group, chunk (l % 16) ^ 2 (row), the swizzle the transposed reads expect.
__device__ __forceinline__ uint32_t dma_v_lane_offset(size_t tok_stride, int lane) {
  const int row_in = lane >> 4;
  const int chunk = (lane & 15) ^ (2 * row_in);
  return (uint32_t)(((size_t)row_in * tok_stride + 8 * chunk) * 2);
}

// K tile as MFMA A operands: k[T][c] = K[token 16T + r][dims 32c + 8gq .. +8];
// lane_off = (r * tok_stride + 8 gq) * 2 bytes.
template <bool kNT = false>
__device__ __forceinline__ void load_k(const uint16_t* __restrict__ kbase, size_t tok_stride,
                                       uint32_t lane_off, i16x8 (&kf)[4][4]) {
#pragma unroll
  for (int T = 0; T < 4; ++T) {
    const char* rows = reinterpret_cast<const char*>(kbase + (size_t)(16 * T) * tok_stride);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const i16x8* a = reinterpret_cast<const i16x8*>(rows + lane_off + 64 * c);
      kf[T][c] = kNT ? __builtin_nontemporal_load(a) : *a;
    }
  }
}

// S^T = K Q^T for one block: sc[T][i] is token 16T + 4gq + i of head r.
__device__ __forceinline__ void block_logits(const i16x8 (&kf)[4][4], const i16x8 (&qf)[4],
                                             f32x4 (&sc)[4]) {
#pragma unroll
  for (int T = 0; T < 4; ++T) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c) acc = mfma_bf16(kf[T][c], qf[c], acc);
    sc[T] = acc;
  }
}

// Online softmax over one block's logits and O^T += V^T P^T.  Tokens a > lim
// (past the query position or the sequence) are masked.
__device__ __forceinline__ void block_softmax_pv(f32x4 (&sc)[4], float scale2, int tok0, int lim,
                                                 const uint16_t* vs, WaveState& st) {
  const int lane = threadIdx.x & 63;
  const int gq = lane >> 4;
  // mask + scale (base 2); sc[T][i] is token 16T + 4gq + i of head r
  float mx = -INFINITY;
#pragma unroll
  for (int T = 0; T < 4; ++T)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int a = tok0 + 16 * T + 4 * gq + i;
      const float x = (a <= lim) ? sc[T][i] * scale2 : -INFINITY;
      sc[T][i] = x;
      mx = fmaxf(mx, x);
    }
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  // a block with no visible token leaves the state unchanged (-inf stays -inf)
  const float m_new = fmaxf(st.m, mx);
  const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
  const float alpha = __builtin_amdgcn_exp2f(st.m - m_use);  // 0 while st.m = -inf
  float rs = 0.f;
  i16x8 ph[2], pl[2];
#pragma unroll
  for (int T = 0; T < 4; ++T)
#pragma unroll
    for (int i = 0; i < 4; i += 2) {
      // p = 2^(x - m) (0 for masked tokens), split p = hi + lo into two bf16
      const f32x2 p = {__builtin_amdgcn_exp2f(sc[T][i] - m_use),
                       __builtin_amdgcn_exp2f(sc[T][i + 1] - m_use)};
      rs += p[0] + p[1];
      const bf16x2 hb = __builtin_convertvector(p, bf16x2);  // round to nearest even
      const f32x2 hf = __builtin_convertvector(hb, f32x2);
      const bf16x2 lb = __builtin_convertvector(p - hf, bf16x2);
      const uint32_t hw = __builtin_bit_cast(uint32_t, hb), lw = __builtin_bit_cast(uint32_t, lb);
      ph[T >> 1][(T & 1) * 4 + i] = (short)(hw & 0xFFFFu);
      ph[T >> 1][(T & 1) * 4 + i + 1] = (short)(hw >> 16);
      pl[T >> 1][(T & 1) * 4 + i] = (short)(lw & 0xFFFFu);
      pl[T >> 1][(T & 1) * 4 + i + 1] = (short)(lw >> 16);
    }
  rs += __shfl_xor(rs, 16, 64);
  rs += __shfl_xor(rs, 32, 64);
  st.l = st.l * alpha + rs;
  st.m = m_new;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) st.o[dt] *= alpha;

  // O^T += V^T . P^T.  k-slot s = 4h + i of lane group gq <-> token 16 (2 ks + h) + 4 gq + i.
  // ds_read_b64_tr_b16: within a 16-lane group, lane 4a+b receives element i
  // from the 4 u16 at the address of lane 4i+a, offset b.  Lane 4i+a therefore
  // points at token 16 (2 ks + h) + 4 gq + i, dims 16 dt + 4a .. +3, and lane
  // (gq, r) receives V[token(s)][16 dt + r] for its four slots.
  const int ti = (lane >> 2) & 3, ta = lane & 3;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      i16x8 va;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int t = 16 * (2 * ks + h) + 4 * gq + ti;
        const int slot = 2 * (dt ^ ti) + (ta >> 1);  // chunk (2 dt + ta/2) ^ 2 (t & 3)
        const uint16_t* a = vs + t * 128 + 8 * slot + 4 * (ta & 1);
        const i16x4 v4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)a);
        va[4 * h + 0] = v4[0];
        va[4 * h + 1] = v4[1];
        va[4 * h + 2] = v4[2];
        va[4 * h + 3] = v4[3];
      }
      st.o[dt] = mfma_bf16(va, ph[ks], st.o[dt]);
      st.o[dt] = mfma_bf16(va, pl[ks], st.o[dt]);
    }
  }
}

// One selected block for one wave: S^T = K Q^T, online softmax, O^T += V^T P^T.
__device__ __forceinline__ void attend_block(const i16x8 (&kf)[4][4], const i16x8 (&qf)[4],
                                             float scale2, int tok0, int lim, const uint16_t* vs,
                                             WaveState& st) {
  f32x4 sc[4];
  block_logits(kf, qf, sc);
  block_softmax_pv(sc, scale2, tok0, lim, vs, st);
}

}  // namespace tile
}  // namespace dsa

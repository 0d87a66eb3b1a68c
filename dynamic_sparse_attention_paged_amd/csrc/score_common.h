// Device helpers for exact FP8 indexer scoring (shared by the scoring and
// the fused scoring + selection kernels).  What is computed is described in
// index_score.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "dsa_internal.h"

namespace dsa {

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

template <int kByte>
__device__ __forceinline__ float e4m3_to_f32(uint32_t word) {
  return __builtin_amdgcn_cvt_f32_fp8((int)word, kByte);
}

__device__ __forceinline__ float e4m3_byte_to_f32(uint32_t word, int byte) {
  switch (byte) {
    case 0: return e4m3_to_f32<0>(word);
    case 1: return e4m3_to_f32<1>(word);
    case 2: return e4m3_to_f32<2>(word);
    default: return e4m3_to_f32<3>(word);
  }
}

__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  // v_cvt_pk_fp8_f32: round to nearest even into OCP E4M3; |x| <= 448 here.
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x, 0.0f, 0, false) & 0xFFu;
}

// Quantize the query's indexer heads into LDS.  qv[d * HP + h] holds the
// float64 value of the E4M3 code (zero for padded heads h >= hi).  Each
// head's max |q| is reduced by one wave (shuffles, no LDS atomics).
template <int DI, int HP>
__device__ void load_query(const QView& Q, int qi, double* qv, double* sq, double* w, int* expo) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = tid >> 6, nwaves = blockDim.x >> 6;
  const int hi = Q.hi;
  const uint16_t* src = Q.q_idx + (size_t)qi * hi * DI;
  for (int h = wave; h < HP; h += nwaves) {
    float a = 0.f;
    if (h < hi) {
#pragma unroll
      for (int e = lane; e < DI; e += 64) a = fmaxf(a, fabsf(bf16_to_f32(src[h * DI + e])));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
    if (lane == 0) {
      int e = 0;
      double wh = 0.0;
      if (h < hi) {
        if (a != 0.0f) {
          int E;
          const float f = frexpf(a, &E);  // a = f 2^E, f in [0.5, 1)
          e = (f <= 0.875f) ? E - 9 : E - 8;
        }
        wh = (double)Q.w[(size_t)qi * hi + h];
      }
      expo[h] = e;
      sq[h] = ldexp(1.0, e);
      w[h] = wh;
    }
  }
  __syncthreads();
  for (int e = tid; e < DI * HP; e += blockDim.x) {
    const int d = e / HP, h = e % HP;
    double val = 0.0;
    if (h < hi) {
      const float x = ldexpf(bf16_to_f32(src[h * DI + d]), -expo[h]);  // exact
      val = (double)e4m3_to_f32<0>(f32_to_e4m3(x));
    }
    qv[e] = val;
  }
  __syncthreads();
}

// Four lanes per block: lane group gq = lane / 16 owns dims
// [gq DI/4, (gq+1) DI/4) of the key row of block (lane % 16) of the wave.
template <int DI>
struct KeyQuarter {
  uint4 w[DI / 64];
  float ks;
  int p;
};

// Request the block-table entry, key quarter and scale of logical block j.
template <int DI>
__device__ __forceinline__ void fetch_key_quarter(const KvView& kv, int s, int j, int gq,
                                                  KeyQuarter<DI>& kq) {
  kq.p = kv.table[(size_t)s * kv.maxb + j];
  const uint4* krow =
      reinterpret_cast<const uint4*>(kv.idx_keys + (size_t)kq.p * DI + gq * (DI / 4));
#pragma unroll
  for (int i = 0; i < DI / 64; ++i) kq.w[i] = krow[i];
  kq.ks = gq == 0 ? kv.idx_scale[kq.p] : 0.f;
}

// Exact scores of the NB blocks whose key quarters this lane holds (blocks
// not fetched must hold zero key words); the results are meaningful in lane
// group 0.  Each float64 query value read from
// LDS feeds NB blocks.  Partial float64 dot products of exact products are
// exact, so combining the four quarters in any order is exact; the epilogue
// is evaluated in float64 in ascending head order, unfused.
template <int DI, int HP, int NB>
__device__ __forceinline__ void score_quarters(const KeyQuarter<DI> (&kq)[NB], int gq,
                                               const double* qv, const double* sq,
                                               const double* wq, float (&S_out)[NB]) {
  double acc[NB][HP];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int h = 0; h < HP; ++h) acc[b][h] = 0.0;
#pragma unroll
  for (int i = 0; i < DI / 64; ++i) {
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) {
#pragma unroll
      for (int bt = 0; bt < 4; ++bt) {
        const int d = gq * (DI / 4) + i * 16 + wd * 4 + bt;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const uint32_t words[4] = {kq[b].w[i].x, kq[b].w[i].y, kq[b].w[i].z, kq[b].w[i].w};
          const double kd = (double)e4m3_byte_to_f32(words[wd], bt);
#pragma unroll
          for (int h = 0; h < HP; ++h) acc[b][h] = fma(qv[d * HP + h], kd, acc[b][h]);
        }
      }
    }
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) {
#pragma unroll
    for (int h = 0; h < HP; ++h) {
      acc[b][h] += __shfl_xor(acc[b][h], 16, 64);
      acc[b][h] += __shfl_xor(acc[b][h], 32, 64);
    }
    const double ks = (double)kq[b].ks;
    double S = 0.0;
    {
#pragma clang fp contract(off)
#pragma unroll
      for (int h = 0; h < HP; ++h) {
        const double t = (sq[h] * ks) * acc[b][h];
        const double r = t > 0.0 ? t : 0.0;
        S = S + wq[h] * r;
      }
    }
    S_out[b] = (float)S;
  }
}

// Exact scores of chunk `chunk` of query qi: logical blocks chunk 64 NB ..
// + 64 NB, by a workgroup of four waves.  Lanes: four per block (key
// quarters), each lane holding NB blocks 16 apart, so that wave w covers
// blocks 16 NB w .. + 16 NB of the chunk and lane l's block b is
// j(b) = chunk 64 NB + 16 NB w + l % 16 + 16 b.  Block-table entries, key
// quarters and scales are requested first, before the query position is
// known (physical ids clamped into the pool, so the speculative reads stay in
// bounds), so that the table -> key chain overlaps the position read and the
// query prologue.  Returns false, uniformly and before any LDS use, when the
// whole chunk lies past the query's local block; otherwise S[b] (meaningful
// in lane group 0) is block j(b)'s score and visible[b] whether j(b) is at or
// below the local block (and inside the table row).  qv, sq, wq, expo: LDS
// of load_query.
template <int DI, int HP, int NB>
__device__ __forceinline__ bool score_chunk(const KvView& kv, const QView& Q, int qi, int chunk,
                                            double* qv, double* sq, double* wq, int* expo,
                                            float (&S)[NB], bool (&visible)[NB], int& local) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int gq = lane >> 4;
  const int j0 = chunk * 64 * NB + wave * 16 * NB + (lane & 15);
  const int s = query_seq(Q, qi);
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
  local = pos >> kv.bs_shift;
  if (chunk * 64 * NB > local) return false;
  // invisible blocks score zero key words (their result is ignored)
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
  load_query<DI, HP>(Q, qi, qv, sq, wq, expo);
  score_quarters<DI, HP, NB>(kq, gq, qv, sq, wq, S);
  return true;
}

}  // namespace dsa

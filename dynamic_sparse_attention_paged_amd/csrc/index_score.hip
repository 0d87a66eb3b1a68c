// Indexer scoring: one coarse FP8 key per KV block, scored against the query.
//
// What is computed ([P1] "Day-0 Adaptation for Massive LLMs...", section
// 4(1) "Index Selection"; [P5] "Day-0 Readiness for Trillion-Parameter
// Models...", "Index Selection Path": a lightweight inner product with
// low-precision inputs), for query q and visible logical block j with
// physical block p = table[s][j]:
//
//   sq[h] = 2^e[h], the smallest power of two with max|q_idx[h,:]| <= 448 sq[h]
//   q8[h,:] = E4M3(q_idx[h,:] / sq[h])              (round to nearest even)
//   D[h] = sum_d q8[h,d] k8[p,d]                     (exact)
//   S = sum_{h ascending} w[h] * max(0, (sq[h] * ks[p]) * D[h])   in float64,
//   stored rounded to fp32.
//
// Exactness: every E4M3 value is a multiple of 2^-9 below 2^9, so products
// are multiples of 2^-18 below 2^18 and any partial sum of <= 128 of them
// fits in 43 bits; float64 FMA accumulation is therefore exact in any order.
// The gfx950 FP8 MFMA does not accumulate exactly (it aligns products to the
// largest one and drops low bits), so it cannot reproduce these scores.
//
// Mapping: four lanes per logical block, each owning a quarter of the key
// row (16 or 32 B, read with 16 B loads); 16 blocks per wave.  The query's
// decoded FP8 values live in LDS as float64 [dI][HP]; a read serves the 16
// lanes of a quarter with one broadcast address.
#include <hip/hip_runtime.h>
#include <math.h>

#include "dsa_internal.h"

namespace dsa {
namespace {

constexpr int kScoreThreads = 256;
constexpr int kBlocksPerWg = 64;  // 4 lanes per block

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
// float64 value of the E4M3 code (zero for padded heads h >= hi).
template <int DI, int HP>
__device__ void load_query(const QView& Q, int qi, double* qv, double* sq, double* w,
                           uint32_t* amax_bits, int* expo) {
  const int tid = threadIdx.x;
  const int hi = Q.hi;
  const uint16_t* src = Q.q_idx + (size_t)qi * hi * DI;
  if (tid < HP) amax_bits[tid] = 0u;
  __syncthreads();
  for (int e = tid; e < hi * DI; e += blockDim.x) {
    const float x = fabsf(bf16_to_f32(src[e]));
    atomicMax(&amax_bits[e / DI], __builtin_bit_cast(uint32_t, x));
  }
  __syncthreads();
  if (tid < HP) {
    int e = 0;
    double wh = 0.0;
    if (tid < hi) {
      const float a = __builtin_bit_cast(float, amax_bits[tid]);
      if (a != 0.0f) {
        int E;
        const float f = frexpf(a, &E);  // a = f 2^E, f in [0.5, 1)
        e = (f <= 0.875f) ? E - 9 : E - 8;
      }
      wh = (double)Q.w[(size_t)qi * hi + tid];
    }
    expo[tid] = e;
    sq[tid] = ldexp(1.0, e);
    w[tid] = wh;
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

// Lanes: 4 per block (dims DI/4 each), 16 blocks per wave, 64 per workgroup.
// Partial dot products of exact products are exact in float64, so the order
// in which the four lanes' partials are combined does not matter.
template <int DI, int HP>
__global__ __launch_bounds__(kScoreThreads) void index_score_exact(KvView kv, QView Q,
                                                                   float* __restrict__ scores) {
  __shared__ double qv[DI * HP];
  __shared__ double sq[HP], wq[HP];
  __shared__ uint32_t amax_bits[HP];
  __shared__ int expo[HP];
  constexpr int kSlice = DI / 4;  // dims per lane

  const int qi = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int gq = lane >> 4;
  const int j = blockIdx.x * kBlocksPerWg + wave * 16 + (lane & 15);
  const int s = query_seq(Q, qi);
  const int len = kv.seq_lens[s];
  const int pos = Q.q_pos ? Q.q_pos[qi] : len - 1;
  const int local = pos / kBlockSize;
  float* row = scores + (size_t)qi * kv.maxb;

  // Workgroups whose blocks are all invisible only write -inf.
  if (blockIdx.x * kBlocksPerWg > local) {
    if (gq == 0 && j < kv.maxb) row[j] = -INFINITY;
    return;
  }
  // Block-table entry, key slice and scale are requested before the query
  // prologue so that their latency overlaps it.
  const bool visible = j <= local && j < kv.maxb;
  int p = 0;
  uint4 kw[kSlice / 16];
  float ks_f = 0.f;
  if (visible) {
    p = kv.table[(size_t)s * kv.maxb + j];
    const uint4* krow = reinterpret_cast<const uint4*>(kv.idx_keys + (size_t)p * DI + gq * kSlice);
#pragma unroll
    for (int i = 0; i < kSlice / 16; ++i) kw[i] = krow[i];
    if (gq == 0) ks_f = kv.idx_scale[p];
  }
  load_query<DI, HP>(Q, qi, qv, sq, wq, amax_bits, expo);
  double acc[HP];
#pragma unroll
  for (int h = 0; h < HP; ++h) acc[h] = 0.0;
  if (visible) {
#pragma unroll
    for (int i = 0; i < kSlice / 16; ++i) {
      const uint32_t words[4] = {kw[i].x, kw[i].y, kw[i].z, kw[i].w};
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int d = gq * kSlice + i * 16 + wd * 4 + b;
          const double kd = (double)e4m3_byte_to_f32(words[wd], b);
#pragma unroll
          for (int h = 0; h < HP; ++h) acc[h] = fma(qv[d * HP + h], kd, acc[h]);
        }
      }
    }
  }
  // combine the four dim slices (exact)
#pragma unroll
  for (int h = 0; h < HP; ++h) {
    acc[h] += __shfl_xor(acc[h], 16, 64);
    acc[h] += __shfl_xor(acc[h], 32, 64);
  }
  if (gq != 0 || j >= kv.maxb) return;
  if (!visible) {
    row[j] = -INFINITY;
    return;
  }
  const double ks = (double)ks_f;
  double S = 0.0;
  {
#pragma clang fp contract(off)
#pragma unroll
    for (int h = 0; h < HP; ++h) {
      const double t = (sq[h] * ks) * acc[h];
      const double r = t > 0.0 ? t : 0.0;
      S = S + wq[h] * r;
    }
  }
  row[j] = (float)S;
}

template <int DI, int HP>
hipError_t launch_t(const KvView& kv, const QView& Q, float* scores, hipStream_t st) {
  dim3 grid((kv.maxb + kBlocksPerWg - 1) / kBlocksPerWg, Q.nq);
  hipLaunchKernelGGL((index_score_exact<DI, HP>), grid, dim3(kScoreThreads), 0, st, kv, Q,
                     scores);
  return hipGetLastError();
}

template <int DI>
hipError_t launch_di(const KvView& kv, const QView& Q, float* scores, hipStream_t st) {
  if (Q.hi <= 1) return launch_t<DI, 1>(kv, Q, scores, st);
  if (Q.hi <= 2) return launch_t<DI, 2>(kv, Q, scores, st);
  if (Q.hi <= 4) return launch_t<DI, 4>(kv, Q, scores, st);
  if (Q.hi <= 8) return launch_t<DI, 8>(kv, Q, scores, st);
  return launch_t<DI, 16>(kv, Q, scores, st);
}

}  // namespace

hipError_t launch_index_score(const KvView& kv, const QView& Q, float* scores, hipStream_t st) {
  if (kv.idx_dim == 64) return launch_di<64>(kv, Q, scores, st);
  return launch_di<128>(kv, Q, scores, st);
}

}  // namespace dsa

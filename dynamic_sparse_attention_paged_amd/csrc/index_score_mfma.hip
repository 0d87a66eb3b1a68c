// Exact FP8 indexer scoring on the int8 matrix cores, for batches of many
// queries (chunked prefill).
//
// What is computed is exactly what index_score.hip computes ([P1] "Day-0
// Adaptation for Massive LLMs...", section 4(1); [P5] "Day-0 Readiness for
// Trillion-Parameter Models...", "Index Selection Path"; prefill batches the
// selection for many queries, [P5] "Differentiated Adaptation of Prefill and
// Decode"):
//   S[q, j] = sum_{h ascending} w[q,h] * max(0, (sq[q,h] * ks[p]) * D[q,h,j]),
//   D[q,h,j] = sum_d q8[q,h,d] k8[p,d]                (exact),
// evaluated in float64 and rounded to fp32.
//
// Exactness on the matrix cores.  Every E4M3 value is n * 2^-9 with an
// integer |n| <= 229376 < 2^18.  Writing |n| in base 128 gives three digits
// (|n| & 127, (|n| >> 7) & 127, |n| >> 14), each carrying the sign of n, so
// every digit fits in int8.  With query digits a_i and key digits b_j,
//   D * 2^18 = sum_{c=0..4} 2^(7c) G_c,   G_c = sum_{i+j=c} sum_d a_i[d] b_j[d],
// and each G_c is a sum of at most 3 * 128 products of magnitude < 2^14, so
// v_mfma_i32_16x16x64_i8 accumulates it exactly in int32.  (The FP8 MFMA
// aligns products to the largest one and drops low bits, so it is not used.)
// Cost: nine digit-pair products, i.e. nine times the int8 MFMA work of a
// single FP8 contraction.
//
// Tiling (MFMA rows = (query, indexer head), columns = blocks, k = dims):
// a workgroup is 4 waves x 8 queries (HP = 8) or 16 queries (HP = 4), over a
// range of 512 blocks.  Query digits stay in registers for the whole block
// loop; each 16-block tile's key digits are built from the E4M3 codes through
// a 256-entry table in LDS.  The epilogue combines the five int32 sums
// exactly, applies scales and ReLU in float64 and sums the heads in
// ascending order within the lane that holds them.
#include <hip/hip_runtime.h>
#include <math.h>

#include "dsa_internal.h"

namespace dsa {
namespace {

typedef __attribute__((ext_vector_type(4))) int i32x4;

constexpr int kMfmaWaves = 4;
constexpr int kRowTiles = 4;           // 16-row MFMA tiles per wave
constexpr int kBlocksPerWg = 512;      // block range of one workgroup

__device__ __forceinline__ float bf16f(uint16_t b) { return __builtin_bit_cast(float, (uint32_t)b << 16); }

// Signed base-128 digits of the E4M3 code c, packed as int8 in bytes 0..2.
__device__ __forceinline__ uint32_t digits_of_code(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const uint32_t n = e == 0 ? m : (8u + m) << (e - 1);  // |value| * 2^9
  int d0 = (int)(n & 127u), d1 = (int)((n >> 7) & 127u), d2 = (int)(n >> 14);
  if (c & 0x80u) {
    d0 = -d0;
    d1 = -d1;
    d2 = -d2;
  }
  return ((uint32_t)(d0 & 0xFF)) | ((uint32_t)(d1 & 0xFF) << 8) | ((uint32_t)(d2 & 0xFF) << 16);
}

// The three digit planes of four codes packed in `w` (one code per byte):
// one table lookup per code, then byte permutes gather digit p of the four
// codes into plane word p.
__device__ __forceinline__ void planes_of_word(const uint32_t* lut, uint32_t w, uint32_t& p0,
                                               uint32_t& p1, uint32_t& p2) {
  const uint32_t l0 = lut[w & 0xFFu], l1 = lut[(w >> 8) & 0xFFu];
  const uint32_t l2 = lut[(w >> 16) & 0xFFu], l3 = lut[w >> 24];
  // perm(hi, lo, sel): byte i of the result is byte sel_i of {hi:lo}
  // (0..3 from lo, 4..7 from hi, 0x0c gives zero)
  const uint32_t a01 = __builtin_amdgcn_perm(l1, l0, 0x05010400u);  // l0.d0 l1.d0 l0.d1 l1.d1
  const uint32_t a23 = __builtin_amdgcn_perm(l3, l2, 0x05010400u);
  const uint32_t b01 = __builtin_amdgcn_perm(l1, l0, 0x0c0c0602u);  // l0.d2 l1.d2
  const uint32_t b23 = __builtin_amdgcn_perm(l3, l2, 0x0c0c0602u);
  p0 = __builtin_amdgcn_perm(a23, a01, 0x05040100u);
  p1 = __builtin_amdgcn_perm(a23, a01, 0x07060302u);
  p2 = __builtin_amdgcn_perm(b23, b01, 0x05040100u);
}

__device__ __forceinline__ void planes_of(const uint32_t* lut, const uint4& w, i32x4 (&pl)[3]) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t a, b, c;
    planes_of_word(lut, ws[i], a, b, c);
    pl[0][i] = (int)a;
    pl[1][i] = (int)b;
    pl[2][i] = (int)c;
  }
}

__device__ __forceinline__ i32x4 mfma_i8(const i32x4& a, const i32x4& b, const i32x4& c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// grid (ceil(maxb / kBlocksPerWg), ceil(Nq / queries per workgroup)), block 256.
//
// Rows of the MFMA tiles: with T = HP / 4 tiles per group of four queries,
// row r of tile t is query 4 (t / T) + r / 4 of the wave, indexer head
// 4 (t % T) + r % 4.  Lane (g, c) of the result (g = lane / 16) then holds
// heads 4 (t % T) .. +3 of query 4 (t / T) + g for block c, so the ascending
// head sum of a (query, block) pair stays within one lane.
template <int DI, int HP>
__global__ __launch_bounds__(64 * kMfmaWaves) __attribute__((amdgpu_waves_per_eu(2)))
void index_score_i8(KvView kv, QView Q, float* __restrict__ scores) {
  constexpr int KC = DI / 64;          // 64-wide k chunks
  constexpr int T = HP / 4;            // tiles per group of four queries
  constexpr int kQPerWave = 4 * kRowTiles / T;
  constexpr int kQPerWg = kMfmaWaves * kQPerWave;
  __shared__ uint32_t lut[256];
  __shared__ double wsq[kQPerWg * HP];  // w * sq * 2^-18 per (query, head)

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int gq = lane >> 4, r = lane & 15;
  for (int c = threadIdx.x; c < 256; c += 64 * kMfmaWaves) lut[c] = digits_of_code((uint32_t)c);
  __syncthreads();

  const int q_wave0 = blockIdx.y * kQPerWg + wave * kQPerWave;  // first query of this wave
  const int j_begin = blockIdx.x * kBlocksPerWg;
  const int j_end = min(kv.maxb, j_begin + kBlocksPerWg);
  int loc[kQPerWave], seq[kQPerWave];
#pragma unroll
  for (int t = 0; t < kQPerWave; ++t) {
    const int q = q_wave0 + t;
    if (q < Q.nq) {
      seq[t] = query_seq(Q, q);
      const int pos = Q.q_pos ? Q.q_pos[q] : kv.seq_lens[seq[t]] - 1;
      loc[t] = pos / kBlockSize;
    } else {
      seq[t] = -1;
      loc[t] = -1;
    }
  }

  // ---- query digits (A operands): lane (gq, r) holds row r of each tile,
  // dims 16 gq .. +16 of every 64-wide chunk.
  i32x4 qa[kRowTiles][KC][3];
#pragma unroll
  for (int t = 0; t < kRowTiles; ++t) {
    const int qloc = 4 * (t / T) + r / 4;  // query within the wave
    const int h = 4 * (t % T) + r % 4;
    const int q = q_wave0 + qloc;
    const bool live = q < Q.nq;
    float x[KC][16];
    float amax = 0.f;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      uint4 raw[2] = {make_uint4(0u, 0u, 0u, 0u), make_uint4(0u, 0u, 0u, 0u)};
      if (live) {
        const uint4* src = reinterpret_cast<const uint4*>(
            Q.q_idx + ((size_t)q * HP + h) * DI + 64 * kc + 16 * gq);
        raw[0] = src[0];
        raw[1] = src[1];
      }
      const uint32_t wv[8] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w,
                              raw[1].x, raw[1].y, raw[1].z, raw[1].w};
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        x[kc][e] = bf16f((uint16_t)(wv[e >> 1] >> (16 * (e & 1))));
        amax = fmaxf(amax, fabsf(x[kc][e]));
      }
    }
    // the four lanes holding row r cover all DI dims of (query, head)
    amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
    int ex = 0;
    if (amax != 0.f) {
      int E;
      const float f = frexpf(amax, &E);  // amax = f 2^E, f in [0.5, 1)
      ex = (f <= 0.875f) ? E - 9 : E - 8;
    }
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      uint32_t codes[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float y = ldexpf(x[kc][e], -ex);  // exact
        const uint32_t code =
            (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y, 0.0f, 0, false) & 0xFFu;  // RNE
        codes[e >> 2] |= code << (8 * (e & 3));
      }
      planes_of(lut, make_uint4(codes[0], codes[1], codes[2], codes[3]), qa[t][kc]);
    }
    // Scale 2^ex of (query, head) folded into its weight, with the 2^-18 of
    // the digit products: both are powers of two, so w (2^ex (ks D)) and
    // (w 2^(ex-18)) (ks D') round alike (D' = 2^18 D, no overflow or
    // underflow in float64 for finite fp32 / bf16 inputs).
    if (gq == 0)
      wsq[wave * kQPerWave * HP + qloc * HP + h] =
          live ? ldexp((double)Q.w[(size_t)q * HP + h], ex - 18) : 0.0;
  }
  __syncthreads();
  const double* wsw = wsq + wave * kQPerWave * HP;

  // This lane's queries in the epilogue: 4 g + gq for group g = t / T.
  constexpr int kGroups = kRowTiles / T;
  int my_loc[kGroups];
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    my_loc[g] = loc[4 * g];
#pragma unroll
    for (int i = 1; i < 4; ++i)
      if (gq == i) my_loc[g] = loc[4 * g + i];
  }

  // One pass per distinct sequence among the wave's queries (a prefill chunk
  // has one): the key tile of a block comes from that sequence's table row.
  uint32_t pending = 0u;
#pragma unroll
  for (int t = 0; t < kQPerWave; ++t) pending |= (seq[t] >= 0) ? (1u << t) : 0u;
  while (pending) {
    int s_u = -1;
#pragma unroll
    for (int t = kQPerWave - 1; t >= 0; --t)
      if ((pending >> t) & 1u) s_u = seq[t];
    uint32_t members = 0u;
    int lmax = -1;
#pragma unroll
    for (int t = 0; t < kQPerWave; ++t)
      if (seq[t] == s_u) {
        members |= 1u << t;
        lmax = max(lmax, loc[t]);
      }
    pending &= ~members;

    for (int jt = j_begin; jt < j_end; jt += 16) {
      const int j = jt + r;  // this lane's block (column of every tile)
      if (jt > lmax) {
        // invisible to every query of this sequence: only -inf
        if (j < j_end && gq == 0) {
#pragma unroll
          for (int t = 0; t < kQPerWave; ++t)
            if ((members >> t) & 1u) scores[(size_t)(q_wave0 + t) * kv.maxb + j] = -INFINITY;
        }
        continue;
      }
      // key digits (B operands) of block j: dims 16 gq .. +16 of each chunk
      const bool jv = j < j_end && j <= lmax;
      uint4 kw[KC];
      float ks = 0.f;
      if (jv) {
        const int p = kv.table[(size_t)s_u * kv.maxb + j];
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
          kw[kc] = *reinterpret_cast<const uint4*>(kv.idx_keys + (size_t)p * DI + 64 * kc + 16 * gq);
        ks = kv.idx_scale[p];
      } else {
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) kw[kc] = make_uint4(0u, 0u, 0u, 0u);
      }
      i32x4 kb[KC][3];
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) planes_of(lut, kw[kc], kb[kc]);
      const double ksd = (double)ks;

      double S = 0.0;
#pragma unroll
      for (int t = 0; t < kRowTiles; ++t) {
        i32x4 G[5];
#pragma unroll
        for (int c = 0; c < 5; ++c) G[c] = i32x4{0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 3; ++i)
#pragma unroll
          for (int jj = 0; jj < 3; ++jj)
#pragma unroll
            for (int kc = 0; kc < KC; ++kc)
              G[i + jj] = mfma_i8(qa[t][kc][i], kb[kc][jj], G[i + jj]);
        const int qloc = 4 * (t / T) + gq;
        if (t % T == 0) S = 0.0;
        {
#pragma clang fp contract(off)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            // D' = G0 + 2^7 G1 + 2^14 G2 + 2^21 G3 + 2^28 G4 = lo + 2^14 hi, with
            // |lo|, |hi| < 2^30 (|G_c| < 2^23 for DI <= 128; |G4| < 2^15 since
            // top digits are at most 14), so lo and hi are exact in int32 and
            // D' = lo + 2^14 hi (|D'| < 2^44) is exact in float64.
            const int lo = G[0][i4] + G[1][i4] * 128;
            const int hi = G[2][i4] + G[3][i4] * 128 + G[4][i4] * 16384;
            const double D = fma((double)hi, 16384.0, (double)lo);
            const double y = ksd * D;
            const double rr = y > 0.0 ? y : 0.0;
            S = S + wsw[qloc * HP + 4 * (t % T) + i4] * rr;
          }
        }
        if (t % T == T - 1) {
          const int q = q_wave0 + qloc;
          if (((members >> qloc) & 1u) && j < j_end)
            scores[(size_t)q * kv.maxb + j] = (j <= my_loc[t / T]) ? (float)S : -INFINITY;
        }
      }
    }
  }
}

template <int DI, int HP>
hipError_t launch_t(const KvView& kv, const QView& Q, float* scores, hipStream_t st) {
  constexpr int kQPerWg = kMfmaWaves * kRowTiles * (16 / HP);
  const dim3 grid((kv.maxb + kBlocksPerWg - 1) / kBlocksPerWg, (Q.nq + kQPerWg - 1) / kQPerWg);
  hipLaunchKernelGGL((index_score_i8<DI, HP>), grid, dim3(64 * kMfmaWaves), 0, st, kv, Q, scores);
  return hipGetLastError();
}

}  // namespace

bool index_score_mfma_supported(const KvView& kv, const QView& Q) {
  // many queries of one sequence (a prefill chunk); 4 or 8 indexer heads
  return Q.q_seq != nullptr && Q.nq >= 256 && (Q.hi == 4 || Q.hi == 8) &&
         (kv.idx_dim == 64 || kv.idx_dim == 128);
}

hipError_t launch_index_score_mfma(const KvView& kv, const QView& Q, float* scores,
                                   hipStream_t st) {
  if (Q.hi == 4) {
    return kv.idx_dim == 64 ? launch_t<64, 4>(kv, Q, scores, st) : launch_t<128, 4>(kv, Q, scores, st);
  }
  return kv.idx_dim == 64 ? launch_t<64, 8>(kv, Q, scores, st) : launch_t<128, 8>(kv, Q, scores, st);
}

}  // namespace dsa

// Exact indexer scores of one query's visible blocks, computed by one
// workgroup on the int8 matrix cores and left in LDS (shared by the fused
// scoring + selection kernel and the decode attention kernel that scores and
// selects its own blocks).
//
// What is computed ([P1] "Day-0 Adaptation for Massive LLMs...", section 4(1)
// "Index Selection"; [P5] "Day-0 Readiness for Trillion-Parameter Models...",
// "Index Selection Path"):
//   S[j] = sum_{h ascending} w[h] * max(0, (sq[h] * ks[p]) * D[h, j])  (float64,
//   stored as fp32), D[h, j] = <q8[h, :], k8[p, :]> exact, p = table[s][j],
// the same value, bit for bit, as index_score.hip.  D is formed from base-128
// digit planes (digit_mfma.h): MFMA rows are the query's indexer heads,
// columns 16 blocks, k the key dims; the five int32 digit sums are combined
// by Horner's rule and the epilogue follows the float64 order head by head.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>

#include "digit_mfma.h"
#include "dsa_internal.h"
#include "select_common.h"

namespace dsa {

// The query operand: lane (gq, r) holds indexer head r (rows r >= HI are
// zero) at dims 16 gq .. +16 of every 64-wide chunk.
template <int DI>
struct QueryRows {
  static constexpr int KC = DI / 64;
  uint4 raw[KC][2];
  float w;
  bool live;

  // Issue the loads (first, so they overlap the caller's other set-up).
  __device__ __forceinline__ void fetch(const QView& Q, int qi, int lane) {
    const int gq = lane >> 4, r = lane & 15;
    live = r < Q.hi;
    const uint4* src =
        reinterpret_cast<const uint4*>(Q.q_idx + ((size_t)qi * Q.hi + (live ? r : 0)) * DI);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      raw[kc][0] = live ? src[8 * kc + 2 * gq] : make_uint4(0u, 0u, 0u, 0u);
      raw[kc][1] = live ? src[8 * kc + 2 * gq + 1] : make_uint4(0u, 0u, 0u, 0u);
    }
    w = live ? Q.w[(size_t)qi * Q.hi + r] : 0.f;
  }

  // Two queries' rows at once (at most hp heads each, 2 hp <= 16): lane
  // (gq, r) takes head r of query q_a for r < hp and head r - hp of query
  // q_b for hp <= r < 2 hp.  A query < 0, and heads past HI, give zero rows.
  __device__ __forceinline__ void fetch_pair(const QView& Q, int q_a, int q_b, int hp,
                                             int lane) {
    const int gq = lane >> 4, r = lane & 15;
    const bool second = r >= hp;
    const int qi = second ? q_b : q_a, h = second ? r - hp : r;
    live = qi >= 0 && h < Q.hi && r < 2 * hp;
    const uint4* src = reinterpret_cast<const uint4*>(
        Q.q_idx + ((size_t)(live ? qi : 0) * Q.hi + (live ? h : 0)) * DI);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      raw[kc][0] = live ? src[8 * kc + 2 * gq] : make_uint4(0u, 0u, 0u, 0u);
      raw[kc][1] = live ? src[8 * kc + 2 * gq + 1] : make_uint4(0u, 0u, 0u, 0u);
    }
    w = live ? Q.w[(size_t)qi * Q.hi + h] : 0.f;
  }

  // Quantize each head to E4M3 with its power-of-two scale 2^e (the smallest
  // with max |q| <= 448 2^e; round to nearest even) and split the codes into
  // digit planes.  When write_w, lane group 0 stores w[r] 2^(e - 18) to
  // wsq[r]: the power-of-two scales move only exponents, so w (2^e (ks D))
  // and (w 2^(e-18)) (ks D 2^18) round alike.
  __device__ __forceinline__ void build(const uint32_t* lut, int lane, bool write_w, double* wsq,
                                        i32x4 (&qa)[KC][3]) const {
    const int gq = lane >> 4, r = lane & 15;
    float x[KC][16];
    float amax = 0.f;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const uint32_t wv[8] = {raw[kc][0].x, raw[kc][0].y, raw[kc][0].z, raw[kc][0].w,
                              raw[kc][1].x, raw[kc][1].y, raw[kc][1].z, raw[kc][1].w};
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        x[kc][e] = bf16f((uint16_t)(wv[e >> 1] >> (16 * (e & 1))));
        amax = fmaxf(amax, fabsf(x[kc][e]));
      }
    }
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
      planes_of(lut, make_uint4(codes[0], codes[1], codes[2], codes[3]), qa[kc]);
    }
    if (write_w && gq == 0) wsq[r] = ldexp((double)w, ex - 18);
  }
};

// The exact scores of one 16-block column tile: kw / ks hold this lane's
// key words (dims 16 gq .. +16 of every 64-wide chunk) and scale of block
// column r, qa the query's digit planes, wh[i4] = wsq[4 gq + i4].  Returns,
// in lane group HP / 4 - 1, the float64 score of column r (the ascending head
// sum runs through the lane groups in order).
template <int DI, int HP>
__device__ __forceinline__ double tile_score_i8(const i32x4 (&qa)[DI / 64][3],
                                                const uint4 (&kw)[DI / 64], float ks,
                                                const uint32_t* lut, const double (&wh)[4],
                                                int lane) {
  constexpr int KC = DI / 64;
  constexpr int kGroups = HP / 4;  // lane groups holding heads
  const int gq = lane >> 4;
  i32x4 kb[KC][3];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) planes_of(lut, kw[kc], kb[kc]);
  // hi = G2 + 2^7 (G3 + 2^7 G4), lo = G0 + 2^7 G1 (exact in int32, |D| 2^18 < 2^44)
  i32x4 h = i32x4{0, 0, 0, 0}, l = i32x4{0, 0, 0, 0};
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) h = mfma_i8(qa[kc][2], kb[kc][2], h);
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) l = mfma_i8(qa[kc][0], kb[kc][1], l);
  h = h * 128;
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    h = mfma_i8(qa[kc][1], kb[kc][2], h);
    h = mfma_i8(qa[kc][2], kb[kc][1], h);
    l = mfma_i8(qa[kc][1], kb[kc][0], l);
  }
  h = h * 128;
  l = l * 128;
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    h = mfma_i8(qa[kc][0], kb[kc][2], h);
    h = mfma_i8(qa[kc][1], kb[kc][1], h);
    h = mfma_i8(qa[kc][2], kb[kc][0], h);
    l = mfma_i8(qa[kc][0], kb[kc][0], l);
  }
  // Lane (gq, r) holds heads 4 gq .. +3 of block column r; ks of that block
  // sits in every lane of column r.  Group g continues the sum of group g - 1.
  const double ksd = (double)ks;
  double acc = 0.0;
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    double run = 0.0;
    if (g > 0) run = __shfl(acc, (lane + 48) & 63, 64);  // the same column, group g - 1
    if (gq == g) {
#pragma clang fp contract(off)
      acc = run;
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const double D = fma((double)h[i4], 16384.0, (double)l[i4]);
        const double y = ksd * D;
        const double rr = y > 0.0 ? y : 0.0;
        acc = acc + wh[i4] * rr;
      }
    }
  }
  return acc;
}

// Scores of blocks 0 .. local into sc[sc_slot(j)], by kWaves waves: 16-block
// column tiles, tile t on wave t % kWaves.  tab[0 .. local] holds the
// sequence's block-table row, lut the digit table and wsq the head weights
// (all visible to the calling waves).  HP (4, 8 or 16) >= HI rows per tile.
template <int DI, int HP, int kWaves>
__device__ __forceinline__ void score_tiles_i8(const KvView& kv, const i32x4 (&qa)[DI / 64][3],
                                               int wave, int lane, int local, const uint32_t* lut,
                                               const int* tab, const double* wsq, float* sc) {
  constexpr int KC = DI / 64;
  constexpr int kGroups = HP / 4;
  const int gq = lane >> 4, r = lane & 15;
  const int ntiles = local / 16 + 1;
  double wh[4];
#pragma unroll
  for (int i4 = 0; i4 < 4; ++i4) wh[i4] = wsq[(4 * gq + i4) & 15];
  // Key rows of a wave's tiles come in groups of kPre tiles, the next group
  // requested while the current one is on the matrix cores.
  constexpr int kPre = 4;
  const int nt_w = ntiles > wave ? (ntiles - wave + kWaves - 1) / kWaves : 0;
  auto fetch = [&](int i, uint4 (&kw)[KC], float& ks) {
    const int j = 16 * (wave + kWaves * i) + r;
    if (i < nt_w && j <= local) {
      const int p = tab[j];
      const uint4* krow = reinterpret_cast<const uint4*>(kv.idx_keys + (size_t)p * DI + 16 * gq);
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) kw[kc] = krow[4 * kc];
      ks = kv.idx_scale[p];
    } else {
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) kw[kc] = make_uint4(0u, 0u, 0u, 0u);
      ks = 0.f;
    }
  };
  auto score_tile = [&](int i, const uint4 (&kw)[KC], float ks) {
    const int j = 16 * (wave + kWaves * i) + r;
    const double acc = tile_score_i8<DI, HP>(qa, kw, ks, lut, wh, lane);
    if (gq == kGroups - 1 && i < nt_w && j <= local) sc[sc_slot(j)] = (float)acc;
  };
  uint4 kwA[kPre][KC], kwB[kPre][KC];
  float ksA[kPre], ksB[kPre];
#pragma unroll
  for (int u = 0; u < kPre; ++u) fetch(u, kwA[u], ksA[u]);
  for (int i0 = 0; i0 < nt_w; i0 += 2 * kPre) {
#pragma unroll
    for (int u = 0; u < kPre; ++u) fetch(i0 + kPre + u, kwB[u], ksB[u]);
#pragma unroll
    for (int u = 0; u < kPre; ++u) score_tile(i0 + u, kwA[u], ksA[u]);
    if (i0 + kPre >= nt_w) break;
#pragma unroll
    for (int u = 0; u < kPre; ++u) fetch(i0 + 2 * kPre + u, kwA[u], ksA[u]);
#pragma unroll
    for (int u = 0; u < kPre; ++u) score_tile(i0 + kPre + u, kwB[u], ksB[u]);
  }
}

// Exact scores of chunk `chunk` of query qi, logical blocks chunk 64 kT ..
// + 64 kT, by a workgroup of four waves on the int8 matrix cores, into
// sc[j - chunk 64 kT] (LDS, 64 kT floats; entries of blocks past the local
// block are not meaningful).  Wave w scores the 16-block tiles w, w + 4, ..,
// w + 4 (kT - 1) of the chunk; each lane reads the block-table entries of
// its kT columns itself (clamped into the row and the pool, so that reads of
// invisible blocks stay in bounds), before the query's position is known.
// lut (256 words) and wsq (16 doubles) are LDS scratch.  Returns false,
// uniformly, when the whole chunk lies past the local block (sc untouched);
// every thread must call it.
template <int DI, int HP, int kT = 4>
__device__ __forceinline__ bool score_chunk_i8(const KvView& kv, const QView& Q, int qi, int chunk,
                                               uint32_t* lut, double* wsq, float* sc, int& local) {
  constexpr int KC = DI / 64;
  constexpr int kGroups = HP / 4;
  constexpr int kChunkBlocks = 64 * kT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int gq = lane >> 4, r = lane & 15;
  const int s = query_seq(Q, qi);
  QueryRows<DI> qr;
  qr.fetch(Q, qi, lane);
  const int len = kv.seq_lens[s];
  const int pos = Q.q_pos ? Q.q_pos[qi] : len - 1;
  const int32_t* trow = kv.table + (size_t)s * kv.maxb;
  int p[kT];
#pragma unroll
  for (int i = 0; i < kT; ++i) {
    const int j = chunk * kChunkBlocks + 16 * (wave + 4 * i) + r;
    p[i] = min(max(trow[min(j, kv.maxb - 1)], 0), kv.num_blocks - 1);
  }
  uint4 kw[kT][KC];
  float ks[kT];
#pragma unroll
  for (int i = 0; i < kT; ++i) {
    const uint4* krow = reinterpret_cast<const uint4*>(kv.idx_keys + (size_t)p[i] * DI + 16 * gq);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) kw[i][kc] = krow[4 * kc];
    ks[i] = kv.idx_scale[p[i]];
  }
  for (int c = threadIdx.x; c < 256; c += blockDim.x) lut[c] = digits_of_code((uint32_t)c);
  __syncthreads();
  local = pos >> kv.bs_shift;
  if (chunk * kChunkBlocks > local) return false;
  i32x4 qa[KC][3];
  qr.build(lut, lane, wave == 0, wsq, qa);
  __syncthreads();
  double wh[4];
#pragma unroll
  for (int i4 = 0; i4 < 4; ++i4) wh[i4] = wsq[(4 * gq + i4) & 15];
#pragma unroll
  for (int i = 0; i < kT; ++i) {
    const double acc = tile_score_i8<DI, HP>(qa, kw[i], ks[i], lut, wh, lane);
    if (gq == kGroups - 1) sc[16 * (wave + 4 * i) + r] = (float)acc;
  }
  return true;
}

}  // namespace dsa

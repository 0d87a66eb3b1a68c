// Indexer scoring and Top-K selection of one query in one workgroup, for
// decode batches whose sequences have at most kFusedMaxBlocks blocks (short
// contexts: one CU scores all of a query's blocks faster than a separate
// scoring launch, a score round trip through memory and a selection launch;
// longer contexts spread the scoring over many workgroups instead).
//
// What is computed is exactly what index_score.hip followed by topk.hip
// compute ([P1] "Day-0 Adaptation for Massive LLMs...", section 4(1) "Index
// Selection"; [P5] "Day-0 Readiness for Trillion-Parameter Models...",
// "Index Selection Path": a lightweight low-precision inner product per
// block, then the Top-K blocks with the local block always kept, ids in
// increasing order):
//   S[j] = sum_{h ascending} w[h] * max(0, (sq[h] * ks[p]) * D[h, j])  (float64,
//   stored as fp32), D exact; then the local block plus the K - 1 best other
//   visible blocks, equal scores going to the lower id.
// The scores never leave LDS.  D is formed on the int8 matrix cores from
// base-128 digit planes (digit_mfma.h): rows of the MFMA tiles are the
// query's indexer heads, columns 16 blocks, k the key dims; the five int32
// digit sums are combined by Horner's rule and the epilogue follows the
// oracle's float64 order, head by head.
#include <hip/hip_runtime.h>
#include <math.h>

#include "digit_mfma.h"
#include "dsa_internal.h"
#include "select_common.h"

namespace dsa {
namespace {

constexpr int kFusedWaves = 8;
constexpr int kFusedMaxBlocks = 256;  // visible blocks per query held in LDS
constexpr int kSelM = kFusedMaxBlocks / 64;

// LDS slot of block j's score: XOR-swizzled within each group of 32, so
// the selection's reads of 32 consecutive scores per lane hit distinct banks.
__device__ __forceinline__ int sc_slot(int j) { return j ^ ((j >> 5) & 31); }

// One wave: the need best of candidates 0 .. n - 1 (scores in LDS), ties to
// the lower id, written to out[0 .. need) in increasing id order.
template <int M>
__device__ __forceinline__ void select_from_lds(const float* sc, int n, int need, uint4* hist4,
                                                int32_t* out) {
  const int lane = threadIdx.x & 63;
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
}

// grid (Nq), block 256.  HP (4, 8 or 16) >= HI rows per tile; rows >= HI
// are zero and weigh zero.
template <int DI, int HP>
__global__ __launch_bounds__(64 * kFusedWaves) void index_topk_i8(KvView kv, QView Q, int top_k,
                                                                  int32_t* __restrict__ out_idx,
                                                                  int32_t* __restrict__ out_cnt) {
  constexpr int KC = DI / 64;
  constexpr int kGroups = HP / 4;  // lane groups holding heads
  __shared__ uint32_t lut[256];
  __shared__ float sc[kFusedMaxBlocks];
  __shared__ int tab[kFusedMaxBlocks];  // the sequence's block-table row
  __shared__ double wsq[16];
  __shared__ uint4 hist4[64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gq = lane >> 4, r = lane & 15;
  const int qi = blockIdx.x;
  const int s = query_seq(Q, qi);
  const int hi = Q.hi;

  // query row r = indexer head r: dims 16 gq .. +16 of every 64-wide chunk
  uint4 raw[KC][2];
  const bool live_row = r < hi;
  {
    const uint4* src =
        reinterpret_cast<const uint4*>(Q.q_idx + ((size_t)qi * hi + (live_row ? r : 0)) * DI);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      raw[kc][0] = live_row ? src[8 * kc + 2 * gq] : make_uint4(0u, 0u, 0u, 0u);
      raw[kc][1] = live_row ? src[8 * kc + 2 * gq + 1] : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  const float wrow = live_row ? Q.w[(size_t)qi * hi + r] : 0.f;
  const int len = kv.seq_lens[s];
  const int pos = Q.q_pos ? Q.q_pos[qi] : len - 1;
  const int local = pos / kBlockSize;  // visible blocks: 0 .. local
  for (int c = tid; c < 256; c += 64 * kFusedWaves) lut[c] = digits_of_code((uint32_t)c);
  for (int j = tid; j <= local; j += 64 * kFusedWaves) tab[j] = kv.table[(size_t)s * kv.maxb + j];
  __syncthreads();

  // ---- query digits (A operand), quantized per head
  i32x4 qa[KC][3];
  {
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
    // w * 2^(e - 18): the power-of-two scales move only exponents, so
    // w (2^e (ks D)) and (w 2^(e-18)) (ks D 2^18) round alike.
    if (wave == 0 && gq == 0) wsq[r] = ldexp((double)wrow, ex - 18);
  }
  __syncthreads();

  // ---- scores of the visible blocks 0 .. local (16-block column tiles,
  // tile t on wave t % kFusedWaves), into LDS.  local < kFusedMaxBlocks (host check).
  const int ntiles = local / 16 + 1;
  double wh[4];
#pragma unroll
  for (int i4 = 0; i4 < 4; ++i4) wh[i4] = wsq[(4 * gq + i4) & 15];
  // Key rows of a wave's tiles come in groups of kPre tiles, the next group
  // requested while the current one is on the matrix cores.
  constexpr int kPre = 4;
  const int nt_w = ntiles > wave ? (ntiles - wave + kFusedWaves - 1) / kFusedWaves : 0;
  auto fetch = [&](int i, uint4 (&kw)[KC], float& ks) {
    const int j = 16 * (wave + kFusedWaves * i) + r;
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
    const int j = 16 * (wave + kFusedWaves * i) + r;
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
    // Lane (gq, r) holds heads 4 gq .. +3 of block j (column r); ks of block
    // j sits in every lane of column r.  The ascending head sum runs through
    // the lane groups in order: group g continues the sum of group g - 1.
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
  __syncthreads();

  // ---- Top-K on one wave, keys from LDS
  if (wave != 0) return;
  const int n = local;  // candidates 0 .. local - 1 (the local block is kept anyway)
  const int need = top_k - 1;
  int32_t* out = out_idx + (size_t)qi * top_k;
  if (n <= need) {
    for (int i = lane; i < top_k; i += 64) out[i] = i <= local ? i : -1;
    if (lane == 0) out_cnt[qi] = local + 1;
    return;
  }
  if (need == 0) {
    if (lane == 0) {
      out[0] = local;
      out_cnt[qi] = 1;
    }
    return;
  }
  if (n <= 64 * 2) {
    select_from_lds<2>(sc, n, need, hist4, out);
  } else {
    select_from_lds<kSelM>(sc, n, need, hist4, out);
  }
  if (lane == 0) {
    out[need] = local;
    out_cnt[qi] = top_k;
  }
}

template <int DI>
hipError_t launch_di(const KvView& kv, const QView& Q, int top_k, int32_t* idx, int32_t* cnt,
                     hipStream_t st) {
  const dim3 grid(Q.nq), block(64 * kFusedWaves);
  if (Q.hi <= 4) {
    hipLaunchKernelGGL((index_topk_i8<DI, 4>), grid, block, 0, st, kv, Q, top_k, idx, cnt);
  } else if (Q.hi <= 8) {
    hipLaunchKernelGGL((index_topk_i8<DI, 8>), grid, block, 0, st, kv, Q, top_k, idx, cnt);
  } else {
    hipLaunchKernelGGL((index_topk_i8<DI, 16>), grid, block, 0, st, kv, Q, top_k, idx, cnt);
  }
  return hipGetLastError();
}

}  // namespace

bool index_topk_fused_supported(const KvView& kv, const QView& Q) {
  // every query's blocks fit the LDS score array (short contexts); few enough
  // queries that the many-query scorer would not be chosen
  return kv.maxb <= kFusedMaxBlocks && Q.nq >= 1 && !index_score_mfma_supported(kv, Q) &&
         (kv.idx_dim == 64 || kv.idx_dim == 128) && Q.hi >= 1 && Q.hi <= 16;
}

hipError_t launch_index_topk_fused(const KvView& kv, const QView& Q, int top_k, int32_t* idx,
                                   int32_t* cnt, hipStream_t st) {
  return kv.idx_dim == 64 ? launch_di<64>(kv, Q, top_k, idx, cnt, st)
                          : launch_di<128>(kv, Q, top_k, idx, cnt, st);
}

}  // namespace dsa

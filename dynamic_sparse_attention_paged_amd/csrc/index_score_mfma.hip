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
#include "digit_mfma.h"

namespace dsa {
namespace {

constexpr int kMfmaWaves = 4;
constexpr int kRowTiles = 4;           // 16-row MFMA tiles per wave
constexpr int kMaxSpan = 2048;         // largest block range of one workgroup
constexpr int kWgSlots = 2 * 256;      // resident workgroups: two per CU

constexpr int kSuper = 64;  // blocks per super-tile (four 16-block MFMA column tiles)

// Byte offset of the 16-byte B operand of lane (g, c) for column tile ct,
// k chunk kc and digit plane pl within one staged super-tile: a wave's 64
// lanes read 1 KiB of consecutive LDS.
template <int KC>
__device__ __forceinline__ int kd_offset(int ct, int kc, int pl, int g, int c) {
  return ((((ct * KC + kc) * 3 + pl) * 4 + g) * 16 + c) * 16;
}

// grid (ceil(maxb / span), ceil(Nq / queries per workgroup)), block 256;
// span (a multiple of 64, at most kMaxSpan) is the workgroup's block range.
//
// Rows of the MFMA tiles: with T = HP / 4 tiles per group of four queries,
// row r of tile t is query 4 (t / T) + r / 4 of the wave, indexer head
// 4 (t % T) + r % 4.  Lane (g, c) of the result (g = lane / 16) then holds
// heads 4 (t % T) .. +3 of query 4 (t / T) + g for block c, so the ascending
// head sum of a (query, block) pair stays within one lane.
//
// Columns: the workgroup walks its block range in super-tiles of 64 blocks.
// All 256 threads fetch a super-tile's key rows (thread t: block t / 4, a
// quarter of the dims), turn them into digit planes and stage them in LDS
// (double-buffered; the next super-tile's keys are in flight while the
// current one is on the matrix cores).  Within a wave, column tile n's
// epilogue (float64, VALU) is interleaved with column tile n + 1's MFMAs.
template <int DI, int HP>
__global__ __launch_bounds__(64 * kMfmaWaves) __attribute__((amdgpu_waves_per_eu(2)))
void index_score_i8(KvView kv, QView Q, float* __restrict__ scores, int span) {
  constexpr int KC = DI / 64;          // 64-wide k chunks
  constexpr int T = HP / 4;            // tiles per group of four queries
  constexpr int kQPerWave = 4 * kRowTiles / T;
  constexpr int kQPerWg = kMfmaWaves * kQPerWave;
  constexpr int kGroups = kRowTiles / T;
  constexpr int kBufBytes = kSuper * DI * 3;
  __shared__ uint32_t lut[256];
  __shared__ double wsq[kQPerWg * HP];  // w * 2^(e - 18) per (query, head)
  __shared__ int seq_s[kQPerWg], loc_s[kQPerWg];
  __shared__ int tab[kMaxSpan];         // block-table slice of the current sequence
  __shared__ float ks_s[2][kSuper];
  __shared__ __attribute__((aligned(16))) uint8_t kd[2][kBufBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in a scalar register
  const int gq = lane >> 4, r = lane & 15;
  const int q_wg0 = blockIdx.y * kQPerWg;
  const int q_wave0 = q_wg0 + wave * kQPerWave;  // first query of this wave
  const int j_begin = blockIdx.x * span;
  const int j_end = min(kv.maxb, j_begin + span);

  // ---- all global reads of the query side first (one round trip):
  // lane (gq, r) holds row r of each tile, dims 16 gq .. +16 of every
  // 64-wide chunk.
  uint4 raw[kRowTiles][KC][2];
  float wrow[kRowTiles];
#pragma unroll
  for (int t = 0; t < kRowTiles; ++t) {
    const int q = q_wave0 + 4 * (t / T) + r / 4;
    const int h = 4 * (t % T) + r % 4;
    const bool live = q < Q.nq;
    const uint4* src = reinterpret_cast<const uint4*>(Q.q_idx + ((size_t)(live ? q : 0) * HP + h) * DI);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      raw[t][kc][0] = live ? src[8 * kc + 2 * gq] : make_uint4(0u, 0u, 0u, 0u);
      raw[t][kc][1] = live ? src[8 * kc + 2 * gq + 1] : make_uint4(0u, 0u, 0u, 0u);
    }
    wrow[t] = live ? Q.w[(size_t)q * HP + h] : 0.f;
  }
  for (int c = tid; c < 256; c += 64 * kMfmaWaves) lut[c] = digits_of_code((uint32_t)c);
  if (tid < kQPerWg) {
    const int q = q_wg0 + tid;
    int sq = -1, lq = -1;
    if (q < Q.nq) {
      sq = query_seq(Q, q);
      const int pos = Q.q_pos ? Q.q_pos[q] : kv.seq_lens[sq] - 1;
      lq = pos >> kv.bs_shift;
    }
    seq_s[tid] = sq;
    loc_s[tid] = lq;
  }
  __syncthreads();

  // ---- query digits (A operands), quantized per (query, head)
  i32x4 qa[kRowTiles][KC][3];
#pragma unroll
  for (int t = 0; t < kRowTiles; ++t) {
    const int qloc = 4 * (t / T) + r / 4;  // query within the wave
    const int h = 4 * (t % T) + r % 4;
    float x[KC][16];
    float amax = 0.f;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const uint32_t wv[8] = {raw[t][kc][0].x, raw[t][kc][0].y, raw[t][kc][0].z, raw[t][kc][0].w,
                              raw[t][kc][1].x, raw[t][kc][1].y, raw[t][kc][1].z, raw[t][kc][1].w};
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
    if (gq == 0) wsq[wave * kQPerWave * HP + qloc * HP + h] = ldexp((double)wrow[t], ex - 18);
  }
  const double* wsw = wsq + wave * kQPerWave * HP;

  // This lane's queries in the epilogue: 4 g + gq for group g = t / T.
  int my_loc[kGroups];
#pragma unroll
  for (int g = 0; g < kGroups; ++g) my_loc[g] = loc_s[wave * kQPerWave + 4 * g + gq];

  // Scores of this wave's queries go through a buffer resource: a store
  // whose offset lies past its range is dropped, so lanes with nothing to
  // write need no branch.
  const uint32_t wave_bytes = (uint32_t)(kQPerWave * kv.maxb) * 4u;
  const __amdgpu_buffer_rsrc_t out_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      scores + (size_t)min(q_wave0, Q.nq) * kv.maxb, 0, (int)wave_bytes, 0x00020000);

  // staging role: block sb of a super-tile, dims (DI / 4) sd .. +DI/4
  const int sb = tid >> 2, sd = tid & 3;

  // One pass per distinct sequence among the workgroup's queries (a prefill
  // chunk has one): the key tiles come from that sequence's table row.
  // Every thread evaluates the same loop bounds.
  uint64_t pending = 0u;
  for (int t = 0; t < kQPerWg; ++t) pending |= (seq_s[t] >= 0) ? (1ull << t) : 0ull;
  while (pending) {
    const int s_u = seq_s[__builtin_ctzll(pending)];
    uint64_t members = 0u;
    int lmax = -1;
    for (int t = 0; t < kQPerWg; ++t)
      if (seq_s[t] == s_u) {
        members |= 1ull << t;
        lmax = max(lmax, loc_s[t]);
      }
    pending &= ~members;
    const uint32_t wmembers = (uint32_t)(members >> (wave * kQPerWave));
    // blocks [j_begin, j_lim) are visible to some query of the pass
    const int j_lim = max(j_begin, min(j_end, lmax + 1));
    __syncthreads();  // previous pass done with tab, kd and ks_s
    for (int i = tid; i < j_lim - j_begin; i += 64 * kMfmaWaves)
      tab[i] = kv.table[(size_t)s_u * kv.maxb + j_begin + i];
    __syncthreads();

    const int nst = (j_lim - j_begin + kSuper - 1) / kSuper;
    uint4 kw[KC];
    float ksn = 0.f;
    auto fetch = [&](int st) {
      const int jl = st * kSuper + sb;  // block within the workgroup's range
      if (j_begin + jl < j_lim) {
        const int p = tab[jl];
        const uint4* src = reinterpret_cast<const uint4*>(kv.idx_keys + (size_t)p * DI + (DI / 4) * sd);
#pragma unroll
        for (int u = 0; u < KC; ++u) kw[u] = src[u];
        ksn = kv.idx_scale[p];
      } else {
#pragma unroll
        for (int u = 0; u < KC; ++u) kw[u] = make_uint4(0u, 0u, 0u, 0u);
        ksn = 0.f;
      }
    };
    auto stage = [&](int buf) {
#pragma unroll
      for (int u = 0; u < KC; ++u) {
        const int d0 = (DI / 4) * sd + 16 * u;
        i32x4 pl[3];
        planes_of(lut, kw[u], pl);
#pragma unroll
        for (int p3 = 0; p3 < 3; ++p3)
          *reinterpret_cast<i32x4*>(&kd[buf][kd_offset<KC>(sb >> 4, d0 >> 6, p3, (d0 >> 4) & 3,
                                                           sb & 15)]) = pl[p3];
      }
      if (sd == 0) ks_s[buf][sb] = ksn;
    };

    // Column tile n's digit sums are finished (scaled, summed over heads,
    // stored) while tile n + 1 is on the matrix cores.  The four tiles of a
    // super-tile alternate between two accumulator sets; a set's pending
    // tile starts at block jA / jB (-1: none).  Tiles past j_lim run on zero
    // keys and store nothing.
    i32x4 hiA[kRowTiles], loA[kRowTiles], hiB[kRowTiles], loB[kRowTiles];
    double ksA = 0.0, ksB = 0.0;
    int jA = -1, jB = -1;
    auto finish = [&](const i32x4 (&hiP)[kRowTiles], const i32x4 (&loP)[kRowTiles], double ksP,
                      int jP) {
      const int j = jP + r;
#pragma unroll
      for (int g = 0; g < kGroups; ++g) {
        const int qloc = 4 * g + gq;
        double S = 0.0;
        {
#pragma clang fp contract(off)
#pragma unroll
          for (int tt = 0; tt < T; ++tt) {
            const int t = g * T + tt;
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
              // D' = lo + 2^14 hi exactly (|D'| < 2^44)
              const double D = fma((double)hiP[t][i4], 16384.0, (double)loP[t][i4]);
              const double y = ksP * D;
              const double rr = y > 0.0 ? y : 0.0;
              S = S + wsw[qloc * HP + 4 * tt + i4] * rr;
            }
          }
        }
        const bool valid = (jP >= 0) & (((wmembers >> qloc) & 1u) != 0u) & (j < j_lim);
        const float val = (j <= my_loc[g]) ? (float)S : -INFINITY;
        const uint32_t off = valid ? (uint32_t)(qloc * kv.maxb + j) * 4u : 0x80000000u;
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, val), out_rsrc, off, 0, 0);
      }
    };
    // Digit sums of column tile ct of the staged super-tile by Horner's rule
    // in the accumulator:
    //   hi = G2 + 2^7 (G3 + 2^7 G4),   lo = G0 + 2^7 G1,
    // with G_c = sum_{i+j=c} <a_i, b_j>.  |G_c| < 2^23 for DI <= 128 and
    // |G4| < 2^15 (top digits are at most 15), so every partial value stays
    // below 2^31 in magnitude: exact in int32.
    auto digit_sums = [&](int buf, int ct, i32x4 (&hiC)[kRowTiles], i32x4 (&loC)[kRowTiles]) {
      i32x4 kb[KC][3];
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
#pragma unroll
        for (int pl = 0; pl < 3; ++pl)
          kb[kc][pl] = *reinterpret_cast<const i32x4*>(&kd[buf][kd_offset<KC>(ct, kc, pl, gq, r)]);
#pragma unroll
      for (int t = 0; t < kRowTiles; ++t) {
        i32x4 h = i32x4{0, 0, 0, 0}, l = i32x4{0, 0, 0, 0};
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) h = mfma_i8(qa[t][kc][2], kb[kc][2], h);
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) l = mfma_i8(qa[t][kc][0], kb[kc][1], l);
        h = h * 128;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          h = mfma_i8(qa[t][kc][1], kb[kc][2], h);
          h = mfma_i8(qa[t][kc][2], kb[kc][1], h);
          l = mfma_i8(qa[t][kc][1], kb[kc][0], l);
        }
        h = h * 128;
        l = l * 128;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          h = mfma_i8(qa[t][kc][0], kb[kc][2], h);
          h = mfma_i8(qa[t][kc][1], kb[kc][1], h);
          h = mfma_i8(qa[t][kc][2], kb[kc][0], h);
          l = mfma_i8(qa[t][kc][0], kb[kc][0], l);
        }
        hiC[t] = h;
        loC[t] = l;
      }
    };
    // issue order within a column tile: one MFMA, then two VALU instructions
    // (of the previous tile's epilogue)
    auto interleave = [&]() {
#pragma unroll
      for (int i = 0; i < 9 * KC * kRowTiles; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
      }
    };

    if (nst > 0) {
      fetch(0);
      stage(0);
    }
    __syncthreads();
    for (int st = 0; st < nst; ++st) {
      const int buf = st & 1;
      if (st + 1 < nst) fetch(st + 1);  // in flight during this super-tile's MFMAs
      const int j0 = j_begin + st * kSuper;
      finish(hiB, loB, ksB, jB);
      digit_sums(buf, 0, hiA, loA);
      interleave();
      ksA = (double)ks_s[buf][r];
      jA = j0;
      finish(hiA, loA, ksA, jA);
      digit_sums(buf, 1, hiB, loB);
      interleave();
      ksB = (double)ks_s[buf][16 + r];
      jB = j0 + 16;
      finish(hiB, loB, ksB, jB);
      digit_sums(buf, 2, hiA, loA);
      interleave();
      ksA = (double)ks_s[buf][32 + r];
      jA = j0 + 32;
      finish(hiA, loA, ksA, jA);
      digit_sums(buf, 3, hiB, loB);
      interleave();
      ksB = (double)ks_s[buf][48 + r];
      jB = j0 + 48;
      if (st + 1 < nst) stage(buf ^ 1);
      __syncthreads();
    }
    finish(hiB, loB, ksB, jB);  // last column tile of the pass
    // blocks past every query of the pass: -inf
    for (int j = j_lim + lane; j < j_end; j += 64) {
#pragma unroll
      for (int t = 0; t < kQPerWave; ++t)
        if ((wmembers >> t) & 1u) scores[(size_t)(q_wave0 + t) * kv.maxb + j] = -INFINITY;
    }
  }
}

template <int DI, int HP>
hipError_t launch_t(const KvView& kv, const QView& Q, float* scores, hipStream_t st) {
  constexpr int kQPerWg = kMfmaWaves * kRowTiles * (16 / HP);
  const int ny = (Q.nq + kQPerWg - 1) / kQPerWg;
  // Block range per workgroup: enough workgroups to fill the resident slots
  // once (two per CU), in whole super-tiles, at most kMaxSpan blocks.
  const int nx_want = (kWgSlots + ny - 1) / ny;
  int span = (kv.maxb + nx_want - 1) / nx_want;
  span = ((span + kSuper - 1) / kSuper) * kSuper;
  span = span < kSuper ? kSuper : (span > kMaxSpan ? kMaxSpan : span);
  const dim3 grid((kv.maxb + span - 1) / span, ny);
  hipLaunchKernelGGL((index_score_i8<DI, HP>), grid, dim3(64 * kMfmaWaves), 0, st, kv, Q, scores,
                     span);
  return hipGetLastError();
}

}  // namespace

bool index_score_mfma_supported(const KvView& kv, const QView& Q) {
  // many queries with explicit sequences and positions (a prefill chunk; the
  // kernel walks the blocks once per distinct sequence of a workgroup), 4 or
  // 8 indexer heads; a wave's score rows must fit one buffer resource (32-bit
  // byte range)
  return Q.q_seq != nullptr && Q.q_pos != nullptr && Q.nq >= 256 && (Q.hi == 4 || Q.hi == 8) &&
         (kv.idx_dim == 64 || kv.idx_dim == 128) && kv.maxb <= (1 << 24);
}

hipError_t launch_index_score_mfma(const KvView& kv, const QView& Q, float* scores,
                                   hipStream_t st) {
  if (Q.hi == 4) {
    return kv.idx_dim == 64 ? launch_t<64, 4>(kv, Q, scores, st) : launch_t<128, 4>(kv, Q, scores, st);
  }
  return kv.idx_dim == 64 ? launch_t<64, 8>(kv, Q, scores, st) : launch_t<128, 8>(kv, Q, scores, st);
}

}  // namespace dsa

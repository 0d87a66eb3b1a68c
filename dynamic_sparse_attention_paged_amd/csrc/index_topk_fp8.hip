// Indexer scoring and Top-K selection of many queries (a prefill chunk) in one
// launch, with the scores kept in LDS: approximate scores on the FP8 matrix
// cores, a bound on their error, and exact scores only for the few blocks
// that the bound cannot place on either side of the Top-K boundary.
//
// What is computed ([P1] "Day-0 Adaptation for Massive LLMs...", section 4(1)
// "Index Selection" and section 4(3): prefill scoring is compute-intensive
// and the inner product should not write intermediates to memory; [P3]
// "Day-0 Adaptation for Trillion-Parameter Models...", section 4.1: Top-K
// fused with the scoring before it; [P5] "Day-0 Readiness...", "Index
// Selection Path": low-precision scoring inputs) is exactly what
// index_score.hip followed by topk.hip compute: for query q at position pos
// and each visible block j < l = pos / block_size,
//   S[j] = sum_h w[h] max(0, (sq[h] ks[p]) D[h, j])  (float64, rounded to fp32),
//   D[h, j] = <q8[h, :], k8[p, :]> exact,  p = table[s][j],
// then the local block l plus the K - 1 best others (equal fp32 scores to the
// lower id), ids ascending.
//
// How.  One workgroup holds kQB = 8 queries.
//  1. Every (query, head) row of E4M3 codes q8 becomes FP8 MFMA operand rows.
//     A 16 x 16 x 128 tile of v_mfma_scale_f32_16x16x128_f8f6f4 (unit
//     scales) has rows (query 4 g + r / 4, head 4 t + r % 4) for row tile t of
//     query group g, so that lane (column c, group r / 4) receives heads
//     4 t .. 4 t + 3 of one query in every row tile of the group: the head sum
//     stays inside the lane.  Columns are 16 blocks, k the 128 key dims.
//  2. Approximate score  S^[j] = ks[p] sum_h a[h] max(0, D^[h, j]),  a[h] =
//     w[h] sq[h], into LDS.
//  3. Error bound.  The matrix unit's products of E4M3 values are exact; it
//     sums them in groups of eight, each group aligned to its largest product
//     and truncated toward zero 13 bits below that product's exponent, and
//     combines the group sums at fp32 precision or better (characterized with
//     dsa_probe_fp8_mfma: structured cases land exactly on this rule and 1.5
//     million random outputs never exceed it).  Each lane's 32 operand
//     bytes are four aligned runs of eight consecutive k, so every group is
//     eight consecutive key dims of one lane's codes.  For one instruction,
//     with e_g the exponent of group g's largest product and Mq[g] the
//     largest |q8| among the group's eight dims (max|k8| <= 448),
//       |D^ - D| <= sum_g 7 truncated products x 2^(e_g - 13)
//                   + 2^-13 max|q8| max|k8|
//               <= 448 2^-13 (7 sum_g Mq[g] + max|q8[h]|).
//     With fp32 epilogue rounding (2^-12 of 448 max|q8| per head) the
//     approximate score obeys
//       |S^[j] - S[j]| <= E = 448 ks_max 2^-13 sum_h |a[h]| (7 sum_g Mq[h, g] + 3 max|q8[h]|),
//     ks_max the largest key scale among the blocks the workgroup scores.
//     As sum_g Mq[g] <= 16 max|q8|, E never exceeds 448 ks_max (2^-6 +
//     2^-12) sum_h |a[h]| max|q8[h]| (the bound with every group at the
//     row's maximum); for N(0, 1) rows it is ~0.57 of that.
//  4. Selection.  T = the (K-1)-th largest S^ (wave radix select).  A block
//     with S^ > T + 2E (+ slack) beats every block that can beat it except at
//     most K - 2, so it is kept; one with S^ < T - 2E (- slack) is beaten by
//     at least K - 1 blocks, so it is dropped.  The slack keeps both sides at
//     least a few fp32 ulps apart, so rounding the scores to fp32 cannot turn
//     a strict order into a tie.  Only the blocks in between ("uncertain":
//     a handful per query at the chunked-prefill shape) are scored exactly,
//     on the int8 matrix cores from base-128 digit planes (digit_mfma.h,
//     bit-exact fp32 scores), and the remaining picks are made among them by
//     (exact score desc, id asc).  The result is therefore the exact
//     selection whatever the approximate scores were, as long as the bound
//     holds.
//  A workgroup whose queries belong to several sequences scores once per
//  sequence (the key columns follow that sequence's table row).
#include <float.h>
#include <hip/hip_runtime.h>
#include <math.h>

#include "dsa_internal.h"
#include "score_i8_lds.h"
#include "select_common.h"

namespace dsa {
namespace {

typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kQB = 8;            // queries per workgroup (two groups of four)
constexpr int kMaxBlocks = 2048;  // blocks per sequence: scores of kQB queries in LDS
constexpr int kPitch = kMaxBlocks + 16;  // rows 16 banks apart
constexpr int kListCap = 256;     // undecided blocks ranked from a list (more: every block rescored)
constexpr int kChunk = 2;         // column tiles per pipeline step
// the error bound's unit: 448 ks_max 2^-13 per unit of |a| (7 sum_g Mq + 3 max|q8|)
constexpr float kErrUnit = 448.f * 0.0001220703125f;

// max(x, 0) in one instruction (v_med3_f32) for finite x
__device__ __forceinline__ float relu(float x) { return __builtin_amdgcn_fmed3f(x, 0.f, FLT_MAX); }

__device__ __forceinline__ float key_float(uint32_t k) {
  const uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __builtin_bit_cast(float, u);
}

// Score rows in LDS are read lane-major (lane l: candidates 32 l .. 32 l + 31,
// eight 16 B reads).  Block j is stored at slot j with its 16 B quad index
// (bits 2-4) XORed with bits 5-7, so that the eight lanes of a 128 B group
// read eight different quads of the 32 banks at every step.
__device__ __forceinline__ int row_slot(int j) { return j ^ (((j >> 5) & 7) << 2); }

// v[m] = score of candidate 32 lane + m (slots as row_slot; row 16 B aligned)
__device__ __forceinline__ void read_row_lanes(const float* row, int lane, float (&v)[32]) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float4 x =
        *reinterpret_cast<const float4*>(row + 32 * lane + 4 * (k ^ (lane & 7)));
    v[4 * k] = x.x;
    v[4 * k + 1] = x.y;
    v[4 * k + 2] = x.z;
    v[4 * k + 3] = x.w;
  }
}

// E4M3 codes of one row's 32 values x[0 .. 32) scaled by 2^-e, four a word.
__device__ __forceinline__ void codes_of(const float (&x)[32], int e, int (&c)[8]) {
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    uint32_t v = 0u;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const float y = ldexpf(x[4 * w + b], -e);  // exact
      v |= ((uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y, 0.0f, 0, false) & 0xFFu) << (8 * b);
    }
    c[w] = (int)v;
  }
}

// Exact scores of blocks j by one wave, written to row[row_slot(j)]: j =
// list[e] for e in [0, n) (list != nullptr), or j = e (list == nullptr).  The int8 digit-plane products of score_i8_lds.h over 16-block tiles
// gathered from the list; the scores are the oracle's float64 values rounded
// to fp32.  When two queries' heads fit the 16 matrix rows (2 HP <= 16), rows
// HP .. 2 HP - 1 of qa hold a second query's heads (QueryRows::fetch_pair),
// whose scores of the same blocks go to row_b; a null row or row_b leaves
// that query's scores unstored.
template <int DI, int HP>
__device__ __forceinline__ void rescore_list(const KvView& kv, const i32x4 (&qa)[DI / 64][3], int lane,
                             const uint16_t* list, int n, const int32_t* trow,
                             const uint32_t* lut, const double* wsq, float* row, float* row_b) {
  constexpr int KC = DI / 64;
  constexpr int kGroups = HP / 4;                  // lane groups holding one query's heads
  constexpr int kAll = 2 * HP <= 16 ? 2 * kGroups : kGroups;
  const int gq = lane >> 4, r = lane & 15;
  double wh[4];
#pragma unroll
  for (int i4 = 0; i4 < 4; ++i4) wh[i4] = wsq[(4 * gq + i4) & 15];
  // eight 16-block tiles at a time (typically both lists of a query pair):
  // list entries, then table entries, then key rows, each level's loads all
  // in flight together
  constexpr int kTiles = 8;
  for (int t0 = 0; t0 < n; t0 += 16 * kTiles) {
    int j[kTiles], p[kTiles];
    // (columns past the list repeat its last entry: every load is in range
    // and unconditional, and their results are not stored)
#pragma unroll
    for (int u = 0; u < kTiles; ++u) {
      const int e = min(t0 + 16 * u + r, n - 1);
      j[u] = list ? (int)list[e] : e;
    }
#pragma unroll
    for (int u = 0; u < kTiles; ++u) p[u] = trow[j[u]];
    uint4 kw[kTiles][KC];
    float ks[kTiles];
#pragma unroll
    for (int u = 0; u < kTiles; ++u) {
      const uint4* krow = reinterpret_cast<const uint4*>(kv.idx_keys + (size_t)p[u] * DI + 16 * gq);
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) kw[u][kc] = krow[4 * kc];
      ks[u] = kv.idx_scale[p[u]];
    }
#pragma unroll
    for (int u = 0; u < kTiles; ++u) {
      if (t0 + 16 * u >= n) break;  // uniform
      i32x4 kb[KC][3];
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) planes_of(lut, kw[u][kc], kb[kc]);
      // hi = G2 + 2^7 (G3 + 2^7 G4), lo = G0 + 2^7 G1: exact in int32
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
      // the float64 epilogue in ascending head order, as the oracle evaluates it
      const double ksd = (double)ks[u];
      double acc = 0.0;
#pragma unroll
      for (int g = 0; g < kAll; ++g) {
        double run = 0.0;
        // the same column, group g - 1 (the second query's sum starts afresh)
        if (g > 0 && g != kGroups) run = __shfl(acc, (lane + 48) & 63, 64);
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
      const bool col = t0 + 16 * u + r < n;
      if (row != nullptr && gq == kGroups - 1 && col) row[row_slot(j[u])] = (float)acc;
      if (kAll > kGroups && row_b != nullptr && gq == kAll - 1 && col)
        row_b[row_slot(j[u])] = (float)acc;
    }
  }
}

// One query's selection state after its classification (per lane: the
// candidates 32 lane .. 32 lane + 31 as bits 0 .. 31 of each mask).
struct Sel {
  int q = -1;  // < 0: nothing left to do (no query, or its output is written)
  int n = 0, local = 0;
  uint32_t valid_m = 0u, in_m = 0u, unc_m = 0u;
  int n_unc = 0, r_need = 0, lbase = 0;  // undecided ids at list [lbase, lbase + n_unc)
  __device__ bool rescore() const { return q >= 0 && r_need < n_unc; }
  // too many undecided blocks for the list: every candidate scored exactly
  __device__ bool all_exact() const { return rescore() && n_unc > kListCap; }
};

// grid (ceil(Nq / kQB)), block 256.  HP (4, 8 or 16) >= HI heads a query.
template <int DI, int HP>
__global__ __launch_bounds__(kThreads, 2) void index_topk_fp8(KvView kv, QView Q, int top_k,
                                                              int32_t* __restrict__ out_idx,
                                                              int32_t* __restrict__ out_cnt) {
  constexpr int NT = HP / 4;         // row tiles per query group
  constexpr int NRT = (kQB / 4) * NT;  // row tiles per workgroup
  constexpr int KC = DI / 64;
  // score rows, then one slot per lane for the stores of columns that hold no
  // candidate (so that the epilogue needs no branch)
  __shared__ float sc[kQB * kPitch + kThreads];
  __shared__ uint16_t list_s[kWaves][2 * kListCap];  // a wave's two queries' lists
  __shared__ uint4 hist4[kWaves][64];  // radix histograms (wave_select)
  __shared__ uint32_t bins_s[kWaves][64];
  __shared__ uint32_t lut[256];
  __shared__ float a_s[kQB][16], am_s[kQB][16];
  __shared__ double wsq_s[kWaves][16];
  __shared__ float cq_s[kQB], ksmax_s[kWaves];
  __shared__ int seq_s[kQB], n_s[kQB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, kg = lane >> 4;
  const int q0 = blockIdx.x * kQB;

  if (tid < kQB) {
    const int q = q0 + tid;
    int s = -1, n = -1;
    if (q < Q.nq) {
      s = query_seq(Q, q);
      const int len = kv.seq_lens[s];
      const int pos = Q.q_pos ? Q.q_pos[q] : len - 1;
      n = pos >> kv.bs_shift;  // the local block; candidates 0 .. n - 1
    }
    seq_s[tid] = s;
    n_s[tid] = n;
  }
  for (int c = tid; c < 256; c += kThreads) lut[c] = digits_of_code((uint32_t)c);

  // ---- 1. query rows as FP8 operands: wave w quantizes row tiles w, w + 4,
  // .. and stages them in LDS (the start of the score rows, which the main
  // loop writes only after every wave has its operands)
  i32x8* a_stage = reinterpret_cast<i32x8*>(sc);  // [NRT][64 lanes]
  static_assert(NRT * 64 * 32 <= kQB * kPitch * 4, "operand staging fits the score rows");
  for (int rt = wave; rt < NRT; rt += kWaves) {
    const int g4 = rt / NT, t = rt % NT;
    const int ql = 4 * g4 + (r >> 2), h = 4 * t + (r & 3);
    const int q = q0 + ql;
    const bool live = q < Q.nq && h < Q.hi;
    float x[32];
    uint4 raw[2][2];
    const uint4* src =
        reinterpret_cast<const uint4*>(Q.q_idx + ((size_t)(live ? q : 0) * Q.hi + (live ? h : 0)) * DI);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const bool ok = live && (hf * 64 < DI);
      raw[hf][0] = ok ? src[8 * hf + 2 * kg] : make_uint4(0u, 0u, 0u, 0u);
      raw[hf][1] = ok ? src[8 * hf + 2 * kg + 1] : make_uint4(0u, 0u, 0u, 0u);
    }
    float amax = 0.f, gmax[4] = {0.f, 0.f, 0.f, 0.f};  // gmax[m]: max |x[8 m .. 8 m + 8)|
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const uint32_t wv[8] = {raw[hf][0].x, raw[hf][0].y, raw[hf][0].z, raw[hf][0].w,
                              raw[hf][1].x, raw[hf][1].y, raw[hf][1].z, raw[hf][1].w};
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        x[16 * hf + e] = bf16f((uint16_t)(wv[e >> 1] >> (16 * (e & 1))));
        gmax[(16 * hf + e) >> 3] = fmaxf(gmax[(16 * hf + e) >> 3], fabsf(x[16 * hf + e]));
      }
    }
    amax = fmaxf(fmaxf(gmax[0], gmax[1]), fmaxf(gmax[2], gmax[3]));
    amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
    // sum of the row's 16 group maxima (each lane holds four groups)
    float gsum = (gmax[0] + gmax[1]) + (gmax[2] + gmax[3]);
    gsum += __shfl_xor(gsum, 16, 64);
    gsum += __shfl_xor(gsum, 32, 64);
    int ex = 0;
    if (amax != 0.f) {
      int E;
      const float f = frexpf(amax, &E);  // amax = f 2^E, f in [0.5, 1)
      ex = (f <= 0.875f) ? E - 9 : E - 8;  // the smallest e with amax <= 448 2^e
    }
    int c[8];
    codes_of(x, ex, c);
    a_stage[rt * 64 + lane] = i32x8{c[0], c[1], c[2], c[3], c[4], c[5], c[6], c[7]};
    if (kg == 0) {
      const float a = live ? ldexpf(Q.w[(size_t)q * Q.hi + h], ex) : 0.f;
      // A code's magnitude exceeds its value's by at most 2^-4 of it (normal
      // codes) or 2^-10 (subnormal ones): max |q8| <= 1.0625 amax 2^-e (amax
      // 2^-e > 224), and the 16 group maxima sum to at most
      // 1.0625 gsum 2^-e + 16 2^-10.
      const float mq = ldexpf(amax, -ex) * 1.0625f;
      const float gq = ldexpf(gsum, -ex) * 1.0625f + 0.015625f;
      a_s[ql][h] = a;
      am_s[ql][h] = fabsf(a) * (7.f * gq + 3.f * mq);
    }
  }
  __syncthreads();
  i32x8 A[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) A[rt] = a_stage[rt * 64 + lane];
  __syncthreads();
  if (tid < kQB) {
    float t = 0.f;
    for (int h = 0; h < HP; ++h) t += am_s[tid][h];
    cq_s[tid] = t * (kErrUnit * 1.0001f);
  }
  // epilogue weights of the lane's query in each group
  float aw[kQB / 4][HP];
#pragma unroll
  for (int g4 = 0; g4 < kQB / 4; ++g4)
#pragma unroll
    for (int h = 0; h < HP; ++h) aw[g4][h] = a_s[4 * g4 + kg][h];

  // ---- 2. approximate scores into LDS, one pass per sequence of the workgroup
  float ksmax = 0.f;
  uint32_t done = 0u;
  for (;;) {
    int sq_seq = -1, nmax = 0;
    uint32_t pass = 0u;
#pragma unroll
    for (int ql = 0; ql < kQB; ++ql) {
      const int s = seq_s[ql];
      if (s < 0 || ((done >> ql) & 1u)) continue;
      if (sq_seq < 0) sq_seq = s;
      if (s == sq_seq) {
        pass |= 1u << ql;
        nmax = max(nmax, n_s[ql]);
      }
    }
    if (sq_seq < 0) break;
    done |= pass;
    const int32_t* trow = kv.table + (size_t)sq_seq * kv.maxb;
    const int nct = (nmax + 15) >> 4;  // column tiles holding candidates
    const int nt_w = nct > wave ? (nct - wave + kWaves - 1) / kWaves : 0;
    if (nt_w == 0) continue;           // uniform over the wave (nmax >= 1 below)
    const int nch = (nt_w + kChunk - 1) / kChunk;
    const int jlast = nmax - 1;
    // Loads are unconditional: columns past the candidates (and the tiles a
    // pipeline step fetches beyond the last one) read the last candidate's
    // entry, and their results are discarded.  Straight-line loads let the
    // compiler wait for exactly the ones a step consumes.
    auto load_tab = [&](int ch, int (&tb)[kChunk]) {
#pragma unroll
      for (int u = 0; u < kChunk; ++u) {
        const int i = ch * kChunk + u;
        tb[u] = trow[min(16 * (wave + kWaves * i) + r, jlast)];
      }
    };
    auto load_keys = [&](const int (&tb)[kChunk], i32x8 (&B)[kChunk], float (&ks)[kChunk]) {
#pragma unroll
      for (int u = 0; u < kChunk; ++u) {
        const uint8_t* kr = kv.idx_keys + (size_t)tb[u] * DI;
        const uint4 lo = *reinterpret_cast<const uint4*>(kr + 16 * kg);
        const uint4 hi = DI == 128 ? *reinterpret_cast<const uint4*>(kr + 64 + 16 * kg)
                                   : make_uint4(0u, 0u, 0u, 0u);
        B[u] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                     (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        ks[u] = kv.idx_scale[tb[u]];
      }
    };
    auto mfmas = [&](const i32x8& B, f32x4 (&acc)[NRT]) {
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
        acc[rt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            A[rt], B, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
    };
    auto epilogue = [&](int i, float ks, const f32x4 (&acc)[NRT]) {
      const int j = 16 * (wave + kWaves * i) + r;
      const bool ok = i < nt_w && j < nmax;
      ksmax = fmaxf(ksmax, ok ? ks : 0.f);
#pragma unroll
      for (int g4 = 0; g4 < kQB / 4; ++g4) {
        float tsum = 0.f;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4)
            tsum = fmaf(aw[g4][4 * t + i4], relu(acc[g4 * NT + t][i4]), tsum);
        const int ql = 4 * g4 + kg;
        const bool st = ok && ((pass >> ql) & 1u);
        sc[st ? ql * kPitch + row_slot(j) : kQB * kPitch + tid] = ks * tsum;
      }
    };
    // the MFMAs of tile u + 1 are issued before the epilogue of tile u, so the
    // matrix cores run while the vector units finish the previous tile
    auto compute = [&](int ch, const i32x8 (&B)[kChunk], const float (&ks)[kChunk]) {
      f32x4 acc0[NRT], acc1[NRT];
      mfmas(B[0], acc0);
#pragma unroll
      for (int u = 0; u < kChunk; u += 2) {
        if (u + 1 < kChunk) mfmas(B[u + 1], acc1);
        epilogue(ch * kChunk + u, ks[u], acc0);
        if (u + 1 >= kChunk) break;
        if (u + 2 < kChunk) mfmas(B[u + 2], acc0);
        epilogue(ch * kChunk + u + 1, ks[u + 1], acc1);
      }
    };
    // Software pipeline, three stages: table entries three chunks ahead, key
    // rows two chunks ahead (four column tiles in flight: the key rows are
    // scattered and their latency is long; eight, with four-tile chunks, took
    // 224 registers a lane and measured slower).  Vector-memory loads complete in
    // order, so each step issues the table loads of chunk c + 3 before the
    // key loads of chunk c + 2 (whose table entries came a step earlier):
    // waiting for those entries then never waits for keys still in use.
    int tbA[kChunk], tbB[kChunk], tbC[kChunk];
    i32x8 BA[kChunk], BB[kChunk], BC[kChunk];
    float ksA[kChunk], ksB[kChunk], ksC[kChunk];
    load_tab(0, tbA);
    load_tab(1, tbB);
    load_tab(2, tbC);
    load_keys(tbA, BA, ksA);
    load_keys(tbB, BB, ksB);
    for (int ch = 0; ch < nch; ch += 3) {
      load_tab(ch + 3, tbA);
      load_keys(tbC, BC, ksC);
      compute(ch, BA, ksA);
      if (ch + 1 >= nch) break;
      load_tab(ch + 4, tbB);
      load_keys(tbA, BA, ksA);
      compute(ch + 1, BB, ksB);
      if (ch + 2 >= nch) break;
      load_tab(ch + 5, tbC);
      load_keys(tbB, BB, ksB);
      compute(ch + 2, BC, ksC);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ksmax = fmaxf(ksmax, __shfl_xor(ksmax, off, 64));
  if (lane == 0) ksmax_s[wave] = ksmax;
  __syncthreads();
  float ksm = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) ksm = fmaxf(ksm, ksmax_s[w]);

  // ---- 3. selection.  Wave w selects queries ql = w and w + kWaves, each
  // classified on its own.  The exact rescoring of both runs as one pass when
  // their heads fit the 16 matrix rows together (2 HP <= 16) and they share a
  // table row; otherwise one list at a time.
  constexpr bool kPair = 2 * HP <= 16;
  const int need = top_k - 1;
  uint16_t* const lists = list_s[wave];
  auto lds_sync = [&]() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
    wave_lds_fence();
  };

  // Approximate-score classification of query ql: certainly in, undecided
  // (its ids, ascending, to lists[lbase ..]) or out.  Writes the output of the
  // cases that need no choice and returns q = -1 for them.
  auto classify = [&](int ql, int lbase) -> Sel {
    Sel S;
    S.lbase = lbase;
    const int q = q0 + ql;
    if (q >= Q.nq) return S;
    const int n = n_s[ql], local = n;
    int32_t* out = out_idx + (size_t)q * top_k;
    if (n <= need) {
      for (int i = lane; i < top_k; i += 64) out[i] = i <= local ? i : -1;
      if (lane == 0) out_cnt[q] = local + 1;
      return S;
    }
    if (need == 0) {
      if (lane == 0) {
        out[0] = local;
        out_cnt[q] = 1;
      }
      return S;
    }
    const float* row = sc + ql * kPitch;
    // lane l owns candidates 32 l .. 32 l + 31: decisions become per-lane bit
    // masks, and one wave prefix sum over their counts places each lane's
    // ids, which keeps every list ascending
    const int c0 = 32 * lane;
    const uint32_t valid_m =
        n - c0 >= 32 ? 0xFFFFFFFFu : (n - c0 <= 0 ? 0u : (1u << (n - c0)) - 1u);
    float v[32];
    read_row_lanes(row, lane, v);
    float mx = -INFINITY;
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      v[m] = ((valid_m >> m) & 1u) ? v[m] : -INFINITY;
      mx = fmaxf(mx, v[m]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    // bracket the need-th largest S^: a histogram of 64 bins of width delta
    // below the maximum (bin = floor((max - S^) / delta)); the bin b holding
    // rank `need` gives T_lo = max - (b + 1) delta and T_hi = max - b delta,
    // each widened by eps for the rounding of the bin arithmetic, so that
    // #{S^ >= T_lo} >= need and #{S^ > T_hi} <= need - 1.
    const float E = cq_s[ql] * ksm;  // |S^ - S| <= E for every candidate
    float delta = fmaxf(4.f * E, fmaxf(fabsf(mx) * 1.1920929e-07f, 1e-30f));
    int b_star = -1;
    float T_lo = 0.f, T_hi = 0.f;
    uint32_t above = 0u;  // candidates in the bins before b_star
    for (int tries = 0; tries < 40; ++tries) {  // delta x8 a try: ends once 64 bins hold rank need
      bins_s[wave][lane] = 0u;
      lds_sync();
      const float inv = 1.f / delta;
#pragma unroll
      for (int m = 0; m < 32; ++m) {
        const float b = (mx - v[m]) * inv;  // +inf for the padding
        if (b < 64.f) atomicAdd(&bins_s[wave][(int)b], 1u);
      }
      lds_sync();
      const uint32_t cum = wave_incl_scan(bins_s[wave][lane]);
      const unsigned long long hit = __ballot(cum >= (uint32_t)need);
      if (hit) {
        b_star = __builtin_ffsll((long long)hit) - 1;
        above = b_star > 0 ? (uint32_t)__shfl((int)cum, b_star - 1, 64) : 0u;
        break;
      }
      delta *= 8.f;
    }
    // the rank-need bin split once more into 64: the bracket narrows to
    // delta / 64 (bins of the same (max - S^) / delta, so membership agrees)
    float f_lo = 1.f, f_hi = 0.f;  // bracket = bins [b_star + f_hi, b_star + f_lo) of width delta
    if (b_star >= 0) {
      bins_s[wave][lane] = 0u;
      lds_sync();
      const float inv = 1.f / delta, bs = (float)b_star;
#pragma unroll
      for (int m = 0; m < 32; ++m) {
        const float b = (mx - v[m]) * inv;
        // b - bs is exact here (Sterbenz, or bs = 0), so the sub-bin is < 64
        if (b >= bs && b < bs + 1.f) atomicAdd(&bins_s[wave][(int)((b - bs) * 64.f)], 1u);
      }
      lds_sync();
      const uint32_t cum = above + wave_incl_scan(bins_s[wave][lane]);
      const int fb = __builtin_ffsll((long long)__ballot(cum >= (uint32_t)need)) - 1;
      f_hi = (float)fb * 0.015625f;
      f_lo = (float)(fb + 1) * 0.015625f;
      const float eps = (fabsf(mx) + 65.f * delta) * 9.5367431640625e-07f;  // 2^-20
      T_lo = mx - (bs + f_lo) * delta - eps;
      T_hi = mx - (bs + f_hi) * delta + eps;
    }
    // (b_star < 0 only if delta overflowed: then every candidate is undecided)
    const float slack = (fabsf(mx) + fabsf(T_lo) + 2.f * E) * 9.5367431640625e-07f + 1e-30f;
    const float hi_thr = b_star >= 0 ? T_hi + 2.f * E + slack : INFINITY;
    const float lo_thr = b_star >= 0 ? T_lo - 2.f * E - slack : -INFINITY;
    // certainly in: S^ > hi_thr; undecided: lo_thr <= S^ <= hi_thr
    uint32_t in_m = 0u, ge_m = 0u;
#pragma unroll
    for (int m = 0; m < 32; ++m) {
      in_m |= v[m] > hi_thr ? 1u << m : 0u;
      ge_m |= v[m] >= lo_thr ? 1u << m : 0u;
    }
    in_m &= valid_m;
    const uint32_t unc_m = ge_m & valid_m & ~in_m;
    // one scan for both counts: undecided in the low 16 bits, certainly-in above
    const uint32_t cu = (uint32_t)__builtin_popcount(unc_m);
    const uint32_t incl = wave_incl_scan(cu | ((uint32_t)__builtin_popcount(in_m) << 16));
    const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    const int n_in = (int)(tot >> 16), n_unc = (int)(tot & 0xFFFFu);
    // the undecided ids, ascending (a list longer than kListCap is not used:
    // its last slot may hold any id)
    int at = (int)(incl & 0xFFFFu) - (int)cu;
    for (uint32_t mm = unc_m; mm; mm &= mm - 1u, ++at)
      lists[lbase + min(at, kListCap - 1)] = (uint16_t)(c0 + __builtin_ctz(mm));
    S.q = q;
    S.n = n;
    S.local = local;
    S.valid_m = valid_m;
    S.in_m = in_m;
    S.unc_m = unc_m;
    S.n_unc = n_unc;
    S.r_need = need - n_in;
    return S;
  };

  // The kept candidates of a classified query (exact scores of its undecided
  // blocks already in its row), in ascending id, then the local block.
  auto finish = [&](const Sel& S, int ql) {
    int32_t* out = out_idx + (size_t)S.q * top_k;
    const float* row = sc + ql * kPitch;
    const int c0 = 32 * lane;
    if (S.all_exact()) {
      float x[32];
      read_row_lanes(row, lane, x);
      uint32_t k[32];
#pragma unroll
      for (int m = 0; m < 32; ++m) k[m] = ((S.valid_m >> m) & 1u) ? order_key(x[m]) : 0u;
      uint32_t T, take_eq, o;
      wave_select<32>(k, S.valid_m, (uint32_t)need, hist4[wave], T, take_eq);
      const uint32_t keep = wave_keep<32>(k, S.valid_m, T, take_eq, &o);
#pragma unroll
      for (int m = 0; m < 32; ++m)
        if ((keep >> m) & 1u) out[o++] = c0 + m;
    } else {
      uint32_t keep_m = S.in_m | S.unc_m;  // every undecided block needed (r_need >= n_unc)
      if (S.rescore()) {
        // the r_need best listed blocks by (exact score desc, id asc), marked
        // in a wave-private mask word per owning lane
        uint32_t* chosen = bins_s[wave];
        chosen[lane] = 0u;
        lds_sync();
        const uint16_t* list = lists + S.lbase;
        uint32_t k2[4], valid2 = 0u;
        int c2[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {  // lane l: list entries 4 l .. 4 l + 3 (ascending ids)
          const int e = 4 * lane + i;
          c2[i] = e < S.n_unc ? (int)list[e] : 0;
          k2[i] = e < S.n_unc ? order_key(row[row_slot(c2[i])]) : 0u;
          valid2 |= (e < S.n_unc) ? (1u << i) : 0u;
        }
        uint32_t T2, take2, o2;
        wave_select<4>(k2, valid2, (uint32_t)S.r_need, hist4[wave], T2, take2);
        const uint32_t keep2 = wave_keep<4>(k2, valid2, T2, take2, &o2);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if ((keep2 >> i) & 1u) atomicOr(&chosen[c2[i] >> 5], 1u << (c2[i] & 31));
        lds_sync();
        keep_m = S.in_m | (chosen[lane] & S.unc_m);
      }
      const uint32_t ck = (uint32_t)__builtin_popcount(keep_m);
      int o = (int)(wave_incl_scan(ck) - ck);
      for (uint32_t mm = keep_m; mm; mm &= mm - 1u) out[o++] = c0 + __builtin_ctz(mm);
    }
    if (lane == 0) {
      out[need] = S.local;  // the largest visible id: last in ascending order
      out_cnt[S.q] = top_k;
    }
  };

  if constexpr (kPair) {
    const int qla = wave, qlb = wave + kWaves;
    // both queries' rows for the exact rescoring, requested first so that
    // they arrive during the classification
    QueryRows<DI> qr;
    qr.fetch_pair(Q, q0 + qla < Q.nq ? q0 + qla : -1, q0 + qlb < Q.nq ? q0 + qlb : -1, HP, lane);
    const Sel A = classify(qla, 0);
    const bool la = A.rescore() && !A.all_exact();  // A rescored from its list
    const Sel B = classify(qlb, la ? A.n_unc : 0);  // B's list right after A's
    const bool lb = B.rescore() && !B.all_exact();
    if (A.rescore() || B.rescore()) {
      i32x4 qa[KC][3];
      qr.build(lut, lane, true, wsq_s[wave], qa);
      lds_sync();  // wsq and the lists written
      float* rowa = sc + qla * kPitch;
      float* rowb = sc + qlb * kPitch;
      const int32_t* trowa = kv.table + (size_t)seq_s[qla] * kv.maxb;
      const int32_t* trowb = kv.table + (size_t)seq_s[qlb] * kv.maxb;
      // one pass over both lists when the queries share a table row: each
      // query's exact scores of all listed blocks go to its own row (those of
      // the other query's blocks are never read)
      const bool joint = la && lb && seq_s[qla] == seq_s[qlb];
      // Up to four jobs through one call site: A's and B's candidates all
      // scored exactly (all_exact), A's list (or both lists), B's list.
      for (int jb = 0; jb < 4; ++jb) {
        const uint16_t* list = nullptr;
        int cnt = 0;
        const int32_t* trow = trowa;
        float* ra = nullptr;
        float* rb = nullptr;
        if (jb == 0 && A.all_exact()) {
          cnt = A.n;
          ra = rowa;
        } else if (jb == 1 && B.all_exact()) {
          cnt = B.n;
          trow = trowb;
          rb = rowb;
        } else if (jb == 2 && la) {
          list = lists + A.lbase;
          cnt = joint ? A.n_unc + B.n_unc : A.n_unc;
          ra = rowa;
          rb = joint ? rowb : nullptr;
        } else if (jb == 3 && lb && !joint) {
          list = lists + B.lbase;
          cnt = B.n_unc;
          trow = trowb;
          rb = rowb;
        }
        if (cnt > 0) rescore_list<DI, HP>(kv, qa, lane, list, cnt, trow, lut, wsq_s[wave], ra, rb);
      }
      lds_sync();
    }
    if (A.q >= 0) finish(A, qla);
    if (B.q >= 0) finish(B, qlb);
  } else {
    for (int ql = wave; ql < kQB; ql += kWaves) {
      if (q0 + ql >= Q.nq) break;
      QueryRows<DI> qr;
      qr.fetch(Q, q0 + ql, lane);
      const Sel S = classify(ql, 0);
      if (S.rescore()) {
        i32x4 qa[KC][3];
        qr.build(lut, lane, true, wsq_s[wave], qa);
        lds_sync();  // wsq and the list written
        // the listed blocks, or (all_exact) every candidate
        rescore_list<DI, HP>(kv, qa, lane, S.all_exact() ? nullptr : lists,
                             S.all_exact() ? S.n : S.n_unc,
                             kv.table + (size_t)seq_s[ql] * kv.maxb, lut, wsq_s[wave],
                             sc + ql * kPitch, nullptr);
        lds_sync();
      }
      if (S.q >= 0) finish(S, ql);
    }
  }
}

template <int DI>
hipError_t launch_di(const KvView& kv, const QView& Q, int top_k, int32_t* idx, int32_t* cnt,
                     hipStream_t st) {
  const dim3 grid((Q.nq + kQB - 1) / kQB), block(kThreads);
  if (Q.hi <= 4)
    hipLaunchKernelGGL((index_topk_fp8<DI, 4>), grid, block, 0, st, kv, Q, top_k, idx, cnt);
  else if (Q.hi <= 8)
    hipLaunchKernelGGL((index_topk_fp8<DI, 8>), grid, block, 0, st, kv, Q, top_k, idx, cnt);
  else
    hipLaunchKernelGGL((index_topk_fp8<DI, 16>), grid, block, 0, st, kv, Q, top_k, idx, cnt);
  return hipGetLastError();
}

}  // namespace

bool index_topk_fp8_supported(const KvView& kv, const QView& Q) {
  // many queries (a prefill chunk): a workgroup per 8 queries, every
  // sequence's scores in LDS
  return Q.nq >= 256 && kv.maxb <= kMaxBlocks && (kv.idx_dim == 64 || kv.idx_dim == 128) &&
         Q.hi >= 1 && Q.hi <= 16;
}

hipError_t launch_index_topk_fp8(const KvView& kv, const QView& Q, int top_k, int32_t* idx,
                                 int32_t* cnt, hipStream_t st) {
  return kv.idx_dim == 64 ? launch_di<64>(kv, Q, top_k, idx, cnt, st)
                          : launch_di<128>(kv, Q, top_k, idx, cnt, st);
}

}  // namespace dsa

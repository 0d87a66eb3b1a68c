// Sparse attention over the gathered K/V of the selected blocks.
//
// What is computed ([P1] "Day-0 Adaptation for Massive LLMs...", section
// 4(3): gather the selected blocks, then sparse attention; [P4] "Day-0
// Adaptation for Large Language Models...", full-vs-sparse table: only the
// index-selected pairs, otherwise the full-attention formula; [P5] "KV Cache
// Layout": whole blocks read through the block table): for query head h with
// KV head g = h / G (G = Hq / Hkv), over the tokens t of the selected blocks
// with position j*block_size + t <= pos and < seq_len,
//   x_t = scale <q_h, K_t>,  out_h = sum_t e^(x_t - m) V_t / sum_t e^(x_t - m),
//   lse_h = m + ln sum_t e^(x_t - m).
//
// Decode is HBM-bound: one (query, KV head, split) per workgroup, four waves,
// each wave streaming 64-token tiles of head g (K and V rows of 256 B at a
// 2 KiB stride; a block of 128, 256 or 512 tokens is 2, 4 or 8 consecutive
// tiles).  Per tile and wave, with the G query heads of g as the 16 MFMA
// columns:
//   S^T[64 tok x 16 heads] = K[64 x 128] . Q^T        16 x mfma 16x16x32 bf16
//   online softmax per head (lane's head = lane % 16 in every tile)
//   O^T[128 x 16] += V^T[128 x 64] . P^T[64 x 16]       32 x mfma (P = hi + lo bf16)
// K is an MFMA operand straight from global memory (8 consecutive dims per
// lane).  V must be read with 8 tokens per lane, so it is staged in LDS.
// P is split into a bf16 high part and a bf16 residual, which keeps the
// softmax weights at ~16 significant bits through the bf16 MFMA.
// The four waves' states, then (if split) the workgroups' states, are merged
// with the usual max / rescale rule; logits are kept in base 2.
#include <hip/hip_runtime.h>
#include <math.h>

#include <atomic>

#include "attn_tile.h"
#include "cand_common.h"
#include "dsa_internal.h"
#include "score_common.h"
#include "score_i8_lds.h"
#include "select_common.h"

namespace dsa {
namespace {

#ifdef DSA_WAVE_CLOCKS
// Diagnostic build only (not part of the library's default build): every
// attention wave records its start and end on the constant-rate wall clock
// (100 MHz on MI355X; dsa_wave_clock_khz gives the rate) with the raw HW_ID
// and XCC_ID hardware registers, indexed by
// ((KV head * Nq + query) * splits + split) * waves + wave, for timelines of
// one launch.
constexpr long kClockWaves = 1 << 16;
__device__ unsigned long long g_wave_clock[kClockWaves][2];
__device__ unsigned int g_wave_where[kClockWaves][2];
#endif

// split partials: one record per (query, head, split): m, l, o[128], two
// floats of padding (16-byte records)
constexpr int kPartStride = kHeadDim + 4;
constexpr int kMaxSelectBlocks = 2048;  // selection inside attention: up to 2048 blocks
constexpr int kMaxScoredBlocks = 256;  // scoring inside attention: up to 256 blocks
// where the attention kernel gets its blocks from (see sparse_attn_split)
constexpr int kAttnGiven = 0, kAttnSelect = 1, kAttnScore = 2, kAttnCand = 3;

using namespace tile;

// grid (splits, Nq, Hkv), block 64 W.  splits > 1: partials [Nq][Hq][splits] records
// kVBufs = 2: each wave double-buffers V in LDS, and the next block's K and V
// are requested as soon as the current block's K has gone through the
// logits MFMAs, so they arrive while the softmax and P V run.
//
// kMode says where the selected blocks come from:
//   kAttnGiven  idx / cnt, as written by the Top-K kernels;
//   kAttnSelect chosen here from the query's scores (one wave, into LDS; the
//               same rule as topk.hip), each workgroup of the query repeating
//               the cheap selection;
//   kAttnScore  scored here as well: the workgroup computes its query's exact
//               indexer scores into LDS on the int8 matrix cores (the same
//               values as index_score.hip, score_i8_lds.h), then selects as
//               above; the block-table row stays in LDS for the gather;
//   kAttnCand   chosen here from the per-workgroup candidate lists of a long
//               context (cand_common.h; `scores` points at the lists), merged
//               by all waves with the same rule.
// With kAttnSelect / kAttnScore, workgroup (0, q, 0) also writes the
// selection to idx_out / cnt_out when those are given.  DI and HP (index
// key length, indexer heads rounded up to 4, 8 or 16) matter for kAttnScore only.
//
// kNT: the K/V tiles are read with the non-temporal cache policy (decode: each
// selected block is streamed once per call); prefill keeps plain loads, since
// the blocks its queries select overlap and are served again from the caches.
//
// attn_unit is one workgroup's work, split sp of query qi and KV head g.
// kAttnGiven: the selection is given_sel[0 .. given_n).  kCohOut: the split
// partials are written with agent-coherent stores (another workgroup of the
// same launch merges them).
template <int kAttnWaves, int kVBufs, int kMode, int DI, int HP, bool kNT, bool kCohOut = false>
__device__ __forceinline__ void attn_unit(
    const KvView& kv, const QView& Q, const int32_t* given_sel, int given_n,
    const float* __restrict__ scores, int32_t* __restrict__ idx_out, int32_t* __restrict__ cnt_out,
    int top_k, float scale2, int splits, float* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ partials, const int sp, const int qi, const int g) {
  constexpr bool kSelects = kMode != kAttnGiven;
  constexpr bool kScores = kMode == kAttnScore;
  // V staging: vs_a, and with kVBufs = 2 vs_b, one 16 KiB block per wave each
  // (two arrays, so that the buffer being read and the one being filled are
  // distinct objects)
  __shared__ uint16_t vs_a[kAttnWaves][64 * kHeadDim];
  __shared__ uint16_t vs_b[kVBufs == 2 ? kAttnWaves : 1][kVBufs == 2 ? 64 * kHeadDim : 8];
  __shared__ float wm[kAttnWaves][16], wl[kAttnWaves][16];
  __shared__ float wf_s[kAttnWaves][16], hl_s[16];  // the waves' merge, per head
  __shared__ int32_t sel_lds[kSelects ? kMaxSelectBlocks : 1];
  __shared__ uint4 hist4[kSelects ? 64 : 1];
  __shared__ int tab[kScores ? kMaxScoredBlocks : 1];
  __shared__ int cnt_lds;

  uint16_t* const vbase = &vs_a[0][0];  // kAttnWaves x 64 x 128 bf16
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // scalar: uniform addresses
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, gq = lane >> 4;
  const int G = Q.hq / kv.num_kv_heads;
  const int s = query_seq(Q, qi);
  constexpr int kDI = DI > 0 ? DI : 64;
  constexpr int kHP = HP > 0 ? HP : 4;
  QueryRows<kDI> qr;
  if (kScores) qr.fetch(Q, qi, lane);  // first: the longest chain starts here
  const int len = kv.seq_lens[s];
  const int pos = Q.q_pos ? Q.q_pos[qi] : len - 1;
  int n_sel;
  const int32_t* sel;
  const int32_t* trow = kv.table + (size_t)s * kv.maxb;
  if (kScores) {
    // Scoring scratch (digit table, scores, head weights) lives in the V
    // staging area, which is free until the gather starts.
    uint32_t* lut = reinterpret_cast<uint32_t*>(vbase);
    float* sc = reinterpret_cast<float*>(lut + 256);
    double* wsq = reinterpret_cast<double*>(sc + kMaxScoredBlocks);
    const int local = pos >> kv.bs_shift;  // <= maxb - 1 < kMaxScoredBlocks (host check)
    for (int c = threadIdx.x; c < 256; c += 64 * kAttnWaves) lut[c] = digits_of_code((uint32_t)c);
    for (int j = threadIdx.x; j <= local; j += 64 * kAttnWaves) tab[j] = trow[j];
    __syncthreads();
    i32x4 qa[kDI / 64][3];
    qr.build(lut, lane, wave == 0, wsq, qa);
    __syncthreads();
    score_tiles_i8<kDI, kHP, kAttnWaves>(kv, qa, wave, lane, local, lut, tab, wsq, sc);
    __syncthreads();
    if (wave == 0) {
      const int c = local <= 64 * 2 ? select_lds_blocks<2>(sc, local, top_k, hist4, sel_lds)
                                    : select_lds_blocks<4>(sc, local, top_k, hist4, sel_lds);
      if (lane == 0) cnt_lds = c;
    }
    trow = tab;
  }
  if (kMode == kAttnSelect) {
    if (wave == 0) {
      const int local = pos >> kv.bs_shift;  // <= maxb - 1 < kMaxSelectBlocks
      const float* row = scores + (size_t)qi * kv.maxb;
      int c;
      if (local <= 64 * 2) {
        c = select_query_blocks<2>(row, kv.maxb, local, top_k, hist4, sel_lds);
      } else if (local <= 64 * 8) {
        c = select_query_blocks<8>(row, kv.maxb, local, top_k, hist4, sel_lds);
      } else {
        c = select_query_blocks<32>(row, kv.maxb, local, top_k, hist4, sel_lds);
      }
      if (lane == 0) cnt_lds = c;
    }
  }
  if (kMode == kAttnCand) {
    const int local = pos >> kv.bs_shift;
    const int need = top_k - 1;
    if (local <= need || need == 0) {  // uniform over the workgroup
      if (wave == 0) {
        const int c = need == 0 ? 1 : local + 1;
        for (int i = lane; i < top_k; i += 64)
          sel_lds[i] = need == 0 ? (i == 0 ? local : -1) : (i <= local ? i : -1);
        if (lane == 0) cnt_lds = c;
      }
    } else {
      // merge scratch in the V staging area, free until the gather starts
      uint32_t* ck = reinterpret_cast<uint32_t*>(vbase);
      int32_t* cj = reinterpret_cast<int32_t*>(ck + kMergeMaxCand);
      int* off = cj + kMergeMaxCand;
      uint32_t* k2 = reinterpret_cast<uint32_t*>(off + kMergeMaxCand + 4);
      int32_t* j2 = reinterpret_cast<int32_t*>(k2 + kMergeMaxCand);
      int32_t* cpos = j2 + kMergeMaxCand;
      int* n2 = cpos + kMergeMaxCand;
      uint4* h4 = reinterpret_cast<uint4*>(n2 + 16);
      int* rc = reinterpret_cast<int*>(h4 + kAttnWaves * 64);
      static_assert((6 * kMergeMaxCand + 4 + 16 + kCandScratchExtraWords) * 4 +
                            kAttnWaves * 64 * 16 <= kAttnWaves * 64 * kHeadDim * 2,
                    "merge scratch fits the V staging area");
      const CandScratch S{ck, cj, off, k2, j2, cpos, n2, h4, rc};
      const int nwg = (kv.maxb + kCandBlocks - 1) / kCandBlocks;
      const int c = merge_candidate_lists<kAttnWaves>(const_cast<float*>(scores), nwg, need, qi,
                                                      S, sel_lds);
      if (wave == 0) {  // c == need: the lists hold at least need candidates below local
        if (lane == 0) {
          sel_lds[c] = local;
          cnt_lds = c + 1;
        }
        for (int i = c + 1 + lane; i < top_k; i += 64) sel_lds[i] = -1;
      }
    }
  }
  if (kSelects) {
    __syncthreads();
    n_sel = cnt_lds;
    sel = sel_lds;
    if (sp == 0 && g == 0) {  // each output optional on its own
      if (idx_out)
        for (int i = threadIdx.x; i < top_k; i += 64 * kAttnWaves)
          idx_out[(size_t)qi * top_k + i] = sel_lds[i];
      if (cnt_out && threadIdx.x == 0) cnt_out[qi] = n_sel;
    }
  } else {
    n_sel = given_n;
    sel = given_sel;
  }
  // A block of 64 m tokens (m = 1, 2, 4, 8) is m tiles of 64 tokens; the
  // splits and the waves share tiles.  The last selected block (the query's
  // own block, in the Top-K kernels' ascending lists) contributes only its
  // tiles up to the query's last visible token, and at least one.
  const int lim = min(pos, len - 1);  // last attended token
  const int sub_shift = kv.bs_shift - 6;
  int n_items = n_sel << sub_shift;
  if (sub_shift > 0 && n_sel > 0) {
    const int vis = (lim >> 6) - (sel[n_sel - 1] << sub_shift) + 1;
    n_items -= (1 << sub_shift) - min(max(vis, 1), 1 << sub_shift);
  }
  const int per = ((top_k << sub_shift) + splits - 1) / splits;
  const int b0 = sp * per, b1 = min(n_items, b0 + per);

  // Q^T fragments (B operand): column = head r of group g, k = dims 32c + 8gq .. +8
  i16x8 qf[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if (r < G) {
      qf[c] = *reinterpret_cast<const i16x8*>(Q.q + ((size_t)qi * Q.hq + g * G + r) * kHeadDim +
                                             32 * c + 8 * gq);
    } else {
      qf[c] = i16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  WaveState st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) st.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint16_t* vs = vbase + wave * 64 * kHeadDim;
  const size_t tok_stride = kv_tok_stride(kv);
  const uint32_t v_off = dma_v_lane_offset(tok_stride, lane);
  const uint32_t k_off = (uint32_t)(((size_t)r * tok_stride + 8 * gq) * 2);

  // The wave's tiles are b0 + wave + W i.  Their logical tile ids (my_j) and
  // their tiles in the pool (my_p: physical block * m + tile within it) are
  // fetched up front, one per lane (64 at a time), so that the loop never
  // waits on a dependent table read before issuing tile loads.
  const int nmine = b1 > b0 + wave ? (b1 - b0 - wave + kAttnWaves - 1) / kAttnWaves : 0;
  for (int c0 = 0; c0 < nmine; c0 += 64) {
    const int cn = min(64, nmine - c0);
    int my_j = 0, my_p = 0;
    if (lane < cn) {
      const int item = b0 + wave + kAttnWaves * (c0 + lane);
      const int jb = sel[item >> sub_shift], h = item & ((1 << sub_shift) - 1);
      my_j = (jb << sub_shift) | h;
      my_p = (trow[jb] << sub_shift) | h;
    }
    if constexpr (kVBufs == 1) {
      for (int i = 0; i < cn; ++i) {
        const int j = __builtin_amdgcn_readlane(my_j, i);
        const int p = __builtin_amdgcn_readlane(my_p, i);
        const size_t base = kv_tile_base(kv, p, g);
        // previous block's LDS reads are complete before the DMA overwrites vs
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        __builtin_amdgcn_wave_barrier();
        dma_v<kNT>(kv.v + base, tok_stride, v_off, vs);
        i16x8 kf[4][4];
        load_k<kNT>(kv.k + base, tok_stride, k_off, kf);
        __builtin_amdgcn_s_waitcnt(0);  // V in LDS and K in registers
        __builtin_amdgcn_wave_barrier();
        attend_block(kf, qf, scale2, j * kBlockSize, lim, vs, st);
      }
    } else {
      // K two blocks ahead in registers (ka / kb), V one block ahead in LDS
      // (vs_a / vs_b).  Issue order: K_0, V_0, K_1, then per block t, after
      // its logits: V_{t+1}, K_{t+2}.  So at the top of every block but the
      // last, exactly K_{t+1}'s 16 loads were issued after V_t, and vmcnt(16)
      // means K_t and V_t have landed (vector memory counts complete in
      // order); the last block waits for everything.  The order of these
      // issues is pinned (compiler and scheduling barriers), and the waits are
      // explicit because the LDS written by global_load_lds is not a register
      // the compiler can track.  The step's V buffers are __restrict__: the
      // one being filled is never the one being read, which keeps the
      // compiler from draining every load before the P V reads.
      i16x8 ka[4][4], kb[4][4];
      auto base_of = [&](int t) {
        const int p = __builtin_amdgcn_readlane(my_p, t);
        return kv_tile_base(kv, p, g);
      };
      auto pin_order = [] {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
      };
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): earlier LDS reads of the buffers done
      __builtin_amdgcn_wave_barrier();
      auto prime = [&](uint16_t* __restrict__ v0) {
        const size_t b = base_of(0);
        load_k<kNT>(kv.k + b, tok_stride, k_off, ka);
        pin_order();
        dma_v<kNT>(kv.v + b, tok_stride, v_off, v0);
        pin_order();
        if (cn > 1) load_k<kNT>(kv.k + base_of(1), tok_stride, k_off, kb);
        pin_order();
      };
      // a block with a successor
      auto step = [&](int t, i16x8 (&kcur)[4][4], uint16_t* __restrict__ vcur,
                      uint16_t* __restrict__ vnext) {
        const int j = __builtin_amdgcn_readlane(my_j, t);
        __builtin_amdgcn_s_waitcnt(0x4070);  // vmcnt(16) lgkmcnt(0): K_t, V_t landed
        __builtin_amdgcn_wave_barrier();
        pin_order();
        f32x4 sc[4];
        block_logits(kcur, qf, sc);
        // vnext was last read by block t - 1's P V, finished at the wait above
        dma_v<kNT>(kv.v + base_of(t + 1), tok_stride, v_off, vnext);
        pin_order();
        if (t + 2 < cn) load_k<kNT>(kv.k + base_of(t + 2), tok_stride, k_off, kcur);
        pin_order();
        block_softmax_pv(sc, scale2, j * kBlockSize, lim, vcur, st);
      };
      auto last = [&](int t, i16x8 (&kcur)[4][4], uint16_t* vcur) {
        const int j = __builtin_amdgcn_readlane(my_j, t);
        __builtin_amdgcn_s_waitcnt(0);  // everything landed
        __builtin_amdgcn_wave_barrier();
        pin_order();
        f32x4 sc[4];
        block_logits(kcur, qf, sc);
        block_softmax_pv(sc, scale2, j * kBlockSize, lim, vcur, st);
      };
      prime(vs_a[wave]);
      int t = 0;
      for (; t + 2 < cn; t += 2) {
        step(t, ka, vs_a[wave], vs_b[wave]);
        step(t + 1, kb, vs_b[wave], vs_a[wave]);
      }
      if (t + 1 < cn) {  // two blocks left
        step(t, ka, vs_a[wave], vs_b[wave]);
        last(t + 1, kb, vs_b[wave]);
      } else {  // one block left
        last(t, ka, vs_a[wave]);
      }
    }
  }

  // ---- merge the four waves through LDS (reusing the V staging area)
  __syncthreads();
  float* wo = reinterpret_cast<float*>(vbase);  // [wave][16 heads][128]
  if (gq == 0) {
    wm[wave][r] = st.m;
    wl[wave][r] = st.l;
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) wo[(wave * 16 + r) * kHeadDim + 16 * dt + 4 * gq + i] = st.o[dt][i];
  __syncthreads();
  // per head: the waves' maximum, each wave's scale 2^(m_w - M) and the
  // scaled sum L, once (not per output element)
  if ((int)threadIdx.x < G) {
    const int h = threadIdx.x;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, wm[w][h]);
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
      // wave accumulators are unnormalised: sum_t 2^(x_t - m_w) V_t
      const float mw = wm[w][h];
      const float f = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
      wf_s[w][h] = f;
      L += f * wl[w][h];
    }
    hl_s[h] = L;
    const int hg = g * G + h;
    if (splits == 1) {
      if (lse) lse[(size_t)qi * Q.hq + hg] = (M + log2f(L)) * kLn2;
    } else {
      float* pp = partials + (((size_t)qi * Q.hq + hg) * splits + sp) * kPartStride;
      st_maybe_coh<kCohOut>(pp, M);
      st_maybe_coh<kCohOut>(pp + 1, L);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < G * kHeadDim; e += 64 * kAttnWaves) {
    const int h = e / kHeadDim, d = e % kHeadDim;
    float O = 0.f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) O += wf_s[w][h] * wo[(w * 16 + h) * kHeadDim + d];
    const float L = hl_s[h];
    const int hg = g * G + h;
    if (splits == 1) {
      out[((size_t)qi * Q.hq + hg) * kHeadDim + d] = O / L;
    } else {
      float* pp = partials + (((size_t)qi * Q.hq + hg) * splits + sp) * kPartStride;
      st_maybe_coh<kCohOut>(pp + 2 + d, (L > 0.f) ? O / L : 0.f);
    }
  }
}

__device__ __forceinline__ uint32_t add_agent(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// this wave's stores are complete, and no memory access moves across
__device__ __forceinline__ void stores_done() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// (m, l) pairs of a fused split merge held in LDS: G heads x splits
constexpr int kFusedMergeMaxGS = 512;

// done != nullptr (splits > 1, G splits <= kFusedMergeMaxGS): the split
// partials are merged in this launch, by the last of a (query, KV head)'s
// splits to finish: each split writes its partials with agent-coherent
// stores, waits for them to complete and adds one to the pair's counter (a
// 256-byte line of its own, zeroed before the launch); the one that brings
// it to splits reads the partials back with coherent loads and writes out /
// lse with the merge_splits rule, then zeroes the counter.  No workgroup
// waits for another.
template <int kAttnWaves, int kVBufs, int kMode, int DI, int HP, bool kNT>
__global__ __launch_bounds__(64 * kAttnWaves) void sparse_attn_split(
    KvView kv, QView Q, const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt,
    const float* __restrict__ scores, int32_t* __restrict__ idx_out, int32_t* __restrict__ cnt_out,
    int top_k, float scale2, int splits, float* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ partials, uint32_t* __restrict__ done) {
  const int qi = blockIdx.y, g = blockIdx.z;
  const int32_t* given_sel = kMode == kAttnGiven ? idx + (size_t)qi * top_k : nullptr;
  const int given_n = kMode == kAttnGiven ? cnt[qi] : 0;
  constexpr bool kFuse = kMode == kAttnCand;
#ifdef DSA_WAVE_CLOCKS
  const unsigned long long t_start = wall_clock64();
#endif
  attn_unit<kAttnWaves, kVBufs, kMode, DI, HP, kNT, kFuse>(kv, Q, given_sel, given_n, scores,
                                                           idx_out, cnt_out, top_k, scale2, splits,
                                                           out, lse, partials, blockIdx.x, qi, g);
#ifdef DSA_WAVE_CLOCKS
  {
    const unsigned long long t_end = wall_clock64();
    const long wid = (((long)blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x) *
                         kAttnWaves + (threadIdx.x >> 6);
    if ((threadIdx.x & 63) == 0 && wid < kClockWaves) {
      g_wave_clock[wid][0] = t_start;
      g_wave_clock[wid][1] = t_end;
      g_wave_where[wid][0] = __builtin_amdgcn_s_getreg((31 << 11) | 4);   // HW_ID, 32 bits
      g_wave_where[wid][1] = __builtin_amdgcn_s_getreg((15 << 11) | 20);  // XCC_ID, 16 bits
    }
  }
#endif
  if (!kFuse || done == nullptr || splits == 1) return;
  __shared__ float ml[2 * kFusedMergeMaxGS];
  __shared__ float wf[kFusedMergeMaxGS];
  __shared__ float hM[kFusedMergeMaxGS / 2], hL[kFusedMergeMaxGS / 2];  // per head (splits >= 2)
  __shared__ int last_s;
  const int tid = threadIdx.x;
  uint32_t* ctr = done + ((size_t)qi * kv.num_kv_heads + g) * kDoneLineWords;
  stores_done();
  __syncthreads();
  if (tid == 0) last_s = add_agent(ctr, 1u) == (uint32_t)(splits - 1);
  __syncthreads();
  if (!__builtin_amdgcn_readfirstlane(last_s)) return;
  const int G = Q.hq / kv.num_kv_heads;
  const float* grp = partials + ((size_t)qi * Q.hq + g * G) * splits * kPartStride;
  // kE output elements a thread, eight splits' o values at a time.  The
  // first group's o values are requested together with every (head,
  // split)'s m and l, so that a G <= 8, splits <= 8 merge waits for one
  // round trip to memory.
  constexpr int kE = 4, kT = 64 * kAttnWaves;
  static_assert(kFusedMergeMaxGS <= 2 * kT, "at most two (m, l) pairs a thread");
  const int GH = G * kHeadDim, GS = G * splits;
  auto load_o = [&](int e0, int i0, float (&o)[kE][8]) {
#pragma unroll
    for (int x = 0; x < kE; ++x) {
      const int e = min(e0 + x * kT, GH - 1);
      const float* po = grp + ((size_t)(e / kHeadDim) * splits) * kPartStride + 2 + e % kHeadDim;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        o[x][u] = i0 + u < splits ? ld_maybe_coh<true>(po + (size_t)(i0 + u) * kPartStride) : 0.f;
    }
  };
  float o[kE][8];
  {
    // (GS <= kFusedMergeMaxGS = 2 kT: at most two pairs a thread)
    float mv[2], lv[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int t = tid + k * kT;
      mv[k] = t < GS ? ld_maybe_coh<true>(grp + (size_t)t * kPartStride) : 0.f;
      lv[k] = t < GS ? ld_maybe_coh<true>(grp + (size_t)t * kPartStride + 1) : 0.f;
    }
    load_o(tid, 0, o);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int t = tid + k * kT;
      if (t < GS) {
        ml[2 * t] = mv[k];
        ml[2 * t + 1] = lv[k];
      }
    }
  }
  __syncthreads();
  if (tid == 0) st_maybe_coh<true>(ctr, 0u);
  // per (head, split): its weight l 2^(m - M) (M the head's maximum m), and
  // per head the sum L of its weights, in split order -- the merge_splits
  // rule, evaluated once per head instead of once per output element
  for (int t = tid; t < GS; t += kT) {
    const int h = t / splits, i = t - h * splits;
    const float* hm = ml + 2 * h * splits;
    float M = -INFINITY;
    for (int k = 0; k < splits; ++k) M = fmaxf(M, hm[2 * k]);
    const float m = hm[2 * i];
    wf[t] = (m == -INFINITY) ? 0.f : hm[2 * i + 1] * exp2f(m - M);
    if (i == 0) hM[h] = M;
  }
  __syncthreads();
  for (int h = tid; h < G; h += kT) {
    float L = 0.f;
    for (int i = 0; i < splits; ++i) L += wf[h * splits + i];
    hL[h] = L;
    if (lse) lse[(size_t)qi * Q.hq + g * G + h] = (hM[h] + log2f(L)) * kLn2;
  }
  __syncthreads();
  for (int e0 = tid; e0 < GH; e0 += kE * kT) {
    float O[kE];
#pragma unroll
    for (int x = 0; x < kE; ++x) O[x] = 0.f;
    for (int i0 = 0; i0 < splits; i0 += 8) {
      if (e0 != tid || i0 != 0) load_o(e0, i0, o);  // (the first group is loaded)
#pragma unroll
      for (int x = 0; x < kE; ++x) {
        const int e = min(e0 + x * kT, GH - 1);
        const float* hw = wf + (e / kHeadDim) * splits;
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (i0 + u < splits) O[x] += hw[i0 + u] * o[x][u];
      }
    }
#pragma unroll
    for (int x = 0; x < kE; ++x) {
      const int e = e0 + x * kT;
      if (e >= GH) break;
      const int h = e / kHeadDim, d = e % kHeadDim;
      out[((size_t)qi * Q.hq + g * G + h) * kHeadDim + d] = O[x] / hL[h];
    }
  }
}

// grid (Nq * Hq), block 128: merge the split partials of one (query, head).
__global__ __launch_bounds__(kHeadDim) void merge_splits(const float* __restrict__ partials,
                                                         int splits, float* __restrict__ out,
                                                         float* __restrict__ lse) {
  const int qh = blockIdx.x;
  const int d = threadIdx.x;
  const float* pp = partials + (size_t)qh * splits * kPartStride;
  float M = -INFINITY;
  for (int i = 0; i < splits; ++i) M = fmaxf(M, pp[i * kPartStride]);
  float L = 0.f, O = 0.f;
  for (int i = 0; i < splits; ++i) {
    const float* q = pp + i * kPartStride;
    const float f = (q[0] == -INFINITY) ? 0.f : q[1] * exp2f(q[0] - M);
    L += f;
    O += f * q[2 + d];
  }
  out[(size_t)qh * kHeadDim + d] = O / L;
  if (lse && d == 0) lse[qh] = (M + log2f(L)) * kLn2;
}

}  // namespace

int device_cu_count() {
  // queried once per device; a device that cannot be queried (no GPU) plans
  // for MI355X's 256 compute units
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
    n = 256;
  cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

AttnPlan attn_plan(int nq, int hkv, int tiles, bool prefill) {
  const int kNumCUs = device_cu_count();
  AttnPlan a;
  const long units = (long)nq * hkv;
  // Enough (query, KV head) pairs to give every CU a workgroup: no split.
  // Otherwise the selected tiles are split across workgroups until every
  // CU has one.
  // Four waves, each double-buffering V (eight single-buffered waves measured
  // no faster for batched decode and 13% slower for a chunked prefill of 8192
  // queries, whose gather is latency-bound).
  a.waves = 4;
  a.splits = 1;
  a.stream = !prefill;
  if (!prefill && tiles <= 8 && units < kNumCUs) {
    // at most eight 64-token tiles: one per wave of one eight-wave
    // workgroup, with no split partials and no merge launch
    a.waves = 8;
    return a;
  }
  if (!prefill && units > 0 && units < kNumCUs) {
    int splits = (int)((kNumCUs + units - 1) / units);
    const int max_splits = (tiles + a.waves - 1) / a.waves;  // >= one tile per wave
    a.splits = splits < max_splits ? splits : max_splits;
    if (a.splits < 1) a.splits = 1;
  }
  return a;
}

size_t attn_partials_bytes(int nq, int hq, int splits) {
  if (splits <= 1) return 0;
  return (size_t)nq * hq * splits * kPartStride * sizeof(float);
}

hipError_t launch_merge(const QView& Q, const float* partials, int splits, float* out, float* lse,
                        hipStream_t st) {
  hipLaunchKernelGGL(merge_splits, dim3(Q.nq * Q.hq), dim3(kHeadDim), 0, st, partials, splits, out,
                     lse);
  return hipGetLastError();
}

hipError_t launch_sparse_attn(const KvView& kv, const QView& Q, const int32_t* idx,
                              const int32_t* cnt, int top_k, float scale, float* out, float* lse,
                              float* partials, AttnPlan plan, hipStream_t st) {
  const float scale2 = scale * kLog2e;
  // KV head slowest: workgroups in flight together work on one head's blocks,
  // so the blocks that many queries select stay in the last-level cache.
  const dim3 grid(plan.splits, Q.nq, kv.num_kv_heads);
  if (plan.waves == 8) {
    hipLaunchKernelGGL((sparse_attn_split<8, 1, kAttnGiven, 0, 0, true>), grid, dim3(512), 0, st, kv,
                       Q, idx, cnt, nullptr, nullptr, nullptr, top_k, scale2, plan.splits, out, lse,
                       partials, nullptr);
  } else if (plan.stream) {
    hipLaunchKernelGGL((sparse_attn_split<4, 2, kAttnGiven, 0, 0, true>), grid, dim3(256), 0, st, kv,
                       Q, idx, cnt, nullptr, nullptr, nullptr, top_k, scale2, plan.splits, out, lse,
                       partials, nullptr);
  } else {
    hipLaunchKernelGGL((sparse_attn_split<4, 2, kAttnGiven, 0, 0, false>), grid, dim3(256), 0, st, kv,
                       Q, idx, cnt, nullptr, nullptr, nullptr, top_k, scale2, plan.splits, out, lse,
                       partials, nullptr);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.splits == 1) return e;
  return launch_merge(Q, partials, plan.splits, out, lse, st);
}

bool attn_select_supported(const KvView& kv, const QView& Q, int top_k, const AttnPlan& plan) {
  // The selection (top_k entries, -1 padded) and the candidates live in LDS.
  // Every workgroup of a query repeats the selection before its gather, which
  // pays only while the grid is one round of workgroups (measured, host
  // launches: 32 queries x 512 blocks, one round, 55.4 us a step against 58.6
  // us with a Top-K launch; 128 queries x up to 2048 blocks, four rounds,
  // 393.8 us against 379.7 us).
  const long wgs = (long)Q.nq * kv.num_kv_heads * plan.splits;
  return plan.waves == 4 && kv.maxb <= kMaxSelectBlocks && top_k <= kMaxSelectBlocks &&
         Q.nq >= 1 && wgs <= device_cu_count();
}

hipError_t launch_sparse_attn_select(const KvView& kv, const QView& Q, const float* scores,
                                     int top_k, float scale, float* out, float* lse,
                                     float* partials, AttnPlan plan, int32_t* idx_out,
                                     int32_t* cnt_out, hipStream_t st) {
  const float scale2 = scale * kLog2e;
  const dim3 grid(plan.splits, Q.nq, kv.num_kv_heads);
  hipLaunchKernelGGL((sparse_attn_split<4, 2, kAttnSelect, 0, 0, true>), grid, dim3(256), 0, st, kv, Q, nullptr,
                     nullptr, scores, idx_out, cnt_out, top_k, scale2, plan.splits, out, lse,
                     partials, nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.splits == 1) return e;
  return launch_merge(Q, partials, plan.splits, out, lse, st);
}

namespace {

template <int kWaves, int kVBufs, int DI>
hipError_t launch_scored_di(const KvView& kv, const QView& Q, int top_k, float scale2,
                            float* out, float* lse, float* partials, int splits,
                            int32_t* idx_out, int32_t* cnt_out, hipStream_t st) {
  const dim3 grid(splits, Q.nq, kv.num_kv_heads), block(64 * kWaves);
  if (Q.hi <= 4) {
    hipLaunchKernelGGL((sparse_attn_split<kWaves, kVBufs, kAttnScore, DI, 4, true>), grid, block, 0, st,
                       kv, Q, nullptr, nullptr, nullptr, idx_out, cnt_out, top_k, scale2, splits,
                       out, lse, partials, nullptr);
  } else if (Q.hi <= 8) {
    hipLaunchKernelGGL((sparse_attn_split<kWaves, kVBufs, kAttnScore, DI, 8, true>), grid, block, 0, st,
                       kv, Q, nullptr, nullptr, nullptr, idx_out, cnt_out, top_k, scale2, splits,
                       out, lse, partials, nullptr);
  } else {
    hipLaunchKernelGGL((sparse_attn_split<kWaves, kVBufs, kAttnScore, DI, 16, true>), grid, block, 0,
                       st, kv, Q, nullptr, nullptr, nullptr, idx_out, cnt_out, top_k, scale2,
                       splits, out, lse, partials, nullptr);
  }
  return hipGetLastError();
}

}  // namespace

bool attn_score_supported(const KvView& kv, const QView& Q, int top_k, const AttnPlan& plan) {
  // Every workgroup of a query repeats the query's scoring, so this pays only
  // while that work is small and the grid is a single round of workgroups
  // (measured: 32 queries x 64-256 blocks 3-4 us faster per step than a
  // separate scoring launch; 512 blocks, or four rounds of workgroups, slower).
  // The block-table row, the scores (in the V staging area) and the selection
  // live in LDS.
  const long wgs = (long)Q.nq * kv.num_kv_heads * plan.splits;
  return (plan.waves == 4 || plan.waves == 8) && kv.maxb <= kMaxScoredBlocks &&
         wgs <= device_cu_count() &&
         top_k <= kMaxSelectBlocks && (kv.idx_dim == 64 || kv.idx_dim == 128) && Q.hi >= 1 &&
         Q.hi <= 16 && Q.nq >= 1 && !index_score_mfma_supported(kv, Q);
}

hipError_t launch_sparse_attn_score(const KvView& kv, const QView& Q, int top_k, float scale,
                                    float* out, float* lse, float* partials, AttnPlan plan,
                                    int32_t* idx_out, int32_t* cnt_out, hipStream_t st) {
  const float scale2 = scale * kLog2e;
  hipError_t e;
  if (plan.waves == 8) {
    e = kv.idx_dim == 64
            ? launch_scored_di<8, 1, 64>(kv, Q, top_k, scale2, out, lse, partials, plan.splits,
                                         idx_out, cnt_out, st)
            : launch_scored_di<8, 1, 128>(kv, Q, top_k, scale2, out, lse, partials, plan.splits,
                                          idx_out, cnt_out, st);
  } else {
    e = kv.idx_dim == 64
            ? launch_scored_di<4, 2, 64>(kv, Q, top_k, scale2, out, lse, partials, plan.splits,
                                         idx_out, cnt_out, st)
            : launch_scored_di<4, 2, 128>(kv, Q, top_k, scale2, out, lse, partials, plan.splits,
                                          idx_out, cnt_out, st);
  }
  if (e != hipSuccess || plan.splits == 1) return e;
  return launch_merge(Q, partials, plan.splits, out, lse, st);
}

bool attn_cand_supported(const KvView& kv, const QView& Q, int top_k, const AttnPlan& plan) {
  // the merge scratch lives in the V staging area of the four-wave kernel and
  // the selection (top_k entries) in LDS
  return plan.waves == 4 && top_k <= kMaxSelectBlocks && index_cand_topk_supported(kv, Q, top_k);
}

size_t attn_done_bytes(int nq, int hkv) {
  return (size_t)nq * hkv * kDoneLineWords * sizeof(uint32_t);
}

bool attn_fused_merge(const QView& Q, int hkv, const AttnPlan& plan) {
  return plan.splits > 1 && (long)(Q.hq / hkv) * plan.splits <= kFusedMergeMaxGS;
}

hipError_t launch_sparse_attn_cand(const KvView& kv, const QView& Q, float* ws, int top_k,
                                   float scale, float* out, float* lse, float* partials,
                                   AttnPlan plan, int32_t* idx_out, int32_t* cnt_out,
                                   uint32_t* done, hipStream_t st) {
  const float scale2 = scale * kLog2e;
  const dim3 grid(plan.splits, Q.nq, kv.num_kv_heads);
  const bool fused = done != nullptr && attn_fused_merge(Q, kv.num_kv_heads, plan);
  hipLaunchKernelGGL((sparse_attn_split<4, 2, kAttnCand, 0, 0, true>), grid, dim3(256), 0, st, kv, Q,
                     nullptr, nullptr, ws, idx_out, cnt_out, top_k, scale2, plan.splits, out, lse,
                     partials, fused ? done : nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.splits == 1 || fused) return e;
  return launch_merge(Q, partials, plan.splits, out, lse, st);
}

}  // namespace dsa

#ifdef DSA_WAVE_CLOCKS
// Copies the first n waves' records of the last instrumented launch:
// clocks [n][2] (start, end), where [n][2] (HW_ID, XCC_ID).  0 on success.
extern "C" int dsa_wave_clocks_read(unsigned long long* clocks, unsigned int* where, int n) {
  if (!clocks || !where || n < 1 || n > dsa::kClockWaves) return -1;
  if (hipMemcpyFromSymbol(clocks, HIP_SYMBOL(dsa::g_wave_clock), sizeof(unsigned long long) * 2 * n,
                          0, hipMemcpyDeviceToHost) != hipSuccess)
    return -6;
  if (hipMemcpyFromSymbol(where, HIP_SYMBOL(dsa::g_wave_where), sizeof(unsigned int) * 2 * n, 0,
                          hipMemcpyDeviceToHost) != hipSuccess)
    return -6;
  return 0;
}

// The current device's wall-clock rate in kHz (the stamps' unit).  0 on success.
extern "C" int dsa_wave_clock_khz(int* khz) {
  int dev = 0;
  if (!khz) return -1;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
    return -6;
  return 0;
}
#endif

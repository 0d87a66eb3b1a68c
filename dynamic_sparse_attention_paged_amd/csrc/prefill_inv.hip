// Block-inverted prefill attention: each gathered 64-token tile of the pool is
// read once per KV head and attended by every query that selected it.
//
// [P1] "Day-0 Adaptation for Massive LLMs...", section 4(3): prefill is
// compute-intensive, and scoring, block selection and attention can be fused
// into one pipeline; [P3] "Day-0 Adaptation for Trillion-Parameter Models...",
// section 4.3: index selection fused with the attention inside blocks, to
// amortize the selection; [P5] "Day-0 Readiness...", "Differentiated
// Adaptation of Prefill and Decode": batch the prefill's sparse selection.
// Sharing each gathered block among the queries that chose it is how this
// kernel turns the prefill gather into matrix-core work.  The result is the
// same attention as the per-query kernel (attn.hip): for each query head,
// softmax over the tokens of its selected blocks up to its position.
//
// A prefill chunk's queries select their blocks independently, so one block is
// typically chosen by many queries of the chunk (8192 queries x 64 picks over a
// 2048-block context: ~256 each).  Here the selection is transposed into a
// CSR list "pool tile -> (query, pick)" (a count, a one-workgroup scan, a
// scatter), and one workgroup per (tile, KV head) keeps the tile's K in
// registers and V in LDS while its waves sweep the tile's queries, 16 / G
// queries per MFMA tile (G query heads per KV head).  Every (query, pick,
// head) leaves one partial softmax state {o[128], m, l} (base 2), and a merge
// kernel combines each query's partials in pick order, so the result does
// not depend on the order of the CSR entries.
#include <hip/hip_runtime.h>
#include <math.h>

#include "attn_tile.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

using namespace tile;

constexpr int kInvThreads = 256;  // four waves
constexpr int kScanThreads = 1024;

// The selected tiles of query q: blocks idx[q][0 .. cnt) as 2^sub tiles each,
// the last block only up to the query's last visible token (at least one).
struct QueryItems {
  int s, lim, n, sub;
};

__device__ __forceinline__ QueryItems query_items(const KvView& kv, const QView& Q,
                                                  const int32_t* __restrict__ idx,
                                                  const int32_t* __restrict__ cnt, int top_k,
                                                  int q) {
  QueryItems r;
  r.s = query_seq(Q, q);
  const int len = kv.seq_lens[r.s];
  const int pos = Q.q_pos ? Q.q_pos[q] : len - 1;
  r.lim = min(pos, len - 1);
  r.sub = kv.bs_shift - 6;
  const int c = cnt[q];
  r.n = c << r.sub;
  if (r.sub > 0 && c > 0) {
    const int vis = (r.lim >> 6) - (idx[(size_t)q * top_k + c - 1] << r.sub) + 1;
    r.n -= (1 << r.sub) - min(max(vis, 1), 1 << r.sub);
  }
  return r;
}

__global__ __launch_bounds__(kInvThreads) void inv_zero(int32_t* __restrict__ a, long n) {
  for (long i = (long)blockIdx.x * kInvThreads + threadIdx.x; i < n;
       i += (long)gridDim.x * kInvThreads)
    a[i] = 0;
}

// One thread per (query, item slot): count the entries of every pool tile
// (kScatter = false), or place each entry into its tile's list (true).
template <bool kScatter>
__global__ __launch_bounds__(kInvThreads) void inv_entries(
    KvView kv, QView Q, const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt,
    int top_k, int items_max, int32_t* __restrict__ count_or_cursor,
    int32_t* __restrict__ n_items, int4* __restrict__ entries) {
  const long total = (long)Q.nq * items_max;
  for (long t = (long)blockIdx.x * kInvThreads + threadIdx.x; t < total;
       t += (long)gridDim.x * kInvThreads) {
    const int q = (int)(t / items_max), it = (int)(t - (long)q * items_max);
    const QueryItems qi = query_items(kv, Q, idx, cnt, top_k, q);
    if (!kScatter && it == 0) n_items[q] = qi.n;
    if (it >= qi.n) continue;
    const int jb = idx[(size_t)q * top_k + (it >> qi.sub)];
    const int h = it & ((1 << qi.sub) - 1);
    const int p = kv.table[(size_t)qi.s * kv.maxb + jb];
    const int tile = (p << qi.sub) | h;
    if (kScatter) {
      const int at = atomicAdd(&count_or_cursor[tile], 1);
      entries[at] = make_int4(q, it, ((jb << qi.sub) | h) * kBlockSize, qi.lim);
    } else {
      atomicAdd(&count_or_cursor[tile], 1);
    }
  }
}

// Inclusive scan of (count, count != 0) over a wave.
__device__ __forceinline__ int2 wave_incl_scan(int2 v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int a = __shfl_up(v.x, d, 64), b = __shfl_up(v.y, d, 64);
    if (lane >= d) {
      v.x += a;
      v.y += b;
    }
  }
  return v;
}

// One workgroup: offset[t] = sum of count[< t] (offset[T] = total), cursor =
// offset, the non-empty tiles in ascending order in tiles[0 .. *n_tiles), and
// the sentinel entry.
__global__ __launch_bounds__(kScanThreads) void inv_scan(const int32_t* __restrict__ count,
                                                          int T, int32_t* __restrict__ offset,
                                                          int32_t* __restrict__ cursor,
                                                          int32_t* __restrict__ tiles,
                                                          int32_t* __restrict__ n_tiles,
                                                          int4* __restrict__ sentinel, int nq) {
  __shared__ int2 wsum[kScanThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (T + kScanThreads - 1) / kScanThreads;
  const int beg = min(T, tid * per), end = min(T, beg + per);
  int2 mine = make_int2(0, 0);
  for (int i = beg; i < end; ++i) {
    const int c = count[i];
    mine.x += c;
    mine.y += c != 0;
  }
  const int2 inc = wave_incl_scan(mine);
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int2 before = make_int2(0, 0);
  for (int w = 0; w < wave; ++w) {
    before.x += wsum[w].x;
    before.y += wsum[w].y;
  }
  int run = before.x + inc.x - mine.x, k = before.y + inc.y - mine.y;
  for (int i = beg; i < end; ++i) {
    const int c = count[i];
    offset[i] = run;
    cursor[i] = run;
    if (c) tiles[k++] = i;
    run += c;
  }
  if (tid == kScanThreads - 1) {
    offset[T] = run;
    *n_tiles = k;
    *sentinel = make_int4(nq, 0, 0, -1);  // the entry of columns without one
  }
}

// grid (tile slots, Hkv), block 256.  Workgroup (x, g): pool tile tiles[x],
// KV head g.  kQPT queries per MFMA tile: column r is query entry r / G and
// head r % G of group g (G = 16 / kQPT); kQPT = 1: column r < G is head r.
template <int kQPT>
__global__ __launch_bounds__(kInvThreads) void inv_attend(
    KvView kv, QView Q, const int32_t* __restrict__ tiles, const int32_t* __restrict__ n_tiles,
    const int32_t* __restrict__ offset, int4* entries, int sentinel,
    int items_max,
    float scale2, float* __restrict__ part_o, float2* __restrict__ part_ml) {
  __shared__ uint16_t vs[64 * kHeadDim];
  if ((int)blockIdx.x >= *n_tiles) return;  // the whole workgroup
  const int tile_id = tiles[blockIdx.x];
  const int g = blockIdx.y;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, gq = lane >> 4;
  const int G = Q.hq / kv.num_kv_heads;
  const int e0 = offset[tile_id], e1 = offset[tile_id + 1];
  const size_t tok_stride = kv_tok_stride(kv);
  const size_t base = kv_tile_base(kv, tile_id, g);

  // V: wave w brings token rows 16 w .. 16 w + 15 into LDS; K: every wave
  // holds the whole tile in registers for all of its query tiles.
  {
    const uint32_t v_off = dma_v_lane_offset(tok_stride, lane);
#pragma unroll
    for (int u = 4 * wave; u < 4 * wave + 4; ++u) {
      const char* rows = reinterpret_cast<const char*>(kv.v + base + (size_t)(4 * u) * tok_stride);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint16_t*>(rows + v_off),
                                       (lds_void_t*)(vs + 512 * u), 16, 0, 0);
    }
  }
  i16x8 kf[4][4];
  load_k(kv.k + base, tok_stride, (uint32_t)(((size_t)r * tok_stride + 8 * gq) * 2), kf);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  constexpr int kG = kQPT > 1 ? 16 / kQPT : 1;
  const int ce = kQPT > 1 ? r / kG : 0;       // entry of the column within the MFMA tile
  const int hl = kQPT > 1 ? r - ce * kG : r;  // head of the column within group g
  const bool col_ok = hl < G;
  // Software pipeline over MFMA tiles, unrolled by two with two register sets
  // (no copies between iterations): while a tile computes, the Q rows of the
  // next one and the entries of the one after are in flight.  The body has no
  // branches, so the compiler's waits stay partial: a column without an entry
  // reads the sentinel entry {query Nq, pick 0, lim -1} (every token masked),
  // whose partial rows lie in a trash region past the last query's, and its
  // Q row is read from query Nq - 1.  entries is not declared read-only: that
  // keeps the compiler from re-reading an entry (with a full wait) instead of
  // holding it in a register.
  auto entry_at = [&](int e) {
    const int my_e = e + ce;
    return entries[(col_ok && my_e < e1) ? my_e : sentinel];
  };
  // Columns past the group's heads (hl >= G, only with kQPT = 1 and G not a
  // power of two) read head G - 1 of the group: rows g * G .. g * G + G - 1
  // lie inside query qq's Hq heads, so no read leaves the caller's Q buffer.
  const int hl_q = min(hl, G - 1);
  auto load_q = [&](const int4& en, i16x8 (&qf)[4]) {
    const int qq = min(en.x, Q.nq - 1);
    const uint16_t* qp = Q.q + ((size_t)qq * Q.hq + g * G + hl_q) * kHeadDim + 8 * gq;
#pragma unroll
    for (int c = 0; c < 4; ++c) qf[c] = *reinterpret_cast<const i16x8*>(qp + 32 * c);
  };
  auto compute = [&](const int4& en, const i16x8 (&qf)[4]) {
    f32x4 sc[4];
    block_logits(kf, qf, sc);
    WaveState st;
    st.m = -INFINITY;
    st.l = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) st.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    block_softmax_pv(sc, scale2, en.z, en.w, vs, st);
    // partial rows [head][query][pick]: a query's picks of one head are
    // contiguous, and the workgroups running together (one KV head: the tile
    // index varies fastest in the grid) write into one head group's region
    const size_t row = ((size_t)(g * G + hl) * (Q.nq + 1) + en.x) * items_max + en.y;
    // (plain stores: the two 64 B halves of a row's 128 B line, written by
    // consecutive instructions, merge in L2; streaming stores measured 23%
    // more HBM write traffic)
    float* pr = part_o + row * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<f32x4*>(pr + 16 * dt + 4 * gq) = st.o[dt];
    part_ml[row] = make_float2(st.m, st.l);  // the column's four lanes hold the same values
  };
  // keeps the scheduler from sinking the prefetches down to their uses
  auto pin_order = [] {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  constexpr int kStep = 4 * kQPT;
  int e = e0 + wave * kQPT;
  if (e >= e1) return;
  // The first tile is peeled, so that the loop is entered with the same
  // loads and stores in flight as at its back edge.
  int4 enA = entry_at(e), enB = entry_at(e + kStep);
  i16x8 qfA[4], qfB[4];
  load_q(enA, qfA);
  load_q(enB, qfB);
  int4 enA2 = entry_at(e + 2 * kStep);
  pin_order();
  compute(enA, qfA);
  if (e + kStep >= e1) return;
  for (;;) {
    load_q(enA2, qfA);
    const int4 enB2 = entry_at(e + 3 * kStep);
    pin_order();
    compute(enB, qfB);
    e += 2 * kStep;
    if (e >= e1) break;
    load_q(enB2, qfB);
    const int4 enA3 = entry_at(e + 2 * kStep);
    pin_order();
    compute(enA2, qfA);
    if (e + kStep >= e1) break;
    enB = enB2;
    enA2 = enA3;
  }
}

// grid (Nq, Hq), one wave: combine query q's partials of head h in pick order.
// The picks' (m, l) are read one per lane; lane l then sums dims 2l, 2l + 1 of
// the o rows, o being unnormalized (sum of 2^(x - m) V):
//   O = sum_k 2^(m_k - M) o_k,  L = sum_k 2^(m_k - M) l_k,  out = O / L.
__global__ __launch_bounds__(64) void inv_merge(const float* __restrict__ part_o,
                                                const float2* __restrict__ part_ml,
                                                const int32_t* __restrict__ n_items,
                                                int items_max, int hq, float* __restrict__ out,
                                                float* __restrict__ lse) {
  const int q = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const int n = n_items[q];
  const size_t qh = (size_t)q * hq + h;
  const size_t hq_row = ((size_t)h * (gridDim.x + 1) + q) * items_max;  // [head][query (+ sentinel)][pick]
  const float* po = part_o + hq_row * kHeadDim + 2 * lane;
  const float2* pml = part_ml + hq_row;
  float M = -INFINITY;
  for (int c0 = 0; c0 < n; c0 += 64)
    if (c0 + lane < n) M = fmaxf(M, pml[c0 + lane].x);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  float Lp = 0.f;
  float2 O = make_float2(0.f, 0.f);
  for (int c0 = 0; c0 < n; c0 += 64) {
    float f = 0.f;
    if (c0 + lane < n) {
      const float2 ml = pml[c0 + lane];
      f = (ml.x == -INFINITY) ? 0.f : exp2f(ml.x - M);
      Lp += f * ml.y;
    }
    const int cn = min(64, n - c0);
    const float* rows = po + (size_t)c0 * kHeadDim;
    auto fj = [&](int j) {
      return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, f), j));
    };
    auto row = [&](int j) {
      return __builtin_nontemporal_load(reinterpret_cast<const f32x2*>(rows + (size_t)j * kHeadDim));
    };
    int j = 0;
    for (; j + 8 <= cn; j += 8) {  // eight rows in flight, summed in pick order
      f32x2 o[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) o[u] = row(j + u);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        O.x += fj(j + u) * o[u][0];
        O.y += fj(j + u) * o[u][1];
      }
    }
    for (; j < cn; ++j) {
      const f32x2 o = row(j);
      O.x += fj(j) * o[0];
      O.y += fj(j) * o[1];
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) Lp += __shfl_xor(Lp, off, 64);
  *reinterpret_cast<float2*>(out + qh * kHeadDim + 2 * lane) = make_float2(O.x / Lp, O.y / Lp);
  if (lse && lane == 0) lse[qh] = (M + log2f(Lp)) * kLn2;
}

template <int kQPT>
void launch_attend(const KvView& kv, const QView& Q, const InvLayout& L, char* ws, float scale2,
                   hipStream_t st) {
  const dim3 grid((unsigned)L.tile_slots, (unsigned)kv.num_kv_heads);
  hipLaunchKernelGGL(inv_attend<kQPT>, grid, dim3(kInvThreads), 0, st, kv, Q,
                     reinterpret_cast<const int32_t*>(ws + L.tiles),
                     reinterpret_cast<const int32_t*>(ws + L.n_tiles),
                     reinterpret_cast<const int32_t*>(ws + L.offset),
                     reinterpret_cast<int4*>(ws + L.entries), (int)L.entries_max,
                     L.items_max, scale2, reinterpret_cast<float*>(ws + L.part_o),
                     reinterpret_cast<float2*>(ws + L.part_ml));
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

// (query, pick) slots: nq * top_k * tiles per block <= 65535 * 4096 * 8 < 2^31,
// so entry indices (and the sentinel's, entries_max) fit in int.
InvLayout inv_layout(const KvView& kv, int nq, int hq, int top_k, size_t base) {
  InvLayout L;
  const int sub = kv.bs_shift - 6;
  L.items_max = top_k << sub;
  L.pool_tiles = (long)kv.num_blocks << sub;
  const long entries = (long)nq * L.items_max;
  L.entries_max = entries;
  L.tile_slots = L.pool_tiles < entries ? L.pool_tiles : entries;
  size_t at = align256(base);
  L.n_items = at;
  at = align256(at + (size_t)nq * 4);
  L.count = at;
  at = align256(at + (size_t)(L.pool_tiles + 1) * 4);
  L.offset = at;
  at = align256(at + (size_t)(L.pool_tiles + 1) * 4);
  L.cursor = at;
  at = align256(at + (size_t)L.pool_tiles * 4);
  L.tiles = at;
  at = align256(at + (size_t)L.pool_tiles * 4);
  L.n_tiles = at;
  at = align256(at + 4);
  // entries, then the sentinel entry
  L.entries = at;
  at = align256(at + (size_t)(entries + 1) * sizeof(int4));
  // partial rows [head][query][pick], each head with the sentinel query Nq
  // after its real ones, plus 16 heads' worth for columns past the last head
  const size_t rows = ((size_t)(hq + 16) * (nq + 1)) * L.items_max;
  L.part_o = at;
  at = align256(at + rows * kHeadDim * sizeof(float));
  L.part_ml = at;
  at = align256(at + rows * sizeof(float2));
  L.total = at;
  return L;
}

bool prefill_inv_supported(const KvView& kv, const QView& Q) {
  const int G = kv.num_kv_heads > 0 ? Q.hq / kv.num_kv_heads : 0;
  return G >= 1 && G <= kMaxGroup && Q.nq >= 1;
}

hipError_t launch_prefill_inv(const KvView& kv, const QView& Q, const int32_t* idx,
                              const int32_t* cnt, int top_k, float scale, float* out, float* lse,
                              char* ws, const InvLayout& L, hipStream_t st) {
  const float scale2 = scale * kLog2e;
  int32_t* n_items = reinterpret_cast<int32_t*>(ws + L.n_items);
  int32_t* count = reinterpret_cast<int32_t*>(ws + L.count);
  int32_t* cursor = reinterpret_cast<int32_t*>(ws + L.cursor);
  int4* entries = reinterpret_cast<int4*>(ws + L.entries);
  const long zn = L.pool_tiles;
  long zg = (zn + kInvThreads - 1) / kInvThreads;
  hipLaunchKernelGGL(inv_zero, dim3((unsigned)(zg > 4096 ? 4096 : zg)), dim3(kInvThreads), 0, st,
                     count, zn);
  const long total = (long)Q.nq * L.items_max;
  long eg = (total + kInvThreads - 1) / kInvThreads;
  const unsigned egu = (unsigned)(eg > 16384 ? 16384 : eg);
  hipLaunchKernelGGL(inv_entries<false>, dim3(egu), dim3(kInvThreads), 0, st, kv, Q, idx, cnt,
                     top_k, L.items_max, count, n_items, entries);
  hipLaunchKernelGGL(inv_scan, dim3(1), dim3(kScanThreads), 0, st, count, (int)L.pool_tiles,
                     reinterpret_cast<int32_t*>(ws + L.offset), cursor,
                     reinterpret_cast<int32_t*>(ws + L.tiles),
                     reinterpret_cast<int32_t*>(ws + L.n_tiles), entries + L.entries_max, Q.nq);
  hipLaunchKernelGGL(inv_entries<true>, dim3(egu), dim3(kInvThreads), 0, st, kv, Q, idx, cnt,
                     top_k, L.items_max, cursor, n_items, entries);
  const int G = Q.hq / kv.num_kv_heads;
  switch (G) {
    case 1: launch_attend<16>(kv, Q, L, ws, scale2, st); break;
    case 2: launch_attend<8>(kv, Q, L, ws, scale2, st); break;
    case 4: launch_attend<4>(kv, Q, L, ws, scale2, st); break;
    case 8: launch_attend<2>(kv, Q, L, ws, scale2, st); break;
    default: launch_attend<1>(kv, Q, L, ws, scale2, st); break;
  }
  hipLaunchKernelGGL(inv_merge, dim3(Q.nq, Q.hq), dim3(64), 0, st,
                     reinterpret_cast<const float*>(ws + L.part_o),
                     reinterpret_cast<const float2*>(ws + L.part_ml), n_items, L.items_max, Q.hq, out,
                     lse);
  return hipGetLastError();
}

}  // namespace dsa

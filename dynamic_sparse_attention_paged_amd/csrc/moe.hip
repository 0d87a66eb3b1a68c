// MXFP4 expert weights: the online MXFP4 -> FP8 conversion into a reused
// workspace, MXFP8 activations, and the grouped expert matmul.
//
// [P1] "Day-0 Adaptation for Massive LLMs...", section 5: expert weights are
// MXFP4 (4-bit elements in fixed blocks with a block-level scale); the routed
// experts' weights are unpacked to FP8 online into a shared workspace and the
// expert matmuls run in FP8 with the block scales, the unpacked layout being
// the matmul's input layout.  [P2] "Day-0 Adaptation for Trillion-Parameter
// LLMs...", sections 3.1-3.2: conversion in registers / shared memory,
// results fed straight to the matrix units, one global FP8 workspace reused
// across layers.  Formats: the OCP MX specification v1.0 (E2M1 elements, E8M0
// scales, blocks of 32).
//
// gfx950 runs the scaled matrix instruction v_mfma_scale_f32_16x16x128_f8f6f4,
// which applies one E8M0 scale per 32-element block of each operand in
// hardware and takes FP8 or FP4 operands.  So the matmul here consumes the
// block scales as they are, from either the FP8 workspace (the pages' path) or
// the MXFP4 weights directly (no workspace: a quarter of the weight bytes of
// unpacking and re-reading).  Operand layout of the 16x16x128 instruction, for
// lane (r, kg), r = lane % 16, kg = lane / 16, over a 128-wide K step:
//   FP8: K [16 kg, 16 kg + 16) and [64 + 16 kg, 64 + 16 kg + 16) (32 bytes);
//   FP4: K [32 kg, 32 kg + 32) (16 bytes, element 2i in the low nibble);
//   the lane's scale operand is the E8M0 scale of block kg, K [32 kg, 32 kg + 32);
//   D[4 kg + i][r] = element i of the lane's result (row: A row, column: B row).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <stdint.h>

#include <type_traits>

#include "dsa_internal.h"

namespace dsa {
namespace {

typedef __attribute__((ext_vector_type(8))) int v8i;
typedef __attribute__((ext_vector_type(4))) int v4i;
typedef __attribute__((ext_vector_type(4))) float v4f;

constexpr int kMoeThreads = 256;
constexpr int kMoeBMSmall = 64;   // pairs per row tile when experts get few pairs (decode)
constexpr int kMoeBMLarge = 128;  // ... and when they get many (prefill): fewer weight re-reads
// output columns per workgroup: four waves x 16 CT (CT column tiles per wave)
constexpr int kScanThreads = 1024;
constexpr int kMoeGroupTiles = 4;  // row tiles whose column blocks run together in the matmul

// E4M3 codes of the 16 E2M1 values (0, 0.5, 1, 1.5, 2, 3, 4, 6 and their
// negatives): E4M3 value (1 + M/8) 2^(E - 7), so 0.5 = E 6, 1 = E 7, 1.5 = E 7
// M 4, 2 = E 8, 3 = E 8 M 4, 4 = E 9, 6 = E 9 M 4; code 8 (-0) is 0x80.
// The magnitudes (codes 0-7) are a byte table held in two registers and
// indexed with v_perm_b32 (four elements per instruction); the sign (code bit
// 3) becomes E4M3 bit 7.
constexpr uint32_t kMagLo = 0x3C383000u;  // E4M3 of E2M1 magnitudes 0, 0.5, 1, 1.5
constexpr uint32_t kMagHi = 0x4C484440u;  // ... 2, 3, 4, 6

// E4M3 codes (one per byte) of the four E2M1 codes in bits 15-0 of x
__device__ __forceinline__ uint32_t e2m1x4_to_e4m3(uint32_t x) {
  const uint32_t spread = (x & 0xFu) | ((x & 0xF0u) << 4) | ((x & 0xF00u) << 8) | ((x & 0xF000u) << 12);
  const uint32_t mag = __builtin_amdgcn_perm(kMagHi, kMagLo, spread & 0x07070707u);
  return mag | ((spread & 0x08080808u) << 4);
}

// One thread per 32-element block of one activation row: MXFP8 with E4M3
// elements.  shared = floor(log2 max|x|) - 8 (clamped to [-127, 127]), scale
// code shared + 127 (0 for a zero block), elements E4M3(x * 2^-shared)
// clamped to +-448, round to nearest even (v_cvt_pk_fp8_f32).  x * 2^-shared
// is exact (a power of two, ldexp), so the only rounding is the conversion.
__global__ __launch_bounds__(kMoeThreads) void mx_quant_act(const uint16_t* __restrict__ x,
                                                            long blocks, uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales) {
  for (long b = (long)blockIdx.x * kMoeThreads + threadIdx.x; b < blocks;
       b += (long)gridDim.x * kMoeThreads) {
    const uint4* src = reinterpret_cast<const uint4*>(x + b * 32);
    float v[32];
    float amax = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 u = src[q];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[8 * q + 2 * i] = __uint_as_float(w[i] << 16);
        v[8 * q + 2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    int s = 0, shared = 0;
    if (amax > 0.f) {
      shared = min(max(__builtin_amdgcn_frexp_expf(amax) - 1 - 8, -127), 127);
      s = shared + 127;
    }
    uint32_t out[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t word = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float y0 = fminf(fmaxf(ldexpf(v[4 * i + 2 * h], -shared), -448.f), 448.f);
        const float y1 = fminf(fmaxf(ldexpf(v[4 * i + 2 * h + 1], -shared), -448.f), 448.f);
        const uint32_t pk = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false) & 0xFFFFu;
        word |= pk << (16 * h);
      }
      out[i] = word;
    }
    uint4* dst = reinterpret_cast<uint4*>(codes + b * 32);
    dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
    dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
    scales[b] = (uint8_t)s;
  }
}

// The online conversion: active expert list[a] -> workspace slot a.  One
// thread per 32-element block: 16 packed bytes in, 32 E4M3 codes out, and the
// block's E8M0 scale copied.
__global__ __launch_bounds__(kMoeThreads) void mxfp4_unpack(
    const uint8_t* __restrict__ w_fp4, const uint8_t* __restrict__ w_scale, int n, int k,
    const int32_t* __restrict__ experts, int n_active, const int32_t* __restrict__ n_active_dev,
    uint8_t* __restrict__ ws_codes, uint8_t* __restrict__ ws_scales) {
  const long per_expert = (long)n * (k / 32);
  const long total = per_expert * (n_active_dev ? min(*n_active_dev, n_active) : n_active);
  for (long b = (long)blockIdx.x * kMoeThreads + threadIdx.x; b < total;
       b += (long)gridDim.x * kMoeThreads) {
    const int a = (int)(b / per_expert);
    const long off = b - (long)a * per_expert;  // block within the expert: row-major [n][k/32]
    const long src_blk = (long)experts[a] * per_expert + off;
    const uint4 p = *reinterpret_cast<const uint4*>(w_fp4 + src_blk * 16);
    const uint32_t w[4] = {p.x, p.y, p.z, p.w};
    uint32_t out[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = e2m1x4_to_e4m3(w[i] & 0xFFFFu);  // elements 8i .. 8i+3
      out[2 * i + 1] = e2m1x4_to_e4m3(w[i] >> 16);  // elements 8i+4 .. 8i+7
    }
    uint4* dst = reinterpret_cast<uint4*>(ws_codes + ((long)a * per_expert + off) * 32);
    dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
    dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
    ws_scales[(long)a * per_expert + off] = w_scale[src_blk];
  }
}

__global__ __launch_bounds__(kMoeThreads) void moe_zero(int32_t* __restrict__ a, int n) {
  for (int i = blockIdx.x * kMoeThreads + threadIdx.x; i < n; i += gridDim.x * kMoeThreads) a[i] = 0;
}

// Count the pairs of every expert (kScatter = false), or place each pair into
// its expert's list (true).  Each workgroup takes chunks of kPairChunk pairs:
// it counts them per expert in LDS (the LDS atomic also gives each pair its
// rank within the chunk), then makes one global atomic per expert and chunk,
// which reserves the chunk's run in the expert's list.  With more experts than
// the LDS table holds, one global atomic per pair.
constexpr int kPairsPerThread = 8;
constexpr int kPairChunk = kPairsPerThread * kMoeThreads;
constexpr int kLdsExperts = 2048;
template <bool kScatter>
__global__ __launch_bounds__(kMoeThreads) void moe_pairs(const int32_t* __restrict__ route,
                                                         int pairs, int num_experts,
                                                         int32_t* __restrict__ count_or_cursor,
                                                         int32_t* __restrict__ list) {
  const int tid = threadIdx.x;
  if (num_experts > kLdsExperts) {
    for (int p = blockIdx.x * kMoeThreads + tid; p < pairs; p += gridDim.x * kMoeThreads) {
      const int e = route[p];
      if (e < 0 || e >= num_experts) continue;
      const int at = atomicAdd(&count_or_cursor[e], 1);
      if (kScatter) list[at] = p;
    }
    return;
  }
  __shared__ int hist[kLdsExperts];
  for (int c0 = blockIdx.x * kPairChunk; c0 < pairs; c0 += gridDim.x * kPairChunk) {
    for (int e = tid; e < num_experts; e += kMoeThreads) hist[e] = 0;
    __syncthreads();
    int ex[kPairsPerThread], rank[kPairsPerThread];
#pragma unroll
    for (int j = 0; j < kPairsPerThread; ++j) {
      const int p = c0 + j * kMoeThreads + tid;
      const int e = p < pairs ? route[p] : -1;
      ex[j] = e >= 0 && e < num_experts ? e : -1;
      rank[j] = ex[j] >= 0 ? atomicAdd(&hist[ex[j]], 1) : 0;
    }
    __syncthreads();
    for (int e = tid; e < num_experts; e += kMoeThreads) {
      const int h = hist[e];
      const int at = h ? atomicAdd(&count_or_cursor[e], h) : 0;
      if (kScatter) hist[e] = at;  // the chunk's first slot in expert e's list
    }
    if (kScatter) {
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kPairsPerThread; ++j)
        if (ex[j] >= 0) list[hist[ex[j]] + rank[j]] = c0 + j * kMoeThreads + tid;
    }
    __syncthreads();  // the table is cleared for the next chunk
  }
}

// One workgroup: offsets of every expert's pair list (cursor = offset), and the
// row tiles of bm pairs: tile i covers list[tile_p0[i] .. tile_p1[i]) of
// expert tile_e[i].
// ... and the routed experts in ascending order: active[a] = e, slot[e] = a
// (-1 for an expert no pair is routed to), *n_active.
__global__ __launch_bounds__(kScanThreads) void moe_scan(const int32_t* __restrict__ count,
                                                         int num_experts,
                                                         int32_t* __restrict__ cursor,
                                                         int32_t* __restrict__ tile_e,
                                                         int32_t* __restrict__ tile_p0,
                                                         int32_t* __restrict__ tile_p1,
                                                         int32_t* __restrict__ n_tiles,
                                                         int32_t* __restrict__ active,
                                                         int32_t* __restrict__ slot,
                                                         int32_t* __restrict__ n_active, int bm) {
  __shared__ int s_off[kScanThreads], s_til[kScanThreads], s_act[kScanThreads];
  const int tid = threadIdx.x;
  const int per = (num_experts + kScanThreads - 1) / kScanThreads;
  const int beg = min(num_experts, tid * per), end = min(num_experts, beg + per);
  int off = 0, til = 0, act = 0;
  for (int e = beg; e < end; ++e) {
    off += count[e];
    til += (count[e] + bm - 1) / bm;
    act += count[e] > 0;
  }
  s_off[tid] = off;
  s_til[tid] = til;
  s_act[tid] = act;
  __syncthreads();
  // inclusive prefix over threads (Hillis-Steele in LDS)
  for (int d = 1; d < kScanThreads; d <<= 1) {
    const int a = tid >= d ? s_off[tid - d] : 0, b = tid >= d ? s_til[tid - d] : 0,
              c = tid >= d ? s_act[tid - d] : 0;
    __syncthreads();
    s_off[tid] += a;
    s_til[tid] += b;
    s_act[tid] += c;
    __syncthreads();
  }
  int o = s_off[tid] - off, t = s_til[tid] - til, q = s_act[tid] - act;
  for (int e = beg; e < end; ++e) {
    const int c = count[e];
    cursor[e] = o;
    for (int m = 0; m < c; m += bm) {
      tile_e[t] = e;
      tile_p0[t] = o + m;
      tile_p1[t] = o + min(c, m + bm);
      ++t;
    }
    if (c > 0) {
      active[q] = e;
      slot[e] = q++;
    } else {
      slot[e] = -1;
    }
    o += c;
  }
  if (tid == kScanThreads - 1) {
    *n_tiles = s_til[tid];
    *n_active = s_act[tid];
  }
}

// One wave per (token, slot) pair not routed to any expert: its output row is zero.
__global__ __launch_bounds__(kMoeThreads) void moe_clear_unrouted(const int32_t* __restrict__ route,
                                                                  int pairs, int num_experts,
                                                                  int n, float* __restrict__ out) {
  const int p = blockIdx.x * (kMoeThreads / 64) + (threadIdx.x >> 6);
  if (p >= pairs) return;
  const int e = route[p];
  if (e >= 0 && e < num_experts) return;
  for (int c = threadIdx.x & 63; c < n; c += 64) out[(size_t)p * n + c] = 0.f;
}

__device__ __forceinline__ v8i load_fp8_operand(const uint8_t* row, int k0, int kg) {
  const v4i lo = *reinterpret_cast<const v4i*>(row + k0 + 16 * kg);
  const v4i hi = *reinterpret_cast<const v4i*>(row + k0 + 64 + 16 * kg);
  return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// grid (row-tile slots x ncb column blocks), block 256.  A work item (row
// tile, column block c) covers the tile's 16 RT pairs of one expert and columns
// [64 CT c, 64 CT (c + 1)); wave w owns 16 CT of them as CT 16-column MFMA
// tiles, over the RT 16-row tiles.  Items are ordered so that each XCD (the
// hardware deals workgroups to its 8 XCDs in turn) takes one contiguous run of
// them, and within a run the column blocks of kMoeGroupTiles consecutive row
// tiles come together: tiles of one expert then read its weight columns, and
// column blocks of one tile its A rows, through the same L2 at about the same
// time (workgroups past the live items exit).  Per K step of 128 KS the
// workgroup stages the tile's A rows (gathered per pair) once in LDS (double
// buffered), each wave reads its B rows straight from memory one step ahead,
// and runs KS x RT x CT scaled MFMAs.  KS = 2 doubles the bytes each wave has
// in flight (for the short tiles, whose B stream is bound by memory latency).
// kFp4: B is the MXFP4 weights; otherwise the FP8 workspace (expert e in slot
// b_slot[e]).  Two waves per SIMD (at most 256 registers a lane; every variant
// launched fits without spills): one wave per SIMD leaves the matrix unit idle
// through every load and barrier.  SV (K % 512 == 0, scale arrays 16 B
// aligned): lane (r, kg) loads 16 B of weight scales of column 16 (kg % CT) + r
// once per 4 K slices of 128, and the lanes trade them by cross-lane reads, instead of four
// 1-byte loads per step that each touch 16 cache lines for 64 bytes; the A
// scales likewise come in 16 B a row per 4 steps.
template <bool kFp4, int RT, int CT, int KS, bool SV>
__global__ __launch_bounds__(kMoeThreads)
__attribute__((amdgpu_waves_per_eu(2))) void moe_gemm(
    const uint8_t* __restrict__ b_codes, const uint8_t* __restrict__ b_scales,
    const int32_t* __restrict__ b_slot, int n, int k, const uint8_t* __restrict__ a_codes,
    const uint8_t* __restrict__ a_scales, int slots, const int32_t* __restrict__ list,
    const int32_t* __restrict__ tile_e, const int32_t* __restrict__ tile_p0,
    const int32_t* __restrict__ tile_p1, const int32_t* __restrict__ n_tiles, int ncb,
    float* __restrict__ out) {
  constexpr int kRows = 16 * RT;
  constexpr int kChunks = 8 * KS;                         // 16 B chunks of a row per K step
  constexpr int kPasses = kRows * kChunks / kMoeThreads;  // chunks each thread stages
  constexpr int kRowsPerPass = kMoeThreads / kChunks;
  // LDS bytes per A row: 128 KS, with the 16 B chunk c of row R stored in slot
  // c ^ swizzle(R): (R / 2) % 8 for rows of 128 B, R % 16 for rows of 256 B.
  // Either way the 16 rows of an MFMA read, and the chunks of a staging write,
  // land on distinct banks.
  constexpr int kPitch = 128 * KS;
  auto swizzle = [](int row) { return KS == 1 ? (row >> 1) & 7 : row & 15; };
  __shared__ __attribute__((aligned(16))) uint8_t a_lds[2][kRows * kPitch];
  // A scales: per step (4 KS bytes a row), or with SV per group of 4 steps (16 B a row)
  constexpr int kScaleRow = SV ? 16 : 4 * KS;
  __shared__ __attribute__((aligned(16))) uint8_t s_lds[2][kRows * kScaleRow];
  const int live_tiles = *n_tiles, live = live_tiles * ncb;
  const int hw = blockIdx.x;
  if (hw >= live) return;  // the whole workgroup
  // XCD x = hw % 8 takes items [x q + min(x, rem), ...) in dispatch order
  const int q = live >> 3, rem = live & 7, x = hw & 7;
  const int item = x * q + min(x, rem) + (hw >> 3);
  const int g0 = item / (kMoeGroupTiles * ncb) * kMoeGroupTiles;
  const int gt = min(kMoeGroupTiles, live_tiles - g0);
  const int within = item - g0 * ncb;
  const int tile = g0 + within % gt, cblk = within / gt;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, kg = lane >> 4;
  const int n0 = (cblk * 4 + wave) * 16 * CT;
  const bool wave_on = n0 < n;  // waves past N still stage A (barriers below)
  const int e = tile_e[tile], p0 = tile_p0[tile], p1 = tile_p1[tile];
  const int slot = kFp4 ? e : b_slot[e];
  const int kb = k / 32;
  // staging: thread tid copies chunk tid % kChunks of rows tid / kChunks +
  // kRowsPerPass q (q < kPasses); rows past the tile repeat the tile's first pair
  const uint8_t* srow[kPasses];
#pragma unroll
  for (int q = 0; q < kPasses; ++q) {
    const int p = p0 + tid / kChunks + kRowsPerPass * q;
    srow[q] = a_codes + (size_t)(list[p < p1 ? p : p0] / slots) * k;
  }
  const uint8_t* sscale = nullptr;  // scale staging: thread tid < kRows copies one row's 4 KS
  if (tid < kRows) {
    const int p = p0 + tid;
    sscale = a_scales + (size_t)(list[p < p1 ? p : p0] / slots) * kb;
  }
  // B rows of this lane: one base per expert, 32-bit offsets within it (n k / 2 < 2^31)
  const int rb = kFp4 ? k / 2 : k;
  const uint8_t* bbase = b_codes + (size_t)slot * n * rb;
  const uint8_t* sbase = b_scales + (size_t)slot * n * kb;
  uint32_t boff[CT], soff[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int col = min(n0 + 16 * ct + r, n - 1);
    boff[ct] = (uint32_t)col * rb;
    soff[ct] = (uint32_t)col * kb;
  }
  auto load_a = [&](int k0, v4i (&st)[kPasses], uint32_t (&sc)[KS]) {
#pragma unroll
    for (int q = 0; q < kPasses; ++q)
      st[q] = *reinterpret_cast<const v4i*>(srow[q] + k0 + 16 * (tid % kChunks));
    if (!SV && tid < kRows) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        sc[ks] = *reinterpret_cast<const uint32_t*>(sscale + k0 / 32 + 4 * ks);
    }
  };
  auto store_a = [&](int buf, const v4i (&st)[kPasses], const uint32_t (&sc)[KS]) {
#pragma unroll
    for (int q = 0; q < kPasses; ++q) {
      const int row = tid / kChunks + kRowsPerPass * q, c = tid % kChunks;
      *reinterpret_cast<v4i*>(&a_lds[buf][row * kPitch + 16 * (c ^ swizzle(row))]) = st[q];
    }
    if (!SV && tid < kRows) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        *reinterpret_cast<uint32_t*>(&s_lds[buf][tid * 4 * KS + 4 * ks]) = sc[ks];
    }
  };
  // SV: the A scales of steps 4 t .. 4 t + 3 (16 B a row) into scale buffer t % 2
  v4i scg = {};
  auto load_a_scales = [&](int t) {
    if (tid < kRows) scg = *reinterpret_cast<const v4i*>(sscale + 16 * t);
  };
  auto store_a_scales = [&](int t) {
    if (tid < kRows) *reinterpret_cast<v4i*>(&s_lds[t & 1][tid * 16]) = scg;
  };
  // FP4 fragments are 16 bytes (the instruction's upper four registers are
  // unused for FP4 and passed as zeros at the call)
  using BFrag = typename std::conditional<kFp4, v4i, v8i>::type;
  auto load_b = [&](int k0, BFrag (&b)[KS][CT], int (&sb)[KS][CT]) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int kk = k0 + 128 * ks;
        if constexpr (kFp4) {
          b[ks][ct] = *reinterpret_cast<const v4i*>(bbase + boff[ct] + kk / 2 + 16 * kg);
        } else {
          b[ks][ct] = load_fp8_operand(bbase + boff[ct], kk, kg);
        }
        if constexpr (!SV) sb[ks][ct] = sbase[soff[ct] + kk / 32 + kg];
      }
  };
  auto operand = [](const BFrag& b) {
    if constexpr (kFp4) return v8i{b[0], b[1], b[2], b[3], 0, 0, 0, 0};
    else return b;
  };
  v4f acc[RT][CT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[rt][ct] = v4f{0.f, 0.f, 0.f, 0.f};

  v4i st[kPasses];
  uint32_t sc[KS] = {};
  load_a(0, st, sc);
  store_a(0, st, sc);
  if constexpr (SV) {
    load_a_scales(0);
    store_a_scales(0);
  }
  BFrag b[KS][CT];
  int sb[KS][CT] = {};
  if (wave_on) load_b(0, b, sb);
  static_assert(CT == 1 || CT == 2 || CT == 4, "column tiles per wave");
  constexpr int G = 4 / KS;  // SV: steps per 16 B scale group (4 slices of K 128)
  // SV: the weight scales of one group for column n0 + 16 (kg % CT) + r
  v4i sg = {}, sgn = {};
  const uint32_t sgoff = (uint32_t)min(n0 + 16 * (kg % CT) + r, n - 1) * kb;
  if (SV && wave_on) sg = *reinterpret_cast<const v4i*>(sbase + sgoff);
  // Drain the prologue's loads here: the loop body reads b only after copying
  // it from the loads of the step before (which it waits for), and without this
  // the compiler's wait at the loop head also covers the loads issued for the
  // next step, which would stall every step on a full memory round trip.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int steps = k / (128 * KS);
  const int swz = swizzle(r);  // of the rows 16 rt + r this lane reads
  for (int s = 0; s < steps; ++s) {
    const int buf = s & 1;
    const bool more = s + 1 < steps;
    BFrag bn[KS][CT];
    int sbn[KS][CT];
    if (more) {
      load_a(128 * KS * (s + 1), st, sc);
      if (SV && (s + 1) % G == 0) load_a_scales((s + 1) / G);
      if (wave_on) load_b(128 * KS * (s + 1), bn, sbn);
      if (SV && wave_on && (s + 1) % G == 0)
        sgn = *reinterpret_cast<const v4i*>(sbase + sgoff + 16 * ((s + 1) / G));
    }
    if (wave_on) {
      int sbv[KS][CT];
      if constexpr (SV) {
        // slice ks of step s: byte kg of word (s % G) KS + ks of lane 16 ct + r
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int u = (s % G) * KS + ks;
          const int word = u == 0 ? sg[0] : u == 1 ? sg[1] : u == 2 ? sg[2] : sg[3];
#pragma unroll
          for (int ct = 0; ct < CT; ++ct)
            sbv[ks][ct] = (__shfl(word, 16 * ct + r) >> (8 * kg)) & 0xff;
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) sbv[ks][ct] = sb[ks][ct];
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const uint8_t* ar = &a_lds[buf][(16 * rt + r) * kPitch];
          const v4i lo = *reinterpret_cast<const v4i*>(ar + 16 * ((8 * ks + kg) ^ swz));
          const v4i hi = *reinterpret_cast<const v4i*>(ar + 16 * ((8 * ks + 4 + kg) ^ swz));
          const v8i a = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          const int sa = SV ? s_lds[(s / G) & 1][(16 * rt + r) * 16 + 4 * ((s % G) * KS + ks) + kg]
                            : s_lds[buf][(16 * rt + r) * 4 * KS + 4 * ks + kg];
#pragma unroll
          for (int ct = 0; ct < CT; ++ct)
            acc[rt][ct] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                a, operand(b[ks][ct]), acc[rt][ct], 0, kFp4 ? 4 : 0, 0, sa, 0, sbv[ks][ct]);
        }
    }
    if (more) {
      store_a(buf ^ 1, st, sc);
      if (SV && (s + 1) % G == 0) store_a_scales((s + 1) / G);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          b[ks][ct] = bn[ks][ct];
          sb[ks][ct] = sbn[ks][ct];
      if (SV && (s + 1) % G == 0) sg = sgn;
        }
    }
    __syncthreads();
  }
  if (!wave_on) return;
  // D[4 kg + i][r]: pair row 16 rt + 4 kg + i, column n0 + 16 ct + r
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p = p0 + 16 * rt + 4 * kg + i;
      if (p >= p1) continue;
      float* orow = out + (size_t)list[p] * n;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int col = n0 + 16 * ct + r;
        if (col < n) orow[col] = acc[rt][ct][i];
      }
    }
}

unsigned grid_for(long work, long cap) {
  long g = (work + kMoeThreads - 1) / kMoeThreads;
  return (unsigned)(g < 1 ? 1 : (g > cap ? cap : g));
}

}  // namespace

hipError_t launch_mx_quant_act(const uint16_t* x, int t, int k, uint8_t* codes, uint8_t* scales,
                               hipStream_t st) {
  const long blocks = (long)t * (k / 32);
  hipLaunchKernelGGL(mx_quant_act, dim3(grid_for(blocks, 65536)), dim3(kMoeThreads), 0, st, x,
                     blocks, codes, scales);
  return hipGetLastError();
}

hipError_t launch_mxfp4_unpack(const MxExperts& w, const int32_t* experts, int n_active,
                               uint8_t* ws_codes, uint8_t* ws_scales, hipStream_t st) {
  const long work = (long)n_active * w.n * (w.k / 32);
  hipLaunchKernelGGL(mxfp4_unpack, dim3(grid_for(work, 65536)), dim3(kMoeThreads), 0, st, w.fp4,
                     w.scale, w.n, w.k, experts, n_active, nullptr, ws_codes, ws_scales);
  return hipGetLastError();
}

MoeLayout moe_layout(const MxExperts& w, int pairs, bool fp8_workspace, size_t base) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const int num_experts = w.num_experts;
  MoeLayout L;
  // tall row tiles once the experts average 96 pairs or more
  L.bm = (long)pairs >= 96L * num_experts ? kMoeBMLarge : kMoeBMSmall;
  L.max_tiles = (pairs + L.bm - 1) / L.bm + num_experts;
  L.max_active = num_experts < pairs ? num_experts : pairs;
  size_t at = al(base);
  L.active = at;
  at = al(at + (size_t)num_experts * 4);
  L.slot = at;
  at = al(at + (size_t)num_experts * 4);
  L.n_active = at;
  at = al(at + 4);
  // the FP8 workspace: the routed experts' weights, one slot each
  L.ws_codes = at;
  if (fp8_workspace) at = al(at + (size_t)L.max_active * w.n * w.k);
  L.ws_scales = at;
  if (fp8_workspace) at = al(at + (size_t)L.max_active * w.n * (w.k / 32));
  L.count = at;
  at = al(at + (size_t)num_experts * 4);
  L.cursor = at;
  at = al(at + (size_t)num_experts * 4);
  L.list = at;
  at = al(at + (size_t)pairs * 4);
  L.tile_e = at;
  at = al(at + (size_t)L.max_tiles * 4);
  L.tile_p0 = at;
  at = al(at + (size_t)L.max_tiles * 4);
  L.tile_p1 = at;
  at = al(at + (size_t)L.max_tiles * 4);
  L.n_tiles = at;
  at = al(at + 4);
  L.total = at;
  return L;
}

hipError_t launch_moe_gemm(const MxExperts& w, bool fp8_workspace, const uint8_t* a_codes,
                           const uint8_t* a_scales, int t, const int32_t* route, int slots,
                           float* out, char* ws, const MoeLayout& L, hipStream_t st) {
  const int pairs = t * slots;
  int32_t* count = reinterpret_cast<int32_t*>(ws + L.count);
  int32_t* cursor = reinterpret_cast<int32_t*>(ws + L.cursor);
  int32_t* list = reinterpret_cast<int32_t*>(ws + L.list);
  int32_t* te = reinterpret_cast<int32_t*>(ws + L.tile_e);
  int32_t* tp0 = reinterpret_cast<int32_t*>(ws + L.tile_p0);
  int32_t* tp1 = reinterpret_cast<int32_t*>(ws + L.tile_p1);
  int32_t* nt = reinterpret_cast<int32_t*>(ws + L.n_tiles);
  hipLaunchKernelGGL(moe_zero, dim3(grid_for(w.num_experts, 64)), dim3(kMoeThreads), 0, st, count,
                     w.num_experts);
  const unsigned pair_grid = (unsigned)std::max(1, std::min(1024, (pairs + kPairChunk - 1) / kPairChunk));
  hipLaunchKernelGGL(moe_pairs<false>, dim3(pair_grid), dim3(kMoeThreads), 0, st, route, pairs,
                     w.num_experts, count, list);
  int32_t* active = reinterpret_cast<int32_t*>(ws + L.active);
  int32_t* slot = reinterpret_cast<int32_t*>(ws + L.slot);
  int32_t* n_active = reinterpret_cast<int32_t*>(ws + L.n_active);
  hipLaunchKernelGGL(moe_scan, dim3(1), dim3(kScanThreads), 0, st, count, w.num_experts, cursor,
                     te, tp0, tp1, nt, active, slot, n_active, L.bm);
  hipLaunchKernelGGL(moe_pairs<true>, dim3(pair_grid), dim3(kMoeThreads), 0, st, route, pairs,
                     w.num_experts, cursor, list);
  hipLaunchKernelGGL(moe_clear_unrouted, dim3((pairs + 3) / 4), dim3(kMoeThreads), 0, st, route,
                     pairs, w.num_experts, w.n, out);
  // tall tiles: 128 pairs x 256 columns (each weight read once per 128 pairs),
  // x 128 columns over the FP8 workspace (twice the B fragment registers);
  // short tiles: 64 pairs x 256 columns (a typical decode expert in one tile)
  const bool tall = L.bm == kMoeBMLarge;
  // short tiles over the FP4 weights take K 256 at a time where K allows (twice
  // the loads in flight; over the FP8 workspace that would spill registers)
  const bool ks2 = w.k % 256 == 0;
  // 16 B scale groups: scale rows a multiple of 16 B, both scale arrays 16 B
  // aligned (the FP8 workspace's are)
  const bool sv = w.k % 512 == 0 && (reinterpret_cast<uintptr_t>(a_scales) & 15) == 0 &&
                  (fp8_workspace || (reinterpret_cast<uintptr_t>(w.scale) & 15) == 0);
  const int wg_cols = tall && fp8_workspace ? 128 : 256;
  const int ncb = (w.n + wg_cols - 1) / wg_cols;
  const dim3 grid((unsigned)((long)L.max_tiles * ncb));
  const uint8_t* bc = w.fp4;
  const uint8_t* bs = w.scale;
  auto launch = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(kMoeThreads), 0, st, bc, bs, slot, w.n, w.k, a_codes,
                       a_scales, slots, list, te, tp0, tp1, nt, ncb, out);
  };
  if (fp8_workspace) {
    // the pages' path: the routed experts unpacked to FP8 into the workspace,
    // then the matmul on the workspace
    uint8_t* wc = reinterpret_cast<uint8_t*>(ws + L.ws_codes);
    uint8_t* wsc = reinterpret_cast<uint8_t*>(ws + L.ws_scales);
    const long work = (long)L.max_active * w.n * (w.k / 32);
    hipLaunchKernelGGL(mxfp4_unpack, dim3(grid_for(work, 65536)), dim3(kMoeThreads), 0, st, w.fp4,
                       w.scale, w.n, w.k, active, L.max_active, n_active, wc, wsc);
    bc = wc;
    bs = wsc;
    if (tall && sv)
      launch(moe_gemm<false, 8, 2, 1, true>);
    else if (tall)
      launch(moe_gemm<false, 8, 2, 1, false>);
    else if (sv)
      launch(moe_gemm<false, 4, 4, 1, true>);
    else
      launch(moe_gemm<false, 4, 4, 1, false>);
  } else {
    if (tall && sv)
      launch(moe_gemm<true, 8, 4, 1, true>);
    else if (tall)
      launch(moe_gemm<true, 8, 4, 1, false>);
    else if (ks2 && sv)
      launch(moe_gemm<true, 4, 4, 2, true>);
    else if (ks2)
      launch(moe_gemm<true, 4, 4, 2, false>);
    else
      launch(moe_gemm<true, 4, 4, 1, false>);
  }
  return hipGetLastError();
}

}  // namespace dsa

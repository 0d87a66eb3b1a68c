// Measurement support: the chip's achievable ceilings, a cache flush, and a
// probe of the FP8 matrix instruction's accumulation.
//
// None of this is on the attention path.  The pages ask that compute-bound
// and memory-bound stages be told apart and profiled ([P5] "Day-0 Readiness
// for Trillion-Parameter Models...", "Verification and Tuning"); a kernel's
// fraction of the published peak means more next to the fraction of what
// the chip sustains in practice:
//   - stream read: every byte of a buffer read once by a grid that fills the
//     chip, 64 B per lane in flight per step (the HBM ceiling of the decode
//     gather, which reads whole 16 KiB runs);
//   - matrix rate: back-to-back independent MFMAs with no memory traffic
//     (FP8 scaled 16x16x128, int8 16x16x64, bf16 16x16x32);
//   - cache flush: writes a scratch buffer so that the next kernel finds none
//     of its inputs in the L2 or the last-level cache;
//   - FP8 MFMA probe: one v_mfma_scale_f32_16x16x128_f8f6f4 per case (E4M3
//     operands, unit scales) so that the host can compare its sums with the
//     exact ones.
#include <hip/hip_runtime.h>

#include <type_traits>
#include <stdint.h>
#include <stdio.h>

#include "../../include/dsa_support.h"

namespace {

typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) short i16x8;

constexpr int kThreads = 256;

// grid-stride over 64 B per lane and step (four independent 16 B loads), XOR
// into one word per thread, which goes to sink[] so the loads stay live.
template <bool kNonTemporal>
__global__ __launch_bounds__(kThreads) void stream_read(const u32x4* __restrict__ p, size_t n16,
                                                        unsigned* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kThreads * 4;
  u32x4 acc = {0u, 0u, 0u, 0u};
  size_t i = ((size_t)blockIdx.x * kThreads + threadIdx.x);
  // lane-contiguous 16 B chunks: chunk c of a step is at base + c * (grid threads)
  const size_t lanes = (size_t)gridDim.x * kThreads;
  for (; i + 3 * lanes < n16; i += stride) {
    u32x4 v[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
      v[c] = kNonTemporal ? __builtin_nontemporal_load(p + i + c * lanes) : p[i + c * lanes];
#pragma unroll
    for (int c = 0; c < 4; ++c) acc ^= v[c];
  }
  for (; i < n16; i += lanes) acc ^= p[i];
  sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

__global__ __launch_bounds__(kThreads) void flush_write(u32x4* __restrict__ p, size_t n16,
                                                        unsigned seed) {
  const size_t lanes = (size_t)gridDim.x * kThreads;
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += lanes)
    p[i] = u32x4{seed, (unsigned)i, seed ^ (unsigned)i, 0u};
}

// kKind 0: FP8 scaled 16x16x128 (65536 flop); 1: int8 16x16x64 (32768 op);
// 2: bf16 16x16x32 (16384 flop).  Eight independent accumulators per wave,
// of the instruction's own type only: with a second, unused accumulator set
// live the compiler shuttles the accumulators between register files every
// iteration and the loop measures those copies instead.
template <int kKind>
__global__ __launch_bounds__(kThreads) void mfma_rate(int iters, float* __restrict__ sink) {
  using E = typename std::conditional<kKind == 1, int, float>::type;
  using Acc = typename std::conditional<kKind == 1, i32x4, f32x4>::type;
  const int lane = threadIdx.x & 63;
  const int x = 0x38383838 ^ (lane << 3);  // E4M3 1.0-ish bytes, lane-varied
  // distinct starting values: eight equal constants let the compiler merge
  // and then re-split the accumulators with copies inside the loop
  Acc acc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) acc[u] = Acc{(E)(lane + u), (E)lane, (E)u, (E)1};
  const i32x8 a8 = {x, x, x, x, x, x, x, x};
  const i32x4 a4 = {x, x, x, x};
  const i16x8 ab = {(short)x, (short)x, (short)x, (short)x, (short)x, (short)x, (short)x, (short)x};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if constexpr (kKind == 0)
        acc[u] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, a8, acc[u], 0, 0, 0, 127, 0,
                                                                    127);
      else if constexpr (kKind == 1)
        acc[u] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a4, a4, acc[u], 0, 0, 0);
      else
        acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ab),
                                                         __builtin_bit_cast(bf16x8, ab), acc[u], 0,
                                                         0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < 8; ++u) s += (float)acc[u][0];
  sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

// One wave per case: D = C + A B with A [16][128], B given as [16 columns][128]
// (E4M3 codes), C and D [16][16] fp32 row-major.  Lane (r, kg) = (lane % 16,
// lane / 16) holds k = 16 kg .. 16 kg + 15 and 64 + 16 kg .. 64 + 16 kg + 15 of
// row r of A and of column r of B; D[4 (lane / 16) + i][lane % 16] is its
// accumulator element i.
__global__ __launch_bounds__(64) void fp8_mfma_cases(const uint8_t* __restrict__ a,
                                                     const uint8_t* __restrict__ b,
                                                     const float* __restrict__ c, int n_cases,
                                                     float* __restrict__ d) {
  const int cs = blockIdx.x;
  if (cs >= n_cases) return;
  const int lane = threadIdx.x, r = lane & 15, kg = lane >> 4;
  const uint8_t* ar = a + ((size_t)cs * 16 + r) * 128;
  const uint8_t* br = b + ((size_t)cs * 16 + r) * 128;
  const i32x4 alo = *reinterpret_cast<const i32x4*>(ar + 16 * kg);
  const i32x4 ahi = *reinterpret_cast<const i32x4*>(ar + 64 + 16 * kg);
  const i32x4 blo = *reinterpret_cast<const i32x4*>(br + 16 * kg);
  const i32x4 bhi = *reinterpret_cast<const i32x4*>(br + 64 + 16 * kg);
  const i32x8 av = {alo[0], alo[1], alo[2], alo[3], ahi[0], ahi[1], ahi[2], ahi[3]};
  const i32x8 bv = {blo[0], blo[1], blo[2], blo[3], bhi[0], bhi[1], bhi[2], bhi[3]};
  f32x4 acc;
  const float* cc = c + (size_t)cs * 256;
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = cc[(4 * kg + i) * 16 + r];
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 0, 0, 0, 127, 0, 127);
  float* dd = d + (size_t)cs * 256;
#pragma unroll
  for (int i = 0; i < 4; ++i) dd[(4 * kg + i) * 16 + r] = acc[i];
}

thread_local char g_msg[256] = "";

int err(hipError_t e) {
  if (e == hipSuccess) return 0;
  snprintf(g_msg, sizeof g_msg, "%s", hipGetErrorString(e));
  return -6;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

extern "C" {

const char* dsa_support_last_error(void) { return g_msg; }

int dsa_probe_stream_read(const void* buf, size_t bytes, int variant, unsigned* sink, int grid,
                          hipStream_t stream) {
  if (!buf || !sink || grid < 1 || bytes < 16) return -1;
  if (!aligned(buf, 16) || bytes % 16) return -4;
  const size_t n16 = bytes / 16;
  const u32x4* p = static_cast<const u32x4*>(buf);
  if (variant == 0)
    hipLaunchKernelGGL(stream_read<false>, dim3(grid), dim3(kThreads), 0, stream, p, n16, sink);
  else
    hipLaunchKernelGGL(stream_read<true>, dim3(grid), dim3(kThreads), 0, stream, p, n16, sink);
  return err(hipGetLastError());
}

int dsa_cache_flush(void* buf, size_t bytes, unsigned seed, hipStream_t stream) {
  if (!buf || bytes < 16) return -1;
  if (!aligned(buf, 16) || bytes % 16) return -4;
  hipLaunchKernelGGL(flush_write, dim3(4096), dim3(kThreads), 0, stream, static_cast<u32x4*>(buf),
                     bytes / 16, seed);
  return err(hipGetLastError());
}

int dsa_probe_mfma_rate(int kind, int iters, int grid, float* sink, hipStream_t stream) {
  if (!sink || grid < 1 || iters < 1) return -1;
  switch (kind) {
    case DSA_PROBE_MFMA_FP8:
      hipLaunchKernelGGL(mfma_rate<0>, dim3(grid), dim3(kThreads), 0, stream, iters, sink);
      break;
    case DSA_PROBE_MFMA_I8:
      hipLaunchKernelGGL(mfma_rate<1>, dim3(grid), dim3(kThreads), 0, stream, iters, sink);
      break;
    case DSA_PROBE_MFMA_BF16:
      hipLaunchKernelGGL(mfma_rate<2>, dim3(grid), dim3(kThreads), 0, stream, iters, sink);
      break;
    default:
      return -3;
  }
  return err(hipGetLastError());
}

int dsa_probe_fp8_mfma(const uint8_t* a, const uint8_t* b, const float* c, int n_cases, float* d,
                       hipStream_t stream) {
  if (!a || !b || !c || !d || n_cases < 1) return -1;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(c, 4) || !aligned(d, 4)) return -4;
  hipLaunchKernelGGL(fp8_mfma_cases, dim3(n_cases), dim3(64), 0, stream, a, b, c, n_cases, d);
  return err(hipGetLastError());
}

}  // extern "C"

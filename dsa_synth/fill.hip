// Device-side filler for the seeded synthetic inputs (input data only).
//
// Implements exactly the stream definition of dsa_synth/gen.py so that the
// host can regenerate any element the device wrote:
//   h(seed, tag, i) = mix64(base + (i + 1) * 0x9E3779B97F4A7C15),
//   base = mix64((seed << 8) | tag),
//   mix64 = the SplitMix64 output function (Steele, Lea, Flood, OOPSLA 2014);
// element e of a bf16-normal tensor is table[(h(seed, tag, e >> 2) >> (16 (e & 3))) & 0xFFFF].
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

uint64_t mix64_host(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// One thread per group of four consecutive elements (one hash).
__global__ void fill_bf16_normal(uint16_t* __restrict__ dst, uint64_t n, uint64_t first_group,
                                 uint64_t base, const uint16_t* __restrict__ table) {
  const uint64_t groups = (n + 3) / 4;
  for (uint64_t g = blockIdx.x * (uint64_t)blockDim.x + threadIdx.x; g < groups;
       g += (uint64_t)gridDim.x * blockDim.x) {
    const uint64_t h = mix64(base + (first_group + g + 1) * 0x9E3779B97F4A7C15ull);
    const uint64_t v0 = table[h & 0xFFFF];
    const uint64_t v1 = table[(h >> 16) & 0xFFFF];
    const uint64_t v2 = table[(h >> 32) & 0xFFFF];
    const uint64_t v3 = table[(h >> 48) & 0xFFFF];
    const uint64_t e = g * 4;
    if (e + 4 <= n) {
      *reinterpret_cast<uint64_t*>(dst + e) = v0 | (v1 << 16) | (v2 << 32) | (v3 << 48);
    } else {
      if (e + 0 < n) dst[e + 0] = (uint16_t)v0;
      if (e + 1 < n) dst[e + 1] = (uint16_t)v1;
      if (e + 2 < n) dst[e + 2] = (uint16_t)v2;
    }
  }
}

}  // namespace

// Fill dst[0..n) (bf16 bits) with elements [offset, offset + n) of the
// normal stream (seed, tag).  dst must be 8-byte aligned, offset a multiple
// of 4.  Returns 0 on success, a hipError_t value otherwise.
extern "C" int dsa_synth_fill_bf16_normal(void* dst, uint64_t n, uint64_t offset, uint64_t seed,
                                          uint32_t tag, const void* table, hipStream_t stream) {
  if (n == 0) return 0;
  if (!dst || !table || (offset & 3) || (reinterpret_cast<uintptr_t>(dst) & 7)) return -1;
  const uint64_t base = mix64_host((seed << 8) | tag);
  const uint64_t groups = (n + 3) / 4;
  uint64_t blocks = (groups + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fill_bf16_normal, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<uint16_t*>(dst), n, offset / 4, base,
                     static_cast<const uint16_t*>(table));
  return (int)hipGetLastError();
}

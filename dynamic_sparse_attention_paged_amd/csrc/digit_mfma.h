// Exact products of E4M3 codes on the int8 matrix cores: every E4M3 value
// is n * 2^-9 with an integer |n| <= 229376 < 2^18, written here as three
// signed base-128 digits (|n| & 127, (|n| >> 7) & 127, |n| >> 14, each with
// the sign of n), so every digit fits in int8 and digit-plane dot products
// accumulate exactly in int32 on v_mfma_i32_16x16x64_i8.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef __attribute__((ext_vector_type(4))) int i32x4;

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

}  // namespace dsa

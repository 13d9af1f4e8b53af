// MXFP4 encoding of one 32-element block (shared by the quantiser kernel and
// the streaming cache append, so both write identical codes).
//
// Pages: pytorch.kr DeepSeek-V4 summary, FP4 QAT paragraph: the indexer's QK
// path runs in FP4 (MXFP4).  The pages give no conversion rule; the reading
// taken is the OCP MX one: the block's shared scale is 2^e, e = floor(log2(
// amax)) - 2 (2: the largest e2m1 exponent), stored as the E8M0 byte e + 127
// clamped to [0, 254] (0 for a block of zeros); each element becomes the e2m1
// value nearest to x / 2^e, ties to the code with an even mantissa bit,
// saturating at 6; zero is code 0 whatever its sign.  Codes are packed two per
// byte, even element low.
//
// floor(log2(amax)) is the biased exponent field of amax (a subnormal or zero
// amax clamps e to -127), and x * 2^-e is exact in fp32 unless it underflows,
// in which case it is far below the first rounding boundary (0.25) anyway, so
// the codes are exact.
#pragma once
#include "common.hpp"

namespace csa {

// nearest e2m1 magnitude code of m >= 0, ties to the even code: the number of
// rounding boundaries below m (a boundary between an odd and the next even
// code counts when m reaches it, the others only when m passes it)
__device__ __forceinline__ uint32_t e2m1_code_of(float m) {
  return (m > 0.25f) + (m >= 0.75f) + (m > 1.25f) + (m >= 1.75f) + (m > 2.5f) + (m >= 3.5f) + (m > 5.0f);
}

// the block's scale exponent e from the bits of its largest magnitude (the
// biased exponent field: 0 for zero or a subnormal, which clamps e to -127)
__device__ __forceinline__ int mxfp4_exponent(uint32_t amax_bits) {
  const int E = (int)(amax_bits >> 23);
  return E == 0 ? -127 : (E - 129 < -127 ? -127 : E - 129);
}
// 2^-e, a normal float for e in [-127, 125]
__device__ __forceinline__ float mxfp4_inverse(int e) { return __uint_as_float((uint32_t)(127 - e) << 23); }
// the 4-bit code of element v given 2^-e
__device__ __forceinline__ uint32_t mxfp4_code(float v, float inv) {
  const float t = v * inv;
  const uint32_t mag = e2m1_code_of(fabsf(t));
  return mag | ((t < 0.f && mag != 0u) ? 8u : 0u);
}

// x: the block's 32 elements (64 bytes of bf16 or 128 of fp32, 16-byte
// aligned) -> 16 code bytes at codes (16-byte aligned) and the E8M0 byte at *scale
template <bool BF16>
__device__ __forceinline__ void mxfp4_block(const uint8_t* x, uint8_t* codes, uint8_t* scale) {
  float v[32];
  if constexpr (BF16) {
    const uint4* p = reinterpret_cast<const uint4*>(x);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 u = p[q];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[8 * q + 2 * i] = __uint_as_float(w[i] << 16);
        v[8 * q + 2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
      }
    }
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(x);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint4 u = p[q];
      v[4 * q] = __uint_as_float(u.x); v[4 * q + 1] = __uint_as_float(u.y);
      v[4 * q + 2] = __uint_as_float(u.z); v[4 * q + 3] = __uint_as_float(u.w);
    }
  }
  uint32_t amax_bits = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t a = __float_as_uint(v[i]) & 0x7fffffffu;
    amax_bits = a > amax_bits ? a : amax_bits;
  }
  const int e = mxfp4_exponent(amax_bits);
  const float inv = mxfp4_inverse(e);
  uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 32; ++i) w[i >> 3] |= mxfp4_code(v[i], inv) << (4 * (i & 7));
  *reinterpret_cast<uint4*>(codes) = make_uint4(w[0], w[1], w[2], w[3]);
  *scale = (uint8_t)(e + 127);
}

}  // namespace csa

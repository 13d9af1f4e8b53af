// MXFP4 quantisation of indexer vectors, the step before the indexer.
//
// Pages: pytorch.kr DeepSeek-V4 summary, FP4 QAT paragraph: the indexer's QK
// path runs in FP4 (MXFP4), dequantisation to FP8 is lossless.  The pages give
// no conversion rule; the reading taken is the OCP MX one: per block of 32
// elements the shared scale is 2^e, e = floor(log2(amax)) - 2 (2: the largest
// e2m1 exponent), stored as the E8M0 byte e + 127 clamped to [0, 254] (0 for a
// block of zeros); each element becomes the e2m1 value nearest to x / 2^e,
// ties to the code with an even mantissa bit, saturating at 6; zero is code 0
// whatever its sign.  Codes are packed two per byte, even element low.
//
// One thread per 32-element block (HBM-bound streaming: 64 or 128 bytes in,
// 17 bytes out).  floor(log2(amax)) is the biased exponent field of amax (a
// subnormal or zero amax clamps e to -127), and x * 2^-e is exact in fp32
// unless it underflows, in which case it is far below the first rounding
// boundary (0.25) anyway, so the codes are exact.
#include "common.hpp"
#include "kernels.hpp"

namespace csa {

// nearest e2m1 magnitude code of m >= 0, ties to the even code: the number of
// rounding boundaries below m (a boundary between an odd and the next even
// code counts when m reaches it, the others only when m passes it)
__device__ __forceinline__ uint32_t e2m1_code_of(float m) {
  return (m > 0.25f) + (m >= 0.75f) + (m > 1.25f) + (m >= 1.75f) + (m > 2.5f) + (m >= 3.5f) + (m > 5.0f);
}

template <bool BF16>
__global__ __launch_bounds__(256) void k_mxfp4_quant(int64_t nblocks, const uint8_t* __restrict__ x,
                                                     uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (blk >= nblocks) return;
  float v[32];
  if constexpr (BF16) {
    const uint4* p = reinterpret_cast<const uint4*>(x + (size_t)blk * 64);
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
    const uint4* p = reinterpret_cast<const uint4*>(x + (size_t)blk * 128);
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
  const int E = (int)(amax_bits >> 23);  // biased exponent of amax; 0 for zero or a subnormal
  const int e = E == 0 ? -127 : (E - 129 < -127 ? -127 : E - 129);
  const float inv = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e, a normal float for e in [-127, 125]
  uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float t = v[i] * inv;
    const uint32_t mag = e2m1_code_of(fabsf(t));
    const uint32_t code = mag | ((t < 0.f && mag != 0u) ? 8u : 0u);
    w[i >> 3] |= code << (4 * (i & 7));
  }
  *reinterpret_cast<uint4*>(codes + (size_t)blk * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  scales[blk] = (uint8_t)(e + 127);
}

int launch_mxfp4_quant(bool bf16, int64_t rows, int dim, const void* x, uint8_t* codes, uint8_t* scales,
                       hipStream_t stream) {
  const int64_t nblocks = rows * (dim / 32);
  if (nblocks == 0) return 0;
  const dim3 grid((unsigned)((nblocks + 255) / 256));
  const hipError_t e = launch(10, kProfBoth, bf16 ? k_mxfp4_quant<true> : k_mxfp4_quant<false>, grid, dim3(256), 0,
                              stream, nblocks, (const uint8_t*)x, codes, scales);
  return e == hipSuccess && hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace csa

// Pooling (compression) kernel: every m consecutive raw rows of a sequence
// become one row, channel by channel, as a softmax-weighted sum over the
// block with per-channel logits (pages: pytorch.kr DeepSeek-V4 summary,
// CSA/HCA section — m consecutive KV entries merged into one, m' >> m for
// HCA; the softmax-weighted rule is the reading taken).
//
// HBM-bound streaming: each thread owns 16 bytes of channels (8 bf16 or 4
// fp32) of one output block and walks the block's m rows; consecutive
// threads cover consecutive 16-byte groups of the same rows, so every load
// is a fully coalesced row segment.  fp32 math, one rounding at the store.
#include "common.hpp"
#include "kernels.hpp"

namespace csa {

template <bool BF16>
struct Vec16 {
  static constexpr int N = BF16 ? 8 : 4;
  __device__ static void load(const void* p, float* v) {
    uint4 u = *reinterpret_cast<const uint4*>(p);
    if constexpr (BF16) {
      uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
      }
    } else {
      v[0] = __uint_as_float(u.x); v[1] = __uint_as_float(u.y);
      v[2] = __uint_as_float(u.z); v[3] = __uint_as_float(u.w);
    }
  }
  __device__ static void store(void* p, const float* v) {
    uint4 u;
    if constexpr (BF16) {
      u.x = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
      u.y = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
      u.z = f32_to_bf16(v[4]) | (f32_to_bf16(v[5]) << 16);
      u.w = f32_to_bf16(v[6]) | (f32_to_bf16(v[7]) << 16);
    } else {
      u.x = __float_as_uint(v[0]); u.y = __float_as_uint(v[1]);
      u.z = __float_as_uint(v[2]); u.w = __float_as_uint(v[3]);
    }
    *reinterpret_cast<uint4*>(p) = u;
  }
};

template <bool BF16>
__global__ __launch_bounds__(256) void k_compress(const int64_t* __restrict__ tok_off,
                                                  const int64_t* __restrict__ pool_off, int m,
                                                  int width, const uint8_t* __restrict__ x,
                                                  const uint8_t* __restrict__ z,
                                                  uint8_t* __restrict__ out) {
  using V = Vec16<BF16>;
  constexpr int N = V::N;
  constexpr int ES = BF16 ? 2 : 4;
  const int b = blockIdx.y;
  const int64_t r0 = tok_off[b];
  const int64_t L = tok_off[b + 1] - r0;
  const int64_t cap = pool_off[b + 1] - pool_off[b];
  const int64_t P = (L / m) < cap ? (L / m) : cap;
  const int groups = width / N;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t j = gid / groups;
  const int g = (int)(gid - j * groups);
  if (j >= P) return;

  const size_t row_bytes = (size_t)width * ES;
  const uint8_t* xp = x + (size_t)(r0 + j * m) * row_bytes + (size_t)g * 16;
  const uint8_t* zp = z + (size_t)(r0 + j * m) * row_bytes + (size_t)g * 16;

  float mx[N], den[N], acc[N];
#pragma unroll
  for (int c = 0; c < N; ++c) { mx[c] = -INFINITY; den[c] = 0.f; acc[c] = 0.f; }

  // online softmax in chunks of up to 8 rows: one rescale per chunk
  for (int i0 = 0; i0 < m; i0 += 8) {
    const int n = (m - i0) < 8 ? (m - i0) : 8;
    float zz[8][N], xx[8][N];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i < n) {
        V::load(zp + (size_t)(i0 + i) * row_bytes, zz[i]);
        V::load(xp + (size_t)(i0 + i) * row_bytes, xx[i]);
      }
    }
#pragma unroll
    for (int c = 0; c < N; ++c) {
      float cm = mx[c];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i < n) cm = fmaxf(cm, zz[i][c]);
      const float alpha = fast_exp2((mx[c] - cm) * kLog2e);  // exp2(-inf) = 0 on the first chunk
      float d = den[c] * alpha, a = acc[c] * alpha;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (i < n) {
          const float e = fast_exp2((zz[i][c] - cm) * kLog2e);
          d += e;
          a = fmaf(e, xx[i][c], a);
        }
      }
      mx[c] = cm; den[c] = d; acc[c] = a;
    }
  }
  float o[N];
#pragma unroll
  for (int c = 0; c < N; ++c) o[c] = acc[c] / den[c];
  V::store(out + (size_t)(pool_off[b] + j) * row_bytes + (size_t)g * 16, o);
}

int launch_compress(bool bf16, int n_seq, const int64_t* tok_off, const int64_t* pool_off,
                    int64_t max_len, int m, int width, const void* x, const void* z, void* out,
                    hipStream_t stream) {
  const int N = bf16 ? 8 : 4;
  const int64_t groups = width / N;
  const int64_t max_blocks = max_len / m;
  if (max_blocks == 0 || n_seq == 0) return 0;
  const int64_t threads = max_blocks * groups;
  dim3 grid((unsigned)((threads + 255) / 256), (unsigned)n_seq);
  prof_begin(5, stream);
  if (bf16)
    hipLaunchKernelGGL(k_compress<true>, grid, dim3(256), 0, stream, tok_off, pool_off, m, width,
                       (const uint8_t*)x, (const uint8_t*)z, (uint8_t*)out);
  else
    hipLaunchKernelGGL(k_compress<false>, grid, dim3(256), 0, stream, tok_off, pool_off, m, width,
                       (const uint8_t*)x, (const uint8_t*)z, (uint8_t*)out);
  prof_end(5, stream);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace csa

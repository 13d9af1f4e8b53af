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
#include "pool_core.hpp"

namespace csa {

template <bool BF16>
__global__ __launch_bounds__(256) void k_compress(const int64_t* __restrict__ tok_off,
                                                  const int64_t* __restrict__ pool_off, int m,
                                                  int width, const uint8_t* __restrict__ x,
                                                  const uint8_t* __restrict__ z,
                                                  uint8_t* __restrict__ out) {
  constexpr int N = Vec16<BF16>::N;
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
  pool_block<BF16>(
      m, [&](int i) { return xp + (size_t)i * row_bytes; }, [&](int i) { return zp + (size_t)i * row_bytes; },
      out + (size_t)(pool_off[b] + j) * row_bytes + (size_t)g * 16);
}

// Short blocks (m <= MAXM <= 8): each thread pools the same 16 bytes of
// channels of BPT consecutive blocks, loading all of their rows before any
// arithmetic, so a thread keeps BPT * 2m loads in flight and the grid needs
// BPT times fewer workgroups.  Same per-channel arithmetic as pool_block
// (pool_core.hpp).
template <bool BF16, int BPT, int MAXM>
__global__ __launch_bounds__(256) void k_compress_short(const int64_t* __restrict__ tok_off,
                                                        const int64_t* __restrict__ pool_off, int m, int width,
                                                        const uint8_t* __restrict__ x, const uint8_t* __restrict__ z,
                                                        uint8_t* __restrict__ out) {
  constexpr int N = Vec16<BF16>::N;
  constexpr int ES = BF16 ? 2 : 4;
  const int b = blockIdx.y;
  const int64_t r0 = tok_off[b];
  const int64_t L = tok_off[b + 1] - r0;
  const int64_t cap = pool_off[b + 1] - pool_off[b];
  const int64_t P = (L / m) < cap ? (L / m) : cap;
  const int groups = width / N;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t jq = gid / groups;
  const int g = (int)(gid - jq * groups);
  const int64_t j0 = jq * BPT;
  if (j0 >= P) return;
  const size_t row_bytes = (size_t)width * ES;
  const uint8_t* xp = x + (size_t)r0 * row_bytes + (size_t)g * 16;
  const uint8_t* zp = z + (size_t)r0 * row_bytes + (size_t)g * 16;
  uint4 xr[BPT][MAXM], zr[BPT][MAXM];
#pragma unroll
  for (int k = 0; k < BPT; ++k) {
    const int64_t j = j0 + k < P ? j0 + k : P - 1;  // blocks past P load the last one (consumed, not stored)
#pragma unroll
    for (int i = 0; i < MAXM; ++i) {
      const int ii = i < m ? i : m - 1;
      const size_t off = (size_t)(j * m + ii) * row_bytes;
      xr[k][i] = *reinterpret_cast<const uint4*>(xp + off);
      zr[k][i] = *reinterpret_cast<const uint4*>(zp + off);
    }
  }
#pragma unroll
  for (int k = 0; k < BPT; ++k) {
    if (j0 + k >= P) {  // loaded (the last block again) but not pooled
#pragma unroll
      for (int i = 0; i < MAXM; ++i) {
        consume_load(xr[k][i].x);
        consume_load(zr[k][i].x);
      }
      continue;
    }
    PoolState<BF16> st;
    pool_reset(st);
    float zz[8][N], xx[8][N];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      Vec16<BF16>::load(&zr[k][i < MAXM ? i : MAXM - 1], zz[i]);
      Vec16<BF16>::load(&xr[k][i < MAXM ? i : MAXM - 1], xx[i]);
    }
    pool_chunk(st, zz, xx, m);
    pool_store<BF16>(st, out + (size_t)(pool_off[b] + j0 + k) * row_bytes + (size_t)g * 16);
  }
}

// Long blocks (m a multiple of kPoolSeg): one thread per (block, 16-row
// segment, 16-byte channel group), every one of its segment's 2 x 16 rows
// loaded before any arithmetic; the segments' states meet in LDS and the
// segment-0 thread folds them left to right, so the result has pool_block's
// bits (the same chunks, the same folds in the same order).  Threads run
// segment-major within a block (consecutive threads: consecutive channel
// groups of one row, so loads coalesce); 256 / (segments x groups) blocks per
// workgroup.
template <bool BF16>
__global__ __launch_bounds__(256) void k_compress_seg(const int64_t* __restrict__ tok_off,
                                                      const int64_t* __restrict__ pool_off, int m, int width,
                                                      const uint8_t* __restrict__ x, const uint8_t* __restrict__ z,
                                                      uint8_t* __restrict__ out) {
  using V = Vec16<BF16>;
  constexpr int N = V::N;
  constexpr int ES = BF16 ? 2 : 4;
  __shared__ float st_s[3][N][256];  // a segment's (max, denominator, sum) per channel, by thread
  const int b = blockIdx.y;
  const int64_t r0 = tok_off[b];
  const int64_t L = tok_off[b + 1] - r0;
  const int64_t cap = pool_off[b + 1] - pool_off[b];
  const int64_t P = (L / m) < cap ? (L / m) : cap;
  const int groups = width / N, segs = m / kPoolSeg, per_block = groups * segs, bpw = 256 / per_block;
  if ((int64_t)blockIdx.x * bpw >= P) return;  // uniform
  const int tid = threadIdx.x;
  const int lb = tid / per_block, rem = tid - lb * per_block;
  const int s = rem / groups, g = rem - s * groups;
  const int64_t j = (int64_t)blockIdx.x * bpw + lb;
  const size_t row_bytes = (size_t)width * ES;
  PoolState<BF16> st;
  if (j < P) {
    const size_t off = (size_t)(r0 + j * m + s * kPoolSeg) * row_bytes + (size_t)g * 16;
    uint4 xr[kPoolSeg], zr[kPoolSeg];
#pragma unroll
    for (int i = 0; i < kPoolSeg; ++i) {
      zr[i] = *reinterpret_cast<const uint4*>(z + off + (size_t)i * row_bytes);
      xr[i] = *reinterpret_cast<const uint4*>(x + off + (size_t)i * row_bytes);
    }
    pool_reset(st);
#pragma unroll
    for (int c0 = 0; c0 < kPoolSeg; c0 += 8) {
      float zz[8][N], xx[8][N];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        V::load(&zr[c0 + i], zz[i]);
        V::load(&xr[c0 + i], xx[i]);
      }
      pool_chunk(st, zz, xx, 8);
    }
#pragma unroll
    for (int c = 0; c < N; ++c) {
      st_s[0][c][tid] = st.mx[c];
      st_s[1][c][tid] = st.den[c];
      st_s[2][c][tid] = st.acc[c];
    }
  }
  __syncthreads();
  if (j < P && s == 0) {
    for (int s2 = 1; s2 < segs; ++s2) {
      const int u = tid + s2 * groups;  // segment s2 of the same block and channel group
      PoolState<BF16> t;
#pragma unroll
      for (int c = 0; c < N; ++c) {
        t.mx[c] = st_s[0][c][u];
        t.den[c] = st_s[1][c][u];
        t.acc[c] = st_s[2][c][u];
      }
      pool_fold(st, t);
    }
    pool_store<BF16>(st, out + (size_t)(pool_off[b] + j) * row_bytes + (size_t)g * 16);
  }
}

int launch_compress(bool bf16, int n_seq, const int64_t* tok_off, const int64_t* pool_off,
                    int64_t max_len, int m, int width, const void* x, const void* z, void* out,
                    hipStream_t stream) {
  const int N = bf16 ? 8 : 4;
  const int64_t groups = width / N;
  const int64_t max_blocks = max_len / m;
  if (max_blocks == 0 || n_seq == 0) return 0;
  hipError_t e;
  if (m <= 8) {
    constexpr int BPT = 2;
    const int64_t threads = (max_blocks + BPT - 1) / BPT * groups;
    dim3 grid((unsigned)((threads + 255) / 256), (unsigned)n_seq);
    auto k = m <= 4 ? (bf16 ? k_compress_short<true, BPT, 4> : k_compress_short<false, BPT, 4>)
                    : (bf16 ? k_compress_short<true, BPT, 8> : k_compress_short<false, BPT, 8>);
    e = launch(5, kProfBoth, k, grid, dim3(256), 0, stream, tok_off, pool_off, m, width, (const uint8_t*)x,
               (const uint8_t*)z, (uint8_t*)out);
  } else if (m % kPoolSeg == 0 && groups * (m / kPoolSeg) <= 256 && 256 % (groups * (m / kPoolSeg)) == 0) {
    const int64_t bpw = 256 / (groups * (m / kPoolSeg));
    dim3 grid((unsigned)((max_blocks + bpw - 1) / bpw), (unsigned)n_seq);
    e = launch(5, kProfBoth, bf16 ? k_compress_seg<true> : k_compress_seg<false>, grid, dim3(256), 0, stream, tok_off,
               pool_off, m, width, (const uint8_t*)x, (const uint8_t*)z, (uint8_t*)out);
  } else {
    const int64_t threads = max_blocks * groups;
    dim3 grid((unsigned)((threads + 255) / 256), (unsigned)n_seq);
    e = launch(5, kProfBoth, bf16 ? k_compress<true> : k_compress<false>, grid, dim3(256), 0, stream, tok_off,
               pool_off, m, width, (const uint8_t*)x, (const uint8_t*)z, (uint8_t*)out);
  }
  return e == hipSuccess && hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace csa

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

int launch_compress(bool bf16, int n_seq, const int64_t* tok_off, const int64_t* pool_off,
                    int64_t max_len, int m, int width, const void* x, const void* z, void* out,
                    hipStream_t stream) {
  const int N = bf16 ? 8 : 4;
  const int64_t groups = width / N;
  const int64_t max_blocks = max_len / m;
  if (max_blocks == 0 || n_seq == 0) return 0;
  const int64_t threads = max_blocks * groups;
  dim3 grid((unsigned)((threads + 255) / 256), (unsigned)n_seq);
  const hipError_t e = launch(5, kProfBoth, bf16 ? k_compress<true> : k_compress<false>, grid, dim3(256), 0, stream,
                              tok_off, pool_off, m, width, (const uint8_t*)x, (const uint8_t*)z, (uint8_t*)out);
  return e == hipSuccess && hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace csa

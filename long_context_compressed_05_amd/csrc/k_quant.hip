// MXFP4 quantisation of indexer vectors, the step before the indexer: one
// thread per 32-element block (HBM-bound streaming: 64 or 128 bytes in, 17
// bytes out).  The conversion rule (OCP MX, the reading taken) and its
// exactness are stated with the block encoder in quant_core.hpp.
#include "common.hpp"
#include "kernels.hpp"
#include "quant_core.hpp"

namespace csa {

template <bool BF16>
__global__ __launch_bounds__(256) void k_mxfp4_quant(int64_t nblocks, const uint8_t* __restrict__ x,
                                                     uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (blk >= nblocks) return;
  mxfp4_block<BF16>(x + (size_t)blk * (BF16 ? 64 : 128), codes + (size_t)blk * 16, scales + blk);
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

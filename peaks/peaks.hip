// Measured peaks of the GPU the benchmark runs on: reference kernels whose
// rates the benchmark reports next to the datasheet peaks, so that every
// roofline fraction can also be read against what this part sustains.
// MEASUREMENT INFRASTRUCTURE ONLY: the benchmark loads it; the product
// library does not.
//
//  - peak_read:      one pass over a buffer with 16-byte loads, each thread
//                    keeping `unroll` loads in flight, a reduction kept live
//                    through one word per workgroup (HBM read bandwidth);
//                    peak_read_chunked: the same, each workgroup streaming a
//                    contiguous span of the buffer;
//  - peak_mfma_fp4:  back-to-back block-scaled FP4 MFMAs (32x32x64, the
//                    indexer's instruction), four independent accumulators
//                    per wave;
//  - peak_mfma_bf16: back-to-back bf16 MFMAs (16x16x32, the attention's
//                    instruction, or 32x32x16);
//  - peak_empty:     a kernel that does nothing (the floor of any launch's
//                    measured duration: dispatch, wave launch, end of kernel);
//  - peak_valu:      `iters` x 256 independent 32-bit VALU adds per wave (four
//                    chains), waves per workgroup as given: the instruction
//                    issue rate of one wave, and of several sharing a SIMD.
// Each call launches one kernel on `stream`; when start/stop are non-null
// they are attached to the dispatch (hipExtLaunchKernel) and time the kernel
// alone.  Returns 0 or -1 (launch failure).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

template <int U>
__global__ __launch_bounds__(256) void k_peak_read(const uint4* __restrict__ p, size_t n16, uint32_t* sink) {
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // keep the loads live: one word per workgroup (lanes folded with atomics in LDS)
  __shared__ uint32_t red;
  if (threadIdx.x == 0) red = 0;
  __syncthreads();
  atomicXor(&red, acc);
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red;
}

// The same pass with each workgroup streaming its own contiguous span of
// `chunk16` elements (the access pattern of the pooling kernels): per step a
// thread loads U elements 256 apart, so a workgroup reads U x 4 KB in order.
template <int U>
__global__ __launch_bounds__(256) void k_peak_read_chunk(const uint4* __restrict__ p, size_t n16, size_t chunk16,
                                                         uint32_t* sink) {
  const size_t begin = (size_t)blockIdx.x * chunk16;
  const size_t end = begin + chunk16 < n16 ? begin + chunk16 : n16;
  uint32_t acc = 0;
  size_t i = begin + threadIdx.x;
  for (; i + (size_t)(U - 1) * 256 < end; i += (size_t)U * 256) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = p[i + (size_t)u * 256];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < end; i += 256) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  __shared__ uint32_t red;
  if (threadIdx.x == 0) red = 0;
  __syncthreads();
  atomicXor(&red, acc);
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red;
}

__global__ __launch_bounds__(256) void k_peak_fp4(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  v8i a = {lane, lane * 3, lane * 5, lane * 7, 0, 0, 0, 0};
  v8i b = {lane * 11, lane * 13, lane * 17, lane * 19, 0, 0, 0, 0};
  v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, 4, 4, 0, 127, 0, 127);
    c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c1, 4, 4, 0, 127, 0, 127);
    c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c2, 4, 4, 0, 127, 0, 127);
    c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c3, 4, 4, 0, 127, 0, 127);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) s += c0[j] + c1[j] + c2[j] + c3[j];
  sink[blockIdx.x * 256 + threadIdx.x] = s;
}

template <bool BIG>
__global__ __launch_bounds__(256) void k_peak_bf16(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  v8bf a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(0.001f * (float)(lane + j));
    b[j] = (__bf16)(0.002f * (float)(lane - j));
  }
  float s = 0.f;
  if constexpr (BIG) {
    v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int i = 0; i < iters; ++i) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) s += c0[j] + c1[j] + c2[j] + c3[j];
  } else {
    v4f c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int i = 0; i < iters; ++i) {
      c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c3, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) s += c0[j] + c1[j] + c2[j] + c3[j];
  }
  sink[blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ __launch_bounds__(1024) void k_peak_empty(uint32_t* sink) {
  if (threadIdx.x == 1023u && blockIdx.x == 0xffffffu) sink[0] = 1u;
}

#define PK_ADD4                                                                                  \
  asm volatile("v_add_u32 %0, %0, %4\n\tv_add_u32 %1, %1, %4\n\tv_add_u32 %2, %2, %4\n\tv_add_u32 %3, %3, %4" \
               : "+v"(x0), "+v"(x1), "+v"(x2), "+v"(x3)                                           \
               : "v"(y));
#define PK_ADD16 PK_ADD4 PK_ADD4 PK_ADD4 PK_ADD4
#define PK_ADD64 PK_ADD16 PK_ADD16 PK_ADD16 PK_ADD16
__global__ __launch_bounds__(1024) void k_peak_valu(int iters, uint32_t y, uint32_t* sink) {
  uint32_t x0 = threadIdx.x, x1 = x0 + 1u, x2 = x0 + 2u, x3 = x0 + 3u;
  for (int i = 0; i < iters; ++i) {
    PK_ADD64 PK_ADD64 PK_ADD64 PK_ADD64
  }
  if ((x0 ^ x1 ^ x2 ^ x3) == 0xdeadbeefu) sink[0] = x0;
}

template <typename... P>
static int go(void (*k)(P...), dim3 grid, void* start, void* stop, void* stream, P... args) {
  void* a[] = {(void*)&args..., nullptr};
  const hipError_t e = hipExtLaunchKernel((const void*)k, grid, dim3(256), a, 0, (hipStream_t)stream,
                                          (hipEvent_t)start, (hipEvent_t)stop, 0);
  return e == hipSuccess ? 0 : -1;
}

extern "C" {

// sink: device word (written only if an impossible value comes out)
int peak_valu(int grid, int block, int iters, uint32_t* sink, void* start, void* stop, void* stream) {
  if (grid < 1 || block < 1 || block > 1024 || iters < 1 || !sink) return -1;
  uint32_t y = 1u;
  void* a[] = {(void*)&iters, (void*)&y, (void*)&sink, nullptr};
  const hipError_t e = hipExtLaunchKernel((const void*)k_peak_valu, dim3(grid), dim3(block), a, 0,
                                          (hipStream_t)stream, (hipEvent_t)start, (hipEvent_t)stop, 0);
  return e == hipSuccess ? 0 : -1;
}

// sink: device word (never written); workgroups of `block` threads (<= 1024)
int peak_empty(int grid, int block, uint32_t* sink, void* start, void* stop, void* stream) {
  if (grid < 1 || block < 1 || block > 1024 || !sink) return -1;
  void* a[] = {(void*)&sink, nullptr};
  const hipError_t e = hipExtLaunchKernel((const void*)k_peak_empty, dim3(grid), dim3(block), a, 0,
                                          (hipStream_t)stream, (hipEvent_t)start, (hipEvent_t)stop, 0);
  return e == hipSuccess ? 0 : -1;
}

// buf: device, bytes a multiple of 16; sink: device, >= grid words; unroll 4, 8 or 16
int peak_read(const void* buf, size_t bytes, int grid, int unroll, uint32_t* sink, void* start, void* stop,
              void* stream) {
  if (!buf || !sink || bytes % 16 != 0 || grid < 1) return -1;
  const uint4* p = (const uint4*)buf;
  const size_t n16 = bytes / 16;
  if (unroll == 4) return go(k_peak_read<4>, dim3(grid), start, stop, stream, p, n16, sink);
  if (unroll == 16) return go(k_peak_read<16>, dim3(grid), start, stop, stream, p, n16, sink);
  return go(k_peak_read<8>, dim3(grid), start, stop, stream, p, n16, sink);
}

// the same with each workgroup reading its own contiguous span (bytes / grid,
// rounded up to 4 KB)
int peak_read_chunked(const void* buf, size_t bytes, int grid, int unroll, uint32_t* sink, void* start, void* stop,
                      void* stream) {
  if (!buf || !sink || bytes % 16 != 0 || grid < 1) return -1;
  const uint4* p = (const uint4*)buf;
  const size_t n16 = bytes / 16;
  const size_t chunk16 = ((n16 + grid - 1) / grid + 255) / 256 * 256;
  if (unroll == 4) return go(k_peak_read_chunk<4>, dim3(grid), start, stop, stream, p, n16, chunk16, sink);
  if (unroll == 16) return go(k_peak_read_chunk<16>, dim3(grid), start, stop, stream, p, n16, chunk16, sink);
  return go(k_peak_read_chunk<8>, dim3(grid), start, stop, stream, p, n16, chunk16, sink);
}

// sink: device, >= grid * 256 floats.  FLOPs = grid * 4 waves * iters * 4 * 2*32*32*64.
int peak_mfma_fp4(int grid, int iters, float* sink, void* start, void* stop, void* stream) {
  if (!sink || grid < 1 || iters < 1) return -1;
  return go(k_peak_fp4, dim3(grid), start, stop, stream, iters, sink);
}

// big = 1: 32x32x16 (FLOPs = grid * 4 * iters * 4 * 2*32*32*16); big = 0: 16x16x32 (2*16*16*32 each)
int peak_mfma_bf16(int grid, int iters, int big, float* sink, void* start, void* stop, void* stream) {
  if (!sink || grid < 1 || iters < 1) return -1;
  if (big) return go(k_peak_bf16<true>, dim3(grid), start, stop, stream, iters, sink);
  return go(k_peak_bf16<false>, dim3(grid), start, stop, stream, iters, sink);
}

}  // extern "C"

// Device-side helpers shared by the libcsa kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// threadIdx.x behind an opaque move: values derived from it are formed where
// they are used instead of being hoisted out of a long outer loop and held in
// registers across all of it
__device__ __forceinline__ int lane_tid() {
  int t = (int)threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16 bits, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

#ifdef CSA_DEBUG
// Debug builds (libcsa_debug.so): kernels check device-side indices before
// they use them and count each violation here (one counter per translation
// unit) instead of reading out of range; csa_debug_checks reads and clears
// the counters.  Release builds compile none of this.
static __device__ unsigned long long g_debug_violations;
__device__ __forceinline__ void debug_violation() { atomicAdd(&g_debug_violations, 1ull); }
// this translation unit's count since the last call, then cleared (synchronous)
static inline unsigned long long debug_take_here() {
  unsigned long long v = 0, z = 0;
  if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_debug_violations), sizeof(v)) != hipSuccess) return ~0ull;
  if (hipMemcpyToSymbol(HIP_SYMBOL(g_debug_violations), &z, sizeof(z)) != hipSuccess) return ~0ull;
  return v;
}
#endif

// Head weight folded into a query block's E8M0 scale: w = 2^e multiplies
// every product of the block, so the block's scale byte becomes qscale + e.
// `u` holds the block's 32 e2m1 codes.  The byte is clamped to E8M0's finite
// range [0, 254], so no 0xFF (NaN) reaches the MFMA: a block whose codes are
// all zero then still adds exactly 0, and a fold of a block with a non-zero
// code that leaves the range is outside the indexer's exactness precondition
// (scales within a few octaves of each other).  A zero weight zeroes the
// codes (its head adds nothing).  The scale depends on the scale byte and the
// weight only, not on the codes, so it never waits for the code load.
__device__ __forceinline__ int fold_head_weight(uint4& u, int qscale, float w) {
  const int wexp = (int)((__float_as_uint(w) >> 23) & 255u);
  if (wexp == 0) u = make_uint4(0u, 0u, 0u, 0u);
  const int e = qscale + wexp - 127;
  return e < 0 ? 0 : (e > 254 ? 254 : e);
}

// Wave-wide inclusive scans on DPP lane moves (row shifts within 16-lane rows,
// then the row broadcasts of lanes 15 and 31): a few VALU operations instead
// of LDS permutes.  Lanes whose source is outside the row take the identity.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t identity, uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)identity, (int)x, CTRL, ROWS, 0xf, false);
}
__device__ __forceinline__ uint32_t wave_incl_add(uint32_t x) {
  x += dpp_mov<0x111>(0u, x);        // row_shr:1
  x += dpp_mov<0x112>(0u, x);        // row_shr:2
  x += dpp_mov<0x114>(0u, x);        // row_shr:4
  x += dpp_mov<0x118>(0u, x);        // row_shr:8
  x += dpp_mov<0x142, 0xa>(0u, x);   // row_bcast:15 -> rows 1, 3
  x += dpp_mov<0x143, 0xc>(0u, x);   // row_bcast:31 -> rows 2, 3
  return x;
}
// wave-wide min and max of x, on every lane
__device__ __forceinline__ void wave_minmax(uint32_t& mn, uint32_t& mx) {
#define CSA_MM_STEP(CTRL, ROWS)                                    \
  {                                                                \
    const uint32_t a_ = dpp_mov<CTRL, ROWS>(0xffffffffu, mn);      \
    const uint32_t b_ = dpp_mov<CTRL, ROWS>(0u, mx);               \
    mn = a_ < mn ? a_ : mn;                                        \
    mx = b_ > mx ? b_ : mx;                                        \
  }
  CSA_MM_STEP(0x111, 0xf) CSA_MM_STEP(0x112, 0xf) CSA_MM_STEP(0x114, 0xf) CSA_MM_STEP(0x118, 0xf)
  CSA_MM_STEP(0x142, 0xa) CSA_MM_STEP(0x143, 0xc)
#undef CSA_MM_STEP
  mn = (uint32_t)__builtin_amdgcn_readlane((int)mn, 63);
  mx = (uint32_t)__builtin_amdgcn_readlane((int)mx, 63);
}

// sequence index of query row `row` given q_off[0..n_seq] (binary search)
__device__ __forceinline__ int seq_of_row(const int64_t* q_off, int n_seq, int64_t row) {
  int lo = 0, hi = n_seq - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (q_off[mid] <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Block-wide search from the top.  Thread t holds the count c of its bin
// range; ranges ascend with t.  Returns in *found (on every thread) the
// thread t* whose range contains the need-th element counted from the top
// (sum over t > t* of c < need <= sum over t >= t*), and in *above that sum
// over t > t*.  Requires blockDim.x % 64 == 0 and total >= need.  `scratch`
// holds at least blockDim.x / 64 + 2 words of LDS.
__device__ __forceinline__ void block_find_from_top(uint32_t c, uint32_t need, uint32_t* scratch,
                                                    int* found, uint32_t* above) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, nw = blockDim.x >> 6;
  uint32_t s = c;  // inclusive suffix sum within the wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t v = __shfl_down(s, off);
    if (lane + off < 64) s += v;
  }
  if (lane == 0) scratch[wave] = s;
  __syncthreads();
  uint32_t higher = 0;
  for (int w = wave + 1; w < nw; ++w) higher += scratch[w];
  const uint32_t incl = s + higher, excl = incl - c;
  if (excl < need && incl >= need) {
    scratch[nw] = (uint32_t)t;
    scratch[nw + 1] = excl;
  }
  __syncthreads();
  *found = (int)scratch[nw];
  *above = scratch[nw + 1];
  __syncthreads();
}

}  // namespace csa

// Pooling of one block of m raw rows into one row (shared by the bulk pooling
// kernel and the streaming cache append, so both produce identical rows).
//
// Pages: pytorch.kr DeepSeek-V4 summary, CSA/HCA section (m consecutive KV
// entries merged into one; m' >> m for HCA).  Rule (the reading taken): for
// each channel c, out[c] = sum_i softmax_i(z_i[c]) * x_i[c], in fp32 with the
// hardware exp2, rounded once at the store.  A thread owns 16 bytes of
// channels (8 bf16 or 4 fp32) of the row.
#pragma once
#include "common.hpp"

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

// 4 bytes of a row (2 bf16 channels or 1 fp32 channel), as a raw word
template <bool BF16>
struct Vec4 {
  static constexpr int N = BF16 ? 2 : 1;
  __device__ static void load(uint32_t u, float* v) {
    if constexpr (BF16) {
      v[0] = __uint_as_float(u << 16);
      v[1] = __uint_as_float(u & 0xffff0000u);
    } else {
      v[0] = __uint_as_float(u);
    }
  }
  __device__ static uint32_t pack(const float* v) {
    if constexpr (BF16) return f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
    else return __float_as_uint(v[0]);
  }
};

// A loaded value that a path does not use is still consumed here (the empty
// asm reads the register, so the compiler waits for the load), so that no
// load is left in flight with its result unused.
__device__ __forceinline__ void consume_load(uint32_t v) { asm volatile("" ::"v"(v)); }

// Pooling state of N channels: running max, denominator, weighted sum.
template <int N>
struct PoolSt {
  float mx[N], den[N], acc[N];
};
template <bool BF16>
using PoolState = PoolSt<Vec16<BF16>::N>;

// A block is pooled in segments of kPoolSeg rows: each segment with an online
// softmax over chunks of up to 8 rows, then the segments folded left to right.
// The bulk kernel folds them in one thread; the streaming append pools the
// segments of a long block in parallel and folds them in the same order, so
// both give the same bits.  Every operation is per channel, so a thread
// holding N channels computes each of them exactly as a thread holding any
// other number of them does.
constexpr int kPoolSeg = 16;

template <int N>
__device__ __forceinline__ void pool_reset(PoolSt<N>& st) {
#pragma unroll
  for (int c = 0; c < N; ++c) { st.mx[c] = -INFINITY; st.den[c] = 0.f; st.acc[c] = 0.f; }
}

// one chunk of n <= 8 rows (logits zz, values xx) into the state: the online
// softmax step every pooling path uses, so all of them give the same bits
template <int N>
__device__ __forceinline__ void pool_chunk(PoolSt<N>& st, const float (&zz)[8][N], const float (&xx)[8][N], int n) {
#pragma unroll
  for (int c = 0; c < N; ++c) {
    float cm = st.mx[c];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i < n) cm = fmaxf(cm, zz[i][c]);
    const float alpha = fast_exp2((st.mx[c] - cm) * kLog2e);  // exp2(-inf) = 0 on the first chunk
    float d = st.den[c] * alpha, a = st.acc[c] * alpha;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i < n) {
        const float e = fast_exp2((zz[i][c] - cm) * kLog2e);
        d += e;
        a = fmaf(e, xx[i][c], a);
      }
    }
    st.mx[c] = cm; st.den[c] = d; st.acc[c] = a;
  }
}

// rows [i0, i1) of the block (1 <= i1 - i0 <= kPoolSeg) -> a fresh state
template <bool BF16, class XRow, class ZRow>
__device__ __forceinline__ void pool_segment(int i0, int i1, XRow xrow, ZRow zrow, PoolState<BF16>& st) {
  using V = Vec16<BF16>;
  constexpr int N = V::N;
  pool_reset(st);
  for (int c0 = i0; c0 < i1; c0 += 8) {
    const int n = (i1 - c0) < 8 ? (i1 - c0) : 8;
    float zz[8][N], xx[8][N];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i < n) {
        V::load(zrow(c0 + i), zz[i]);
        V::load(xrow(c0 + i), xx[i]);
      }
    }
    pool_chunk(st, zz, xx, n);
  }
}

// st <- st folded with the next segment t
template <int N>
__device__ __forceinline__ void pool_fold(PoolSt<N>& st, const PoolSt<N>& t) {
#pragma unroll
  for (int c = 0; c < N; ++c) {
    const float M = fmaxf(st.mx[c], t.mx[c]);
    const float a1 = fast_exp2((st.mx[c] - M) * kLog2e), a2 = fast_exp2((t.mx[c] - M) * kLog2e);
    st.den[c] = st.den[c] * a1 + t.den[c] * a2;
    st.acc[c] = st.acc[c] * a1 + t.acc[c] * a2;
    st.mx[c] = M;
  }
}

// the pooled values of the state's channels
template <int N>
__device__ __forceinline__ void pool_result(const PoolSt<N>& st, float (&o)[N]) {
#pragma unroll
  for (int c = 0; c < N; ++c) o[c] = st.acc[c] / st.den[c];
}
template <bool BF16>
__device__ __forceinline__ void pool_store(const PoolState<BF16>& st, uint8_t* out) {
  float o[Vec16<BF16>::N];
  pool_result(st, o);
  Vec16<BF16>::store(out, o);
}

// xrow(i), zrow(i): this thread's 16 bytes of row i < m of the block's values
// and logits; the whole block in this thread
template <bool BF16, class XRow, class ZRow>
__device__ __forceinline__ void pool_block(int m, XRow xrow, ZRow zrow, uint8_t* out) {
  PoolState<BF16> st;
  pool_segment<BF16>(0, m < kPoolSeg ? m : kPoolSeg, xrow, zrow, st);
  for (int s0 = kPoolSeg; s0 < m; s0 += kPoolSeg) {
    PoolState<BF16> t;
    pool_segment<BF16>(s0, m - s0 < kPoolSeg ? m : s0 + kPoolSeg, xrow, zrow, t);
    pool_fold(st, t);
  }
  pool_store<BF16>(st, out);
}

}  // namespace csa

// MQA attention tile loop on bf16 MFMA, shared by the attention kernels.
//
// One workgroup of 4 waves; wave w owns query-head groups w, w+4, ... (16
// heads each, GPW groups per wave).  A list of key rows ([2][128] bf16: K then
// V) is walked in 64-key tiles: K staged row-major and V transposed in LDS,
// S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_16x16x32_bf16 with fp32
// accumulation and an online softmax in base 2.  The P^T operand uses the key
// order 8g+i <-> 32*kq + (i < 4 ? 4g+i : 16+4g+i-4), which is exactly the set
// of keys each lane already holds in the S^T output, so no shuffles are
// needed.  The next tile's rows are loaded into registers while the current
// tile is computed.
#pragma once
#include "common.hpp"

namespace csa {

constexpr int kKStride = 136;  // LDS row stride (elements) of the K tile
constexpr int kVStride = 72;   // LDS row stride (elements) of the transposed V tile
constexpr int kAttnLdsBytes = 64 * kKStride * 2 + 128 * kVStride * 2 + 64;  // K, V^T, valid flags

template <int GPW>
struct AttnState {
  v8bf qf[GPW][4];
  float m_run[GPW], l_run[GPW];
  v4f O[GPW][8];
};

// q_row: this query's [H][128] bf16 heads.
template <int GPW>
__device__ __forceinline__ void attn_init(AttnState<GPW>& st, const uint8_t* q_row, int H) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l16 = lane & 15, g = lane >> 4;
  const int HG = H >> 4;
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    const int hg = wave + 4 * gi;
    st.m_run[gi] = -INFINITY;
    st.l_run[gi] = 0.f;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) st.O[gi][mt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) {
      if (hg < HG) {
        const uint8_t* qp = q_row + ((size_t)(16 * hg + l16) * 128 + 32 * kq + 8 * g) * 2;
        st.qf[gi][kq] = *reinterpret_cast<const v8bf*>(qp);
      } else {
        st.qf[gi][kq] = v8bf{};
      }
    }
  }
}

// Walk list positions [p_begin, p_end); rowptr(p) gives the [2][128] bf16 row
// of position p or nullptr when masked.  lds: kAttnLdsBytes bytes, 16-aligned.
template <int GPW, class RowPtr>
__device__ __forceinline__ void attn_run(AttnState<GPW>& st, int H, float scale_log2, int64_t p_begin,
                                         int64_t p_end, RowPtr rowptr, uint8_t* lds) {
  uint16_t* Ks = reinterpret_cast<uint16_t*>(lds);
  uint16_t* Vt = Ks + 64 * kKStride;
  uint8_t* valid_s = reinterpret_cast<uint8_t*>(Vt + 128 * kVStride);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int HG = H >> 4;
  const int ch = tid & 15;  // staging: 16-byte chunk ch of keys 2*kp, 2*kp+1, kp in {tid/16, tid/16+16}
  uint4 kr[2][2], vr[2][2];
  bool vl[2][2];
  auto load_tile = [&](int64_t p0) {
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int64_t p = p0 + 2 * ((tid >> 4) + 16 * r) + e;
        const uint8_t* rp = p < p_end ? rowptr(p) : nullptr;
        vl[r][e] = rp != nullptr;
        if (rp) {
          kr[r][e] = *reinterpret_cast<const uint4*>(rp + ch * 16);
          vr[r][e] = *reinterpret_cast<const uint4*>(rp + 256 + ch * 16);
        } else {
          kr[r][e] = make_uint4(0, 0, 0, 0);
          vr[r][e] = make_uint4(0, 0, 0, 0);
        }
      }
  };
  if (p_begin < p_end) load_tile(p_begin);

  for (int64_t p0 = p_begin; p0 < p_end; p0 += 64) {
    __syncthreads();  // the previous tile's LDS reads are done
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int kp = (tid >> 4) + 16 * r;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        *reinterpret_cast<uint4*>(&Ks[(2 * kp + e) * kKStride + ch * 8]) = kr[r][e];
        if (ch == 0) valid_s[2 * kp + e] = vl[r][e] ? 1 : 0;
      }
      const uint32_t v0[4] = {vr[r][0].x, vr[r][0].y, vr[r][0].z, vr[r][0].w};
      const uint32_t v1[4] = {vr[r][1].x, vr[r][1].y, vr[r][1].z, vr[r][1].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t lo = (v0[q] & 0xffffu) | (v1[q] << 16);
        const uint32_t hi = (v0[q] >> 16) | (v1[q] & 0xffff0000u);
        *reinterpret_cast<uint32_t*>(&Vt[(ch * 8 + 2 * q) * kVStride + 2 * kp]) = lo;
        *reinterpret_cast<uint32_t*>(&Vt[(ch * 8 + 2 * q + 1) * kVStride + 2 * kp]) = hi;
      }
    }
    __syncthreads();
    if (p0 + 64 < p_end) load_tile(p0 + 64);  // next tile's loads fly during this tile's math

#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) {
      const int hg = wave + 4 * gi;
      if (hg >= HG) continue;
      float s[4][4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kq = 0; kq < 4; ++kq) {
          const v8bf kf = *reinterpret_cast<const v8bf*>(&Ks[(16 * mt + l16) * kKStride + 32 * kq + 8 * g]);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, st.qf[gi][kq], acc, 0, 0, 0);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v)
          s[mt][v] = valid_s[16 * mt + 4 * g + v] ? acc[v] * scale_log2 : -INFINITY;
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) tmax = fmaxf(tmax, s[mt][v]);
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float mnew = fmaxf(st.m_run[gi], tmax);
      if (mnew == -INFINITY) continue;  // nothing valid so far (uniform: validity is per key)
      const float alpha = fast_exp2(st.m_run[gi] - mnew);
      st.m_run[gi] = mnew;
      float psum = 0.f;
      float pv[4][4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          pv[mt][v] = fast_exp2(s[mt][v] - mnew);
          psum += pv[mt][v];
        }
      st.l_run[gi] = st.l_run[gi] * alpha + psum;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) st.O[gi][mt] *= alpha;
#pragma unroll
      for (int kq = 0; kq < 2; ++kq) {
        v8bf pf;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pf[i] = (__bf16)pv[2 * kq][i];
          pf[4 + i] = (__bf16)pv[2 * kq + 1][i];
        }
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
          const uint16_t* vrow = &Vt[(16 * mt + l16) * kVStride + 32 * kq + 4 * g];
          const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
          const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 16);
          uint4 u = make_uint4(lo.x, lo.y, hi.x, hi.y);
          const v8bf vf = *reinterpret_cast<const v8bf*>(&u);
          st.O[gi][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, st.O[gi][mt], 0, 0, 0);
        }
      }
    }
  }
}

// Finish: normalised bf16 output [H][128] and lse (natural log), or, when
// `partial` is set, the unnormalised (m in log2 units, l, O) partial through
// device-coherent stores if `coherent` (read by other workgroups in the same
// launch) or plain stores.  Lane (l16, g) holds head 16*hg + l16, dims
// 16*mt + 4*g + v.
template <int GPW>
__device__ __forceinline__ void attn_finish(AttnState<GPW>& st, int H, uint8_t* out_row, float* lse_row,
                                            float* part_o, float* part_ml, bool partial, bool coherent) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l16 = lane & 15, g = lane >> 4;
  const int HG = H >> 4;
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    const int hg = wave + 4 * gi;
    if (hg >= HG) continue;
    float l = st.l_run[gi];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const int head = 16 * hg + l16;
    if (!partial) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
      uint8_t* op = out_row + (size_t)head * 128 * 2;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const int d0 = 16 * mt + 4 * g;
        uint2 u;
        u.x = f32_to_bf16(st.O[gi][mt][0] * inv) | (f32_to_bf16(st.O[gi][mt][1] * inv) << 16);
        u.y = f32_to_bf16(st.O[gi][mt][2] * inv) | (f32_to_bf16(st.O[gi][mt][3] * inv) << 16);
        *reinterpret_cast<uint2*>(op + d0 * 2) = u;
      }
      if (lse_row && g == 0) lse_row[head] = l > 0.f ? (st.m_run[gi] + __log2f(l)) * kLn2 : -INFINITY;
    } else {
      float* op = part_o + (size_t)head * 128;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        float* dst = op + 16 * mt + 4 * g;
        if (coherent) {
#pragma unroll
          for (int v = 0; v < 4; ++v)
            __hip_atomic_store(reinterpret_cast<uint32_t*>(dst + v), __float_as_uint(st.O[gi][mt][v]),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
          *reinterpret_cast<v4f*>(dst) = st.O[gi][mt];
        }
      }
      if (g == 0) {
        if (coherent) {
          __hip_atomic_store(reinterpret_cast<uint32_t*>(part_ml + head * 2), __float_as_uint(st.m_run[gi]),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(reinterpret_cast<uint32_t*>(part_ml + head * 2 + 1), __float_as_uint(l),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
          part_ml[head * 2] = st.m_run[gi];
          part_ml[head * 2 + 1] = l;
        }
      }
    }
  }
}

}  // namespace csa

// MQA attention tile loop on bf16 MFMA, shared by the attention kernels.
//
// One workgroup of 4 waves; wave w owns query-head groups w, w+4, ... (16
// heads each, GPW groups per wave).  attn_run_q2 serves two queries of one
// sequence over one key list instead: wave w owns head group w of both, and
// each K and V fragment read from LDS feeds both queries' MFMAs (half the
// LDS reads per FLOP); per-query limits mask the list positions beyond each
// query's visible range.  A list of key rows ([2][128] bf16: K then
// V, 512 B) is walked in 64-key tiles.  Tiles go from memory straight into LDS
// (global_load_lds_dwordx4, no register staging) through NST stages: while
// tile t is computed, tiles t+1 .. t+NST-1 are in flight.
//
// LDS stage layout (32 KB): row r (key), 16-byte chunk c (0..15 K, 16..31 V)
// lives at ((c/4)*4 + r/16) KB + (r%16)*64 + (c%4)*16.  One DMA instruction of
// wave w writes 1 KB: lane L carries row 16w + L/4, chunk 4i + L%4 of
// instruction i, so each lane needs one row address per tile.  With this
// layout both the K fragment reads and the V transpose reads stay inside one
// 1 KB block per instruction.
//
// Per tile and head group: S^T = K Q^T (v_mfma_f32_16x16x32_bf16, K rows as
// the A operand), an online softmax in base 2, then O^T += V^T P^T.  The V^T
// operand comes from the row-major V chunks through ds_read_b64_tr_b16: in
// each 16-lane group, lane a addresses row (key0 + a/4), dims dim0 + 4(a%4)
// and lane j receives dims dim0 + j of keys key0 .. key0+3.  The P^T operand
// uses the key order 8g+i <-> 32*kq + (i < 4 ? 4g+i : 16+4g+i-4), exactly the
// keys each lane already holds in the S^T output, so P needs no shuffles; the
// head-wise max and sum over the four lane groups use v_permlane16_swap and
// v_permlane32_swap.  The running max is only raised (and O, l rescaled) when
// a tile's max exceeds it by more than 2^8, so most tiles skip the rescale;
// the normalised result does not depend on which max is used.  Masked keys
// read a zero row and are excluded through one 64-bit validity word per tile.
#pragma once
#include "common.hpp"

namespace csa {

constexpr int kTileKeys = 64;
constexpr int kStageBytes = kTileKeys * 512;
constexpr int kLazyRescale = 8;  // log2 headroom before the running max is raised

template <int NST>
constexpr int attn_lds_bytes() { return NST * kStageBytes + 8 * NST; }
constexpr int kAttnStages = 2;
constexpr int kAttnLdsBytes = attn_lds_bytes<kAttnStages>();

// A 512-byte row of zeros in device memory (never written): the source of
// masked key rows.
static __device__ __align__(256) uint8_t g_zero_row[512];

template <int GPW>
struct AttnState {
  v8bf qf[GPW][4];
  float m_run[GPW], l_run[GPW];
  v4f O[GPW][8];
};

typedef short v4s_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 16 bytes per lane from global memory to LDS address m0 + 16*lane + OFF
// (and global address + OFF).  The compiler does not see this write: callers
// order it with attn_wait_dma and a barrier.
template <int OFF>
__device__ __forceinline__ void dma16(const uint8_t* gaddr, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off offset:%2"
               :
               : "s"(m0), "v"(gaddr), "i"(OFF)
               : "memory");
}
// at most N of this wave's memory operations still outstanding
template <int N>
__device__ __forceinline__ void attn_wait_dma() {
  if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
}

// q_row: this query's [H][128] bf16 heads.
template <int GPW>
__device__ __forceinline__ void attn_init(AttnState<GPW>& st, const uint8_t* q_row, int H) {
  const int lane = lane_tid() & 63, wave = lane_tid() >> 6, l16 = lane & 15, g = lane >> 4;
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

// DMA of tile t of list positions [p_begin, p_end) into stage s: wave w
// stages rows 16w .. 16w+15 (lane: row 16w + lane/4, chunks 4i + lane%4 of
// instruction i) and writes their validity bits to the stage's mask word.
template <class RowPtr>
__device__ __forceinline__ void attn_issue_tile(int64_t p_begin, int64_t p_end, int64_t t, int s, RowPtr& rowptr,
                                                uint32_t lds_base, uint64_t* masks) {
  const int lane = lane_tid() & 63, wave = lane_tid() >> 6;
  const int row = 16 * wave + (lane >> 2);
  const int64_t p = p_begin + t * kTileKeys + row;
  const uint8_t* rp = p < p_end ? rowptr(p) : nullptr;
  const uint64_t vb = __ballot(rp != nullptr);
  const uint8_t* src = (rp ? rp : g_zero_row) + 16 * (lane & 3);
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_base + (uint32_t)(s * kStageBytes + wave * 1024));
  dma16<0>(src, m0);
  dma16<64>(src, m0 + 4 * 1024 - 64);
  dma16<128>(src, m0 + 8 * 1024 - 128);
  dma16<192>(src, m0 + 12 * 1024 - 192);
  dma16<256>(src, m0 + 16 * 1024 - 256);
  dma16<320>(src, m0 + 20 * 1024 - 320);
  dma16<384>(src, m0 + 24 * 1024 - 384);
  dma16<448>(src, m0 + 28 * 1024 - 448);
  // rows 16w .. 16w+15 valid bits: lanes 4j
  uint32_t m16 = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) m16 |= (uint32_t)((vb >> (4 * j)) & 1ull) << j;
  if (lane == 0) reinterpret_cast<uint16_t*>(masks + s)[wave] = (uint16_t)m16;
}

// the tile's V^T fragments (lane (l16, g): see the layout notes above)
__device__ __forceinline__ void attn_vt(const uint8_t* cur, int l16, int g, v4s_t (&vt)[8][2][2]) {
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int kq = 0; kq < 2; ++kq)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int a3 = l16 & 3;
        const int off = ((4 + (mt >> 1)) * 4 + 2 * kq + hh) * 1024 + (4 * g + (l16 >> 2)) * 64 +
                        (2 * (mt & 1) + (a3 >> 1)) * 16 + (a3 & 1) * 8;
        vt[mt][kq][hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4s_t*)(const_cast<uint8_t*>(cur) + off));
      }
}

// masked online softmax of one tile's scores and O^T += V^T P^T for one
// group (the same steps as attn_run's, for attn_run_q2)
__device__ __forceinline__ void attn_softmax_pv(float& m_run, float& l_run, v4f (&O)[8], float (&s_)[4][4],
                                                const v4s_t (&vt)[8][2][2], uint64_t vmask, int g,
                                                float scale_log2) {
  if (vmask != ~0ull) {
    const uint64_t my = vmask >> (4 * g);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (!((my >> (16 * mt + v)) & 1ull)) s_[mt][v] = -INFINITY;
  }
  float tmax = -INFINITY;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int v = 0; v < 4; ++v) tmax = fmaxf(tmax, s_[mt][v]);
  tmax = xor32_max(xor16_max(tmax)) * scale_log2;
  if (__ballot(tmax > m_run + (float)kLazyRescale) != 0ull) {
    const float mnew = fmaxf(m_run, tmax);
    const float alpha = fast_exp2(m_run - mnew);  // 0 while nothing was valid
    m_run = mnew;
    l_run *= alpha;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) O[mt] *= alpha;
  }
  if (m_run == -INFINITY) return;  // nothing valid so far (uniform: validity is per key)
  const float mneg = -m_run;
  float psum = 0.f;
  float pv[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      pv[mt][v] = fast_exp2(fmaf(s_[mt][v], scale_log2, mneg));
      psum += pv[mt][v];
    }
  l_run += psum;
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
      const v4s_t both[2] = {vt[mt][kq][0], vt[mt][kq][1]};
      const v8bf vf = *reinterpret_cast<const v8bf*>(both);
      O[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, O[mt], 0, 0, 0);
    }
  }
}

// Walk list positions [p_begin, p_end); rowptr(p) gives the [2][128] bf16 row
// of position p or nullptr when masked.  lds: attn_lds_bytes<NST>() bytes,
// 16-aligned.  Must be called by the whole workgroup; no memory operation of
// the calling thread may be outstanding on entry (the DMA count relies on it).
template <int GPW, int NST = kAttnStages, class RowPtr>
__device__ __forceinline__ void attn_run(AttnState<GPW>& st, int H, float scale_log2, int64_t p_begin,
                                         int64_t p_end, RowPtr rowptr, uint8_t* lds) {
  static_assert(NST == 2 || NST == 3, "two or three stages");
  const int tid = lane_tid(), lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int HG = H >> 4;
  if (p_begin >= p_end) return;
  const int64_t n_tiles = (p_end - p_begin + kTileKeys - 1) / kTileKeys;
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds;
  uint64_t* masks = reinterpret_cast<uint64_t*>(lds + NST * kStageBytes);

  // DMA of tile t into stage s: row 16*wave + lane/4, chunks 4i + lane%4
  auto issue = [&](int64_t t, int s) {
    const int row = 16 * wave + (lane >> 2);
    const int64_t p = p_begin + t * kTileKeys + row;
    const uint8_t* rp = p < p_end ? rowptr(p) : nullptr;
    const uint64_t vb = __ballot(rp != nullptr);
    const uint8_t* src = (rp ? rp : g_zero_row) + 16 * (lane & 3);
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_base + (uint32_t)(s * kStageBytes + wave * 1024));
    dma16<0>(src, m0);
    dma16<64>(src, m0 + 4 * 1024 - 64);
    dma16<128>(src, m0 + 8 * 1024 - 128);
    dma16<192>(src, m0 + 12 * 1024 - 192);
    dma16<256>(src, m0 + 16 * 1024 - 256);
    dma16<320>(src, m0 + 20 * 1024 - 320);
    dma16<384>(src, m0 + 24 * 1024 - 384);
    dma16<448>(src, m0 + 28 * 1024 - 448);
    // rows 16w .. 16w+15 valid bits: lanes 4j
    uint32_t m16 = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) m16 |= (uint32_t)((vb >> (4 * j)) & 1ull) << j;
    if (lane == 0) reinterpret_cast<uint16_t*>(masks + s)[wave] = (uint16_t)m16;
  };

  issue(0, 0);
  if (n_tiles > 1) issue(1, 1);
  if (NST == 3 && n_tiles > 2) issue(2, 2);

  for (int64_t t = 0; t < n_tiles; ++t) {
    const int s = (int)(t % NST);
    const int64_t ahead = n_tiles - 1 - t < NST - 1 ? n_tiles - 1 - t : NST - 1;  // tiles issued after t
    if (ahead >= 2) attn_wait_dma<16>();
    else if (ahead == 1) attn_wait_dma<8>();
    else attn_wait_dma<0>();
    __syncthreads();  // every wave's part of tile t is in LDS (with its validity word)
    const uint8_t* cur = lds + s * kStageBytes;
    const uint64_t vmask = masks[s];

#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) {
      const int hg = wave + 4 * gi;
      if (hg >= HG) continue;
      // S^T: 64 keys x 16 heads; lane holds keys 16 mt + 4 g + v of head l16
      v8bf kf[4][4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int kq = 0; kq < 4; ++kq)
          kf[mt][kq] = *reinterpret_cast<const v8bf*>(cur + (kq * 4 + mt) * 1024 + l16 * 64 + g * 16);
      float s_[4][4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kq = 0; kq < 4; ++kq)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[mt][kq], st.qf[gi][kq], acc, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < 4; ++v) s_[mt][v] = acc[v];
      }
      // V^T fragments, requested before the softmax math
      v4s_t vt[8][2][2];
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int kq = 0; kq < 2; ++kq)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int a3 = l16 & 3;
            const int off = ((4 + (mt >> 1)) * 4 + 2 * kq + hh) * 1024 + (4 * g + (l16 >> 2)) * 64 +
                            (2 * (mt & 1) + (a3 >> 1)) * 16 + (a3 & 1) * 8;
            vt[mt][kq][hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4s_t*)(const_cast<uint8_t*>(cur) + off));
          }
      if (vmask != ~0ull) {
        const uint64_t my = vmask >> (4 * g);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (!((my >> (16 * mt + v)) & 1ull)) s_[mt][v] = -INFINITY;
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) tmax = fmaxf(tmax, s_[mt][v]);
      tmax = xor32_max(xor16_max(tmax)) * scale_log2;
      if (__ballot(tmax > st.m_run[gi] + (float)kLazyRescale) != 0ull) {
        const float mnew = fmaxf(st.m_run[gi], tmax);
        const float alpha = fast_exp2(st.m_run[gi] - mnew);  // 0 while nothing was valid
        st.m_run[gi] = mnew;
        st.l_run[gi] *= alpha;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) st.O[gi][mt] *= alpha;
      }
      if (st.m_run[gi] == -INFINITY) continue;  // nothing valid so far (uniform: validity is per key)
      const float mneg = -st.m_run[gi];
      float psum = 0.f;
      float pv[4][4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          pv[mt][v] = fast_exp2(fmaf(s_[mt][v], scale_log2, mneg));
          psum += pv[mt][v];
        }
      st.l_run[gi] += psum;
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
          const v4s_t both[2] = {vt[mt][kq][0], vt[mt][kq][1]};
          const v8bf vf = *reinterpret_cast<const v8bf*>(both);
          st.O[gi][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, st.O[gi][mt], 0, 0, 0);
        }
      }
    }
    if (t + NST < n_tiles) {
      __syncthreads();  // stage s is read out by every wave
      issue(t + NST, s);
    }
  }
  __syncthreads();  // LDS free for the caller
}

// Two queries of one sequence over one key list (positions [0, p_end)): group
// gi of `st` is query gi's head group `wave`; query gi sees positions < lim[gi]
// only.  Each K fragment feeds both queries' S^T MFMAs and each V^T fragment
// both PV products.  Same entry conditions as attn_run.
template <int NST = kAttnStages, class RowPtr>
__device__ __forceinline__ void attn_run_q2(AttnState<2>& st, float scale_log2, int64_t p_end, const int64_t (&lim)[2],
                                            RowPtr rowptr, uint8_t* lds) {
  static_assert(NST == 2 || NST == 3, "two or three stages");
  const int lane = lane_tid() & 63;
  const int l16 = lane & 15, g = lane >> 4;
  if (p_end <= 0) return;
  const int64_t n_tiles = (p_end + kTileKeys - 1) / kTileKeys;
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds;
  uint64_t* masks = reinterpret_cast<uint64_t*>(lds + NST * kStageBytes);
  auto issue = [&](int64_t t, int s) { attn_issue_tile(0, p_end, t, s, rowptr, lds_base, masks); };
  issue(0, 0);
  if (n_tiles > 1) issue(1, 1);
  if (NST == 3 && n_tiles > 2) issue(2, 2);
  for (int64_t t = 0; t < n_tiles; ++t) {
    const int s = (int)(t % NST);
    const int64_t ahead = n_tiles - 1 - t < NST - 1 ? n_tiles - 1 - t : NST - 1;
    if (ahead >= 2) attn_wait_dma<16>();
    else if (ahead == 1) attn_wait_dma<8>();
    else attn_wait_dma<0>();
    __syncthreads();
    const uint8_t* cur = lds + s * kStageBytes;
    const uint64_t vmask = masks[s];
    const int64_t t0 = t * kTileKeys;
    uint64_t vm[2];
#pragma unroll
    for (int gi = 0; gi < 2; ++gi)
      vm[gi] = lim[gi] <= t0 ? 0ull : (lim[gi] < t0 + kTileKeys ? vmask & ((1ull << (lim[gi] - t0)) - 1ull) : vmask);
    float s0[4][4], s1[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      v8bf kf[4];
#pragma unroll
      for (int kq = 0; kq < 4; ++kq)
        kf[kq] = *reinterpret_cast<const v8bf*>(cur + (kq * 4 + mt) * 1024 + l16 * 64 + g * 16);
      v4f a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kq = 0; kq < 4; ++kq) {
        a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kq], st.qf[0][kq], a0, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kq], st.qf[1][kq], a1, 0, 0, 0);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        s0[mt][v] = a0[v];
        s1[mt][v] = a1[v];
      }
    }
    v4s_t vt[8][2][2];
    attn_vt(cur, l16, g, vt);
    attn_softmax_pv(st.m_run[0], st.l_run[0], st.O[0], s0, vt, vm[0], g, scale_log2);
    attn_softmax_pv(st.m_run[1], st.l_run[1], st.O[1], s1, vt, vm[1], g, scale_log2);
    if (t + NST < n_tiles) {
      __syncthreads();
      issue(t + NST, s);
    }
  }
  __syncthreads();
}

// Finish: normalised bf16 output [H][128] and lse (natural log), or, when
// `partial` is set, the unnormalised (m in log2 units, l, O) partial through
// device-coherent stores if `coherent` (read by other workgroups in the same
// launch) or plain stores.  Lane (l16, g) holds head 16*hg + l16, dims
// 16*mt + 4*g + v.
template <int GPW>
__device__ __forceinline__ void attn_finish(AttnState<GPW>& st, int H, uint8_t* out_row, float* lse_row,
                                            float* part_o, float* part_ml, bool partial, bool coherent) {
  const int lane = lane_tid() & 63, wave = lane_tid() >> 6, l16 = lane & 15, g = lane >> 4;
  const int HG = H >> 4;
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    const int hg = wave + 4 * gi;
    if (hg >= HG) continue;
    const float l = xor32_sum(xor16_sum(st.l_run[gi]));
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

// Exact top-k selection helpers (whole workgroup), shared by the top-k kernels.
#pragma once
#include "common.hpp"

namespace csa {

// need-th largest value among the active entries i < n (val(i), active(i)),
// 8 bits per round from the top.  Returns the exact value; *need_left = how
// many of the entries equal to it are to be taken (>= 1).  bins: 256 words of
// LDS; scratch: blockDim.x/64 + 2 words of LDS.  Every thread must call it.
template <typename ValueFn, typename ActiveFn>
__device__ uint32_t radix_select_desc(uint32_t n, uint32_t need, ValueFn val, ActiveFn active,
                                      uint32_t* need_left, uint32_t* bins, uint32_t* scratch) {
  uint32_t prefix = 0, pmask = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = lane_tid(); i < 256; i += blockDim.x) bins[i] = 0;
    __syncthreads();
    for (uint32_t i = lane_tid(); i < n; i += blockDim.x) {
      if (!active(i)) continue;
      const uint32_t v = val(i);
      if ((v & pmask) == prefix) atomicAdd(&bins[(v >> shift) & 255u], 1u);
    }
    __syncthreads();
    uint32_t c = 0;
    for (int b = lane_tid(); b < 256; b += blockDim.x) c += bins[b];  // one bin per thread (blockDim >= 256)
    int d;
    uint32_t above;
    block_find_from_top(lane_tid() < 256 ? c : 0u, need, scratch, &d, &above);
    prefix |= (uint32_t)d << shift;
    pmask |= 255u << shift;
    need -= above;
  }
  *need_left = need;
  return prefix;
}

// The same selection when every active value already agrees on the bits at
// and above `top` (given in `fixed`): only the low `top` bits are resolved,
// in digits of at most 10 bits (1024 bins).  bins: 1024 words of LDS.
template <typename ValueFn, typename ActiveFn>
__device__ uint32_t radix_select_desc_low(uint32_t n, uint32_t need, int top, uint32_t fixed, ValueFn val,
                                          ActiveFn active, uint32_t* need_left, uint32_t* bins,
                                          uint32_t* scratch) {
  uint32_t prefix = fixed, pmask = top >= 32 ? 0u : ~((1u << top) - 1u);
  const int rounds = (top + 9) / 10;
  const int nt = blockDim.x;
  for (int rd = 0; rd < rounds; ++rd) {
    const int hi = top - rd * ((top + rounds - 1) / rounds);
    const int width = hi < (top + rounds - 1) / rounds ? hi : (top + rounds - 1) / rounds;
    const int shift = hi - width;
    const int nb = 1 << width;
    for (int i = lane_tid(); i < nb; i += nt) bins[i] = 0;
    __syncthreads();
    for (uint32_t i = lane_tid(); i < n; i += nt) {
      if (!active(i)) continue;
      const uint32_t v = val(i);
      if ((v & pmask) == prefix) atomicAdd(&bins[(v >> shift) & (uint32_t)(nb - 1)], 1u);
    }
    __syncthreads();
    // thread t owns bins [t*bpt, (t+1)*bpt)
    const int bpt = (nb + nt - 1) / nt;
    uint32_t c = 0;
    for (int b = 0; b < bpt; ++b) {
      const int bi = lane_tid() * bpt + b;
      if (bi < nb) c += bins[bi];
    }
    int tstar;
    uint32_t above;
    block_find_from_top(c, need, scratch, &tstar, &above);
    if ((int)lane_tid() == tstar) {
      uint32_t cum = above;
      int b = bpt - 1;
      for (; b > 0; --b) {
        const int bi = lane_tid() * bpt + b;
        const uint32_t cb = bi < nb ? bins[bi] : 0u;
        if (cum + cb >= need) break;
        cum += cb;
      }
      scratch[30] = (uint32_t)(lane_tid() * bpt + b);
      scratch[31] = cum;
    }
    __syncthreads();
    const uint32_t digit = scratch[30];
    need -= scratch[31];
    prefix |= digit << shift;
    pmask |= (uint32_t)(nb - 1) << shift;
    __syncthreads();
  }
  *need_left = need;
  return prefix;
}

// Calls emit(rank, j) for every set bit j of an LDS bitmap (nwords words), in
// ascending j, rank counting from 0.  scratch: blockDim.x/64 words of LDS.
template <typename EmitFn>
__device__ void bitmap_emit_ascending(const uint32_t* bitmap, int nwords, uint32_t* scratch, EmitFn emit) {
  const int tid = lane_tid(), lane = tid & 63, wave = tid >> 6;
  const int wpt = (nwords + (int)blockDim.x - 1) / (int)blockDim.x;
  const int w0 = tid * wpt;
  uint32_t cnt = 0;
  for (int i = 0; i < wpt; ++i)
    if (w0 + i < nwords) cnt += __popc(bitmap[w0 + i]);
  uint32_t incl = cnt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  uint32_t pos = incl - cnt;
  for (int w = 0; w < wave; ++w) pos += scratch[w];
  for (int i = 0; i < wpt; ++i) {
    if (w0 + i >= nwords) break;
    uint32_t bits = bitmap[w0 + i];
    while (bits) {
      const int bpos = __ffs(bits) - 1;
      bits &= bits - 1;
      emit(pos++, (w0 + i) * 32 + bpos);
    }
  }
  __syncthreads();
}

}  // namespace csa

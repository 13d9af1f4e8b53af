// MQA attention over a per-query key list with one softmax, used by both
// CSA (selected pooled rows ++ sliding window of raw rows) and HCA (every
// visible heavily-pooled row, optionally ++ a window).
//
// Pages: pytorch.kr DeepSeek-V4 summary, CSA/HCA section (top-k compressed
// entries plus a sliding-window branch; HCA dense over all compressed
// entries); sigco.tistory.com CSA/HCA section; jyp-garden IDEAS (MQA: one
// KV head shared by all query heads).  The single softmax over the union of
// both branches is the reading taken.
//
// Key list of query i (position t, sequence b), position p:
//   p <  seg_a : CSA -> pooled row pool_off[b] + idx[i][p] (padding if < 0)
//                HCA -> pooled row pool_off[b] + p (valid if p < n_vis)
//   p >= seg_a : raw row tok_off[b] + t - W + 1 + (p - seg_a) (valid if >= 0)
// Work item = (query, split of the list).  A split of more than one tile
// runs an online softmax; with several splits per query, partial
// (max, sum, unnormalised output) go to the workspace and k_attn_combine
// merges them by log-sum-exp.
//
// bf16: one workgroup = 4 waves; a wave owns 16 query heads.  Per 64-key
// tile, K rows are staged row-major and V transposed in LDS; S^T = K Q^T and
// O^T += V^T P^T run on v_mfma_f32_16x16x32_bf16 with fp32 accumulation.
// The key order inside the P^T operand is permuted so that each lane feeds
// the MFMA with its own softmax outputs (no cross-lane shuffles).
#include "attn_core.hpp"
#include "common.hpp"
#include "kernels.hpp"

namespace csa {

struct AttnArgs {
  const int64_t* tok_off;
  const int64_t* q_off;
  const int64_t* q_pos;
  const int64_t* pool_off;
  int n_seq;
  int hca;      // 0: CSA (segment A through idx), 1: HCA (segment A contiguous)
  int m_pool;   // HCA block size
  int seg_a;    // CSA: k; HCA: max pooled rows per sequence
  int W;
  int H;
  float scale_log2;
  const uint8_t* q;
  const uint8_t* kv_pool;
  const uint8_t* kv_raw;
  const int32_t* idx;
  uint8_t* out;
  float* lse;
  float* part_o;   // [n_q][splits][H][128]
  float* part_ml;  // [n_q][splits][H][2]
  int splits;
  int ks;          // list positions per split (multiple of 64)
};

struct RowCtx {
  int b;
  int64_t t, n_vis_a, pool_base, tok_base;
#ifdef CSA_DEBUG
  int64_t P;  // pooled rows of the sequence (the range a CSA index must fall in)
#endif
};

__device__ __forceinline__ RowCtx row_ctx(const AttnArgs& a, int64_t row) {
  RowCtx c;
  c.b = seq_of_row(a.q_off, a.n_seq, row);
  c.t = a.q_pos[row];
  c.pool_base = a.pool_off[c.b];
  c.tok_base = a.tok_off[c.b];
#ifdef CSA_DEBUG
  c.P = a.pool_off[c.b + 1] - c.pool_base;
#endif
  if (a.hca) {
    const int64_t P = a.pool_off[c.b + 1] - c.pool_base;
    const int64_t v = (c.t + 1) / a.m_pool;
    c.n_vis_a = v < P ? v : P;
  } else {
    c.n_vis_a = a.seg_a;
  }
  return c;
}

// row pointer of list position p (nullptr = masked), row_bytes = bytes of one [2][d] row
__device__ __forceinline__ const uint8_t* key_row(const AttnArgs& a, const RowCtx& c, int64_t row,
                                                  int64_t p, size_t row_bytes) {
  if (p < a.seg_a) {
    if (a.hca) return p < c.n_vis_a ? a.kv_pool + (size_t)(c.pool_base + p) * row_bytes : nullptr;
    const int32_t j = a.idx[row * a.seg_a + p];
#ifdef CSA_DEBUG
    if (j >= c.P) {
      debug_violation();
      return nullptr;
    }
#endif
    return j >= 0 ? a.kv_pool + (size_t)(c.pool_base + j) * row_bytes : nullptr;
  }
  const int64_t u = c.t - a.W + 1 + (p - a.seg_a);
  if (p >= (int64_t)a.seg_a + a.W || u < 0) return nullptr;
  return a.kv_raw + (size_t)(c.tok_base + u) * row_bytes;
}

// ---------------------------------------------------------------------------
// bf16, MFMA (tile loop in attn_core.hpp)
// ---------------------------------------------------------------------------
// One query's head group per wave over list positions [p_begin, p_end), with
// 48 KB of LDS instead of two 32 KB stages: K single-buffered, V
// double-buffered (kKv1LdsBytes).  Per tile t: wait for K(t) and V(t), read
// the K fragments (S^T MFMAs) and the V^T fragments into registers, barrier,
// DMA of K(t+1) (hidden behind the softmax and PV) and of V(t+2) (a whole
// tile ahead), then the softmax and PV from registers.  So three workgroups
// fit a CU's LDS.  Same arithmetic as attn_run (attn_softmax_pv); same entry
// conditions.
constexpr int kKv1LdsBytes = 3 * 16 * 1024 + 16;

template <class RowPtr>
__device__ __forceinline__ void attn_run_kv1(AttnState<1>& st, float scale_log2, int64_t p_begin, int64_t p_end,
                                             RowPtr rowptr, uint8_t* lds) {
  const int lane = lane_tid() & 63, wave = lane_tid() >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  if (p_begin >= p_end) return;
  const int64_t n_tiles = (p_end - p_begin + kTileKeys - 1) / kTileKeys;
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds;
  uint64_t* masks = reinterpret_cast<uint64_t*>(lds + 3 * 16 * 1024);  // by tile parity
  // row of this lane in tile t (nullptr: masked) and its source address
  auto src_of = [&](int64_t t, const uint8_t** rp_out) {
    const int row = 16 * wave + (lane >> 2);
    const int64_t p = p_begin + t * kTileKeys + row;
    const uint8_t* rp = p < p_end ? rowptr(p) : nullptr;
    *rp_out = rp;
    return (rp ? rp : g_zero_row) + 16 * (lane & 3);
  };
  auto issue_k = [&](int64_t t) {  // K chunks 0..15 -> [0, 16 KB), and the tile's validity word
    const uint8_t* rp;
    const uint8_t* src = src_of(t, &rp);
    const uint64_t vb = __ballot(rp != nullptr);
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_base + (uint32_t)(wave * 1024));
    dma16<0>(src, m0);
    dma16<64>(src, m0 + 4 * 1024 - 64);
    dma16<128>(src, m0 + 8 * 1024 - 128);
    dma16<192>(src, m0 + 12 * 1024 - 192);
    uint32_t m16 = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) m16 |= (uint32_t)((vb >> (4 * j)) & 1ull) << j;
    if (lane == 0) reinterpret_cast<uint16_t*>(masks + (t & 1))[wave] = (uint16_t)m16;
  };
  auto issue_v = [&](int64_t t) {  // V chunks 16..31 -> buffer t & 1 at 16 KB (t & 1 ? 2 : 1)
    const uint8_t* rp;
    const uint8_t* src = src_of(t, &rp);
    const uint32_t vb0 = lds_base + (uint32_t)((1 + (t & 1)) * 16 * 1024);
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(vb0 + (uint32_t)(wave * 1024));
    dma16<256>(src, m0 - 256);
    dma16<320>(src, m0 + 4 * 1024 - 320);
    dma16<384>(src, m0 + 8 * 1024 - 384);
    dma16<448>(src, m0 + 12 * 1024 - 448);
  };
  issue_k(0);
  issue_v(0);
  if (n_tiles > 1) issue_v(1);
  for (int64_t t = 0; t < n_tiles; ++t) {
    // issued after K(t): only V(t+1) (V(t) was issued before K(t))
    if (t + 1 < n_tiles) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // K(t), V(t) and the validity word in LDS
    const uint64_t vmask = masks[t & 1];
    float s_[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      v8bf kf[4];
#pragma unroll
      for (int kq = 0; kq < 4; ++kq)
        kf[kq] = *reinterpret_cast<const v8bf*>(lds + (kq * 4 + mt) * 1024 + l16 * 64 + g * 16);
      v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kq = 0; kq < 4; ++kq) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kq], st.qf[0][kq], acc, 0, 0, 0);
#pragma unroll
      for (int v = 0; v < 4; ++v) s_[mt][v] = acc[v];
    }
    // V^T of tile t: attn_vt addresses V at +16 KB of its base
    v4s_t vt[8][2][2];
    attn_vt(lds + (t & 1) * 16 * 1024, l16, g, vt);
    __syncthreads();  // every wave has read K(t) and V(t) (the barrier waits for its LDS reads)
    if (t + 1 < n_tiles) issue_k(t + 1);
    if (t + 2 < n_tiles) issue_v(t + 2);
    attn_softmax_pv(st.m_run[0], st.l_run[0], st.O[0], s_, vt, vmask, g, scale_log2);
  }
  __syncthreads();
}

constexpr int kMaxSplitKeys = 1024;

template <int GPW>
__global__ __launch_bounds__(256) void k_attn_bf16(AttnArgs a) {
  // one head group per wave (H <= 64): the 48 KB K/V staging (three
  // workgroups per CU); two groups per wave: two 32 KB stages
  __shared__ __align__(16) uint8_t lds[GPW == 1 ? kKv1LdsBytes : kAttnLdsBytes];
  __shared__ int32_t idx_s[kMaxSplitKeys];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.y;
  const int split = blockIdx.x;
  const RowCtx c = row_ctx(a, row);
  const int64_t list_len = (int64_t)a.seg_a + a.W;
  const int64_t p_begin = (int64_t)split * a.ks;
  const int64_t p_end = p_begin + a.ks < list_len ? p_begin + a.ks : list_len;
  constexpr size_t RB = 2 * 128 * 2;  // bytes per [2][128] bf16 row

  // this split's slice of the index row, staged once
  if (!a.hca) {
    for (int64_t p = p_begin + tid; p < p_end && p < a.seg_a; p += 256)
      idx_s[p - p_begin] = a.idx[row * a.seg_a + p];
  }
  __syncthreads();
  auto rowptr = [&](int64_t p) -> const uint8_t* {
    if (p < a.seg_a) {
      if (a.hca) return p < c.n_vis_a ? a.kv_pool + (size_t)(c.pool_base + p) * RB : nullptr;
      const int32_t j = idx_s[p - p_begin];
#ifdef CSA_DEBUG
      if (j >= c.P) {
        debug_violation();
        return nullptr;
      }
#endif
      return j >= 0 ? a.kv_pool + (size_t)(c.pool_base + j) * RB : nullptr;
    }
    const int64_t u = c.t - a.W + 1 + (p - a.seg_a);
    return u >= 0 ? a.kv_raw + (size_t)(c.tok_base + u) * RB : nullptr;
  };
  AttnState<GPW> st;
  attn_init<GPW>(st, a.q + (size_t)row * a.H * 128 * 2, a.H);
  if constexpr (GPW == 1) attn_run_kv1(st, a.scale_log2, p_begin, p_end, rowptr, lds);
  else attn_run<GPW>(st, a.H, a.scale_log2, p_begin, p_end, rowptr, lds);
  const size_t pbase = (size_t)(row * a.splits + split) * a.H;
  attn_finish<GPW>(st, a.H, a.out + (size_t)row * a.H * 128 * 2, a.lse ? a.lse + row * a.H : nullptr,
                   a.part_o ? a.part_o + pbase * 128 : nullptr, a.part_ml ? a.part_ml + pbase * 2 : nullptr,
                   a.splits > 1, false);
}

// HCA without a window over a prefill batch (H = 64, one split per query):
// workgroup y serves rows 2y and 2y+1 of one sequence over the union of their
// visible pooled rows (attn_run_q2: every K and V fragment read from LDS feeds
// both rows; each row masks the positions beyond its own visible count).  A
// pair that straddles two sequences (at most one per sequence boundary), or
// the unpaired last row, is served one row at a time (attn_run).
__global__ __launch_bounds__(256) void k_attn_bf16_pair(AttnArgs a, int64_t n_q) {
  __shared__ __align__(16) uint8_t lds[kAttnLdsBytes];
  const int64_t r0 = 2 * (int64_t)blockIdx.y;
  const bool has1 = r0 + 1 < n_q;
  const RowCtx c0 = row_ctx(a, r0);
  const RowCtx c1 = row_ctx(a, has1 ? r0 + 1 : r0);
  constexpr size_t RB = 2 * 128 * 2;
  if (has1 && c1.b == c0.b) {
    const int64_t n_union = c0.n_vis_a > c1.n_vis_a ? c0.n_vis_a : c1.n_vis_a;
    auto rowptr = [&](int64_t p) -> const uint8_t* {
      return p < n_union ? a.kv_pool + (size_t)(c0.pool_base + p) * RB : nullptr;
    };
    AttnState<2> st;
    {
      const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l16 = lane & 15, g = lane >> 4;
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) {
        st.m_run[gi] = -INFINITY;
        st.l_run[gi] = 0.f;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) st.O[gi][mt] = v4f{0.f, 0.f, 0.f, 0.f};
        const uint8_t* qrow = a.q + (size_t)(r0 + gi) * a.H * 128 * 2;
#pragma unroll
        for (int kq = 0; kq < 4; ++kq)
          st.qf[gi][kq] = *reinterpret_cast<const v8bf*>(qrow + ((size_t)(16 * wave + l16) * 128 + 32 * kq + 8 * g) * 2);
      }
    }
    const int64_t lim[2] = {c0.n_vis_a, c1.n_vis_a};
    attn_run_q2(st, a.scale_log2, n_union, lim, rowptr, lds);
    // each row's head group `wave`: the one-group finish on a copy of its state
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      AttnState<1> one;
      one.m_run[0] = st.m_run[gi];
      one.l_run[0] = st.l_run[gi];
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) one.O[0][mt] = st.O[gi][mt];
      const int64_t row = r0 + gi;
      attn_finish<1>(one, a.H, a.out + (size_t)row * a.H * 128 * 2, a.lse ? a.lse + row * a.H : nullptr, nullptr,
                     nullptr, false, false);
    }
    return;
  }
  for (int j = 0; j < (has1 ? 2 : 1); ++j) {  // uniform
    const RowCtx& c = j == 0 ? c0 : c1;
    const int64_t row = r0 + j;
    auto rowptr = [&](int64_t p) -> const uint8_t* {
      return p < c.n_vis_a ? a.kv_pool + (size_t)(c.pool_base + p) * RB : nullptr;
    };
    AttnState<1> st;
    attn_init<1>(st, a.q + (size_t)row * a.H * 128 * 2, a.H);
    attn_run<1>(st, a.H, a.scale_log2, 0, a.seg_a, rowptr, lds);
    attn_finish<1>(st, a.H, a.out + (size_t)row * a.H * 128 * 2, a.lse ? a.lse + row * a.H : nullptr, nullptr,
                   nullptr, false, false);
  }
}

// ---------------------------------------------------------------------------
// fp32, VALU (small head counts; exact fp32 FMAs)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum_f(float v) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// QLDS (H <= 64): the query's heads are staged in LDS once, so the score
// loop reads them from LDS (a wave's lanes share one head: a broadcast)
// instead of from global memory.  E (a power of two >= H / 2): the outputs a
// thread owns, dims tid & 127 of heads (tid >> 7) + 2e.  A tile's scores
// come from four independent partial dot products per (head, key) over
// 16-byte LDS reads, the softmax runs one wave per head and a lane per key,
// and PV reads each V element once for all of the thread's heads (E
// independent FMA chains), so no step is a long chain of dependent LDS reads.
template <bool QLDS, int E>
__global__ __launch_bounds__(256) void k_attn_f32(AttnArgs a) {
  constexpr int KS = 132, PS = 68;  // row strides (floats): 16-byte aligned rows
  __shared__ __align__(16) float Ks[64][KS];
  __shared__ __align__(16) float Vs[64][128];
  __shared__ __align__(16) float Ps[128][PS];
  __shared__ float m_s[128], l_s[128], al_s[128];
  __shared__ const uint8_t* rowp[64];
  extern __shared__ float qs[];  // [H][128] with QLDS
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.y;
  const int split = blockIdx.x;
  const RowCtx c = row_ctx(a, row);
  const int64_t list_len = (int64_t)a.seg_a + a.W;
  const int64_t p_begin = (int64_t)split * a.ks;
  const int64_t p_end = p_begin + a.ks < list_len ? p_begin + a.ks : list_len;
  const int H = a.H;
  constexpr size_t RB = 2 * 128 * 4;
  const float* qrow = reinterpret_cast<const float*>(a.q) + (size_t)row * H * 128;
  const int d_own = tid & 127, h_own = tid >> 7;  // output e: head h_own + 2e, dim d_own
  float O[E];
#pragma unroll
  for (int e = 0; e < E; ++e) O[e] = 0.f;
  for (int h = tid; h < H; h += 256) { m_s[h] = -INFINITY; l_s[h] = 0.f; }
  if constexpr (QLDS) {
    for (int i = tid; i < H * 32; i += 256)
      reinterpret_cast<float4*>(qs)[i] = reinterpret_cast<const float4*>(qrow)[i];
  }

  for (int64_t p0 = p_begin; p0 < p_end; p0 += 64) {
    if (tid < 64) {
      const int64_t p = p0 + tid;
      rowp[tid] = p < p_end ? key_row(a, c, row, p, RB) : nullptr;
    }
    __syncthreads();
    {  // 64 keys x 64 float4 (K then V): all 16 of a thread's loads, then the stores
      float4 v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int i = tid + 256 * u, key = i >> 6, q4 = i & 63;
        const uint8_t* rp = rowp[key];
        v[u] = rp ? *reinterpret_cast<const float4*>(rp + q4 * 16) : make_float4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int i = tid + 256 * u, key = i >> 6, q4 = i & 63;
        if (q4 < 32) *reinterpret_cast<float4*>(&Ks[key][4 * q4]) = v[u];
        else *reinterpret_cast<float4*>(&Vs[key][4 * (q4 - 32)]) = v[u];
      }
    }
    __syncthreads();
    for (int i = tid; i < H * 64; i += 256) {  // a wave's 64 lanes: one head, 64 keys
      const int h = i >> 6, j = i & 63;
      const float* qh = QLDS ? qs + h * 128 : qrow + h * 128;
      float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll 8
      for (int d = 0; d < 128; d += 4) {
        const float4 q = *reinterpret_cast<const float4*>(qh + d);
        const float4 k = *reinterpret_cast<const float4*>(&Ks[j][d]);
        s0 = fmaf(q.x, k.x, s0);
        s1 = fmaf(q.y, k.y, s1);
        s2 = fmaf(q.z, k.z, s2);
        s3 = fmaf(q.w, k.w, s3);
      }
      Ps[h][j] = rowp[j] ? ((s0 + s1) + (s2 + s3)) * a.scale_log2 : -INFINITY;
    }
    __syncthreads();
    for (int h = wave; h < H; h += 4) {  // wave per head, lane per key
      const float pv = Ps[h][lane];
      const float tmax = wave_max(pv);
      const float mold = m_s[h];
      const float mnew = fmaxf(mold, tmax);
      if (mnew == -INFINITY) {  // nothing valid so far (uniform): adds nothing
        Ps[h][lane] = 0.f;
        if (lane == 0) al_s[h] = 1.f;
        continue;
      }
      const float pj = fast_exp2(pv - mnew);
      Ps[h][lane] = pj;
      const float sum = wave_sum_f(pj);
      if (lane == 0) {
        const float alpha = fast_exp2(mold - mnew);
        m_s[h] = mnew;
        l_s[h] = l_s[h] * alpha + sum;
        al_s[h] = alpha;
      }
    }
    __syncthreads();
    {  // O[e] = O[e] * alpha + sum_j P[h][j] V[j][d], four keys a step
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (h_own + 2 * e < H) O[e] *= al_s[h_own + 2 * e];
#pragma unroll 2
      for (int j = 0; j < 64; j += 4) {
        const float v0 = Vs[j][d_own], v1 = Vs[j + 1][d_own], v2 = Vs[j + 2][d_own], v3 = Vs[j + 3][d_own];
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int h = h_own + 2 * e;
          if (h < H) {
            const float4 pp = *reinterpret_cast<const float4*>(&Ps[h][j]);
            O[e] = fmaf(pp.x, v0, O[e]);
            O[e] = fmaf(pp.y, v1, O[e]);
            O[e] = fmaf(pp.z, v2, O[e]);
            O[e] = fmaf(pp.w, v3, O[e]);
          }
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int h = h_own + 2 * e;
    if (h >= H) continue;
    const int o = h * 128 + d_own;
    const float l = l_s[h];
    if (a.splits == 1) {
      reinterpret_cast<float*>(a.out)[(size_t)row * H * 128 + o] = l > 0.f ? O[e] / l : 0.f;
      if (a.lse && d_own == 0) a.lse[row * H + h] = l > 0.f ? (m_s[h] + __log2f(l)) * kLn2 : -INFINITY;
    } else {
      const size_t base = (size_t)(row * a.splits + split) * H + h;
      a.part_o[base * 128 + d_own] = O[e];
      if (d_own == 0) { a.part_ml[base * 2] = m_s[h]; a.part_ml[base * 2 + 1] = l; }
    }
  }
}

// ---------------------------------------------------------------------------
// log-sum-exp merge of split partials: one workgroup per (query, head), one
// thread per output dim
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(128) void k_attn_combine(const float* __restrict__ part_o,
                                                      const float* __restrict__ part_ml, int splits,
                                                      int H, uint8_t* __restrict__ out,
                                                      float* __restrict__ lse) {
  __shared__ float wsh[128];
  __shared__ float red[2];
  const int64_t row = blockIdx.x;
  const int h = blockIdx.y, d = threadIdx.x, lane = d & 63, wave = d >> 6;
  const float* ml = part_ml + ((size_t)row * splits * H + h) * 2;  // split s at ml[s * H * 2]
  float M = -INFINITY;
  for (int s = d; s < splits; s += 128) M = fmaxf(M, ml[(size_t)s * H * 2]);
  M = wave_max(M);
  if (lane == 0) red[wave] = M;
  __syncthreads();
  M = fmaxf(red[0], red[1]);
  __syncthreads();
  float Lp = 0.f, acc = 0.f;
  if (M != -INFINITY) {
    for (int c0 = 0; c0 < splits; c0 += 128) {
      const int s = c0 + d;
      float wgt = 0.f;
      if (s < splits) {
        const float ms = ml[(size_t)s * H * 2];
        wgt = ms == -INFINITY ? 0.f : fast_exp2(ms - M);
        Lp = fmaf(wgt, ml[(size_t)s * H * 2 + 1], Lp);
      }
      wsh[d] = wgt;
      __syncthreads();
      const int n = splits - c0 < 128 ? splits - c0 : 128;
      const float* po = part_o + (((size_t)row * splits + c0) * H + h) * 128 + d;
      const size_t stride = (size_t)H * 128;
      int i = 0;
      for (; i + 8 <= n; i += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = po[(size_t)(i + u) * stride];
#pragma unroll
        for (int u = 0; u < 8; ++u) acc = fmaf(wsh[i + u], v[u], acc);
      }
      for (; i < n; ++i) acc = fmaf(wsh[i], po[(size_t)i * stride], acc);
      __syncthreads();
    }
  }
  // L = sum of the per-thread partial sums
  for (int o = 32; o >= 1; o >>= 1) Lp += __shfl_xor(Lp, o);
  if (lane == 0) red[wave] = Lp;
  __syncthreads();
  const float L = red[0] + red[1];
  const float v = L > 0.f ? acc / L : 0.f;
  const size_t o = ((size_t)row * H + h) * 128 + d;
  if (BF16) reinterpret_cast<uint16_t*>(out)[o] = (uint16_t)f32_to_bf16(v);
  else reinterpret_cast<float*>(out)[o] = v;
  if (lse && d == 0) lse[row * H + h] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
AttnPlan plan_attn(int64_t n_q, int64_t list_len, int H) {
  // aim for ~256 workgroups, at least one 64-key tile per split (a split's
  // tiles form a dependent chain, so a short list gains more from splits run
  // side by side than the combine costs: 3 splits of 64 against 2 of 128 took
  // the fp32 4096-token decode step from 50 to 42 us), and at most
  // kMaxSplitKeys positions per split (the staged index slice)
  AttnPlan p;
  const int64_t s_min = (list_len + kMaxSplitKeys - 1) / kMaxSplitKeys;
  const int64_t s_max = (list_len + 63) / 64;
  int64_t s = n_q > 0 ? (256 + n_q - 1) / n_q : 1;
  if (s > s_max) s = s_max;
  if (s < s_min) s = s_min;
  if (s < 1) s = 1;
  int64_t ks = (list_len + s - 1) / s;
  ks = ((ks + 63) / 64) * 64;
  if (ks < 64) ks = 64;
  if (ks > kMaxSplitKeys) ks = kMaxSplitKeys;
  s = (list_len + ks - 1) / ks;
  if (s < 1) s = 1;
  p.splits = (int)s;
  p.ks = (int)ks;
  p.ws_bytes = s > 1 ? (size_t)n_q * s * H * (128 + 2) * 4 + 256 : 0;
  return p;
}

#ifdef CSA_DEBUG
unsigned long long debug_take_attn() { return debug_take_here(); }
#endif

int launch_attn(bool bf16, bool hca, int n_seq, int64_t n_q, const int64_t* tok_off,
                const int64_t* q_off, const int64_t* q_pos, const int64_t* pool_off, int m_pool,
                int seg_a, int W, int H, float scale, const void* q, const void* kv_pool,
                const void* kv_raw, const int32_t* idx, void* out, float* lse, void* ws,
                hipStream_t stream) {
  if (n_q == 0) return 0;
  const int64_t list_len = (int64_t)seg_a + W;
  const AttnPlan pl = plan_attn(n_q, list_len, H);
  AttnArgs a;
  a.tok_off = tok_off; a.q_off = q_off; a.q_pos = q_pos; a.pool_off = pool_off;
  a.n_seq = n_seq; a.hca = hca ? 1 : 0; a.m_pool = m_pool; a.seg_a = seg_a; a.W = W; a.H = H;
  a.scale_log2 = scale * kLog2e;
  a.q = (const uint8_t*)q; a.kv_pool = (const uint8_t*)kv_pool; a.kv_raw = (const uint8_t*)kv_raw;
  a.idx = idx; a.out = (uint8_t*)out; a.lse = lse;
  a.part_o = (float*)ws;
  a.part_ml = pl.splits > 1 ? (float*)ws + (size_t)n_q * pl.splits * H * 128 : nullptr;
  a.splits = pl.splits; a.ks = pl.ks;
  if (list_len == 0) {  // every list is empty: the combine writes zeros and -inf
    a.splits = 1;
  }
  if (bf16 && hca && W == 0 && H == 64 && a.splits == 1 && n_q >= 512) {  // prefill HCA: two rows per workgroup
    const hipError_t e = launch(3, kProfBoth, k_attn_bf16_pair, dim3(1u, (unsigned)((n_q + 1) / 2)), dim3(256), 0,
                                stream, a, n_q);
    return e == hipSuccess && hipGetLastError() == hipSuccess ? 0 : -1;
  }
  dim3 grid((unsigned)a.splits, (unsigned)n_q);
  hipError_t e;
  if (!bf16) {  // outputs per thread: the power of two >= H / 2; the query's heads in LDS when H <= 64
    const size_t qb = (size_t)H * 128 * 4;
    if (H <= 8) e = launch(3, kProfBoth, k_attn_f32<true, 4>, grid, dim3(256), qb, stream, a);
    else if (H <= 16) e = launch(3, kProfBoth, k_attn_f32<true, 8>, grid, dim3(256), qb, stream, a);
    else if (H <= 32) e = launch(3, kProfBoth, k_attn_f32<true, 16>, grid, dim3(256), qb, stream, a);
    else if (H <= 64) e = launch(3, kProfBoth, k_attn_f32<true, 32>, grid, dim3(256), qb, stream, a);
    else e = launch(3, kProfBoth, k_attn_f32<false, 64>, grid, dim3(256), 0, stream, a);
  } else {
    e = launch(3, kProfBoth, H > 64 ? k_attn_bf16<2> : k_attn_bf16<1>, grid, dim3(256), 0, stream, a);
  }
  if (e == hipSuccess && a.splits > 1) {
    dim3 gc((unsigned)n_q, (unsigned)H);
    e = launch(4, kProfBoth, bf16 ? k_attn_combine<true> : k_attn_combine<false>, gc, dim3(128), 0, stream,
               (const float*)a.part_o, (const float*)a.part_ml, a.splits, H, a.out, lse);
  }
  return e == hipSuccess && hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace csa

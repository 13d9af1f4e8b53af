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
};

__device__ __forceinline__ RowCtx row_ctx(const AttnArgs& a, int64_t row) {
  RowCtx c;
  c.b = seq_of_row(a.q_off, a.n_seq, row);
  c.t = a.q_pos[row];
  c.pool_base = a.pool_off[c.b];
  c.tok_base = a.tok_off[c.b];
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
    return j >= 0 ? a.kv_pool + (size_t)(c.pool_base + j) * row_bytes : nullptr;
  }
  const int64_t u = c.t - a.W + 1 + (p - a.seg_a);
  if (p >= (int64_t)a.seg_a + a.W || u < 0) return nullptr;
  return a.kv_raw + (size_t)(c.tok_base + u) * row_bytes;
}

// ---------------------------------------------------------------------------
// bf16, MFMA (tile loop in attn_core.hpp)
// ---------------------------------------------------------------------------
constexpr int kMaxSplitKeys = 1024;

template <int GPW>
__global__ __launch_bounds__(256) void k_attn_bf16(AttnArgs a) {
  __shared__ __align__(16) uint8_t lds[kAttnLdsBytes];
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
      return j >= 0 ? a.kv_pool + (size_t)(c.pool_base + j) * RB : nullptr;
    }
    const int64_t u = c.t - a.W + 1 + (p - a.seg_a);
    return u >= 0 ? a.kv_raw + (size_t)(c.tok_base + u) * RB : nullptr;
  };
  AttnState<GPW> st;
  attn_init<GPW>(st, a.q + (size_t)row * a.H * 128 * 2, a.H);
  attn_run<GPW>(st, a.H, a.scale_log2, p_begin, p_end, rowptr, lds);
  const size_t pbase = (size_t)(row * a.splits + split) * a.H;
  attn_finish<GPW>(st, a.H, a.out + (size_t)row * a.H * 128 * 2, a.lse ? a.lse + row * a.H : nullptr,
                   a.part_o ? a.part_o + pbase * 128 : nullptr, a.part_ml ? a.part_ml + pbase * 2 : nullptr,
                   a.splits > 1, false);
}

// ---------------------------------------------------------------------------
// fp32, VALU (small head counts; exact fp32 FMAs)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_attn_f32(AttnArgs a) {
  __shared__ float Ks[64][129];
  __shared__ float Vs[64][128];
  __shared__ float Ps[128][65];
  __shared__ float m_s[128], l_s[128], al_s[128];
  __shared__ const uint8_t* rowp[64];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.y;
  const int split = blockIdx.x;
  const RowCtx c = row_ctx(a, row);
  const int64_t list_len = (int64_t)a.seg_a + a.W;
  const int64_t p_begin = (int64_t)split * a.ks;
  const int64_t p_end = p_begin + a.ks < list_len ? p_begin + a.ks : list_len;
  const int H = a.H;
  constexpr size_t RB = 2 * 128 * 4;
  const float* qrow = reinterpret_cast<const float*>(a.q) + (size_t)row * H * 128;
  constexpr int MAXE = 64;  // H*128/256 outputs per thread at H = 128
  const int n_el = (H * 128 + 255) / 256;
  float O[MAXE];
#pragma unroll
  for (int e = 0; e < MAXE; ++e) O[e] = 0.f;
  for (int h = tid; h < H; h += 256) { m_s[h] = -INFINITY; l_s[h] = 0.f; }

  for (int64_t p0 = p_begin; p0 < p_end; p0 += 64) {
    if (tid < 64) {
      const int64_t p = p0 + tid;
      rowp[tid] = p < p_end ? key_row(a, c, row, p, RB) : nullptr;
    }
    __syncthreads();
    for (int i = tid; i < 64 * 64; i += 256) {  // 64 keys x 64 float4 (K then V)
      const int key = i >> 6, q4 = i & 63;
      const uint8_t* rp = rowp[key];
      float4 v = rp ? *reinterpret_cast<const float4*>(rp + q4 * 16) : make_float4(0, 0, 0, 0);
      if (q4 < 32) {
        Ks[key][4 * q4 + 0] = v.x; Ks[key][4 * q4 + 1] = v.y;
        Ks[key][4 * q4 + 2] = v.z; Ks[key][4 * q4 + 3] = v.w;
      } else {
        *reinterpret_cast<float4*>(&Vs[key][4 * (q4 - 32)]) = v;
      }
    }
    __syncthreads();
    for (int i = tid; i < H * 64; i += 256) {
      const int h = i >> 6, j = i & 63;
      float s = 0.f;
      const float* qh = qrow + h * 128;
      for (int d = 0; d < 128; ++d) s = fmaf(qh[d], Ks[j][d], s);
      Ps[h][j] = rowp[j] ? s * a.scale_log2 : -INFINITY;
    }
    __syncthreads();
    for (int h = tid; h < H; h += 256) {
      float tmax = -INFINITY;
      for (int j = 0; j < 64; ++j) tmax = fmaxf(tmax, Ps[h][j]);
      const float mnew = fmaxf(m_s[h], tmax);
      if (mnew == -INFINITY) { al_s[h] = 1.f; continue; }
      const float alpha = fast_exp2(m_s[h] - mnew);
      float sum = 0.f;
      for (int j = 0; j < 64; ++j) {
        const float pj = fast_exp2(Ps[h][j] - mnew);
        Ps[h][j] = pj;
        sum += pj;
      }
      m_s[h] = mnew;
      l_s[h] = l_s[h] * alpha + sum;
      al_s[h] = alpha;
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < MAXE; ++e) {
      const int o = tid + 256 * e;
      if (e < n_el && o < H * 128) {
        const int h = o >> 7, d = o & 127;
        if (m_s[h] != -INFINITY) {
          float acc = O[e] * al_s[h];
          for (int j = 0; j < 64; ++j) acc = fmaf(Ps[h][j], Vs[j][d], acc);
          O[e] = acc;
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int e = 0; e < MAXE; ++e) {
    const int o = tid + 256 * e;
    if (e >= n_el || o >= H * 128) continue;
    const int h = o >> 7, d = o & 127;
    const float l = l_s[h];
    if (a.splits == 1) {
      reinterpret_cast<float*>(a.out)[(size_t)row * H * 128 + o] = l > 0.f ? O[e] / l : 0.f;
      if (a.lse && d == 0) a.lse[row * H + h] = l > 0.f ? (m_s[h] + __log2f(l)) * kLn2 : -INFINITY;
    } else {
      const size_t base = (size_t)(row * a.splits + split) * H + h;
      a.part_o[base * 128 + d] = O[e];
      if (d == 0) { a.part_ml[base * 2] = m_s[h]; a.part_ml[base * 2 + 1] = l; }
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
  // aim for ~256 workgroups, at least 128 list positions per split (the
  // partial (m, l, o) of a split costs as much as 64 bf16 KV rows), and at
  // most kMaxSplitKeys positions per split (the staged index slice)
  AttnPlan p;
  const int64_t s_min = (list_len + kMaxSplitKeys - 1) / kMaxSplitKeys;
  const int64_t s_max = (list_len + 127) / 128;
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
  dim3 grid((unsigned)a.splits, (unsigned)n_q);
  prof_begin(3, stream);
  if (bf16) {
    if (H > 64) hipLaunchKernelGGL(k_attn_bf16<2>, grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(k_attn_bf16<1>, grid, dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL(k_attn_f32, grid, dim3(256), 0, stream, a);
  }
  prof_end(3, stream);
  if (a.splits > 1) {
    prof_begin(4, stream);
    dim3 gc((unsigned)n_q, (unsigned)H);
    if (bf16)
      hipLaunchKernelGGL(k_attn_combine<true>, gc, dim3(128), 0, stream, a.part_o, a.part_ml, a.splits, H,
                         a.out, lse);
    else
      hipLaunchKernelGGL(k_attn_combine<false>, gc, dim3(128), 0, stream, a.part_o, a.part_ml, a.splits, H,
                         a.out, lse);
    prof_end(4, stream);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace csa

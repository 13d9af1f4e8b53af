// Streaming cache upkeep: one call appends each sequence's new tokens and
// pools every block the append completes.
//
// Pages: sigco.tistory.com, "DeepSeek-V4 paper reading", KV-cache section: the
// cache is kept in three parts, the compressed entries used by CSA/HCA, the
// recent tokens the sliding window reads, and the state of the tail tokens
// that are not yet numerous enough to be compressed.  Here: the raw rows
// [sum capacity][width] hold every token (the window reads the last W of
// them); the tail state is a ring of the latest `ring` tokens' pooling logits
// per sequence (slot p % ring); the pooled caches take one row per completed
// block of m (CSA) or m_hca (HCA) tokens, pooled with the same arithmetic as
// the bulk pooling kernel (pool_core.hpp), so a cache built by appends equals
// one pooled in bulk bit for bit.
//
// Two kernels, in stream order:
//   k_append_pool  copies the new rows into the raw cache and pools the
//                  completed blocks: a block's older tokens come from the raw
//                  cache and the logit ring, its new tokens straight from the
//                  inputs (nothing this kernel reads is written by it).  A
//                  short block is pooled by one thread per 16 bytes of
//                  channels; a long one by a workgroup whose threads pool its
//                  16-row segments in parallel and then fold them in order
//                  (the bulk kernel's order, so the bits agree)
//   k_append_tail  one workgroup per sequence: the newest min(n, ring) tokens'
//                  logits -> the ring, then the sequence's length advances
#include "common.hpp"
#include "kernels.hpp"
#include "pool_core.hpp"

namespace csa {

struct AppendArgs {
  const int64_t* tok_off;
  int64_t* len;
  const int64_t* new_off;
  const uint8_t* x_new;
  const uint8_t* z_new;
  uint8_t* kv_raw;
  uint8_t* z_tail;
  const int64_t* pool_off;
  const int64_t* hpool_off;
  uint8_t* pooled;
  uint8_t* hpooled;
  int width, ring, m, m_hca;
  int64_t narrow_items;  // per sequence, at most: rows to copy + blocks of at most kPoolSeg rows
  int nb_narrow;         // workgroups of the narrow items; each later workgroup pools one long block
  int wide_par;          // long blocks: segments pooled in parallel (1) or in one thread each (0)
};

__device__ __forceinline__ int64_t floordiv_blocks(int64_t p, int m) { return m > 0 ? p / m : 0; }

// The per-sequence view of one append: new rows, and the blocks of each size it completes.
struct AppendSeq {
  int64_t L0, n, r0, cap, c0, nc, h0, nh;
};
__device__ __forceinline__ AppendSeq append_seq(const AppendArgs& a, int b) {
  AppendSeq q;
  q.L0 = a.len[b];
  q.n = a.new_off[b + 1] - a.new_off[b];
  const int64_t L1 = q.L0 + q.n;
  q.r0 = a.tok_off[b];
  q.cap = a.tok_off[b + 1] - q.r0;
  q.c0 = floordiv_blocks(q.L0, a.m);
  q.nc = floordiv_blocks(L1, a.m) - q.c0;
  q.h0 = floordiv_blocks(q.L0, a.m_hca);
  q.nh = floordiv_blocks(L1, a.m_hca) - q.h0;
  return q;
}

// Block j of m rows of sequence b, this thread's 16-byte channel group g:
// older tokens from the raw cache and the logit ring, new ones from the inputs.
template <bool BF16>
struct BlockRows {
  const uint8_t* xo;
  const uint8_t* zo;
  const uint8_t* xn;
  const uint8_t* zn;
  int64_t p0, L0;
  size_t row;
  int ring;
  __device__ const uint8_t* x(int i) const {
    const int64_t p = p0 + i;
    return p < L0 ? xo + (size_t)p * row : xn + (size_t)(p - L0) * row;
  }
  __device__ const uint8_t* z(int i) const {
    const int64_t p = p0 + i;
    return p < L0 ? zo + (size_t)(p % ring) * row : zn + (size_t)(p - L0) * row;
  }
};
template <bool BF16>
__device__ __forceinline__ BlockRows<BF16> block_rows(const AppendArgs& a, int b, const AppendSeq& q, int64_t j,
                                                      int m, int g) {
  constexpr int ES = BF16 ? 2 : 4;
  BlockRows<BF16> br;
  br.row = (size_t)a.width * ES;
  br.xo = a.kv_raw + (size_t)q.r0 * br.row + (size_t)g * 16;
  br.zo = a.z_tail + (size_t)b * a.ring * br.row + (size_t)g * 16;
  br.xn = a.x_new + (size_t)a.new_off[b] * br.row + (size_t)g * 16;
  br.zn = a.z_new + (size_t)a.new_off[b] * br.row + (size_t)g * 16;
  br.p0 = j * m;
  br.L0 = q.L0;
  br.ring = a.ring;
  return br;
}

template <bool BF16>
__global__ __launch_bounds__(256) void k_append_pool(AppendArgs a) {
  constexpr int N = Vec16<BF16>::N;
  constexpr int ES = BF16 ? 2 : 4;
  const int b = blockIdx.y;
  const int groups = a.width / N;
  const size_t row = (size_t)a.width * ES;
  const AppendSeq q = append_seq(a, b);
  const bool csa_narrow = a.m <= kPoolSeg, hca_narrow = a.m_hca <= kPoolSeg;
  if ((int)blockIdx.x < a.nb_narrow) {
    // narrow items: [rows to copy | short CSA blocks | short HCA blocks], a thread per 16 bytes
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int64_t item = gid / groups;
    const int g = (int)(gid - item * groups);
    if (item >= a.narrow_items) return;
    if (item < q.n) {
      if (q.L0 + item < q.cap)
        *reinterpret_cast<uint4*>(a.kv_raw + (size_t)(q.r0 + q.L0 + item) * row + (size_t)g * 16) =
            *reinterpret_cast<const uint4*>(a.x_new + (size_t)(a.new_off[b] + item) * row + (size_t)g * 16);
      return;
    }
    item -= q.n;
    bool hca;
    int64_t j;
    if (csa_narrow && item < q.nc) {
      hca = false;
      j = q.c0 + item;
    } else {
      item -= csa_narrow ? q.nc : 0;
      if (!hca_narrow || a.m_hca == 0 || item >= q.nh) return;
      hca = true;
      j = q.h0 + item;
    }
    const int m = hca ? a.m_hca : a.m;
    const int64_t pcap = hca ? a.hpool_off[b + 1] - a.hpool_off[b] : a.pool_off[b + 1] - a.pool_off[b];
    if (j >= pcap || (j + 1) * m > q.cap) return;
    const BlockRows<BF16> br = block_rows<BF16>(a, b, q, j, m, g);
    pool_block<BF16>(
        m, [&](int i) { return br.x(i); }, [&](int i) { return br.z(i); },
        (hca ? a.hpooled + (size_t)(a.hpool_off[b] + j) * row : a.pooled + (size_t)(a.pool_off[b] + j) * row) +
            (size_t)g * 16);
    return;
  }
  // one long block per workgroup: [long CSA blocks | long HCA blocks]
  int64_t w = (int64_t)blockIdx.x - a.nb_narrow;
  bool hca;
  int64_t j;
  if (!csa_narrow && w < q.nc) {
    hca = false;
    j = q.c0 + w;
  } else {
    w -= csa_narrow ? 0 : q.nc;
    if (hca_narrow || a.m_hca == 0 || w >= q.nh) return;
    hca = true;
    j = q.h0 + w;
  }
  const int m = hca ? a.m_hca : a.m;
  const int64_t pcap = hca ? a.hpool_off[b + 1] - a.hpool_off[b] : a.pool_off[b + 1] - a.pool_off[b];
  if (j >= pcap || (j + 1) * m > q.cap) return;  // uniform over the workgroup
  uint8_t* out = hca ? a.hpooled + (size_t)(a.hpool_off[b] + j) * row : a.pooled + (size_t)(a.pool_off[b] + j) * row;
  const int segs = (m + kPoolSeg - 1) / kPoolSeg;
  if (!a.wide_par) {
    for (int g = threadIdx.x; g < groups; g += blockDim.x) {
      const BlockRows<BF16> br = block_rows<BF16>(a, b, q, j, m, g);
      pool_block<BF16>(m, [&](int i) { return br.x(i); }, [&](int i) { return br.z(i); }, out + (size_t)g * 16);
    }
    return;
  }
  // every segment's state -> LDS [segs][groups], then each channel group folds them in order
  extern __shared__ __align__(16) uint8_t ap_sm[];
  PoolState<BF16>* part = reinterpret_cast<PoolState<BF16>*>(ap_sm);
  for (int t = threadIdx.x; t < segs * groups; t += blockDim.x) {
    const int sg = t / groups, g = t - sg * groups;
    const BlockRows<BF16> br = block_rows<BF16>(a, b, q, j, m, g);
    const int i0 = sg * kPoolSeg, i1 = i0 + kPoolSeg < m ? i0 + kPoolSeg : m;
    pool_segment<BF16>(i0, i1, [&](int i) { return br.x(i); }, [&](int i) { return br.z(i); }, part[t]);
  }
  __syncthreads();
  for (int g = threadIdx.x; g < groups; g += blockDim.x) {
    PoolState<BF16> st = part[g];
    for (int sg = 1; sg < segs; ++sg) pool_fold<BF16>(st, part[sg * groups + g]);
    pool_store<BF16>(st, out + (size_t)g * 16);
  }
}

template <bool BF16>
__global__ __launch_bounds__(256) void k_append_tail(AppendArgs a) {
  constexpr int N = Vec16<BF16>::N;
  constexpr int ES = BF16 ? 2 : 4;
  const int b = blockIdx.x;
  const int groups = a.width / N;
  const size_t row = (size_t)a.width * ES;
  const int64_t L0 = a.len[b];
  const int64_t n = a.new_off[b + 1] - a.new_off[b];
  const int64_t first = n > a.ring ? n - a.ring : 0;  // older new tokens are overwritten in the ring anyway
  const int64_t work = (n - first) * groups;
  for (int64_t t = threadIdx.x; t < work; t += blockDim.x) {
    const int64_t i = first + t / groups;
    const int g = (int)(t % groups);
    const int64_t p = L0 + i;
    *reinterpret_cast<uint4*>(a.z_tail + ((size_t)b * a.ring + (size_t)(p % a.ring)) * row + (size_t)g * 16) =
        *reinterpret_cast<const uint4*>(a.z_new + (size_t)(a.new_off[b] + i) * row + (size_t)g * 16);
  }
  __syncthreads();  // every thread has read len[b]
  if (threadIdx.x == 0) a.len[b] = L0 + n;
}

int launch_append(bool bf16, int n_seq, int width, const int64_t* tok_off, int64_t* len, const int64_t* new_off,
                  int64_t max_new, const void* x_new, const void* z_new, void* kv_raw, void* z_tail, int ring,
                  const int64_t* pool_off, int m, void* pooled, const int64_t* hpool_off, int m_hca, void* hpooled,
                  hipStream_t stream) {
  if (n_seq == 0) return 0;
  AppendArgs a{};
  a.tok_off = tok_off; a.len = len; a.new_off = new_off;
  a.x_new = (const uint8_t*)x_new; a.z_new = (const uint8_t*)z_new;
  a.kv_raw = (uint8_t*)kv_raw; a.z_tail = (uint8_t*)z_tail;
  a.pool_off = pool_off; a.hpool_off = hpool_off; a.pooled = (uint8_t*)pooled; a.hpooled = (uint8_t*)hpooled;
  a.width = width; a.ring = ring; a.m = m; a.m_hca = m_hca;
  const int N = bf16 ? 8 : 4;
  const int groups = width / N;
  // rows to copy plus the short blocks (at most kPoolSeg rows) max_new tokens can complete; long blocks
  // get a workgroup each, their segments pooled in parallel when their states fit 64 KB of LDS
  const int64_t nb_c = max_new / m + 1, nb_h = m_hca > 0 ? max_new / m_hca + 1 : 0;
  a.narrow_items = max_new + (m <= kPoolSeg ? nb_c : 0) + (m_hca > 0 && m_hca <= kPoolSeg ? nb_h : 0);
  const int64_t wide = (m > kPoolSeg ? nb_c : 0) + (m_hca > kPoolSeg ? nb_h : 0);
  a.nb_narrow = (int)((a.narrow_items * groups + 255) / 256);
  const int max_m = m > m_hca ? m : m_hca;
  const size_t state = bf16 ? sizeof(PoolState<true>) : sizeof(PoolState<false>);
  const size_t lds = (size_t)((max_m + kPoolSeg - 1) / kPoolSeg) * groups * state;
  a.wide_par = wide > 0 && lds <= 64 * 1024 ? 1 : 0;
  const size_t lds_launch = a.wide_par ? lds : 0;
  dim3 g1((unsigned)(a.nb_narrow + wide), (unsigned)n_seq);
  hipError_t e = launch(9, kProfStart, bf16 ? k_append_pool<true> : k_append_pool<false>, g1, dim3(256), lds_launch,
                        stream, a);
  if (e == hipSuccess)
    e = launch(9, kProfStop, bf16 ? k_append_tail<true> : k_append_tail<false>, dim3((unsigned)n_seq), dim3(256), 0,
               stream, a);
  return e == hipSuccess && hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace csa

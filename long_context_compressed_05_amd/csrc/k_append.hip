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
// The indexer key of each CSA block the append completes (an input vector of
// kdim elements, the block's key given by the caller: reading D9) is encoded
// in MXFP4 (quant_core.hpp) into the key cache row pool_off[b] + j.
//
// A short append is one launch: k_append_step for a decode-sized one (a few
// tokens per sequence, each task one per thread), else k_append_one (up to 64
// tokens per sequence): a workgroup per sequence copies the rows, pools the
// completed blocks, encodes their keys, and only then (after a barrier)
// writes the ring and advances the length.
// A longer one takes two kernels, in stream order:
//   k_append_pool  copies the new rows into the raw cache and pools the
//                  completed blocks: a block's older tokens come from the raw
//                  cache and the logit ring, its new tokens straight from the
//                  inputs (nothing this kernel reads is written by it).  A
//                  short block is pooled by one thread per 16 bytes of
//                  channels; a long one by several workgroups, each holding a
//                  slice of the channels, whose threads pool its 16-row
//                  segments in parallel and then fold them in order (the bulk
//                  kernel's order, so the bits agree)
//                  (and its last workgroups encode the completed blocks'
//                  keys, a thread per 32-element part)
//   k_append_tail  one workgroup per sequence: the newest min(n, ring)
//                  tokens' logits -> the ring, then the sequence's length
//                  advances
#include "common.hpp"
#include "kernels.hpp"
#include "pool_core.hpp"
#include "quant_core.hpp"

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
  const int64_t* kvec_off;  // [B+1] rows of kvec per sequence (null: no keys to encode)
  const uint8_t* kvec;      // [sum completed CSA blocks][kdim], KV dtype
  uint8_t* k_codes;         // [sum P][kdim / 2]
  uint8_t* k_scales;        // [sum P][kdim / 32]
  int kdim;
  int width, ring, m, m_hca;
  int64_t narrow_items;  // per sequence, at most: blocks of at most kPoolSeg rows (k_append_one: + rows to copy)
  int nb_copy;           // k_append_pool: workgroups copying the new rows (first in the grid)
  int nb_narrow;         // workgroups of the short blocks; then the long blocks' and the keys' workgroups
  int nb_wide;           // workgroups of long blocks; the workgroups after them encode keys (a thread per part)
  int wide_par;          // long blocks: segments pooled in parallel (1) or in one thread each (0)
  int wide_slices;       // k_append_pool: workgroups per long block (channel slices)
  int wide_units;        // k_append_pool: 4-byte channel units per slice
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
  if ((int)blockIdx.x < a.nb_copy) {
    // the new rows -> the raw cache: kCopyPer 16-byte pieces per thread, all loaded before any store
    constexpr int kCopyPer = 4;
    const int64_t pieces = q.n * groups;
    const int64_t t0 = (int64_t)blockIdx.x * blockDim.x * kCopyPer + threadIdx.x;
    if (t0 >= pieces) return;
    const uint8_t* src = a.x_new + (size_t)a.new_off[b] * row;
    uint8_t* dst = a.kv_raw + (size_t)(q.r0 + q.L0) * row;
    uint4 v[kCopyPer];
#pragma unroll
    for (int k = 0; k < kCopyPer; ++k) {
      const int64_t t = t0 + (int64_t)k * blockDim.x;
      const int64_t tt = t < pieces ? t : pieces - 1;
      const int64_t i = tt / groups;
      v[k] = *reinterpret_cast<const uint4*>(src + (size_t)i * row + (size_t)(tt - i * groups) * 16);
    }
#pragma unroll
    for (int k = 0; k < kCopyPer; ++k) {
      const int64_t t = t0 + (int64_t)k * blockDim.x;
      const int64_t i = t / groups;
      if (t < pieces && q.L0 + i < q.cap)
        *reinterpret_cast<uint4*>(dst + (size_t)i * row + (size_t)(t - i * groups) * 16) = v[k];
    }
    return;
  }
  if ((int)blockIdx.x < a.nb_copy + a.nb_narrow) {
    // short blocks: [short CSA blocks | short HCA blocks], a thread per 16 bytes
    const int64_t gid = (int64_t)(blockIdx.x - a.nb_copy) * blockDim.x + threadIdx.x;
    int64_t item = gid / groups;
    const int g = (int)(gid - item * groups);
    if (item >= a.narrow_items) return;
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
  if ((int)blockIdx.x >= a.nb_copy + a.nb_narrow + a.nb_wide) {  // keys: a thread per 32-element part
    if (!a.kvec) return;
    const int parts = a.kdim / 32;
    const int64_t t = (int64_t)(blockIdx.x - a.nb_copy - a.nb_narrow - a.nb_wide) * blockDim.x + threadIdx.x;
    const int64_t i = t / parts;
    const int p = (int)(t - i * parts);
    const int64_t r0 = a.kvec_off[b];
    const int64_t nk = a.kvec_off[b + 1] - r0 < q.nc ? a.kvec_off[b + 1] - r0 : q.nc;
    if (i >= nk || q.c0 + i >= a.pool_off[b + 1] - a.pool_off[b]) return;
    const size_t kr = (size_t)(a.pool_off[b] + q.c0 + i);
    mxfp4_block<BF16>(a.kvec + ((size_t)(r0 + i) * a.kdim + (size_t)p * 32) * ES,
                      a.k_codes + kr * (a.kdim / 2) + (size_t)p * 16, a.k_scales + kr * parts + p);
    return;
  }
  // long blocks: [long CSA blocks | long HCA blocks], each split into
  // wide_slices workgroups by 4-byte channel units; a workgroup pools every
  // 16-row segment of its units in parallel (each thread loading all of its
  // segment's rows before any arithmetic), then folds them in order
  const int64_t wb = (int64_t)blockIdx.x - a.nb_copy - a.nb_narrow;
  int64_t w = wb / a.wide_slices;
  const int slice = (int)(wb - w * a.wide_slices);
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
  constexpr int N4 = Vec4<BF16>::N;
  const int units = (int)(row / 4);
  const int u0 = slice * a.wide_units;
  const int nu = units - u0 < a.wide_units ? units - u0 : a.wide_units;
  if (nu <= 0) return;
  uint8_t* out = hca ? a.hpooled + (size_t)(a.hpool_off[b] + j) * row : a.pooled + (size_t)(a.pool_off[b] + j) * row;
  const int segs = (m + kPoolSeg - 1) / kPoolSeg;
  const uint8_t* xold = a.kv_raw + (size_t)q.r0 * row;
  const uint8_t* zring = a.z_tail + (size_t)b * a.ring * row;
  const uint8_t* xnew = a.x_new + (size_t)a.new_off[b] * row;
  const uint8_t* znew = a.z_new + (size_t)a.new_off[b] * row;
  const int64_t p_blk = j * m;
  const int slot0 = (int)(p_blk % a.ring);  // rows of the block are < m <= ring apart: one wrap at most
  extern __shared__ __align__(16) uint8_t ap_sm[];
  PoolSt<N4>* part = reinterpret_cast<PoolSt<N4>*>(ap_sm);
  for (int task = threadIdx.x; task < segs * nu; task += blockDim.x) {
    const int sg = task / nu, u = u0 + (task - sg * nu);
    const int i0 = sg * kPoolSeg;
    const int ns = m - i0 < kPoolSeg ? m - i0 : kPoolSeg;
    uint32_t xr[kPoolSeg], zr[kPoolSeg];
#pragma unroll
    for (int i = 0; i < kPoolSeg; ++i) {
      const int ii = i0 + (i < ns ? i : ns - 1);  // rows past the segment load its last row (unused)
      const int64_t p = p_blk + ii;
      const int so = slot0 + ii;
      const int slot = so < a.ring ? so : so - a.ring;
      const bool old = p < q.L0;
      xr[i] = *reinterpret_cast<const uint32_t*>((old ? xold + (size_t)p * row : xnew + (size_t)(p - q.L0) * row) +
                                                 (size_t)u * 4);
      zr[i] = *reinterpret_cast<const uint32_t*>((old ? zring + (size_t)slot * row : znew + (size_t)(p - q.L0) * row) +
                                                 (size_t)u * 4);
    }
    PoolSt<N4> st;
    pool_reset(st);
#pragma unroll
    for (int c0 = 0; c0 < kPoolSeg; c0 += 8) {
      if (c0 < ns) {
        float zz[8][N4], xx[8][N4];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          Vec4<BF16>::load(zr[c0 + i], zz[i]);
          Vec4<BF16>::load(xr[c0 + i], xx[i]);
        }
        pool_chunk(st, zz, xx, ns - c0 < 8 ? ns - c0 : 8);
      }
    }
#pragma unroll
    for (int i = 8; i < kPoolSeg; ++i) {  // rows of a second chunk the segment does not have
      consume_load(xr[i]);
      consume_load(zr[i]);
    }
    part[task] = st;
  }
  __syncthreads();
  for (int uu = threadIdx.x; uu < nu; uu += blockDim.x) {
    PoolSt<N4> st = part[uu];
    for (int sg = 1; sg < segs; ++sg) pool_fold(st, part[sg * nu + uu]);
    float o[N4];
    pool_result(st, o);
    *reinterpret_cast<uint32_t*>(out + (size_t)(u0 + uu) * 4) = Vec4<BF16>::pack(o);
  }
}

// the indexer keys of sequence b's completed CSA blocks (blocks j = c0 .. c0 + nc
// of the append) -> MXFP4 rows pool_off[b] + j, a thread per 32-element part
template <bool BF16>
__device__ __forceinline__ void append_keys(const AppendArgs& a, int b, const AppendSeq& q) {
  if (!a.kvec) return;
  constexpr int ES = BF16 ? 2 : 4;
  const int parts = a.kdim / 32;
  const int64_t r0 = a.kvec_off[b];
  const int64_t nk = a.kvec_off[b + 1] - r0 < q.nc ? a.kvec_off[b + 1] - r0 : q.nc;  // vectors given
  const int64_t pcap = a.pool_off[b + 1] - a.pool_off[b];
  for (int64_t t = threadIdx.x; t < nk * parts; t += blockDim.x) {
    const int64_t i = t / parts;
    const int p = (int)(t - i * parts);
    const int64_t j = q.c0 + i;
    if (j >= pcap) continue;
    const size_t kr = (size_t)(a.pool_off[b] + j);
    mxfp4_block<BF16>(a.kvec + ((size_t)(r0 + i) * a.kdim + (size_t)p * 32) * ES,
                      a.k_codes + kr * (a.kdim / 2) + (size_t)p * 16, a.k_scales + kr * parts + p);
  }
}

template <bool BF16>
__global__ __launch_bounds__(1024) void k_append_tail(AppendArgs a) {
  constexpr int N = Vec16<BF16>::N;
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int kPer = 4;  // 16-byte pieces per thread and pass, all loaded before any store
  const int b = blockIdx.x;
  const int groups = a.width / N;
  const size_t row = (size_t)a.width * ES;
  const int64_t L0 = a.len[b];
  const int64_t n = a.new_off[b + 1] - a.new_off[b];
  const int64_t first = n > a.ring ? n - a.ring : 0;  // older new tokens are overwritten in the ring anyway
  const int64_t work = (n - first) * groups;
  const int ring_slot0 = (int)((L0 + first) % a.ring);  // piece t: token first + t / groups, slot one wrap away
  const uint8_t* src = a.z_new + (size_t)(a.new_off[b] + first) * row;
  uint8_t* ring = a.z_tail + (size_t)b * a.ring * row;
  for (int64_t t0 = threadIdx.x; t0 < work; t0 += (int64_t)kPer * blockDim.x) {
    uint4 v[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int64_t t = t0 + (int64_t)k * blockDim.x;
      const int64_t tt = t < work ? t : work - 1;
      const int64_t i = tt / groups;
      v[k] = *reinterpret_cast<const uint4*>(src + (size_t)i * row + (size_t)(tt - i * groups) * 16);
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int64_t t = t0 + (int64_t)k * blockDim.x;
      if (t < work) {
        const int64_t i = t / groups;
        const int64_t so = ring_slot0 + i;  // i < ring: one wrap at most
        const int64_t slot = so < a.ring ? so : so - a.ring;
        *reinterpret_cast<uint4*>(ring + (size_t)slot * row + (size_t)(t - i * groups) * 16) = v[k];
      }
    }
  }
  __syncthreads();  // every thread has read len[b]
  if (threadIdx.x == 0) a.len[b] = L0 + n;
}

// The whole append of sequence b in one workgroup: rows, completed blocks
// (short ones a thread per channel group, long ones by parallel segments
// folded in order, as k_append_pool), their keys; then, after every read of
// the ring and of len[b] is done, the ring and the length.
template <bool BF16>
__global__ __launch_bounds__(256) void k_append_one(AppendArgs a) {
  constexpr int N = Vec16<BF16>::N;
  constexpr int ES = BF16 ? 2 : 4;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int groups = a.width / N;
  const size_t row = (size_t)a.width * ES;
  const AppendSeq q = append_seq(a, b);
  for (int64_t t = tid; t < q.n * groups; t += blockDim.x) {
    const int64_t i = t / groups;
    const int g = (int)(t - i * groups);
    if (q.L0 + i < q.cap)
      *reinterpret_cast<uint4*>(a.kv_raw + (size_t)(q.r0 + q.L0 + i) * row + (size_t)g * 16) =
          *reinterpret_cast<const uint4*>(a.x_new + (size_t)(a.new_off[b] + i) * row + (size_t)g * 16);
  }
  extern __shared__ __align__(16) uint8_t ap_sm[];
  PoolState<BF16>* part = reinterpret_cast<PoolState<BF16>*>(ap_sm);
  for (int kind = 0; kind < 2; ++kind) {
    const bool hca = kind == 1;
    const int m = hca ? a.m_hca : a.m;
    if (m == 0) continue;
    const int64_t j0 = hca ? q.h0 : q.c0, nb = hca ? q.nh : q.nc;
    const int64_t pcap = hca ? a.hpool_off[b + 1] - a.hpool_off[b] : a.pool_off[b + 1] - a.pool_off[b];
    uint8_t* dst = hca ? a.hpooled + (size_t)a.hpool_off[b] * row : a.pooled + (size_t)a.pool_off[b] * row;
    if (m <= kPoolSeg) {
      for (int64_t t = tid; t < nb * groups; t += blockDim.x) {
        const int64_t j = j0 + t / groups;
        const int g = (int)(t % groups);
        if (j >= pcap || (j + 1) * m > q.cap) continue;
        const BlockRows<BF16> br = block_rows<BF16>(a, b, q, j, m, g);
        pool_block<BF16>(m, [&](int i) { return br.x(i); }, [&](int i) { return br.z(i); },
                         dst + (size_t)j * row + (size_t)g * 16);
      }
      continue;
    }
    const int segs = (m + kPoolSeg - 1) / kPoolSeg;
    for (int64_t j = j0; j < j0 + nb; ++j) {  // uniform
      if (j >= pcap || (j + 1) * m > q.cap) continue;
      for (int t = tid; t < segs * groups; t += blockDim.x) {
        const int sg = t / groups, g = t - sg * groups;
        const BlockRows<BF16> br = block_rows<BF16>(a, b, q, j, m, g);
        const int i0 = sg * kPoolSeg, i1 = i0 + kPoolSeg < m ? i0 + kPoolSeg : m;
        pool_segment<BF16>(i0, i1, [&](int i) { return br.x(i); }, [&](int i) { return br.z(i); }, part[t]);
      }
      __syncthreads();
      for (int g = tid; g < groups; g += blockDim.x) {
        PoolState<BF16> st = part[g];
        for (int sg = 1; sg < segs; ++sg) pool_fold(st, part[sg * groups + g]);
        pool_store<BF16>(st, dst + (size_t)j * row + (size_t)g * 16);
      }
      __syncthreads();
    }
  }
  append_keys<BF16>(a, b, q);
  __syncthreads();  // every read of the ring and of len[b] is done
  const int64_t first = q.n > a.ring ? q.n - a.ring : 0;
  for (int64_t t = tid; t < (q.n - first) * groups; t += blockDim.x) {
    const int64_t i = first + t / groups;
    const int g = (int)(t % groups);
    const int64_t p = q.L0 + i;
    *reinterpret_cast<uint4*>(a.z_tail + ((size_t)b * a.ring + (size_t)(p % a.ring)) * row + (size_t)g * 16) =
        *reinterpret_cast<const uint4*>(a.z_new + (size_t)(a.new_off[b] + i) * row + (size_t)g * 16);
  }
  if (tid == 0) a.len[b] = q.L0 + q.n;
}

// A decode-sized append (kernel k_append_step): one workgroup of 1024 threads
// per sequence.  A wave issues about one vector instruction every few cycles,
// so the launch is bounded by the longest instruction stream of any wave, not
// by its few kilobytes of data: every thread pools 4 bytes of channels of one
// 16-row segment of the sequence's one long (HCA) block (segment t / units),
// and the other tasks go to distinct waves: 4 bytes of a short (CSA) block
// (threads from 0), one element of a completed block's key (from 256; the 32
// lanes of a key part find its scale together), 16 bytes of a new row (from
// 512; they also write the ring), and the long block's fold, 4 bytes of
// channels each (from 768).  Every load is issued before any arithmetic.
// After the barrier that ends every read of the ring and of len[b], the fold
// threads fold the segment states in order and the row threads write the
// ring.  The host takes this path when every task fits (at most one long
// block, m <= 8, at most 256 threads per task kind).
constexpr int kStepKeys = 256, kStepRows = 512, kStepFold = 768;  // first threads of the task kinds

template <bool BF16>
__global__ __launch_bounds__(1024) void k_append_step(AppendArgs a) {
  constexpr int N = Vec4<BF16>::N;
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int kMaxM = 8;  // short blocks (CSA) of at most 8 rows on this path
  const int b = blockIdx.x, t = threadIdx.x;
  const size_t row = (size_t)a.width * ES;
  const int units = (int)(row / 4), groups = (int)(row / 16);
  const AppendSeq q = append_seq(a, b);
  const uint8_t* xnew = a.x_new + (size_t)a.new_off[b] * row;
  const uint8_t* znew = a.z_new + (size_t)a.new_off[b] * row;
  const uint8_t* xold = a.kv_raw + (size_t)q.r0 * row;
  const uint8_t* zring = a.z_tail + (size_t)b * a.ring * row;
  // ---- issue every load
  // (1) the long block: rows [i0, i0 + ns) of segment t / units, unit t % units
  const int segs = a.m_hca > 0 ? (a.m_hca + kPoolSeg - 1) / kPoolSeg : 0;
  const int64_t hcap = a.m_hca > 0 ? a.hpool_off[b + 1] - a.hpool_off[b] : 0;
  const bool h_blk = q.nh > 0 && q.h0 < hcap && (q.h0 + 1) * a.m_hca <= q.cap;
  const bool h_do = h_blk && t < segs * units;
  const int hs = t / units, hu = t - hs * units;
  const int i0 = hs * kPoolSeg;
  const int ns = h_do ? (a.m_hca - i0 < kPoolSeg ? a.m_hca - i0 : kPoolSeg) : 0;
  uint32_t hx[kPoolSeg], hz[kPoolSeg];
  // ring slots: a block's first slot (uniform) plus the row's offset in the
  // block, which is below m_hca <= ring, so one wrap at most
  const int hslot0 = a.m_hca > 0 ? (int)((q.h0 * a.m_hca) % a.ring) : 0;
  if (h_do) {
    const int64_t p0 = q.h0 * a.m_hca + i0;
#pragma unroll
    for (int i = 0; i < kPoolSeg; ++i) {
      const int ii = i < ns ? i : ns - 1;  // rows past the segment load its last row (unused)
      const int64_t p = p0 + ii;
      const int so = hslot0 + i0 + ii;
      const int slot = so < a.ring ? so : so - a.ring;
      const bool old = p < q.L0;
      hx[i] = *reinterpret_cast<const uint32_t*>((old ? xold + (size_t)p * row : xnew + (size_t)(p - q.L0) * row) +
                                                 (size_t)hu * 4);
      hz[i] = *reinterpret_cast<const uint32_t*>((old ? zring + (size_t)slot * row : znew + (size_t)(p - q.L0) * row) +
                                                 (size_t)hu * 4);
    }
  }
  // (2) one short block's unit: block c0 + t / units (threads from 0)
  const int64_t cj = q.c0 + t / units;
  const int cu = t % units;
  const int64_t ccap = a.pool_off[b + 1] - a.pool_off[b];
  const bool c_do = t / units < q.nc && cj < ccap && (cj + 1) * a.m <= q.cap;
  uint32_t cx[kMaxM], cz[kMaxM];
  // the first short block's first slot (uniform); the blocks this append
  // completes span fewer than max_new + m <= 2 * ring rows from it
  const int cslot0 = (int)((q.c0 * a.m) % a.ring);
  if (c_do) {
    const int64_t p0 = cj * a.m;
    int cs = cslot0 + (t / units) * a.m;
    cs = cs < a.ring ? cs : cs - a.ring;
#pragma unroll
    for (int i = 0; i < kMaxM; ++i) {
      const int ii = i < a.m ? i : a.m - 1;
      const int64_t p = p0 + ii;
      int slot = cs + ii;
      slot = slot < a.ring ? slot : slot - a.ring;
      slot = slot < a.ring ? slot : slot - a.ring;
      const bool old = p < q.L0;
      cx[i] = *reinterpret_cast<const uint32_t*>((old ? xold + (size_t)p * row : xnew + (size_t)(p - q.L0) * row) +
                                                 (size_t)cu * 4);
      cz[i] = *reinterpret_cast<const uint32_t*>((old ? zring + (size_t)slot * row : znew + (size_t)(p - q.L0) * row) +
                                                 (size_t)cu * 4);
    }
  }
  // (3) 16 bytes of one new row (threads from 512)
  const int tr = t - kStepRows;
  const int64_t ri = tr >= 0 ? tr / groups : 0;
  const int rg = tr >= 0 ? tr % groups : 0;
  const bool r_do = tr >= 0 && ri < q.n;
  uint4 rx = make_uint4(0u, 0u, 0u, 0u), rz = make_uint4(0u, 0u, 0u, 0u);
  if (r_do) {
    rx = *reinterpret_cast<const uint4*>(xnew + (size_t)ri * row + (size_t)rg * 16);
    rz = *reinterpret_cast<const uint4*>(znew + (size_t)ri * row + (size_t)rg * 16);
  }
  // (4, issued last: its lanes
  // exchange values, which waits for every load) one element of a completed block's key vector (threads from 256: key
  // tk / kdim, element tk % kdim)
  const int tk = t - kStepKeys;
  const int64_t kvr = a.kvec ? a.kvec_off[b] : 0;
  const int64_t nk = a.kvec ? (a.kvec_off[b + 1] - kvr < q.nc ? a.kvec_off[b + 1] - kvr : q.nc) : 0;
  const int ki = a.kvec && tk >= 0 ? tk / a.kdim : 0, ke = a.kvec && tk >= 0 ? tk - ki * a.kdim : 0;
  const bool k_do = a.kvec && tk >= 0 && ki < nk && q.c0 + ki < ccap;  // the same for the 32 lanes of a part
  float kval = 0.f;
  if (k_do) {
    const uint8_t* src = a.kvec + ((size_t)(kvr + ki) * a.kdim + (size_t)ke) * ES;
    kval = BF16 ? __uint_as_float((uint32_t)*reinterpret_cast<const uint16_t*>(src) << 16)
                : *reinterpret_cast<const float*>(src);
  }
  // ---- compute and store
  extern __shared__ __align__(16) uint8_t ap_sm[];
  PoolSt<N>* part = reinterpret_cast<PoolSt<N>*>(ap_sm);
  if (h_do) {
    PoolSt<N> st;
    pool_reset(st);
#pragma unroll
    for (int c0 = 0; c0 < kPoolSeg; c0 += 8) {
      if (c0 < ns) {
        float zz[8][N], xx[8][N];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          Vec4<BF16>::load(hz[c0 + i], zz[i]);
          Vec4<BF16>::load(hx[c0 + i], xx[i]);
        }
        pool_chunk(st, zz, xx, ns - c0 < 8 ? ns - c0 : 8);
      }
    }
#pragma unroll
    for (int i = 8; i < kPoolSeg; ++i) {  // rows of a second chunk the segment does not have
      consume_load(hx[i]);
      consume_load(hz[i]);
    }
    part[t] = st;
  }
  if (c_do) {
    PoolSt<N> st;
    pool_reset(st);
    float zz[8][N], xx[8][N];
#pragma unroll
    for (int i = 0; i < kMaxM; ++i) {
      Vec4<BF16>::load(cz[i], zz[i]);
      Vec4<BF16>::load(cx[i], xx[i]);
    }
    pool_chunk(st, zz, xx, a.m);
    float o[N];
    pool_result(st, o);
    *reinterpret_cast<uint32_t*>(a.pooled + (size_t)(a.pool_off[b] + cj) * row + (size_t)cu * 4) = Vec4<BF16>::pack(o);
  }
  if (r_do && q.L0 + ri < q.cap)
    *reinterpret_cast<uint4*>(a.kv_raw + (size_t)(q.r0 + q.L0 + ri) * row + (size_t)rg * 16) = rx;
  if (r_do) {  // a row past the capacity is loaded but not stored
    consume_load(rx.x);
    consume_load(rz.x);
  }
  if (k_do) {
    uint32_t amax = __float_as_uint(kval) & 0x7fffffffu;
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) {
      const uint32_t v = (uint32_t)__shfl_xor((int)amax, o, 32);
      amax = v > amax ? v : amax;
    }
    const int e = mxfp4_exponent(amax);
    uint32_t w = mxfp4_code(kval, mxfp4_inverse(e)) << (4 * (ke & 7));
#pragma unroll
    for (int o = 4; o >= 1; o >>= 1) w |= (uint32_t)__shfl_xor((int)w, o, 32);
    const size_t kr = (size_t)(a.pool_off[b] + q.c0 + ki);
    if ((ke & 7) == 0) *reinterpret_cast<uint32_t*>(a.k_codes + kr * (a.kdim / 2) + (size_t)(ke >> 3) * 4) = w;
    if ((ke & 31) == 0) a.k_scales[kr * (a.kdim / 32) + (ke >> 5)] = (uint8_t)(e + 127);
  }
  __syncthreads();  // every segment state is in LDS; every read of the ring and of len[b] is done
  if (h_blk && t >= kStepFold && t < kStepFold + units) {
    {
      const int u = t - kStepFold;
      PoolSt<N> st = part[u];
      for (int sg = 1; sg < segs; ++sg) pool_fold(st, part[sg * units + u]);
      float o[N];
      pool_result(st, o);
      *reinterpret_cast<uint32_t*>(a.hpooled + (size_t)(a.hpool_off[b] + q.h0) * row + (size_t)u * 4) =
          Vec4<BF16>::pack(o);
    }
  }
  if (r_do) {  // new row ri < max_new <= ring: one wrap at most
    const int rs0 = (int)(q.L0 % a.ring) + (int)ri;
    const int slot = rs0 < a.ring ? rs0 : rs0 - a.ring;
    *reinterpret_cast<uint4*>(a.z_tail + ((size_t)b * a.ring + (size_t)slot) * row + (size_t)rg * 16) = rz;
  }
  if (t == 0) a.len[b] = q.L0 + q.n;
}

int launch_append(bool bf16, int n_seq, int width, const int64_t* tok_off, int64_t* len, const int64_t* new_off,
                  int64_t max_new, const void* x_new, const void* z_new, void* kv_raw, void* z_tail, int ring,
                  const int64_t* pool_off, int m, void* pooled, const int64_t* hpool_off, int m_hca, void* hpooled,
                  const int64_t* kvec_off, const void* kvec, int kdim, uint8_t* k_codes, uint8_t* k_scales,
                  hipStream_t stream) {
  if (n_seq == 0) return 0;
  AppendArgs a{};
  a.kvec_off = kvec_off; a.kvec = (const uint8_t*)kvec; a.kdim = kdim; a.k_codes = k_codes; a.k_scales = k_scales;
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
  // a short append (at most kOneMax new tokens per sequence, long blocks' segment
  // states in 64 KB): one launch, a workgroup per sequence
  constexpr int64_t kOneMax = 64;
  {
    // at most one task of each kind per thread of a 1024-thread workgroup: the
    // long block's segment units, the short blocks' units, key elements and
    // new rows' 16-byte groups
    const int64_t nc_max = max_new / m + 1;
    const int units = groups * 4;
    const int segs = m_hca > 0 ? (m_hca + kPoolSeg - 1) / kPoolSeg : 0;
    const size_t step_lds = (size_t)segs * units * (bf16 ? sizeof(PoolSt<2>) : sizeof(PoolSt<1>));
    const bool fits = m <= 8 && (m_hca == 0 || max_new <= m_hca) && max_new <= ring && max_new * groups <= 256 &&
                      nc_max * units <= 256 && (int64_t)segs * units <= 1024 && nc_max * kdim <= 256 &&
                      units <= 256 && step_lds <= 64 * 1024;
    if (fits) {
      const hipError_t e1 = launch(9, kProfBoth, bf16 ? k_append_step<true> : k_append_step<false>,
                                   dim3((unsigned)n_seq), dim3(1024), step_lds, stream, a);
      return e1 == hipSuccess && hipGetLastError() == hipSuccess ? 0 : -1;
    }
  }
  if (max_new <= kOneMax && (wide == 0 || a.wide_par)) {
    const hipError_t e1 = launch(9, kProfBoth, bf16 ? k_append_one<true> : k_append_one<false>, dim3((unsigned)n_seq),
                                 dim3(256), wide > 0 ? lds : 0, stream, a);
    return e1 == hipSuccess && hipGetLastError() == hipSuccess ? 0 : -1;
  }
  // long blocks: slices of wide_units channel units, segs x units tasks per
  // 256-thread workgroup (more segments than 256: a loop)
  {
    const int units = groups * 4;
    const int segs_max = (max_m + kPoolSeg - 1) / kPoolSeg;
    int U = 256 / segs_max;
    U = U < 1 ? 1 : (U > units ? units : U);
    a.wide_units = U;
    a.wide_slices = (units + U - 1) / U;
  }
  a.nb_wide = (int)(wide * a.wide_slices);
  // the multi-kernel path copies rows in workgroups of their own (4 pieces per thread)
  // and numbers the short blocks alone
  a.narrow_items -= max_new;
  a.nb_narrow = (int)((a.narrow_items * groups + 255) / 256);
  a.nb_copy = (int)((max_new * groups + 1023) / 1024);
  const size_t wide_lds = wide > 0 ? (size_t)((max_m + kPoolSeg - 1) / kPoolSeg) * a.wide_units *
                                         (bf16 ? sizeof(PoolSt<2>) : sizeof(PoolSt<1>)) : 0;
  const int64_t nb_keys = kvec ? (nb_c * (kdim / 32) + 255) / 256 : 0;
  dim3 g1((unsigned)(a.nb_copy + a.nb_narrow + a.nb_wide + nb_keys), (unsigned)n_seq);
  hipError_t e = launch(9, kProfStart, bf16 ? k_append_pool<true> : k_append_pool<false>, g1, dim3(256), wide_lds,
                        stream, a);
  if (e == hipSuccess)
    e = launch(9, kProfStop, bf16 ? k_append_tail<true> : k_append_tail<false>, dim3((unsigned)n_seq), dim3(1024), 0,
               stream, a);
  return e == hipSuccess && hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace csa

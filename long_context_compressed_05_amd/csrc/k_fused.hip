// Fused CSA + HCA decode step: one cooperative launch per step.
//
// The whole decode hot path runs in one persistent kernel whose workgroups
// are all co-resident.  Every workgroup w runs, in order:
//   score   chunk w of the (row, chunk) list: C pooled entries of one query's
//           visible range, MXFP4 MFMA scores -> sort keys kept in LDS, and an
//           LDS histogram of key >> 19; then it publishes a summary: the
//           nonzero bins at or above its local k-th bin (at most k pairs, and
//           every bin at or above the row's threshold bin is complete in it)
//   reduce  (chunk 0 of each row) merge the row's summaries, find the
//           threshold bin b1 and the count above it, publish them
//   emit    keys above bin b1 -> the chunk's list of definite indices, keys
//           in bin b1 -> its candidate list, both in ascending index order
//   items   taken from [CSA selected splits | CSA window splits | HCA splits |
//           CSA merges | HCA merges], item i on workgroup i mod G:
//     CSA selected split: the exact k-th key and lowest-index ties among the
//           row's candidates (in LDS), the row's selected set as an LDS
//           bitmap, the split's slice of the ascending list, attention over it
//     window / HCA split: attention over raw window rows / pooled HCA rows
//     merge: log-sum-exp merge of the row's split partials, 4 heads per item
//
// Synchronisation.  Cross-workgroup words are 64 bits: the launch's tag in
// the high half, the payload in the low half, written with device-coherent
// (sc1) stores and polled with device-coherent loads until the tag matches,
// so neither clearing nor store ordering between words is needed.  The tag is
// one more than the epoch word at the start of the workspace; the last
// workgroup to finish (a returning atomic on the exit count) advances it.
// Attention partials are plain data: the producer drains its stores
// (s_waitcnt vmcnt(0)) before it publishes the partial's tagged header.
// Every wait depends only on work of an earlier stage done by workgroups that
// are all resident and never wait for a later stage, so every wait ends; the
// waits are bounded anyway, and hitting the bound sets the error word (read
// and cleared by csa_hca_decode_check) and skips the workgroup's remaining work.
#include "attn_core.hpp"
#include "common.hpp"
#include "kernels.hpp"
#include "select_core.hpp"

namespace csa {

constexpr int kFMaxC = 3072;         // score entries per workgroup (keys in LDS)
constexpr int kFBins = 4096;         // key >> 19
constexpr int kFMaxSplit = 256;      // list positions per attention item
constexpr int kFCandLds = 4096;      // candidates staged in LDS
constexpr int kFMaxVisible = 262144;  // visible pooled entries per query (18-bit indices)
constexpr int kFMaxRows = 64;
constexpr int kFMaxSlots = 512;      // score chunks per row
constexpr int kFRankMax = 1024;      // candidates ranked by direct comparison (< kFCandLds - 16)
constexpr uint32_t kSpinLimit = 1u << 20;
constexpr int kTopPairs = 16;       // summary pairs per chunk read in the first round
constexpr int kThrStride = 64;      // threshold words 512 bytes apart (no shared line among pollers)

// control words at the start of the workspace
enum { W_EPOCH = 0, W_EXIT = 1, W_ERROR = 2, W_CTL = 64 };

// LDS layout (dynamic)
constexpr int kOffKeys = 0;                                 // uint32 [kFMaxC]; later slot prefix sums
constexpr int kOffIdx = kOffKeys + kFMaxC * 4;              // int32 [kFMaxSplit]
constexpr int kOffScr = kOffIdx + kFMaxSplit * 4;           // uint32 [64]
constexpr int kOffU = kOffScr + 64 * 4;                     // union region
constexpr int kOffCand = kOffU;                             // uint2 [kFCandLds]
constexpr int kOffRadix = kOffCand + kFCandLds * 8;         // uint32 [1024] radix bins
constexpr int kOffComp = kOffRadix + 1024 * 4;             // uint64 [kFRankMax + 16] order keys
constexpr int kSelEnd = kOffComp + (1024 + 16) * 8;
constexpr int kAttnEnd = kOffU + kAttnLdsBytes;
constexpr int kFusedLds = kSelEnd > kAttnEnd ? kSelEnd : kAttnEnd;
static_assert((kFMaxSlots + 1) * 3 * 4 <= kFMaxC * 4, "slot prefix sums alias the key region");
static_assert(kOffU % 16 == 0, "attention LDS must be 16-byte aligned");
static_assert(kFBins * 4 <= kFCandLds * 8, "histogram fits the union region");

// scratch word indices (0..39 are used by the block scans)
enum { S_TAG = 40, S_FLAG, S_B1, S_ABOVE, S_FLOOR, S_KSTAR, S_JSTAR };

struct FusedArgs {
  const int64_t* tok_off;
  const int64_t* q_pos;
  const int64_t* pool_off;
  const int64_t* hpool_off;
  int R, m, m_hca, H, k, W, W_hca;
  float scale_log2;
  int64_t max_pool, max_hpool;
  const uint8_t* q_codes;
  const uint8_t* q_scales;
  const float* w;
  const uint8_t* k_codes;
  const uint8_t* k_scales;
  const uint8_t* q;
  const uint8_t* kv_pool;
  const uint8_t* kv_hpool;
  const uint8_t* kv_raw;
  int32_t* idx;
  uint8_t* csa_out;
  float* csa_lse;
  uint8_t* hca_out;
  float* hca_lse;
  // plan
  int C, n_sc;                 // entries per score chunk, chunks per row
  int cs, n_cs_sel, n_cs_win;  // CSA split size, selected splits, window splits (per row)
  int hs, n_hs;                // HCA split size, splits per row
  int def_cap;                 // definite slots per chunk = min(C, k)
  // workspace
  uint32_t* ctl;
  uint64_t* sum_hdr;   // [R*n_sc]
  uint64_t* sum;       // [R*n_sc][k]
  uint64_t* thr;       // [R][kThrStride], word 0 used
  uint64_t* emit_hdr;  // [R*n_sc]
  uint64_t* defw;      // [R*n_sc][def_cap]
  uint64_t* candw;     // [R*n_sc][2*C]
  uint64_t* part_hdr;  // [R][n_cs_sel + n_cs_win + n_hs]
  float* csa_po;       // [R][n_cs][H][128]
  float* csa_pml;      // [R][n_cs][H][2]
  float* hca_po;
  float* hca_pml;
};

struct FRow {
  int64_t t, n_vis, n_vis_h, pbase, hbase, tok_base;
};

__device__ __forceinline__ FRow row_info(const FusedArgs& a, int r) {
  FRow f;
  f.t = a.q_pos[r];
  f.pbase = a.pool_off[r];
  f.hbase = a.hpool_off[r];
  f.tok_base = a.tok_off[r];
  const int64_t P = a.pool_off[r + 1] - f.pbase, Ph = a.hpool_off[r + 1] - f.hbase;
  const int64_t v = (f.t + 1) / a.m, vh = (f.t + 1) / a.m_hca;
  f.n_vis = v < P ? v : P;
  f.n_vis_h = vh < Ph ? vh : Ph;
  return f;
}

__device__ __forceinline__ uint32_t ld_dev(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void vm_drain() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ uint64_t tagged(uint32_t tag, uint32_t payload) {
  return ((uint64_t)tag << 32) | payload;
}

// Device-coherent (sc1) loads and stores through a buffer descriptor over the
// workspace: ordinary (non-atomic) memory operations, so the compiler keeps
// many of them in flight, with the same cache policy as agent-scope atomics.
typedef unsigned int v2u_t __attribute__((ext_vector_type(2)));
typedef unsigned int v4u_t __attribute__((ext_vector_type(4)));
constexpr int kSc1 = 16;  // cache-policy operand: sc1
struct Coh {
  __amdgpu_buffer_rsrc_t r;
  const uint8_t* base;
};
__device__ __forceinline__ Coh make_coh(const void* base) {
  return Coh{__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, 0x00020000),
             reinterpret_cast<const uint8_t*>(base)};
}
__device__ __forceinline__ uint32_t coh_off(const Coh& c, const void* p) {
  return (uint32_t)(reinterpret_cast<const uint8_t*>(p) - c.base);
}
__device__ __forceinline__ uint64_t coh_ld64(const Coh& c, const void* p) {
  const v2u_t v = __builtin_amdgcn_raw_buffer_load_b64(c.r, coh_off(c, p), 0, kSc1);
  return (uint64_t)v[0] | ((uint64_t)v[1] << 32);
}
__device__ __forceinline__ uint32_t coh_ld32(const Coh& c, const void* p) {
  return __builtin_amdgcn_raw_buffer_load_b32(c.r, coh_off(c, p), 0, kSc1);
}
__device__ __forceinline__ v4u_t coh_ld128(const Coh& c, const void* p) {
  return __builtin_amdgcn_raw_buffer_load_b128(c.r, coh_off(c, p), 0, kSc1);
}
__device__ __forceinline__ void coh_st128(const Coh& c, void* p, v4u_t v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, c.r, coh_off(c, p), 0, kSc1);
}

struct FCtx {
  const FusedArgs* a;
  uint8_t* smem;
  uint32_t* scr;
  uint32_t tag;
  Coh coh;
};

__device__ __forceinline__ void set_error(const FCtx& x) { atomicOr(x.a->ctl + W_ERROR, 1u); }
__device__ __forceinline__ bool error_seen(const FCtx& x) { return ld_dev(x.a->ctl + W_ERROR) != 0; }

// this thread spins until the tagged word at p carries the launch's tag and
// returns its payload; after the bound (or once an error was reported) it
// sets *fail and returns 0
__device__ __forceinline__ uint32_t poll_word(const FCtx& x, const uint64_t* p, bool* fail) {
  uint64_t v = coh_ld64(x.coh, p);
  uint32_t n = 0;
  while ((uint32_t)(v >> 32) != x.tag) {
    ++n;
    if (n >= kSpinLimit || ((n & 1023u) == 0 && error_seen(x))) {
      if (n >= kSpinLimit) set_error(x);
      *fail = true;
      return 0;
    }
    __builtin_amdgcn_s_sleep(2);
    v = coh_ld64(x.coh, p);
  }
  return (uint32_t)v;
}

// N tagged words read at once; words whose tag has not arrived yet are read
// again (all in one bounded retry loop)
template <int N>
__device__ __forceinline__ void read_tagged(const FCtx& x, const uint64_t* const (&p)[N], const bool (&use)[N],
                                            uint32_t (&out)[N], bool* fail) {
  uint64_t v[N];
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = use[i] ? coh_ld64(x.coh, p[i]) : tagged(x.tag, 0u);
  uint32_t n = 0;
  for (;;) {
    bool late = false;
#pragma unroll
    for (int i = 0; i < N; ++i) late |= (uint32_t)(v[i] >> 32) != x.tag;
    if (!late) break;
    if (++n >= kSpinLimit || ((n & 1023u) == 0 && error_seen(x))) {
      if (n >= kSpinLimit) set_error(x);
      *fail = true;
      break;
    }
    __builtin_amdgcn_s_sleep(2);
#pragma unroll
    for (int i = 0; i < N; ++i)
      if ((uint32_t)(v[i] >> 32) != x.tag) v[i] = coh_ld64(x.coh, p[i]);
  }
#pragma unroll
  for (int i = 0; i < N; ++i) out[i] = (uint32_t)v[i];
}

// exclusive scan of cnt[0..n) in place (LDS, n <= 1024), total at cnt[n]
__device__ __forceinline__ void block_exscan(uint32_t* cnt, int n, uint32_t* scr) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t v[4], tot = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = 4 * tid + i;
    v[i] = j < n ? cnt[j] : 0u;
    tot += v[i];
  }
  uint32_t incl = tot;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t u = __shfl_up(incl, off);
    if (lane >= off) incl += u;
  }
  if (lane == 63) scr[wave] = incl;
  __syncthreads();
  uint32_t run = incl - tot;
  for (int w2 = 0; w2 < wave; ++w2) run += scr[w2];
  const uint32_t all = scr[0] + scr[1] + scr[2] + scr[3];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = 4 * tid + i;
    if (j < n) cnt[j] = run;
    run += v[i];
  }
  if (tid == 0) cnt[n] = all;
  __syncthreads();
}

// index of the last entry of off[0..n) (ascending) that is <= i
__device__ __forceinline__ int upper_slot(const uint32_t* off, int n, uint32_t i) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= i) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// workgroup-wide: true when no thread's wait failed
__device__ __forceinline__ bool all_ok(const FCtx& x, bool fail) {
  if (threadIdx.x == 0) x.scr[S_FLAG] = 0;
  __syncthreads();
  if (fail) x.scr[S_FLAG] = 1;
  __syncthreads();
  const bool ok = x.scr[S_FLAG] == 0;
  __syncthreads();
  return ok;
}

// k-th largest bin over a 4096-bin LDS histogram (thread t owns bins 16t..16t+15):
// returns the bin, *above = entries in higher bins.  need >= 1 and <= total.
// Returns kFBins + 1 when the histogram holds fewer than need entries.
__device__ __forceinline__ uint32_t kth_bin(const uint32_t* hist, uint32_t need, uint32_t* scr, uint32_t* above) {
  const int tid = threadIdx.x;
  uint32_t cnt[16], tot = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    cnt[i] = hist[tid * 16 + i];
    tot += cnt[i];
  }
  if (tid == 0) scr[4] = 0xffffffffu;  // block_find_from_top's result word for 4 waves
  __syncthreads();
  int tstar;
  uint32_t ab;
  block_find_from_top(tot, need, scr, &tstar, &ab);
  if (tstar < 0) {
    *above = 0;
    return kFBins + 1;
  }
  if (tid == tstar) {  // walk this thread's bins downwards (unrolled: no dynamic register indexing)
    uint32_t cum = ab, asel = 0;
    int bsel = -1;
#pragma unroll
    for (int bi = 15; bi >= 1; --bi) {
      if (bsel < 0) {
        if (cum + cnt[bi] >= need) {
          bsel = bi;
          asel = cum;
        } else {
          cum += cnt[bi];
        }
      }
    }
    if (bsel < 0) {
      bsel = 0;
      asel = cum;
    }
    scr[S_B1] = (uint32_t)(tid * 16 + bsel);
    scr[S_ABOVE] = asel;
  }
  __syncthreads();
  const uint32_t b = scr[S_B1];
  *above = scr[S_ABOVE];
  __syncthreads();
  return b;
}

// ---------------------------------------------------------------------------
// score: chunk c of row r -> keys in LDS, local histogram, published summary
// ---------------------------------------------------------------------------
__device__ __forceinline__ void phase_score(const FCtx& x, int r, int c, const FRow& f, int64_t j0, int64_t j1) {
  const FusedArgs& a = *x.a;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, kb = lane >> 5;
  uint32_t* keys_s = reinterpret_cast<uint32_t*>(x.smem + kOffKeys);
  uint32_t* hist = reinterpret_cast<uint32_t*>(x.smem + kOffU);
  for (int i = tid; i < kFBins; i += 256) hist[i] = 0;
  // A operand: rows 0..3 = the query's 4 heads, K block lane/32
  v8i av = {0, 0, 0, 0, 0, 0, 0, 0};
  int asc = 127;
  if ((lane & 31) < 4) {
    const int64_t qrow = (int64_t)r * 4 + (lane & 3);
    const uint4 u = *reinterpret_cast<const uint4*>(a.q_codes + qrow * 32 + kb * 16);
    av[0] = (int)u.x; av[1] = (int)u.y; av[2] = (int)u.z; av[3] = (int)u.w;
    const int we = (int)((__float_as_uint(a.w[qrow]) >> 23) & 255u) - 127;
    asc = (int)a.q_scales[qrow * 2 + kb] + we;  // w_h = 2^we folded into the block scale
  }
  __syncthreads();  // histogram zeroed
  // 32-entry MFMA tiles; wave w takes tiles w, w+4, ...; 16 tiles per wave per batch of loads
  const int n = (int)(j1 - j0);
  const int ntiles = (n + 31) >> 5;
  for (int tb = 0; tb < ntiles; tb += 64) {
    uint4 kcv[16];
    int ksv[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int tile = tb + 4 * u + wave;
      const int64_t j = j0 + (int64_t)tile * 32 + (lane & 31);
      kcv[u] = make_uint4(0, 0, 0, 0);
      ksv[u] = 127;
      if (tile < ntiles && j < j1) {
        kcv[u] = *reinterpret_cast<const uint4*>(a.k_codes + (f.pbase + j) * 32 + kb * 16);
        ksv[u] = a.k_scales[(f.pbase + j) * 2 + kb];
      }
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int tile = tb + 4 * u + wave;
      if (tile >= ntiles) continue;  // uniform per wave
      v8i bv = {(int)kcv[u].x, (int)kcv[u].y, (int)kcv[u].z, (int)kcv[u].w, 0, 0, 0, 0};
      v16f acc = {};
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 4, 4, 0, asc, 0, ksv[u]);
      const int jl = tile * 32 + lane;  // local index
      if (lane < 32 && jl < n) {
        const float r0 = __int_as_float(max(__float_as_int(acc[0]), 0));
        const float r1 = __int_as_float(max(__float_as_int(acc[1]), 0));
        const float r2 = __int_as_float(max(__float_as_int(acc[2]), 0));
        const float r3 = __int_as_float(max(__float_as_int(acc[3]), 0));
        const uint32_t key = __float_as_uint((r0 + r1) + (r2 + r3));
        keys_s[jl] = key;
        atomicAdd(&hist[key >> 19], 1u);
      }
    }
  }
  __syncthreads();
  // local k-th bin: report the nonzero bins at or above it
  int bw = 0;
  const uint32_t need = n < a.k ? (uint32_t)n : (uint32_t)a.k;
  if (need > 0) {
    uint32_t ab;
    bw = (int)kth_bin(hist, need, x.scr, &ab);
  }
  uint32_t cnt[16], mine = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    cnt[i] = hist[tid * 16 + i];
    mine += (tid * 16 + i >= bw && cnt[i] != 0) ? 1u : 0u;
  }
  // output position: pairs of higher threads come first (descending bins)
  uint32_t s = mine;  // inclusive suffix sum within the wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t v = __shfl_down(s, off);
    if (lane + off < 64) s += v;
  }
  if (lane == 0) x.scr[8 + wave] = s;
  __syncthreads();
  uint32_t higher = 0;
  for (int w2 = wave + 1; w2 < 4; ++w2) higher += x.scr[8 + w2];
  uint32_t pos = s - mine + higher;
  const uint32_t npairs = x.scr[8] + x.scr[9] + x.scr[10] + x.scr[11];
  const size_t slot = (size_t)r * a.n_sc + c;
  uint64_t* dst = a.sum + slot * a.k;
  for (int i = 15; i >= 0; --i) {
    const int bin = tid * 16 + i;
    if (bin >= bw && cnt[i] != 0) st_dev64(dst + pos++, tagged(x.tag, ((uint32_t)bin << 20) | cnt[i]));
  }
  if (tid == 0) st_dev64(a.sum_hdr + slot, tagged(x.tag, npairs));
  __syncthreads();
}

// ---------------------------------------------------------------------------
// reduce (chunk 0 of row r): threshold bin of the row
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool phase_reduce(const FCtx& x, int r, const FRow& f) {
  const FusedArgs& a = *x.a;
  const int tid = threadIdx.x;
  uint32_t* hist = reinterpret_cast<uint32_t*>(x.smem + kOffU);
  uint32_t* np = hist + kFBins;  // pairs per chunk
  for (int i = tid; i < kFBins; i += 256) hist[i] = 0;
  if (tid == 0) x.scr[S_FLOOR] = 0;
  bool fail = false;
  for (int sl = tid; sl < a.n_sc && !fail; sl += 256) np[sl] = poll_word(x, a.sum_hdr + (size_t)r * a.n_sc + sl, &fail);
  if (!all_ok(x, fail)) return false;
  const uint64_t* rowsum = a.sum + (size_t)r * a.n_sc * a.k;
  // Round 1: the top kTopPairs pairs of every chunk.  The counts are then complete at and
  // above the highest last-read bin of the truncated chunks (the floor).
  const int nq = a.n_sc * kTopPairs;
  for (int base = 0; base < nq && !fail; base += 256 * 8) {
    const uint64_t* pp[8];
    bool use[8];
    uint32_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = base + tid + 256 * u, sl = i / kTopPairs, j = i % kTopPairs;
      use[u] = i < nq && (uint32_t)j < np[sl < a.n_sc ? sl : 0];
      pp[u] = rowsum + (size_t)(use[u] ? sl : 0) * a.k + (use[u] ? j : 0);
    }
    read_tagged<8>(x, pp, use, v, &fail);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (!use[u] || fail) continue;
      const int i = base + tid + 256 * u, sl = i / kTopPairs, j = i % kTopPairs;
      atomicAdd(&hist[v[u] >> 20], v[u] & 0xfffffu);
      if (j == kTopPairs - 1 && np[sl] > (uint32_t)kTopPairs) atomicMax(&x.scr[S_FLOOR], v[u] >> 20);
    }
  }
  if (!all_ok(x, fail)) return false;
  const uint32_t k_eff = (uint32_t)(f.n_vis < a.k ? f.n_vis : a.k);
  uint32_t b1 = kFBins, above = 0;  // k_eff == 0: nothing is selected
  if (k_eff > 0) {
    const uint32_t floor_bin = x.scr[S_FLOOR];
    b1 = kth_bin(hist, k_eff, x.scr, &above);
    if (b1 > kFBins || b1 < floor_bin) {
      // Round 2 (rare): the rest of the truncated chunks' pairs, one chunk per thread
      for (int sl = tid; sl < a.n_sc && !fail; sl += 256) {
        const uint32_t n = np[sl];
        for (uint32_t j0 = kTopPairs; j0 < n && !fail; j0 += 8) {
          const uint64_t* pp[8];
          bool use[8];
          uint32_t v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            use[u] = j0 + u < n;
            pp[u] = rowsum + (size_t)sl * a.k + (use[u] ? j0 + u : 0);
          }
          read_tagged<8>(x, pp, use, v, &fail);
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (use[u] && !fail) atomicAdd(&hist[v[u] >> 20], v[u] & 0xfffffu);
        }
      }
      if (!all_ok(x, fail)) return false;
      b1 = kth_bin(hist, k_eff, x.scr, &above);
    }
  }
  if (tid == 0) st_dev64(a.thr + (size_t)r * kThrStride, tagged(x.tag, (above << 13) | b1));
  __syncthreads();
  return true;
}

// ---------------------------------------------------------------------------
// emit: definite indices and candidates of chunk c, ascending
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool phase_emit(const FCtx& x, int r, int c, int n) {
  const FusedArgs& a = *x.a;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  bool fail = false;
  if (tid == 0) x.scr[S_B1] = poll_word(x, a.thr + (size_t)r * kThrStride, &fail) & 0x1fffu;
  if (!all_ok(x, fail)) return false;
  const uint32_t b1 = x.scr[S_B1];
  const uint32_t* keys_s = reinterpret_cast<const uint32_t*>(x.smem + kOffKeys);
  // thread t owns local entries [t*E, t*E + E)
  const int E = (n + 255) / 256;
  const int e0 = tid * E;
  uint32_t ng = 0, ne = 0;
  for (int i = 0; i < E; ++i) {
    const int jl = e0 + i;
    if (jl < n) {
      const uint32_t bin = keys_s[jl] >> 19;
      ng += bin > b1 ? 1u : 0u;
      ne += bin == b1 ? 1u : 0u;
    }
  }
  uint32_t sg = ng, se = ne;  // inclusive prefix within the wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t vg = __shfl_up(sg, off), ve = __shfl_up(se, off);
    if (lane >= off) {
      sg += vg;
      se += ve;
    }
  }
  if (lane == 63) {
    x.scr[wave] = sg;
    x.scr[4 + wave] = se;
  }
  __syncthreads();
  uint32_t pg = sg - ng, pe = se - ne;
  for (int w2 = 0; w2 < wave; ++w2) {
    pg += x.scr[w2];
    pe += x.scr[4 + w2];
  }
  const uint32_t tg = x.scr[0] + x.scr[1] + x.scr[2] + x.scr[3];
  const uint32_t te = x.scr[4] + x.scr[5] + x.scr[6] + x.scr[7];
  const size_t slot = (size_t)r * a.n_sc + c;
  uint64_t* dd = a.defw + slot * a.def_cap;
  uint64_t* cd = a.candw + slot * 2 * a.C;
  const uint32_t jbase = (uint32_t)c * (uint32_t)a.C;
  for (int i = 0; i < E; ++i) {
    const int jl = e0 + i;
    if (jl < n) {
      const uint32_t key = keys_s[jl];
      const uint32_t bin = key >> 19;
      if (bin > b1) {
        st_dev64(dd + pg++, tagged(x.tag, jbase + (uint32_t)jl));
      } else if (bin == b1) {
        st_dev64(cd + 2 * pe, tagged(x.tag, jbase + (uint32_t)jl));
        st_dev64(cd + 2 * pe + 1, tagged(x.tag, key));
        ++pe;
      }
    }
  }
  if (tid == 0) st_dev64(a.emit_hdr + slot, tagged(x.tag, (tg << 12) | te));
  __syncthreads();
  return true;
}

// ---------------------------------------------------------------------------
// attention items
// ---------------------------------------------------------------------------
// unnormalised partial (O, m in log2 units, l) of one split, then its tagged header
__device__ __forceinline__ void write_partial(const FCtx& x, AttnState<1>& st, int r, int pi, bool hca) {
  const FusedArgs& a = *x.a;
  const int n_cs = a.n_cs_sel + a.n_cs_win;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l16 = lane & 15, g = lane >> 4;
  float* po;
  float* pml;
  if (hca) {
    const size_t pb = ((size_t)r * a.n_hs + pi) * a.H;
    po = a.hca_po + pb * 128;
    pml = a.hca_pml + pb * 2;
  } else {
    const size_t pb = ((size_t)r * n_cs + pi) * a.H;
    po = a.csa_po + pb * 128;
    pml = a.csa_pml + pb * 2;
  }
  if (wave < (a.H >> 4)) {
    const float l = xor32_sum(xor16_sum(st.l_run[0]));
    const int head = 16 * wave + l16;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const v4f o = st.O[0][mt];
      const v4u_t u = {__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]), __float_as_uint(o[3])};
      coh_st128(x.coh, po + (size_t)head * 128 + 16 * mt + 4 * g, u);
    }
    if (g == 0)
      __builtin_amdgcn_raw_buffer_store_b64(v2u_t{__float_as_uint(st.m_run[0]), __float_as_uint(l)}, x.coh.r,
                                            coh_off(x.coh, pml + head * 2), 0, kSc1);
  }
  vm_drain();
  __syncthreads();
  if (threadIdx.x == 0)
    st_dev64(a.part_hdr + (size_t)r * (n_cs + a.n_hs) + (hca ? n_cs : 0) + pi, tagged(x.tag, 1u));
}

// Selection for CSA split s of row r: the split's slice of the ascending
// selected list -> idx_s (and, for split 0, the whole row -> idx).  false on a
// failed wait.
//
// The row's selected set is every definite index plus the candidates (keys in
// the threshold bin) that come first in (key descending, index ascending)
// order, need = k_eff - definites of them.  The need-th candidate (K*, j*) is
// found by ranking every candidate against all others (at most kFRankMax
// candidates) or by a radix select; candidate (key, j) is chosen when
// key > K* or (key == K* and j <= j*).  Chunks cover ascending index ranges,
// so the position of a selected index is the selected count of the earlier
// chunks plus its rank among its own chunk's definites and chosen candidates,
// both of which are stored in ascending order.
__device__ __forceinline__ bool select_split(const FCtx& x, int r, int s, const FRow& f) {
  const FusedArgs& a = *x.a;
  const int tid = threadIdx.x;
  const int64_t p_begin = (int64_t)s * a.cs;
  const int64_t p_end = p_begin + a.cs < a.k ? p_begin + a.cs : a.k;
  const int k_eff = (int)(f.n_vis < a.k ? f.n_vis : a.k);
  int32_t* idx_s = reinterpret_cast<int32_t*>(x.smem + kOffIdx);
  int32_t* idx_out = a.idx + (size_t)r * a.k;
  for (int i = tid; i < a.cs; i += 256) idx_s[i] = -1;
  const bool needs_sel = (s == 0) || (p_begin < k_eff);
  if (needs_sel && k_eff > 0) {
    // per-chunk counts -> exclusive prefix sums (LDS, over the key region)
    uint32_t* def_off = reinterpret_cast<uint32_t*>(x.smem + kOffKeys);
    uint32_t* cand_off = def_off + (kFMaxSlots + 1);
    uint32_t* sel_off = cand_off + (kFMaxSlots + 1);
    bool fail = false;
    if (tid == 0) x.scr[S_B1] = poll_word(x, a.thr + (size_t)r * kThrStride, &fail) & 0x1fffu;
    for (int sl = tid; sl < a.n_sc && !fail; sl += 256) {
      const uint32_t v = poll_word(x, a.emit_hdr + (size_t)r * a.n_sc + sl, &fail);
      def_off[sl] = v >> 12;
      cand_off[sl] = v & 0xfffu;
    }
    if (!all_ok(x, fail)) return false;
    const uint32_t b1 = x.scr[S_B1];
    block_exscan(def_off, a.n_sc, x.scr);
    block_exscan(cand_off, a.n_sc, x.scr);
    const uint32_t n_def = def_off[a.n_sc], n_c = cand_off[a.n_sc];
    const uint32_t need = (uint32_t)k_eff - n_def;
    uint2* cand_s = reinterpret_cast<uint2*>(x.smem + kOffCand);
    const bool in_lds = n_c <= (uint32_t)kFCandLds;
    auto cand_src = [&](uint32_t i) -> const uint64_t* {
      const int sl = upper_slot(cand_off, a.n_sc, i);
      return a.candw + ((size_t)r * a.n_sc + sl) * 2 * a.C + 2 * (i - cand_off[sl]);
    };
    // candidate i of the row: (key, index)
    auto cand_global = [&](uint32_t i, bool* fl) -> uint2 {
      const uint64_t* src = cand_src(i);
      const uint32_t j = poll_word(x, src, fl);
      const uint32_t key = poll_word(x, src + 1, fl);
      return make_uint2(key, j);
    };
    if (in_lds) {  // one chunk per thread, 8 candidates (16 words) per round
      for (int sl = tid; sl < a.n_sc && !fail; sl += 256) {
        const uint32_t c0 = cand_off[sl], nc = cand_off[sl + 1] - c0;
        const uint64_t* src = a.candw + ((size_t)r * a.n_sc + sl) * 2 * a.C;
        for (uint32_t i0 = 0; i0 < nc && !fail; i0 += 8) {
          const uint64_t* pp[16];
          bool use[16];
          uint32_t v[16];
#pragma unroll
          for (int u = 0; u < 16; ++u) {
            use[u] = i0 + (u >> 1) < nc;
            pp[u] = src + (use[u] ? 2 * (i0 + (u >> 1)) + (u & 1) : 0);
          }
          read_tagged<16>(x, pp, use, v, &fail);
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (use[2 * u]) cand_s[c0 + i0 + u] = make_uint2(v[2 * u + 1], v[2 * u]);
        }
      }
    }
    if (!all_ok(x, fail)) return false;
    // the need-th candidate (K*, j*)
    if (tid == 0) {
      x.scr[S_KSTAR] = 0xffffffffu;  // need == 0: no candidate is chosen
      x.scr[S_JSTAR] = 0;
    }
    __syncthreads();
    if (need > 0) {
      if (in_lds && n_c <= (uint32_t)kFRankMax) {
        // order key (key, ~index): larger ranks first.  Padded to a multiple of 16 with
        // zero keys, which rank after every candidate.
        uint64_t* comp = reinterpret_cast<uint64_t*>(x.smem + kOffComp);
        const uint32_t n_pad = (n_c + 15) & ~15u;
        for (uint32_t i = tid; i < n_pad; i += 256)
          comp[i] = i < n_c ? ((uint64_t)cand_s[i].x << 32) | (uint32_t)~cand_s[i].y : 0ull;
        __syncthreads();
        for (uint32_t i = tid; i < n_c; i += 256) {
          const uint64_t ci = comp[i];
          uint32_t rank = 0;
          for (uint32_t j0 = 0; j0 < n_pad; j0 += 16) {
            uint64_t q[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) q[u] = comp[j0 + u];
#pragma unroll
            for (int u = 0; u < 16; ++u) rank += q[u] > ci ? 1u : 0u;
          }
          if (rank == need - 1) {
            x.scr[S_KSTAR] = (uint32_t)(ci >> 32);
            x.scr[S_JSTAR] = ~(uint32_t)ci;
          }
        }
      } else {
        // every candidate key shares its top 13 bits (bin b1); every index < 2^18, so ~index
        // starts with 14 ones.  A tie class too large for LDS is re-read from the workspace.
        bool fl = false;
        uint32_t* bins = reinterpret_cast<uint32_t*>(x.smem + kOffRadix);
        auto cand = [&](uint32_t i) -> uint2 { return in_lds ? cand_s[i] : cand_global(i, &fl); };
        uint32_t rr, r2;
        const uint32_t ks = radix_select_desc_low(n_c, need, 19, b1 << 19, [&](uint32_t i) { return cand(i).x; },
                                                  [&](uint32_t) { return true; }, &rr, bins, x.scr);
        const uint32_t js = radix_select_desc_low(n_c, rr, 18, 0xfffc0000u, [&](uint32_t i) { return ~cand(i).y; },
                                                  [&](uint32_t i) { return cand(i).x == ks; }, &r2, bins, x.scr);
        if (tid == 0) {
          x.scr[S_KSTAR] = ks;
          x.scr[S_JSTAR] = ~js;
        }
      }
    }
    __syncthreads();
    const uint32_t kstar = x.scr[S_KSTAR], jstar = x.scr[S_JSTAR];
    auto chosen = [&](uint2 c) { return c.x > kstar || (c.x == kstar && c.y <= jstar); };
    // selected count per chunk -> offsets
    for (int sl = tid; sl < a.n_sc; sl += 256) {
      uint32_t cnt = def_off[sl + 1] - def_off[sl];
      const uint32_t c0 = cand_off[sl], c1 = cand_off[sl + 1];
      for (uint32_t i = c0; i < c1; ++i) {
        bool fl = false;
        cnt += chosen(in_lds ? cand_s[i] : cand_global(i, &fl)) ? 1u : 0u;
      }
      sel_off[sl] = cnt;
    }
    __syncthreads();
    block_exscan(sel_off, a.n_sc, x.scr);
    // chunks overlapping this split's positions (every chunk for split 0): ordered merge
    for (int sl = tid; sl < a.n_sc && !fail; sl += 256) {
      uint32_t pos = sel_off[sl];
      const uint32_t pend = sel_off[sl + 1];
      if (pos == pend || (s != 0 && ((int64_t)pos >= p_end || (int64_t)pend <= p_begin))) continue;
      auto emit = [&](uint32_t j) {
        if ((int64_t)pos >= p_begin && (int64_t)pos < p_end) idx_s[pos - p_begin] = (int32_t)j;
        if (s == 0 && pos < (uint32_t)a.k) idx_out[pos] = (int32_t)j;
        ++pos;
      };
      const uint32_t nd = def_off[sl + 1] - def_off[sl];
      const uint32_t c1 = cand_off[sl + 1];
      uint32_t m = cand_off[sl];
      auto next_chosen = [&]() -> uint32_t {  // index of the next chosen candidate, or ~0
        for (; m < c1; ++m) {
          bool fl = false;
          const uint2 c = in_lds ? cand_s[m] : cand_global(m, &fl);
          if (chosen(c)) return c.y;
        }
        return 0xffffffffu;
      };
      uint32_t cn = next_chosen();
      const uint64_t* src = a.defw + ((size_t)r * a.n_sc + sl) * a.def_cap;
      for (uint32_t i0 = 0; i0 < nd && !fail; i0 += 16) {
        const uint64_t* pp[16];
        bool use[16];
        uint32_t v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          use[u] = i0 + u < nd;
          pp[u] = src + (use[u] ? i0 + u : 0);
        }
        read_tagged<16>(x, pp, use, v, &fail);
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          if (!use[u]) continue;
          while (cn < v[u]) {
            emit(cn);
            ++m;
            cn = next_chosen();
          }
          emit(v[u]);
        }
      }
      while (cn != 0xffffffffu) {
        emit(cn);
        ++m;
        cn = next_chosen();
      }
    }
    if (!all_ok(x, fail)) return false;
  }
  if (s == 0)
    for (int i = k_eff + tid; i < a.k; i += 256) idx_out[i] = -1;
  __syncthreads();
  return true;
}

// Attention item: CSA selected split (kind 0, rows through idx_s), CSA window
// split (kind 1) or HCA split (kind 2) of row r, then its partial.
__device__ __forceinline__ void attend_item(const FCtx& x, int r, int kind, int s, const FRow& f) {
  const FusedArgs& a = *x.a;
  int64_t p_begin, p_end;
  int pi = s;
  if (kind == 0) {
    p_begin = (int64_t)s * a.cs;
    p_end = p_begin + a.cs < a.k ? p_begin + a.cs : a.k;
  } else if (kind == 1) {
    p_begin = (int64_t)s * a.cs;
    p_end = p_begin + a.cs < a.W ? p_begin + a.cs : a.W;
    pi = a.n_cs_sel + s;
  } else {
    const int64_t list_len = a.max_hpool + a.W_hca;
    p_begin = (int64_t)s * a.hs;
    p_end = p_begin + a.hs < list_len ? p_begin + a.hs : list_len;
  }
  const int32_t* idx_s = reinterpret_cast<const int32_t*>(x.smem + kOffIdx);
  constexpr size_t RB = 2 * 128 * 2;
  auto rowptr = [&](int64_t p) -> const uint8_t* {
    if (kind == 0) {
      const int32_t j = idx_s[p - p_begin];
      return j >= 0 ? a.kv_pool + (size_t)(f.pbase + j) * RB : nullptr;
    }
    if (kind == 1) {
      const int64_t u = f.t - a.W + 1 + p;
      return u >= 0 ? a.kv_raw + (size_t)(f.tok_base + u) * RB : nullptr;
    }
    if (p < a.max_hpool) return p < f.n_vis_h ? a.kv_hpool + (size_t)(f.hbase + p) * RB : nullptr;
    const int64_t u = f.t - a.W_hca + 1 + (p - a.max_hpool);
    return u >= 0 ? a.kv_raw + (size_t)(f.tok_base + u) * RB : nullptr;
  };
  AttnState<1> st;
  attn_init<1>(st, a.q + (size_t)r * a.H * 128 * 2, a.H);
  attn_run<1>(st, a.H, a.scale_log2, p_begin, p_end, rowptr, x.smem + kOffU);
  write_partial(x, st, r, pi, kind == 2);
}

// merge of 4 heads (h0 .. h0+3) of one row: thread = (head, 2 dims)
__device__ __forceinline__ void item_merge(const FCtx& x, bool hca, int r, int h0) {
  const FusedArgs& a = *x.a;
  const int tid = threadIdx.x;
  const int n_cs = a.n_cs_sel + a.n_cs_win;
  const int n = hca ? a.n_hs : n_cs;
  const uint64_t* hdr = a.part_hdr + (size_t)r * (n_cs + a.n_hs) + (hca ? n_cs : 0);
  bool fail = false;
  for (int s = tid; s < n && !fail; s += 256) (void)poll_word(x, hdr + s, &fail);
  if (!all_ok(x, fail)) return;
  const float* po = hca ? a.hca_po : a.csa_po;
  const float* pml = hca ? a.hca_pml : a.csa_pml;
  uint8_t* out = hca ? a.hca_out : a.csa_out;
  float* lse = hca ? a.hca_lse : a.csa_lse;
  // (m, l) of every split for the 4 heads -> LDS [4][n]
  uint2* ml_s = reinterpret_cast<uint2*>(x.smem + kOffU);
  for (int q0 = 0; q0 < 4 * n; q0 += 256 * 8) {
    uint64_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int q = q0 + tid + 256 * u;
      v[u] = q < 4 * n ? coh_ld64(x.coh, pml + (((size_t)r * n + (q >> 2)) * a.H + h0 + (q & 3)) * 2) : 0ull;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int q = q0 + tid + 256 * u;
      if (q < 4 * n) ml_s[(q & 3) * n + (q >> 2)] = make_uint2((uint32_t)v[u], (uint32_t)(v[u] >> 32));
    }
  }
  __syncthreads();
  const int hh = tid >> 6, h = h0 + hh, d = (tid & 63) * 2;
  const uint2* mlh = ml_s + hh * n;
  float M = -INFINITY;
  for (int s = 0; s < n; ++s) M = fmaxf(M, __uint_as_float(mlh[s].x));
  float L = 0.f, acc0 = 0.f, acc1 = 0.f;
  if (M != -INFINITY) {
    for (int s0 = 0; s0 < n; s0 += 32) {
      uint64_t ov[32];
#pragma unroll
      for (int u = 0; u < 32; ++u) {
        const int s = s0 + u;
        ov[u] = s < n && __uint_as_float(mlh[s].x) != -INFINITY
                    ? coh_ld64(x.coh, po + (((size_t)r * n + s) * a.H + h) * 128 + d)
                    : 0ull;
      }
#pragma unroll
      for (int u = 0; u < 32; ++u) {
        const int s = s0 + u;
        if (s >= n) continue;
        const float ms = __uint_as_float(mlh[s].x);
        if (ms == -INFINITY) continue;
        const float wgt = fast_exp2(ms - M);
        L = fmaf(wgt, __uint_as_float(mlh[s].y), L);
        acc0 = fmaf(wgt, __uint_as_float((uint32_t)ov[u]), acc0);
        acc1 = fmaf(wgt, __uint_as_float((uint32_t)(ov[u] >> 32)), acc1);
      }
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint32_t* o = reinterpret_cast<uint32_t*>(out + (((size_t)r * a.H + h) * 128 + d) * 2);
  *o = f32_to_bf16(acc0 * inv) | (f32_to_bf16(acc1 * inv) << 16);
  if (lse && d == 0) lse[(size_t)r * a.H + h] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_decode_fused(FusedArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  uint32_t* scr = reinterpret_cast<uint32_t*>(smem + kOffScr);
  if (threadIdx.x == 0) {
    uint32_t tag = ld_dev(a.ctl + W_EPOCH) + 1u;
    if (tag == 0) tag = 1;
    scr[S_TAG] = tag;
  }
  __syncthreads();
  const FCtx x{&a, smem, scr, scr[S_TAG], make_coh(a.ctl)};
  __syncthreads();
  const int G = (int)gridDim.x, w = (int)blockIdx.x;
  bool ok = true;
  // ---- score / reduce / emit: chunk w
  if (w < a.R * a.n_sc) {
    const int r = w / a.n_sc, c = w % a.n_sc;
    const FRow f = row_info(a, r);
    int64_t j0 = (int64_t)c * a.C, j1 = j0 + a.C;
    if (j1 > f.n_vis) j1 = f.n_vis;
    if (j0 > j1) j0 = j1;
    phase_score(x, r, c, f, j0, j1);
    if (c == 0) ok = phase_reduce(x, r, f);
    if (ok) ok = phase_emit(x, r, c, (int)(j1 - j0));
  }
  // ---- items
  if (ok) {
    const int R = a.R, nM = a.H / 4;
    const int64_t e1 = (int64_t)R * a.n_cs_sel, e2 = e1 + (int64_t)R * a.n_cs_win,
                  e3 = e2 + (int64_t)R * a.n_hs, e4 = e3 + (int64_t)R * nM, total = e4 + (int64_t)R * nM;
    for (int64_t it = w; it < total; it += G) {
      __syncthreads();
      if (error_seen(x)) break;
      if (it >= e3) {
        const bool hca = it >= e4;
        const int64_t m = it - (hca ? e4 : e3);
        item_merge(x, hca, (int)(m / nM), (int)(m % nM) * 4);
        continue;
      }
      const int kind = it < e1 ? 0 : it < e2 ? 1 : 2;
      const int64_t q = it - (kind == 0 ? 0 : kind == 1 ? e1 : e2);
      const int r = (int)(q % R), s = (int)(q / R);
      const FRow f = row_info(a, r);
      if (kind == 0 && !select_split(x, r, s, f)) continue;
      attend_item(x, r, kind, s, f);
    }
  }
  // ---- the last workgroup out advances the epoch
  __syncthreads();
  if (threadIdx.x == 0) {
    vm_drain();
    if (atomicAdd(a.ctl + W_EXIT, 1u) == (uint32_t)G - 1) {
      st_dev(a.ctl + W_EXIT, 0u);
      st_dev(a.ctl + W_EPOCH, x.tag);
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
static int g_fused_grid = 0;

static int fused_grid() {
  if (g_fused_grid > 0) return g_fused_grid;
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipFuncSetAttribute((const void*)k_decode_fused, hipFuncAttributeMaxDynamicSharedMemorySize, kFusedLds) !=
      hipSuccess)
    return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)k_decode_fused, 256, kFusedLds) != hipSuccess)
    return 0;
  if (per_cu < 1) return 0;
  g_fused_grid = cus * per_cu;
  return g_fused_grid;
}

static int split_count(int64_t len, int64_t size) { return len <= 0 ? 0 : (int)((len + size - 1) / size); }

FusedPlan plan_fused(int64_t R, int64_t max_pool, int64_t max_hpool, int H, int k, int W, int W_hca) {
  FusedPlan p{};
  const int G = fused_grid();
  p.grid = G;
  // score chunk: the smallest multiple of 256 (>= 1024) that gives every chunk its own workgroup
  int64_t C = 1024;
  if (G > 0) {
    const int64_t per = (R * max_pool + G - 1) / G;
    if (per > C) C = ((per + 255) / 256) * 256;
  }
  p.C = (int)(C > kFMaxC ? kFMaxC + 1 : C);
  p.n_sc = max_pool > 0 ? (int)((max_pool + C - 1) / C) : 1;
  p.cs = 64;
  p.n_cs_sel = split_count(k, p.cs);
  p.n_cs_win = split_count(W, p.cs);
  if (p.n_cs_sel + p.n_cs_win == 0) p.n_cs_win = 1;
  p.hs = 128;
  p.n_hs = split_count(max_hpool + W_hca, p.hs);
  if (p.n_hs == 0) p.n_hs = 1;
  p.def_cap = (int)(p.C < k ? p.C : k);
  auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
  const size_t slots = (size_t)R * p.n_sc;
  const int n_cs = p.n_cs_sel + p.n_cs_win;
  size_t s = 0;
  s += al(W_CTL * 4);
  s += al(slots * 8);
  s += al(slots * k * 8);
  s += al((size_t)R * kThrStride * 8);
  s += al(slots * 8);
  s += al(slots * p.def_cap * 8);
  s += al(slots * 2 * p.C * 8);
  s += al((size_t)R * (n_cs + p.n_hs) * 8);
  s += al((size_t)R * n_cs * H * 128 * 4);
  s += al((size_t)R * n_cs * H * 2 * 4);
  s += al((size_t)R * p.n_hs * H * 128 * 4);
  s += al((size_t)R * p.n_hs * H * 2 * 4);
  p.ws_bytes = s;
  return p;
}

int fused_supported(int64_t R, int64_t max_pool, int64_t max_hpool, int H, int k, int W, int W_hca) {
  if (R < 1 || R > kFMaxRows || max_pool > (int64_t)kFMaxVisible || H % 16 != 0 || H > 64 || H < 16) return 0;
  const FusedPlan p = plan_fused(R, max_pool, max_hpool, H, k, W, W_hca);
  if (p.grid <= 0 || p.C > kFMaxC || p.n_sc > kFMaxSlots || (int64_t)R * p.n_sc > p.grid) return 0;
  return 1;
}

size_t fused_error_word_offset() { return W_ERROR * 4; }

int launch_fused(int R, const int64_t* tok_off, const int64_t* q_pos, const int64_t* pool_off,
                 const int64_t* hpool_off, int64_t max_pool, int64_t max_hpool, int m, int m_hca, int H,
                 float scale, int k, int W, int W_hca, const uint8_t* q_codes, const uint8_t* q_scales,
                 const float* w, const uint8_t* k_codes, const uint8_t* k_scales, const void* q,
                 const void* kv_pool, const void* kv_hpool, const void* kv_raw, int32_t* idx, void* csa_out,
                 float* csa_lse, void* hca_out, float* hca_lse, void* ws, hipStream_t stream) {
  const FusedPlan pl = plan_fused(R, max_pool, max_hpool, H, k, W, W_hca);
  if (pl.grid <= 0 || pl.C > kFMaxC || (int64_t)R * pl.n_sc > pl.grid) return -1;
  uint8_t* p = (uint8_t*)ws;
  auto take = [&](size_t bytes) {
    uint8_t* q0 = p;
    p += (bytes + 255) & ~(size_t)255;
    return q0;
  };
  const size_t slots = (size_t)R * pl.n_sc;
  const int n_cs = pl.n_cs_sel + pl.n_cs_win;
  FusedArgs a;
  a.tok_off = tok_off; a.q_pos = q_pos; a.pool_off = pool_off; a.hpool_off = hpool_off;
  a.R = R; a.m = m; a.m_hca = m_hca; a.H = H; a.k = k; a.W = W; a.W_hca = W_hca;
  a.scale_log2 = scale * kLog2e;
  a.max_pool = max_pool; a.max_hpool = max_hpool;
  a.q_codes = q_codes; a.q_scales = q_scales; a.w = w; a.k_codes = k_codes; a.k_scales = k_scales;
  a.q = (const uint8_t*)q; a.kv_pool = (const uint8_t*)kv_pool; a.kv_hpool = (const uint8_t*)kv_hpool;
  a.kv_raw = (const uint8_t*)kv_raw;
  a.idx = idx; a.csa_out = (uint8_t*)csa_out; a.csa_lse = csa_lse; a.hca_out = (uint8_t*)hca_out; a.hca_lse = hca_lse;
  a.C = pl.C; a.n_sc = pl.n_sc; a.cs = pl.cs; a.n_cs_sel = pl.n_cs_sel; a.n_cs_win = pl.n_cs_win;
  a.hs = pl.hs; a.n_hs = pl.n_hs; a.def_cap = pl.def_cap;
  a.ctl = (uint32_t*)take(W_CTL * 4);
  a.sum_hdr = (uint64_t*)take(slots * 8);
  a.sum = (uint64_t*)take(slots * k * 8);
  a.thr = (uint64_t*)take((size_t)R * kThrStride * 8);
  a.emit_hdr = (uint64_t*)take(slots * 8);
  a.defw = (uint64_t*)take(slots * pl.def_cap * 8);
  a.candw = (uint64_t*)take(slots * 2 * pl.C * 8);
  a.part_hdr = (uint64_t*)take((size_t)R * (n_cs + pl.n_hs) * 8);
  a.csa_po = (float*)take((size_t)R * n_cs * H * 128 * 4);
  a.csa_pml = (float*)take((size_t)R * n_cs * H * 2 * 4);
  a.hca_po = (float*)take((size_t)R * pl.n_hs * H * 128 * 4);
  a.hca_pml = (float*)take((size_t)R * pl.n_hs * H * 2 * 4);
  void* args[] = {&a};
  prof_begin(6, stream);
  const hipError_t e = hipLaunchCooperativeKernel((const void*)k_decode_fused, dim3((unsigned)pl.grid), dim3(256),
                                                  args, kFusedLds, stream);
  prof_end(6, stream);
  if (e != hipSuccess) return -1;
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace csa

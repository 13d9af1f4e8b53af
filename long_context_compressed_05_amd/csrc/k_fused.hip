// Fused CSA + HCA decode step: one launch per step.
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
constexpr int kFEntLds = 6144;       // emitted entries of a row staged in LDS
constexpr int kFMaxVisible = 262144;  // visible pooled entries per query (18-bit indices)
constexpr int kFMaxRows = 64;
constexpr int kFMaxSlots = 512;      // score chunks per row
constexpr int kFRankMax = 2032;      // threshold-bin entries ranked by direct comparison
constexpr uint32_t kSpinLimit = 1u << 20;

// control words at the start of the workspace
enum { W_EPOCH = 0, W_EXIT = 1, W_ERROR = 2, W_TICKET = 3, W_CTL = 64 };

// LDS layout (dynamic)
constexpr int kOffKeys = 0;                                 // uint32 [kFMaxC]; later per-chunk arrays
constexpr int kOffIdx = kOffKeys + kFMaxC * 4;              // int32 [kFMaxSplit]
constexpr int kOffScr = kOffIdx + kFMaxSplit * 4;           // uint32 [64]
constexpr int kOffU = kOffScr + 64 * 4;                     // union region
constexpr int kOffEnt = kOffU;                              // uint64 [kFEntLds] order keys of emitted entries
constexpr int kOffHist = kOffEnt + kFEntLds * 8;            // uint32 [kFBins]; then uint64 [kFRankMax + 16]
constexpr int kSelEnd = kOffHist + kFBins * 4;
constexpr int kAttnEnd = kOffU + kAttnLdsBytes;
constexpr int kFusedLds = kSelEnd > kAttnEnd ? kSelEnd : kAttnEnd;
static_assert((kFMaxSlots + 1) * 3 * 4 <= kFMaxC * 4, "per-chunk arrays alias the key region");
static_assert(kOffU % 16 == 0, "attention LDS must be 16-byte aligned");
static_assert((kFRankMax + 16) * 8 <= kFBins * 4, "ranked entries reuse the histogram");

// scratch word indices (0..39 are used by the block scans)
enum { S_TAG = 40, S_FLAG, S_B1, S_ABOVE, S_NB1, S_CSTAR_LO, S_CSTAR_HI, S_BAD, S_TICKET };

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
  int rounds;                  // work units taken per workgroup (rounds * grid >= all units)
  int hs, n_hs;                // HCA split size, splits per row
  int emit_q, emit_max;        // per chunk: entries at or above the local emit_q-th bin, at most emit_max
  int64_t key_stride;          // keys row stride (multiple of 4)
  // workspace
  uint32_t* ctl;
  uint32_t* keys;      // [R][key_stride] sort keys (read only by the exact fallback)
  uint64_t* ent_hdr;   // [R*n_sc] tagged: count | bin << 12 | truncated << 25
  uint64_t* ent;       // [R*n_sc][emit_max] (key << 32) | index, ascending index
  uint64_t* part_hdr;  // [R][n_cs_sel + n_cs_win + n_hs]
  float* csa_po;       // [R][n_cs][H][128]
  float* csa_pml;      // [R][n_cs][H][2]
  float* hca_po;
  float* hca_pml;
};

// The arguments are read through a kernarg-segment pointer that is laundered
// at the top of every work round, so each field is re-read with a scalar load
// where it is used instead of being held in registers across the whole loop.
using KArgs = const __attribute__((address_space(4))) FusedArgs;

struct FRow {
  int64_t t, n_vis, n_vis_h, pbase, hbase, tok_base;
};

__device__ __forceinline__ FRow row_info(KArgs& a, int r) {
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

__device__ __forceinline__ uint32_t n_vis_u32(const FRow& f) { return (uint32_t)f.n_vis; }
// A value every lane holds identically (an LDS broadcast): made scalar so that
// the compiler sees control flow on it as uniform (barriers inside stay aligned).
__device__ __forceinline__ uint32_t uni(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

struct FCtx {
  KArgs* a;
  uint8_t* smem;
  uint32_t* scr;
  uint32_t tag;
  Coh coh;
};

// error word: bit 0 = a wait hit its bound, bits 1.. = which wait (see the callers)
__device__ __forceinline__ void set_error(const FCtx& x, uint32_t code) { atomicOr(x.a->ctl + W_ERROR, 1u | code); }
__device__ __forceinline__ bool error_seen(const FCtx& x) { return ld_dev(x.a->ctl + W_ERROR) != 0; }

// this thread spins until the tagged word at p carries the launch's tag and
// returns its payload; after the bound (or once an error was reported) it
// sets *fail and returns 0
__device__ __forceinline__ uint32_t poll_word(const FCtx& x, const uint64_t* p, bool* fail, uint32_t code = 0) {
  uint64_t v = coh_ld64(x.coh, p);
  uint32_t n = 0;
  while ((uint32_t)(v >> 32) != x.tag) {
    ++n;
    if (n >= kSpinLimit || ((n & 1023u) == 0 && error_seen(x))) {
      if (n >= kSpinLimit) set_error(x, code);
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
      if (n >= kSpinLimit) set_error(x, 0);
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
  const int tid = lane_tid(), lane = tid & 63, wave = tid >> 6;
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
  if (lane_tid() == 0) x.scr[S_FLAG] = 0;
  __syncthreads();
  if (fail) x.scr[S_FLAG] = 1;
  __syncthreads();
  const bool ok = uni(x.scr[S_FLAG]) == 0;
  __syncthreads();
  return ok;
}

// k-th largest bin over a 4096-bin LDS histogram (thread t owns bins 16t..16t+15):
// returns the bin, *above = entries in higher bins.  need >= 1 and <= total.
// Returns kFBins + 1 when the histogram holds fewer than need entries.
__device__ __forceinline__ uint32_t kth_bin(const uint32_t* hist, uint32_t need, uint32_t* scr, uint32_t* above) {
  const int tid = lane_tid();
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
  if ((int)uni((uint32_t)tstar) < 0) {
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
  const uint32_t b = uni(scr[S_B1]);
  *above = uni(scr[S_ABOVE]);
  __syncthreads();
  return b;
}

// ---------------------------------------------------------------------------
// score: chunk c of row r -> keys in LDS, local histogram, published summary
// ---------------------------------------------------------------------------
__device__ __forceinline__ void phase_score(const FCtx& x, int r, int c, const FRow& f, int64_t j0, int64_t j1) {
  KArgs& a = *x.a;
  const int tid = lane_tid(), lane = tid & 63, wave = tid >> 6, kb = lane >> 5;
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
  // keys -> workspace (read only by the exact fallback), 16 bytes per store
  {
    uint32_t* gk = a.keys + (size_t)r * a.key_stride + j0;
    for (int i = 4 * tid; i < n; i += 1024) {
      if (i + 3 < n) {
        const v4u_t u = {keys_s[i], keys_s[i + 1], keys_s[i + 2], keys_s[i + 3]};
        coh_st128(x.coh, gk + i, u);
      } else {
        for (int e = i; e < n; ++e)
          __builtin_amdgcn_raw_buffer_store_b32(keys_s[e], x.coh.r, coh_off(x.coh, gk + e), 0, kSc1);
      }
    }
  }
  // local emit_q-th bin bq: every entry above it, and entries in it while room remains
  const uint32_t q = n < a.emit_q ? (uint32_t)n : (uint32_t)a.emit_q;
  uint32_t bq = 0, ab = 0;
  if (q > 0) bq = kth_bin(hist, q, x.scr, &ab);
  const int E = (n + 255) / 256;  // thread t owns local entries [t*E, t*E + E)
  const int e0 = tid * E;
  uint32_t ng = 0, ne = 0;
  for (int i = 0; i < E; ++i) {
    const int jl = e0 + i;
    if (jl < n) {
      const uint32_t bin = keys_s[jl] >> 19;
      ng += bin > bq ? 1u : 0u;
      ne += bin == bq ? 1u : 0u;
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
  const uint32_t cap_eq = (uint32_t)a.emit_max - tg;  // tg < q <= emit_q < emit_max
  const uint32_t n_emit = tg + (te < cap_eq ? te : cap_eq);
  const size_t slot = (size_t)r * a.n_sc + c;
  uint64_t* dst = a.ent + slot * a.emit_max;
  const uint32_t jbase = (uint32_t)c * (uint32_t)a.C;
  uint32_t pos = pg + (pe < cap_eq ? pe : cap_eq);
  for (int i = 0; i < E; ++i) {
    const int jl = e0 + i;
    if (jl < n) {
      const uint32_t key = keys_s[jl], bin = key >> 19;
      bool take = bin > bq;
      if (bin == bq) take = pe++ < cap_eq;
      if (take) {
        const uint64_t w64 = ((uint64_t)key << 32) | (jbase + (uint32_t)jl);
        __builtin_amdgcn_raw_buffer_store_b64(v2u_t{(uint32_t)w64, (uint32_t)(w64 >> 32)}, x.coh.r,
                                              coh_off(x.coh, dst + pos), 0, kSc1);
        ++pos;
      }
    }
  }
  vm_drain();
  __syncthreads();
  if (tid == 0) st_dev64(a.ent_hdr + slot, tagged(x.tag, n_emit | (bq << 12) | ((te > cap_eq ? 1u : 0u) << 25)));
}

// ---------------------------------------------------------------------------
// attention items
// ---------------------------------------------------------------------------
// unnormalised partial (O, m in log2 units, l) of one split, then its tagged header
__device__ __forceinline__ void write_partial(const FCtx& x, AttnState<1>& st, int r, int pi, bool hca) {
  KArgs& a = *x.a;
  const int n_cs = a.n_cs_sel + a.n_cs_win;
  const int lane = lane_tid() & 63, wave = lane_tid() >> 6, l16 = lane & 15, g = lane >> 4;
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
  if (lane_tid() == 0)
    st_dev64(a.part_hdr + (size_t)r * (n_cs + a.n_hs) + (hca ? n_cs : 0) + pi, tagged(x.tag, 1u));
}

// Selection for CSA split s of row r: the split's slice of the ascending
// selected list -> idx_s (and, for split 0, the whole row -> idx).  false on a
// failed wait.
//
// The selected set is the k_eff first entries in (key descending, index
// ascending) order, i.e. the entries whose order key (key << 32 | ~index) is
// at least that of the k_eff-th one, c*.  Each score chunk emitted every entry
// above its local emit_q-th bin bq (and that bin's entries up to emit_max,
// else it is marked truncated).  From the emitted entries of the row: b1 = the
// bin of the k_eff-th largest, and c* = the need-th largest order key in bin
// b1.  This is exact when every chunk emitted all its entries in bins >= b1:
// bq <= b1 (bq < b1 when truncated).  Otherwise c* comes from an exact radix
// select over the row's stored keys.  Chunks cover ascending index ranges and
// emit in index order, so the position of a selected index is the selected
// count of the earlier chunks plus its rank within its chunk.
__device__ __forceinline__ bool select_split(const FCtx& x, int r, int s, const FRow& f) {
  KArgs& a = *x.a;
  const int tid = lane_tid();
  const int64_t p_begin = (int64_t)s * a.cs;
  const int64_t p_end = p_begin + a.cs < a.k ? p_begin + a.cs : a.k;
  const int k_eff = (int)(f.n_vis < a.k ? f.n_vis : a.k);
  int32_t* idx_s = reinterpret_cast<int32_t*>(x.smem + kOffIdx);
  int32_t* idx_out = a.idx + (size_t)r * a.k;
  for (int i = tid; i < a.cs; i += 256) idx_s[i] = -1;
  const bool needs_sel = (s == 0) || (p_begin < k_eff);
  if (needs_sel && k_eff > 0) {
    uint32_t* e_off = reinterpret_cast<uint32_t*>(x.smem + kOffKeys);  // per chunk, LDS
    uint32_t* e_bq = e_off + (kFMaxSlots + 1);
    uint32_t* sel_off = e_bq + (kFMaxSlots + 1);
    uint64_t* ent_s = reinterpret_cast<uint64_t*>(x.smem + kOffEnt);
    uint32_t* hist = reinterpret_cast<uint32_t*>(x.smem + kOffHist);
    const uint64_t* rowent = a.ent + (size_t)r * a.n_sc * a.emit_max;
    const uint32_t* rowkeys = a.keys + (size_t)r * a.key_stride;
    bool fail = false;
    for (int sl = tid; sl < a.n_sc && !fail; sl += 256) {
      const uint32_t v = poll_word(x, a.ent_hdr + (size_t)r * a.n_sc + sl, &fail, 2u);
      e_off[sl] = v & 0xfffu;
      e_bq[sl] = v >> 12;  // bin | truncated << 13
    }
    for (int i = tid; i < kFBins; i += 256) hist[i] = 0;
    if (tid == 0) x.scr[S_BAD] = 0;
    if (!all_ok(x, fail)) return false;
    block_exscan(e_off, a.n_sc, x.scr);
    const uint32_t n_ent = uni(e_off[a.n_sc]);
    bool exact = n_ent <= (uint32_t)kFEntLds && n_ent >= (uint32_t)k_eff;
    if (exact) {
      // emitted entries -> LDS order keys, in global index order: wave w takes chunks
      // w, w+4, ..., lane = entry within the chunk, 16 chunks in flight
      const int lane = tid & 63, wave = tid >> 6;
      for (int i0 = 0; i0 < a.emit_max; i0 += 64) {
        const uint32_t i = (uint32_t)(i0 + lane);
        for (int sb = wave; sb < a.n_sc; sb += 64) {
          uint64_t v[16];
#pragma unroll
          for (int u = 0; u < 16; ++u) {
            const int sl = sb + 4 * u;
            v[u] = (sl < a.n_sc && i < e_off[sl + 1] - e_off[sl]) ? coh_ld64(x.coh, rowent + (size_t)sl * a.emit_max + i)
                                                                  : 0ull;
          }
#pragma unroll
          for (int u = 0; u < 16; ++u) {
            const int sl = sb + 4 * u;
            if (sl < a.n_sc && i < e_off[sl + 1] - e_off[sl]) {
              const uint32_t key = (uint32_t)(v[u] >> 32), j = (uint32_t)v[u];
              ent_s[e_off[sl] + i] = ((uint64_t)key << 32) | (uint32_t)~j;
              atomicAdd(&hist[key >> 19], 1u);
            }
          }
        }
      }
      __syncthreads();
      uint32_t above = 0;
      const uint32_t b1 = kth_bin(hist, (uint32_t)k_eff, x.scr, &above);
      // every chunk must have emitted all of its entries in bins >= b1
      for (int sl = tid; sl < a.n_sc; sl += 256) {
        const uint32_t bq = e_bq[sl] & 0x1fffu, trunc = e_bq[sl] >> 13;
        if (trunc ? bq >= b1 : bq > b1) x.scr[S_BAD] = 1;
      }
      if (tid == 0) x.scr[S_NB1] = 0;
      __syncthreads();
      exact = uni(x.scr[S_BAD]) == 0;
      if (exact) {
        // the bin-b1 entries, ranked by order key (the histogram area is free now)
        uint64_t* comp = reinterpret_cast<uint64_t*>(x.smem + kOffHist);
        for (uint32_t i0 = 0; i0 < n_ent; i0 += 256) {
          const uint32_t i = i0 + tid;
          const uint64_t e = i < n_ent ? ent_s[i] : 0ull;
          const bool hit = i < n_ent && (uint32_t)(e >> 51) == b1;
          const uint64_t m = __ballot(hit);
          uint32_t base = 0;
          if ((tid & 63) == 0 && m) base = atomicAdd(&x.scr[S_NB1], (uint32_t)__popcll(m));
          base = __shfl(base, 0);
          const uint32_t slot_i = base + (uint32_t)__popcll(m & ((1ull << (tid & 63)) - 1ull));
          if (hit && slot_i < (uint32_t)kFRankMax) comp[slot_i] = e;
        }
        __syncthreads();
        const uint32_t nb = uni(x.scr[S_NB1]);
        exact = nb <= (uint32_t)kFRankMax;
        if (exact) {
          const uint32_t need = (uint32_t)k_eff - above;  // >= 1
          const uint32_t n_pad = (nb + 15) & ~15u;
          for (uint32_t i = nb + tid; i < n_pad; i += 256) comp[i] = 0ull;
          __syncthreads();
          for (uint32_t i = tid; i < nb; i += 256) {
            const uint64_t ci = comp[i];
            uint32_t rank = 0;
            for (uint32_t j0 = 0; j0 < n_pad; j0 += 16) {
              uint64_t qv[16];
#pragma unroll
              for (int u = 0; u < 16; ++u) qv[u] = comp[j0 + u];
#pragma unroll
              for (int u = 0; u < 16; ++u) rank += qv[u] > ci ? 1u : 0u;
            }
            if (rank == need - 1) {
              x.scr[S_CSTAR_LO] = (uint32_t)ci;
              x.scr[S_CSTAR_HI] = (uint32_t)(ci >> 32);
            }
          }
          __syncthreads();
        }
      }
    }
    if (!exact) {
      // exact radix select over the row's stored keys: the k_eff-th largest key K*, then
      // the (need_left)-th smallest index among keys equal to K* (indices < 2^18)
      uint32_t* bins = hist;
      uint32_t nl;
      const uint32_t n_vis = (uint32_t)f.n_vis;
      const uint32_t kstar = radix_select_desc(
          n_vis, (uint32_t)k_eff, [&](uint32_t i) { return coh_ld32(x.coh, rowkeys + i); },
          [&](uint32_t) { return true; }, &nl, bins, x.scr);
      uint32_t nl2;
      const uint32_t njstar = radix_select_desc_low(
          n_vis, nl, 18, 0xfffc0000u, [&](uint32_t i) { return ~i; },
          [&](uint32_t i) { return coh_ld32(x.coh, rowkeys + i) == kstar; }, &nl2, bins, x.scr);
      if (tid == 0) {
        x.scr[S_CSTAR_LO] = njstar;
        x.scr[S_CSTAR_HI] = kstar;
      }
      __syncthreads();
    }
    const uint64_t cstar = ((uint64_t)uni(x.scr[S_CSTAR_HI]) << 32) | uni(x.scr[S_CSTAR_LO]);
    auto emit_at = [&](uint32_t pos, uint32_t j) {
      if ((int64_t)pos >= p_begin && (int64_t)pos < p_end) idx_s[pos - p_begin] = (int32_t)j;
      if (s == 0 && pos < (uint32_t)a.k) idx_out[pos] = (int32_t)j;
    };
    if (exact) {
      // the entries are in index order: position = selected entries before it.  Thread t
      // owns entries [t*M, t*M + M); one block scan of the per-thread counts.
      const uint32_t M = (n_ent + 255) / 256, m0 = tid * M;
      uint32_t cnt = 0;
      for (uint32_t i = m0; i < m0 + M && i < n_ent; ++i) cnt += ent_s[i] >= cstar ? 1u : 0u;
      sel_off[tid] = cnt;
      __syncthreads();
      block_exscan(sel_off, 256, x.scr);
      uint32_t pos = sel_off[tid];
      const uint32_t pend = sel_off[tid + 1];
      if (pos < pend && (s == 0 || ((int64_t)pos < p_end && (int64_t)pend > p_begin))) {
        for (uint32_t i = m0; i < m0 + M && i < n_ent; ++i) {
          const uint64_t e = ent_s[i];
          if (e >= cstar) emit_at(pos++, ~(uint32_t)e);
        }
      }
    } else {
      const int C = a.C;
      const uint32_t nv = n_vis_u32(f);
      // selected count per chunk -> offsets, then the chunks in index order
      for (int sl = tid; sl < a.n_sc; sl += 256) {
        uint32_t cnt = 0;
        const uint32_t jb = (uint32_t)sl * C, je = jb + C < nv ? jb + C : nv;
        for (uint32_t j = jb; j < je; ++j)
          cnt += (((uint64_t)coh_ld32(x.coh, rowkeys + j) << 32) | (uint32_t)~j) >= cstar ? 1u : 0u;
        sel_off[sl] = cnt;
      }
      __syncthreads();
      block_exscan(sel_off, a.n_sc, x.scr);
      for (int sl = tid; sl < a.n_sc; sl += 256) {
        uint32_t pos = sel_off[sl];
        const uint32_t pend = sel_off[sl + 1];
        if (pos == pend || (s != 0 && ((int64_t)pos >= p_end || (int64_t)pend <= p_begin))) continue;
        const uint32_t jb = (uint32_t)sl * C, je = jb + C < nv ? jb + C : nv;
        for (uint32_t j = jb; j < je; ++j)
          if ((((uint64_t)coh_ld32(x.coh, rowkeys + j) << 32) | (uint32_t)~j) >= cstar) emit_at(pos++, j);
      }
    }
    __syncthreads();
  }
  if (s == 0)
    for (int i = k_eff + tid; i < a.k; i += 256) idx_out[i] = -1;
  __syncthreads();
  return true;
}

// Attention item: CSA selected split (kind 0, rows through idx_s), CSA window
// split (kind 1) or HCA split (kind 2) of row r, then its partial.
__device__ __forceinline__ void attend_item(const FCtx& x, int r, int kind, int s, const FRow& f) {
  KArgs& a = *x.a;
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
  constexpr uint64_t RB = 2 * 128 * 2;
  // Row addresses from 32-bit offsets against per-row bases: list positions
  // below `split` are pooled rows (selected ones for kind 0, HCA rows for
  // kind 2), the rest are window tokens t - W + 1 + (p - split).
  const uint8_t* pool_base = kind == 0 ? a.kv_pool + (size_t)f.pbase * RB : a.kv_hpool + (size_t)f.hbase * RB;
  const uint8_t* raw_base = a.kv_raw + (size_t)f.tok_base * RB;
  const int32_t pb32 = (int32_t)p_begin;
  const int32_t split = kind == 1 ? 0 : (int32_t)a.max_hpool;
  const int32_t hi_pool = (int32_t)f.n_vis_h;
  const int32_t win_off = (int32_t)(f.t + 1 - (kind == 1 ? a.W : a.W_hca)) - split;
  auto rowptr = [&](int64_t p64) -> const uint8_t* {
    const int32_t p = (int32_t)p64;
    if (kind == 0) {
      const int32_t j = idx_s[p - pb32];
      return j >= 0 ? pool_base + (uint64_t)(uint32_t)j * RB : nullptr;
    }
    if (p < split) return p < hi_pool ? pool_base + (uint64_t)(uint32_t)p * RB : nullptr;
    const int32_t u = p + win_off;
    return u >= 0 ? raw_base + (uint64_t)(uint32_t)u * RB : nullptr;
  };
  AttnState<1> st;
  attn_init<1>(st, a.q + (size_t)r * a.H * 128 * 2, a.H);
  attn_run<1>(st, a.H, a.scale_log2, p_begin, p_end, rowptr, x.smem + kOffU);
  write_partial(x, st, r, pi, kind == 2);
}

// merge of 4 heads (h0 .. h0+3) of one row: thread = (head, 2 dims)
__device__ __forceinline__ void item_merge(const FCtx& x, bool hca, int r, int h0) {
  KArgs& a = *x.a;
  const int tid = lane_tid();
  const int n_cs = a.n_cs_sel + a.n_cs_win;
  const int n = hca ? a.n_hs : n_cs;
  const uint64_t* hdr = a.part_hdr + (size_t)r * (n_cs + a.n_hs) + (hca ? n_cs : 0);
  bool fail = false;
  for (int s = tid; s < n && !fail; s += 256) (void)poll_word(x, hdr + s, &fail, hca ? 8u : 4u);
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
  if (lane_tid() == 0) {
    uint32_t tag = ld_dev(a.ctl + W_EPOCH) + 1u;
    if (tag == 0) tag = 1;
    scr[S_TAG] = tag;
  }
  __syncthreads();
  const uint32_t tag = uni(scr[S_TAG]);
  __syncthreads();
  const int rounds = a.rounds;
  // Work units in dependency order: the R * n_sc score chunks, then the items
  // [CSA selected splits | CSA window splits | HCA splits | CSA merges | HCA
  // merges].  Units are handed out in that order through one returning atomic,
  // and a unit only waits for units of lower number, whose holders are already
  // running: every wait ends whatever the residency of the grid.
  // Every workgroup runs the same number of rounds (rounds * grid >= total), so
  // the loop bound is uniform; a round whose unit number is past the end (or
  // that follows a reported error) does nothing.
  for (int round = 0; round < rounds; ++round) {
    KArgs* ap = (KArgs*)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(ap));
    KArgs& A = *ap;
    const FCtx x{ap, smem, scr, tag, make_coh(A.ctl)};
    const int R = A.R, nM = A.H / 4;
    const int64_t nS = (int64_t)R * A.n_sc;
    const int64_t e1 = nS + (int64_t)R * A.n_cs_sel, e2 = e1 + (int64_t)R * A.n_cs_win,
                  e3 = e2 + (int64_t)R * A.n_hs, e4 = e3 + (int64_t)R * nM, total = e4 + (int64_t)R * nM;
    if (lane_tid() == 0) scr[S_TICKET] = error_seen(x) ? 0xffffffffu : atomicAdd(A.ctl + W_TICKET, 1u);
    __syncthreads();
    const int64_t it = uni(scr[S_TICKET]);
    __syncthreads();
    if (it >= total) {
      // nothing to do this round
    } else if (it < nS) {
      const int r = (int)(it / A.n_sc), c = (int)(it % A.n_sc);
      const FRow f = row_info(A, r);
      int64_t j0 = (int64_t)c * A.C, j1 = j0 + A.C;
      if (j1 > f.n_vis) j1 = f.n_vis;
      if (j0 > j1) j0 = j1;
      phase_score(x, r, c, f, j0, j1);
    } else if (it >= e3) {
      const bool hca = it >= e4;
      const int64_t m = it - (hca ? e4 : e3);
      item_merge(x, hca, (int)(m / nM), (int)(m % nM) * 4);
    } else {
      const int kind = it < e1 ? 0 : it < e2 ? 1 : 2;
      const int64_t q = it - (kind == 0 ? nS : kind == 1 ? e1 : e2);
      const int r = (int)(q % R), s = (int)(q / R);
      const FRow f = row_info(A, r);
      const bool ok = kind != 0 || select_split(x, r, s, f);
      if (ok) attend_item(x, r, kind, s, f);
    }
  }
  const int G = (int)gridDim.x;
  // ---- the last workgroup out advances the epoch
  __syncthreads();
  if (lane_tid() == 0) {
    vm_drain();
    if (atomicAdd(a.ctl + W_EXIT, 1u) == (uint32_t)G - 1) {
      st_dev(a.ctl + W_EXIT, 0u);
      st_dev(a.ctl + W_TICKET, 0u);
      st_dev(a.ctl + W_EPOCH, tag);
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
  // emitted per chunk: about twice a chunk's expected share of the top-k, plus slack
  const int64_t share = p.n_sc > 0 ? ((int64_t)k + p.n_sc - 1) / p.n_sc : k;
  int64_t q = 2 * share + 16;
  if (q > p.C) q = p.C;
  int64_t qm = q + 16;
  if (qm > p.C) qm = p.C;
  p.emit_q = (int)q;
  p.emit_max = (int)qm;
  p.key_stride = (max_pool + 3) & ~(int64_t)3;
  auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
  const size_t slots = (size_t)R * p.n_sc;
  const int n_cs = p.n_cs_sel + p.n_cs_win;
  size_t s = 0;
  s += al(W_CTL * 4);
  s += al((size_t)R * p.key_stride * 4);
  s += al(slots * 8);
  s += al(slots * p.emit_max * 8);
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
  a.hs = pl.hs; a.n_hs = pl.n_hs;
  a.emit_q = pl.emit_q; a.emit_max = pl.emit_max; a.key_stride = pl.key_stride;
  {
    const int64_t units = (int64_t)R * pl.n_sc + (int64_t)R * (pl.n_cs_sel + pl.n_cs_win + pl.n_hs) +
                          2 * (int64_t)R * (H / 4);
    a.rounds = (int)((units + pl.grid - 1) / pl.grid);
  }
  a.ctl = (uint32_t*)take(W_CTL * 4);
  a.keys = (uint32_t*)take((size_t)R * pl.key_stride * 4);
  a.ent_hdr = (uint64_t*)take(slots * 8);
  a.ent = (uint64_t*)take(slots * pl.emit_max * 8);
  a.part_hdr = (uint64_t*)take((size_t)R * (n_cs + pl.n_hs) * 8);
  a.csa_po = (float*)take((size_t)R * n_cs * H * 128 * 4);
  a.csa_pml = (float*)take((size_t)R * n_cs * H * 2 * 4);
  a.hca_po = (float*)take((size_t)R * pl.n_hs * H * 128 * 4);
  a.hca_pml = (float*)take((size_t)R * pl.n_hs * H * 2 * 4);
  void* args[] = {&a};
  prof_begin(6, stream);
  // an ordinary launch: correctness does not depend on all workgroups being resident
  const hipError_t e =
      hipLaunchKernel((const void*)k_decode_fused, dim3((unsigned)pl.grid), dim3(256), args, kFusedLds, stream);
  prof_end(6, stream);
  if (e != hipSuccess) return -1;
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace csa

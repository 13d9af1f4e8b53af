// Fused CSA + HCA decode step: one launch per step.
//
// The whole decode hot path runs in one kernel whose workgroups (one per CU)
// take work units in dependency order:
//   score   chunk c of row r: one of the row's nsc equal parts of the query's
//           visible range (nsc <= n_sc), MXFP4 MFMA scores -> u32 sort keys
//           in LDS, each counted into fixed bins as it is made; the bin
//           holding the chunk's Lm-th largest key (refined by one radix pass
//           when that bin is crowded) gives a threshold tau; every entry with
//           key >= tau (at most L of them) is written to the chunk's L list
//           positions in ascending index order, each position a tagged entry
//           (empty ones included), with tau beside them; then the chunk's
//           keys are stored for the exact fallback
//   group   CSA group g of row r (cg consecutive chunks, about 64 selected
//           entries, 128 beyond 8 rows): reads the whole row's lists (one
//           round of loads), warms the caches with the rows listed at its own
//           positions, finds K* = the k_eff-th largest listed key (radix
//           select in LDS), checks that every truncated chunk has tau <= K*
//           (else the row's first group runs an exact radix select over the
//           stored keys and publishes it), ranks its own positions' taken
//           entries (cutting ties in list = index order), attends over those
//           pooled rows, writes its partial and its slice of idx
//   window / HCA split: attention over raw window rows / pooled HCA rows
//   merge   log-sum-exp merge of a row's split partials, 4 heads per unit
// (units: [score chunks | CSA groups | window splits | HCA splits | HCA
// merges | CSA merges]).
//
// Synchronisation.  Cross-workgroup words are 64 bits: the launch's tag in
// the high half, the payload in the low half, written with device-coherent
// (sc1) stores and polled with device-coherent loads until the tag matches,
// so neither clearing nor store ordering between words is needed.  The tag is
// one more than the epoch word at the start of the workspace; the last
// workgroup to finish (a returning atomic on the exit count) advances it.
// Attention partials are plain data: the producer drains its stores
// (s_waitcnt vmcnt(0)) before it publishes the partial's tagged header.
// Forward progress: units wait only for units of lower number.  Every unit
// after the first round is claimed from the ticket counter by a workgroup
// that is running; a first-round score chunk (assigned by workgroup id) may
// belong to a workgroup not yet dispatched, so a CSA group that finds a chunk's
// list missing for steal_polls polls computes that chunk itself and then runs
// again.  Every wait therefore ends whatever the residency; the waits are
// bounded anyway, and hitting the bound sets the error word (read and cleared
// by csa_hca_decode_check) and skips the workgroup's remaining work.
#include <atomic>
#include <cstdlib>

#include "attn_core.hpp"
#include "common.hpp"
#include "kernels.hpp"
#include "select_core.hpp"

namespace csa {

constexpr int kFMaxC = 4096;         // score entries per workgroup (keys in LDS)
constexpr int kFKPT = kFMaxC / 256;  // keys per thread in a chunk
constexpr int kFHist = 2048;         // radix digit bins (11 bits)
constexpr int kFEntLds = 6144;       // list positions of a row (n_sc * lst)
constexpr int kFEPT = kFEntLds / 256;  // list positions per thread in a group's selection
constexpr int kFMaxSel = 1024;       // selected rows of one CSA group (k <= kFMaxSel)
constexpr int kFMaxVisible = 262144;  // visible pooled entries per query (18-bit indices)
constexpr int kFMaxRows = 64;
constexpr int kFMaxSlots = 512;      // score chunks per row
constexpr uint32_t kSpinLimit = 1u << 20;
static_assert(kFMaxVisible / 1024 <= kFMaxSlots, "every plan's chunk count fits (chunks hold at least 1024 entries)");

// control words at the start of the workspace
enum { W_EPOCH = 0, W_EXIT = 1, W_ERROR = 2, W_TICKET = 3, W_FALLBACK = 4, W_CTL = 64 };

// LDS layout (dynamic).  The key region holds a score chunk's keys, or the
// per-chunk arrays of a row (counts, thresholds) and a CSA group's selected
// rows; the union region holds the attention stages, or the radix histograms,
// or a score chunk's staged list.
constexpr int kFKeyPad = kFMaxC + kFMaxC / 16;  // key slots: entry j at j + j/16 (runs of 16 start on distinct banks)
constexpr int kFBins = 4096;                    // fixed score bins: a key's bits 30..19 (16 bins per octave)
constexpr int kFBinPad = kFBins + kFBins / 16;  // bin b at b + b/16
constexpr int kOffKeys = 0;                                 // uint32 [kFKeyPad]
constexpr int kOffSel = kOffKeys + 3 * (kFMaxSlots + 8) * 4;  // int32 [kFMaxSel] (aliases the chunk keys)
constexpr int kOffScr = kOffKeys + kFKeyPad * 4;            // uint32 [64]
constexpr int kOffU = kOffScr + 64 * 4;                     // union region
constexpr int kOffHist = kOffU + kFEntLds * 4;              // uint32 [2][kFHist] + [64] lane trash words
constexpr int kSelEnd = kOffHist + (2 * kFHist + 64) * 4;
constexpr int kAttnEnd = kOffU + kAttnLdsBytes;
constexpr int kFusedLds0 = kSelEnd > kAttnEnd ? kSelEnd : kAttnEnd;
// The launch's per-row work counts (built once per workgroup before it decodes
// its first ticket; no phase writes this region): row-major exclusive starts of
// the ticket-phase score chunks and of the HCA splits, each row's HCA split
// count, the two totals and whether every row has all n_hs splits.
enum { T_EB = 0, T_EH = 64, T_NHS = 128, T_UB = 192, T_UH, T_UNIH, T_WORDS = 196 };
constexpr int kOffTab = (kFusedLds0 + 15) & ~15;
constexpr int kFusedLds = kOffTab + T_WORDS * 4;
static_assert(kFMaxRows <= 64, "the row table holds one row per lane of a wave");
constexpr int kOffSelP = kOffSel + (kFMaxSel + 64) * 4;    // int32 [kFMaxSel] physical rows (paged caches)
static_assert(kOffSel + (kFMaxSel + 64) * 4 <= kOffScr, "a group's selected rows (+ 64 dummy slots) fit the key region");
static_assert(kOffSelP + kFMaxSel * 4 <= kOffScr, "the selected rows' physical rows fit the key region");
static_assert(kOffU % 16 == 0 && kOffHist % 16 == 0, "LDS regions must be 16-byte aligned");
static_assert(kFMaxC * 8 <= kAttnLdsBytes, "a score chunk's staged list fits the union region");
static_assert(kFBinPad * 4 <= kOffHist - kOffU && kFBinPad % 4 == 0, "a score chunk's fixed bins fit below the radix histograms");
static_assert((kFBinPad + kFMaxC / 32 + 1) * 4 <= kOffHist - kOffU, "a score chunk's page ids (pages of >= 32 rows) fit after its bins");
static_assert(2 * kFEntLds * 4 <= kAttnLdsBytes, "a row's keys and indices by position fit the union region");
static_assert(kFEPT % 4 == 0 && kFEntLds % 4 == 0, "positions are read 16 bytes at a time");
static_assert(kFusedLds <= 160 * 1024, "one workgroup per CU");

typedef unsigned int v2u_t __attribute__((ext_vector_type(2)));
typedef unsigned int v4u_t __attribute__((ext_vector_type(4)));
constexpr uint32_t kNoKey = 0xffffffffu;  // empty list position (scores are finite and >= 0)

// scratch word indices (0..19 are used by the block scans and searches, 20..35
// by the CSA group's first reduction)
enum { S_TAG = 40, S_FLAG, S_DIGIT, S_ABOVE, S_CNT, S_BAD, S_TICKET, S_KEY, S_CUT, S_OFF, S_STEAL, S_PENDC, S_PENDG, S_END };

struct FusedArgs {
  const int64_t* tok_off;
  const int64_t* q_pos;
  const int64_t* pool_off;
  const int64_t* hpool_off;
  const int32_t* pre_seq;  // [R] or null: the sequence whose cache holds this one's prefix (-1: none)
  const int64_t* pre_tok;  // [R] or null: the shared prefix's length in tokens
  // paged pooled caches (ptab null: contiguous, by pool_off / hpool_off): pooled
  // row j of row r is row ptab[r][j >> lg_page] << lg_page | (j & page mask) of
  // kv_pool (and of the indexer keys); HCA rows likewise through hptab
  const int32_t* ptab;     // [R][max_pages]
  const int64_t* plen;     // [R] pooled rows per row
  const int32_t* hptab;    // [R][max_hpages]
  const int64_t* hplen;    // [R]
  int max_pages, max_hpages, lg_page, lg_hpage;
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
  int cs, n_cs_sel, n_cs_win;  // window split size; CSA groups and window splits per row
  int cg;                      // score chunks per CSA group
  int rounds;                  // work units taken per workgroup (rounds * grid >= all units)
  int first_units;             // first-round score chunks assigned by workgroup id (min(score chunks, grid))
  int hpm;                     // heads per merge unit (4, or 16 beyond 8 rows)
  int steal_polls;             // list polls after which a group computes a missing score chunk itself
  int hs, n_hs;                // HCA split size, splits per row
  int lst_min, lst;            // per chunk: listed entries, at least lst_min (when it has them), at most lst (4 | lst)
  int64_t key_stride;          // keys row stride (multiple of 4)
  // workspace
  uint32_t* ctl;
  uint32_t* keys;      // [R][key_stride] sort keys (read only by the exact fallback)
  uint64_t* key_hdr;   // [R*n_sc] tagged: the chunk's keys are in keys
  v4u_t* lent;         // [R*n_sc][lst] list entries {tag, key, tag, index}, ascending index;
                       // positions past the chunk's count hold kNoKey
  uint64_t* ltau;      // [R*n_sc] tagged: the chunk's listing threshold (0 when it listed all)
  uint64_t* row_k;     // [R] tagged: K* (exact selection over the stored keys only)
  uint64_t* row_cut;   // [R] tagged: index of the last taken entry equal to K* (same)
  uint64_t* grp_off;   // [R][n_cs_sel] tagged: output position of the group's first selected entry (same)
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

// A row's logical cache entries: a shared prefix (pre_p pooled rows, pre_h
// HCA rows, pre_t raw tokens, held in another sequence's cache from ppbase /
// phbase / ptbase), then the row's own segment (from pbase / hbase /
// tok_base).  Without a prefix the pre_ counts are 0.
struct FRow {
  int64_t t, n_vis, n_vis_h, pbase, hbase, tok_base;
  int64_t pre_p, pre_h, pre_t, ppbase, phbase, ptbase;
};
// physical pooled row (and indexer key row) of logical pooled entry j
__device__ __forceinline__ int64_t pool_row(const FRow& f, int64_t j) {
  return j < f.pre_p ? f.ppbase + j : f.pbase + (j - f.pre_p);
}
// the same through row r's page table (paged caches)
__device__ __forceinline__ int64_t paged_row(const int32_t* tab_row, int lg, int64_t j) {
  return ((int64_t)tab_row[j >> lg] << lg) | (j & (((int64_t)1 << lg) - 1));
}

__device__ __forceinline__ FRow row_info(KArgs& a, int r, bool paged) {
  FRow f;
  f.t = a.q_pos[r];
  f.tok_base = a.tok_off[r];
  f.pre_p = f.pre_h = f.pre_t = 0;
  f.ppbase = f.phbase = f.ptbase = 0;
  if (paged) {  // pooled rows through the page tables, counts clamped to what they map
    f.pbase = f.hbase = 0;
    const int64_t cp = (int64_t)a.max_pages << a.lg_page, ch = (int64_t)a.max_hpages << a.lg_hpage;
    const int64_t P = a.plen[r] < cp ? a.plen[r] : cp, Ph = a.hplen[r] < ch ? a.hplen[r] : ch;
    const int64_t v = (f.t + 1) / a.m, vh = (f.t + 1) / a.m_hca;
    f.n_vis = v < P ? v : P;
    f.n_vis_h = vh < Ph ? vh : Ph;
    return f;
  }
  f.pbase = a.pool_off[r];
  f.hbase = a.hpool_off[r];
  if (a.pre_seq) {
    const int32_t s = a.pre_seq[r];
    const int64_t T = a.pre_tok[r];
    if (s >= 0 && s < a.R && s != r && T > 0) {
      // clamped to what the holder stores, so every read stays in its segment
      f.ppbase = a.pool_off[s];
      f.phbase = a.hpool_off[s];
      f.ptbase = a.tok_off[s];
      const int64_t sp = a.pool_off[s + 1] - f.ppbase, sh = a.hpool_off[s + 1] - f.phbase;
      const int64_t st = a.tok_off[s + 1] - f.ptbase;
      f.pre_p = T / a.m < sp ? T / a.m : sp;
      f.pre_h = T / a.m_hca < sh ? T / a.m_hca : sh;
      f.pre_t = T < st ? T : st;
    }
  }
  const int64_t P = f.pre_p + a.pool_off[r + 1] - f.pbase, Ph = f.pre_h + a.hpool_off[r + 1] - f.hbase;
  const int64_t v = (f.t + 1) / a.m, vh = (f.t + 1) / a.m_hca;
  f.n_vis = v < P ? v : P;
  f.n_vis_h = vh < Ph ? vh : Ph;
  return f;
}

// A row's score chunks and lists.  The row's visible range is split evenly
// into as few chunks as keep each at most the plan's C entries (nsc <= the
// plan's n_sc; a multiple of 32 entries each), and the row's n_sc * lst list
// positions are shared by its chunks: L positions per chunk, at least Lm of
// them filled when the chunk has that many entries.  A short row thus has few
// chunks with long lists, and every row's per-chunk share of the top-k is
// covered the same way.
struct RowLayout {
  int nsc;
  int64_t C;
  uint32_t L, Lm, npos;
};
__device__ __forceinline__ RowLayout row_layout(KArgs& a, const FRow& f) {
  RowLayout o;
  const int64_t nv = f.n_vis > 0 ? f.n_vis : 1;
  int64_t n = (nv + a.C - 1) / a.C;
  o.nsc = (int)(n < 1 ? 1 : (n > a.n_sc ? a.n_sc : n));
  int64_t c = ((nv + o.nsc - 1) / o.nsc + 31) & ~(int64_t)31;
  o.C = c > a.C ? a.C : c;
  uint32_t L = (uint32_t)(((int64_t)a.n_sc * a.lst / o.nsc) & ~(int64_t)3);
  if (L > (uint32_t)o.C) L = (uint32_t)o.C;
  o.L = L;
  const uint32_t share = (uint32_t)((a.k + o.nsc - 1) / o.nsc);
  const uint32_t Lm = 2 * share + 16;
  o.Lm = Lm < L ? Lm : L;
  o.npos = (uint32_t)o.nsc * L;
  return o;
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
  bool paged;  // pooled caches through page tables (a compile-time constant of the kernel)
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
  const uint32_t incl = wave_incl_add(tot);
  if (lane == 63) scr[wave] = incl;
  __syncthreads();
  const uint4 wt = *reinterpret_cast<const uint4*>(scr);
  uint32_t run = incl - tot + (wave > 0 ? wt.x : 0u) + (wave > 1 ? wt.y : 0u) + (wave > 2 ? wt.z : 0u);
  const uint32_t all = wt.x + wt.y + wt.z + wt.w;
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

// exclusive prefix of v over the workgroup (thread order); *total = the sum
__device__ __forceinline__ uint32_t block_exscan_val(uint32_t v, uint32_t* scr, uint32_t* total) {
  const int tid = lane_tid(), lane = tid & 63, wave = tid >> 6;
  const uint32_t incl = wave_incl_add(v);
  if (lane == 63) scr[16 + wave] = incl;
  __syncthreads();
  const uint4 w = *reinterpret_cast<const uint4*>(scr + 16);  // one LDS read for the four wave totals
  const uint32_t run = incl - v + (wave > 0 ? w.x : 0u) + (wave > 1 ? w.y : 0u) + (wave > 2 ? w.z : 0u);
  *total = uni(w.x + w.y + w.z + w.w);
  __syncthreads();
  return run;
}

// [lo, hi] = the range of the workgroup's valid keys (each thread holds NK in
// registers, key i valid when bit i of vm is set; at least one valid key in
// the workgroup).
// Also clears the two 2048-bin histograms at hist (16-byte aligned).
template <int NK>
__device__ __forceinline__ void key_range(const uint32_t (&kv)[NK], uint32_t vm, uint32_t* hist, uint32_t* scr,
                                          uint32_t* lo, uint32_t* hi) {
  const int tid = lane_tid(), lane = tid & 63, wave = tid >> 6;
  uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    const bool v = (vm >> i) & 1u;
    mn = v && kv[i] < mn ? kv[i] : mn;
    mx = v && kv[i] > mx ? kv[i] : mx;
  }
  wave_minmax(mn, mx);
  if (lane == 0) {
    scr[8 + wave] = mn;
    scr[12 + wave] = mx;
  }
  for (int i = tid; i < 2 * kFHist / 4; i += 256) reinterpret_cast<uint4*>(hist)[i] = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();
  const uint4 l4 = *reinterpret_cast<const uint4*>(scr + 8), h4 = *reinterpret_cast<const uint4*>(scr + 12);
  const uint32_t l01 = l4.x < l4.y ? l4.x : l4.y, l23 = l4.z < l4.w ? l4.z : l4.w;
  const uint32_t h01 = h4.x > h4.y ? h4.x : h4.y, h23 = h4.z > h4.w ? h4.z : h4.w;
  *lo = uni(l01 < l23 ? l01 : l23);
  *hi = uni(h01 > h23 ? h01 : h23);
}

// One radix pass over the keys in [lo, hi] (lo < hi), cut into at most 2048
// bins of width 2^shift: the bin that holds the need-th largest of them
// (need <= their count) -> [*blo, *bhi], *above = keys above that bin, *cnt =
// keys in it.  hist: 2048 zeroed words, left zeroed; trash: 64 words that
// take the counts of keys outside the range (one per lane: the count loop
// has no branches and no colliding atomics on them).
template <int NK>
__device__ __forceinline__ void radix_pass(const uint32_t (&kv)[NK], uint32_t vm, uint32_t need, uint32_t* hist,
                                           uint32_t* trash, uint32_t* scr, uint32_t lo, uint32_t hi, uint32_t* blo,
                                           uint32_t* bhi, uint32_t* above, uint32_t* cnt) {
  const int tid = lane_tid(), lane = tid & 63, wave = tid >> 6;
  const uint32_t span = hi - lo;
  const int nbits = 32 - __clz((int)span);
  const int shift = nbits > 11 ? nbits - 11 : 0;
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    const bool in = ((vm >> i) & 1u) && kv[i] >= lo && kv[i] <= hi;
    atomicAdd(in ? hist + ((kv[i] - lo) >> shift) : trash + lane, 1u);
  }
  __syncthreads();
  uint32_t c[8], tot = 0;
  {
    uint4* h4 = reinterpret_cast<uint4*>(hist + 8 * tid);
    const uint4 a0 = h4[0], a1 = h4[1];
    h4[0] = make_uint4(0u, 0u, 0u, 0u);
    h4[1] = make_uint4(0u, 0u, 0u, 0u);
    c[0] = a0.x; c[1] = a0.y; c[2] = a0.z; c[3] = a0.w;
    c[4] = a1.x; c[5] = a1.y; c[6] = a1.z; c[7] = a1.w;
  }
#pragma unroll
  for (int b = 0; b < 8; ++b) tot += c[b];
  const uint32_t incl = wave_incl_add(tot);
  if (lane == 63) scr[wave] = incl;
  __syncthreads();
  const uint4 wt = *reinterpret_cast<const uint4*>(scr);
  const uint32_t all = wt.x + wt.y + wt.z + wt.w;
  const uint32_t below = incl - tot + (wave > 0 ? wt.x : 0u) + (wave > 1 ? wt.y : 0u) + (wave > 2 ? wt.z : 0u);
  const uint32_t sup = all - below - tot;  // keys in bins above this thread's 8
  if (sup < need && sup + tot >= need) {  // walk this thread's bins downwards (unrolled)
    uint32_t cum = sup, asel = 0;
    int bsel = -1;
#pragma unroll
    for (int b = 7; b >= 1; --b) {
      if (bsel < 0) {
        if (cum + c[b] >= need) {
          bsel = b;
          asel = cum;
        } else {
          cum += c[b];
        }
      }
    }
    if (bsel < 0) {
      bsel = 0;
      asel = cum;
    }
    uint32_t cb = c[0];
#pragma unroll
    for (int b = 1; b < 8; ++b) cb = b == bsel ? c[b] : cb;
    scr[S_DIGIT] = (uint32_t)(8 * tid + bsel);
    scr[S_ABOVE] = asel;
    scr[S_CNT] = cb;
  }
  __syncthreads();
  const uint32_t digit = uni(scr[S_DIGIT]);
  *above = uni(scr[S_ABOVE]);
  *cnt = uni(scr[S_CNT]);
  const uint32_t nlo = lo + (digit << shift);
  const uint32_t width_m1 = (uint32_t)(((uint64_t)1 << shift) - 1u);
  *blo = nlo;
  *bhi = hi - nlo > width_m1 ? nlo + width_m1 : hi;
}

// The need-th largest key (1 <= need <= number of valid keys) among the
// workgroup's keys, each thread holding NK of them in registers (key i valid
// when bit i of vm is set): radix select over the keys' own range, each pass narrowing it to one
// of at most 2048 bins (so keys spread over the bins whatever their
// magnitude), at most 3 passes.  Returns the key; *gt = the keys above it.
// A pass that leaves one key in the range ends the search.  *eq = the keys
// equal to it (n_valid when they are all equal).  hist: 2 x 2048 + 64 words of
// LDS, 16-byte aligned.
template <int NK>
__device__ __forceinline__ uint32_t kth_key_in(const uint32_t (&kv)[NK], uint32_t vm, uint32_t need, uint32_t n_valid,
                                               uint32_t* hist, uint32_t* scr, uint32_t* gt, uint32_t* eq,
                                               uint32_t lo, uint32_t hi);
template <int NK>
__device__ __forceinline__ uint32_t kth_key(const uint32_t (&kv)[NK], uint32_t vm, uint32_t need, uint32_t n_valid,
                                            uint32_t* hist, uint32_t* scr, uint32_t* gt, uint32_t* eq) {
  uint32_t lo, hi;
  key_range<NK>(kv, vm, hist, scr, &lo, &hi);
  return kth_key_in<NK>(kv, vm, need, n_valid, hist, scr, gt, eq, lo, hi);
}
// The same search when the keys' range [lo, hi] is known and both histograms
// are zeroed (and a barrier has ordered that before the first pass).
template <int NK>
__device__ __forceinline__ uint32_t kth_key_in(const uint32_t (&kv)[NK], uint32_t vm, uint32_t need, uint32_t n_valid,
                                               uint32_t* hist, uint32_t* scr, uint32_t* gt, uint32_t* eq,
                                               uint32_t lo, uint32_t hi) {
  uint32_t above_all = 0, in_range = n_valid;
#pragma unroll 1
  for (int pass = 0; pass < 3 && lo != hi; ++pass) {
    uint32_t blo, bhi, above, cnt;
    radix_pass<NK>(kv, vm, need, hist + (pass & 1) * kFHist, hist + 2 * kFHist, scr, lo, hi, &blo, &bhi, &above,
                   &cnt);
    need -= above;
    above_all += above;
    lo = blo;
    hi = bhi;
    in_range = cnt;
    if (cnt == 1u && lo != hi) {  // the one key in [lo, hi]
#pragma unroll
      for (int i = 0; i < NK; ++i)
        if (((vm >> i) & 1u) && kv[i] >= lo && kv[i] <= hi) scr[S_KEY] = kv[i];
      __syncthreads();
      lo = hi = uni(scr[S_KEY]);
      __syncthreads();
    } else if (cnt <= 64u && lo != hi) {
      // few keys left in [lo, hi]: gather them (in no particular order) and
      // rank each against the others instead of another pass; the key with
      // (greater < need <= greater + equal) is the answer
      uint32_t* cand = hist + (pass & 1 ? 0 : kFHist);  // the idle histogram
      uint32_t inr = 0;  // this thread's keys in [lo, hi]
#pragma unroll
      for (int i = 0; i < NK; ++i) inr |= (((vm >> i) & 1u) && kv[i] >= lo && kv[i] <= hi) ? (1u << i) : 0u;
      uint32_t n_in;
      uint32_t at = block_exscan_val((uint32_t)__builtin_popcount(inr), scr, &n_in);  // n_in == cnt
#pragma unroll
      for (int i = 0; i < NK; ++i)
        if ((inr >> i) & 1u) cand[at++] = kv[i];
      __syncthreads();
      const int tid = lane_tid();
      if (tid < (int)cnt) {
        const uint32_t mine = cand[tid];
        uint32_t g = 0, e = 0;
        for (uint32_t j = 0; j < cnt; ++j) {
          const uint32_t o = cand[j];
          g += o > mine ? 1u : 0u;
          e += o == mine ? 1u : 0u;
        }
        if (g < need && g + e >= need) {  // equal keys write the same words
          scr[S_KEY] = mine;
          scr[S_ABOVE] = g;
          scr[S_CNT] = e;
        }
      }
      __syncthreads();
      lo = hi = uni(scr[S_KEY]);
      above_all += uni(scr[S_ABOVE]);
      in_range = uni(scr[S_CNT]);
      __syncthreads();
    }
  }
  *gt = above_all;
  *eq = in_range;
  return lo;
}

// ---------------------------------------------------------------------------
// score: chunk c of row r -> keys in LDS and in the workspace, then the
// chunk's list: its lst largest entries in (key descending, index ascending)
// order, stored in ascending index order, and the list's tagged header
// ---------------------------------------------------------------------------
__device__ __forceinline__ void phase_score(const FCtx& x, int r, int c, const FRow& f, int64_t j0, int64_t j1) {
  KArgs& a = *x.a;
  const int tid = lane_tid(), lane = tid & 63, wave = tid >> 6, kb = lane >> 5;
  uint32_t* keys_s = reinterpret_cast<uint32_t*>(x.smem + kOffKeys);
  uint32_t* hist = reinterpret_cast<uint32_t*>(x.smem + kOffHist);
  // A operand: rows 0..3 = the query's 4 heads, K block lane/32
  v8i av = {0, 0, 0, 0, 0, 0, 0, 0};
  int asc = 127;
  if ((lane & 31) < 4) {
    const int64_t qrow = (int64_t)r * 4 + (lane & 3);
    uint4 u = *reinterpret_cast<const uint4*>(a.q_codes + qrow * 32 + kb * 16);
    asc = fold_head_weight(u, (int)a.q_scales[qrow * 2 + kb], a.w[qrow]);  // w_h folded into the block scale
    av[0] = (int)u.x; av[1] = (int)u.y; av[2] = (int)u.z; av[3] = (int)u.w;
  }
  // 32-entry MFMA tiles; wave w takes tiles w, w+4, ...; 16 tiles per wave per batch of loads
  const int n = (int)(j1 - j0);
  const int ntiles = (n + 31) >> 5;
  const RowLayout lay = row_layout(a, f);
  const uint32_t L = lay.L;
  const bool trunc = (uint32_t)n > L;
  // a truncated chunk counts its keys into fixed bins as they are made (the
  // LDS atomics hide under the key stream)
  uint32_t* fh = reinterpret_cast<uint32_t*>(x.smem + kOffU);
  // paged caches: the chunk's page ids -> LDS first (the key loads need them)
  const bool paged = x.paged;
  const int lg = a.lg_page;
  uint32_t* pg_s = fh + kFBinPad;
  int64_t pfirst = 0;
  if (paged) {
    const int32_t* trow = a.ptab + (size_t)r * a.max_pages;
    pfirst = j0 >> lg;
    const int64_t npg = j1 > j0 ? ((j1 - 1) >> lg) - pfirst + 1 : 0;  // j1 <= n_vis <= max_pages << lg
    for (int64_t i = tid; i < npg; i += 256) pg_s[i] = (uint32_t)trow[pfirst + i];
    __syncthreads();
  }
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
        const int64_t pj = paged ? (((int64_t)pg_s[(j >> lg) - pfirst] << lg) | (j & (((int64_t)1 << lg) - 1)))
                                 : pool_row(f, j);
        kcv[u] = *reinterpret_cast<const uint4*>(a.k_codes + pj * 32 + kb * 16);
        ksv[u] = a.k_scales[pj * 2 + kb];
      }
    }
    if (tb == 0 && trunc) {  // cleared while the first loads are in flight
      for (int i = tid; i < kFBinPad / 4; i += 256) reinterpret_cast<uint4*>(fh)[i] = make_uint4(0u, 0u, 0u, 0u);
      __syncthreads();
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
        // ReLU on the bit pattern (also maps -0 to +0), then the head sum
        const float r0 = __int_as_float(max(__float_as_int(acc[0]), 0));
        const float r1 = __int_as_float(max(__float_as_int(acc[1]), 0));
        const float r2 = __int_as_float(max(__float_as_int(acc[2]), 0));
        const float r3 = __int_as_float(max(__float_as_int(acc[3]), 0));
        const uint32_t key = __float_as_uint((r0 + r1) + (r2 + r3));
        keys_s[jl + (jl >> 4)] = key;
        if (trunc) atomicAdd(fh + (key >> 19) + (key >> 23), 1u);  // bin key >> 19, padded
      }
    }
  }
  __syncthreads();
  // thread t owns the local entries [t*M, t*M + M)
  const int M = (n + 255) >> 8;
  const int e0 = tid * M;
  const int nv = n - e0 < 0 ? 0 : (n - e0 < M ? n - e0 : M);
  uint32_t kv[kFKPT];
#pragma unroll
  for (int i = 0; i < kFKPT; ++i) kv[i] = i < nv ? keys_s[e0 + i + ((e0 + i) >> 4)] : 0u;
  // The list: every entry with key >= tau, where tau is the lower edge of the
  // fixed bin holding the chunk's lst_min-th largest key when listing that bin
  // stays within lst entries; otherwise one radix pass over that bin's key
  // range places tau at the lower edge of the sub-bin holding it, or of the
  // sub-bin above it when listing that one would pass lst entries.  Chunks with
  // at most lst entries list them all.
  uint32_t tau = 0;
  if (trunc) {
    const uint32_t need = lay.Lm;  // <= L < n
    // thread t: bins [16t, 16t + 16), in keys-descending order from the top thread
    uint32_t hc[16], tot = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      hc[i] = fh[17 * tid + i];
      tot += hc[i];
    }
    const uint32_t incl = wave_incl_add(tot);
    if (lane == 63) x.scr[wave] = incl;
    __syncthreads();
    const uint4 wt = *reinterpret_cast<const uint4*>(x.scr);
    const uint32_t all = wt.x + wt.y + wt.z + wt.w;
    const uint32_t below = incl - tot + (wave > 0 ? wt.x : 0u) + (wave > 1 ? wt.y : 0u) + (wave > 2 ? wt.z : 0u);
    const uint32_t sup = all - below - tot;  // keys in the bins above this thread's
    if (sup < need && sup + tot >= need) {
      uint32_t cum = sup, asel = 0, bsel = 0, csel = 0;
      bool found = false;
#pragma unroll
      for (int b = 15; b >= 0; --b) {
        if (!found) {
          if (cum + hc[b] >= need) {
            found = true;
            bsel = (uint32_t)b;
            asel = cum;
            csel = hc[b];
          } else {
            cum += hc[b];
          }
        }
      }
      x.scr[S_DIGIT] = 16u * (uint32_t)tid + bsel;
      x.scr[S_ABOVE] = asel;
      x.scr[S_CNT] = csel;
    }
    __syncthreads();
    const uint32_t bin = uni(x.scr[S_DIGIT]), above = uni(x.scr[S_ABOVE]), cnt = uni(x.scr[S_CNT]);
    if (above + cnt <= L) {
      tau = bin << 19;
    } else {
      const uint32_t vm = (1u << nv) - 1u;
      for (int i = tid; i < kFHist / 4; i += 256) reinterpret_cast<uint4*>(hist)[i] = make_uint4(0u, 0u, 0u, 0u);
      __syncthreads();
      uint32_t blo, bhi, ab2, cnt2;
      radix_pass<kFKPT>(kv, vm, need - above, hist, hist + 2 * kFHist, x.scr, bin << 19, ((bin + 1u) << 19) - 1u, &blo,
                        &bhi, &ab2, &cnt2);
      tau = above + ab2 + cnt2 <= L ? blo : bhi + 1u;
    }
  }
  uint32_t cg = 0;
#pragma unroll
  for (int i = 0; i < kFKPT; ++i) cg += (i < nv && kv[i] >= tau) ? 1u : 0u;
  uint32_t n_list;
  uint32_t pos = block_exscan_val(cg, x.scr, &n_list);
  // the listed (key, index) pairs in ascending index order -> LDS (the
  // histograms are no longer needed), then every list position -> workspace
  uint2* lst_s = reinterpret_cast<uint2*>(x.smem + kOffU);
  const uint32_t jbase = (uint32_t)(c * lay.C) + (uint32_t)e0;
#pragma unroll
  for (int i = 0; i < kFKPT; ++i)
    if (i < nv && kv[i] >= tau) lst_s[pos++] = make_uint2(kv[i], jbase + (uint32_t)i);
  __syncthreads();
  const size_t slot = (size_t)r * a.n_sc + c;
  v4u_t* dst = a.lent + (size_t)r * a.n_sc * a.lst + (size_t)c * L;
  for (uint32_t t = (uint32_t)tid; t < L; t += 256) {
    const uint2 e = t < n_list ? lst_s[t] : make_uint2(kNoKey, kNoKey);
    coh_st128(x.coh, dst + t, v4u_t{x.tag, e.x, x.tag, e.y});
  }
  if (tid == 0) st_dev64(a.ltau + slot, tagged(x.tag, n_list < (uint32_t)n ? tau : 0u));
  // then all the keys -> workspace, read only by the exact fallback: stored after the
  // list is published (their drain would hold the list back), with a header of their own
  {
    uint32_t* gk = a.keys + (size_t)r * a.key_stride + j0;
    for (int i = 4 * tid; i < n; i += 1024) {
      if (i + 3 < n) {
        const uint32_t* k4 = keys_s + i + (i >> 4);  // i % 16 <= 12: the four share one run
        const v4u_t u = {k4[0], k4[1], k4[2], k4[3]};
        coh_st128(x.coh, gk + i, u);
      } else {
        for (int e = i; e < n; ++e)
          __builtin_amdgcn_raw_buffer_store_b32(keys_s[e + (e >> 4)], x.coh.r, coh_off(x.coh, gk + e), 0, kSc1);
      }
    }
  }
  vm_drain();
  __syncthreads();
  if (tid == 0) st_dev64(a.key_hdr + slot, tagged(x.tag, 1u));
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

// Per-chunk thresholds of a row, or per-chunk counts, in LDS (key region).
__device__ __forceinline__ uint32_t* row_cnts(const FCtx& x) { return reinterpret_cast<uint32_t*>(x.smem + kOffKeys); }
__device__ __forceinline__ uint32_t* row_taus(const FCtx& x) { return row_cnts(x) + (kFMaxSlots + 8); }

__device__ __forceinline__ uint32_t lanes_below(uint64_t b) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
}

// Exact selection of row r over all of its stored keys, when its chunks' lists
// cannot decide it (run by the row's first CSA group).  The k_eff-th entry in
// (key descending, index ascending) order is found by a radix select over the
// keys and then over the indices of the entries equal to its key; published:
// row_k = K*, row_cut = its index, and each CSA group's output offset.
__device__ __forceinline__ bool row_fallback(const FCtx& x, int r, const FRow& f, int k_eff) {
  KArgs& a = *x.a;
  const int tid = lane_tid();
  const int ngrp = a.n_cs_sel, cgs = a.cg;
  const RowLayout lay = row_layout(a, f);
  const int nsc = lay.nsc;
  uint32_t* hist = reinterpret_cast<uint32_t*>(x.smem + kOffHist);
  if (tid == 0) atomicAdd(a.ctl + W_FALLBACK, 1u);
  {
    bool kfail = false;
    for (int sl = tid; sl < nsc && !kfail; sl += 256) (void)poll_word(x, a.key_hdr + (size_t)r * a.n_sc + sl, &kfail, 64u);
    if (!all_ok(x, kfail)) return false;
  }
  const uint32_t* rowkeys = a.keys + (size_t)r * a.key_stride;
  uint32_t nl;
  const uint32_t n_vis = n_vis_u32(f);
  const uint32_t kstar = radix_select_desc(
      n_vis, (uint32_t)k_eff, [&](uint32_t i) { return coh_ld32(x.coh, rowkeys + i); }, [&](uint32_t) { return true; },
      &nl, hist, x.scr);
  uint32_t nl2;
  const uint32_t njstar = radix_select_desc_low(
      n_vis, nl, 18, 0xfffc0000u, [&](uint32_t i) { return ~i; },
      [&](uint32_t i) { return coh_ld32(x.coh, rowkeys + i) == kstar; }, &nl2, hist, x.scr);
  if (tid == 0) {
    st_dev64(a.row_k + r, tagged(x.tag, kstar));
    st_dev64(a.row_cut + r, tagged(x.tag, ~njstar & 0x3ffffu));
  }
  const uint64_t cstar = ((uint64_t)kstar << 32) | njstar;
  // selected count per chunk -> offsets at the group starts
  const uint32_t C = (uint32_t)lay.C;
  uint32_t* e_sel = row_taus(x);
  for (int sl = tid; sl < nsc; sl += 256) {
    uint32_t cnt = 0;
    const uint32_t jb = (uint32_t)sl * C, je = jb + C < n_vis ? jb + C : n_vis;
    for (uint32_t j = jb; j < je; ++j)
      cnt += (((uint64_t)coh_ld32(x.coh, rowkeys + j) << 32) | (uint32_t)~j) >= cstar ? 1u : 0u;
    e_sel[sl] = cnt;
  }
  __syncthreads();
  block_exscan(e_sel, nsc, x.scr);
  for (int g = tid; g < ngrp; g += 256)
    st_dev64(a.grp_off + (size_t)r * ngrp + g, tagged(x.tag, e_sel[g * cgs < nsc ? g * cgs : nsc]));
  __syncthreads();
  return true;
}

// CSA group g of row r: score chunks [c0, c1) = [g*cg, g*cg + cg).  The row
// takes the k_eff first entries in (key descending, index ascending) order.
// Each score chunk listed every entry whose key is at least its threshold tau
// (all of its entries when it has at most lst), in ascending index order, at
// list positions chunk * lst + rank, so positions ascend with the index.  The
// group reads the whole row's lists and thresholds (every group of the row
// computes the same result): K* = the k_eff-th largest listed key; the row
// takes every listed entry above K* and the r_eq = k_eff - (listed keys above
// K*) listed entries equal to K* of lowest position.  This is the exact
// selection when every truncated chunk has tau <= K*: each entry of the row
// with key >= K* is then listed, so the listed keys >= K* are all of the
// row's, ties included.  Otherwise the row's first group runs the exact
// selection over the stored keys (row_fallback) and every group takes its
// entries from the stored keys.  Result: the group's selected indices in
// ascending order -> LDS, their count (or -1 on a failed wait, or -2 with the
// number of a score chunk of the row to compute first in *off_out), and their
// output offset in the row's idx -> *off_out; the entries sit at
// sel_s[*base_out ..] (the exact path stores them at their output rank).
// (*phys_out: with paged caches, whether the selected rows' physical rows are
// already in LDS beside them)
__device__ __forceinline__ int group_select(const FCtx& x, int r, int g, const FRow& f, uint32_t* off_out,
                                            uint32_t* base_out, bool* phys_out) {
  KArgs& a = *x.a;
  const int tid = lane_tid();
  const int cgs = a.cg;
  const int k_eff = (int)(f.n_vis < a.k ? f.n_vis : a.k);
  // the group's share of the row's list positions: the plan's chunks [g*cg, g*cg + cg)
  // times lst (positions past the row's npos hold nothing)
  const int pc0 = g * cgs < a.n_sc ? g * cgs : a.n_sc, pc1 = pc0 + cgs < a.n_sc ? pc0 + cgs : a.n_sc;
  const uint32_t P0 = (uint32_t)(pc0 * a.lst), P1 = (uint32_t)(pc1 * a.lst);
  const RowLayout lay = row_layout(a, f);
  const int nsc = lay.nsc;
  const uint32_t npos = lay.npos;
  // in the exact fallback the group takes the row's chunks [c0, c1)
  const int c0 = g * cgs < nsc ? g * cgs : nsc, c1 = c0 + cgs < nsc ? c0 + cgs : nsc;
  int32_t* sel_s = reinterpret_cast<int32_t*>(x.smem + kOffSel);
  uint32_t* e_tau = row_taus(x);
  uint32_t* hist = reinterpret_cast<uint32_t*>(x.smem + kOffHist);
  if (g == 0) {
    int32_t* idx_out = a.idx + (size_t)r * a.k;
    for (int i = k_eff + tid; i < a.k; i += 256) idx_out[i] = -1;
  }
  *base_out = 0;
  if (k_eff == 0) {  // nothing visible: every list is empty
    *off_out = 0;
    return 0;
  }
  // the row's lists: thread t holds positions u * 256 + t (keys and indices in
  // registers), and the chunks' thresholds -> LDS
  const v4u_t* lrow = a.lent + (size_t)r * a.n_sc * a.lst;
  const uint64_t* trow = a.ltau + (size_t)r * a.n_sc;  // chunk c's word at r * n_sc + c (the plan's n_sc)
  uint32_t kv[kFEPT], ix[kFEPT];
  uint32_t vm = 0;
  bool fail = false, steal = false;
  uint32_t steal_c = 0xffffffffu;  // the lowest chunk this thread found missing (when it gave up waiting)
  {
    v4u_t e[kFEPT];
#pragma unroll
    for (int u = 0; u < kFEPT; ++u) {
      const uint32_t p = (uint32_t)(u * 256 + tid);
      e[u] = p < npos ? coh_ld128(x.coh, lrow + p) : v4u_t{x.tag, kNoKey, x.tag, kNoKey};
    }
    uint64_t tw0 = tid < nsc ? coh_ld64(x.coh, trow + tid) : tagged(x.tag, 0u);
    uint64_t tw1 = tid + 256 < nsc ? coh_ld64(x.coh, trow + tid + 256) : tagged(x.tag, 0u);
    // entries not written yet are all read again together (one bounded retry loop)
    for (uint32_t n = 0;;) {
      bool late = (uint32_t)(tw0 >> 32) != x.tag || (uint32_t)(tw1 >> 32) != x.tag;
#pragma unroll
      for (int u = 0; u < kFEPT; ++u) late |= e[u][0] != x.tag || e[u][2] != x.tag;
      if (!late) break;
      if (++n >= (uint32_t)a.steal_polls) {  // far longer than a running chunk takes
        steal = true;
        break;
      }
      if (n >= kSpinLimit || ((n & 1023u) == 0 && error_seen(x))) {
        if (n >= kSpinLimit) set_error(x, 2u);
        fail = true;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
#pragma unroll
      for (int u = 0; u < kFEPT; ++u)
        if (e[u][0] != x.tag || e[u][2] != x.tag) e[u] = coh_ld128(x.coh, lrow + u * 256 + tid);
      if ((uint32_t)(tw0 >> 32) != x.tag) tw0 = coh_ld64(x.coh, trow + tid);
      if ((uint32_t)(tw1 >> 32) != x.tag) tw1 = coh_ld64(x.coh, trow + tid + 256);
    }
    if (steal) {
      if ((uint32_t)(tw0 >> 32) != x.tag) steal_c = (uint32_t)tid;
      if ((uint32_t)(tw1 >> 32) != x.tag && (uint32_t)tid + 256u < steal_c) steal_c = (uint32_t)tid + 256u;
#pragma unroll
      for (int u = 0; u < kFEPT; ++u) {
        const uint32_t c = (uint32_t)(u * 256 + tid) / lay.L;
        if ((e[u][0] != x.tag || e[u][2] != x.tag) && c < steal_c) steal_c = c;
      }
    }
#pragma unroll
    for (int u = 0; u < kFEPT; ++u) {
      kv[u] = fail || steal ? kNoKey : e[u][1];
      ix[u] = e[u][3];
      vm |= kv[u] != kNoKey ? (1u << u) : 0u;
    }
    if (tid < nsc) e_tau[tid] = (uint32_t)tw0;
    if (tid + 256 < nsc) e_tau[tid + 256] = (uint32_t)tw1;
  }
  // Warm the caches with the rows listed at the group's first 256 positions
  // (its selected rows are among them when P1 - P0 <= 256) while K* is found:
  // one word of each 128-byte line, consumed only once the ranks are known.
  uint32_t warm0 = 0, warm1 = 0, warm2 = 0, warm3 = 0;
  const int uw = (int)(P0 >> 8);
  int32_t pr_w = 0;  // the physical row of this thread's entry at slot uw (when it is listed)
  *phys_out = false;
  {
    uint32_t kw = kNoKey, iw = 0;
#pragma unroll
    for (int v = 0; v < kFEPT; ++v) {
      kw = v == uw ? kv[v] : kw;
      iw = v == uw ? ix[v] : iw;
    }
    const uint32_t p = (uint32_t)(uw * 256 + tid);
    if (kw != kNoKey && p >= P0 && p < P1) {  // a listed entry: iw < the row's visible count
      const int64_t pr = x.paged ? paged_row(a.ptab + (size_t)r * a.max_pages, a.lg_page, iw) : pool_row(f, iw);
      pr_w = (int32_t)pr;
      const uint32_t* row = reinterpret_cast<const uint32_t*>(a.kv_pool + (size_t)pr * 512u);
      warm0 = row[0];
      warm1 = row[32];
      warm2 = row[64];
      warm3 = row[96];
    }
  }
  // A chunk whose list is still missing after that long may belong to a
  // first-round workgroup that has not started (another kernel holds its CU):
  // the group has the lowest such chunk computed by its own workgroup and is
  // run again.  A score chunk is a pure function of the inputs, so a second
  // run of it (by a late owner) rewrites identical words.
  // One round of wave reductions and one barrier give every thread the
  // failure and steal flags, the number of listed entries and their key
  // range (K*'s first pass needs no range pass of its own); the radix
  // histograms are cleared beside them.
  uint32_t wfail, wsteal, n_ent, klo, khi;
  {
    const int lane = tid & 63, wave = tid >> 6;
    uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
    for (int u = 0; u < kFEPT; ++u) {
      const bool v = (vm >> u) & 1u;
      mn = v && kv[u] < mn ? kv[u] : mn;
      mx = v && kv[u] > mx ? kv[u] : mx;
    }
    wave_minmax(mn, mx);
    uint32_t st = steal ? steal_c : 0xffffffffu, st_hi = 0u;
    wave_minmax(st, st_hi);
    const uint32_t cnt = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_add((uint32_t)__builtin_popcount(vm)), 63);
    const bool wf = __ballot(fail) != 0ull;
    for (int i = tid; i < 2 * kFHist / 4; i += 256) reinterpret_cast<uint4*>(hist)[i] = make_uint4(0u, 0u, 0u, 0u);
    if (tid == 0) x.scr[S_BAD] = 0;
    if (lane == 0) *reinterpret_cast<uint4*>(x.scr + 20 + 4 * wave) = make_uint4(cnt, mn, mx, wf ? 0xfffffffeu : st);
    __syncthreads();
    const uint4 r0 = *reinterpret_cast<const uint4*>(x.scr + 20), r1 = *reinterpret_cast<const uint4*>(x.scr + 24);
    const uint4 r2 = *reinterpret_cast<const uint4*>(x.scr + 28), r3 = *reinterpret_cast<const uint4*>(x.scr + 32);
    n_ent = uni(r0.x + r1.x + r2.x + r3.x);
    klo = uni(min(min(r0.y, r1.y), min(r2.y, r3.y)));
    khi = uni(max(max(r0.z, r1.z), max(r2.z, r3.z)));
    wfail = (r0.w == 0xfffffffeu || r1.w == 0xfffffffeu || r2.w == 0xfffffffeu || r3.w == 0xfffffffeu) ? 1u : 0u;
    wsteal = uni(min(min(r0.w, r1.w), min(r2.w, r3.w)));
  }
  if (wfail) return -1;
  if (wsteal != 0xffffffffu) {
    *off_out = wsteal;
    return -2;
  }
  bool exact = n_ent >= (uint32_t)k_eff;
  uint32_t kstar = 0, gt_all = 0, eq_all = 0;
  uint32_t* lk = reinterpret_cast<uint32_t*>(x.smem + kOffU);  // [npos] keys by position
  uint32_t* li = lk + kFEntLds;                                 // [npos] indices by position
  if (exact) {
    if (npos <= 16u * 256u) {
      uint32_t kv16[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) kv16[u] = kv[u];
      kstar = kth_key_in<16>(kv16, vm & 0xffffu, (uint32_t)k_eff, n_ent, hist, x.scr, &gt_all, &eq_all, klo, khi);
    } else {
      kstar = kth_key_in<kFEPT>(kv, vm, (uint32_t)k_eff, n_ent, hist, x.scr, &gt_all, &eq_all, klo, khi);
    }
    for (int sl = tid; sl < nsc; sl += 256)
      if (e_tau[sl] > kstar) x.scr[S_BAD] = 1;
    if (gt_all + eq_all == (uint32_t)k_eff) {
      // every listed entry equal to K* is taken, so the row takes exactly the
      // listed entries with key >= K*: one scan in position order (slot u,
      // then thread) ranks the group's own positions, and its first field
      // counts the taken positions below P0 (the group's output offset)
      const int32_t ks = (int32_t)kstar;
      uint32_t pre = 0;
#pragma unroll
      for (int u = 0; u < kFEPT; ++u) pre += ((int32_t)kv[u] >= ks && (uint32_t)(u * 256 + tid) < P0) ? 1u : 0u;
      const int u0 = (int)(P0 >> 8), u1r = (int)((P1 + 255u) >> 8), u1 = u1r > u0 ? u1r : u0 + 1;
      uint32_t off = 0, run = 0;
      for (int u = u0; u < u1; ++u) {  // uniform; one slot when the group's positions are one 256-aligned run
        uint32_t ku = kNoKey, iu = 0;
#pragma unroll
        for (int v = 0; v < kFEPT; ++v) {
          ku = v == u ? kv[v] : ku;
          iu = v == u ? ix[v] : iu;
        }
        const uint32_t p = (uint32_t)(u * 256 + tid);
        const bool take = (int32_t)ku >= ks && p >= P0 && p < P1;
        uint32_t tot;
        const uint32_t ex = block_exscan_val((take ? 1u : 0u) | (u == u0 ? pre << 16 : 0u), x.scr, &tot);
        if (u == u0) off = tot >> 16;
        if (take) {
          sel_s[off + run + (ex & 0xffffu)] = (int32_t)iu;
          if (x.paged)  // the physical row beside it: from the warm-up at slot uw, else looked up
            reinterpret_cast<int32_t*>(x.smem + kOffSelP)[off + run + (ex & 0xffffu)] =
                u == uw ? pr_w : (int32_t)paged_row(a.ptab + (size_t)r * a.max_pages, a.lg_page, iu);
        }
        run += tot & 0xffffu;
      }
      exact = uni(x.scr[S_BAD]) == 0u;  // the scans' barriers ordered the threshold checks
      __syncthreads();
      if (exact) {
        asm volatile("" ::"v"(warm0), "v"(warm1), "v"(warm2), "v"(warm3));
        *off_out = off;
        *base_out = off;
        *phys_out = x.paged;
        return (int)run;
      }
    }
  }
  if (exact) {
    // to contiguous ownership (the histograms are free again): thread t takes
    // positions [t*M, t*M + M), so position order is thread order
    // (unconditional: kFEPT * 256 = kFEntLds, and positions past npos hold kNoKey)
#pragma unroll
    for (int u = 0; u < kFEPT; ++u) {
      const uint32_t p = (uint32_t)(u * 256 + tid);
      lk[p] = kv[u];
      li[p] = ix[u];
    }
    __syncthreads();
    exact = uni(x.scr[S_BAD]) == 0u;
  }
  if (exact) {
    const uint32_t r_eq = (uint32_t)k_eff - gt_all;  // >= 1
    constexpr uint32_t M = kFEPT;  // positions per thread (16-byte aligned runs)
    const uint32_t m0 = (uint32_t)tid * M;
    uint32_t ck[kFEPT], ci[kFEPT];
#pragma unroll
    for (int e4 = 0; e4 < kFEPT / 4; ++e4) {
      const uint32_t q = m0 + 4u * (uint32_t)e4;
      const uint4 kk = q < npos ? *reinterpret_cast<const uint4*>(lk + q) : make_uint4(kNoKey, kNoKey, kNoKey, kNoKey);
      const uint4 ii = q < npos ? *reinterpret_cast<const uint4*>(li + q) : make_uint4(0u, 0u, 0u, 0u);
      ck[4 * e4] = kk.x; ck[4 * e4 + 1] = kk.y; ck[4 * e4 + 2] = kk.z; ck[4 * e4 + 3] = kk.w;
      ci[4 * e4] = ii.x; ci[4 * e4 + 1] = ii.y; ci[4 * e4 + 2] = ii.z; ci[4 * e4 + 3] = ii.w;
    }
    // empty positions hold kNoKey, which is -1 as a signed value: below every
    // key (finite scores are >= 0) and never equal to K*
    const int32_t ks = (int32_t)kstar;
    uint32_t cgt = 0, ceq = 0;
#pragma unroll
    for (int e = 0; e < kFEPT; ++e) {
      cgt += (int32_t)ck[e] > ks ? 1u : 0u;
      ceq += ck[e] == kstar ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t pre = block_exscan_val(cgt | (ceq << 16), x.scr, &tot);
    const uint32_t pre_gt = pre & 0xffffu, pre_eq = pre >> 16;
    if (pre_eq < r_eq && pre_eq + ceq >= r_eq) {  // this thread holds the r_eq-th entry equal to K*
      uint32_t e2 = pre_eq, cut = 0;
#pragma unroll
      for (int e = 0; e < kFEPT; ++e)
        if (ck[e] == kstar && ++e2 == r_eq) cut = m0 + (uint32_t)e;
      x.scr[S_CUT] = cut;
    }
    __syncthreads();
    const uint32_t pcut = uni(x.scr[S_CUT]);
    // each taken entry's output rank: the taken entries before this thread,
    // then its own in position order; the group's entries go to sel_s[rank]
    const uint32_t rank0 = pre_gt + (pre_eq < r_eq ? pre_eq : r_eq);
    uint32_t rank = rank0, tkm = 0;
    int32_t* const dummy = sel_s + kFMaxSel + (tid & 63);  // the stores of entries not taken
#pragma unroll
    for (int e = 0; e < kFEPT; ++e) {
      const uint32_t p = m0 + (uint32_t)e;
      const uint32_t tk = ((int32_t)ck[e] > ks ? 1u : 0u) | (ck[e] == kstar && p <= pcut ? 1u : 0u);
      const bool mine = tk != 0u && p >= P0 && p < P1;
      *(mine ? sel_s + rank : dummy) = (int32_t)ci[e];
      tkm |= tk << e;
      rank += tk;
    }
    if (P0 - m0 < M) x.scr[S_OFF] = rank0 + (uint32_t)__builtin_popcount(tkm & ((1u << (P0 - m0)) - 1u));
    if (P1 - m0 < M) x.scr[S_END] = rank0 + (uint32_t)__builtin_popcount(tkm & ((1u << (P1 - m0)) - 1u));
    if (tid == 0 && P0 >= npos) x.scr[S_OFF] = (uint32_t)k_eff;
    if (tid == 0 && P1 >= npos) x.scr[S_END] = (uint32_t)k_eff;
    __syncthreads();
    const uint32_t off = uni(x.scr[S_OFF]);
    *off_out = off;
    *base_out = off;
    return (int)(uni(x.scr[S_END]) - off);
  }
  // not decidable from the lists: the exact selection over the stored keys
  if (g == 0 && !row_fallback(x, r, f, k_eff)) return -1;
  uint32_t w3[3];
  {
    const uint64_t* const pw[3] = {a.row_k + r, a.row_cut + r, a.grp_off + (size_t)r * a.n_cs_sel + g};
    const bool use[3] = {true, true, true};
    if (tid == 0) {
      read_tagged<3>(x, pw, use, w3, &fail);
      x.scr[S_KEY] = w3[0];
      x.scr[S_CUT] = w3[1];
      x.scr[S_DIGIT] = w3[2];
    }
  }
  if (!all_ok(x, fail)) return -1;
  const uint32_t kstar_f = uni(x.scr[S_KEY]), jstar = uni(x.scr[S_CUT]);
  *off_out = uni(x.scr[S_DIGIT]);
  // the order key (key, ~index) of every visible entry of the group's chunks
  bool kfail = false;
  for (int sl = c0 + tid; sl < c1 && !kfail; sl += 256) (void)poll_word(x, a.key_hdr + (size_t)r * a.n_sc + sl, &kfail, 64u);
  if (!all_ok(x, kfail)) return -1;
  const uint64_t cstar = ((uint64_t)kstar_f << 32) | (uint32_t)~jstar;
  const uint32_t* rowkeys = a.keys + (size_t)r * a.key_stride;
  const uint32_t C = (uint32_t)lay.C, nvis = n_vis_u32(f);
  const uint32_t jb = (uint32_t)c0 * C, je = (uint32_t)c1 * C < nvis ? (uint32_t)c1 * C : nvis;
  const uint32_t n = je > jb ? je - jb : 0u;
  const uint32_t M = (n + 255) >> 8, m0 = (uint32_t)tid * M;
  uint32_t cntf = 0, tot;
  for (uint32_t i = 0; i < M; ++i) {
    const uint32_t j = jb + m0 + i;
    if (m0 + i < n) cntf += (((uint64_t)coh_ld32(x.coh, rowkeys + j) << 32) | (uint32_t)~j) >= cstar ? 1u : 0u;
  }
  uint32_t pos = block_exscan_val(cntf, x.scr, &tot);
  for (uint32_t i = 0; i < M; ++i) {
    const uint32_t j = jb + m0 + i;
    if (m0 + i < n && (((uint64_t)coh_ld32(x.coh, rowkeys + j) << 32) | (uint32_t)~j) >= cstar)
      sel_s[pos++] = (int32_t)j;
  }
  __syncthreads();
  return (int)tot;
}

// the group's selected indices -> idx at its output offset
__device__ __forceinline__ void group_write_idx(const FCtx& x, int r, uint32_t off, int n_sel, uint32_t base) {
  KArgs& a = *x.a;
  const int tid = lane_tid();
  const int32_t* sel_s = reinterpret_cast<const int32_t*>(x.smem + kOffSel) + base;
  int32_t* dst = a.idx + (size_t)r * a.k + off;
  for (int i = tid; i < n_sel && off + (uint32_t)i < (uint32_t)a.k; i += 256) dst[i] = sel_s[i];
}

// Attention item: CSA group (kind 0, its n_sel selected rows in LDS), CSA
// window split (kind 1) or HCA split (kind 2) of row r, then its partial.
__device__ __forceinline__ void attend_item(const FCtx& x, int r, int kind, int s, const FRow& f, int n_sel,
                                            uint32_t sel_base = 0) {
  KArgs& a = *x.a;
  int64_t p_begin, p_end;
  int pi = s;
  if (kind == 0) {
    p_begin = 0;
    p_end = n_sel;
  } else if (kind == 1) {
    p_begin = (int64_t)s * a.cs;
    p_end = p_begin + a.cs < a.W ? p_begin + a.cs : a.W;
    pi = a.n_cs_sel + s;
  } else {
    const int64_t list_len = a.max_hpool + a.W_hca;
    p_begin = (int64_t)s * a.hs;
    p_end = p_begin + a.hs < list_len ? p_begin + a.hs : list_len;
    if (a.W_hca == 0 && p_end > f.n_vis_h) p_end = f.n_vis_h > p_begin ? f.n_vis_h : p_begin;  // past the row's rows
  }
  const int32_t* idx_s = reinterpret_cast<const int32_t*>(x.smem + kOffSel) + sel_base;
  constexpr uint64_t RB = 2 * 128 * 2;
  // Row addresses from 32-bit offsets against per-row bases: list positions
  // below `split` are pooled rows (selected ones for kind 0, HCA rows for
  // kind 2), the rest are window tokens t - W + 1 + (p - split).  Logical
  // rows below the shared prefix's count come from the prefix holder.
  const uint8_t* pool_base = kind == 0 ? a.kv_pool + (size_t)f.pbase * RB : a.kv_hpool + (size_t)f.hbase * RB;
  const uint8_t* pre_pool = kind == 0 ? a.kv_pool + (size_t)f.ppbase * RB : a.kv_hpool + (size_t)f.phbase * RB;
  const int32_t pre_pool_n = (int32_t)(kind == 0 ? f.pre_p : f.pre_h);
  const uint8_t* raw_base = a.kv_raw + (size_t)f.tok_base * RB;
  const uint8_t* pre_raw = a.kv_raw + (size_t)f.ptbase * RB;
  const int32_t pre_raw_n = (int32_t)f.pre_t;
  const int32_t pb32 = (int32_t)p_begin;
  const int32_t split = kind == 1 ? 0 : (int32_t)a.max_hpool;
  const int32_t hi_pool = (int32_t)f.n_vis_h;
  const int32_t win_off = (int32_t)(f.t + 1 - (kind == 1 ? a.W : a.W_hca)) - split;
  auto pooled = [&](int32_t j) -> const uint8_t* {
    return j < pre_pool_n ? pre_pool + (uint64_t)(uint32_t)j * RB
                          : pool_base + (uint64_t)(uint32_t)(j - pre_pool_n) * RB;
  };
  // paged caches: CSA groups read the physical rows their selection was
  // translated to; an HCA split takes its range's page ids into LDS first
  const bool paged = x.paged;
  const int32_t* idx_p = reinterpret_cast<const int32_t*>(x.smem + kOffSelP) + sel_base;
  uint32_t* hpg_s = reinterpret_cast<uint32_t*>(x.smem + kOffSel);
  const int hlg = a.lg_hpage;
  const int32_t hfirst = (int32_t)(p_begin >> hlg);
  if (paged && kind == 2) {
    const int64_t pe = p_end < f.n_vis_h ? p_end : f.n_vis_h;  // <= max_hpages << hlg
    const int64_t npg = pe > p_begin ? ((pe - 1) >> hlg) - hfirst + 1 : 0;
    const int32_t* trow = a.hptab + (size_t)r * a.max_hpages;
    for (int64_t i = lane_tid(); i < npg; i += 256) hpg_s[i] = (uint32_t)trow[hfirst + i];
    __syncthreads();
  }
  auto rowptr = [&](int64_t p64) -> const uint8_t* {
    const int32_t p = (int32_t)p64;
    if (kind == 0) {
      const int32_t j = idx_s[p - pb32];
      if (j < 0) return nullptr;
#ifdef CSA_DEBUG
      if (j >= (int32_t)f.n_vis) {
        debug_violation();
        return nullptr;
      }
#endif
      return paged ? a.kv_pool + (uint64_t)(uint32_t)idx_p[p - pb32] * RB : pooled(j);
    }
    if (p < split) {
      if (p >= hi_pool) return nullptr;
      if (!paged) return pooled(p);
      const uint32_t pr = (hpg_s[(p >> hlg) - hfirst] << hlg) | ((uint32_t)p & ((1u << hlg) - 1u));
      return a.kv_hpool + (uint64_t)pr * RB;
    }
    const int32_t u = p + win_off;
    if (u < 0) return nullptr;
    return u < pre_raw_n ? pre_raw + (uint64_t)(uint32_t)u * RB : raw_base + (uint64_t)(uint32_t)(u - pre_raw_n) * RB;
  };
  AttnState<1> st;
  attn_init<1>(st, a.q + (size_t)r * a.H * 128 * 2, a.H);
  attn_run<1>(st, a.H, a.scale_log2, p_begin, p_end, rowptr, x.smem + kOffU);
  write_partial(x, st, r, pi, kind == 2);
}

// merge of 4 heads (h0 .. h0+3) of one row: thread = (head, 2 dims)
// HPM (8 or 16) heads of row r from head h0: 256 / HPM threads per head,
// HPM / 2 output dims per thread
template <int HPM>
__device__ __forceinline__ void merge_heads(const FCtx& x, bool hca, int r, int h0, int n) {
  KArgs& a = *x.a;
  const int tid = lane_tid();
  const int n_cs = a.n_cs_sel + a.n_cs_win;
  const int ns = hca ? a.n_hs : n_cs;  // partial slots per row
  const float* po = hca ? a.hca_po : a.csa_po;
  const float* pml = hca ? a.hca_pml : a.csa_pml;
  uint8_t* out = hca ? a.hca_out : a.csa_out;
  float* lse = hca ? a.hca_lse : a.csa_lse;
  // every split's (m, l) of this thread's head and its output values, all
  // loaded at once (one round of loads per SB splits), merged online
  constexpr int TPH = 256 / HPM, DPT = 128 / TPH;  // threads per head, dims per thread
  const int hh = tid / TPH, h = h0 + hh, d = (tid % TPH) * DPT;
  constexpr int SB = HPM == 8 ? 16 : 8;
  float M = -INFINITY, L = 0.f, acc[DPT];
#pragma unroll
  for (int i = 0; i < DPT; ++i) acc[i] = 0.f;
  for (int s0 = 0; s0 < n; s0 += SB) {
    uint64_t mlv[SB];
    uint32_t ov[SB][DPT];
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      const int s = s0 + u;
      const size_t pb = ((size_t)r * ns + s) * a.H + h;
      mlv[u] = s < n ? coh_ld64(x.coh, pml + pb * 2) : (uint64_t)__float_as_uint(-INFINITY);
#pragma unroll
      for (int i = 0; i < DPT; i += 2) {
        const uint64_t v = s < n ? coh_ld64(x.coh, po + pb * 128 + d + i) : 0ull;
        ov[u][i] = (uint32_t)v;
        ov[u][i + 1] = (uint32_t)(v >> 32);
      }
    }
    float Mc = M;
#pragma unroll
    for (int u = 0; u < SB; ++u) Mc = fmaxf(Mc, __uint_as_float((uint32_t)mlv[u]));
    if (Mc == -INFINITY) continue;
    const float sc = M == -INFINITY ? 0.f : fast_exp2(M - Mc);
    L *= sc;
#pragma unroll
    for (int i = 0; i < DPT; ++i) acc[i] *= sc;
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      const float ms = __uint_as_float((uint32_t)mlv[u]);
      const float wgt = ms == -INFINITY ? 0.f : fast_exp2(ms - Mc);
      L = fmaf(wgt, __uint_as_float((uint32_t)(mlv[u] >> 32)), L);
#pragma unroll
      for (int i = 0; i < DPT; ++i) acc[i] = fmaf(wgt, __uint_as_float(ov[u][i]), acc[i]);
    }
    M = Mc;
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint32_t* o = reinterpret_cast<uint32_t*>(out + (((size_t)r * a.H + h) * 128 + d) * 2);
#pragma unroll
  for (int i = 0; i < DPT; i += 2) o[i / 2] = f32_to_bf16(acc[i] * inv) | (f32_to_bf16(acc[i + 1] * inv) << 16);
  if (lse && d == 0) lse[(size_t)r * a.H + h] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
}

// merge unit: a.hpm heads of row r from head h0 (4, or 16 for batches of many
// rows) over the row's first n partials (its n_cs CSA ones, or the HCA splits
// that were handed out for it; slots past those are not written)
__device__ __forceinline__ void item_merge(const FCtx& x, bool hca, int r, int h0, int n) {
  KArgs& a = *x.a;
  const int tid = lane_tid();
  const int n_cs = a.n_cs_sel + a.n_cs_win;
  const int ns = hca ? a.n_hs : n_cs;  // partial slots per row
  const uint64_t* hdr = a.part_hdr + (size_t)r * (n_cs + a.n_hs) + (hca ? n_cs : 0);
  bool fail = false;
  for (int s = tid; s < n && !fail; s += 256) (void)poll_word(x, hdr + s, &fail, hca ? 8u : 4u);
  if (!all_ok(x, fail)) return;
  if (a.hpm == 16) {
    merge_heads<16>(x, hca, r, h0, n);
    return;
  }
  if (a.hpm == 8) {
    merge_heads<8>(x, hca, r, h0, n);
    return;
  }
  // 4 heads: a thread per head and 2 dims, 24 splits per round of loads
  const float* po = hca ? a.hca_po : a.csa_po;
  const float* pml = hca ? a.hca_pml : a.csa_pml;
  uint8_t* out = hca ? a.hca_out : a.csa_out;
  float* lse = hca ? a.hca_lse : a.csa_lse;
  const int hh = tid >> 6, h = h0 + hh, d = (tid & 63) * 2;
  constexpr int SB = 24;
  float M = -INFINITY, L = 0.f, acc0 = 0.f, acc1 = 0.f;
  for (int s0 = 0; s0 < n; s0 += SB) {
    uint64_t mlv[SB], ov[SB];
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      const int s = s0 + u;
      const size_t pb = ((size_t)r * ns + s) * a.H + h;
      mlv[u] = s < n ? coh_ld64(x.coh, pml + pb * 2) : (uint64_t)__float_as_uint(-INFINITY);
      ov[u] = s < n ? coh_ld64(x.coh, po + pb * 128 + d) : 0ull;
    }
    float Mc = M;
#pragma unroll
    for (int u = 0; u < SB; ++u) Mc = fmaxf(Mc, __uint_as_float((uint32_t)mlv[u]));
    if (Mc == -INFINITY) continue;
    const float sc = M == -INFINITY ? 0.f : fast_exp2(M - Mc);
    L *= sc;
    acc0 *= sc;
    acc1 *= sc;
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      const float ms = __uint_as_float((uint32_t)mlv[u]);
      const float wgt = ms == -INFINITY ? 0.f : fast_exp2(ms - Mc);
      L = fmaf(wgt, __uint_as_float((uint32_t)(mlv[u] >> 32)), L);
      acc0 = fmaf(wgt, __uint_as_float((uint32_t)ov[u]), acc0);
      acc1 = fmaf(wgt, __uint_as_float((uint32_t)(ov[u] >> 32)), acc1);
    }
    M = Mc;
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint32_t* o = reinterpret_cast<uint32_t*>(out + (((size_t)r * a.H + h) * 128 + d) * 2);
  *o = f32_to_bf16(acc0 * inv) | (f32_to_bf16(acc1 * inv) << 16);
  if (lse && d == 0) lse[(size_t)r * a.H + h] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
}

// The row table, built by a workgroup before it decodes its first ticket when
// the plan has more score chunks than the first round takes (wave 0, lane r =
// row r): of row r's score chunks, those not numbered below
// `first` (the first round's chunks, numbered c * R + r) and its HCA splits
// (every split of the plan when the HCA list ends in a window, otherwise
// those that hold visible rows), with their row-major exclusive starts.  The
// ticket units are numbered over these counts, so the empty chunks and
// splits of short rows in a ragged batch are never handed out.
__device__ __forceinline__ void build_row_table(const FCtx& x, uint32_t first) {
  KArgs& a = *x.a;
  uint32_t* tab = reinterpret_cast<uint32_t*>(x.smem + kOffTab);
  const int r = lane_tid();
  if (r < 64) {
    const int R = a.R;
    uint32_t eb = 0, eh = 0;
    if (r < R) {
      // the chunk count of row_layout (the visible count is at most
      // kFMaxVisible, so 32-bit arithmetic is exact) and the splits holding
      // visible HCA rows (at most the plan's n_hs)
      const FRow f = row_info(a, r, x.paged);
      const uint32_t nv = f.n_vis > 1 ? (uint32_t)f.n_vis : 1u, C = (uint32_t)a.C;
      uint32_t nsc = (nv + C - 1u) / C;
      nsc = nsc > (uint32_t)a.n_sc ? (uint32_t)a.n_sc : nsc;
      const uint32_t c0 = first > (uint32_t)r ? (first - (uint32_t)r + (uint32_t)R - 1u) / (uint32_t)R : 0u;
      eb = nsc > c0 ? nsc - c0 : 0u;
      if (a.W_hca > 0) {
        eh = (uint32_t)a.n_hs;
      } else {
        const int64_t cap = (int64_t)a.n_hs * a.hs;
        const uint32_t nh = (uint32_t)(f.n_vis_h < cap ? f.n_vis_h : cap), hs = (uint32_t)a.hs;
        eh = (nh + hs - 1u) / hs;
      }
    }
    const uint32_t ib = wave_incl_add(eb), ih = wave_incl_add(eh);
    tab[T_EB + r] = ib - eb;
    tab[T_EH + r] = ih - eh;
    tab[T_NHS + r] = eh;
    const bool uni_h = __ballot(r < R && eh != (uint32_t)a.n_hs) == 0ull;
    if (r == 63) {
      tab[T_UB] = ib;
      tab[T_UH] = ih;
      tab[T_UNIH] = uni_h ? 1u : 0u;
    }
  }
  __syncthreads();
}

// The row holding unit j of a row-major count table with exclusive starts
// `starts` (R rows): the last row whose start is <= j (rows with no units
// share the next row's start and are passed over).  Each wave computes it
// (one LDS read per lane and a ballot); the result is the same in all.
__device__ __forceinline__ int table_row(const uint32_t* starts, int R, uint32_t j) {
  const int l = lane_tid() & 63;
  const bool le = l < R && starts[l] <= j;
  return (int)__builtin_popcountll(__ballot(le)) - 1;
}

// ---------------------------------------------------------------------------
// kPaged: the pooled caches are read through page tables (csa_hca_decode_paged)
// (one workgroup per CU, so one wave per SIMD: the compiler is told so and
// schedules without a second wave's register budget in mind)
// kCompact: the plan has more score chunks than the first round takes, so the
// ticket units are numbered over the row table (otherwise the table is
// compiled out and the plan's numbering is used)
template <bool kPaged, bool kCompact>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_decode_fused(FusedArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  uint32_t* scr = reinterpret_cast<uint32_t*>(smem + kOffScr);
  // the launch's tag: every thread loads the epoch word; the load is waited for
  // at the tag's first use (a first-round score chunk: when it publishes)
  const uint32_t tag0 = ld_dev(a.ctl + W_EPOCH) + 1u;
  const uint32_t tag = tag0 == 0u ? 1u : tag0;
  const int rounds = a.rounds;
  // Work units in dependency order: [score chunks | CSA groups | CSA window
  // splits | HCA splits | HCA merges | CSA merges].  The score chunks stream
  // first on every workgroup; the HCA stream then runs beside the
  // latency-bound selection chain.  The first-round score chunks (the first
  // min(score chunks, grid) units) are taken by workgroup id, so their key
  // streams start at once; every other unit number comes from one returning
  // atomic on a ticket counter, taken by a running workgroup one round ahead,
  // so those units are handed out in arrival order and are only ever held by
  // workgroups that have started.  A workgroup runs its units in the order it
  // holds them (ascending), and a unit only waits for units of lower number.
  // The only units a workgroup can hold before it starts are first-round
  // score chunks, and nothing waits for them blindly: a CSA group that has
  // waited far longer than a running chunk takes (steal_polls polls) computes
  // the missing chunk itself (a chunk is a pure function of the inputs, so
  // its late owner only rewrites the same words) and runs again.  So the
  // lowest unfinished unit is either such a chunk, computed by whoever waits
  // for it, or held by a running workgroup whose earlier units are done and
  // never waits: every wait ends however many of the grid's workgroups are
  // resident at a time.  The first-round chunks are numbered c * R + r over
  // the plan's n_sc chunks per row (those of short rows past the row's own
  // chunk count do nothing); when the plan has more chunks than the first
  // round takes, the ticket units are numbered over what each row has (the
  // row table), so a ragged batch hands out no empty chunk or HCA split.  A
  // workgroup stops at its first ticket past the last unit;
  // `rounds` bounds the rounds (rounds * grid covers every unit of the plan),
  // plus two for every chunk it computes for one of its groups.  (Unit
  // numbers fit 32 bits: the plan bounds them far below.)
  const uint32_t first = (uint32_t)a.first_units;
  const bool by_id = blockIdx.x < first;
  // lane 0: the unit number of the next ticket (fetched one unit ahead) and the
  // claims still to make; a group that has its workgroup compute a missing
  // chunk leaves the chunk and itself in two LDS words, taken before the next
  // ticket (no other state is carried from round to round)
  uint32_t next_ticket = 0;  // lane 0: the unit number of the next round, fetched one round ahead
  if (!by_id && lane_tid() == 0) next_ticket = first + atomicAdd(a.ctl + W_TICKET, 1u);
  // 1: run the chunk in scr[S_PENDC] (for a group of this workgroup), 2: then
  // that group (scr[S_PENDG]) again; such rounds claim nothing and do not count
  int pend = 0;
  bool tab_ready = false;  // the row table (uniform: every thread takes the same path)
  for (int round = 0; round < rounds; ++round) {
    KArgs* ap = (KArgs*)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(ap));
    KArgs& A = *ap;
    const FCtx x{ap, smem, scr, tag, make_coh(A.ctl), kPaged};
    const int R = A.R, nM = A.H / A.hpm;
    int64_t it;
    // a score chunk numbered c * R + r: the first round's, or one computed for a group
    bool old_chunk = false;
    if (pend != 0) {
      it = (int64_t)uni(scr[pend == 1 ? S_PENDC : S_PENDG]);
      old_chunk = pend == 1;
    } else {
      if (round == 0 && by_id) {
        it = (int64_t)blockIdx.x;
        old_chunk = true;
      } else {
        if (lane_tid() == 0) scr[S_TICKET] = next_ticket;
        __syncthreads();
        it = (int64_t)uni(scr[S_TICKET]);
        __syncthreads();
      }
      // claim the next round's unit now: the returning atomic's latency overlaps
      // this round's work.  A workgroup still runs its units in claim order.
      // (The compact form claims once the unit is decoded, below.)
      if (!kCompact && round + 1 < rounds && lane_tid() == 0) next_ticket = first + atomicAdd(A.ctl + W_TICKET, 1u);
    }
    // Ticket units (t = it - first), in dependency order: [the rows' remaining
    // score chunks | CSA groups | CSA window splits | HCA splits | HCA merges |
    // CSA merges]; units only wait for units of lower number.  When every
    // chunk of the plan ran in the first round (R * n_sc <= first, as in
    // batches of equal long rows) the units are the plan's (HCA splits
    // split-major, R * n_hs of them, those past a row's rows doing nothing);
    // otherwise they are numbered over the row table, which leaves out the
    // empty chunks and HCA splits of short rows (a ragged batch) at the cost
    // of building the table (one round of loads) before the first ticket.
    // The unit is decoded first (kind, row, index), then run from one call
    // site per kind (each phase is inlined once).
    int kind;  // 0 score chunk, 1 CSA group, 2 CSA window split, 3 HCA split, 4 HCA merge, 5 CSA merge
    int r, ui;
    int n_merge = 0;
    if (old_chunk) {
      // chunk-major: every row's first chunks come first (a short row uses fewer chunks)
      kind = 0;
      ui = (int)(it / R);
      r = (int)(it % R);
    } else {
      constexpr bool compact = kCompact;
      if (compact && !tab_ready) {  // once per workgroup
        build_row_table(x, first);
        tab_ready = true;
      }
      const uint32_t* tab = reinterpret_cast<const uint32_t*>(smem + kOffTab);
      const int64_t t = it - (int64_t)first;
      const int64_t t_grp = compact ? (int64_t)tab[T_UB] : 0;
      const int64_t t_win = t_grp + (int64_t)R * A.n_cs_sel, t_hca = t_win + (int64_t)R * A.n_cs_win;
      const int64_t t_mh = t_hca + (compact ? (int64_t)tab[T_UH] : (int64_t)R * A.n_hs);
      const int64_t t_mc = t_mh + (int64_t)R * nM, t_end = t_mc + (int64_t)R * nM;
      if (t >= t_end) break;  // every unit is handed out: no further claims
      if (t < t_grp) {
        kind = 0;
        r = table_row(tab + T_EB, R, (uint32_t)t);
        const uint32_t c0 = first > (uint32_t)r ? (first - (uint32_t)r + (uint32_t)R - 1u) / (uint32_t)R : 0u;
        ui = (int)(c0 + ((uint32_t)t - tab[T_EB + r]));
      } else if (t >= t_mh) {
        kind = t < t_mc ? 4 : 5;
        const int64_t m = t - (kind == 4 ? t_mh : t_mc);
        r = (int)(m / nM);
        ui = (int)(m % nM) * A.hpm;
        n_merge = kind == 4 ? (compact ? (int)tab[T_NHS + r] : A.n_hs) : A.n_cs_sel + A.n_cs_win;
      } else if (t < t_hca) {
        kind = t < t_win ? 1 : 2;
        const int64_t q = t - (kind == 1 ? t_grp : t_win);
        r = (int)(q % R);
        ui = (int)(q / R);
      } else {  // HCA split: split-major when every row has all of them, else row-major
        kind = 3;
        const uint32_t j = (uint32_t)(t - t_hca);
        if (!compact || tab[T_UNIH] != 0u) {
          r = (int)(j % (uint32_t)R);
          ui = (int)(j / (uint32_t)R);
        } else {
          r = table_row(tab + T_EH, R, j);
          ui = (int)(j - tab[T_EH + r]);
        }
      }
    }
    // In the compact form (ragged batches) a CSA group's workgroup claims its
    // next unit only once its group is done: a group ends late, and group
    // workgroups arrive first for the next round's tickets, so the units they
    // would hold start last (ragged 32 rows: 65.3 -> 55.6 us; with equal rows
    // it measured no better).  Every other unit claims the next one now.
    if (kCompact && pend == 0 && kind != 1 && round + 1 < rounds && lane_tid() == 0)
      next_ticket = first + atomicAdd(A.ctl + W_TICKET, 1u);
    if (kind == 0) {  // score chunk ui of row r
      const FRow f = row_info(A, r, kPaged);
      const RowLayout lay = row_layout(A, f);
      if (ui < lay.nsc) {
        int64_t j0 = (int64_t)ui * lay.C, j1 = j0 + lay.C;
        if (j1 > f.n_vis) j1 = f.n_vis;
        if (j0 > j1) j0 = j1;
        phase_score(x, r, ui, f, j0, j1);
      }
      if (pend == 1) {  // computed for a group of this workgroup: out before it reads them back
        vm_drain();
        __syncthreads();
        pend = 2;
      }
    } else if (kind >= 4) {
      item_merge(x, kind == 4, r, ui, n_merge);
    } else if (kind == 1) {
      const int g = ui;
      const FRow f = row_info(A, r, kPaged);
      uint32_t off = 0, base = 0;
      bool phys = false;
      const int n_sel = group_select(x, r, g, f, &off, &base, &phys);
      pend = 0;
      if (n_sel == -2) {  // run the row's missing chunk `off`, then this group again
        if (lane_tid() == 0) {
          scr[S_PENDC] = (uint32_t)((int64_t)off * R + r);
          scr[S_PENDG] = (uint32_t)it;
        }
        __syncthreads();
        pend = 1;
        round -= 2;  // two rounds of their own (the chunk, the group again): no claims, not counted
      } else if (n_sel >= 0) {
        if (kPaged && !phys) {  // paged caches: the selected rows' physical rows -> LDS
          const int32_t* sel_s = reinterpret_cast<const int32_t*>(smem + kOffSel) + base;
          int32_t* sel_p = reinterpret_cast<int32_t*>(smem + kOffSelP) + base;
          const int32_t* trow = A.ptab + (size_t)r * A.max_pages;
          for (int i = lane_tid(); i < n_sel; i += 256) sel_p[i] = (int32_t)paged_row(trow, A.lg_page, sel_s[i]);
          __syncthreads();
        }
        attend_item(x, r, 0, g, f, n_sel, base);
        group_write_idx(x, r, off, n_sel, base);
      }
      if (kCompact && n_sel != -2 && round + 1 < rounds && lane_tid() == 0)
        next_ticket = first + atomicAdd(A.ctl + W_TICKET, 1u);
    } else {
      // a CSA window split (attend_item's kind 1) or an HCA split (its kind 2)
      attend_item(x, r, kind == 2 ? 1 : 2, ui, row_info(A, r, kPaged), 0);
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
// grid size per device (0 = not known yet): the occupancy query runs once
// per device; concurrent first calls compute the same value, so a relaxed
// atomic store is enough
constexpr int kMaxDevices = 64;
static std::atomic<int> g_fused_grid[kMaxDevices];

static int fused_grid() {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < kMaxDevices) {
    const int g = g_fused_grid[dev].load(std::memory_order_relaxed);
    if (g > 0) return g;
  }
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipFuncSetAttribute((const void*)k_decode_fused<false, false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                          kFusedLds0) != hipSuccess ||
      hipFuncSetAttribute((const void*)k_decode_fused<true, false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                          kFusedLds0) != hipSuccess ||
      hipFuncSetAttribute((const void*)k_decode_fused<false, true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                          kFusedLds) != hipSuccess ||
      hipFuncSetAttribute((const void*)k_decode_fused<true, true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                          kFusedLds) != hipSuccess)
    return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)k_decode_fused<false, true>, 256, kFusedLds) !=
      hipSuccess)
    return 0;
  if (per_cu < 1 || cus < 1) return 0;
  // One workgroup per CU: two score workgroups sharing a CU's memory pipeline
  // finish far apart (the second one's stores drain late), and the selection
  // waits for the last chunk of every row.
  if (dev < kMaxDevices) g_fused_grid[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Polls of a CSA group's list wait after which it computes a missing score
// chunk itself: far longer than a running chunk takes (each poll is a
// device-coherent load), so it only happens when the chunk's workgroup has not
// started.  CSA_FUSED_STEAL_POLLS (1 .. 2^19) overrides it; a small value
// makes groups compute chunks that are merely late, which changes no output.
static int steal_polls() {
  const char* e = std::getenv("CSA_FUSED_STEAL_POLLS");
  if (e && *e) {
    const long v = std::strtol(e, nullptr, 10);
    if (v >= 1 && v < (long)kSpinLimit) return (int)v;
  }
  return 4096;
}

static int split_count(int64_t len, int64_t size) { return len <= 0 ? 0 : (int)((len + size - 1) / size); }

#ifdef CSA_DEBUG
unsigned long long debug_take_fused() { return debug_take_here(); }
#endif

FusedPlan plan_fused(int64_t R, int64_t max_pool, int64_t max_hpool, int H, int k, int W, int W_hca) {
  FusedPlan p{};
  const int G = fused_grid();
  p.grid = G;
  p.cs = 128;
  p.n_cs_win = split_count(W, p.cs);
  p.hs = 256;
  p.n_hs = split_count(max_hpool + W_hca, p.hs);
  if (p.n_hs == 0) p.n_hs = 1;
  // score chunk: the smallest multiple of 256 (>= 1024) that gives every chunk a
  // workgroup of its own (more chunks than workgroups: later rounds take the rest)
  int64_t C = 1024;
  if (G > 0) {
    const int64_t per = (R * max_pool + G - 1) / G;
    if (per > C) C = ((per + 255) / 256) * 256;
  }
  p.C = (int)(C > kFMaxC ? kFMaxC : C);
  p.n_sc = max_pool > 0 ? (int)((max_pool + p.C - 1) / p.C) : 1;
  // CSA groups: consecutive chunks holding about 64 selected entries each for
  // up to 8 rows, 128 for more (measured: fewer, longer groups pay off once
  // the rows' groups would take more than a quarter of the grid)
  const int per_group = R > 8 ? 128 : 64;
  const int64_t want = split_count(k, per_group) > 0 ? split_count(k, per_group) : 1;
  p.cg = (int)((p.n_sc + want - 1) / want);
  if (p.cg < 1) p.cg = 1;
  p.n_cs_sel = (p.n_sc + p.cg - 1) / p.cg;
  // heads per merge unit: as many as keep a unit's partials near 66 KB (at
  // most 128 partials of one head), so batches of many short rows need fewer
  // units (each unit is one claim on the ticket counter, whose returning
  // atomics are served one at a time) while long rows keep their merges spread
  {
    const int nmax = p.n_cs_sel + p.n_cs_win > p.n_hs ? p.n_cs_sel + p.n_cs_win : p.n_hs;
    p.hpm = nmax * 16 <= 128 && H % 16 == 0 ? 16 : (nmax * 8 <= 128 && H % 8 == 0 ? 8 : 4);
  }
  // listed per chunk: about twice a chunk's expected share of the top-k plus
  // slack, and room for 16 more (a threshold bin's worth); the stride is a
  // multiple of 4, so lists are read 16 bytes at a time, and the row's listed
  // keys fit its LDS staging.  Short lists only make the exact fallback more
  // likely.
  const int64_t share = p.n_sc > 0 ? ((int64_t)k + p.n_sc - 1) / p.n_sc : k;
  int64_t Lm = 2 * share + 16;
  int64_t L = Lm + 16;
  if (L * p.n_sc > kFEntLds) L = kFEntLds / p.n_sc;
  L &= ~(int64_t)3;
  if (L < 4) L = 4;
  if (L > p.C) L = p.C;
  if (Lm > L) Lm = L;
  p.lst_min = (int)Lm;
  p.lst = (int)L;
  p.key_stride = (max_pool + 3) & ~(int64_t)3;
  auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
  const size_t slots = (size_t)R * p.n_sc;
  const int n_cs = p.n_cs_sel + p.n_cs_win;
  size_t s = 0;
  s += al(W_CTL * 4);
  s += al((size_t)R * p.key_stride * 4);
  s += al(slots * 8);
  s += al(slots * p.lst * 16);
  s += al(slots * 8);
  s += al((size_t)R * 8);
  s += al((size_t)R * 8);
  s += al((size_t)R * p.n_cs_sel * 8);
  s += al((size_t)R * (n_cs + p.n_hs) * 8);
  s += al((size_t)R * n_cs * H * 128 * 4);
  s += al((size_t)R * n_cs * H * 2 * 4);
  s += al((size_t)R * p.n_hs * H * 128 * 4);
  s += al((size_t)R * p.n_hs * H * 2 * 4);
  p.ws_bytes = s;
  return p;
}

int fused_supported(int64_t R, int64_t max_pool, int64_t max_hpool, int H, int k, int W, int W_hca) {
  if (R < 1 || R > kFMaxRows || max_pool > (int64_t)kFMaxVisible || H % 16 != 0 || H > 64 || H < 16 || k > kFMaxSel)
    return 0;
  // the plan always fits: C <= kFMaxC and n_sc <= kFMaxVisible / 1024 <= kFMaxSlots
  return plan_fused(R, max_pool, max_hpool, H, k, W, W_hca).grid > 0 ? 1 : 0;
}

size_t fused_error_word_offset() { return W_ERROR * 4; }
size_t fused_fallback_word_offset() { return W_FALLBACK * 4; }

int launch_fused(int R, const int64_t* tok_off, const int64_t* q_pos, const int64_t* pool_off,
                 const int64_t* hpool_off, const int32_t* pre_seq, const int64_t* pre_tok, const FusedPaging* paging,
                 int64_t max_pool, int64_t max_hpool, int m, int m_hca, int H,
                 float scale, int k, int W, int W_hca, const uint8_t* q_codes, const uint8_t* q_scales,
                 const float* w, const uint8_t* k_codes, const uint8_t* k_scales, const void* q,
                 const void* kv_pool, const void* kv_hpool, const void* kv_raw, int32_t* idx, void* csa_out,
                 float* csa_lse, void* hca_out, float* hca_lse, void* ws, hipStream_t stream) {
  const FusedPlan pl = plan_fused(R, max_pool, max_hpool, H, k, W, W_hca);
  if (pl.grid <= 0) return -1;
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
  a.pre_seq = pre_seq; a.pre_tok = pre_tok;
  a.ptab = nullptr; a.plen = nullptr; a.hptab = nullptr; a.hplen = nullptr;
  a.max_pages = a.max_hpages = 0; a.lg_page = a.lg_hpage = 0;
  if (paging) {
    a.ptab = paging->ptab; a.plen = paging->plen; a.max_pages = paging->max_pages;
    a.hptab = paging->hptab; a.hplen = paging->hplen; a.max_hpages = paging->max_hpages;
    a.lg_page = __builtin_ctz((unsigned)paging->page_rows);
    a.lg_hpage = __builtin_ctz((unsigned)paging->hpage_rows);
  }
  a.R = R; a.m = m; a.m_hca = m_hca; a.H = H; a.k = k; a.W = W; a.W_hca = W_hca;
  a.scale_log2 = scale * kLog2e;
  a.max_pool = max_pool; a.max_hpool = max_hpool;
  a.q_codes = q_codes; a.q_scales = q_scales; a.w = w; a.k_codes = k_codes; a.k_scales = k_scales;
  a.q = (const uint8_t*)q; a.kv_pool = (const uint8_t*)kv_pool; a.kv_hpool = (const uint8_t*)kv_hpool;
  a.kv_raw = (const uint8_t*)kv_raw;
  a.idx = idx; a.csa_out = (uint8_t*)csa_out; a.csa_lse = csa_lse; a.hca_out = (uint8_t*)hca_out; a.hca_lse = hca_lse;
  a.C = pl.C; a.n_sc = pl.n_sc; a.cs = pl.cs; a.n_cs_sel = pl.n_cs_sel; a.n_cs_win = pl.n_cs_win; a.cg = pl.cg;
  a.hs = pl.hs; a.n_hs = pl.n_hs; a.hpm = pl.hpm;
  a.lst_min = pl.lst_min; a.lst = pl.lst; a.key_stride = pl.key_stride;
  {
    const int64_t units = (int64_t)R * pl.n_sc + (int64_t)R * (pl.n_cs_sel + pl.n_cs_win + pl.n_hs) +
                          2 * (int64_t)R * (H / pl.hpm);
    a.rounds = (int)((units + pl.grid - 1) / pl.grid);
    const int64_t chunks = (int64_t)R * pl.n_sc;
    a.first_units = (int)(chunks < pl.grid ? chunks : pl.grid);
    a.steal_polls = steal_polls();
  }
  a.ctl = (uint32_t*)take(W_CTL * 4);
  a.keys = (uint32_t*)take((size_t)R * pl.key_stride * 4);
  a.key_hdr = (uint64_t*)take(slots * 8);
  a.lent = (v4u_t*)take(slots * pl.lst * 16);
  a.ltau = (uint64_t*)take(slots * 8);
  a.row_k = (uint64_t*)take((size_t)R * 8);
  a.row_cut = (uint64_t*)take((size_t)R * 8);
  a.grp_off = (uint64_t*)take((size_t)R * pl.n_cs_sel * 8);
  a.part_hdr = (uint64_t*)take((size_t)R * (n_cs + pl.n_hs) * 8);
  a.csa_po = (float*)take((size_t)R * n_cs * H * 128 * 4);
  a.csa_pml = (float*)take((size_t)R * n_cs * H * 2 * 4);
  a.hca_po = (float*)take((size_t)R * pl.n_hs * H * 128 * 4);
  a.hca_pml = (float*)take((size_t)R * pl.n_hs * H * 2 * 4);
  // an ordinary launch of one workgroup per CU
  // the row table only when some chunks are left past the first round (a.first_units)
  const bool compact = (int64_t)R * pl.n_sc > (int64_t)a.first_units;
  const hipError_t e =
      compact ? launch(6, kProfBoth, paging ? k_decode_fused<true, true> : k_decode_fused<false, true>,
                       dim3((unsigned)pl.grid), dim3(256), kFusedLds, stream, a)
              : launch(6, kProfBoth, paging ? k_decode_fused<true, false> : k_decode_fused<false, false>,
                       dim3((unsigned)pl.grid), dim3(256), kFusedLds0, stream, a);
  if (e != hipSuccess) return -1;
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace csa

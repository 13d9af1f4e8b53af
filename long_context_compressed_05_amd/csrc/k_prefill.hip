// Lightning-indexer top-k for prefill batches (many queries per sequence),
// without materialising the score matrix.
//
// Pages: jyp-garden EP 95 notes, IDEAS (the Lightning Indexer keeps only the
// top-k compressed blocks); sigco.tistory.com CSA/HCA section (the indexer
// picks the blocks most relevant to each query); pytorch.kr FP4 QAT section
// (the indexer QK path is MXFP4).  Same score and order as the decode path:
//     S(i, j) = sum_h w[i][h] * max(0, qhat[i][h] . khat[j]),
// the k largest under (S descending, j ascending), indices in ascending order.
//
// Three kernels:
//  1. k_pf_thresh: per block of 4 queries of one sequence, the scores of a
//     sample of the keys (runs of 32 consecutive keys, one run every
//     32 * stride keys: 1 key in stride, each run one coalesced tile) -> LDS;
//     per query (one wave, one radix pass over the range of its visible
//     samples' nonzero scores) tau = the lower edge of the bin holding the
//     need_s-th largest sample score, need_s = ceil(2 k / stride), so that
//     about 2 k keys are >= tau; tau = 0 when the query sees at most k keys or
//     too few samples.
//  2. k_pf_score: every visible score exactly once on the block-scaled FP4
//     MFMA (8 queries x 4 heads x 32 keys per MFMA, two MFMAs per key tile),
//     compared with its query's tau: the output is a candidate bitmap, one bit
//     per (query, visible key).  This is the scoring pass; no score is stored.
//  3. k_pf_select: one wave per query: the candidates from its bitmap (in
//     ascending index order), their scores again (MFMA on the gathered keys),
//     K* = the k_eff-th largest by a radix select in the wave's LDS, then the
//     selected indices, in order.  Exact whenever at least k_eff keys are >=
//     tau (then K* >= tau and every key >= K* is a candidate); otherwise, or
//     when the candidates overflow the wave's LDS, the wave runs an exact
//     radix select over all of the query's visible keys, scored again on each
//     pass (slow, and only for such queries).  It also returns the query's
//     threshold and bitmap words to zero, so the workspace is left zero-filled.
//
// MFMA operands: A rows (lane & 31) = query slot (lane & 31) >> 2 and head
// lane & 3, K half lane >> 5; the power-of-two head weight is folded into the
// query's block scale.  B: key lane & 31, K half lane >> 5.  Output register
// 4s + h of lane l holds query slot 2s + (l >> 5), head h, key l & 31.  Every
// product and partial sum is a small dyadic rational, so the fp32 sums are
// exact and the score bit pattern (ReLU as an integer max, which also maps -0
// to +0) is an exact sort key.
#include <atomic>

#include "common.hpp"
#include "kernels.hpp"

namespace csa {

constexpr int kPfRowsT = 8;        // queries per threshold block: one per wave (one MFMA A operand)
constexpr int kPfThreads = 64 * kPfRowsT;
constexpr int kPfRows = 16;        // queries per score block (two MFMA A operands)
constexpr int kPfKeysWG = 4096;    // keys per scoring workgroup, at least (a multiple of 128)
constexpr int kPfSampleMax = 2048;  // sample keys per query
constexpr int kPfCand = 2048;      // candidates per query held in a wave's LDS
constexpr int kPfBins = 1024;      // wave radix-select bins
constexpr int kPfWaveHist = kPfBins + 64;  // + one trash word per lane
// the selection kernel's per-wave histogram: 256 bins (+ trash), so that a
// wave's LDS (2048 candidates + histogram) stays under 10 KB and every
// two-wave workgroup of a 4096-query chunk is resident at once (8 per CU)
constexpr int kSelBins = 256;
constexpr int kSelWaveHist = kSelBins + 64;
constexpr int kPfMinQ = 16;        // queries per sequence from which this path is used

struct PfArgs {
  const int64_t* q_off;
  const int64_t* q_pos;
  const int64_t* pool_off;
  int n_seq, bps, bps_t, m, k, stride, ns_max, bw;
  int kw;  // keys per scoring workgroup (a multiple of 128: 32-key tiles, 4 waves)
  int64_t n_q, max_pool;
  const uint8_t* q_codes;
  const uint8_t* q_scales;
  const float* w;
  const uint8_t* k_codes;
  const uint8_t* k_scales;
  uint32_t* tau;     // [n_q]
  uint32_t* bitmap;  // [n_q][bw]
  int32_t* idx;      // [n_q][k]
};

__device__ __forceinline__ int64_t pf_nvis(int64_t t, int m, int64_t P) {
  const int64_t v = (t + 1) / m;
  return v < P ? v : P;
}

// A operand: query slots [0, nslots) are rows row0 + slot, the others zero
__device__ __forceinline__ void pf_load_a(const PfArgs& a, int64_t row0, int nslots, int lane, v8i& av, int& asc) {
  const int slot = (lane & 31) >> 2, head = lane & 3, kb = lane >> 5;
  av = v8i{0, 0, 0, 0, 0, 0, 0, 0};
  asc = 127;
  if (slot < nslots) {
    const int64_t qrow = (row0 + slot) * 4 + head;
    uint4 u = *reinterpret_cast<const uint4*>(a.q_codes + qrow * 32 + kb * 16);
    asc = fold_head_weight(u, (int)a.q_scales[qrow * 2 + kb], a.w[qrow]);  // w_h folded into the block scale
    av[0] = (int)u.x; av[1] = (int)u.y; av[2] = (int)u.z; av[3] = (int)u.w;
  }
}

// B operand of pooled row gj (codes half lane >> 5), or zero
__device__ __forceinline__ void pf_load_b(const PfArgs& a, int64_t gj, bool ok, int kb, uint4& kc, int& ks) {
  kc = make_uint4(0u, 0u, 0u, 0u);
  ks = 127;
  if (ok) {
    kc = *reinterpret_cast<const uint4*>(a.k_codes + gj * 32 + kb * 16);
    ks = a.k_scales[gj * 2 + kb];
  }
}

__device__ __forceinline__ v16f pf_mfma(const v8i& av, int asc, const uint4& kc, int ks) {
  const v8i bv = {(int)kc.x, (int)kc.y, (int)kc.z, (int)kc.w, 0, 0, 0, 0};
  v16f acc = {};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 4, 4, 0, asc, 0, ks);
}

// sort key of score index s of this lane (query slot 2s + lane/32)
__device__ __forceinline__ uint32_t pf_key(const v16f& acc, int s) {
  const float r0 = __int_as_float(max(__float_as_int(acc[4 * s + 0]), 0));
  const float r1 = __int_as_float(max(__float_as_int(acc[4 * s + 1]), 0));
  const float r2 = __int_as_float(max(__float_as_int(acc[4 * s + 2]), 0));
  const float r3 = __int_as_float(max(__float_as_int(acc[4 * s + 3]), 0));
  return __float_as_uint((r0 + r1) + (r2 + r3));
}

// The candidate test key >= tau of score index s, in 7 operations instead of
// the key's 8.  For reals, max(a, 0) + max(b, 0) = max(a + b, a, b) whenever
// that is positive, and the sum is 0 otherwise; the same holds for the rounded
// sums (rounding is monotonic, and a + b rounds to a when b is 0), so
//   v = max3(p01 + p23, p01, p23),  p01 = max3(x0 + x1, x0, x1)  (p23 alike)
// equals the key's value (x0 + x1 ... in the key's order) when it is positive
// and is <= 0 exactly when the key is 0.  The maxima compare bit patterns as
// signed integers: right whenever one operand is positive, and a non-positive
// result is all that matters otherwise.  The test is then v >= tau as signed
// bit patterns, with tau = 0 (every key passes) mapped to INT_MIN
// (pf_tau_signed).
__device__ __forceinline__ int pf_tau_signed(uint32_t tau) {
  return tau == 0u ? (int)0x80000000u : (int)(tau < 0x7fffffffu ? tau : 0x7fffffffu);
}
__device__ __forceinline__ int pf_relu_sum_bits(const v16f& acc, int s) {
  const float x0 = acc[4 * s + 0], x1 = acc[4 * s + 1], x2 = acc[4 * s + 2], x3 = acc[4 * s + 3];
  const int p01 = max(max(__float_as_int(x0 + x1), __float_as_int(x0)), __float_as_int(x1));
  const int p23 = max(max(__float_as_int(x2 + x3), __float_as_int(x2)), __float_as_int(x3));
  return max(max(__float_as_int(__int_as_float(p01) + __int_as_float(p23)), p01), p23);
}

// candidate mask of score index E & 3 of MFMA output c (this lane's query
// E = 4 o + s: the query of lanes 0-31 is slot 2E, of lanes 32-63 slot 2E + 1);
// WHOLE: every query sees the tile's 32 keys; tq: thresholds by pf_tau_signed
template <int E, bool WHOLE>
__device__ __forceinline__ uint64_t pf_mask(const v16f& c, int j, const int (&nq)[kPfRows / 2],
                                            const int (&tq)[kPfRows / 2]) {
  const int v = pf_relu_sum_bits(c, E & 3);
  return __builtin_amdgcn_ballot_w64(WHOLE ? v >= tq[E] : (j < nq[E] && v >= tq[E]));
}

// one tile's 16 candidate words (query slot L in lane L): the 8 ballots' halves
// go straight from the scalar masks into lanes 0..15 with v_writelane; the
// masks are written by VALU compares, so the block starts with the wait states
// a VALU-written SGPR needs before v_writelane may read it
template <bool WHOLE>
__device__ __forceinline__ uint32_t pf_tile_word(const v8i (&av)[2], const int (&asc)[2], const uint4& kc, int ks,
                                                 int j, const int (&nq)[kPfRows / 2],
                                                 const int (&tq)[kPfRows / 2]) {
  uint64_t m[8];
  {
    const v16f c = pf_mfma(av[0], asc[0], kc, ks);
    m[0] = pf_mask<0, WHOLE>(c, j, nq, tq);
    m[1] = pf_mask<1, WHOLE>(c, j, nq, tq);
    m[2] = pf_mask<2, WHOLE>(c, j, nq, tq);
    m[3] = pf_mask<3, WHOLE>(c, j, nq, tq);
  }
  {
    const v16f c = pf_mfma(av[1], asc[1], kc, ks);
    m[4] = pf_mask<4, WHOLE>(c, j, nq, tq);
    m[5] = pf_mask<5, WHOLE>(c, j, nq, tq);
    m[6] = pf_mask<6, WHOLE>(c, j, nq, tq);
    m[7] = pf_mask<7, WHOLE>(c, j, nq, tq);
  }
  uint32_t word = 0u;
  asm("s_nop 4\n\t"
      "v_writelane_b32 %0, %1, 0\n\tv_writelane_b32 %0, %2, 1\n\t"
      "v_writelane_b32 %0, %3, 2\n\tv_writelane_b32 %0, %4, 3\n\t"
      "v_writelane_b32 %0, %5, 4\n\tv_writelane_b32 %0, %6, 5\n\t"
      "v_writelane_b32 %0, %7, 6\n\tv_writelane_b32 %0, %8, 7\n\t"
      "v_writelane_b32 %0, %9, 8\n\tv_writelane_b32 %0, %10, 9\n\t"
      "v_writelane_b32 %0, %11, 10\n\tv_writelane_b32 %0, %12, 11\n\t"
      "v_writelane_b32 %0, %13, 12\n\tv_writelane_b32 %0, %14, 13\n\t"
      "v_writelane_b32 %0, %15, 14\n\tv_writelane_b32 %0, %16, 15"
      : "+v"(word)
      : "s"((uint32_t)m[0]), "s"((uint32_t)(m[0] >> 32)), "s"((uint32_t)m[1]), "s"((uint32_t)(m[1] >> 32)),
        "s"((uint32_t)m[2]), "s"((uint32_t)(m[2] >> 32)), "s"((uint32_t)m[3]), "s"((uint32_t)(m[3] >> 32)),
        "s"((uint32_t)m[4]), "s"((uint32_t)(m[4] >> 32)), "s"((uint32_t)m[5]), "s"((uint32_t)(m[5] >> 32)),
        "s"((uint32_t)m[6]), "s"((uint32_t)(m[6] >> 32)), "s"((uint32_t)m[7]), "s"((uint32_t)(m[7] >> 32)));
  return word;
}

// The need-th largest (1 <= need <= valid count) of the wave's keys, lane l
// holding kv[i] (valid when bit i of vm is set): radix select over the keys'
// own range in at most 1024 bins per pass, in the wave's LDS (hist: 1024
// zeroed words, left zeroed, + 64 trash words); only slots i < nk (uniform)
// are looked at.  No barriers.  *gt = the keys above the result.  With
// MAXPASS < 4 the result is the lower edge of the last bin found, a value
// with at least `need` keys at or above it; otherwise a pass that leaves at
// most 64 keys in its bin is finished by ranking them against each other.
template <int NK, int MAXPASS = 4, int BINS = kPfBins>
__device__ __forceinline__ uint32_t wave_kth(const uint32_t (&kv)[NK], uint32_t vm, int nk, uint32_t need,
                                             uint32_t* hist, uint32_t* gt) {
  static_assert(BINS == 1024 || BINS == 256, "1024 or 256 bins");
  constexpr int LOGB = BINS == 1024 ? 10 : 8, BPL = BINS / 64;  // bins per lane
  const int lane = lane_tid() & 63;
  uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    if (i >= nk) break;  // uniform: only the slots in use
    const bool v = (vm >> i) & 1u;
    lo = v && kv[i] < lo ? kv[i] : lo;
    hi = v && kv[i] > hi ? kv[i] : hi;
  }
  wave_minmax(lo, hi);
  uint32_t above_all = 0;
#pragma unroll 1
  for (int pass = 0; pass < MAXPASS && lo != hi; ++pass) {
    const uint32_t span = hi - lo;
    const int nbits = 32 - __clz((int)span);
    const int shift = nbits > LOGB ? nbits - LOGB : 0;
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      if (i >= nk) break;
      const bool in = ((vm >> i) & 1u) && kv[i] >= lo && kv[i] <= hi;
      atomicAdd(in ? hist + ((kv[i] - lo) >> shift) : hist + BINS + lane, 1u);
    }
    // lane l owns bins [BINS - BPL (l + 1), BINS - BPL l): lane 0 the top ones
    const int base = BINS - BPL * (lane + 1);
    uint32_t c[BPL], tot = 0;
#pragma unroll
    for (int b = 0; b < BPL; ++b) {
      c[b] = hist[base + b];
      hist[base + b] = 0u;
      tot += c[b];
    }
    const uint32_t incl = wave_incl_add(tot), excl = incl - tot;
    uint32_t cum = excl, asel = 0, cb = 0;
    int bsel = -1;
#pragma unroll
    for (int b = BPL - 1; b >= 0; --b) {
      if (bsel < 0) {
        if (cum + c[b] >= need || b == 0) {
          bsel = b;
          asel = cum;
          cb = c[b];
        } else {
          cum += c[b];
        }
      }
    }
    const uint64_t fl = __ballot(excl < need && incl >= need);
    const int src = (int)__builtin_ctzll(fl);
    const uint32_t digit = (uint32_t)__builtin_amdgcn_readlane(base + bsel, src);
    const uint32_t above = (uint32_t)__builtin_amdgcn_readlane((int)asel, src);
    const uint32_t cnt = (uint32_t)__builtin_amdgcn_readlane((int)cb, src);
    need -= above;
    above_all += above;
    const uint32_t nlo = lo + (digit << shift);
    const uint32_t width_m1 = (uint32_t)(((uint64_t)1 << shift) - 1u);
    hi = hi - nlo > width_m1 ? nlo + width_m1 : hi;
    lo = nlo;
    if (cnt == 1u && lo != hi) {  // the one key in [lo, hi]
      uint32_t v = 0u;
#pragma unroll
      for (int i = 0; i < NK; ++i) v = (((vm >> i) & 1u) && kv[i] >= lo && kv[i] <= hi) ? kv[i] : v;
      uint32_t dummy = 0xffffffffu;
      wave_minmax(dummy, v);
      lo = hi = v;
    } else if (MAXPASS > 1 && cnt <= 64u && lo != hi) {
      // at most 64 keys left in [lo, hi]: gather them into the (zeroed) bins
      // and rank each against the others instead of another pass; the key
      // with (greater < need <= greater + equal) is the answer
      uint32_t at = 0;
      const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
      for (int i = 0; i < NK; ++i) {
        if (i >= nk) break;
        const bool in = ((vm >> i) & 1u) && kv[i] >= lo && kv[i] <= hi;
        const uint64_t m = __ballot(in);
        if (in) hist[at + (uint32_t)__popcll(m & below)] = kv[i];
        at += (uint32_t)__popcll(m);
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's stores, before its lanes read them
      const uint32_t mine = lane < (int)cnt ? hist[lane] : 0u;
      uint32_t g = 0, e = 0;
      for (uint32_t j = 0; j < cnt; ++j) {
        const uint32_t o = hist[j];
        g += o > mine ? 1u : 0u;
        e += o == mine ? 1u : 0u;
      }
      const uint64_t hit = __ballot(lane < (int)cnt && g < need && g + e >= need);
      const int src = (int)__builtin_ctzll(hit);
      const uint32_t v = (uint32_t)__builtin_amdgcn_readlane((int)mine, src);
      above_all += (uint32_t)__builtin_amdgcn_readlane((int)g, src);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // every lane's reads, before the bins are cleared
      if (lane < (int)cnt) hist[lane] = 0u;
      lo = hi = v;
    }
  }
  *gt = above_all;
  return lo;
}

// ---------------------------------------------------------------------------
// 1. thresholds from a sample of key runs
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kPfThreads) void k_pf_thresh(PfArgs a) {
  extern __shared__ __align__(16) uint32_t pf_sm[];
  uint32_t* ss = pf_sm;                                          // [kPfRowsT][ns_max]
  uint32_t* wh = pf_sm + (size_t)kPfRowsT * a.ns_max;            // [kPfRowsT][kPfWaveHist]
  const int tid = threadIdx.x, lane = tid & 63, kb = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int b = blockIdx.x / a.bps_t, t = blockIdx.x % a.bps_t;
  const int64_t row0 = a.q_off[b] + (int64_t)t * kPfRowsT, row_end = a.q_off[b + 1];
  const int nrows = (int)(row0 >= row_end ? 0 : (row_end - row0 < kPfRowsT ? row_end - row0 : kPfRowsT));
  if (nrows == 0) return;
  const int64_t pbase = a.pool_off[b], P = a.pool_off[b + 1] - pbase;
  __builtin_amdgcn_s_setprio(3);  // lowered for the radix pass (waves of a SIMD progress together)
  for (int i = tid; i < kPfRowsT * kPfWaveHist; i += kPfThreads) wh[i] = 0u;
  v8i a0;
  int s0;
  pf_load_a(a, row0, nrows, lane, a0, s0);
  // sample tile u: keys [u * span, u * span + 32) of the sequence's P (the
  // queries' own visible limits are applied per query below, so the loads do
  // not wait for the positions); at most 64 tiles (the stride is >= P / 2048)
  const int64_t st = a.stride, span = 32 * st;
  const int ntiles = (int)((P + span - 1) / span);  // ntiles * 32 <= ns_max
  // up to 16 tiles per wave in flight: the whole sample takes one round of loads
  constexpr int kTB = 16;
  for (int tb = wave; tb < ntiles; tb += kPfRowsT * kTB) {
    uint4 kc[kTB];
    int ks[kTB];
#pragma unroll
    for (int u = 0; u < kTB; ++u) {
      // 32-bit: P <= max_pool <= 2^30 (checked at the boundary), so j < 2^31
      const int j = (tb + kPfRowsT * u) * (int)span + (lane & 31);
      pf_load_b(a, pbase + j, tb + kPfRowsT * u < ntiles && j < (int)P, kb, kc[u], ks[u]);
    }
#pragma unroll
    for (int u = 0; u < kTB; ++u) {
      const int tile = tb + kPfRowsT * u;
      if (tile >= ntiles) break;
      const int i = tile * 32 + (lane & 31);
      const v16f c0 = pf_mfma(a0, s0, kc[u], ks[u]);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int q = 2 * s + (lane >> 5);
        if (q < nrows) ss[(size_t)q * a.ns_max + i] = pf_key(c0, s);
      }
    }
  }
  __syncthreads();
  __builtin_amdgcn_s_setprio(1);
  uint32_t* hist = wh + wave * kPfWaveHist;
  for (int q = wave; q < nrows; q += kPfRowsT) {
    const int64_t row = row0 + q;
    const int64_t nvis = pf_nvis(a.q_pos[row], a.m, P);
    const int64_t k_eff = nvis < a.k ? nvis : a.k;
    // samples of keys < nvis: the runs below nvis / span whole, then the first
    // min(32, nvis % span) of the next, so slots [0, nsq)
    const int64_t rem = nvis % span;
    const int nsq = (int)(nvis / span * 32 + (rem < 32 ? rem : 32));
    const int64_t need_s = (2 * k_eff + st - 1) / st;
    uint32_t tau = 0u;
    if (k_eff < nvis && need_s >= 1 && need_s <= nsq) {
      uint32_t kv[kPfSampleMax / 64];
      uint32_t vm = 0;
#pragma unroll
      for (int e = 0; e < kPfSampleMax / 64; ++e) {
        const int c = e * 64 + lane;
        const bool v = c < nsq;
        kv[e] = v ? ss[(size_t)q * a.ns_max + c] : 0u;
        vm |= v ? (1u << e) : 0u;
      }
      // One radix pass over the range of the sample's nonzero scores (a score
      // is 0 when every head's dot product is <= 0): the lower edge of the
      // sample bin holding the need_s-th largest, so at least need_s samples
      // are >= it (the exact order statistic is not needed).  With 1024 bins
      // over that range a bin spans a few percent of a score, so the bin
      // edge adds few candidates.  When fewer than need_s samples are
      // nonzero, tau = 0 (every visible key is a candidate).
#pragma unroll
      for (int e = 0; e < kPfSampleMax / 64; ++e) vm &= kv[e] != 0u ? 0xffffffffu : ~(1u << e);
      uint32_t nz = (uint32_t)__builtin_popcount(vm);
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) nz += (uint32_t)__shfl_xor((int)nz, o);
      if (nz >= (uint32_t)need_s) {
        uint32_t gt;
        tau = wave_kth<kPfSampleMax / 64, 1>(kv, vm, (nsq + 63) >> 6, (uint32_t)need_s, hist, &gt);
      }
    }
    if (lane == 0) a.tau[row] = tau;
  }
}

// ---------------------------------------------------------------------------
// 2. every visible score once -> candidate bitmap
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_pf_score(PfArgs a) {
  const int tid = threadIdx.x, lane = tid & 63, kb = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int b = blockIdx.y / a.bps, t = blockIdx.y % a.bps;
  const int64_t row0 = a.q_off[b] + (int64_t)t * kPfRows, row_end = a.q_off[b + 1];
  const int nrows = (int)(row0 >= row_end ? 0 : (row_end - row0 < kPfRows ? row_end - row0 : kPfRows));
  if (nrows == 0) return;
  const int64_t pbase = a.pool_off[b], P = a.pool_off[b + 1] - pbase;
  const int64_t jr0 = (int64_t)blockIdx.x * a.kw;
  // this lane's 16 queries: slot 8u + 2s + lane/32 of A operand u, score index s
  constexpr int kE = kPfRows / 2;
  int tq[kE];  // thresholds by pf_tau_signed
  int nq[kE];
  int nmax = 0, nmin = 0x7fffffff;
#pragma unroll
  for (int e = 0; e < kE; ++e) {
    const int q = 8 * (e >> 2) + 2 * (e & 3) + (lane >> 5);
    const bool v = q < nrows;
    tq[e] = pf_tau_signed(v ? a.tau[row0 + q] : 0xffffffffu);
    nq[e] = v ? (int)pf_nvis(a.q_pos[row0 + q], a.m, P) : 0;
    nmax = nq[e] > nmax ? nq[e] : nmax;
    nmin = v && nq[e] < nmin ? nq[e] : nmin;
  }
  {  // over the wave (lanes 0-31 and 32-63 hold different queries)
    uint32_t mn = (uint32_t)nmin, mx = (uint32_t)nmax;
    wave_minmax(mn, mx);
    nmin = (int)mn;
    nmax = (int)mx;
  }
  const int64_t nvis_max = nmax;
  if (jr0 >= nvis_max) return;
  v8i av[kPfRows / 8];
  int asc[kPfRows / 8];
#pragma unroll
  for (int u = 0; u < kPfRows / 8; ++u) pf_load_a(a, row0 + 8 * u, nrows - 8 * u, lane, av[u], asc[u]);
  // word lane L < kPfRows holds the bits of query L (= 8u + 2s + h for ballot (u, s), half h)
  uint32_t* bm_row = a.bitmap + (size_t)(row0 + ((lane & 31) < nrows ? (lane & 31) : 0)) * a.bw;
  const int kT = a.kw / 32 / 4;  // tiles per wave
  constexpr int kB = 8;          // tiles per wave in flight
#pragma unroll 1
  for (int ub = 0; ub < kT; ub += kB) {
    {  // a wave further along issues after those behind it (waves of a SIMD
       // otherwise issue oldest first, and the youngest one finishes alone)
      const int pb = ub / kB;
      if (pb == 0) __builtin_amdgcn_s_setprio(3);
      else if (pb == 1) __builtin_amdgcn_s_setprio(2);
      else if (pb == 2) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
    }
    uint4 kc[kB];
    int ks[kB];
    // a batch whose tiles every query sees whole: straight-line code (no
    // branch between its tiles, so the compiler schedules across them and
    // each tile waits only for its own loads), its 16 words per tile stored
    // after the batch
    const int64_t jlast = jr0 + (int64_t)(wave + 4 * (ub + kB - 1)) * 32;
    if (ub + kB <= kT && jlast + 32 <= (int64_t)nmin) {  // uniform per wave
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        const int64_t j = jr0 + (int64_t)(wave + 4 * (ub + u)) * 32 + (lane & 31);
        kc[u] = *reinterpret_cast<const uint4*>(a.k_codes + (pbase + j) * 32 + kb * 16);
        ks[u] = a.k_scales[(pbase + j) * 2 + kb];
      }
      uint32_t words[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        const int j = (int)(jr0 + (int64_t)(wave + 4 * (ub + u)) * 32) + (lane & 31);
        words[u] = pf_tile_word<true>(av, asc, kc[u], ks[u], j, nq, tq);
      }
      if (lane < nrows && lane < kPfRows) {
#pragma unroll
        for (int u = 0; u < kB; ++u) bm_row[(jr0 >> 5) + wave + 4 * (ub + u)] = words[u];
      }
      continue;
    }
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const int64_t j = jr0 + (int64_t)(wave + 4 * (ub + u)) * 32 + (lane & 31);
      pf_load_b(a, pbase + j, ub + u < kT && j < nvis_max, kb, kc[u], ks[u]);
    }
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const int64_t jt = jr0 + (int64_t)(wave + 4 * (ub + u)) * 32;
      if (ub + u >= kT || jt >= nvis_max) break;
      const int j = (int)jt + (lane & 31);
      const bool whole = jt + 32 <= (int64_t)nmin;  // every query sees the whole tile
      static_assert(kPfRows == 16, "two MFMA A operands");
      const uint32_t word = whole ? pf_tile_word<true>(av, asc, kc[u], ks[u], j, nq, tq)
                                  : pf_tile_word<false>(av, asc, kc[u], ks[u], j, nq, tq);
      if (lane < nrows && lane < kPfRows) bm_row[jt >> 5] = word;
    }
  }
}

// ---------------------------------------------------------------------------
// 3. per query: exact top-k among the candidates (or over all keys)
// ---------------------------------------------------------------------------
// exact radix select over all visible keys of one query, scored again on
// every pass, then the selection in ascending index order
__device__ void pf_select_all(const PfArgs& a, int64_t row, int64_t pbase, int64_t nvis, uint32_t k_eff,
                              uint32_t* hist, int32_t* idx) {
  const int lane = lane_tid() & 63, kb = lane >> 5;
  v8i av;
  int asc;
  pf_load_a(a, row, 1, lane, av, asc);
  const int64_t ntiles = (nvis + 31) >> 5;
  uint32_t prefix = 0, pmask = 0, need = k_eff;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int64_t tt = 0; tt < ntiles; ++tt) {
      const int64_t j = tt * 32 + (lane & 31);
      uint4 kc;
      int ks;
      pf_load_b(a, pbase + j, j < nvis, kb, kc, ks);
      const uint32_t key = pf_key(pf_mfma(av, asc, kc, ks), 0);
      const bool in = lane < 32 && j < nvis && (key & pmask) == prefix;
      atomicAdd(in ? hist + ((key >> shift) & 255u) : hist + kSelBins + lane, 1u);
    }
    // 256 bins: lane l owns bins [252 - 4 l, 256 - 4 l)
    const int base = 252 - 4 * lane;
    uint32_t c[4], tot = 0;
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
      c[bb] = hist[base + bb];
      hist[base + bb] = 0u;
      tot += c[bb];
    }
    const uint32_t incl = wave_incl_add(tot), excl = incl - tot;
    uint32_t cum = excl, asel = 0;
    int bsel = -1;
#pragma unroll
    for (int bb = 3; bb >= 0; --bb) {
      if (bsel < 0) {
        if (cum + c[bb] >= need || bb == 0) {
          bsel = bb;
          asel = cum;
        } else {
          cum += c[bb];
        }
      }
    }
    const uint64_t fl = __ballot(excl < need && incl >= need);
    const int src = (int)__builtin_ctzll(fl);
    const uint32_t digit = (uint32_t)__builtin_amdgcn_readlane(base + bsel, src);
    need -= (uint32_t)__builtin_amdgcn_readlane((int)asel, src);
    prefix |= digit << shift;
    pmask |= 255u << shift;
  }
  // prefix = K*; take every key above it and the first `need` keys equal to it
  uint32_t n_sel = 0, n_tie = 0;
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  for (int64_t tt = 0; tt < ntiles; ++tt) {
    const int64_t j = tt * 32 + (lane & 31);
    uint4 kc;
    int ks;
    pf_load_b(a, pbase + j, j < nvis, kb, kc, ks);
    const uint32_t key = pf_key(pf_mfma(av, asc, kc, ks), 0);
    const bool ok = lane < 32 && j < nvis;
    const bool eq = ok && key == prefix;
    const uint64_t me = __ballot(eq);
    const uint32_t tie_rank = n_tie + (uint32_t)__popcll(me & below);
    const bool sel = ok && (key > prefix || (eq && tie_rank < need));
    const uint64_t ms = __ballot(sel);
    if (sel) idx[n_sel + (uint32_t)__popcll(ms & below)] = (int32_t)j;
    n_sel += (uint32_t)__popcll(ms);
    n_tie += (uint32_t)__popcll(me);
  }
}

__global__ __launch_bounds__(128) void k_pf_select(PfArgs a) {
  extern __shared__ __align__(16) uint32_t pf_sm[];
  const int tid = threadIdx.x, lane = tid & 63, kb = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  uint32_t* cand_j = pf_sm + (size_t)wave * (kPfCand + kSelWaveHist);
  uint32_t* hist = cand_j + kPfCand;
  for (int i = lane; i < kSelWaveHist; i += 64) hist[i] = 0u;
  const int64_t row = (int64_t)blockIdx.x * 2 + wave;
  if (row >= a.n_q) return;  // wave-level work only: no block barriers below
  const int b = seq_of_row(a.q_off, a.n_seq, row);
  const int64_t pbase = a.pool_off[b], P = a.pool_off[b + 1] - pbase;
  const int64_t nvis = pf_nvis(a.q_pos[row], a.m, P);
  const uint32_t k_eff = (uint32_t)(nvis < a.k ? nvis : a.k);
  int32_t* idx = a.idx + row * a.k;
  for (int i = (int)k_eff + lane; i < a.k; i += 64) idx[i] = -1;
  if (k_eff == 0) {
    if (lane == 0) a.tau[row] = 0u;
    return;
  }
  // candidates: the bitmap's set bits.  Word g * 64 + l goes to lane l (words
  // of a group of 64 are adjacent, so a run of dense words spreads over the
  // lanes and a group's extraction takes as many steps as its densest word
  // has bits); groups read 16 at a time (all loads of a batch in flight)
  const uint32_t* bm = a.bitmap + (size_t)row * a.bw;
  uint32_t* bmw = a.bitmap + (size_t)row * a.bw;
  const int nw = (int)((nvis + 31) >> 5), ng = (nw + 63) >> 6;
  constexpr int kWB = 16;
  uint32_t wv[kWB];
  uint32_t cnt = 0;
  for (int g0 = 0; g0 < ng; g0 += kWB) {
#pragma unroll
    for (int i = 0; i < kWB; ++i) {
      const int w = (g0 + i) * 64 + lane;
      wv[i] = (g0 + i < ng && w < nw) ? bm[w] : 0u;
    }
#pragma unroll
    for (int i = 0; i < kWB; ++i) cnt += (uint32_t)__popc(wv[i]);
  }
  // issue priority falls as a wave's phases complete (count, re-score, K*),
  // so the waves of a SIMD progress together rather than oldest first
  __builtin_amdgcn_s_setprio(3);
  const uint32_t n_c = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_add(cnt), 63);
  // the workspace is left zero-filled: this query's threshold and bitmap words
  if (lane == 0) a.tau[row] = 0u;
  if (n_c < k_eff || n_c > (uint32_t)kPfCand) {
    for (int w = lane; w < nw; w += 64) bmw[w] = 0u;
    pf_select_all(a, row, pbase, nvis, k_eff, hist, idx);
    return;
  }
  uint32_t run = 0;  // candidates of the groups before
  for (int g0 = 0; g0 < ng; g0 += kWB) {
    if (ng > kWB) {  // more than one batch: read this one again
#pragma unroll
      for (int i = 0; i < kWB; ++i) {
        const int w = (g0 + i) * 64 + lane;
        wv[i] = (g0 + i < ng && w < nw) ? bm[w] : 0u;
      }
    }
#pragma unroll
    for (int i = 0; i < kWB; ++i) {
      if (g0 + i >= ng) break;  // uniform
      const int w = (g0 + i) * 64 + lane;
      if (w < nw) bmw[w] = 0u;
      const uint32_t c = (uint32_t)__popc(wv[i]);
      const uint32_t incl = wave_incl_add(c);
      uint32_t pos = run + incl - c;
      run += (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
      uint32_t bits = wv[i];
      while (bits) {
        const int bpos = __ffs(bits) - 1;
        bits &= bits - 1u;
        cand_j[pos++] = (uint32_t)(w * 32 + bpos);
      }
    }
  }
  __builtin_amdgcn_s_setprio(2);
  // the candidates' scores again: query slot 0 of the MFMA, 32 candidates per tile;
  // tiles 2e and 2e + 1 fill register slot e (lanes 0-31 and 32-63)
  v8i av;
  int asc;
  pf_load_a(a, row, 1, lane, av, asc);
  constexpr int NK = kPfCand / 64;
  uint32_t kv[NK];
  uint32_t vm = 0;
  const int nk = (int)((n_c + 63) >> 6);
#pragma unroll
  for (int e0 = 0; e0 < NK; e0 += 4) {  // 8 tiles (4 register slots) in flight
    if (e0 >= nk) break;
    uint4 kc[8];
    int ks[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t c = (uint32_t)(2 * e0 + u) * 32u + (uint32_t)(lane & 31);
      const bool ok = c < n_c;
      pf_load_b(a, pbase + (ok ? (int64_t)cand_j[c] : 0), ok, kb, kc[u], ks[u]);
    }
#pragma unroll
    for (int u = 0; u < 8; u += 2) {
      const uint32_t k_even = pf_key(pf_mfma(av, asc, kc[u], ks[u]), 0);
      const uint32_t k_odd = pf_key(pf_mfma(av, asc, kc[u + 1], ks[u + 1]), 0);
      // lanes 0-31 of k_odd -> lanes 32-63 of the slot
      const uint32_t hi_half = (uint32_t)__shfl_xor((int)k_odd, 32);
      const int e = e0 + u / 2;
      kv[e] = lane < 32 ? k_even : hi_half;
      const bool v = (uint32_t)(e * 64 + lane) < n_c;
      vm |= v ? (1u << e) : 0u;
    }
  }
  uint32_t gt;
  __builtin_amdgcn_s_setprio(1);
  const uint32_t kstar = wave_kth<NK, 4, kSelBins>(kv, vm, nk, k_eff, hist, &gt);
  __builtin_amdgcn_s_setprio(0);
  const uint32_t r_eq = k_eff - gt;
  // candidates are in ascending index order: a selected one goes to the count of
  // selected ones before it
  uint32_t n_sel = 0, n_tie = 0;
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int e = 0; e < NK; ++e) {
    if (e >= nk) break;
    const bool v = (vm >> e) & 1u;
    const bool eq = v && kv[e] == kstar;
    const uint64_t me = __ballot(eq);
    const uint32_t tie_rank = n_tie + (uint32_t)__popcll(me & below);
    const bool sel = v && (kv[e] > kstar || (eq && tie_rank < r_eq));
    const uint64_t ms = __ballot(sel);
    if (sel) idx[n_sel + (uint32_t)__popcll(ms & below)] = (int32_t)cand_j[e * 64 + lane];
    n_sel += (uint32_t)__popcll(ms);
    n_tie += (uint32_t)__popcll(me);
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
int prefill_path(int64_t max_q_per_seq) { return max_q_per_seq >= kPfMinQ ? 1 : 0; }

// keys per scoring workgroup: the grid (key blocks x query blocks) is sized to
// a whole number of rounds of resident workgroups, so no last round runs the
// chip partly empty
static std::atomic<int> g_pf_capacity[64];  // resident scoring workgroups per device (0 = not known yet)

static int pf_keys_per_wg(int64_t max_pool, int64_t qblocks) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  int capacity = dev < 64 ? g_pf_capacity[dev].load(std::memory_order_relaxed) : 0;
  if (capacity == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)k_pf_score, 256, 0) == hipSuccess &&
        cus > 0 && per_cu > 0)
      capacity = cus * per_cu;
    else
      capacity = 1024;
    if (dev < 64) g_pf_capacity[dev].store(capacity, std::memory_order_relaxed);
  }
  const int64_t quads = (max_pool + 127) / 128;  // 128-key units
  if (quads <= 0 || qblocks <= 0) return kPfKeysWG;
  // fewest key blocks that reach a whole round, then as many rounds as keep >= kPfKeysWG keys per block
  int64_t rounds = 1;
  for (;;) {
    const int64_t nx = (rounds * capacity + qblocks - 1) / qblocks;
    const int64_t per = (quads + nx - 1) / nx;
    if (per * 128 < kPfKeysWG || nx >= quads) break;
    const int64_t nx2 = ((rounds + 1) * capacity + qblocks - 1) / qblocks;
    const int64_t per2 = (quads + nx2 - 1) / nx2;
    if (per2 * 128 < kPfKeysWG) break;
    ++rounds;
  }
  const int64_t nx = (rounds * capacity + qblocks - 1) / qblocks;
  int64_t per = (quads + nx - 1) / nx;
  if (per < 1) per = 1;
  return (int)(per * 128);
}

static int pf_stride(int64_t max_pool) {
  int64_t s = (max_pool + kPfSampleMax - 1) / kPfSampleMax;
  return (int)(s < 16 ? 16 : s);
}

size_t prefill_ws_bytes(int64_t n_q, int64_t max_pool) {
  const size_t bw = (size_t)((max_pool + 31) / 32);
  return (((size_t)n_q * 4 + 255) & ~(size_t)255) + (size_t)n_q * (bw ? bw : 1) * 4;
}

int launch_prefill_topk(int n_seq, int64_t n_q, int64_t max_q_per_seq, const int64_t* q_off,
                        const int64_t* q_pos, const int64_t* pool_off, int64_t max_pool, int m, int k,
                        const uint8_t* q_codes, const uint8_t* q_scales, const float* w,
                        const uint8_t* k_codes, const uint8_t* k_scales, int32_t* idx, void* ws,
                        hipStream_t stream) {
  if (n_q == 0) return 0;
  PfArgs a{};
  a.q_off = q_off; a.q_pos = q_pos; a.pool_off = pool_off;
  a.n_seq = n_seq;
  a.bps = (int)((max_q_per_seq + kPfRows - 1) / kPfRows);
  a.bps_t = (int)((max_q_per_seq + kPfRowsT - 1) / kPfRowsT);
  a.m = m; a.k = k;
  a.stride = pf_stride(max_pool);
  // sample slots: 32 per run of the longest sequence (<= kPfSampleMax, since
  // stride >= max_pool / kPfSampleMax)
  a.ns_max = (int)((max_pool + 32 * (int64_t)a.stride - 1) / (32 * (int64_t)a.stride)) * 32;
  if (a.ns_max < 32) a.ns_max = 32;
  a.bw = (int)((max_pool + 31) / 32);
  a.n_q = n_q; a.max_pool = max_pool;
  a.q_codes = q_codes; a.q_scales = q_scales; a.w = w; a.k_codes = k_codes; a.k_scales = k_scales;
  uint8_t* p = (uint8_t*)ws;
  a.tau = (uint32_t*)p;
  a.bitmap = (uint32_t*)(p + (((size_t)n_q * 4 + 255) & ~(size_t)255));
  a.idx = idx;
  const size_t lds1 = ((size_t)kPfRowsT * a.ns_max + kPfRowsT * kPfWaveHist) * 4;
  const size_t lds3 = (size_t)2 * (kPfCand + kSelWaveHist) * 4;
  static_assert((size_t)2 * (kPfCand + kSelWaveHist) * 4 * 8 <= 160 * 1024, "8 selection workgroups per CU");
  // the threshold kernel's LDS can exceed the default dynamic limit (idempotent,
  // so concurrent first calls need no ordering)
  (void)hipFuncSetAttribute((const void*)k_pf_thresh, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)(((size_t)kPfRowsT * kPfSampleMax + kPfRowsT * kPfWaveHist) * 4));
  static_assert(((size_t)kPfRowsT * kPfSampleMax + kPfRowsT * kPfWaveHist) * 4 <= 160 * 1024,
                "the threshold block's samples and histograms fit a CU's LDS");
  const unsigned nblk = (unsigned)(n_seq * a.bps);
  hipError_t e = launch(7, kProfBoth, k_pf_thresh, dim3((unsigned)(n_seq * a.bps_t)), dim3(kPfThreads), lds1, stream, a);
  a.kw = pf_keys_per_wg(max_pool, (int64_t)nblk);
  dim3 g2((unsigned)((max_pool + a.kw - 1) / a.kw), nblk);
  if (g2.x == 0) g2.x = 1;
  if (e == hipSuccess) e = launch(0, kProfBoth, k_pf_score, g2, dim3(256), 0, stream, a);
  if (e == hipSuccess) e = launch(8, kProfBoth, k_pf_select, dim3((unsigned)((n_q + 1) / 2)), dim3(128), lds3, stream, a);
  return e == hipSuccess && hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace csa

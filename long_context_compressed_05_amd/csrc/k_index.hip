// Lightning-indexer scoring and exact per-query top-k.
//
// Pages: jyp-garden EP 95 notes, IDEAS (KV compressed to 1/4, the Lightning
// Indexer keeps only the top-k); sigco.tistory.com CSA/HCA section (the
// indexer looks for the blocks most relevant to the current token and only
// the top candidates are attended); pytorch.kr FP4 QAT section (the indexer
// QK path is MXFP4).  Score (reading taken):
//     S(i, j) = sum_h w[i][h] * max(0, qhat[i][h] . khat[j])
// with MXFP4 operands, ties broken toward the lower j.
//
// Scoring runs on the gfx950 block-scaled MFMA (32x32x64, FP4 x FP4, one
// E8M0 scale per lane per 32-element K block).  The A operand holds up to 8
// queries x 4 heads (32 rows), the B operand 32 keys; the power-of-two head
// weight is folded into the query block scale, so the MFMA output already
// carries w_h.  Every product and partial sum is a small dyadic rational, so
// the fp32 accumulation is exact and the score bit pattern is an exact sort
// key (ReLU is an integer max on the bit pattern, which also maps -0 to +0).
//
// This is the path for decode batches (few queries per sequence); batches with
// many queries per sequence take the prefill path (k_prefill.hip), which keeps
// no score matrix.  Selection is a radix select on those 32-bit keys:
//   1. k_idx_score: keys to the workspace + a 4096-bin histogram of the top
//      13 key bits per query (LDS, merged into one of `nrep` global replicas
//      picked by workgroup id, i.e. per XCD, to spread the atomics); the last
//      workgroup of a query tile finds the threshold bin b1;
//   2. k_idx_select: entries above b1 are selected outright, entries in b1
//      become candidates;
//   3. k_idx_final: exact k-th key K* among the candidates, then the lowest
//      indices among entries equal to K*, then the ascending index order
//      (an LDS bitmap of the visible range, or a bitonic sort when the range
//      is too large for LDS).  It also returns the workspace to all-zero.
// Batches whose sequences have at most kSmallPool pooled entries take one
// launch instead (k_idx_small, below).
#include "common.hpp"
#include "kernels.hpp"
#include "select_core.hpp"

namespace csa {

constexpr int kNBins = 4096;  // key >> 19: 8 exponent + 4 mantissa bits (sign is 0)
constexpr int kBinShift = 19;
constexpr int kScoreIter = 8;                       // 32-key MFMA groups per wave
constexpr int kScoreChunk = 4 * 32 * kScoreIter;    // keys per score workgroup
constexpr int kSelChunk = 4096;                     // keys per select workgroup
constexpr int kSelPerThread = kSelChunk / 256;
constexpr uint32_t kNoBin = 0xffffffffu;
constexpr int kBitmapMaxBytes = 64 * 1024;         // LDS bitmap of the visible range
constexpr int kCandLds = 4096;                     // candidates staged in LDS (else read from L2)

__device__ __forceinline__ int64_t n_visible(int64_t t, int m, int64_t P) {
  int64_t v = (t + 1) / m;
  return v < P ? v : P;
}

// Threshold bin of one query over `nrep` histogram replicas: the bin b1 with
// count(bin > b1) < need <= count(bin >= b1).  Whole 256-thread block.
__device__ void find_threshold(const uint32_t* hist, int nrep, uint32_t need, uint32_t* info_out) {
  __shared__ uint32_t scratch[8];
  const int t = threadIdx.x;
  uint32_t loc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) loc[i] = 0;
  for (int r = 0; r < nrep; ++r) {
#pragma unroll
    for (int i = 0; i < 16; ++i) loc[i] += hist[r * kNBins + t * 16 + i];
  }
  uint32_t c = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) c += loc[i];
  int tstar;
  uint32_t above;
  block_find_from_top(c, need, scratch, &tstar, &above);
  if (t == tstar) {
    uint32_t cum = above;
    int bi = 15;
    for (; bi > 0; --bi) {
      if (cum + loc[bi] >= need) break;
      cum += loc[bi];
    }
    info_out[0] = (uint32_t)(t * 16 + bi);
    info_out[1] = cum;
  }
  __syncthreads();
}

struct ScoreArgs {
  const int64_t* q_off;
  const int64_t* q_pos;
  const int64_t* pool_off;
  int n_seq, tiles_per_seq, qt, m, nrep;
  int64_t max_pool;
  const uint8_t* q_codes;
  const uint8_t* q_scales;
  const float* w;
  const uint8_t* k_codes;
  const uint8_t* k_scales;
  uint32_t* keys;
  uint32_t* hist;
};

__global__ __launch_bounds__(256) void k_idx_score(ScoreArgs a) {
  extern __shared__ uint32_t lhist[];  // qt * kNBins/2 words, two 16-bit counters per word
  __shared__ int64_t nvis_s[8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tile = blockIdx.y;
  const int b = tile / a.tiles_per_seq;
  const int64_t row0 = a.q_off[b] + (int64_t)(tile % a.tiles_per_seq) * a.qt;
  const int64_t row_end_seq = a.q_off[b + 1];
  const int nrows = (int)(row0 >= row_end_seq ? 0 : (row_end_seq - row0 < a.qt ? row_end_seq - row0 : a.qt));
  if (nrows == 0) return;  // an empty tile: no query waits on it
  const int64_t pbase = a.pool_off[b];
  const int64_t P = a.pool_off[b + 1] - pbase;
  if (tid < 8) nvis_s[tid] = tid < nrows ? n_visible(a.q_pos[row0 + tid], a.m, P) : 0;
  for (int i = tid; i < a.qt * (kNBins / 2); i += 256) lhist[i] = 0;
  __syncthreads();
  int64_t nvis_max = 0;
  for (int r = 0; r < nrows; ++r) nvis_max = nvis_s[r] > nvis_max ? nvis_s[r] : nvis_max;

  // A operand: row (lane%32) = query slot * 4 + head, K block lane/32
  const int slot_a = (lane & 31) >> 2, head_a = lane & 3, kb = lane >> 5;
  v8i av = {0, 0, 0, 0, 0, 0, 0, 0};
  int asc = 127;
  if (slot_a < nrows) {
    const int64_t qrow = (row0 + slot_a) * 4 + head_a;
    uint4 u = *reinterpret_cast<const uint4*>(a.q_codes + qrow * 32 + kb * 16);
    asc = fold_head_weight(u, (int)a.q_scales[qrow * 2 + kb], a.w[qrow]);  // w_h folded into the block scale
    av[0] = (int)u.x; av[1] = (int)u.y; av[2] = (int)u.z; av[3] = (int)u.w;
  }

  const int64_t jc0 = (int64_t)blockIdx.x * kScoreChunk;
  if (jc0 < nvis_max) {
    // issue all key loads of this wave first, then the MFMAs
    uint4 kcv[kScoreIter];
    int ksv[kScoreIter];
#pragma unroll
    for (int it = 0; it < kScoreIter; ++it) {
      const int64_t j = jc0 + (int64_t)(wave * kScoreIter + it) * 32 + (lane & 31);
      kcv[it] = make_uint4(0, 0, 0, 0);
      ksv[it] = 127;
      if (j < nvis_max) {
        kcv[it] = *reinterpret_cast<const uint4*>(a.k_codes + (pbase + j) * 32 + kb * 16);
        ksv[it] = a.k_scales[(pbase + j) * 2 + kb];
      }
    }
#pragma unroll
    for (int it = 0; it < kScoreIter; ++it) {
      const int64_t jbase = jc0 + (int64_t)(wave * kScoreIter + it) * 32;
      if (jbase >= nvis_max) break;
      v8i bv = {(int)kcv[it].x, (int)kcv[it].y, (int)kcv[it].z, (int)kcv[it].w, 0, 0, 0, 0};
      v16f acc = {};
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 4, 4, 0, asc, 0, ksv[it]);
      const int64_t j = jbase + (lane & 31);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int slot = 2 * s + (lane >> 5);
        if (slot < nrows && j < nvis_s[slot]) {
          float r0 = __int_as_float(max(__float_as_int(acc[4 * s + 0]), 0));
          float r1 = __int_as_float(max(__float_as_int(acc[4 * s + 1]), 0));
          float r2 = __int_as_float(max(__float_as_int(acc[4 * s + 2]), 0));
          float r3 = __int_as_float(max(__float_as_int(acc[4 * s + 3]), 0));
          const uint32_t key = __float_as_uint((r0 + r1) + (r2 + r3));
          a.keys[(row0 + slot) * a.max_pool + j] = key;
          const uint32_t bin = key >> kBinShift;
          atomicAdd(&lhist[slot * (kNBins / 2) + (bin >> 1)], 1u << ((bin & 1u) * 16));
        }
      }
    }
  }
  __syncthreads();
  const int rep = (int)((blockIdx.x + (int64_t)gridDim.x * blockIdx.y) % a.nrep);
  for (int r = 0; r < nrows; ++r) {
    uint32_t* gh = a.hist + ((row0 + r) * a.nrep + rep) * kNBins;
    for (int wi = tid; wi < kNBins / 2; wi += 256) {
      const uint32_t v = lhist[r * (kNBins / 2) + wi];
      if (v & 0xffffu) atomicAdd(gh + 2 * wi, v & 0xffffu);
      if (v >> 16) atomicAdd(gh + 2 * wi + 1, v >> 16);
    }
  }
}

// The same scores from bf16 indexer vectors (the higher-precision indexer
// the FP4 path is compared with; same definition, S = sum_h w_h * max(0,
// q_h . k), with bf16 operands and fp32 accumulation): v_mfma_f32_32x32x16_bf16,
// A = up to 8 queries x 4 heads (lane & 31 = slot * 4 + head), B = 32 keys,
// K = 64 in four steps of 16; the output layout is the FP4 kernel's, so the
// epilogue, the keys and the histogram are the same and the selection kernels
// that follow are shared.  The head weights multiply the ReLU'd dots in fp32.
struct ScoreArgsBf16 {
  const int64_t* q_off;
  const int64_t* q_pos;
  const int64_t* pool_off;
  int n_seq, tiles_per_seq, qt, m, nrep;
  int64_t max_pool;
  const uint16_t* q;  // [n_q][4][64]
  const float* w;     // [n_q][4]
  const uint16_t* k;  // [sum P][64]
  uint32_t* keys;
  uint32_t* hist;
};

__global__ __launch_bounds__(256) void k_idx_score_bf16(ScoreArgsBf16 a) {
  extern __shared__ uint32_t lhist[];  // qt * kNBins/2 words, two 16-bit counters per word
  __shared__ int64_t nvis_s[8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tile = blockIdx.y;
  const int b = tile / a.tiles_per_seq;
  const int64_t row0 = a.q_off[b] + (int64_t)(tile % a.tiles_per_seq) * a.qt;
  const int64_t row_end_seq = a.q_off[b + 1];
  const int nrows = (int)(row0 >= row_end_seq ? 0 : (row_end_seq - row0 < a.qt ? row_end_seq - row0 : a.qt));
  if (nrows == 0) return;
  const int64_t pbase = a.pool_off[b];
  const int64_t P = a.pool_off[b + 1] - pbase;
  if (tid < 8) nvis_s[tid] = tid < nrows ? n_visible(a.q_pos[row0 + tid], a.m, P) : 0;
  for (int i = tid; i < a.qt * (kNBins / 2); i += 256) lhist[i] = 0;
  __syncthreads();
  int64_t nvis_max = 0;
  for (int r = 0; r < nrows; ++r) nvis_max = nvis_s[r] > nvis_max ? nvis_s[r] : nvis_max;
  // A operand, k-step s: row (lane & 31) = slot * 4 + head, dims 16 s + 8 (lane >> 5) .. + 8
  const int slot_a = (lane & 31) >> 2, head_a = lane & 3, half = lane >> 5;
  v8bf av[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    av[st] = v8bf{};
    if (slot_a < nrows)
      av[st] = *reinterpret_cast<const v8bf*>(a.q + ((row0 + slot_a) * 4 + head_a) * 64 + 16 * st + 8 * half);
  }
  // this lane's output rows: slot 2 s + half, head h -> weight
  float wq[4][4];
#pragma unroll
  for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int slot = 2 * s2 + half;
      wq[s2][h] = slot < nrows ? a.w[(row0 + slot) * 4 + h] : 0.f;
    }
  const int64_t jc0 = (int64_t)blockIdx.x * kScoreChunk;
  if (jc0 < nvis_max) {
#pragma unroll 1
    for (int it0 = 0; it0 < kScoreIter; it0 += 4) {  // 4 key tiles (16 KB per wave) in flight
      v8bf kv[4][4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t j = jc0 + (int64_t)(wave * kScoreIter + it0 + u) * 32 + (lane & 31);
#pragma unroll
        for (int st = 0; st < 4; ++st)
          kv[u][st] = j < nvis_max ? *reinterpret_cast<const v8bf*>(a.k + (pbase + j) * 64 + 16 * st + 8 * half)
                                   : v8bf{};
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t jbase = jc0 + (int64_t)(wave * kScoreIter + it0 + u) * 32;
        if (jbase >= nvis_max) break;
        v16f acc = {};
#pragma unroll
        for (int st = 0; st < 4; ++st) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[st], kv[u][st], acc, 0, 0, 0);
        const int64_t j = jbase + (lane & 31);
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
          const int slot = 2 * s2 + half;
          if (slot < nrows && j < nvis_s[slot]) {
            const float r0 = wq[s2][0] * __int_as_float(max(__float_as_int(acc[4 * s2 + 0]), 0));
            const float r1 = wq[s2][1] * __int_as_float(max(__float_as_int(acc[4 * s2 + 1]), 0));
            const float r2 = wq[s2][2] * __int_as_float(max(__float_as_int(acc[4 * s2 + 2]), 0));
            const float r3 = wq[s2][3] * __int_as_float(max(__float_as_int(acc[4 * s2 + 3]), 0));
            const uint32_t key = __float_as_uint((r0 + r1) + (r2 + r3));
            a.keys[(row0 + slot) * a.max_pool + j] = key;
            const uint32_t bin = key >> kBinShift;
            atomicAdd(&lhist[slot * (kNBins / 2) + (bin >> 1)], 1u << ((bin & 1u) * 16));
          }
        }
      }
    }
  }
  __syncthreads();
  const int rep = (int)((blockIdx.x + (int64_t)gridDim.x * blockIdx.y) % a.nrep);
  for (int r = 0; r < nrows; ++r) {
    uint32_t* gh = a.hist + ((row0 + r) * a.nrep + rep) * kNBins;
    for (int wi = tid; wi < kNBins / 2; wi += 256) {
      const uint32_t v = lhist[r * (kNBins / 2) + wi];
      if (v & 0xffffu) atomicAdd(gh + 2 * wi, v & 0xffffu);
      if (v >> 16) atomicAdd(gh + 2 * wi + 1, v >> 16);
    }
  }
}

// threshold bin of every query (one workgroup per query); runs after the
// scoring kernel so its histogram merges are complete and visible
__global__ __launch_bounds__(256) void k_idx_threshold(const int64_t* q_off, const int64_t* q_pos,
                                                       const int64_t* pool_off, int n_seq, int m, int k,
                                                       int nrep, const uint32_t* hist, uint32_t* info) {
  const int64_t row = blockIdx.x;
  const int b = seq_of_row(q_off, n_seq, row);
  const int64_t P = pool_off[b + 1] - pool_off[b];
  const int64_t nvis = n_visible(q_pos[row], m, P);
  const int64_t kk = nvis < k ? nvis : k;
  if (kk == 0) {
    if (threadIdx.x == 0) { info[row * 2] = kNoBin; info[row * 2 + 1] = 0; }
    return;
  }
  find_threshold(hist + row * nrep * kNBins, nrep, (uint32_t)kk, info + row * 2);
}

struct SelectArgs {
  const int64_t* q_off;
  const int64_t* q_pos;
  const int64_t* pool_off;
  int n_seq, m, k;
  int64_t max_pool;
  const uint32_t* keys;
  const uint32_t* info;
  uint32_t* counts;
  int32_t* def;
  uint2* cand;
};

__global__ __launch_bounds__(256) void k_idx_select(SelectArgs a) {
  const int64_t row = blockIdx.y;
  const uint32_t b1 = a.info[row * 2];
  if (b1 == kNoBin) return;
  const int b = seq_of_row(a.q_off, a.n_seq, row);
  const int64_t P = a.pool_off[b + 1] - a.pool_off[b];
  const int64_t nvis = n_visible(a.q_pos[row], a.m, P);
  const int64_t j0 = (int64_t)blockIdx.x * kSelChunk;
  if (j0 >= nvis) return;
  const int lane = threadIdx.x & 63;
  const uint32_t* keys = a.keys + row * a.max_pool;
  uint32_t kv[kSelPerThread];
#pragma unroll
  for (int i = 0; i < kSelPerThread; ++i) {  // all loads first
    const int64_t j = j0 + i * 256 + threadIdx.x;
    kv[i] = j < nvis ? keys[j] : 0u;
  }
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // pass 1: per-wave counts; one atomic per list per workgroup
  __shared__ uint32_t wcount[2][4], wbase[2];
  uint32_t ng = 0, ne = 0;
#pragma unroll
  for (int i = 0; i < kSelPerThread; ++i) {
    const int64_t j = j0 + i * 256 + threadIdx.x;
    const bool ok = j < nvis;
    const uint32_t bin = kv[i] >> kBinShift;
    ng += (uint32_t)__popcll(__ballot(ok && bin > b1));
    ne += (uint32_t)__popcll(__ballot(ok && bin == b1));
  }
  const int wave = threadIdx.x >> 6;
  if (lane == 0) { wcount[0][wave] = ng; wcount[1][wave] = ne; }
  __syncthreads();
  if (threadIdx.x < 2) {
    const uint32_t tot = wcount[threadIdx.x][0] + wcount[threadIdx.x][1] + wcount[threadIdx.x][2] +
                         wcount[threadIdx.x][3];
    wbase[threadIdx.x] = tot ? atomicAdd(a.counts + row * 4 + threadIdx.x, tot) : 0u;
  }
  __syncthreads();
  uint32_t pg = wbase[0], pe = wbase[1];
  for (int w = 0; w < wave; ++w) { pg += wcount[0][w]; pe += wcount[1][w]; }
  // pass 2: write in the same order
#pragma unroll
  for (int i = 0; i < kSelPerThread; ++i) {
    const int64_t j = j0 + i * 256 + threadIdx.x;
    const bool ok = j < nvis;
    const uint32_t bin = kv[i] >> kBinShift;
    const bool gt = ok && bin > b1, eq = ok && bin == b1;
    const uint64_t mg = __ballot(gt), me = __ballot(eq);
    if (gt) a.def[row * a.k + pg + __popcll(mg & below)] = (int32_t)j;
    if (eq) a.cand[row * a.max_pool + pe + __popcll(me & below)] = make_uint2(kv[i], (uint32_t)j);
    pg += (uint32_t)__popcll(mg);
    pe += (uint32_t)__popcll(me);
  }
}

struct FinalArgs {
  const int64_t* q_off;
  const int64_t* q_pos;
  const int64_t* pool_off;
  int n_seq, m, k, nrep, use_bitmap;
  int64_t max_pool;
  uint32_t* counts;
  uint32_t* hist;
  const int32_t* def;
  const uint2* cand;
  int32_t* idx;
};

__global__ __launch_bounds__(1024) void k_idx_final(FinalArgs a) {
  extern __shared__ uint32_t bitmap[];  // ceil(max_pool / 32) words when use_bitmap
  __shared__ int32_t outj[4096];
  __shared__ uint2 cand_s[kCandLds];
  __shared__ uint32_t bins[1024];
  __shared__ uint32_t scratch[32];
  __shared__ uint32_t n_out, n_eq;
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int b = seq_of_row(a.q_off, a.n_seq, row);
  const int64_t P = a.pool_off[b + 1] - a.pool_off[b];
  const int64_t nvis = n_visible(a.q_pos[row], a.m, P);
  const int k_eff = (int)(nvis < a.k ? nvis : a.k);
  int32_t* idx = a.idx + row * a.k;
  if (k_eff > 0) {
    const uint32_t n_def = a.counts[row * 4 + 0];
    const uint32_t n_c = a.counts[row * 4 + 1];
    const uint32_t need = (uint32_t)k_eff - n_def;  // >= 1 by the choice of b1
    const uint2* cand = a.cand + row * a.max_pool;
    if (n_c <= (uint32_t)kCandLds) {  // stage the candidates once
      for (uint32_t i = tid; i < n_c; i += blockDim.x) cand_s[i] = cand[i];
      __syncthreads();
      cand = cand_s;
    }
    // Every candidate lies in the threshold bin b1 (its key >> kBinShift), so
    // only the keys' low kBinShift bits are left to resolve (two rounds of
    // at most 10 bits instead of four of 8 over the whole key).
    const uint32_t fixed = cand[0].x & ~((1u << kBinShift) - 1u);
    uint32_t r;
    const uint32_t kstar = radix_select_desc_low(
        n_c, need, kBinShift, fixed, [&](uint32_t i) { return cand[i].x; }, [&](uint32_t) { return true; }, &r,
        bins, scratch);
    // r of the candidates equal to K* are taken: all of them unless ties are
    // cut, and then the r lowest indices (the largest complements ~j, whose
    // bits above the index width are all ones)
    if (tid == 0) n_eq = 0;
    __syncthreads();
    {
      uint32_t e = 0;
      for (uint32_t i = tid; i < n_c; i += blockDim.x) e += cand[i].x == kstar ? 1u : 0u;
      if (e) atomicAdd(&n_eq, e);
    }
    __syncthreads();
    uint32_t jstar = 0;  // every tie taken
    if (n_eq > r) {
      const int ibits = a.max_pool > 1 ? 64 - __clzll((unsigned long long)(a.max_pool - 1)) : 0;
      uint32_t r2;
      jstar = radix_select_desc_low(
          n_c, r, ibits, ibits >= 32 ? 0u : (~0u << ibits), [&](uint32_t i) { return ~cand[i].y; },
          [&](uint32_t i) { return cand[i].x == kstar; }, &r2, bins, scratch);
    }
    auto chosen = [&](uint2 c) { return c.x > kstar || (c.x == kstar && ~c.y >= jstar); };
    if (a.use_bitmap) {
      // ascending order from a bitmap of the visible range
      const int nwords = (int)((nvis + 31) >> 5);
      for (int i = tid; i < nwords; i += blockDim.x) bitmap[i] = 0;
      __syncthreads();
      for (uint32_t i = tid; i < n_def; i += blockDim.x) {
        const int32_t j = a.def[row * a.k + i];
        atomicOr(&bitmap[j >> 5], 1u << (j & 31));
      }
      for (uint32_t i = tid; i < n_c; i += blockDim.x) {
        const uint2 c = cand[i];
        if (chosen(c)) atomicOr(&bitmap[c.y >> 5], 1u << (c.y & 31));
      }
      __syncthreads();
      bitmap_emit_ascending(bitmap, nwords, scratch, [&](uint32_t pos, int32_t j) { idx[pos] = j; });
    } else {
      if (tid == 0) n_out = n_def;
      for (uint32_t i = tid; i < n_def; i += blockDim.x) outj[i] = a.def[row * a.k + i];
      __syncthreads();
      for (uint32_t i = tid; i < n_c; i += blockDim.x) {
        const uint2 c = cand[i];
        if (chosen(c)) outj[atomicAdd(&n_out, 1u)] = (int32_t)c.y;
      }
      __syncthreads();
      // bitonic sort of outj[0..k_eff) ascending, padded to a power of two
      int N = 1;
      while (N < k_eff) N <<= 1;
      for (int i = k_eff + tid; i < N; i += blockDim.x) outj[i] = 0x7fffffff;
      __syncthreads();
      for (int size = 2; size <= N; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
          for (int i = tid; i < N / 2; i += blockDim.x) {
            const int lo = 2 * i - (i & (stride - 1));
            const int hi = lo + stride;
            const bool up = ((lo & size) == 0);
            const int32_t x = outj[lo], y = outj[hi];
            if ((x > y) == up) { outj[lo] = y; outj[hi] = x; }
          }
          __syncthreads();
        }
      }
      for (int i = tid; i < k_eff; i += blockDim.x) idx[i] = outj[i];
    }
  }
  for (int i = k_eff + tid; i < a.k; i += blockDim.x) idx[i] = -1;
  // return this query's workspace rows to zero for the next call
  uint32_t* h = a.hist + row * a.nrep * kNBins;
  for (int i = tid; i < a.nrep * kNBins; i += blockDim.x) h[i] = 0;
  if (tid < 2) a.counts[row * 4 + tid] = 0;
}

static int hist_replicas(int64_t n_q, int64_t max_pool) {
  const int64_t chunks = (max_pool + kScoreChunk - 1) / kScoreChunk;
  return (chunks >= 32 && n_q <= 256) ? 8 : 1;
}

size_t index_ws_bytes(int64_t n_q, int64_t max_q_per_seq, int64_t max_pool, int k) {
  if (prefill_path(max_q_per_seq)) return prefill_ws_bytes(n_q, max_pool);
  const int nrep = hist_replicas(n_q, max_pool);
  size_t s = 0;
  auto add = [&](size_t bytes) { s += (bytes + 255) & ~(size_t)255; };
  add((size_t)n_q * nrep * kNBins * 4);  // hist replicas (zero invariant)
  add((size_t)n_q * 4 * 4);              // counts (zero invariant)
  add((size_t)n_q * 2 * 4);              // info
  add((size_t)n_q * max_pool * 4);       // keys
  add((size_t)n_q * k * 4);              // def
  add((size_t)n_q * max_pool * 8);       // cand
  return s;
}

// A query whose sequence has at most kSmallPool pooled entries (a short
// decode cache) is selected by one workgroup in one launch: its visible keys
// are scored into LDS (4 waves, 32-key MFMA tiles), K* is found by a radix
// select over the keys' own range (the bits above it are common to every key),
// ties at K* are cut at the lowest indices (a second select over the
// complemented indices, only when some are left out), and the chosen entries
// are emitted in ascending order from an LDS bitmap.  The workspace is not
// touched (it stays zero-filled).
constexpr int kSmallPool = 4096;

struct SmallArgs {
  const int64_t* q_off;
  const int64_t* q_pos;
  const int64_t* pool_off;
  int n_seq, m, k;
  const uint8_t* q_codes;
  const uint8_t* q_scales;
  const float* w;
  const uint8_t* k_codes;
  const uint8_t* k_scales;
  int32_t* idx;
};

constexpr int kSmallWaves = 4;
__global__ __launch_bounds__(64 * kSmallWaves) void k_idx_small(SmallArgs a) {
  __shared__ uint32_t keys_s[kSmallPool];
  __shared__ uint32_t bins[1024];
  __shared__ uint32_t bitmap[kSmallPool / 32];
  __shared__ uint32_t scratch[32];
  __shared__ uint32_t red[2][kSmallWaves];
  __shared__ uint32_t n_eq;
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = seq_of_row(a.q_off, a.n_seq, row);
  const int64_t pbase = a.pool_off[b], P = a.pool_off[b + 1] - pbase;
  int64_t nv = n_visible(a.q_pos[row], a.m, P);
  const int nvis = (int)(nv < kSmallPool ? nv : kSmallPool);  // P <= max_pool <= kSmallPool
  const int k_eff = nvis < a.k ? nvis : a.k;
  int32_t* idx = a.idx + row * a.k;
  for (int i = k_eff + tid; i < a.k; i += blockDim.x) idx[i] = -1;
  if (k_eff == nvis) {  // every visible entry is taken (none when nothing is visible)
    for (int i = tid; i < nvis; i += blockDim.x) idx[i] = i;
    return;
  }
  // scores: A = this query's 4 heads (slot 0), B = 32 keys; wave w takes tiles
  // w, w + kSmallWaves, ..., in batches of 8 whose loads all go out first
  const int kb = lane >> 5;
  v8i av = {0, 0, 0, 0, 0, 0, 0, 0};
  int asc = 127;
  if (((lane & 31) >> 2) == 0) {
    const int64_t qrow = row * 4 + (lane & 3);
    uint4 u = *reinterpret_cast<const uint4*>(a.q_codes + qrow * 32 + kb * 16);
    asc = fold_head_weight(u, (int)a.q_scales[qrow * 2 + kb], a.w[qrow]);  // w_h folded into the block scale
    av[0] = (int)u.x; av[1] = (int)u.y; av[2] = (int)u.z; av[3] = (int)u.w;
  }
  constexpr int kB = 8;  // tiles per wave in flight
  const int ntiles = (nvis + 31) >> 5;
  uint32_t mn = 0xffffffffu, mx = 0u;
  for (int t0 = wave; t0 < ntiles; t0 += kSmallWaves * kB) {
    uint4 kcv[kB];
    int ksv[kB];
#pragma unroll
    for (int it = 0; it < kB; ++it) {
      const int j = (t0 + kSmallWaves * it) * 32 + (lane & 31);
      kcv[it] = make_uint4(0u, 0u, 0u, 0u);
      ksv[it] = 127;
      if (j < nvis) {
        kcv[it] = *reinterpret_cast<const uint4*>(a.k_codes + (pbase + j) * 32 + kb * 16);
        ksv[it] = a.k_scales[(pbase + j) * 2 + kb];
      }
    }
#pragma unroll
    for (int it = 0; it < kB; ++it) {
      const int tile = t0 + kSmallWaves * it;
      if (tile >= ntiles) break;  // uniform per wave
      const v8i bv = {(int)kcv[it].x, (int)kcv[it].y, (int)kcv[it].z, (int)kcv[it].w, 0, 0, 0, 0};
      v16f acc = {};
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 4, 4, 0, asc, 0, ksv[it]);
      const int j = tile * 32 + (lane & 31);
      if (lane < 32 && j < nvis) {  // slot 0: lanes 0-31, score index 0
        const float r0 = __int_as_float(max(__float_as_int(acc[0]), 0));
        const float r1 = __int_as_float(max(__float_as_int(acc[1]), 0));
        const float r2 = __int_as_float(max(__float_as_int(acc[2]), 0));
        const float r3 = __int_as_float(max(__float_as_int(acc[3]), 0));
        const uint32_t key = __float_as_uint((r0 + r1) + (r2 + r3));
        keys_s[j] = key;
        mn = key < mn ? key : mn;
        mx = key > mx ? key : mx;
      }
    }
  }
  wave_minmax(mn, mx);
  if (lane == 0) {
    red[0][wave] = mn;
    red[1][wave] = mx;
  }
  for (int i = tid; i < kSmallPool / 32; i += blockDim.x) bitmap[i] = 0u;
  if (tid == 0) n_eq = 0u;
  __syncthreads();
  uint32_t lo = 0xffffffffu, hi = 0u;
  for (int wv = 0; wv < kSmallWaves; ++wv) {
    lo = red[0][wv] < lo ? red[0][wv] : lo;
    hi = red[1][wv] > hi ? red[1][wv] : hi;
  }
  // every key lies in [lo, hi], so the bits above the highest one in which lo
  // and hi differ are common to all of them
  const int top = lo == hi ? 0 : 32 - __clz((int)(lo ^ hi));
  const uint32_t fixed = top >= 32 ? 0u : (lo & ~((1u << top) - 1u));
  uint32_t r;
  const uint32_t kstar = radix_select_desc_low(
      (uint32_t)nvis, (uint32_t)k_eff, top, fixed, [&](uint32_t i) { return keys_s[i]; },
      [&](uint32_t) { return true; }, &r, bins, scratch);
  {
    uint32_t e = 0;
    for (int i = tid; i < nvis; i += blockDim.x) e += keys_s[i] == kstar ? 1u : 0u;
    if (e) atomicAdd(&n_eq, e);
  }
  __syncthreads();
  // r of the entries equal to K* are taken: all of them, or the r lowest indices
  uint32_t jstar = 0;
  if (n_eq > r) {
    const int ibits = 32 - __clz(nvis - 1);  // nvis >= 2 here
    uint32_t r2;
    jstar = radix_select_desc_low(
        (uint32_t)nvis, r, ibits, ~0u << ibits, [&](uint32_t i) { return ~i; },
        [&](uint32_t i) { return keys_s[i] == kstar; }, &r2, bins, scratch);
  }
  for (int i = tid; i < nvis; i += blockDim.x) {
    const uint32_t key = keys_s[i];
    if (key > kstar || (key == kstar && ~(uint32_t)i >= jstar)) atomicOr(&bitmap[i >> 5], 1u << (i & 31));
  }
  __syncthreads();
  bitmap_emit_ascending(bitmap, (nvis + 31) >> 5, scratch, [&](uint32_t pos, int32_t j) { idx[pos] = j; });
}

// the decode-batch chain: scoring (FP4, or bf16 when q_bf16 is set), threshold,
// selection, final
static int decode_topk(int n_seq, int64_t n_q, int64_t max_q_per_seq, const int64_t* q_off, const int64_t* q_pos,
                       const int64_t* pool_off, int64_t max_pool, int m, int k, const uint8_t* q_codes,
                       const uint8_t* q_scales, const float* w, const uint8_t* k_codes, const uint8_t* k_scales,
                       const uint16_t* q_bf16, const uint16_t* k_bf16, int32_t* idx, void* ws, hipStream_t stream) {
  const int nrep = hist_replicas(n_q, max_pool);
  uint8_t* p = (uint8_t*)ws;
  auto take = [&](size_t bytes) { uint8_t* r = p; p += (bytes + 255) & ~(size_t)255; return r; };
  uint32_t* hist = (uint32_t*)take((size_t)n_q * nrep * kNBins * 4);
  uint32_t* counts = (uint32_t*)take((size_t)n_q * 4 * 4);
  uint32_t* info = (uint32_t*)take((size_t)n_q * 2 * 4);
  uint32_t* keys = (uint32_t*)take((size_t)n_q * max_pool * 4);
  int32_t* def = (int32_t*)take((size_t)n_q * k * 4);
  uint2* cand = (uint2*)take((size_t)n_q * max_pool * 8);
  if (n_q == 0) return 0;

  if (!q_bf16 && max_pool <= kSmallPool) {  // short caches: one workgroup per query, one launch
    SmallArgs sm{q_off, q_pos, pool_off, n_seq, m, k, q_codes, q_scales, w, k_codes, k_scales, idx};
    const hipError_t e = launch(2, kProfBoth, k_idx_small, dim3((unsigned)n_q), dim3(64 * kSmallWaves), 0, stream, sm);
    return e == hipSuccess && hipGetLastError() == hipSuccess ? 0 : -1;
  }
  const int qt = max_q_per_seq > 1 ? 8 : 1;
  const int tiles_per_seq = (int)((max_q_per_seq + qt - 1) / qt);
  dim3 g1((unsigned)((max_pool + kScoreChunk - 1) / kScoreChunk), (unsigned)(n_seq * tiles_per_seq));
  if (g1.x == 0) g1.x = 1;
  hipError_t e;
  if (q_bf16) {
    ScoreArgsBf16 sb{q_off, q_pos, pool_off, n_seq, tiles_per_seq, qt, m, nrep, max_pool, q_bf16, w, k_bf16, keys, hist};
    e = launch(0, kProfBoth, k_idx_score_bf16, g1, dim3(256), (size_t)qt * (kNBins / 2) * 4, stream, sb);
  } else {
    ScoreArgs sa{q_off, q_pos, pool_off, n_seq, tiles_per_seq, qt, m, nrep, max_pool, q_codes,
                 q_scales, w, k_codes, k_scales, keys, hist};
    e = launch(0, kProfBoth, k_idx_score, g1, dim3(256), (size_t)qt * (kNBins / 2) * 4, stream, sa);
  }
  if (e == hipSuccess)
    e = launch(-1, kProfNone, k_idx_threshold, dim3((unsigned)n_q), dim3(256), 0, stream, q_off, q_pos, pool_off,
               n_seq, m, k, nrep, (const uint32_t*)hist, info);
  SelectArgs se{q_off, q_pos, pool_off, n_seq, m, k, max_pool, keys, info, counts, def, cand};
  dim3 g2((unsigned)((max_pool + kSelChunk - 1) / kSelChunk), (unsigned)n_q);
  if (g2.x == 0) g2.x = 1;
  if (e == hipSuccess) e = launch(1, kProfBoth, k_idx_select, g2, dim3(256), 0, stream, se);
  const size_t bm_bytes = (size_t)((max_pool + 31) / 32) * 4;
  const int use_bitmap = bm_bytes <= (size_t)kBitmapMaxBytes ? 1 : 0;
  FinalArgs fa{q_off, q_pos, pool_off, n_seq, m, k, nrep, use_bitmap, max_pool, counts, hist, def, cand, idx};
  // allow the bitmap beyond the default dynamic LDS limit (idempotent, per call:
  // it holds for whichever device is current)
  (void)hipFuncSetAttribute((const void*)k_idx_final, hipFuncAttributeMaxDynamicSharedMemorySize, kBitmapMaxBytes);
  if (e == hipSuccess)
    e = launch(2, kProfBoth, k_idx_final, dim3((unsigned)n_q), dim3(1024), use_bitmap ? bm_bytes : 0, stream, fa);
  return e == hipSuccess && hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_index_topk(int n_seq, int64_t n_q, int64_t max_q_per_seq, const int64_t* q_off,
                      const int64_t* q_pos, const int64_t* pool_off, int64_t max_pool, int m,
                      int k, const uint8_t* q_codes, const uint8_t* q_scales, const float* w,
                      const uint8_t* k_codes, const uint8_t* k_scales, int32_t* idx, void* ws,
                      hipStream_t stream) {
  if (prefill_path(max_q_per_seq))
    return launch_prefill_topk(n_seq, n_q, max_q_per_seq, q_off, q_pos, pool_off, max_pool, m, k, q_codes, q_scales,
                               w, k_codes, k_scales, idx, ws, stream);
  return decode_topk(n_seq, n_q, max_q_per_seq, q_off, q_pos, pool_off, max_pool, m, k, q_codes, q_scales, w, k_codes,
                     k_scales, nullptr, nullptr, idx, ws, stream);
}

int launch_index_topk_bf16(int n_seq, int64_t n_q, int64_t max_q_per_seq, const int64_t* q_off, const int64_t* q_pos,
                           const int64_t* pool_off, int64_t max_pool, int m, int k, const uint16_t* q, const float* w,
                           const uint16_t* keys, int32_t* idx, void* ws, hipStream_t stream) {
  return decode_topk(n_seq, n_q, max_q_per_seq, q_off, q_pos, pool_off, max_pool, m, k, nullptr, nullptr, w, nullptr,
                     nullptr, q, keys, idx, ws, stream);
}

}  // namespace csa

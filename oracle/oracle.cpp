/*
 * CPU ORACLE for compressed sparse attention (CSA) and heavily compressed
 * attention (HCA).  TEST INFRASTRUCTURE ONLY: tests, the smoke check and the
 * benchmark's CPU-baseline leg may call it; the product path never does.
 * It shares no code, header, table or helper with the HIP library.
 *
 * Plain, slow, obviously-correct C++.  Floating point is fp64 throughout; the
 * lightning-indexer score is computed exactly, twice, by independent routes
 * (128-bit integers and fp64), which must agree.
 *
 * Sources (pages on DeepSeek-V4):
 *  - discuss.pytorch.kr "DeepSeek-V4 series" summary, section on CSA and HCA:
 *    CSA merges m consecutive KV entries into one, applies DeepSeek Sparse
 *    Attention so that each query attends only to its top-k compressed
 *    entries, and adds a sliding-window branch of recent tokens; HCA merges
 *    m' >> m entries and runs dense attention with no sparse selection.
 *  - same page, section on FP4 quantisation-aware training: the indexer QK
 *    path runs in FP4 (MXFP4).
 *  - sigco.tistory.com "DeepSeek-V4 paper reading", section on CSA and HCA:
 *    compress the context blockwise, an indexer finds the blocks relevant to
 *    the current token, only the top candidates are attended, recent tokens
 *    are kept by a sliding window; HCA attends to all compressed entries.
 *  - jyp-garden EP 95 notes (IDEAS): KV compressed to one quarter, then the
 *    Lightning Indexer picks the top-k; V4 uses multi-query attention.
 * Where the pages leave a step open the reading taken is stated at the step.
 *
 * Layouts: raw KV rows are [L][2][d] (K half, then V half); pooling logits Z
 * use the same layout; pooled rows are [P][2][d].  dtype code 0 = fp32,
 * 1 = bf16 bit patterns.  Indexer vectors are MXFP4: packed e2m1 codes (even
 * element in the low nibble) with one E8M0 scale byte per 32 elements.
 */
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <utility>
#include <vector>

namespace {

double load_elem(int dt, const void* base, int64_t i) {
  if (dt == 0) return (double)static_cast<const float*>(base)[i];
  uint32_t bits = (uint32_t) static_cast<const uint16_t*>(base)[i] << 16;
  float f;
  std::memcpy(&f, &bits, 4);
  return (double)f;
}

/* OCP MX FP4 (E2M1): sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0.
 * Exponent field 0 is subnormal: value = m * 2^(1-1) * 1/2. */
double e2m1_value(int code) {
  int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  double mag = (e == 0) ? 0.5 * m : std::ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -mag : mag;
}

/* the same value times two, as an integer (all e2m1 values are multiples of 1/2) */
int e2m1_twice(int code) { return (int)std::lround(2.0 * e2m1_value(code)); }

int nibble(const uint8_t* packed, int i) { return (packed[i >> 1] >> ((i & 1) * 4)) & 15; }

bool is_pow2(float w, int* e) {
  if (!(w > 0.0f) || !std::isfinite(w)) return false;
  int ex;
  double fr = std::frexp((double)w, &ex);
  if (fr != 0.5) return false;
  *e = ex - 1;
  return true;
}

/* Pooling of one block (compression step).  The pages say m consecutive KV
 * entries become one; the rule used is a per-channel softmax over the block's
 * logits followed by the weighted sum of the block's rows. */
void pool_block(int dt, const void* x, const void* z, int64_t row0, int m, int C, double* out) {
  for (int c = 0; c < C; ++c) {
    double mu = -std::numeric_limits<double>::infinity();
    for (int i = 0; i < m; ++i) mu = std::max(mu, load_elem(dt, z, (row0 + i) * C + c));
    double num = 0.0, den = 0.0;
    for (int i = 0; i < m; ++i) {
      double e = std::exp(load_elem(dt, z, (row0 + i) * C + c) - mu);
      num += e * load_elem(dt, x, (row0 + i) * C + c);
      den += e;
    }
    out[c] = num / den;
  }
}

/* Attention with one softmax over an explicit key/value list (fp64). */
void attend(int H, int d, double scale, const double* q, int64_t n, const double* keys,
            const double* vals, double* out, double* lse) {
  std::vector<double> logit((size_t)std::max<int64_t>(n, 1));
  for (int h = 0; h < H; ++h) {
    double* o = out + (int64_t)h * d;
    if (n == 0) { /* empty key set: zero output, lse = -inf */
      for (int c = 0; c < d; ++c) o[c] = 0.0;
      if (lse) lse[h] = -std::numeric_limits<double>::infinity();
      continue;
    }
    double M = -std::numeric_limits<double>::infinity();
    for (int64_t j = 0; j < n; ++j) {
      double s = 0.0;
      for (int c = 0; c < d; ++c) s += q[(int64_t)h * d + c] * keys[j * d + c];
      logit[j] = scale * s;
      M = std::max(M, logit[j]);
    }
    double den = 0.0;
    for (int c = 0; c < d; ++c) o[c] = 0.0;
    for (int64_t j = 0; j < n; ++j) {
      double e = std::exp(logit[j] - M);
      den += e;
      for (int c = 0; c < d; ++c) o[c] += e * vals[j * d + c];
    }
    for (int c = 0; c < d; ++c) o[c] /= den;
    if (lse) lse[h] = M + std::log(den);
  }
}

struct ScoreResult {
  double s;      /* exact score */
  bool f32_exact; /* a fp32 evaluation in any summation order is exact */
  bool ok;        /* the two exact routes agree */
};

/* Lightning-indexer score of one key for one query:
 *   S = sum_h w_h * max(0, sum_c q[h][c] * k[c])
 * over MXFP4 values (code value times the 2^(e-127) scale of its 32-block). */
/* whether v << sh (v >= 0) stays below 2^125, so that a few such terms still
 * add up inside a signed 128-bit integer */
bool shl_fits(__int128 v, int sh) {
  if (v < 0 || sh < 0) return false;
  int bits = 0;
  for (__int128 t = v; t != 0; t >>= 1) ++bits;
  return bits + sh <= 125;
}

ScoreResult index_score(int H_I, int d_I, const uint8_t* qc, const uint8_t* qs, const float* w,
                        const uint8_t* kc, const uint8_t* ks) {
  ScoreResult r{0.0, true, true};
  const int nb = d_I / 32;
  /* route 1: fp64 on decoded values */
  double s64 = 0.0;
  for (int h = 0; h < H_I; ++h) {
    double dot = 0.0;
    for (int c = 0; c < d_I; ++c) {
      double qv = e2m1_value(nibble(qc + h * (d_I / 2), c)) * std::ldexp(1.0, (int)qs[h * nb + c / 32] - 127);
      double kv = e2m1_value(nibble(kc, c)) * std::ldexp(1.0, (int)ks[c / 32] - 127);
      dot += qv * kv;
    }
    s64 += (double)w[h] * std::max(0.0, dot);
  }
  /* route 2: 128-bit integers.  A product of two e2m1 values times their
   * scales is (2a)(2b) * 2^(eq+ek-256), so each block's dot is an integer
   * times 2^(eq+ek-256). */
  __int128 tot = 0;
  int tot_e = 0;
  bool have = false, all_pow2 = true;
  double min_unit_all = std::numeric_limits<double>::infinity();
  std::vector<long long> blk((size_t)nb);
  std::vector<int> bexp((size_t)nb);
  std::vector<char> nonzero((size_t)nb);
  for (int h = 0; h < H_I; ++h) {
    int we;
    if (!is_pow2(w[h], &we)) { all_pow2 = false; we = 0; }
    /* per block: the integer sum of its products (2a)(2b), their exponent
     * eq+ek-256, and whether any product is non-zero.  A block whose
     * products are all zero adds exactly nothing, whatever its scales, so it
     * takes no part in the dot's unit 2^emin. */
    int emin = 1 << 30;
    double abs_sum = 0.0;
    for (int b = 0; b < nb; ++b) {
      blk[b] = 0;
      nonzero[b] = 0;
      bexp[b] = (int)qs[h * nb + b] + (int)ks[b] - 256;
      for (int c = b * 32; c < b * 32 + 32; ++c) {
        int pa = e2m1_twice(nibble(qc + h * (d_I / 2), c)) * e2m1_twice(nibble(kc, c));
        blk[b] += pa;
        if (pa != 0) nonzero[b] = 1;
        abs_sum += std::ldexp((double)std::abs(pa), bexp[b]);
      }
      if (nonzero[b]) emin = std::min(emin, bexp[b]);
    }
    if (emin == (1 << 30)) continue; /* every product is zero: the dot is 0 */
    __int128 dot = 0;
    for (int b = 0; b < nb; ++b) {
      if (!nonzero[b]) continue;
      int sh = bexp[b] - emin;
      if (sh > 90) { r.ok = false; sh = 90; } /* beyond what 128 bits can check */
      dot += (__int128)blk[b] * ((__int128)1 << sh);
    }
    /* fp32 exactness of this head's dot in any order: every partial sum is a
     * multiple of 2^emin bounded by abs_sum, so it needs abs_sum < 2^(24+emin) */
    if (abs_sum >= std::ldexp(1.0, 24 + emin)) r.f32_exact = false;
    if (dot <= 0) continue;
    int e = emin + we;
    min_unit_all = std::min(min_unit_all, std::ldexp(1.0, e));
    if (!have) { tot = dot; tot_e = e; have = true; }
    else if (!r.ok) continue; /* already beyond what 128 bits can check */
    else if (e >= tot_e) {
      if (!shl_fits(dot, e - tot_e)) r.ok = false;
      else tot += dot << (e - tot_e);
    } else {
      if (!shl_fits(tot, tot_e - e)) r.ok = false;
      else { tot = (tot << (tot_e - e)) + dot; tot_e = e; }
    }
  }
  if (all_pow2) { /* the integer route needs power-of-two head weights */
    double sint = have ? std::ldexp((double)tot, tot_e) : 0.0;
    if ((__int128)(double)tot != tot) r.ok = false; /* too wide for the fp64 comparison */
    if (sint != s64) r.ok = false;
  } else {
    r.f32_exact = false;
  }
  /* head sum: non-negative terms, all multiples of the smallest unit */
  if (have && s64 >= min_unit_all * 16777216.0) r.f32_exact = false;
  r.s = s64;
  return r;
}

/* Top-k: the k visible entries first under (score descending, index
 * ascending); emitted in ascending index order and padded with -1. */
void topk(int64_t n, const double* S, int k, int32_t* idx) {
  std::vector<std::pair<double, int64_t>> v((size_t)n);
  for (int64_t j = 0; j < n; ++j) v[(size_t)j] = {S[j], j};
  std::sort(v.begin(), v.end(), [](const std::pair<double, int64_t>& a, const std::pair<double, int64_t>& b) {
    if (a.first != b.first) return a.first > b.first;
    return a.second < b.second;
  });
  int64_t keep = std::min<int64_t>(k, n);
  std::vector<int32_t> sel((size_t)keep);
  for (int64_t i = 0; i < keep; ++i) sel[(size_t)i] = (int32_t)v[(size_t)i].second;
  std::sort(sel.begin(), sel.end());
  for (int i = 0; i < k; ++i) idx[i] = i < keep ? sel[(size_t)i] : -1;
}

void raw_half(int dt, const void* kv, int64_t row, int d, int half, double* dst) {
  for (int c = 0; c < d; ++c) dst[c] = load_elem(dt, kv, row * 2 * d + half * d + c);
}

}  // namespace

extern "C" {

double orc_e2m1_value(int code) { return e2m1_value(code & 15); }

double orc_e8m0_value(int byte) {
  if ((byte & 255) == 255) return std::numeric_limits<double>::quiet_NaN();
  return std::ldexp(1.0, (byte & 255) - 127);
}

/* Pool n_rows/m whole blocks of C channels (tail rows that do not fill a block
 * are not pooled; they are covered by the sliding window). */
int orc_pool(int dt, int64_t n_rows, int C, int m, const void* x, const void* z, double* out) {
  if (m < 1 || C < 1 || n_rows < 0) return -1;
  int64_t P = n_rows / m;
  for (int64_t j = 0; j < P; ++j) pool_block(dt, x, z, j * m, m, C, out + j * C);
  return 0;
}

/* Exact indexer scores of n_keys keys for one query.  Returns 0, or -2 when
 * the two exact routes disagree.  exact_f32[j] (nullable) tells whether a
 * fp32 evaluation of key j is guaranteed exact in any summation order. */
int orc_index_scores(int64_t n_keys, int H_I, int d_I, const uint8_t* qc, const uint8_t* qs,
                     const float* w, const uint8_t* kc, const uint8_t* ks, double* S,
                     int32_t* exact_f32) {
  if (d_I % 32 != 0 || H_I < 1) return -1;
  int rc = 0;
  for (int64_t j = 0; j < n_keys; ++j) {
    ScoreResult r = index_score(H_I, d_I, qc, qs, w, kc + j * (d_I / 2), ks + j * (d_I / 32));
    S[j] = r.s;
    if (exact_f32) exact_f32[j] = r.f32_exact ? 1 : 0;
    if (!r.ok) rc = -2;
  }
  return rc;
}

/* The indexer score with bf16 operands (the higher-precision indexer the
 * MXFP4 one is compared with; pytorch.kr FP4 QAT section: the FP4 indexer is
 * set against a higher-precision selector):
 *   S = sum_h w_h * max(0, sum_c q[h][c] * k[c])
 * q [H_I][d_I] and keys [n][d_I] as bf16 bit patterns.  Every product of two
 * bf16 values is exact in fp64 (8 + 8 significand bits); the sum runs in fp64
 * in index order. */
int orc_index_scores_bf16(int64_t n_keys, int H_I, int d_I, const uint16_t* q, const float* w,
                          const uint16_t* keys, double* S) {
  if (H_I < 1 || d_I < 1 || n_keys < 0) return -1;
  for (int64_t j = 0; j < n_keys; ++j) {
    double s = 0.0;
    for (int h = 0; h < H_I; ++h) {
      double dot = 0.0;
      for (int c = 0; c < d_I; ++c)
        dot += load_elem(1, q, (int64_t)h * d_I + c) * load_elem(1, keys, j * d_I + c);
      s += (double)w[h] * std::max(0.0, dot);
    }
    S[j] = s;
  }
  return 0;
}

int orc_topk(int64_t n, const double* S, int k, int32_t* idx) {
  if (k < 1 || n < 0) return -1;
  topk(n, S, k, idx);
  return 0;
}

int orc_attend(int H, int d, double scale, const double* q, int64_t n, const double* keys,
               const double* vals, double* out, double* lse) {
  if (H < 1 || d < 1 || n < 0) return -1;
  attend(H, d, scale, q, n, keys, vals, out, lse);
  return 0;
}

/* End-to-end CSA for one query at position t of one sequence.
 *  1. visible compressed entries: block j covers tokens jm..jm+m-1 and is
 *     visible iff it ends at or before t, so n_vis = floor((t+1)/m);
 *  2. indexer scores of the visible entries (exact);
 *  3. top-k of the scores, ties to the lower index;
 *  4. keys/values = the selected pooled rows followed by the raw rows of the
 *     last W tokens up to t (max(0,t-W+1)..t), concatenated without dedup;
 *  5. one softmax over that list.
 * pooled (nullable) is a prebuilt fp64 pooled cache [P][2d]; when NULL the
 * selected blocks are pooled here from kv/z. */
int orc_csa_query(int dt, int d, int H, int m, int W, int k, double scale, int64_t t,
                  const void* kv, const void* z, const double* pooled, const void* q,
                  int H_I, int d_I, const uint8_t* qc, const uint8_t* qs, const float* w,
                  const uint8_t* kc, const uint8_t* ks, double* out, double* lse, int32_t* idx) {
  if (m < 1 || W < 0 || k < 1 || t < 0 || d < 1 || H < 1) return -1;
  const int C = 2 * d;
  int64_t n_vis = (t + 1) / m;
  std::vector<double> S((size_t)n_vis);
  int rc = orc_index_scores(n_vis, H_I, d_I, qc, qs, w, kc, ks, S.data(), nullptr);
  if (rc) return rc;
  topk(n_vis, S.data(), k, idx);
  int64_t n_sel = std::min<int64_t>(k, n_vis);
  int64_t w0 = std::max<int64_t>(0, t - W + 1);
  int64_t n_win = (W > 0) ? t - w0 + 1 : 0;
  int64_t n = n_sel + n_win;
  std::vector<double> keys((size_t)(n * d)), vals((size_t)(n * d)), row((size_t)C), qd((size_t)H * d);
  for (int64_t i = 0; i < n_sel; ++i) {
    const double* pr;
    if (pooled) pr = pooled + (int64_t)idx[i] * C;
    else { pool_block(dt, kv, z, (int64_t)idx[i] * m, m, C, row.data()); pr = row.data(); }
    std::copy(pr, pr + d, keys.begin() + i * d);
    std::copy(pr + d, pr + C, vals.begin() + i * d);
  }
  for (int64_t i = 0; i < n_win; ++i) {
    raw_half(dt, kv, w0 + i, d, 0, keys.data() + (n_sel + i) * d);
    raw_half(dt, kv, w0 + i, d, 1, vals.data() + (n_sel + i) * d);
  }
  for (int64_t i = 0; i < (int64_t)H * d; ++i) qd[(size_t)i] = load_elem(dt, q, i);
  attend(H, d, scale, qd.data(), n, keys.data(), vals.data(), out, lse);
  return 0;
}

/* End-to-end HCA for one query at position t: dense attention over every
 * visible m'-pooled entry (j < floor((t+1)/m')), optionally followed by a
 * window of the last W_h raw tokens (W_h = 0: no window). */
int orc_hca_query(int dt, int d, int H, int m_h, int W_h, double scale, int64_t t, const void* kv,
                  const void* z, const double* hpooled, const void* q, double* out, double* lse) {
  if (m_h < 1 || W_h < 0 || t < 0 || d < 1 || H < 1) return -1;
  const int C = 2 * d;
  int64_t n_vis = (t + 1) / m_h;
  int64_t w0 = std::max<int64_t>(0, t - W_h + 1);
  int64_t n_win = (W_h > 0) ? t - w0 + 1 : 0;
  int64_t n = n_vis + n_win;
  std::vector<double> keys((size_t)(n * d)), vals((size_t)(n * d)), row((size_t)C), qd((size_t)H * d);
  for (int64_t j = 0; j < n_vis; ++j) {
    const double* pr;
    if (hpooled) pr = hpooled + j * C;
    else { pool_block(dt, kv, z, j * m_h, m_h, C, row.data()); pr = row.data(); }
    std::copy(pr, pr + d, keys.begin() + j * d);
    std::copy(pr + d, pr + C, vals.begin() + j * d);
  }
  for (int64_t i = 0; i < n_win; ++i) {
    raw_half(dt, kv, w0 + i, d, 0, keys.data() + (n_vis + i) * d);
    raw_half(dt, kv, w0 + i, d, 1, vals.data() + (n_vis + i) * d);
  }
  for (int64_t i = 0; i < (int64_t)H * d; ++i) qd[(size_t)i] = load_elem(dt, q, i);
  attend(H, d, scale, qd.data(), n, keys.data(), vals.data(), out, lse);
  return 0;
}

/* Stage-wise CSA attention on given inputs: a pooled cache [P][2d] in the KV
 * dtype and a given index list (entries < 0 are padding and skipped). */
int orc_csa_attend_given(int dt, int d, int H, int W, double scale, int64_t t, const void* kv,
                         const void* pooled, const int32_t* idx, int k, const void* q, double* out,
                         double* lse) {
  if (W < 0 || t < 0 || k < 0) return -1;
  int64_t w0 = std::max<int64_t>(0, t - W + 1);
  int64_t n_win = (W > 0) ? t - w0 + 1 : 0;
  std::vector<int32_t> sel;
  for (int i = 0; i < k; ++i)
    if (idx[i] >= 0) sel.push_back(idx[i]);
  int64_t n = (int64_t)sel.size() + n_win;
  std::vector<double> keys((size_t)(n * d)), vals((size_t)(n * d)), qd((size_t)H * d);
  for (size_t i = 0; i < sel.size(); ++i) {
    raw_half(dt, pooled, sel[i], d, 0, keys.data() + i * d);
    raw_half(dt, pooled, sel[i], d, 1, vals.data() + i * d);
  }
  for (int64_t i = 0; i < n_win; ++i) {
    raw_half(dt, kv, w0 + i, d, 0, keys.data() + ((int64_t)sel.size() + i) * d);
    raw_half(dt, kv, w0 + i, d, 1, vals.data() + ((int64_t)sel.size() + i) * d);
  }
  for (int64_t i = 0; i < (int64_t)H * d; ++i) qd[(size_t)i] = load_elem(dt, q, i);
  attend(H, d, scale, qd.data(), n, keys.data(), vals.data(), out, lse);
  return 0;
}

/* Stage-wise HCA attention on a given pooled cache [P'][2d] in the KV dtype. */
int orc_hca_attend_given(int dt, int d, int H, int m_h, int W_h, double scale, int64_t t,
                         const void* kv, const void* hpooled, const void* q, double* out,
                         double* lse) {
  if (m_h < 1 || W_h < 0 || t < 0) return -1;
  int64_t n_vis = (t + 1) / m_h;
  int64_t w0 = std::max<int64_t>(0, t - W_h + 1);
  int64_t n_win = (W_h > 0) ? t - w0 + 1 : 0;
  int64_t n = n_vis + n_win;
  std::vector<double> keys((size_t)(n * d)), vals((size_t)(n * d)), qd((size_t)H * d);
  for (int64_t j = 0; j < n_vis; ++j) {
    raw_half(dt, hpooled, j, d, 0, keys.data() + j * d);
    raw_half(dt, hpooled, j, d, 1, vals.data() + j * d);
  }
  for (int64_t i = 0; i < n_win; ++i) {
    raw_half(dt, kv, w0 + i, d, 0, keys.data() + (n_vis + i) * d);
    raw_half(dt, kv, w0 + i, d, 1, vals.data() + (n_vis + i) * d);
  }
  for (int64_t i = 0; i < (int64_t)H * d; ++i) qd[(size_t)i] = load_elem(dt, q, i);
  attend(H, d, scale, qd.data(), n, keys.data(), vals.data(), out, lse);
  return 0;
}

/* MXFP4 quantisation of rows of `dim` elements (dim a multiple of 32), the
 * step before the indexer: the pages put the indexer's QK path in MXFP4
 * (pytorch.kr, FP4 QAT paragraph) but give no conversion rule; the reading
 * taken is the OCP MX one, written out here from its definition:
 *  - per block of 32 elements, the shared scale is 2^e with
 *    e = floor(log2(amax)) - 2, 2 being the largest exponent of an e2m1
 *    value (6 = 1.5 * 2^2), amax the block's largest magnitude; stored as the
 *    E8M0 byte e + 127, clamped to [0, 254]; a block of zeros takes byte 0;
 *  - each element x becomes the e2m1 value nearest to x / 2^e, ties going to
 *    the code with an even mantissa bit, magnitudes above 6 saturating to 6;
 *    the sign bit is set only for a non-zero negative result, so zero is
 *    always code 0;
 *  - codes are packed two per byte, the even element in the low nibble.
 * x: [rows][dim] in dtype dt; codes [rows][dim/2]; scales [rows][dim/32]. */
int orc_mxfp4_quantize(int64_t rows, int dim, int dt, const void* x, uint8_t* codes, uint8_t* scales) {
  if (rows < 0 || dim < 32 || dim % 32 != 0) return -1;
  for (int64_t r = 0; r < rows; ++r) {
    for (int blk = 0; blk < dim / 32; ++blk) {
      const int64_t base = r * dim + blk * 32;
      double amax = 0.0;
      for (int i = 0; i < 32; ++i) amax = std::max(amax, std::fabs(load_elem(dt, x, base + i)));
      int e = -127;
      if (amax > 0.0) {
        int ex;
        (void)std::frexp(amax, &ex);  /* amax = f * 2^ex with f in [0.5, 1): floor(log2 amax) = ex - 1 */
        e = std::max(-127, std::min(127, (ex - 1) - 2));
      }
      scales[r * (dim / 32) + blk] = (uint8_t)(e + 127);
      for (int i = 0; i < 32; ++i) {
        const double v = std::ldexp(load_elem(dt, x, base + i), -e);
        const double mag = std::fabs(v);
        int best = 0;
        double best_err = std::numeric_limits<double>::infinity();
        for (int c = 0; c < 8; ++c) {  /* nearest magnitude; a tie keeps the even code */
          const double err = std::fabs(mag - e2m1_value(c));
          if (err < best_err || (err == best_err && (c & 1) == 0)) {
            best = c;
            best_err = err;
          }
        }
        const int code = best | ((v < 0.0 && best != 0) ? 8 : 0);
        const int64_t byte = r * (dim / 2) + blk * 16 + i / 2;
        if (i % 2 == 0) codes[byte] = (uint8_t)code;
        else codes[byte] = (uint8_t)(codes[byte] | (code << 4));
      }
    }
  }
  return 0;
}

}  // extern "C"

// Sanitizer driver for the oracle -- TEST INFRASTRUCTURE ONLY.
//
// Runs every exported oracle function on small inputs (both KV dtypes, empty
// and degenerate sizes, k above the visible count, windows clipped at the
// sequence start) so that a build of oracle.cpp with AddressSanitizer and
// UndefinedBehaviorSanitizer sees all of its code paths.  It checks no
// values (the pins do that); a sanitizer report or a non-zero return is the
// failure.  Built and run by tests/test_sanitizers.py.
#include <cstdint>
#include <cstdio>
#include <vector>

extern "C" {
double orc_e2m1_value(int code);
double orc_e8m0_value(int byte);
int orc_pool(int dt, int64_t n_rows, int C, int m, const void* x, const void* z, double* out);
int orc_index_scores(int64_t n_keys, int H_I, int d_I, const uint8_t* qc, const uint8_t* qs, const float* w,
                     const uint8_t* kc, const uint8_t* ks, double* S, int32_t* exact_f32);
int orc_index_scores_bf16(int64_t n_keys, int H_I, int d_I, const uint16_t* q, const float* w,
                          const uint16_t* keys, double* S);
int orc_topk(int64_t n, const double* S, int k, int32_t* idx);
int orc_attend(int H, int d, double scale, const double* q, int64_t n, const double* keys, const double* vals,
               double* out, double* lse);
int orc_csa_query(int dt, int d, int H, int m, int W, int k, double scale, int64_t t, const void* kv, const void* z,
                  const double* pooled, const void* q, int H_I, int d_I, const uint8_t* qc, const uint8_t* qs,
                  const float* w, const uint8_t* kc, const uint8_t* ks, double* out, double* lse, int32_t* idx);
int orc_hca_query(int dt, int d, int H, int m_h, int W_h, double scale, int64_t t, const void* kv, const void* z,
                  const double* hpooled, const void* q, double* out, double* lse);
int orc_csa_attend_given(int dt, int d, int H, int W, double scale, int64_t t, const void* kv, const void* pooled,
                         const int32_t* idx, int k, const void* q, double* out, double* lse);
int orc_hca_attend_given(int dt, int d, int H, int m_h, int W_h, double scale, int64_t t, const void* kv,
                         const void* hpooled, const void* q, double* out, double* lse);
int orc_mxfp4_quantize(int64_t rows, int dim, int dt, const void* x, uint8_t* codes, uint8_t* scales);
}

namespace {

uint64_t g_state = 0x2545F4914F6CDD1DULL;
uint32_t next_u32() {  // xorshift64*: input bits only
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return (uint32_t)((g_state * 0x2545F4914F6CDD1DULL) >> 32);
}
float small_float() { return (float)((int)(next_u32() % 17) - 8) * 0.125f; }
uint16_t bf16_bits(float f) {  // values here are exact in bf16
  uint32_t u;
  __builtin_memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

int failures = 0;
void expect_ok(int rc, const char* what) {
  if (rc != 0) {
    std::fprintf(stderr, "%s returned %d\n", what, rc);
    ++failures;
  }
}

// KV-dtype buffer of n elements: fp32 (dt 0) or bf16 bits (dt 1)
struct KvBuf {
  std::vector<float> f;
  std::vector<uint16_t> h;
  KvBuf(int dt, size_t n) {
    f.resize(n);
    h.resize(n);
    for (size_t i = 0; i < n; ++i) {
      f[i] = small_float();
      h[i] = bf16_bits(f[i]);
    }
    (void)dt;
  }
  const void* ptr(int dt) const { return dt == 0 ? (const void*)f.data() : (const void*)h.data(); }
};

void run_dtype(int dt) {
  const int d = 8, H = 2, C = 2 * d, H_I = 4, d_I = 64;
  for (int64_t L : {0, 1, 3, 31, 64}) {
    KvBuf kv(dt, (size_t)(L * C + 1)), z(dt, (size_t)(L * C + 1)), q(dt, (size_t)(H * d));
    for (int m : {1, 3, 4, 8}) {
      const int64_t P = L / m;
      std::vector<double> pooled((size_t)(P * C + 1));
      expect_ok(orc_pool(dt, L, C, m, kv.ptr(dt), z.ptr(dt), pooled.data()), "orc_pool");
      if (L == 0) continue;
      std::vector<uint8_t> qc((size_t)H_I * d_I / 2), qs((size_t)H_I * d_I / 32);
      std::vector<uint8_t> kc((size_t)(P * d_I / 2 + 1)), ks((size_t)(P * d_I / 32 + 1));
      std::vector<float> w(H_I, 1.0f);
      for (auto& b : qc) b = (uint8_t)next_u32();
      for (auto& b : qs) b = (uint8_t)(125 + next_u32() % 5);
      for (auto& b : kc) b = (uint8_t)next_u32();
      for (auto& b : ks) b = (uint8_t)(125 + next_u32() % 5);
      w[1] = 0.5f;
      w[2] = 2.0f;
      std::vector<double> out((size_t)H * d), lse(H);
      for (int k : {1, 5, 100}) {
        std::vector<int32_t> idx(k);
        for (int W : {0, 3, 100}) {
          const int64_t t = L - 1;
          expect_ok(orc_csa_query(dt, d, H, m, W, k, 0.35, t, kv.ptr(dt), z.ptr(dt), nullptr, q.ptr(dt), H_I, d_I,
                                  qc.data(), qs.data(), w.data(), kc.data(), ks.data(), out.data(), lse.data(),
                                  idx.data()),
                    "orc_csa_query");
          expect_ok(orc_csa_query(dt, d, H, m, W, k, 0.35, t, kv.ptr(dt), z.ptr(dt), pooled.data(), q.ptr(dt), H_I,
                                  d_I, qc.data(), qs.data(), w.data(), kc.data(), ks.data(), out.data(), lse.data(),
                                  idx.data()),
                    "orc_csa_query (pooled)");
          expect_ok(orc_hca_query(dt, d, H, m, W, 0.35, t, kv.ptr(dt), z.ptr(dt), nullptr, q.ptr(dt), out.data(),
                                  lse.data()),
                    "orc_hca_query");
          expect_ok(orc_hca_query(dt, d, H, m, W, 0.35, t, kv.ptr(dt), z.ptr(dt), pooled.data(), q.ptr(dt),
                                  out.data(), lse.data()),
                    "orc_hca_query (pooled)");
          // the given-index attention on a pooled cache in the KV dtype
          KvBuf pk(dt, (size_t)(P * C + 1));
          std::vector<int32_t> gi(k);
          for (int i = 0; i < k; ++i) gi[i] = (P > 0 && i < P) ? (int32_t)(next_u32() % P) : -1;
          expect_ok(orc_csa_attend_given(dt, d, H, W, 0.35, t, kv.ptr(dt), pk.ptr(dt), gi.data(), k, q.ptr(dt),
                                         out.data(), lse.data()),
                    "orc_csa_attend_given");
          expect_ok(orc_hca_attend_given(dt, d, H, m, W, 0.35, t, kv.ptr(dt), pk.ptr(dt), q.ptr(dt), out.data(),
                                         lse.data()),
                    "orc_hca_attend_given");
        }
      }
    }
  }
  // quantiser: rows of 32 and 64 elements, zeros and large values included
  for (int dim : {32, 64}) {
    KvBuf x(dt, (size_t)(5 * dim));
    for (int i = 0; i < dim; ++i) {
      x.f[i] = 0.0f;
      x.h[i] = 0;
    }
    x.f[dim] = 1e30f;
    x.h[dim] = bf16_bits(1e30f);
    std::vector<uint8_t> codes((size_t)(5 * dim / 2)), scales((size_t)(5 * dim / 32));
    expect_ok(orc_mxfp4_quantize(5, dim, dt, x.ptr(dt), codes.data(), scales.data()), "orc_mxfp4_quantize");
  }
}

}  // namespace

int main() {
  double acc = 0;
  for (int c = 0; c < 16; ++c) acc += orc_e2m1_value(c);
  for (int b = 0; b < 255; ++b) acc += orc_e8m0_value(b) > 0 ? 1 : 0;
  // indexer scores on both routes, exactness flags, bf16 scores, top-k
  const int H_I = 4, d_I = 64;
  for (int64_t n : {0, 1, 50}) {
    std::vector<uint8_t> qc((size_t)H_I * d_I / 2), qs((size_t)H_I * d_I / 32);
    std::vector<uint8_t> kc((size_t)(n * d_I / 2 + 1)), ks((size_t)(n * d_I / 32 + 1));
    for (auto& b : qc) b = (uint8_t)next_u32();
    for (auto& b : qs) b = (uint8_t)(125 + next_u32() % 5);
    for (auto& b : kc) b = (uint8_t)next_u32();
    for (auto& b : ks) b = (uint8_t)(125 + next_u32() % 5);
    std::vector<float> w = {0.5f, 1.0f, 2.0f, 0.0f};
    std::vector<double> S((size_t)n + 1);
    std::vector<int32_t> ex((size_t)n + 1);
    expect_ok(orc_index_scores(n, H_I, d_I, qc.data(), qs.data(), w.data(), kc.data(), ks.data(), S.data(),
                               ex.data()),
              "orc_index_scores");
    // scales spread over 100 octaves and a zero-scale block: beyond what the
    // exact route can confirm, which it reports (-2) without overflowing
    for (auto& b : qs) b = (uint8_t)(27 + next_u32() % 200);
    for (auto& b : ks) b = (uint8_t)(27 + next_u32() % 200);
    qs[0] = 0;
    const int rc = orc_index_scores(n, H_I, d_I, qc.data(), qs.data(), w.data(), kc.data(), ks.data(), S.data(),
                                    ex.data());
    if (rc != 0 && rc != -2) expect_ok(rc, "orc_index_scores (wide scales)");
    std::vector<uint16_t> qb((size_t)H_I * d_I), kb((size_t)(n * d_I + 1));
    for (auto& v : qb) v = bf16_bits(small_float());
    for (auto& v : kb) v = bf16_bits(small_float());
    expect_ok(orc_index_scores_bf16(n, H_I, d_I, qb.data(), w.data(), kb.data(), S.data()), "orc_index_scores_bf16");
    for (int k : {1, 7, 64}) {
      std::vector<int32_t> idx(k);
      expect_ok(orc_topk(n, S.data(), k, idx.data()), "orc_topk");
    }
  }
  // plain attention, empty key list included
  for (int64_t n : {0, 1, 9}) {
    std::vector<double> q(16), keys((size_t)(n * 8 + 1)), vals((size_t)(n * 8 + 1)), out(16), lse(2);
    for (auto& v : q) v = small_float();
    for (auto& v : keys) v = small_float();
    for (auto& v : vals) v = small_float();
    expect_ok(orc_attend(2, 8, 0.5, q.data(), n, keys.data(), vals.data(), out.data(), lse.data()), "orc_attend");
  }
  run_dtype(0);
  run_dtype(1);
  std::printf("sanitize_check: %d failures (checksum %g)\n", failures, acc);
  return failures == 0 ? 0 : 1;
}

// Host-side sanitizer driver for libcsa's C ABI (test infrastructure).
//
// Linked against the library's objects built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host side only, it calls every entry
// point on a machine without a GPU: invalid arguments (each rejected by the
// host validation), valid ones (which get as far as the device check), and
// the workspace queries over extreme shapes (up to 2^30 pooled entries,
// 4096-way top-k, 2^24 queries), so the planning arithmetic runs under the
// overflow checks.  A sanitizer report or an unexpected status fails the run.
// Built and run by tests/test_abi_host_sanitizers.py.
#include <cstdint>
#include <cstdio>

#include "../include/csa.h"

static int failures = 0;
static void expect(bool ok, const char* what, int rc) {
  if (!ok) {
    std::fprintf(stderr, "%s: unexpected status %d (%s)\n", what, rc, csa_last_error());
    ++failures;
  }
}

int main() {
  // fake device pointers: never dereferenced (validation or the device check stops first)
  int64_t* P = reinterpret_cast<int64_t*>(0x10000);
  void* V = reinterpret_cast<void*>(0x10000);
  uint8_t* U = reinterpret_cast<uint8_t*>(0x10000);
  float* F = reinterpret_cast<float*>(0x10000);
  int32_t* I = reinterpret_cast<int32_t*>(0x10000);
  for (int s = -6; s <= 1; ++s) (void)csa_status_string(s);
  uint64_t viol = 0;
  int rc = csa_debug_checks(&viol);
  expect(rc == CSA_ERR_UNSUPPORTED || rc == CSA_ERR_DEVICE || rc == CSA_OK, "csa_debug_checks", rc);
  rc = csa_debug_checks(nullptr);
  expect(rc == CSA_ERR_INVALID, "csa_debug_checks(NULL)", rc);

  // workspace queries over extreme shapes: must not overflow
  const int64_t nqs[] = {1, 64, 4096, 1 << 24};
  const int64_t pools[] = {0, 1, 262144, (int64_t)1 << 30};
  for (int64_t nq : nqs) {
    for (int64_t maxq : {(int64_t)1, (int64_t)16, nq}) {
      if (maxq > nq) continue;
      csa_batch b{(int32_t)((nq + maxq - 1) / maxq), nq, (int64_t)1 << 30, maxq, P, P, P};
      for (int64_t mp : pools) {
        for (int k : {1, 1024, 4096, 4097}) {
          size_t n = 0;
          rc = csa_index_topk_workspace(&b, mp, k, &n);
          expect(rc == CSA_OK || rc == CSA_ERR_INVALID || rc == CSA_ERR_UNSUPPORTED, "index workspace", rc);
          rc = csa_hca_decode_workspace(&b, mp, mp / 32, 64, 128, k, 128, 0, &n);
          expect(rc <= 0, "decode workspace", rc);
        }
        size_t n = 0;
        rc = hca_attn_workspace(CSA_BF16, &b, mp, 64, 128, 128, &n);
        expect(rc == CSA_OK || rc == CSA_ERR_INVALID, "hca workspace", rc);
      }
      for (int k : {0, 64, 4096}) {
        size_t n = 0;
        rc = csa_sparse_attn_workspace(CSA_BF16, &b, 64, 128, 128, k, &n);
        expect(rc == CSA_OK, "sparse workspace", rc);
        rc = csa_sparse_attn_workspace(CSA_F32, &b, 24, 128, 0, k, &n);
        expect(rc == CSA_OK, "sparse workspace f32", rc);
      }
    }
  }

  // every entry point: an invalid call, then a valid one (no device here)
  csa_batch b{2, 2, 4096, 1, P, P, P};
  const size_t big = (size_t)1 << 40;
  rc = csa_compress(CSA_BF16, 1, P, P, 16, 0, 256, V, V, V, nullptr);
  expect(rc == CSA_ERR_INVALID, "compress m=0", rc);
  rc = csa_compress(CSA_BF16, 1, P, P, 16, 4, 256, V, V, V, nullptr);
  expect(rc == CSA_ERR_DEVICE, "compress", rc);
  rc = csa_cache_append(CSA_BF16, 1, 256, P, P, P, 1, V, V, V, V, 2, P, 4, V, P, 128, V, nullptr, nullptr, 0, nullptr,
                        nullptr, nullptr);
  expect(rc == CSA_ERR_INVALID, "append ring < m_hca", rc);
  rc = csa_cache_append(CSA_BF16, 1, 256, P, P, P, 1, V, V, V, V, 128, P, 4, V, P, 128, V, P, V, 64, U, U, nullptr);
  expect(rc == CSA_ERR_DEVICE, "append", rc);
  rc = csa_mxfp4_quantize(CSA_F32, 8, 48, V, U, U, nullptr);
  expect(rc == CSA_ERR_INVALID || rc == CSA_ERR_UNSUPPORTED, "quantize dim 48", rc);
  rc = csa_mxfp4_quantize(CSA_F32, 8, 64, V, U, U, nullptr);
  expect(rc == CSA_ERR_DEVICE, "quantize", rc);
  rc = csa_index_topk(&b, P, 1000, 4, 8, 64, 64, U, U, F, U, U, I, V, big, nullptr);
  expect(rc == CSA_ERR_UNSUPPORTED, "index 8 heads", rc);
  rc = csa_index_topk(&b, P, 1000, 4, 4, 64, 64, U, U, F, U, U, I, V, big, nullptr);
  expect(rc == CSA_ERR_DEVICE, "index", rc);
  rc = csa_index_topk_bf16(&b, P, 1000, 4, 4, 64, 0, V, F, V, I, V, big, nullptr);
  expect(rc == CSA_ERR_INVALID, "index bf16 k=0", rc);
  rc = csa_index_topk_bf16(&b, P, 1000, 4, 4, 64, 64, V, F, V, I, V, big, nullptr);
  expect(rc == CSA_ERR_DEVICE, "index bf16", rc);
  rc = csa_sparse_attn(CSA_BF16, &b, P, 24, 128, 0.1f, 128, 64, V, V, V, I, V, F, V, big, nullptr);
  expect(rc == CSA_ERR_UNSUPPORTED, "sparse H=24 bf16", rc);
  rc = csa_sparse_attn(CSA_BF16, &b, P, 64, 128, 0.1f, 128, 64, V, V, V, I, V, F, V, big, nullptr);
  expect(rc == CSA_ERR_DEVICE, "sparse", rc);
  rc = hca_attn(CSA_BF16, &b, P, 512, 0, 64, 128, 0.1f, 0, V, V, V, V, F, V, big, nullptr);
  expect(rc == CSA_ERR_INVALID, "hca m'=0", rc);
  rc = hca_attn(CSA_BF16, &b, P, 512, 128, 64, 128, 0.1f, 0, V, V, V, V, F, V, big, nullptr);
  expect(rc == CSA_ERR_DEVICE, "hca", rc);
  rc = csa_hca_decode(&b, P, 262144, P, 8192, 4, 128, 64, 128, 0.1f, 2048, 128, 0, U, U, F, U, U, V, V, V, V, I, V,
                      F, V, F, V, big, nullptr);
  expect(rc == CSA_ERR_UNSUPPORTED || rc == CSA_ERR_DEVICE, "decode k=2048", rc);  // sizing needs the device
  rc = csa_hca_decode(&b, P, 262144, P, 8192, 4, 128, 64, 128, 0.1f, 1024, 128, 0, U, U, F, U, U, V, V, V, V, I, V,
                      F, V, F, V, big, nullptr);
  expect(rc == CSA_ERR_DEVICE, "decode", rc);
  rc = csa_hca_decode_noalloc(&b, P, 262144, P, 8192, 4, 128, 64, 128, 0.1f, 1024, 128, 0, U, U, F, U, U, V, V, V, V,
                              I, V, F, V, F, nullptr);
  expect(rc == CSA_ERR_DEVICE, "decode noalloc", rc);
  rc = csa_hca_decode_shared(&b, I, P, P, 262144, P, 8192, 4, 128, 64, 128, 0.1f, 1024, 128, 0, U, U, F, U, U, V, V,
                             V, V, I, V, F, V, F, V, big, nullptr);
  expect(rc == CSA_ERR_DEVICE, "decode shared", rc);
  rc = csa_hca_decode_paged(&b, 100, I, 64, P, 64, I, 64, P, 262144, 8192, 4, 128, 64, 128, 0.1f, 1024, 128, 0, U, U,
                            F, U, U, V, V, V, V, I, V, F, V, F, V, big, nullptr);
  expect(rc == CSA_ERR_INVALID, "decode paged page_rows=100", rc);
  rc = csa_hca_decode_paged(&b, 256, I, 1024, P, 64, I, 128, P, 262144, 8192, 4, 128, 64, 128, 0.1f, 1024, 128, 0, U,
                            U, F, U, U, V, V, V, V, I, V, F, V, F, V, big, nullptr);
  expect(rc == CSA_ERR_DEVICE, "decode paged", rc);
  uint32_t rows = 0;
  rc = csa_hca_decode_fallbacks(nullptr, nullptr, &rows);
  expect(rc == CSA_ERR_INVALID, "fallbacks NULL", rc);
  rc = csa_hca_decode_check(nullptr, nullptr, nullptr);
  expect(rc == CSA_ERR_INVALID, "check NULL", rc);
  rc = csa_profile_events(99, nullptr, nullptr);
  expect(rc == CSA_ERR_INVALID, "profile id 99", rc);
  rc = csa_profile_events(0, nullptr, nullptr);
  expect(rc == CSA_OK, "profile clear", rc);
  std::printf("abi_host_sanitize: %d failures\n", failures);
  return failures == 0 ? 0 : 1;
}

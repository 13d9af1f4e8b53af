// C ABI of libcsa: host-side validation, workspace sizing and launches.
// Declarations, argument meaning and error behaviour: include/csa.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/csa.h"
#include "kernels.hpp"

namespace {

thread_local char g_err[512] = "";
thread_local hipEvent_t g_prof[CSA_K_COUNT][2] = {};

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// 0 = unknown, 1 = gfx950, 2 = other / unusable
std::atomic<int> g_dev_state[64];

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fail(CSA_ERR_DEVICE, "no HIP device available");
  }
  if (dev < 64) {
    int s = g_dev_state[dev].load(std::memory_order_relaxed);
    if (s == 1) return CSA_OK;
    if (s == 2) return fail(CSA_ERR_DEVICE, "device %d is not gfx950", dev);
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return fail(CSA_ERR_DEVICE, "hipGetDeviceProperties failed on device %d", dev);
  }
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) g_dev_state[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  if (!ok) return fail(CSA_ERR_DEVICE, "device %d is %s, libcsa is built for gfx950", dev, prop.gcnArchName);
  return CSA_OK;
}

int check_batch(const csa_batch* b) {
  if (!b) return fail(CSA_ERR_INVALID, "batch descriptor is NULL");
  if (b->n_seq < 1) return fail(CSA_ERR_INVALID, "n_seq must be >= 1 (got %d)", b->n_seq);
  if (b->n_q < 0 || b->max_len < 0 || b->max_q_per_seq < 0)
    return fail(CSA_ERR_INVALID, "negative batch sizes");
  if (b->n_q > 0 && b->max_q_per_seq < 1)
    return fail(CSA_ERR_INVALID, "max_q_per_seq must be >= 1 when n_q > 0");
  if (b->n_q > (int64_t)b->n_seq * b->max_q_per_seq)
    return fail(CSA_ERR_INVALID, "n_q exceeds n_seq * max_q_per_seq");
  if (!b->tok_off || !b->q_off || (b->n_q > 0 && !b->q_pos))
    return fail(CSA_ERR_INVALID, "batch offset arrays must not be NULL");
  if (b->n_q > 0x7fffffffLL) return fail(CSA_ERR_UNSUPPORTED, "n_q too large");
  return CSA_OK;
}

int launched(int rc) {
  if (rc != 0) {
    (void)hipGetLastError();
    return fail(CSA_ERR_DEVICE, "kernel launch failed");
  }
  return CSA_OK;
}

}  // namespace

namespace csa {
hipEvent_t prof_event(int id, int stop) { return g_prof[id][stop ? 1 : 0]; }
}  // namespace csa

extern "C" {

int csa_hca_decode_workspace(const csa_batch* b, int64_t max_pool, int64_t max_hpool, int H, int d,
                             int k, int W, int W_hca, size_t* bytes) {
  int rc = check_batch(b);
  if (rc) return rc;
  if (!bytes || k < 1 || k > 4096 || W < 0 || W_hca < 0 || max_pool < 0 || max_hpool < 0)
    return fail(CSA_ERR_INVALID, "bytes NULL or k / W / W_hca / sizes out of range");
  rc = check_device();
  if (rc) return rc;
  if (d != 128 || !csa::fused_supported(b->n_q, max_pool, max_hpool, H, k, W, W_hca))
    return fail(CSA_ERR_UNSUPPORTED, "fused decode needs d = 128, 16 <= H <= 64 with H %% 16 == 0, k <= 1024, "
                                     "max_pool <= 262144 and 1..64 queries");
  *bytes = csa::plan_fused(b->n_q, max_pool, max_hpool, H, k, W, W_hca).ws_bytes;
  return CSA_OK;
}

static int hca_decode_impl(const csa_batch* b, const int32_t* pre_seq, const int64_t* pre_tok,
                           const csa::FusedPaging* paging,
                           const int64_t* pool_off, int64_t max_pool, const int64_t* hpool_off, int64_t max_hpool,
                           int m, int m_hca, int H, int d, float scale, int k, int W, int W_hca,
                           const uint8_t* q_codes, const uint8_t* q_scales, const float* w, const uint8_t* k_codes,
                           const uint8_t* k_scales, const void* q, const void* kv_pool, const void* kv_pool_hca,
                           const void* kv_raw, int32_t* idx, void* csa_out, float* csa_lse, void* hca_out,
                           float* hca_lse, void* ws, size_t ws_bytes, void* stream, bool noalloc = false) {
  int rc = check_batch(b);
  if (rc) return rc;
  if (b->n_q != b->n_seq || b->max_q_per_seq != 1)
    return fail(CSA_ERR_UNSUPPORTED, "fused decode needs exactly one query per sequence");
  if (m < 1 || m_hca < 1) return fail(CSA_ERR_INVALID, "block sizes must be >= 1");
  if (k < 1 || k > 4096 || W < 0 || W_hca < 0) return fail(CSA_ERR_INVALID, "k / W / W_hca out of range");
  if (max_pool < 0 || max_hpool < 0 || max_hpool > 0x7fffffffLL) return fail(CSA_ERR_INVALID, "sizes out of range");
  rc = check_device();
  if (rc) return rc;
  if (d != 128 || !csa::fused_supported(b->n_q, max_pool, max_hpool, H, k, W, W_hca))
    return fail(CSA_ERR_UNSUPPORTED, "fused decode needs d = 128, 16 <= H <= 64 with H %% 16 == 0, k <= 1024, "
                                     "max_pool <= 262144 and 1..64 queries");
  if ((!paging && (!pool_off || !hpool_off)) || !q_codes || !q_scales || !w || !k_codes || !k_scales || !q || !kv_pool ||
      (max_hpool > 0 && !kv_pool_hca) || ((W > 0 || W_hca > 0) && !kv_raw) || !idx || !csa_out || !hca_out)
    return fail(CSA_ERR_INVALID, "NULL pointer argument");
  if (!aligned16(q_codes) || !aligned16(k_codes) || !aligned16(q) || !aligned16(kv_pool) ||
      !aligned16(kv_pool_hca) || !aligned16(kv_raw) || !aligned16(csa_out) || !aligned16(hca_out))
    return fail(CSA_ERR_INVALID, "codes, q, caches and outputs must be 16-byte aligned");
  if (noalloc) {  // the library's static scratch (cleared here when the layout changes)
    const char* err = "";
    rc = csa::noalloc_prepare((int)b->n_q, max_pool, max_hpool, H, k, W, W_hca, (hipStream_t)stream, &ws, &ws_bytes,
                              &err);
    if (rc) return fail(rc, "%s", err);
  }
  const size_t need = csa::plan_fused(b->n_q, max_pool, max_hpool, H, k, W, W_hca).ws_bytes;
  if (!ws || ws_bytes < need)
    return fail(CSA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  if (csa::launch_fused((int)b->n_q, b->tok_off, b->q_pos, pool_off, hpool_off, pre_seq, pre_tok, paging, max_pool,
                        max_hpool, m, m_hca, H,
                        scale, k, W, W_hca, q_codes, q_scales, w, k_codes, k_scales, q, kv_pool, kv_pool_hca,
                        kv_raw, idx, csa_out, csa_lse, hca_out, hca_lse, ws, (hipStream_t)stream) != 0) {
    (void)hipGetLastError();
    return fail(CSA_ERR_DEVICE, "launch of the fused decode kernel failed");
  }
  return CSA_OK;
}

int csa_hca_decode(const csa_batch* b, const int64_t* pool_off, int64_t max_pool,
                   const int64_t* hpool_off, int64_t max_hpool, int m, int m_hca, int H, int d,
                   float scale, int k, int W, int W_hca, const uint8_t* q_codes,
                   const uint8_t* q_scales, const float* w, const uint8_t* k_codes,
                   const uint8_t* k_scales, const void* q, const void* kv_pool,
                   const void* kv_pool_hca, const void* kv_raw, int32_t* idx, void* csa_out,
                   float* csa_lse, void* hca_out, float* hca_lse, void* ws, size_t ws_bytes,
                   void* stream) {
  return hca_decode_impl(b, nullptr, nullptr, nullptr, pool_off, max_pool, hpool_off, max_hpool, m, m_hca, H, d, scale, k, W,
                         W_hca, q_codes, q_scales, w, k_codes, k_scales, q, kv_pool, kv_pool_hca, kv_raw, idx,
                         csa_out, csa_lse, hca_out, hca_lse, ws, ws_bytes, stream);
}

int csa_hca_decode_noalloc(const csa_batch* b, const int64_t* pool_off, int64_t max_pool,
                           const int64_t* hpool_off, int64_t max_hpool, int m, int m_hca, int H, int d,
                           float scale, int k, int W, int W_hca, const uint8_t* q_codes,
                           const uint8_t* q_scales, const float* w, const uint8_t* k_codes,
                           const uint8_t* k_scales, const void* q, const void* kv_pool,
                           const void* kv_pool_hca, const void* kv_raw, int32_t* idx, void* csa_out,
                           float* csa_lse, void* hca_out, float* hca_lse, void* stream) {
  return hca_decode_impl(b, nullptr, nullptr, nullptr, pool_off, max_pool, hpool_off, max_hpool, m, m_hca, H, d, scale, k,
                         W, W_hca, q_codes, q_scales, w, k_codes, k_scales, q, kv_pool, kv_pool_hca, kv_raw, idx,
                         csa_out, csa_lse, hca_out, hca_lse, nullptr, 0, stream, true);
}

int csa_hca_decode_shared(const csa_batch* b, const int32_t* prefix_seq, const int64_t* prefix_tokens,
                          const int64_t* pool_off, int64_t max_pool, const int64_t* hpool_off, int64_t max_hpool,
                          int m, int m_hca, int H, int d, float scale, int k, int W, int W_hca,
                          const uint8_t* q_codes, const uint8_t* q_scales, const float* w,
                          const uint8_t* k_codes, const uint8_t* k_scales, const void* q, const void* kv_pool,
                          const void* kv_pool_hca, const void* kv_raw, int32_t* idx, void* csa_out,
                          float* csa_lse, void* hca_out, float* hca_lse, void* ws, size_t ws_bytes,
                          void* stream) {
  if (!prefix_seq || !prefix_tokens) return fail(CSA_ERR_INVALID, "NULL prefix array");
  return hca_decode_impl(b, prefix_seq, prefix_tokens, nullptr, pool_off, max_pool, hpool_off, max_hpool, m, m_hca, H, d,
                         scale, k, W, W_hca, q_codes, q_scales, w, k_codes, k_scales, q, kv_pool, kv_pool_hca,
                         kv_raw, idx, csa_out, csa_lse, hca_out, hca_lse, ws, ws_bytes, stream);
}

int csa_hca_decode_paged(const csa_batch* b, int page_rows, const int32_t* page_table, int max_pages,
                         const int64_t* pooled_rows, int hca_page_rows, const int32_t* hca_page_table,
                         int max_hca_pages, const int64_t* hca_pooled_rows, int64_t max_pool, int64_t max_hpool,
                         int m, int m_hca, int H, int d, float scale, int k, int W, int W_hca,
                         const uint8_t* q_codes, const uint8_t* q_scales, const float* w,
                         const uint8_t* k_codes, const uint8_t* k_scales, const void* q, const void* kv_pool,
                         const void* kv_pool_hca, const void* kv_raw, int32_t* idx, void* csa_out,
                         float* csa_lse, void* hca_out, float* hca_lse, void* ws, size_t ws_bytes,
                         void* stream) {
  if (!page_table || !pooled_rows || !hca_page_table || !hca_pooled_rows)
    return fail(CSA_ERR_INVALID, "NULL page table or pooled-row count");
  auto pow2 = [](int v) { return v >= 32 && (v & (v - 1)) == 0; };
  if (!pow2(page_rows) || !pow2(hca_page_rows))
    return fail(CSA_ERR_INVALID, "page sizes must be powers of two of at least 32 rows");
  if (max_pages < 1 || max_hca_pages < 1) return fail(CSA_ERR_INVALID, "page tables need at least one column");
  if ((int64_t)max_pages * page_rows < max_pool || (int64_t)max_hca_pages * hca_page_rows < max_hpool)
    return fail(CSA_ERR_INVALID, "the page tables map fewer rows than max_pool / max_hpool");
  const csa::FusedPaging pg{page_table, pooled_rows, max_pages, page_rows,
                            hca_page_table, hca_pooled_rows, max_hca_pages, hca_page_rows};
  return hca_decode_impl(b, nullptr, nullptr, &pg, nullptr, max_pool, nullptr, max_hpool, m, m_hca, H, d, scale, k, W,
                         W_hca, q_codes, q_scales, w, k_codes, k_scales, q, kv_pool, kv_pool_hca, kv_raw, idx,
                         csa_out, csa_lse, hca_out, hca_lse, ws, ws_bytes, stream);
}

int csa_hca_decode_check(const csa_batch* b, const void* ws, void* stream) {
  int rc = check_batch(b);
  if (rc) return rc;
  if (!ws) return fail(CSA_ERR_INVALID, "ws is NULL");
  rc = check_device();
  if (rc) return rc;
  // the error word sits among the control words at the start of the workspace
  uint32_t* errp = (uint32_t*)((uint8_t*)ws + csa::fused_error_word_offset());
  uint32_t ctl[4] = {0, 0, 0, 0};  // epoch, exit count, error word, work counter
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess ||
      hipMemcpy(ctl, ws, sizeof(ctl), hipMemcpyDeviceToHost) != hipSuccess) {
    (void)hipGetLastError();
    return fail(CSA_ERR_DEVICE, "could not read the decode status word");
  }
  if (ctl[2]) {
    const uint32_t zero = 0;
    (void)hipMemcpy(errp, &zero, 4, hipMemcpyHostToDevice);
    return fail(CSA_ERR_DEVICE,
                "a fused decode launch hit its internal wait bound (code 0x%x; epoch %u, exit %u, work %u); its outputs "
                "are invalid",
                ctl[2], ctl[0], ctl[1], ctl[3]);
  }
  return CSA_OK;
}

int csa_hca_decode_fallbacks(const void* ws, void* stream, uint32_t* rows) {
  if (!ws || !rows) return fail(CSA_ERR_INVALID, "ws and rows must not be NULL");
  int rc = check_device();
  if (rc) return rc;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess ||
      hipMemcpy(rows, (const uint8_t*)ws + csa::fused_fallback_word_offset(), 4, hipMemcpyDeviceToHost) !=
          hipSuccess) {
    (void)hipGetLastError();
    return fail(CSA_ERR_DEVICE, "could not read the decode fallback count");
  }
  return CSA_OK;
}

int csa_profile_events(int kernel_id, void* start, void* stop) {
  if (kernel_id < 0 || kernel_id >= CSA_K_COUNT) return fail(CSA_ERR_INVALID, "unknown kernel id %d", kernel_id);
  if ((start == nullptr) != (stop == nullptr)) return fail(CSA_ERR_INVALID, "pass both events or neither");
  g_prof[kernel_id][0] = (hipEvent_t)start;
  g_prof[kernel_id][1] = (hipEvent_t)stop;
  return CSA_OK;
}


const char* csa_status_string(int status) {
  switch (status) {
    case CSA_OK: return "CSA_OK";
    case CSA_ERR_INVALID: return "CSA_ERR_INVALID: invalid argument";
    case CSA_ERR_UNSUPPORTED: return "CSA_ERR_UNSUPPORTED: unsupported shape or dtype";
    case CSA_ERR_WORKSPACE: return "CSA_ERR_WORKSPACE: workspace missing or too small";
    case CSA_ERR_DEVICE: return "CSA_ERR_DEVICE: no usable gfx950 device or launch failure";
    default: return "unknown csa status";
  }
}

const char* csa_last_error(void) { return g_err; }

int csa_debug_checks(uint64_t* violations) {
  if (!violations) return fail(CSA_ERR_INVALID, "violations must not be NULL");
#ifdef CSA_DEBUG
  const unsigned long long a = csa::debug_take_attn(), f = csa::debug_take_fused();
  if (a == ~0ull || f == ~0ull) return fail(CSA_ERR_DEVICE, "could not read the debug counters");
  *violations = (uint64_t)(a + f);
  return CSA_OK;
#else
  *violations = 0;
  return fail(CSA_ERR_UNSUPPORTED, "a release build: no device-side checks compiled (build with --debug)");
#endif
}

int csa_compress(int dtype, int32_t n_seq, const int64_t* tok_off, const int64_t* pool_off,
                 int64_t max_len, int m, int width, const void* x, const void* z, void* out,
                 void* stream) {
  if (dtype != CSA_F32 && dtype != CSA_BF16) return fail(CSA_ERR_UNSUPPORTED, "dtype %d", dtype);
  if (n_seq < 1) return fail(CSA_ERR_INVALID, "n_seq must be >= 1");
  if (!tok_off || !pool_off || !x || !z || !out) return fail(CSA_ERR_INVALID, "NULL pointer argument");
  if (m < 1) return fail(CSA_ERR_INVALID, "block size m must be >= 1 (got %d)", m);
  if (width < 1 || width % 8 != 0) return fail(CSA_ERR_INVALID, "width must be a positive multiple of 8");
  if (max_len < 0) return fail(CSA_ERR_INVALID, "max_len must be >= 0");
  if (!aligned16(x) || !aligned16(z) || !aligned16(out))
    return fail(CSA_ERR_INVALID, "x, z and out must be 16-byte aligned");
  int rc = check_device();
  if (rc) return rc;
  return launched(csa::launch_compress(dtype == CSA_BF16, n_seq, tok_off, pool_off, max_len, m,
                                       width, x, z, out, (hipStream_t)stream));
}

int csa_cache_append(int dtype, int32_t n_seq, int width, const int64_t* tok_off, int64_t* len,
                     const int64_t* new_off, int64_t max_new, const void* x_new, const void* z_new, void* kv_raw,
                     void* z_tail, int ring, const int64_t* pool_off, int m, void* pooled,
                     const int64_t* hpool_off, int m_hca, void* hpooled, const int64_t* kvec_off, const void* kvec,
                     int kdim, uint8_t* k_codes, uint8_t* k_scales, void* stream) {
  if (dtype != CSA_F32 && dtype != CSA_BF16) return fail(CSA_ERR_UNSUPPORTED, "dtype %d", dtype);
  if (n_seq < 1) return fail(CSA_ERR_INVALID, "n_seq must be >= 1");
  if (width < 1 || width % 8 != 0) return fail(CSA_ERR_INVALID, "width must be a positive multiple of 8");
  if (m < 1) return fail(CSA_ERR_INVALID, "block size m must be >= 1 (got %d)", m);
  if (m_hca < 0) return fail(CSA_ERR_INVALID, "m_hca must be >= 0 (got %d)", m_hca);
  if (max_new < 0) return fail(CSA_ERR_INVALID, "max_new must be >= 0");
  if (ring < m || ring < m_hca)
    return fail(CSA_ERR_INVALID, "ring (%d) must be >= m (%d) and >= m_hca (%d)", ring, m, m_hca);
  if (!tok_off || !len || !new_off || !x_new || !z_new || !kv_raw || !z_tail || !pool_off || !pooled)
    return fail(CSA_ERR_INVALID, "NULL pointer argument");
  if (m_hca > 0 && (!hpool_off || !hpooled)) return fail(CSA_ERR_INVALID, "m_hca > 0 needs hpool_off and hpooled");
  if (!aligned16(x_new) || !aligned16(z_new) || !aligned16(kv_raw) || !aligned16(z_tail) || !aligned16(pooled) ||
      (m_hca > 0 && !aligned16(hpooled)))
    return fail(CSA_ERR_INVALID, "row buffers must be 16-byte aligned");
  if (kvec) {
    if (!kvec_off || !k_codes || !k_scales) return fail(CSA_ERR_INVALID, "kvec needs kvec_off, k_codes and k_scales");
    if (kdim < 32 || kdim % 32 != 0) return fail(CSA_ERR_INVALID, "kdim must be a positive multiple of 32 (got %d)", kdim);
    if (!aligned16(kvec) || !aligned16(k_codes)) return fail(CSA_ERR_INVALID, "kvec and k_codes must be 16-byte aligned");
  }
  if (max_new == 0) return CSA_OK;
  int rc = check_device();
  if (rc) return rc;
  return launched(csa::launch_append(dtype == CSA_BF16, n_seq, width, tok_off, len, new_off, max_new, x_new, z_new,
                                     kv_raw, z_tail, ring, pool_off, m, pooled, hpool_off, m_hca, hpooled, kvec_off,
                                     kvec, kvec ? kdim : 0, k_codes, k_scales, (hipStream_t)stream));
}

int csa_mxfp4_quantize(int dtype, int64_t rows, int dim, const void* x, uint8_t* codes, uint8_t* scales,
                       void* stream) {
  if (dtype != CSA_F32 && dtype != CSA_BF16) return fail(CSA_ERR_UNSUPPORTED, "dtype %d", dtype);
  if (rows < 0) return fail(CSA_ERR_INVALID, "rows must be >= 0");
  if (dim < 32 || dim % 32 != 0) return fail(CSA_ERR_INVALID, "dim must be a positive multiple of 32 (got %d)", dim);
  if (!x || !codes || !scales) return fail(CSA_ERR_INVALID, "NULL pointer argument");
  if (!aligned16(x) || !aligned16(codes)) return fail(CSA_ERR_INVALID, "x and codes must be 16-byte aligned");
  if (rows == 0) return CSA_OK;
  int rc = check_device();
  if (rc) return rc;
  return launched(csa::launch_mxfp4_quant(dtype == CSA_BF16, rows, dim, x, codes, scales, (hipStream_t)stream));
}

int csa_index_topk_workspace(const csa_batch* b, int64_t max_pool, int k, size_t* bytes) {
  int rc = check_batch(b);
  if (rc) return rc;
  if (!bytes) return fail(CSA_ERR_INVALID, "bytes is NULL");
  if (max_pool < 0) return fail(CSA_ERR_INVALID, "max_pool must be >= 0");
  if (k < 1 || k > 4096) return fail(CSA_ERR_INVALID, "k must be in [1, 4096] (got %d)", k);
  *bytes = csa::index_ws_bytes(b->n_q, b->max_q_per_seq, max_pool, k);
  return CSA_OK;
}

int csa_index_topk(const csa_batch* b, const int64_t* pool_off, int64_t max_pool, int m,
                   int n_heads, int dim, int k, const uint8_t* q_codes, const uint8_t* q_scales,
                   const float* w, const uint8_t* k_codes, const uint8_t* k_scales, int32_t* idx,
                   void* ws, size_t ws_bytes, void* stream) {
  int rc = check_batch(b);
  if (rc) return rc;
  if (n_heads != 4 || dim != 64)
    return fail(CSA_ERR_UNSUPPORTED, "indexer shape %d heads x %d dims (supported: 4 x 64)", n_heads, dim);
  if (m < 1) return fail(CSA_ERR_INVALID, "block size m must be >= 1");
  if (k < 1 || k > 4096) return fail(CSA_ERR_INVALID, "k must be in [1, 4096] (got %d)", k);
  if (max_pool < 0 || max_pool > (1LL << 30)) return fail(CSA_ERR_INVALID, "max_pool out of range");
  if (!pool_off || !q_codes || !q_scales || !w || !k_codes || !k_scales || !idx)
    return fail(CSA_ERR_INVALID, "NULL pointer argument");
  if (!aligned16(q_codes) || !aligned16(k_codes))
    return fail(CSA_ERR_INVALID, "q_codes and k_codes must be 16-byte aligned");
  const size_t need = csa::index_ws_bytes(b->n_q, b->max_q_per_seq, max_pool, k);
  if (!ws || ws_bytes < need)
    return fail(CSA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  rc = check_device();
  if (rc) return rc;
  return launched(csa::launch_index_topk(b->n_seq, b->n_q, b->max_q_per_seq, b->q_off, b->q_pos,
                                         pool_off, max_pool, m, k, q_codes, q_scales, w, k_codes,
                                         k_scales, idx, ws, (hipStream_t)stream));
}

int csa_index_topk_bf16(const csa_batch* b, const int64_t* pool_off, int64_t max_pool, int m, int n_heads, int dim,
                        int k, const void* q, const float* w, const void* keys, int32_t* idx, void* ws,
                        size_t ws_bytes, void* stream) {
  int rc = check_batch(b);
  if (rc) return rc;
  if (n_heads != 4 || dim != 64)
    return fail(CSA_ERR_UNSUPPORTED, "indexer shape %d heads x %d dims (supported: 4 x 64)", n_heads, dim);
  if (csa::prefill_path(b->max_q_per_seq))
    return fail(CSA_ERR_UNSUPPORTED, "the bf16 indexer takes decode batches only (max_q_per_seq < 16)");
  if (m < 1) return fail(CSA_ERR_INVALID, "block size m must be >= 1");
  if (k < 1 || k > 4096) return fail(CSA_ERR_INVALID, "k must be in [1, 4096] (got %d)", k);
  if (max_pool < 0 || max_pool > (1LL << 30)) return fail(CSA_ERR_INVALID, "max_pool out of range");
  if (!pool_off || !q || !w || !keys || !idx) return fail(CSA_ERR_INVALID, "NULL pointer argument");
  if (!aligned16(q) || !aligned16(keys)) return fail(CSA_ERR_INVALID, "q and keys must be 16-byte aligned");
  const size_t need = csa::index_ws_bytes(b->n_q, b->max_q_per_seq, max_pool, k);
  if (!ws || ws_bytes < need)
    return fail(CSA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  rc = check_device();
  if (rc) return rc;
  return launched(csa::launch_index_topk_bf16(b->n_seq, b->n_q, b->max_q_per_seq, b->q_off, b->q_pos, pool_off,
                                              max_pool, m, k, (const uint16_t*)q, w, (const uint16_t*)keys, idx, ws,
                                              (hipStream_t)stream));
}

static int check_attn_shape(int dtype, int H, int d) {
  if (dtype != CSA_F32 && dtype != CSA_BF16) return fail(CSA_ERR_UNSUPPORTED, "dtype %d", dtype);
  if (d != 128) return fail(CSA_ERR_UNSUPPORTED, "head dim %d (supported: 128)", d);
  if (H < 1 || H > 128) return fail(CSA_ERR_UNSUPPORTED, "H = %d (supported: 1..128)", H);
  if (dtype == CSA_BF16 && H % 16 != 0) return fail(CSA_ERR_UNSUPPORTED, "bf16 needs H %% 16 == 0");
  return CSA_OK;
}

int csa_sparse_attn_workspace(int dtype, const csa_batch* b, int H, int d, int W, int k,
                              size_t* bytes) {
  int rc = check_batch(b);
  if (rc) return rc;
  rc = check_attn_shape(dtype, H, d);
  if (rc) return rc;
  if (!bytes || W < 0 || k < 0) return fail(CSA_ERR_INVALID, "bytes NULL or negative W/k");
  *bytes = csa::plan_attn(b->n_q, (int64_t)k + W, H).ws_bytes;
  return CSA_OK;
}

int csa_sparse_attn(int dtype, const csa_batch* b, const int64_t* pool_off, int H, int d,
                    float scale, int W, int k, const void* q, const void* kv_pool,
                    const void* kv_raw, const int32_t* idx, void* out, float* lse, void* ws,
                    size_t ws_bytes, void* stream) {
  int rc = check_batch(b);
  if (rc) return rc;
  rc = check_attn_shape(dtype, H, d);
  if (rc) return rc;
  if (W < 0 || k < 0) return fail(CSA_ERR_INVALID, "W and k must be >= 0");
  if (!pool_off || !q || !out || (k > 0 && (!kv_pool || !idx)) || (W > 0 && !kv_raw))
    return fail(CSA_ERR_INVALID, "NULL pointer argument");
  if (!aligned16(q) || !aligned16(kv_pool) || !aligned16(kv_raw) || !aligned16(out))
    return fail(CSA_ERR_INVALID, "q, kv_pool, kv_raw and out must be 16-byte aligned");
  const size_t need = csa::plan_attn(b->n_q, (int64_t)k + W, H).ws_bytes;
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(CSA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  rc = check_device();
  if (rc) return rc;
  return launched(csa::launch_attn(dtype == CSA_BF16, false, b->n_seq, b->n_q, b->tok_off, b->q_off,
                                   b->q_pos, pool_off, 1, k, W, H, scale, q, kv_pool, kv_raw, idx,
                                   out, lse, ws, (hipStream_t)stream));
}

int hca_attn_workspace(int dtype, const csa_batch* b, int64_t max_hpool, int H, int d, int W_hca,
                       size_t* bytes) {
  int rc = check_batch(b);
  if (rc) return rc;
  rc = check_attn_shape(dtype, H, d);
  if (rc) return rc;
  if (!bytes || W_hca < 0 || max_hpool < 0 || max_hpool > 0x7fffffffLL)
    return fail(CSA_ERR_INVALID, "bytes NULL or W_hca / max_hpool out of range");
  *bytes = csa::plan_attn(b->n_q, max_hpool + W_hca, H).ws_bytes;
  return CSA_OK;
}

int hca_attn(int dtype, const csa_batch* b, const int64_t* hpool_off, int64_t max_hpool,
             int m_hca, int H, int d, float scale, int W_hca, const void* q,
             const void* kv_pool_hca, const void* kv_raw, void* out, float* lse, void* ws,
             size_t ws_bytes, void* stream) {
  int rc = check_batch(b);
  if (rc) return rc;
  rc = check_attn_shape(dtype, H, d);
  if (rc) return rc;
  if (m_hca < 1) return fail(CSA_ERR_INVALID, "m_hca must be >= 1");
  if (W_hca < 0 || max_hpool < 0 || max_hpool > 0x7fffffffLL)
    return fail(CSA_ERR_INVALID, "W_hca / max_hpool out of range");
  if (!hpool_off || !q || !out || (max_hpool > 0 && !kv_pool_hca) || (W_hca > 0 && !kv_raw))
    return fail(CSA_ERR_INVALID, "NULL pointer argument");
  if (!aligned16(q) || !aligned16(kv_pool_hca) || !aligned16(kv_raw) || !aligned16(out))
    return fail(CSA_ERR_INVALID, "q, kv_pool_hca, kv_raw and out must be 16-byte aligned");
  const size_t need = csa::plan_attn(b->n_q, max_hpool + W_hca, H).ws_bytes;
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(CSA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  rc = check_device();
  if (rc) return rc;
  return launched(csa::launch_attn(dtype == CSA_BF16, true, b->n_seq, b->n_q, b->tok_off, b->q_off,
                                   b->q_pos, hpool_off, m_hca, (int)max_hpool, W_hca, H, scale, q,
                                   kv_pool_hca, kv_raw, nullptr, out, lse, ws, (hipStream_t)stream));
}

}  // extern "C"

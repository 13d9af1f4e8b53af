// Host-side launchers of the libcsa kernels (internal to the library).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa {

// Tracing hook: the caller's events for one internal kernel id (thread-local;
// null when none are set).  Every kernel is launched through launch() below:
// when the hook holds events for the launch's id they are handed to
// hipExtLaunchKernel, which attaches them to the dispatch itself, so they time
// the kernel's execution on the GPU (as a kernel trace does), not its enqueue;
// otherwise it is a plain hipLaunchKernel.  `mark` says which of the id's
// events a launch carries: the start for the first of several launches, the
// stop for the last, both for a single one.
hipEvent_t prof_event(int kernel_id, int stop);
enum { kProfNone = 0, kProfStart = 1, kProfStop = 2, kProfBoth = 3 };
template <class T>
struct launch_arg {
  using type = T;
};
template <typename... P>
inline hipError_t launch(int kernel_id, int mark, void (*k)(P...), dim3 grid, dim3 block, size_t lds,
                         hipStream_t stream, typename launch_arg<P>::type... args) {
  void* a[] = {(void*)&args..., nullptr};
  hipEvent_t e0 = (mark & kProfStart) ? prof_event(kernel_id, 0) : nullptr;
  hipEvent_t e1 = (mark & kProfStop) ? prof_event(kernel_id, 1) : nullptr;
  if (e0 || e1) return hipExtLaunchKernel((const void*)k, grid, block, a, lds, stream, e0, e1, 0);
  return hipLaunchKernel((const void*)k, grid, block, a, lds, stream);
}

int launch_compress(bool bf16, int n_seq, const int64_t* tok_off, const int64_t* pool_off,
                    int64_t max_len, int m, int width, const void* x, const void* z, void* out,
                    hipStream_t stream);

int launch_append(bool bf16, int n_seq, int width, const int64_t* tok_off, int64_t* len, const int64_t* new_off,
                  int64_t max_new, const void* x_new, const void* z_new, void* kv_raw, void* z_tail, int ring,
                  const int64_t* pool_off, int m, void* pooled, const int64_t* hpool_off, int m_hca, void* hpooled,
                  const int64_t* kvec_off, const void* kvec, int kdim, uint8_t* k_codes, uint8_t* k_scales,
                  hipStream_t stream);

int launch_mxfp4_quant(bool bf16, int64_t rows, int dim, const void* x, uint8_t* codes, uint8_t* scales,
                       hipStream_t stream);

size_t index_ws_bytes(int64_t n_q, int64_t max_q_per_seq, int64_t max_pool, int k);
int prefill_path(int64_t max_q_per_seq);
size_t prefill_ws_bytes(int64_t n_q, int64_t max_pool);
int launch_prefill_topk(int n_seq, int64_t n_q, int64_t max_q_per_seq, const int64_t* q_off,
                        const int64_t* q_pos, const int64_t* pool_off, int64_t max_pool, int m, int k,
                        const uint8_t* q_codes, const uint8_t* q_scales, const float* w,
                        const uint8_t* k_codes, const uint8_t* k_scales, int32_t* idx, void* ws,
                        hipStream_t stream);
int launch_index_topk(int n_seq, int64_t n_q, int64_t max_q_per_seq, const int64_t* q_off,
                      const int64_t* q_pos, const int64_t* pool_off, int64_t max_pool, int m,
                      int k, const uint8_t* q_codes, const uint8_t* q_scales, const float* w,
                      const uint8_t* k_codes, const uint8_t* k_scales, int32_t* idx, void* ws,
                      hipStream_t stream);

// decode batches only (max_q_per_seq below the prefill threshold); workspace as
// launch_index_topk's for such batches
int launch_index_topk_bf16(int n_seq, int64_t n_q, int64_t max_q_per_seq, const int64_t* q_off, const int64_t* q_pos,
                           const int64_t* pool_off, int64_t max_pool, int m, int k, const uint16_t* q, const float* w,
                           const uint16_t* keys, int32_t* idx, void* ws, hipStream_t stream);

struct AttnPlan {
  int splits;
  int ks;
  size_t ws_bytes;
};
AttnPlan plan_attn(int64_t n_q, int64_t list_len, int H);
int launch_attn(bool bf16, bool hca, int n_seq, int64_t n_q, const int64_t* tok_off,
                const int64_t* q_off, const int64_t* q_pos, const int64_t* pool_off, int m_pool,
                int seg_a, int W, int H, float scale, const void* q, const void* kv_pool,
                const void* kv_raw, const int32_t* idx, void* out, float* lse, void* ws,
                hipStream_t stream);

struct FusedPlan {
  int grid;                     // workgroups of the launch (CUs x workgroups per CU)
  int C, n_sc;                  // score entries per chunk, chunks per row
  int cs, n_cs_sel, n_cs_win;   // window split size; CSA groups and window splits per row
  int cg;                       // score chunks per CSA group
  int hs, n_hs;                 // HCA split size, splits per row
  int lst_min, lst;             // per score chunk: entries listed, at least lst_min, at most lst
  int hpm;                      // heads per merge unit
  int64_t key_stride;
  size_t ws_bytes;
};
FusedPlan plan_fused(int64_t R, int64_t max_pool, int64_t max_hpool, int H, int k, int W, int W_hca);
int fused_supported(int64_t R, int64_t max_pool, int64_t max_hpool, int H, int k, int W, int W_hca);
size_t fused_error_word_offset();
size_t fused_fallback_word_offset();
// paged pooled caches for the fused decode (page_rows / hpage_rows powers of two >= 32)
struct FusedPaging {
  const int32_t* ptab;
  const int64_t* plen;
  int max_pages, page_rows;
  const int32_t* hptab;
  const int64_t* hplen;
  int max_hpages, hpage_rows;
};
// the static scratch of the no-allocation decode entry point (noalloc.hip):
// its device address on the current device, cleared first when the layout
// differs from the last launch's on this device
int noalloc_prepare(int R, int64_t max_pool, int64_t max_hpool, int H, int k, int W, int W_hca, hipStream_t stream,
                    void** ws, size_t* ws_bytes, const char** err);
int launch_fused(int R, const int64_t* tok_off, const int64_t* q_pos, const int64_t* pool_off,
                 const int64_t* hpool_off, const int32_t* pre_seq, const int64_t* pre_tok, const FusedPaging* paging,
                 int64_t max_pool, int64_t max_hpool, int m, int m_hca, int H,
                 float scale, int k, int W, int W_hca, const uint8_t* q_codes, const uint8_t* q_scales,
                 const float* w, const uint8_t* k_codes, const uint8_t* k_scales, const void* q,
                 const void* kv_pool, const void* kv_hpool, const void* kv_raw, int32_t* idx, void* csa_out,
                 float* csa_lse, void* hca_out, float* hca_lse, void* ws, hipStream_t stream);

#ifdef CSA_DEBUG
// violations counted by the debug checks since the last call, cleared (synchronous)
unsigned long long debug_take_attn();
unsigned long long debug_take_fused();
#endif

}  // namespace csa

/*
 * csa.h — C ABI of libcsa.so: compressed sparse attention (CSA) and heavily
 * compressed attention (HCA) on AMD Instinct MI355X (gfx950).
 *
 * The method (pages on DeepSeek-V4):
 *  - discuss.pytorch.kr, "DeepSeek-V4 series" summary, CSA/HCA section: CSA
 *    compresses every m consecutive KV entries into one, lets each query
 *    attend only to its top-k compressed entries (DeepSeek Sparse Attention
 *    on the compressed sequence) and adds a sliding-window branch of recent
 *    tokens; HCA compresses m' >> m entries into one and attends densely to
 *    all of them, with no sparse selection.
 *  - same page, FP4 QAT section: the indexer's QK path is MXFP4.
 *  - sigco.tistory.com, "DeepSeek-V4 paper reading", CSA/HCA section: block
 *    compression, an indexer that finds the blocks relevant to the current
 *    token, attention over the top candidates, a sliding window of recent
 *    tokens; HCA attends to every compressed entry.  KV-cache section: the
 *    cache is split into compressed entries, the window, and the tail of
 *    tokens not yet numerous enough to form a block; a cache computed for a
 *    shared prefix is kept and reused by later requests over it.
 *  - jyp-garden EP 95 notes, IDEAS: multi-query attention (one shared KV head).
 *
 * Conventions for every entry point
 *  - Pointers are DEVICE pointers unless a comment says "host".  The caller
 *    owns all memory, including workspaces; the library allocates and frees
 *    nothing and keeps no pointer after a call returns.  Its only state is
 *    per-device caches (whether the device is a gfx950, workgroups resident
 *    per CU; computed once per device, race-free atomics), the profiling
 *    hook's events, and for csa_hca_decode_noalloc a static scratch array
 *    per device.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *    default stream).  The library never synchronises.  Calls on different
 *    streams may run concurrently if they do not share a workspace.
 *  - Return value: CSA_OK (0) or a negative csa_status.  Arguments are
 *    validated on the host before anything is enqueued; a rejected call
 *    enqueues nothing.  csa_last_error() returns a thread-local message for
 *    the last failed call on the calling thread.
 *  - Device data (offsets, positions, codes) is trusted: out-of-range values
 *    there are undefined behaviour, not reported errors.
 *  - Layouts: raw KV rows [sum L][2][d] (K half first, V half at element d);
 *    pooled rows [sum P][2][d] in the same layout; queries [n_q][H][d];
 *    outputs [n_q][H][d] in the KV dtype; lse [n_q][H] fp32.
 *  - Supported shapes: d = 128; H <= 128 (bf16 needs H % 16 == 0); indexer
 *    4 heads x 64 dims.  Everything else returns CSA_ERR_UNSUPPORTED.
 */
#ifndef CSA_H
#define CSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CSA_OK = 0,
  CSA_ERR_INVALID = -1,     /* null pointer, negative size, inconsistent arguments */
  CSA_ERR_UNSUPPORTED = -2, /* valid but not implemented (dtype, d, H, indexer shape) */
  CSA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than the queried size   */
  CSA_ERR_DEVICE = -4       /* no usable gfx950 device, or a HIP launch failed       */
} csa_status;

typedef enum { CSA_F32 = 0, CSA_BF16 = 1 } csa_dtype;

/* A batch of sequences and the query rows that belong to them.
 * Sequence b owns raw rows [tok_off[b], tok_off[b+1]) (length L_b) and query
 * rows [q_off[b], q_off[b+1]); query i sits at position q_pos[i] inside its
 * sequence, 0 <= q_pos[i] < L_b.  The host scalars bound the device arrays
 * and size the launch grids; they must be >= the true values. */
typedef struct {
  int32_t n_seq;            /* host: number of sequences B >= 1                  */
  int64_t n_q;              /* host: total query rows (= q_off[B])               */
  int64_t max_len;          /* host: max_b L_b                                   */
  int64_t max_q_per_seq;    /* host: max_b (q_off[b+1] - q_off[b])               */
  const int64_t* tok_off;   /* device [B+1]                                      */
  const int64_t* q_off;     /* device [B+1]                                      */
  const int64_t* q_pos;     /* device [n_q]                                      */
} csa_batch;

/* Status code -> static string (host; never fails). */
const char* csa_status_string(int status);

/* Thread-local description of the last failed call on this thread (host). */
const char* csa_last_error(void);

/* Debug builds only.  In a library compiled with CSA_DEBUG (libcsa_debug.so,
 * `python -m long_context_compressed_05_amd.build --debug`), the kernels check
 * device-side indices before using them (every CSA list index given to
 * csa_sparse_attn against its sequence's pooled rows; every row a fused
 * decode step's selection gathers against the query's visible entries) and
 * count each violation instead of reading out of range (the entry is then
 * treated as padding).  csa_debug_checks stores the count since the last
 * call in *violations and clears it; it synchronises the current device.
 * Errors: CSA_ERR_INVALID for a NULL pointer, CSA_ERR_UNSUPPORTED in a
 * release build (no checks compiled), CSA_ERR_DEVICE when the counters
 * cannot be read. */
int csa_debug_checks(uint64_t* violations);

/* ------------------------------------------------------------------------
 * csa_compress — pooling of m consecutive raw rows into one row.
 * Pages: pytorch.kr CSA/HCA section (m consecutive KV entries become one;
 * m' >> m for HCA); sigco CSA/HCA section (blockwise compression).  Rule
 * (the reading taken; the pages give none): for block j of sequence b and
 * channel c, out[j][c] = sum_i softmax_i(z[jm+i][c]) * x[jm+i][c], i < m,
 * computed in fp32 and rounded once to the KV dtype.
 *
 * Sequence b's rows [tok_off[b], tok_off[b+1]) are pooled in whole blocks of
 * m starting at tok_off[b] (the start must sit on a block boundary of the
 * sequence's absolute positions when appending a chunk); trailing rows that
 * do not fill a block are not pooled (they stay visible through the window).
 * Block j of sequence b is written to row pool_off[b] + j of `out`, for
 * j < min(floor(L_b/m), pool_off[b+1] - pool_off[b]).
 *   x, z      [sum L][width] in `dtype`  (width = 2d: the K and V channels
 *             each with their own logits)
 *   out       [sum P][width] in `dtype`
 * Errors: CSA_ERR_INVALID for null pointers, m < 1, width < 1 or not a
 * multiple of 8; CSA_ERR_UNSUPPORTED for other dtypes.
 * ---------------------------------------------------------------------- */
int csa_compress(int dtype, int32_t n_seq, const int64_t* tok_off, const int64_t* pool_off,
                 int64_t max_len, int m, int width, const void* x, const void* z, void* out,
                 void* stream);

/* ------------------------------------------------------------------------
 * csa_cache_append — streaming cache upkeep: append each sequence's new
 * tokens and pool every block the append completes.
 * Pages: sigco.tistory.com KV-cache section (the cache is split into the
 * compressed entries CSA/HCA read, the recent tokens the sliding window reads,
 * and the state of the tail tokens not yet numerous enough to compress);
 * pooling rule as csa_compress.  For sequence b with L = len[b] tokens cached
 * and n = new_off[b+1] - new_off[b] new ones:
 *   - raw row tok_off[b] + L + i <- x_new row new_off[b] + i   (i < n); the
 *     raw rows [tok_off[b], tok_off[b+1]) are the sequence's capacity and the
 *     window reads the last W of them;
 *   - every block j of m tokens with L < (j+1)*m <= L + n is pooled into
 *     pooled row pool_off[b] + j, and likewise every block of m_hca tokens
 *     into hpooled row hpool_off[b] + j (m_hca = 0: no HCA pooling); the rows
 *     are bit-identical to csa_compress over the whole sequence;
 *   - the tail state z_tail [n_seq][ring][width] keeps the pooling logits of
 *     the latest `ring` tokens (token p at slot p % ring): it must hold them
 *     for the tokens cached so far before the call, and does after it;
 *   - the indexer key of each CSA block j the append completes (c0 <= j <
 *     c0 + nc, c0 = floor(L/m), nc = floor((L+n)/m) - c0) is the caller's
 *     vector kvec row kvec_off[b] + (j - c0) (kdim elements in `dtype`; the
 *     pages give no source for it, so it is an input), encoded in MXFP4 as
 *     csa_mxfp4_quantize does into k_codes / k_scales row pool_off[b] + j
 *     (at most kvec_off[b+1] - kvec_off[b] blocks); kvec = NULL: no keys;
 *   - len[b] += n.
 * x_new, z_new [sum n][width] (values; pooling logits) in `dtype`; kv_raw
 * [capacity][width]; pooled / hpooled [rows][width]; kvec [sum nc][kdim],
 * kvec_off [B+1] device; k_codes [sum P][kdim/2], k_scales [sum P][kdim/32].
 * Writes past a sequence's raw or pooled capacity are skipped.  An append of
 * at most 64 tokens per sequence is one launch (a workgroup per sequence);
 * a longer one takes two.  Calls on one set of caches must be ordered (one
 * stream).
 * Errors: CSA_ERR_INVALID for null pointers, width not a positive multiple of
 * 8, m < 1, m_hca < 0, ring < max(m, m_hca), max_new < 0, unaligned rows,
 * kvec without kvec_off / k_codes / k_scales, kdim not a positive multiple
 * of 32; CSA_ERR_UNSUPPORTED for other dtypes.
 * ---------------------------------------------------------------------- */
int csa_cache_append(int dtype, int32_t n_seq, int width, const int64_t* tok_off, int64_t* len,
                     const int64_t* new_off, int64_t max_new, const void* x_new, const void* z_new, void* kv_raw,
                     void* z_tail, int ring, const int64_t* pool_off, int m, void* pooled,
                     const int64_t* hpool_off, int m_hca, void* hpooled, const int64_t* kvec_off, const void* kvec,
                     int kdim, uint8_t* k_codes, uint8_t* k_scales, void* stream);

/* ------------------------------------------------------------------------
 * csa_mxfp4_quantize — MXFP4 encoding of indexer vectors (the input format of
 * csa_index_topk and csa_hca_decode).
 * Pages: pytorch.kr FP4 QAT section (the indexer QK path is MXFP4).  The pages
 * give no conversion rule; the OCP MX one is taken: per block of 32 elements
 * the scale is 2^e with e = floor(log2(amax)) - 2, stored as the E8M0 byte
 * e + 127 clamped to [0, 254] (0 for an all-zero block); each element becomes
 * the e2m1 value nearest to x / 2^e, ties to the code with an even mantissa
 * bit, magnitudes above 6 saturating to 6; zero is code 0 whatever its sign.
 *   x       [rows][dim] in `dtype` (dim a multiple of 32), 16-byte aligned
 *   codes   [rows][dim/2] (two codes per byte, even element in the low
 *           nibble), 16-byte aligned; scales [rows][dim/32]
 * Indexer queries are rows of n_heads * 64, keys rows of 64.  Deterministic;
 * bit-identical to the definition above for every finite input.
 * Errors: CSA_ERR_INVALID for null pointers, rows < 0, dim not a positive
 * multiple of 32, unaligned x or codes; CSA_ERR_UNSUPPORTED for other dtypes.
 * ---------------------------------------------------------------------- */
int csa_mxfp4_quantize(int dtype, int64_t rows, int dim, const void* x, uint8_t* codes, uint8_t* scales,
                       void* stream);

/* ------------------------------------------------------------------------
 * csa_index_topk — lightning-indexer scores and per-query top-k.
 * Pages: jyp-garden IDEAS (KV compressed to 1/4, the Lightning Indexer keeps
 * only the top-k); sigco CSA/HCA section (the indexer finds relevant blocks,
 * only the top candidates are used); pytorch.kr FP4 QAT section (MXFP4 on the
 * indexer QK path).  Score of pooled entry j for query i (reading taken):
 *     S = sum_h w[i][h] * max(0, sum_c qhat[i][h][c] * khat[j][c])
 * with MXFP4 operands: e2m1 codes packed two per byte (even element in the
 * low nibble) and one E8M0 scale byte per 32 elements.  Visible entries of a
 * query at position t are j < min(floor((t+1)/m), P_b) (a block is visible
 * once it ends at or before t).  The k entries first under (S descending,
 * j ascending) are written to idx[i][0..k_eff) in ascending j, k_eff =
 * min(k, visible), and idx[i][k_eff..k) = -1.  Indices are relative to the
 * sequence's first pooled row pool_off[b].
 *   q_codes  [n_q][n_heads][dim/2]   q_scales [n_q][n_heads][dim/32]
 *   w        [n_q][n_heads] fp32, each an exact positive power of two or
 *            zero; it is folded into the query's block scales (byte + log2 w),
 *            so for a block with a non-zero code the folded byte must stay in
 *            E8M0's finite range [0, 254] (else it is clamped there and the
 *            scores are no longer those of the definition).  A block whose
 *            codes are all zero (+0 or -0) may carry any scale byte, 0
 *            included, and a zero weight drops its head.  Negative weights
 *            are not supported (the sign would be dropped).
 *   k_codes  [sum P][dim/2]          k_scales [sum P][dim/32]
 *   idx      [n_q][k] int32 (output)
 *   ws       workspace of >= csa_index_topk_workspace() bytes, ZERO-FILLED
 *            before its first use.  Every successful call returns the parts
 *            that must start at zero (histograms, counters, candidate bitmaps)
 *            to zero, so later calls reuse it without clearing; the rest is
 *            scratch that each call writes before reading (a failed launch may
 *            leave it dirty: re-zero it then).
 * Exactness: scores are formed in fp32 and compared as bit patterns.  They
 * are exact, and the selection therefore matches exact arithmetic bit for
 * bit, when every per-head dot and the head sum are representable, e.g. all
 * partial sums stay below 2^24 units of their smallest block product, which
 * holds for scale exponents within a few powers of two of each other.
 * Errors: CSA_ERR_UNSUPPORTED unless n_heads = 4 and dim = 64;
 * CSA_ERR_INVALID for null pointers, k < 1 or k > 4096, m < 1;
 * CSA_ERR_WORKSPACE when ws_bytes is too small.
 * ---------------------------------------------------------------------- */
int csa_index_topk_workspace(const csa_batch* b, int64_t max_pool, int k, size_t* bytes);
int csa_index_topk(const csa_batch* b, const int64_t* pool_off, int64_t max_pool, int m,
                   int n_heads, int dim, int k, const uint8_t* q_codes, const uint8_t* q_scales,
                   const float* w, const uint8_t* k_codes, const uint8_t* k_scales, int32_t* idx,
                   void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * csa_index_topk_bf16 — the same indexer with bf16 operands: the
 * higher-precision indexer the MXFP4 path is measured against.
 * Pages: pytorch.kr FP4 QAT section (the indexer QK path is FP4, with a
 * speed-up over a higher-precision selector at high recall).  Score of pooled
 * entry j for query i: S = sum_h w[i][h] * max(0, sum_c q[i][h][c] * key[j][c])
 * with bf16 q and keys, fp32 products and accumulation (exact when every
 * partial sum is representable, e.g. small-integer multiples of one power of
 * two); same visibility, order (S descending, j ascending), output layout and
 * workspace rules as csa_index_topk.  Decode batches only (max_q_per_seq < 16).
 *   q     [n_q][4][64] bf16     w [n_q][4] fp32 (exact powers of two keep
 *                               the products exact)
 *   keys  [sum P][64] bf16      idx [n_q][k] int32 (output)
 *   ws    >= csa_index_topk_workspace() bytes for the same batch, zero-filled
 *         before first use (left so by every successful call).
 * Errors: as csa_index_topk; CSA_ERR_UNSUPPORTED also for prefill batches.
 * ---------------------------------------------------------------------- */
int csa_index_topk_bf16(const csa_batch* b, const int64_t* pool_off, int64_t max_pool, int m, int n_heads, int dim,
                        int k, const void* q, const float* w, const void* keys, int32_t* idx, void* ws,
                        size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * csa_sparse_attn — MQA attention over the selected pooled rows plus the
 * sliding window, with ONE softmax.
 * Pages: pytorch.kr CSA/HCA section (attend to the top-k compressed entries;
 * a sliding-window branch keeps local detail); sigco CSA/HCA section (recent
 * tokens kept by a sliding window); jyp-garden IDEAS (MQA).  For query i at
 * position t in sequence b and head h the key list is
 *     [pooled row pool_off[b] + idx[i][s] for s < k_eff]  ++
 *     [raw row tok_off[b] + u for u = max(0, t-W+1) .. t]
 * (concatenated, no de-duplication; entries with idx < 0 are padding and
 * must come after the valid ones), and
 *     out[i][h] = sum_n softmax_n(scale * q[i][h] . key_n) * value_n,
 *     lse[i][h] = log sum_n exp(scale * q[i][h] . key_n).
 * An empty list gives out = 0 and lse = -inf.
 *   q [n_q][H][d], kv_pool [sum P][2][d], kv_raw [sum L][2][d], idx [n_q][k],
 *   out [n_q][H][d] (KV dtype), lse [n_q][H] fp32 or NULL,
 *   ws  >= csa_sparse_attn_workspace() bytes (no zero-fill needed).
 * Errors: CSA_ERR_INVALID for null pointers, W < 0, k < 0; CSA_ERR_UNSUPPORTED
 * for d != 128, H > 128, bf16 with H % 16 != 0; CSA_ERR_WORKSPACE.
 * ---------------------------------------------------------------------- */
int csa_sparse_attn_workspace(int dtype, const csa_batch* b, int H, int d, int W, int k,
                              size_t* bytes);
int csa_sparse_attn(int dtype, const csa_batch* b, const int64_t* pool_off, int H, int d,
                    float scale, int W, int k, const void* q, const void* kv_pool,
                    const void* kv_raw, const int32_t* idx, void* out, float* lse, void* ws,
                    size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * hca_attn — dense MQA attention over every visible m'-pooled row.
 * Pages: pytorch.kr CSA/HCA section (m' >> m, dense attention without
 * sparse selection); sigco CSA/HCA section (attention over all compressed
 * entries).  For query i at position t the key list is the pooled rows
 * j < min(floor((t+1)/m_hca), P'_b) followed, when W_hca > 0, by the raw
 * rows of the last W_hca tokens up to t (W_hca = 0: no window, the reading
 * taken for pure HCA).  Same softmax, outputs and empty-list rule as
 * csa_sparse_attn.
 *   kv_pool_hca [sum P'][2][d]; kv_raw may be NULL iff W_hca == 0.
 * ---------------------------------------------------------------------- */
int hca_attn_workspace(int dtype, const csa_batch* b, int64_t max_hpool, int H, int d, int W_hca,
                       size_t* bytes);
int hca_attn(int dtype, const csa_batch* b, const int64_t* hpool_off, int64_t max_hpool,
             int m_hca, int H, int d, float scale, int W_hca, const void* q,
             const void* kv_pool_hca, const void* kv_raw, void* out, float* lse, void* ws,
             size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * csa_hca_decode — one decode step of a CSA + HCA layer in ONE launch:
 * csa_index_topk, csa_sparse_attn and hca_attn of the same arguments, fused
 * into a single persistent kernel (one workgroup per compute unit, work units
 * handed out in dependency order) so that the HCA stream overlaps the top-k
 * chain and no launch gaps separate the stages.  Same definitions and
 * outputs as the three separate calls (pages as cited there); bit-identical
 * top-k.  Decode batches only: one query per sequence (n_q == n_seq,
 * q_off[b] == b), bf16, H % 16 == 0 and 16 <= H <= 64, d = 128, indexer
 * 4 x 64, k <= 1024, max_pool <= 262144 and at most 64 queries; otherwise
 * CSA_ERR_UNSUPPORTED (use the separate calls).  Indexer inputs (w included)
 * as csa_index_topk.
 *   kv_pool [sum P][2][d] (block m), kv_pool_hca [sum P'][2][d] (block m_hca),
 *   kv_raw [sum L][2][d]; idx [n_q][k]; csa_out/hca_out [n_q][H][d] bf16;
 *   csa_lse/hca_lse [n_q][H] fp32 or NULL.
 *   ws: >= csa_hca_decode_workspace() bytes, ZERO-FILLED before first use and
 *       reusable by later launches of the same shapes (a launch-epoch tag in
 *       ws tells one launch's words from another's); re-zero it when the
 *       shapes change.  Launches sharing a ws must be ordered (one stream).
 * The launch's workgroups take their work units from a counter in arrival
 * order, and a unit only waits for units handed out before it, so every wait
 * ends even when only some of the workgroups are resident at a time (another
 * kernel holding compute units only delays the step).  The waits are bounded
 * all the same: if one ever runs out the step's outputs are invalid and an
 * error word in ws is set, which csa_hca_decode_check() reports.
 * ---------------------------------------------------------------------- */
int csa_hca_decode_workspace(const csa_batch* b, int64_t max_pool, int64_t max_hpool, int H, int d,
                             int k, int W, int W_hca, size_t* bytes);
int csa_hca_decode(const csa_batch* b, const int64_t* pool_off, int64_t max_pool,
                   const int64_t* hpool_off, int64_t max_hpool, int m, int m_hca, int H, int d,
                   float scale, int k, int W, int W_hca, const uint8_t* q_codes,
                   const uint8_t* q_scales, const float* w, const uint8_t* k_codes,
                   const uint8_t* k_scales, const void* q, const void* kv_pool,
                   const void* kv_pool_hca, const void* kv_raw, int32_t* idx, void* csa_out,
                   float* csa_lse, void* hca_out, float* hca_lse, void* ws, size_t ws_bytes,
                   void* stream);

/* ------------------------------------------------------------------------
 * csa_hca_decode_noalloc — csa_hca_decode without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  It allocates
 * nothing: the step's workspace is a static scratch array of 64 MiB that the
 * library holds on each GPU it runs on until the process ends.  Arguments,
 * outputs and errors as csa_hca_decode (bit-identical results), plus
 * CSA_ERR_UNSUPPORTED when the step needs more than the 64 MiB
 * (csa_hca_decode_workspace() tells the size: 4 x 1M-token sequences need
 * about 11 MB).  Before the first call on a device, and before a call whose
 * shapes (n_q, max_pool, max_hpool, H, k, W, W_hca) differ from the previous
 * call's on that device, a small kernel on `stream` clears the bytes the step
 * uses.  Every call on a GPU shares that GPU's array and keeps the last
 * call's contents: calls that overlap on one GPU (different streams or host
 * threads) race and their results are undefined; order them on one stream.
 * The wait-bound error word of this variant is not readable by the caller.
 * ---------------------------------------------------------------------- */
int csa_hca_decode_noalloc(const csa_batch* b, const int64_t* pool_off, int64_t max_pool,
                           const int64_t* hpool_off, int64_t max_hpool, int m, int m_hca, int H, int d,
                           float scale, int k, int W, int W_hca, const uint8_t* q_codes,
                           const uint8_t* q_scales, const float* w, const uint8_t* k_codes,
                           const uint8_t* k_scales, const void* q, const void* kv_pool,
                           const void* kv_pool_hca, const void* kv_raw, int32_t* idx, void* csa_out,
                           float* csa_lse, void* hca_out, float* hca_lse, void* stream);

/* ------------------------------------------------------------------------
 * csa_hca_decode_shared — csa_hca_decode over caches whose leading part is
 * shared with another sequence (a prefix cache).
 * Pages: sigco.tistory.com KV-cache section (requests with a common prefix
 * reuse the cache already computed for it, so several questions over one long
 * document do not rebuild it); the shared part here is device-resident.
 * Sequence b with p = prefix_seq[b] >= 0 and T = prefix_tokens[b] > 0 reads
 * the first T tokens of its logical sequence from sequence p's cache: its
 * logical pooled row j (indexer key row j alike) is pooled row pool_off[p] + j
 * when j < T/m, else pool_off[b] + (j - T/m); its HCA row j is hpool_off[p] + j
 * when j < T/m_hca, else hpool_off[b] + (j - T/m_hca); its raw token u (window
 * rows) is tok_off[p] + u when u < T, else tok_off[b] + (u - T).  So b stores
 * only its own rows after the prefix, and its logical pooled count is
 * T/m + (pool_off[b+1] - pool_off[b]) (HCA alike).  q_pos, idx (indices into
 * the logical pooled rows) and every output are those of csa_hca_decode on
 * the logical sequence; the result is bit-identical to csa_hca_decode over
 * caches holding each logical sequence contiguously.
 *   prefix_seq [n_seq] int32 device (-1: no prefix); prefix_tokens [n_seq]
 *   int64 device.  T need not be a multiple of m or m_hca: a block that
 *   straddles T is b's own first pooled row (b's cache pools it from the
 *   prefix's last tokens and its own first ones).  p's cache should hold at
 *   least T tokens' rows and p should have no prefix of its own; the kernel
 *   clamps each count to what p stores (reads never leave p's rows) and
 *   ignores p outside [0, n_seq) or p == b, but the result is only
 *   meaningful when these hold.  max_pool / max_hpool bound the logical
 *   counts.  Other arguments, workspace and errors as csa_hca_decode;
 *   CSA_ERR_INVALID also for a NULL prefix array.
 * ---------------------------------------------------------------------- */
int csa_hca_decode_shared(const csa_batch* b, const int32_t* prefix_seq, const int64_t* prefix_tokens,
                          const int64_t* pool_off, int64_t max_pool, const int64_t* hpool_off, int64_t max_hpool,
                          int m, int m_hca, int H, int d, float scale, int k, int W, int W_hca,
                          const uint8_t* q_codes, const uint8_t* q_scales, const float* w,
                          const uint8_t* k_codes, const uint8_t* k_scales, const void* q, const void* kv_pool,
                          const void* kv_pool_hca, const void* kv_raw, int32_t* idx, void* csa_out,
                          float* csa_lse, void* hca_out, float* hca_lse, void* ws, size_t ws_bytes,
                          void* stream);

/* ------------------------------------------------------------------------
 * csa_hca_decode_paged — csa_hca_decode over paged pooled caches.
 * Pages: sigco.tistory.com KV-cache section (the compressed caches are kept
 * apart from the window and the tail, and a prefix's cache is reused by later
 * requests): here the compressed caches live in fixed-size pages that
 * sequences map through page tables, so pages can be allocated one at a time
 * as a sequence grows and a shared prefix's pages can appear in several
 * tables (see also csa_hca_decode_shared).
 * Sequence b's pooled row j (block m; and its indexer key row, paged the same
 * way) is row page_table[b][j / page_rows] * page_rows + j % page_rows of
 * kv_pool / k_codes / k_scales, for j < pooled_rows[b]; its HCA row j (block
 * m_hca) is row hca_page_table[b][j / hca_page_rows] * hca_page_rows +
 * j % hca_page_rows of kv_pool_hca, for j < hca_pooled_rows[b].  Raw rows
 * (window) stay contiguous: tok_off[b] + u.  Outputs, idx (indices into the
 * logical pooled rows) and exactness are those of csa_hca_decode over the
 * same logical caches, bit for bit.
 *   page_table [n_seq][max_pages] int32 device, hca_page_table
 *   [n_seq][max_hca_pages]; pooled_rows, hca_pooled_rows [n_seq] int64
 *   device.  page_rows and hca_page_rows: powers of two, >= 32.  The kernel
 *   clamps each count to what its table maps; page ids are trusted.
 *   max_pool / max_hpool bound the pooled counts (and the tables must map
 *   them).  Other arguments, workspace and errors as csa_hca_decode (its
 *   pool_off / hpool_off are replaced by the tables); CSA_ERR_INVALID also for
 *   NULL tables or counts, page sizes that are not powers of two >= 32,
 *   tables with no column, or tables mapping fewer rows than max_pool /
 *   max_hpool.
 * ---------------------------------------------------------------------- */
int csa_hca_decode_paged(const csa_batch* b, int page_rows, const int32_t* page_table, int max_pages,
                         const int64_t* pooled_rows, int hca_page_rows, const int32_t* hca_page_table,
                         int max_hca_pages, const int64_t* hca_pooled_rows, int64_t max_pool, int64_t max_hpool,
                         int m, int m_hca, int H, int d, float scale, int k, int W, int W_hca,
                         const uint8_t* q_codes, const uint8_t* q_scales, const float* w,
                         const uint8_t* k_codes, const uint8_t* k_scales, const void* q, const void* kv_pool,
                         const void* kv_pool_hca, const void* kv_raw, int32_t* idx, void* csa_out,
                         float* csa_lse, void* hca_out, float* hca_lse, void* ws, size_t ws_bytes,
                         void* stream);

/* Synchronises `stream`, then returns CSA_OK if no csa_hca_decode launch on
 * workspace `ws` hit its wait bound since the last check, else
 * CSA_ERR_DEVICE; clears the word.  (The only synchronising call.) */
int csa_hca_decode_check(const csa_batch* b, const void* ws, void* stream);

/* Synchronises `stream`, then stores in *rows how many row selections of the
 * csa_hca_decode launches on `ws` (since it was zero-filled) could not be
 * proved exact from the score chunks' candidate lists and took the exact
 * radix select over all of the row's keys instead (same result, slower).
 * ws and rows non-NULL (rows is a host pointer), else CSA_ERR_INVALID. */
int csa_hca_decode_fallbacks(const void* ws, void* stream, uint32_t* rows);

/* ------------------------------------------------------------------------
 * csa_profile_events — tracing hook (host).  Until cleared, every launch of
 * internal kernel `kernel_id` made by the calling thread carries the two
 * events: they are attached to the dispatch itself (hipExtLaunchKernel), so
 * hipEventElapsedTime(start, stop) is the kernel's execution time on the GPU,
 * as a kernel trace reports it, without the enqueue (for an id that covers
 * two kernels, from the first one's start to the second one's end).
 * start/stop are hipEvent_t handles owned by the caller; pass NULL, NULL to
 * clear.  Kernel ids: CSA_K_IDX_SCORE (indexer scoring), CSA_K_IDX_SELECT,
 * CSA_K_IDX_FINAL (top-k passes of decode batches; for caches of at most
 * 4096 pooled entries per sequence the one-launch top-k), CSA_K_ATTN (attention
 * main kernel, CSA or HCA), CSA_K_ATTN_COMBINE (split merge), CSA_K_COMPRESS,
 * CSA_K_FUSED, CSA_K_PF_THRESH and CSA_K_PF_SELECT (threshold and selection
 * kernels of prefill batches; their scoring kernel is CSA_K_IDX_SCORE),
 * CSA_K_APPEND (both kernels of csa_cache_append), CSA_K_QUANT
 * (csa_mxfp4_quantize).
 * Errors: CSA_ERR_INVALID for an unknown id or exactly one NULL event.
 * ---------------------------------------------------------------------- */
enum {
  CSA_K_IDX_SCORE = 0,
  CSA_K_IDX_SELECT = 1,
  CSA_K_IDX_FINAL = 2,
  CSA_K_ATTN = 3,
  CSA_K_ATTN_COMBINE = 4,
  CSA_K_COMPRESS = 5,
  CSA_K_FUSED = 6,
  CSA_K_PF_THRESH = 7,
  CSA_K_PF_SELECT = 8,
  CSA_K_APPEND = 9,
  CSA_K_QUANT = 10,
  CSA_K_COUNT = 11
};
int csa_profile_events(int kernel_id, void* start, void* stop);

#ifdef __cplusplus
}
#endif
#endif /* CSA_H */

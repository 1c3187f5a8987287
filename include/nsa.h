/*
 * nsa.h -- C ABI of the MI355X (gfx950) sparse-attention decode library.
 *
 * One step of DeepSeek native / DeepSeek sparse attention (NSA / DSA) per
 * query row:
 *   indexer logits -> length-masked top-k -> page-table transform ->
 *   MLA attention over the selected KV slots of a shared 576-wide latent.
 *
 * Source pages cited below, by title:
 *   [nsa-fork]  "nsa_backend.py (EngineX-Hygon sglang fork)"
 *   [dsa-main]  "dsa_backend.py (sglang main)"
 *   [nsa-diff]  "nsa_backend.py (sglang 0.5.3rc2 -> 0.5.4 diff)"
 *
 * Conventions shared by every call
 *   - Pointers named as device pointers must point to device memory of the
 *     current HIP device; pointers named as host pointers to host memory.
 *   - The caller owns every buffer. The library never allocates, frees, or
 *     synchronises with the host; all work is enqueued on `stream` (a
 *     hipStream_t; NULL is the default stream) and the call returns at once.
 *   - Integer index tensors are int32. Strides are in elements.
 *   - Index rows use -1 for unused entries, valid entries first.
 *   - Every call returns NSA_OK (0) or a negative status. Arguments are
 *     checked on the host before anything is launched; on error nothing is
 *     launched and nsa_last_error() describes the problem. No call aborts.
 *   - Device-side data the host cannot check (index values, page ids, slot
 *     ids, request indices, pool rows) is bounds-checked in the kernels: an
 *     out-of-range id is treated as absent (see each call), never
 *     dereferenced, and recorded as an NSA_DEVERR_* bit that
 *     nsa_check_device_errors() reports.
 */
#ifndef NSA_H_
#define NSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes -------------------------------------------------------- */
#define NSA_OK 0
#define NSA_ERR_INVALID_ARG (-1)  /* null pointer, negative size, bad stride */
#define NSA_ERR_UNSUPPORTED (-2)  /* shape / dtype / page size not supported */
#define NSA_ERR_WORKSPACE (-3)    /* workspace missing or too small */
#define NSA_ERR_LAUNCH (-4)       /* the HIP runtime rejected a launch */

/* ---- enums ---------------------------------------------------------------- */
#define NSA_MODE_DECODE 0
#define NSA_MODE_EXTEND 1
#define NSA_MODE_TARGET_VERIFY 2
#define NSA_MODE_DRAFT_EXTEND 3     /* draft model, per-request accepted + 1 */
#define NSA_MODE_DRAFT_EXTEND_V2 4  /* draft model, draft_token_num each */

#define NSA_DTYPE_FP32 0
#define NSA_DTYPE_BF16 1
#define NSA_DTYPE_FP8_E4M3 2  /* OCP e4m3fn */

#define NSA_KV_BF16_576 0     /* latent row = 576 bf16 (1152 bytes) */
#define NSA_KV_FP8_656 1      /* latent row = 656 bytes, see quantize below */

#define NSA_PAGE_SIZE 64
#define NSA_D_QK 576
#define NSA_D_V 512

/* Thread-local description of the last error returned on this thread
 * ("" when the last call succeeded). The string stays valid until the next
 * call on the same thread. */
const char* nsa_last_error(void);

/* Library version as an integer (major*10000 + minor*100 + patch). */
int nsa_version(void);

/* ---- device-side errors ------------------------------------------------------
 * The DSA page validates the page table against the KV-cache capacity before
 * an extend ([dsa-main] init_forward_metadata, extend branch: the largest
 * token slot must lie below the pool's capacity). Here every kernel checks
 * the ids it reads from device memory and, for one out of range, records
 * one of these bits in a device word (one per library translation unit, per
 * device) while treating the id as absent:
 */
#define NSA_DEVERR_PAGE_ID 0x1   /* indexer: a page id outside [0, num_pages) */
#define NSA_DEVERR_SLOT 0x2      /* a KV slot outside [0, num_slots) other than -1
                                    (attention, quantize-on-write, paged
                                    dequantisation) */
#define NSA_DEVERR_REQUEST 0x4   /* a token_to_req entry outside [0, rows of the
                                    page table) (indexer, top-k, transform,
                                    ragged metadata) */
#define NSA_DEVERR_POOL_ROW 0x8  /* metadata: a req_pool_indices entry outside
                                    [0, pool_rows) */
#define NSA_DEVERR_INDEX 0x10    /* transform: a top-k index at or past its
                                    table's width */
/* Waits for `stream`, then returns the OR of the NSA_DEVERR_* bits recorded
 * on the current device since the last call (>= 0) and clears them, or a
 * negative status if the HIP runtime fails. It synchronises with the host, so
 * it belongs in debug paths and tests, not inside a captured graph. Calls
 * that overlap on other streams may add bits while it runs. */
int nsa_check_device_errors(void* stream);

/* ---- a0: per-forward metadata ------------------------------------------------
 * Defined by [nsa-fork] NSAMetadata, compute_cu_seqlens,
 * _transform_table_1_to_real and NativeSparseAttnBackend.init_forward_metadata;
 * [dsa-main] DeepseekSparseAttnBackend.init_forward_metadata (decode,
 * target-verify and extend branches) and _cal_indexer_k_start_end (per-token
 * batch index); [nsa-diff] target-verify metadata; [dsa-main]
 * init_forward_metadata draft-extend branch and the draft-extend-v2 branch of
 * init_forward_metadata_replay_cuda_graph (draft-extend rows are per token,
 * as in target-verify, and seq_lens already count the new tokens).
 *
 * Inputs (device, int32):
 *   seq_lens[bs]          KV length per request (extend, draft-extend:
 *                         including the new tokens; target-verify: excluding
 *                         the drafts).
 *   extend_lens[bs]       new tokens per request (EXTEND and DRAFT_EXTEND,
 *                         else ignored / NULL).
 *   req_to_token          [pool_rows, rtt_stride] token -> physical slot.
 *   req_pool_indices[bs]  each request's row of req_to_token; a row outside
 *                         [0, pool_rows) gives -1 page ids in its tables
 *                         (NSA_DEVERR_POOL_ROW).
 * Host scalars:
 *   mode                  NSA_MODE_*.
 *   draft_token_num       tokens per request of TARGET_VERIFY and
 *                         DRAFT_EXTEND_V2 (>= 1), else ignored.
 *   topk                  selection size (clip for nsa_cache_seqlens).
 *   page_size             must be 64.
 *   max_seqlen_k          host bound >= every cache seqlen; sizes the tables.
 *   num_q_rows            T: bs (decode), bs*draft (verify, draft-extend
 *                         v2), sum of extend_lens (extend, draft-extend).
 *                         Extend modes: rows past sum(extend_lens) get
 *                         length 0 (seqlens_expanded, nsa_cache_seqlens),
 *                         token_to_req 0 and the running
 *                         nsa_cu_seqlens_k total, so a T above the sum is
 *                         harmless; rows past T are never written.
 * Outputs (device, int32, caller-allocated):
 *   cache_seqlens[bs]         seq_lens (+ draft_token_num in verify).
 *   cu_seqlens_k[bs+1]        [0, cumsum(cache_seqlens)].
 *   cu_seqlens_q              decode, verify, draft-extend: [T+1] =
 *                             arange(T+1) (every verify or draft-extend token
 *                             is its own query row);
 *                             extend: [bs+1] = [0, cumsum(extend_lens)].
 *   seqlens_expanded[T]       visible KV length of each query row: decode =
 *                             cache_seqlens; other modes: kv_len - q_len + 1
 *                             ... kv_len per request.
 *   nsa_cache_seqlens[T]      min(seqlens_expanded, topk).
 *   nsa_cu_seqlens_k[T+1]     [0, cumsum(nsa_cache_seqlens)].
 *   nsa_cu_seqlens_q[T+1]     arange(T+1).
 *   real_page_table           [bs, rpt_stride], columns
 *                             p < ceil(max_seqlen_k/64) written with
 *                             req_to_token[row, 64 p] >> 6 (one row per
 *                             request; the pages repeat it per draft token).
 *   token_to_req[T]           request of each query row.
 *   page_table_1              optional [bs, pt1_stride] copy of
 *                             req_to_token[row, :max_seqlen_k]; NULL to skip
 *                             (the wide table the DSA page drops in its fused
 *                             decode graphs).
 * Host must ensure rtt_stride >= max_seqlen_k, pt1_stride >= max_seqlen_k
 * and rpt_stride >= ceil(max_seqlen_k/64); req_to_token must have at least
 * max_seqlen_k readable columns in every row named by req_pool_indices.
 */
int nsa_build_metadata(int mode, int bs, int draft_token_num, int topk,
                       int page_size, const int32_t* seq_lens,
                       const int32_t* extend_lens, const int32_t* req_to_token,
                       int64_t rtt_stride, int64_t pool_rows,
                       const int32_t* req_pool_indices,
                       int max_seqlen_k, int num_q_rows,
                       int32_t* cache_seqlens, int32_t* cu_seqlens_k,
                       int32_t* cu_seqlens_q, int32_t* seqlens_expanded,
                       int32_t* nsa_cache_seqlens, int32_t* nsa_cu_seqlens_k,
                       int32_t* nsa_cu_seqlens_q, int32_t* real_page_table,
                       int64_t rpt_stride, int32_t* token_to_req,
                       int32_t* page_table_1, int64_t pt1_stride,
                       void* stream);

/* ---- a1: indexer logits ("paged MQA logits") -----------------------------------
 * The indexer reads the index-key cache through the 64-token page table
 * ([nsa-fork] NSAIndexerMetadata.get_page_table_64) for the row's expanded
 * seqlen ([dsa-main] _to_2d_context_lens: one context length per row).
 * Scoring formula (the indexer itself is not on the pages; reading adopted):
 *   logits[t, s] = kscale[s] * sum_h weights[t, h] * max(0, q[t,h,:] . k[s,:])
 * for s < min(seqlens_expanded[t], max_seqlen_k). Positions at or past that
 * length are NOT written.
 *
 *   q                [T, Hi, Di] row-major; fp8 e4m3 codes (q_dtype
 *                    NSA_DTYPE_FP8_E4M3) or fp32 (NSA_DTYPE_FP32). Any
 *                    query-side scale is folded into weights by the caller.
 *   weights          [T, Hi] fp32.
 *                    q, weights and the keys are finite (fp8 NaN codes
 *                    0x7F / 0xFF are outside the contract: their logits
 *                    are unspecified).
 *   k_index_cache    [num_pages] pages of 64 tokens; page bytes =
 *                    64*Di*elem (keys, row-major [64][Di]) + 64*4 (fp32
 *                    per-token scales). k_dtype must equal q_dtype.
 *   real_page_table  [num_reqs, rpt_stride] page ids per request; a page id
 *                    outside [0, num_pages) yields -inf logits for its 64
 *                    positions (NSA_DEVERR_PAGE_ID).
 *                    The fp8 path needs num_pages >= 1 (it reads page 0 in
 *                    place of an absent page); 0 is NSA_ERR_INVALID_ARG there.
 *   token_to_req[T], seqlens_expanded[T]  from nsa_build_metadata; a row
 *                    whose token_to_req lies outside [0, num_reqs) is left
 *                    unwritten, as an empty row (NSA_DEVERR_REQUEST).
 *   logits           [T, logits_stride] fp32, logits_stride >= max_seqlen_k.
 *                    Rows that start 256-byte aligned (stride a multiple of
 *                    64) give whole-line stores here and vector loads in
 *                    nsa_topk_transform; any stride is correct.
 * Supported: (fp8, Hi = 64, Di = 128) on the MFMA path; (fp32, Hi <= 64,
 * Di <= 128, Di % 4 == 0). page_size must be 64.
 * The fp8 path assumes each key page is read by one row (decode) and streams
 * the keys with non-temporal loads, which do not keep them in the caches;
 * rows that share pages are served better by nsa_indexer_logits_hist with
 * its rows_per_request hint. Results do not depend on this.
 */
int nsa_indexer_logits(const void* q, int q_dtype, const float* weights,
                       const void* k_index_cache, int k_dtype,
                       int64_t num_pages, const int32_t* real_page_table,
                       int64_t rpt_stride, int64_t num_reqs, const int32_t* token_to_req,
                       const int32_t* seqlens_expanded, int T, int Hi, int Di,
                       int page_size, int max_seqlen_k, float* logits,
                       int64_t logits_stride, void* stream);

/* ---- a2 (+a3 fused): length-masked top-k -----------------------------------------
 * [nsa-fork] NSAIndexerMetadata.topk_transform: fast_topk_v2(logits,
 * lengths, topk) returns logical positions; fast_topk_transform_fused(...)
 * returns physical slots through the page table. Field comment of
 * nsa_cache_seqlens_int32: the effective length is clipped to topk.
 *
 * Row t keeps n = min(lengths[t], max_seqlen_k): if n <= topk every position
 * 0..n-1, else the topk positions with the largest logits[t, 0:n]. The row of
 * `out` holds the kept entries in ascending position order, then -1. Ties at
 * the threshold are broken by ascending position. NaN logits rank lowest.
 *   table == NULL    out holds logical positions.
 *   table != NULL    out holds physical slots: table is the compact page
 *                    table [table_rows, table_stride] (real_page_table) and
 *                    slot = table[token_to_req[t], i >> 6] * 64 + (i & 63);
 *                    a row whose token_to_req lies outside [0, table_rows)
 *                    is written as all -1 (NSA_DEVERR_REQUEST).
 *   workspace        device scratch of nsa_topk_workspace_size() bytes (may
 *                    be NULL when that size is 0).
 */
int nsa_topk_workspace_size(int T, int max_seqlen_k, int topk, size_t* bytes);
int nsa_topk_transform(const float* logits, int64_t logits_stride,
                       const int32_t* lengths, int T, int topk,
                       int max_seqlen_k, const int32_t* table,
                       int64_t table_stride, int64_t table_rows, const int32_t* token_to_req,
                       int page_size, int32_t* out, int64_t out_stride,
                       void* workspace, size_t ws_bytes, void* stream);

/* ---- f1: the top-k histogram fused into the indexer ----------------------------
 * Direction of the pages' folded top-k plan ("dsa_backend.py (sglang main)",
 * _build_topk_v2_plan: top-k work prepared from the same lengths the
 * transform receives): the indexer, which holds every logit anyway, also
 * histograms them, so the top-k reads the logits once instead of twice.
 *
 * nsa_indexer_logits_hist: as nsa_indexer_logits (fp8 path only), and adds
 * to key_hist[t * 4096 + b] the number of positions s < min(L_t,
 * max_seqlen_k) whose logit's order key has top 12 bits b. The order key of
 * x: NaN -> 0; -0 -> +0; otherwise the fp32 bits with the sign bit set for
 * x >= 0 and all bits inverted for x < 0 (so keys order as the floats).
 * key_hist is device memory of T * 4096 uint32, 4-byte aligned, owned by the
 * caller, and must hold zeros on entry (counts are added atomically).
 * rows_per_request: a scheduling hint (the typical number of consecutive
 * rows of one request), not a change of results:
 *   >= 4     rows are scored in groups of 4 consecutive rows; a group whose
 *            rows share one request reads each key page once for all of
 *            them (target-verify, draft-extend v2 with 4 drafts, extend),
 *            a group that mixes requests scores its rows one at a time;
 *   2 or 3   when T is a multiple of it, the blocks of a group that read
 *            the same key pages run back to back on one XCD, so the pages
 *            come from HBM about once per group;
 *   other    per-row order; at most 1 (one row per request, as in
 *            decode) also streams the keys with non-temporal loads, which
 *            do not keep them in the caches for other rows.
 * Every choice gives bit-identical logits and counts.
 *
 * nsa_topk_transform_hist: as nsa_topk_transform, with key_hist from
 * nsa_indexer_logits_hist over the same logits (16-byte aligned). It sets
 * rows 0..T-1 of key_hist back to zero, so one buffer serves every layer. A
 * row whose counts do not add up to its length takes a slower exact path;
 * any other mismatch between key_hist and the logits is the caller's
 * contract (the result is then unspecified but stays in the bounds of `out`).
 *   workspace   optional device scratch of nsa_topk_hist_workspace_size()
 *               bytes, 16-byte aligned, owned by the caller, contents
 *               irrelevant on entry (ws_bytes is its size; smaller is
 *               NSA_ERR_WORKSPACE). With it, a batch of at most 128
 *               rows longer than 16384 positions has its rows classified by
 *               blocks of 16384 positions spread over the whole GPU instead
 *               of one block per row (a second launch then finishes each
 *               row). NULL, or a size of 0 from the query, runs one block
 *               per row. Results are identical either way.
 * nsa_topk_hist_workspace_size: that size for T rows (0 when the split is
 * not used: T > 128, max_seqlen_k <= max(topk, 16384) or > 262144).
 */
int nsa_indexer_logits_hist(const void* q, int q_dtype, const float* weights,
                            const void* k_index_cache, int k_dtype,
                            int64_t num_pages, const int32_t* real_page_table,
                            int64_t rpt_stride, int64_t num_reqs, const int32_t* token_to_req,
                            const int32_t* seqlens_expanded, int T, int Hi,
                            int Di, int page_size, int max_seqlen_k,
                            float* logits, int64_t logits_stride,
                            uint32_t* key_hist, int rows_per_request,
                            void* stream);
int nsa_topk_hist_workspace_size(int T, int max_seqlen_k, int topk,
                                 size_t* bytes);
int nsa_topk_transform_hist(const float* logits, int64_t logits_stride,
                            const int32_t* lengths, int T, int topk,
                            int max_seqlen_k, const int32_t* table,
                            int64_t table_stride, int64_t table_rows, const int32_t* token_to_req,
                            int page_size, uint32_t* key_hist, int32_t* out,
                            int64_t out_stride, void* workspace, size_t ws_bytes,
                            void* stream);

/* ---- a3: page-table transform ---------------------------------------------------
 * [nsa-fork] forward_decode / forward_extend:
 * transform_index_page_table_decode / _prefill(page_table_1, topk_indices,
 * page_size=1). out[t, j] = -1 if idx < 0, else the physical slot of logical
 * position idx of request token_to_req[t]: page_table_1[r, idx] (wide form)
 * or real_page_table[r, idx >> 6] * 64 + (idx & 63) (compact form). Exactly
 * one of page_table_1 / real_page_table must be non-NULL, with table_rows
 * rows. Indices at or past the table width give -1 (NSA_DEVERR_INDEX); a row
 * whose token_to_req lies outside [0, table_rows) is written as all -1
 * (NSA_DEVERR_REQUEST).
 */
int nsa_page_table_transform(const int32_t* topk_indices, int64_t in_stride,
                             int T, int topk, const int32_t* page_table_1,
                             int64_t pt1_stride, int64_t pt1_width,
                             const int32_t* real_page_table,
                             int64_t rpt_stride, int64_t rpt_width,
                             int64_t table_rows, int page_size,
                             const int32_t* token_to_req,
                             int32_t* out, int64_t out_stride, void* stream);

/* ---- a4 / a5: sparse MLA over selected slots ------------------------------------
 * [nsa-fork] _forward_fa3 (semantics: score = q_rope.k_rope + q_nope.c_kv,
 * value = c_kv, over the first nsa_cache_seqlens[t] entries of the
 * transformed table), _forward_flashmla_decode / [dsa-main]
 * _forward_flashmla_kv (q [T, H, 576], cache viewed as [pages, 64, 1, dim],
 * indices width == topk, returns o and lse), _forward_flashmla_sparse.
 *
 *   q            bf16, element (t, h, d) at q[t*q_tok_stride + h*q_head_stride
 *                + d], d < 576 (512 no-rope then 64 rope).
 *   kv_cache     [num_slots] rows: NSA_KV_BF16_576 (576 bf16) or
 *                NSA_KV_FP8_656 (the quantize_k_cache layout).
 *   indices      [T, idx_stride] int32 physical slots, -1 = unused; a slot
 *                outside [0, num_slots) counts as unused (and, unless -1,
 *                sets NSA_DEVERR_SLOT).
 *   nsa_cache_seqlens  optional [T]: only the first nsa_cache_seqlens[t]
 *                entries of row t are read (NULL: all topk entries).
 *   out          [T, H, 512] bf16, contiguous.
 *   lse          optional [T, H] fp32 natural-log log-sum-exp of the scaled
 *                scores (-inf for a row with no valid slot; out = 0 there).
 *   workspace    device scratch >= nsa_sparse_mla_workspace_size(...) bytes.
 * Supported: H in {16, 32, ..., 128}, d_qk = 576, d_v = 512, topk <= 8192,
 * q pointer 16-byte aligned and strides multiples of 8 elements.
 * The result is bit-reproducible (fixed-order combine of KV splits).
 * _decode plans KV splits for small T (decode, verify rows); _extend for
 * many rows (chunked prefill). Both compute the same function.
 */
int nsa_sparse_mla_workspace_size(int T, int H, int topk, int d_v,
                                  size_t* bytes);
int nsa_sparse_mla_decode(const void* q, int64_t q_tok_stride,
                          int64_t q_head_stride, const void* kv_cache,
                          int kv_dtype, int64_t num_slots,
                          const int32_t* indices, int64_t idx_stride,
                          const int32_t* nsa_cache_seqlens, int T, int H,
                          int topk, int d_qk, int d_v, float sm_scale,
                          void* out, float* lse, void* workspace,
                          size_t ws_bytes, void* stream);
int nsa_sparse_mla_extend(const void* q, int64_t q_tok_stride,
                          int64_t q_head_stride, const void* kv_cache,
                          int kv_dtype, int64_t num_slots,
                          const int32_t* indices, int64_t idx_stride,
                          const int32_t* nsa_cache_seqlens, int T, int H,
                          int topk, int d_qk, int d_v, float sm_scale,
                          void* out, float* lse, void* workspace,
                          size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation as nsa_sparse_mla_decode, with its split workspace taken from a
 * fixed device array inside the library (64 MiB, one per GPU, held until the
 * process ends; its device address is looked up once per device). Nothing is
 * allocated. A shape whose plan needs more scratch than that returns
 * NSA_ERR_WORKSPACE. Every call on one GPU uses the same array: calls that
 * overlap on one GPU (on different streams) race and must be serialised by
 * the caller. Arguments and results as nsa_sparse_mla_decode. */
int nsa_sparse_mla_decode_noalloc(const void* q, int64_t q_tok_stride,
                                  int64_t q_head_stride, const void* kv_cache,
                                  int kv_dtype, int64_t num_slots,
                                  const int32_t* indices, int64_t idx_stride,
                                  const int32_t* nsa_cache_seqlens, int T, int H,
                                  int topk, int d_qk, int d_v, float sm_scale,
                                  void* out, float* lse, void* stream);

/* ---- a6: fp8 block-scaled latent cache --------------------------------------------
 * [nsa-fork] _forward_flashmla_decode and [dsa-main] _forward_flashmla_kv
 * call quantize_k_cache(kv_cache) to produce the fp8 cache the decode kernel
 * reads (page size 64). Layout (a reading; the body is not on the pages),
 * one 656-byte row per slot:
 *   [0, 512)    e4m3fn codes of the 512 no-rope values, 4 blocks of 128
 *   [512, 528)  4 fp32 block scales, scale_b = amax_b / 448 (1 if amax_b = 0)
 *   [528, 656)  64 rope values, bf16, copied
 * code = round-to-nearest-even, saturating e4m3fn of (x / scale_b), the
 * division correctly rounded in fp32.
 *   kv_bf16   [num_slots, in_stride] bf16, first 576 elements used.
 *   out       [num_slots, 656] bytes.
 */
int nsa_quantize_k_cache(const void* kv_bf16, int64_t num_slots,
                         int64_t in_stride, void* out, void* stream);

/* ---- f2: quantize-on-write of new latent rows --------------------------------------
 * [dsa-main] forward_extend / forward_decode store each new token's latent
 * row with token_to_kv_pool.set_mla_kv_buffer(layer, cache_loc, k, k_rope)
 * before attention. This call writes row i into slot cache_loc[i] in the
 * cache's own format: for NSA_KV_FP8_656 the 656-byte row is exactly what
 * nsa_quantize_k_cache makes of the 576 values (so the fp8 cache never needs
 * a whole-cache re-quantization), for NSA_KV_BF16_576 the values are copied.
 *   k_nope      [n, nope_stride] bf16, first 512 elements used; 16-byte
 *               aligned, nope_stride >= 512 and a multiple of 8.
 *   k_rope      [n, rope_stride] bf16, first 64 elements used; bf16 cache:
 *               16-byte aligned, rope_stride a multiple of 8.
 *   cache_loc   [n] int32 destination slots; entries outside
 *               [0, num_slots) are skipped (NSA_DEVERR_SLOT). Entries must
 *               be distinct (two rows to one slot race).
 *   kv_cache    [num_slots, 656] bytes or [num_slots, 576] bf16, updated in
 *               place; other slots are not touched.
 * Nothing is allocated; n == 0 is a no-op.
 */
int nsa_set_mla_kv_buffer(const void* k_nope, int64_t nope_stride,
                          const void* k_rope, int64_t rope_stride,
                          const int32_t* cache_loc, int n, void* kv_cache,
                          int kv_dtype, int64_t num_slots, void* stream);

/* ---- f3: the RAGGED extend route ---------------------------------------------------
 * [dsa-main] scores each extend token against the concatenated keys of the
 * batch and attends over a contiguous bf16 copy of the batch's latent rows
 * (init_forward_metadata extend branch: page_table_1_flattened,
 * topk_indices_offset; _cal_indexer_k_start_end: ks / ke; forward_extend
 * RAGGED: the shifted top-k positions and dequantize_k_cache_paged). The
 * route composes with the other calls: nsa_indexer_logits + nsa_topk_transform
 * (no table) give each row's positions relative to its request, which are
 * the positions inside [ks, ke) minus ks; nsa_ragged_index_transform shifts
 * them into the concatenation; nsa_dequantize_k_cache_paged builds the bf16
 * rows of the flattened table; nsa_sparse_mla_extend then reads those rows
 * (NSA_KV_BF16_576) with the shifted positions as slot indices.
 *
 * nsa_ragged_extend_metadata, from the outputs of nsa_build_metadata:
 *   cu_seqlens_k[bs+1], cache_seqlens[bs], seqlens_expanded[T],
 *   token_to_req[T], real_page_table [bs, rpt_stride]  (device, int32);
 *   max_seqlen_k   the host bound used for nsa_build_metadata.
 *   ks[T], ke[T]   the row's window [ks, ke) in the concatenated keys:
 *                  ks = cu_seqlens_k[req], ke = ks + seqlens_expanded.
 *   topk_indices_offset[T]  (nullable) = ks.
 *   page_table_1_flattened  (nullable) [flat_capacity]: entry
 *                  cu_seqlens_k[r] + s = slot of token s of request r, for
 *                  s < cache_seqlens[r]; positions >= flat_capacity are not
 *                  written (size it with the host's sum of cache lengths).
 */
int nsa_ragged_extend_metadata(const int32_t* cu_seqlens_k,
                               const int32_t* cache_seqlens, int bs,
                               const int32_t* seqlens_expanded,
                               const int32_t* token_to_req, int T,
                               const int32_t* real_page_table,
                               int64_t rpt_stride, int max_seqlen_k,
                               int32_t* ks, int32_t* ke,
                               int32_t* topk_indices_offset,
                               int32_t* page_table_1_flattened,
                               int64_t flat_capacity, void* stream);

/* out[t, j] = topk_indices[t, j] + offset[t] where the index is not -1, else
 * -1 (forward_extend, RAGGED). [T, topk] int32 with row strides; in place
 * (out == topk_indices) is allowed. */
int nsa_ragged_index_transform(const int32_t* topk_indices, int64_t in_stride,
                               int T, int topk, const int32_t* offset,
                               int32_t* out, int64_t out_stride, void* stream);

/* dequantize_k_cache_paged: out[i] = bf16 latent row of slot slots[i] of an
 * NSA_KV_FP8_656 cache: each no-rope value = fp32 product of its e4m3 code
 * and block scale, rounded to bf16 (nearest even); the 64 rope values copied;
 * a slot outside [0, num_slots) gives a zero row (a reading: the body is not
 * on the pages; NSA_DEVERR_SLOT). out: [n, out_stride] bf16, out_stride >= 576 and a multiple
 * of 8, 16-byte aligned. */
int nsa_dequantize_k_cache_paged(const void* kv_fp8, int64_t num_slots,
                                 const int32_t* slots, int64_t n, void* out,
                                 int64_t out_stride, void* stream);

/* CSR lists of the entries != -1 of an index matrix [T, topk] (the aiter
 * route's get_valid_kv_indices in [dsa-main]): kv_indptr[T+1] =
 * [0, cumsum(valid count per row)], kv_indices = every row's valid entries
 * in column order, rows in order; entries beyond `capacity` are dropped
 * (kv_indptr still counts them). Three launches (count, scan, write). For
 * rows written by nsa_topk_transform (valid first) kv_indptr equals
 * nsa_cu_seqlens_k. */
int nsa_valid_kv_indices(const int32_t* indices, int64_t idx_stride, int T,
                         int topk, int32_t* kv_indptr, int32_t* kv_indices,
                         int64_t capacity, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NSA_H_ */

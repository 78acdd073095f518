/*
 * saga.h -- C ABI of the SAGA + Atop-N decode-attention library (libsaga.so,
 * HIP, gfx950 / MI355X).
 *
 * One decode step of attention for one layer, for a batch of sequences that
 * share one context length.  The method is the one described on the pages
 * "More Value per Key: Asymmetric Sparse Attention for Faster LLM Decoding"
 * (ai.info AI summary and atlas.scime.ai AI summary):
 *   - SAGA: the number of key heads h_k is chosen independently of the number
 *     of value heads h_v (ai.info summary, Key Contributions 3; atlas summary,
 *     Approach).  Query head i reads key head i / (h_q/h_k) and value head
 *     i / (h_q/h_v) (contiguous grouping).  h_k == h_v is ordinary GQA.
 *   - Atop-N: exact top-N logit thresholds are computed once every n steps
 *     and reused; in between, entries are picked by comparing each logit with
 *     the reused threshold, with no sort (ai.info summary, Key Contributions 2
 *     and Methodology).  The probability-value product then reads only the
 *     selected value rows (ai.info summary, Main Findings, first item).
 *
 * The caller owns the refresh schedule: at steps t with t mod n == 0 call
 * atopn_refresh_decode_step() (or atopn_refresh_thresholds() and then
 * saga_decode_step() with the fresh thresholds); at other steps call
 * saga_decode_step() with the kept ones.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers named *_dev are device pointers (hipMalloc / torch CUDA memory),
 * 16-byte aligned.  The library never allocates, frees, copies between host
 * and device, or synchronises: all work is enqueued on `stream` (a
 * hipStream_t; NULL = the legacy default stream) and the calls are legal
 * inside hipGraph stream capture.  The caller keeps every buffer alive until
 * the enqueued work has finished.  The library holds no state between calls;
 * concurrent calls need distinct workspaces.
 *
 * Layouts (row-major, contiguous; d_k = head_dim, d_v = head_dim_v or, when
 * that is 0, head_dim):
 *   q        bf16 [batch][h_q][d_k]
 *   k_cache  bf16 [batch][h_k][cache_len][d_k]
 *   v_cache  bf16 [batch][h_v][cache_len][d_v]
 *   out      bf16 [batch][h_q][d_v]           (round to nearest even)
 *   thresholds fp32 [batch][h_q]
 * A step attends rows 0 .. ctx_len-1 of each cache head.  Logits are
 * s_j = scale * <q, k_j> computed with fp32 products and sums; softmax and the
 * value sum are fp32.
 *
 * Status codes: every call validates all arguments before enqueuing anything
 * and returns a saga_status; nothing is launched on a non-zero status except
 * SAGA_ERR_HIP, which reports a failed launch (hipGetLastError) after a
 * partial enqueue.
 */
#ifndef SAGA_H
#define SAGA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum saga_status {
    SAGA_OK = 0,
    SAGA_ERR_INVALID_ARGUMENT = 1,   /* null pointer, bad dims, misalignment   */
    SAGA_ERR_UNSUPPORTED = 2,        /* valid but not implemented (head_dim...) */
    SAGA_ERR_WORKSPACE_TOO_SMALL = 3,
    SAGA_ERR_HIP = 4                 /* a kernel launch failed                  */
} saga_status;

/* Problem shape of one layer call.
 *   batch      >= 1
 *   h_q, h_k, h_v >= 1; h_k and h_v each divide h_q; h_q/h_k <= 16;
 *              batch * h_k <= 65535 and batch * h_q * cache_len <= 2^40, else
 *              SAGA_ERR_UNSUPPORTED
 *   head_dim   d_k, the q / key head dimension: 32, 64 or 128
 *   head_dim_v d_v, the value / output head dimension: 32, 64 or 128, or 0
 *              for d_v = d_k.  The key and value dimensions are independent
 *              (the pages compare a Sigma-style (h_k, d_k) = (2, 32) with
 *              SAGA's (1, 64) at h_v = 8, d_v = 64: ai.info summary, Main
 *              Findings, "head count beats head dimension")
 *   ctx_len    rows attended this step, 1 <= ctx_len <= cache_len
 *   cache_len  rows allocated per cache head (the head stride), < 2^27; one
 *              head must stay under 2 GiB (cache_len * max(d_k, d_v) * 2 <
 *              2^31, 8M rows at 128), else SAGA_ERR_UNSUPPORTED
 *   scale      multiplies q.k (use 1/sqrt(d_k) unless it is folded into q) */
typedef struct saga_dims {
    int32_t batch;
    int32_t h_q;
    int32_t h_k;
    int32_t h_v;
    int32_t head_dim;
    int32_t head_dim_v; /* 0: same as head_dim */
    int64_t ctx_len;
    int64_t cache_len;
    float scale;
    float reserved2;    /* must be 0 */
} saga_dims;

/* Bytes of device workspace that every call below needs for `dims` with any
 * ctx_len <= dims->cache_len and the given top_n.  One workspace may be reused
 * by every layer and step issued on one stream.  Returns 0 if the dims are
 * invalid.  Host-only; no device access. */
size_t saga_workspace_bytes(const saga_dims* dims, int32_t top_n);

/*
 * Exact top-N threshold refresh (Atop-N's "exact thresholds every n tokens";
 * ai.info summary, Key Contributions 2 and Methodology).
 *
 * For every (b, i): thresholds_dev[b][i] = the top_n-th largest fp32 logit
 * s[b][i][0..ctx_len) (counting repeated values), or -INFINITY when
 * top_n >= ctx_len.  The value is bit-identical to a logit that
 * saga_decode_step() computes for the same q and k_cache, so comparing with
 * it selects exactly top_n entries when there are no ties (ties at the
 * threshold are all kept).  -0.0 logits are ranked as +0.0.
 *
 * Cost.  One pass over K collects the candidates at or above a pivot taken
 * from a sample of at most 2048 rows (about 1.7 * top_n of them); the answer
 * is then selected among the candidates, in registers up to 8192 per row and
 * by three radix passes over the candidate lists above that, so any top_n
 * costs one K pass plus work proportional to top_n.  Only when the sample
 * misleads (fewer than top_n candidates, rare by construction) does a row
 * recompute its logits, three more passes over its key head.
 *
 *   q_dev, k_cache_dev   inputs, layouts above
 *   thresholds_dev       output fp32 [batch][h_q]
 *   logits_debug_dev     optional output fp32 [batch][h_q][ctx_len] (NULL: skip)
 *   workspace_dev        saga_workspace_bytes(dims, top_n) bytes
 * Errors: INVALID_ARGUMENT (null q/k/thresholds/workspace, top_n < 1, bad
 * dims), UNSUPPORTED, WORKSPACE_TOO_SMALL, HIP.
 */
int atopn_refresh_thresholds(const saga_dims* dims, int32_t top_n, const void* q_dev,
                             const void* k_cache_dev, float* thresholds_dev,
                             float* logits_debug_dev, void* workspace_dev,
                             size_t workspace_bytes, void* stream);

/*
 * One SAGA Atop-N decode step (selection by per-element comparison; sparse
 * probability-value product: ai.info summary, Key Contributions 2, Main
 * Findings first item).
 *
 * For every (b, i), with kappa = i/(h_q/h_k), nu = i/(h_q/h_v):
 *   s_j = scale * <q[b][i], k_cache[b][kappa][j]>          j < ctx_len
 *   S   = { j : s_j >= thresholds[b][i] }                   (fp32 compare)
 *   out[b][i] = sum_{j in S} softmax_S(s)_j * v_cache[b][nu][j]; zero if S = {}
 * Only the value rows in S are read.  The K cache is streamed once per
 * (b, key head) for all of that head's query heads.
 *
 *   thresholds_dev       input fp32 [batch][h_q] (from the last refresh)
 *   out_dev              output bf16 [batch][h_q][d_v]
 *   sel_counts_dev       optional output int32 [batch][h_q] = |S| (NULL: skip)
 *   sel_bitmap_debug_dev optional output uint32 [batch][h_q][ceil(cache_len/32)]:
 *                        bit j%32 of word j/32 set iff j in S; the library
 *                        clears it first (NULL: skip)
 * Errors: as above.
 */
int saga_decode_step(const saga_dims* dims, const void* q_dev, const void* k_cache_dev,
                     const void* v_cache_dev, const float* thresholds_dev, void* out_dev,
                     int32_t* sel_counts_dev, uint32_t* sel_bitmap_debug_dev,
                     void* workspace_dev, size_t workspace_bytes, void* stream);

/*
 * saga_decode_step() without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the workspace is a device array inside
 * the library, SAGA_NOALLOC_SCRATCH_BYTES bytes per device, held by each GPU
 * the library runs on until the process ends.  Results are bit-identical to
 * saga_decode_step() with the same arguments (no selection bitmap here).
 *
 * The call allocates nothing.  Its first call on a device looks the array up
 * (hipGetSymbolAddress, with that device current); make that first call
 * outside stream capture.  Every call on one device shares that device's
 * array: calls that overlap in time on one device (concurrent streams or
 * threads) race on it and must be serialised by the caller.  The array keeps
 * the last call's contents; nothing in it needs to start at zero.
 *
 * Errors: as saga_decode_step(), and SAGA_ERR_WORKSPACE_TOO_SMALL when
 * saga_workspace_bytes(dims, top_n) exceeds SAGA_NOALLOC_SCRATCH_BYTES (for
 * example batch 1 at 128K context fits; batch 16 does not).
 */
#define SAGA_NOALLOC_SCRATCH_BYTES (128u << 20)
int saga_decode_step_noalloc(const saga_dims* dims, const void* q_dev, const void* k_cache_dev,
                             const void* v_cache_dev, const float* thresholds_dev, void* out_dev,
                             int32_t* sel_counts_dev, void* stream);

/*
 * A refresh step in one call: the same results as atopn_refresh_thresholds()
 * followed by saga_decode_step() with the fresh thresholds, with one pass over
 * the K cache instead of two (the refresh's candidate lists already hold every
 * logit >= the new threshold).  This is the step the caller runs at
 * t mod n == 0.
 *
 *   thresholds_dev   output fp32 [batch][h_q] (kept for the following steps)
 *   out_dev          output bf16 [batch][h_q][d_v]
 *   sel_counts_dev   optional output int32 [batch][h_q] (NULL: skip)
 * Errors: as atopn_refresh_thresholds() and saga_decode_step().
 */
int atopn_refresh_decode_step(const saga_dims* dims, int32_t top_n, const void* q_dev,
                              const void* k_cache_dev, const void* v_cache_dev,
                              float* thresholds_dev, void* out_dev, int32_t* sel_counts_dev,
                              void* workspace_dev, size_t workspace_bytes, void* stream);

/*
 * Paged caches with per-sequence lengths (a serving-shaped cache: sequences of
 * different lengths sharing page pools; the step before the method proper,
 * needed to serve batched decode as the pages' batch-16 setting does).
 *
 *   k_pages bf16 [num_pages][h_k][page_rows][d_k]
 *   v_pages bf16 [num_pages][h_v][page_rows][d_v]
 * Row r (0-based, logical) of sequence b is row r % page_rows of page
 * block_table[b][r / page_rows] in both pools.  Sequence b attends rows
 * 0 .. ctx_lens[b]-1 (values outside [0, max_pages * page_rows] are clamped);
 * dims->ctx_len must be >= every ctx_lens[b] (it sizes the work split) and
 * dims->cache_len must equal max_pages * page_rows.  page_rows is a multiple of
 * 256.  A table entry outside [0, num_pages) reads as a page of zero rows that
 * contribute no value row.  Both arrays are device memory read by the kernels
 * (the call may be captured in a graph while they change between replays).
 */
typedef struct saga_paged {
    const int32_t* block_table_dev;  /* [batch][max_pages] page index           */
    const int32_t* ctx_lens_dev;     /* [batch] rows attended per sequence       */
    int32_t page_rows;               /* rows per page, a multiple of 256         */
    int32_t max_pages;               /* block_table row stride                   */
    int64_t num_pages;               /* pages in each pool                       */
    int64_t reserved;                /* must be 0                                */
} saga_paged;

/* The three Atop-N calls above on paged caches.  Same results per sequence as
 * the contiguous calls with ctx_len = ctx_lens[b] (for every b with
 * top_n >= ctx_lens[b], tau = -inf); the workspace is saga_workspace_bytes(dims,
 * top_n).  No debug outputs.  Errors: as the contiguous calls, plus
 * INVALID_ARGUMENT for a null or inconsistent saga_paged. */
int atopn_refresh_thresholds_paged(const saga_dims* dims, const saga_paged* paged, int32_t top_n,
                                   const void* q_dev, const void* k_pages_dev,
                                   float* thresholds_dev, void* workspace_dev,
                                   size_t workspace_bytes, void* stream);
int saga_decode_step_paged(const saga_dims* dims, const saga_paged* paged, const void* q_dev,
                           const void* k_pages_dev, const void* v_pages_dev,
                           const float* thresholds_dev, void* out_dev, int32_t* sel_counts_dev,
                           void* workspace_dev, size_t workspace_bytes, void* stream);
int atopn_refresh_decode_step_paged(const saga_dims* dims, const saga_paged* paged, int32_t top_n,
                                    const void* q_dev, const void* k_pages_dev,
                                    const void* v_pages_dev, float* thresholds_dev, void* out_dev,
                                    int32_t* sel_counts_dev, void* workspace_dev,
                                    size_t workspace_bytes, void* stream);

/*
 * Several query tokens per query head and step (speculative verification,
 * chunked prefill): the pages count the value vectors of a step as
 * h_q x l_q x N, one selection of N per query token.  Token j (0-based) of the
 * step sits at row ctx_len - l_q + j of the caches (the step's own rows are
 * already in them) and attends rows 0 .. ctx_len - l_q + j; it has its own
 * threshold, refreshed on the same schedule.  Per token the results equal the
 * one-token calls with that token's q at ctx_len - (l_q - 1 - j).
 *
 *   q_dev          bf16 [batch][h_q][l_q][d_k]
 *   thresholds_dev fp32 [batch][h_q][l_q]
 *   out_dev        bf16 [batch][h_q][l_q][d_v]
 *   sel_counts_dev optional int32 [batch][h_q][l_q]
 *   workspace      saga_workspace_bytes() of dims with h_q replaced by h_q * l_q
 * Requires 1 <= l_q <= ctx_len and (h_q / h_k) * l_q <= 16 (UNSUPPORTED
 * otherwise).  Errors otherwise as the one-token calls.
 */
int atopn_refresh_thresholds_lq(const saga_dims* dims, int32_t l_q, int32_t top_n,
                                const void* q_dev, const void* k_cache_dev, float* thresholds_dev,
                                void* workspace_dev, size_t workspace_bytes, void* stream);
int saga_decode_step_lq(const saga_dims* dims, int32_t l_q, const void* q_dev,
                        const void* k_cache_dev, const void* v_cache_dev,
                        const float* thresholds_dev, void* out_dev, int32_t* sel_counts_dev,
                        void* workspace_dev, size_t workspace_bytes, void* stream);
int atopn_refresh_decode_step_lq(const saga_dims* dims, int32_t l_q, int32_t top_n,
                                 const void* q_dev, const void* k_cache_dev,
                                 const void* v_cache_dev, float* thresholds_dev, void* out_dev,
                                 int32_t* sel_counts_dev, void* workspace_dev,
                                 size_t workspace_bytes, void* stream);

/*
 * An fp8 K cache (the pages list SAGA as combinable with cache quantization:
 * ai.info summary, Why This Matters).  The dominant K stream then reads one
 * byte per element instead of two; V stays bf16.
 *
 *   k8_cache_dev  [batch][h_k][cache_len][d_k] bytes, each an fp8 E4M3
 *                 value in the OCP 8-bit floating point format (bias 7, no
 *                 infinities, 0x7F / 0xFF are NaN, max 448)
 *   k_scale_dev   fp32 [batch][h_k] device memory: key row r of (b, g) is
 *                 k_scale[b][g] * decode(k8[b][g][r][:])
 * The logits are scale * k_scale[b][kappa(i)] * (q . decode(k8 row)), i.e. the
 * contiguous calls run on the dequantized cache; everything else (thresholds,
 * selection, outputs, workspace size, the debug outputs of the refresh and
 * decode calls) is as the contiguous calls.  The two E4M3 NaN codes are not
 * valid cache contents (results with them are unspecified).  Errors: as the
 * contiguous calls, plus INVALID_ARGUMENT for a null or misaligned
 * k_scale_dev and UNSUPPORTED for d_k = 32.
 */
int atopn_refresh_thresholds_fp8k(const saga_dims* dims, int32_t top_n, const void* q_dev,
                                  const void* k8_cache_dev, const float* k_scale_dev,
                                  float* thresholds_dev, float* logits_debug_dev,
                                  void* workspace_dev, size_t workspace_bytes, void* stream);
int saga_decode_step_fp8k(const saga_dims* dims, const void* q_dev, const void* k8_cache_dev,
                          const float* k_scale_dev, const void* v_cache_dev,
                          const float* thresholds_dev, void* out_dev, int32_t* sel_counts_dev,
                          uint32_t* sel_bitmap_debug_dev, void* workspace_dev,
                          size_t workspace_bytes, void* stream);
int atopn_refresh_decode_step_fp8k(const saga_dims* dims, int32_t top_n, const void* q_dev,
                                   const void* k8_cache_dev, const float* k_scale_dev,
                                   const void* v_cache_dev, float* thresholds_dev, void* out_dev,
                                   int32_t* sel_counts_dev, void* workspace_dev,
                                   size_t workspace_bytes, void* stream);

/*
 * fp8 K and V caches (the same quantization applied to the value cache as
 * well).  The V gather then reads d_v bytes per selected row instead of
 * 2 * d_v.  Thresholds come from atopn_refresh_thresholds_fp8k (they depend
 * on K only).
 *   v8_cache_dev  [batch][h_v][cache_len][d_v] bytes, fp8 E4M3 as k8_cache_dev
 *   v_scale_dev   fp32 [batch][h_v] device memory: value row r of (b, nu) is
 *                 v_scale[b][nu] * decode(v8[b][nu][r][:])
 * Outputs are the contiguous calls' on the dequantized caches (each output
 * row is accumulated on the decoded codes and scaled once by its value head's
 * scale); thresholds, selection, counts and workspace as the fp8 K calls.
 * Errors: as the fp8 K calls, plus INVALID_ARGUMENT for a null or misaligned
 * v_scale_dev.
 */
int saga_decode_step_fp8kv(const saga_dims* dims, const void* q_dev, const void* k8_cache_dev,
                           const float* k_scale_dev, const void* v8_cache_dev,
                           const float* v_scale_dev, const float* thresholds_dev, void* out_dev,
                           int32_t* sel_counts_dev, uint32_t* sel_bitmap_debug_dev,
                           void* workspace_dev, size_t workspace_bytes, void* stream);
int atopn_refresh_decode_step_fp8kv(const saga_dims* dims, int32_t top_n, const void* q_dev,
                                    const void* k8_cache_dev, const float* k_scale_dev,
                                    const void* v8_cache_dev, const float* v_scale_dev,
                                    float* thresholds_dev, void* out_dev,
                                    int32_t* sel_counts_dev, void* workspace_dev,
                                    size_t workspace_bytes, void* stream);

/*
 * Full (dense) decode attention over all ctx_len rows with the same head maps:
 * the full-attention GQA baseline the pages time against when h_k == h_v, and
 * "SAGA full attention" when h_k < h_v (ai.info summary, Main Findings:
 * end-to-end speedups and the merging-alone result).
 *   out[b][i] = softmax(s)_j-weighted sum of v_cache[b][nu][j], j < ctx_len.
 * Additionally requires that each key head's query heads map to 1, 2 or 4
 * value heads with at most 8 query heads per value head (UNSUPPORTED
 * otherwise).
 */
int saga_full_attention(const saga_dims* dims, const void* q_dev, const void* k_cache_dev,
                        const void* v_cache_dev, void* out_dev, void* workspace_dev,
                        size_t workspace_bytes, void* stream);

/* Static, human-readable name of a status code. */
const char* saga_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
int saga_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SAGA_H */

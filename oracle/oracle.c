/*
 * oracle.c -- plain, slow, fp64 CPU oracle for SAGA + Atop-N decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product (the HIP
 * library and its Python binding) never calls it, and this file shares no
 * code, header, table or helper with the product.
 *
 * Sources, cited by page title and section:
 *   [P1] "More Value per Key: Asymmetric Sparse Attention for Faster LLM
 *        Decoding", ai.info AI summary.
 *   [P2] the same paper, atlas.scime.ai AI summary.
 *   [F8] the OCP 8-bit floating point specification (OFP8), format E4M3:
 *        the fp8 key cache ([P1] Why This Matters: SAGA combines with cache
 *        quantization).
 *
 * What is computed (for each layer call, each batch row b, each query head i):
 *   - SAGA head maps: the key-head count h_k and the value-head count h_v are
 *     set independently of each other and of h_q ([P1] Key Contributions 3;
 *     [P2] Approach).  Query head i reads key head i / (h_q/h_k) and value
 *     head i / (h_q/h_v) (contiguous grouping; the pages leave the map open).
 *   - Logits s_j = scale * <q, k_j> over the attended context ([P1] Main
 *     Findings, first item: the query-key product is what remains dominant).
 *   - Atop-N ([P1] Key Contributions 2; Methodology): every n decode steps an
 *     exact top-N threshold is computed (here: sort, take the N-th largest);
 *     between refreshes that threshold is reused and the selected set is the
 *     per-element comparison s_j >= tau, with no sort.
 *   - The probability-value product touches only the selected entries
 *     ([P1] Main Findings, first item); softmax is renormalised over the
 *     selection.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   refresh at steps t with t mod n == 0, starting at t = 0, the fresh
 *   threshold used in the same step; inclusive comparison (ties kept);
 *   N >= ctx gives tau = -inf (select everything); an empty selection gives
 *   the zero vector; inputs are bf16 bit patterns, every product and sum is
 *   done in double.  An fp8 key cache holds E4M3 codes with one fp32 scale
 *   per (batch row, key head); key value = scale * decode(code), and the rest
 *   is the bf16 computation on those values.  The key/query head dimension d
 *   and the value/output head dimension dv are independent ([P1] Main
 *   Findings: a Sigma-style variant trades key heads for key head dimension).
 *
 * Precision: fp64 throughout on exactly the bf16 values the device sees.
 * Parallelism: one OpenMP loop over independent (b, i) pairs; nothing else.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- helpers */

/* A bf16 value is the upper half of an IEEE binary32; widen it exactly. */
static double bf16_to_double(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP E4M3 ([F8]): sign bit, 4 exponent bits (bias 7), 3 mantissa bits.
 * Exponent field 0 is subnormal, (m/8) * 2^-6; the all-ones code S.1111.111
 * is NaN; there are no infinities, so exponent field 15 with m < 7 is an
 * ordinary normal (largest 1.75 * 2^8 = 448). */
static double e4m3_to_double(uint8_t code)
{
    const int sign = code >> 7, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7) return NAN;
    const double mag = e == 0 ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/* A key or value cache [B][H][cache_len][d]: bf16 bit patterns, or E4M3
 * codes with one scale per (batch row, head): element = scale * e4m3(code). */
typedef struct {
    const uint16_t* bf16;
    const uint8_t* e4m3;
    const float* scale;   /* [B][H], with e4m3 */
} kv_cache;

/* Row 0 of one head of a cache. */
typedef struct {
    const uint16_t* bf16;
    const uint8_t* e4m3;
    double scale;
} kv_head;

static kv_head head_of(const kv_cache* kc, int b, int H, int h, int64_t cache_len, int d)
{
    kv_head r = {NULL, NULL, 1.0};
    const int64_t off = (((int64_t)b * H + h) * cache_len) * d;
    if (kc->e4m3) {
        r.e4m3 = kc->e4m3 + off;
        r.scale = (double)kc->scale[(int64_t)b * H + h];
    } else {
        r.bf16 = kc->bf16 + off;
    }
    return r;
}

/* Element idx (= j * d + c) of a head, as a double. */
static double elem_at(const kv_head* k, int64_t idx)
{
    if (k->e4m3) return k->scale * e4m3_to_double(k->e4m3[idx]);
    return bf16_to_double(k->bf16[idx]);
}

static int check_dims(int B, int hq, int hk, int hv, int d, int dv, int64_t cache_len)
{
    if (B < 1 || hq < 1 || hk < 1 || hv < 1 || d < 1 || dv < 1 || cache_len < 1) return 1;
    if (hq % hk != 0 || hq % hv != 0) return 1;
    return 0;
}

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

/* Pointer to row 0 of head h of batch row b in a [B][H][cache_len][d] cache. */
static const uint16_t* cache_head(const uint16_t* cache, int b, int H, int h,
                                  int64_t cache_len, int d)
{
    return cache + (((int64_t)b * H + h) * cache_len) * d;
}

/* s[j] = scale * sum_c q[c] * K[j][c], for j < ctx  (one query head). */
static void head_logits(const uint16_t* q, const kv_head* Kh, int d, int64_t ctx,
                        double scale, double* s)
{
    for (int64_t j = 0; j < ctx; ++j) {
        double acc = 0.0;
        for (int c = 0; c < d; ++c)
            acc += bf16_to_double(q[c]) * elem_at(Kh, j * d + c);
        s[j] = scale * acc;
    }
}

static int cmp_double_desc(const void* a, const void* b)
{
    double x = *(const double*)a, y = *(const double*)b;
    return (x < y) - (x > y);
}

/* The N-th largest of s[0..n), or -inf when N >= n (everything selected). */
static double nth_largest(const double* s, int64_t n, int64_t N)
{
    if (N >= n) return -INFINITY;
    double* tmp = (double*)malloc(sizeof(double) * (size_t)n);
    memcpy(tmp, s, sizeof(double) * (size_t)n);
    qsort(tmp, (size_t)n, sizeof(double), cmp_double_desc);
    double t = tmp[N - 1];
    free(tmp);
    return t;
}

/* Softmax-weighted average of value rows over the entries with sel[j] != 0:
 *   m = max_S s_j, w_j = exp(s_j - m), out = sum_S w_j V_j / sum_S w_j.
 * An empty selection gives out = 0.  Returns |S|. */
static int64_t attend_selected(const double* s, const unsigned char* sel, int64_t ctx,
                               const kv_head* Vh, int dv, double* out)
{
    int64_t count = 0;
    double m = -INFINITY;
    for (int64_t j = 0; j < ctx; ++j)
        if (sel[j]) { ++count; if (s[j] > m) m = s[j]; }
    for (int c = 0; c < dv; ++c) out[c] = 0.0;
    if (count == 0) return 0;
    double denom = 0.0;
    for (int64_t j = 0; j < ctx; ++j) {
        if (!sel[j]) continue;
        double w = exp(s[j] - m);
        denom += w;
        for (int c = 0; c < dv; ++c) out[c] += w * elem_at(Vh, j * dv + c);
    }
    for (int c = 0; c < dv; ++c) out[c] /= denom;
    return count;
}

/* ------------------------------------------------------------- public API */

static int logits_impl(int B, int hq, int hk, int hv, int d, int64_t cache_len, int64_t ctx,
                       double scale, const uint16_t* q, const kv_cache* K, double* s,
                       int nthreads)
{
    if (check_dims(B, hq, hk, hv, d, d, cache_len) || ctx < 1 || ctx > cache_len) return 1;
    set_threads(nthreads);
    const int Gk = hq / hk;
#pragma omp parallel for schedule(dynamic, 1)
    for (int bi = 0; bi < B * hq; ++bi) {
        int b = bi / hq, i = bi % hq;
        const kv_head Kh = head_of(K, b, hk, i / Gk, cache_len, d);
        head_logits(q + (int64_t)bi * d, &Kh, d, ctx, scale, s + (int64_t)bi * ctx);
    }
    return 0;
}

/* Logits of one decode step for every (b, i): out s[B][hq][ctx]. */
int oracle_logits(int B, int hq, int hk, int hv, int d, int64_t cache_len, int64_t ctx,
                  double scale, const uint16_t* q, const uint16_t* K, double* s,
                  int nthreads)
{
    const kv_cache kc = {K, NULL, NULL};
    return logits_impl(B, hq, hk, hv, d, cache_len, ctx, scale, q, &kc, s, nthreads);
}

/* The same with an E4M3 key cache K8 and per-(b, key head) scales k_scale. */
int oracle_logits_e4m3k(int B, int hq, int hk, int hv, int d, int64_t cache_len, int64_t ctx,
                        double scale, const uint16_t* q, const uint8_t* K8,
                        const float* k_scale, double* s, int nthreads)
{
    const kv_cache kc = {NULL, K8, k_scale};
    return logits_impl(B, hq, hk, hv, d, cache_len, ctx, scale, q, &kc, s, nthreads);
}

/* Decode n E4M3 codes ([F8]) to doubles (NaN for the two NaN codes). */
void oracle_e4m3_decode(const uint8_t* codes, int64_t n, double* out)
{
    for (int64_t k = 0; k < n; ++k) out[k] = e4m3_to_double(codes[k]);
}

/* Exact top-N threshold of one logit row: the N-th largest value, -inf if N >= n. */
double oracle_nth_largest(const double* s, int64_t n, int64_t N)
{
    if (n < 1 || N < 1) return NAN;
    return nth_largest(s, n, N);
}

/*
 * Atop-N over T decode steps of one layer ([P1] Key Contributions 2 and
 * Methodology; [P1] Main Findings, first item), for every (b, i):
 *   1. key head kappa = i / (hq/hk), value head nu = i / (hq/hv);
 *   2. s_j = scale * <q_t[b,i], K[b,kappa,j]> for j < ctx[t];
 *   3. if t mod refresh_n == 0: tau = N-th largest s_j (sorted), or -inf when
 *      N >= ctx[t]; otherwise tau is kept from the last refresh;
 *   4. S = { j < ctx[t] : s_j >= tau };
 *   5. out = softmax over S of s, applied to V[b,nu] rows; zero if S is empty.
 *
 *   q      [T][B][hq][d]      bf16 bits      K [B][hk][cache_len][d] bf16 bits
 *   ctx    [T]                rows attended  V [B][hv][cache_len][d] bf16 bits
 *   out    [T][B][hq][d]      double
 *   tau    [T][B][hq]         double  (threshold in force at step t)
 *   count  [T][B][hq]         int64   (|S|)
 *   sel    [T][B][hq][cache_len] uint8, nullable (1 = selected)
 *   logits [T][B][hq][cache_len] double, nullable
 */
static int atopn_run_impl(int B, int hq, int hk, int hv, int d, int dv, int64_t cache_len,
                          int T, const int64_t* ctx, double scale, int64_t top_n,
                          int64_t refresh_n, const uint16_t* q, const kv_cache* K,
                          const kv_cache* V, double* out, double* tau, int64_t* count,
                          unsigned char* sel, double* logits, int nthreads)
{
    if (check_dims(B, hq, hk, hv, d, dv, cache_len) || T < 1 || top_n < 1 || refresh_n < 1)
        return 1;
    for (int t = 0; t < T; ++t)
        if (ctx[t] < 1 || ctx[t] > cache_len) return 1;
    set_threads(nthreads);
    const int Gk = hq / hk, Gv = hq / hv;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
    for (int bi = 0; bi < B * hq; ++bi) {
        const int b = bi / hq, i = bi % hq;
        const kv_head Kh = head_of(K, b, hk, i / Gk, cache_len, d);
        const kv_head Vh = head_of(V, b, hv, i / Gv, cache_len, dv);
        double* s = (double*)malloc(sizeof(double) * (size_t)cache_len);
        unsigned char* S = (unsigned char*)malloc((size_t)cache_len);
        if (!s || !S) { err = 1; free(s); free(S); continue; }
        double threshold = NAN;
        for (int t = 0; t < T; ++t) {
            const int64_t n = ctx[t];
            const int64_t row = (int64_t)t * B * hq + bi;
            head_logits(q + row * d, &Kh, d, n, scale, s);
            if (t % refresh_n == 0) threshold = nth_largest(s, n, top_n);
            for (int64_t j = 0; j < n; ++j) S[j] = (s[j] >= threshold);
            count[row] = attend_selected(s, S, n, &Vh, dv, out + row * dv);
            tau[row] = threshold;
            if (sel) {
                memset(sel + row * cache_len, 0, (size_t)cache_len);
                memcpy(sel + row * cache_len, S, (size_t)n);
            }
            if (logits) {
                for (int64_t j = 0; j < cache_len; ++j)
                    logits[row * cache_len + j] = j < n ? s[j] : 0.0;
            }
        }
        free(s);
        free(S);
    }
    return err;
}

int oracle_atopn_run(int B, int hq, int hk, int hv, int d, int dv, int64_t cache_len,
                     int T, const int64_t* ctx, double scale, int64_t top_n,
                     int64_t refresh_n, const uint16_t* q, const uint16_t* K,
                     const uint16_t* V, double* out, double* tau, int64_t* count,
                     unsigned char* sel, double* logits, int nthreads)
{
    const kv_cache kc = {K, NULL, NULL}, vc = {V, NULL, NULL};
    return atopn_run_impl(B, hq, hk, hv, d, dv, cache_len, T, ctx, scale, top_n, refresh_n, q,
                          &kc, &vc, out, tau, count, sel, logits, nthreads);
}

/* Atop-N as above with an E4M3 key cache K8 [B][hk][cache_len][d] and
 * per-(b, key head) scales k_scale [B][hk]. */
int oracle_atopn_run_e4m3k(int B, int hq, int hk, int hv, int d, int dv, int64_t cache_len,
                           int T, const int64_t* ctx, double scale, int64_t top_n,
                           int64_t refresh_n, const uint16_t* q, const uint8_t* K8,
                           const float* k_scale, const uint16_t* V, double* out, double* tau,
                           int64_t* count, unsigned char* sel, double* logits, int nthreads)
{
    const kv_cache kc = {NULL, K8, k_scale}, vc = {V, NULL, NULL};
    return atopn_run_impl(B, hq, hk, hv, d, dv, cache_len, T, ctx, scale, top_n, refresh_n, q,
                          &kc, &vc, out, tau, count, sel, logits, nthreads);
}

/* Atop-N with E4M3 key and value caches: K8 [B][hk][cache_len][d] with
 * k_scale [B][hk], V8 [B][hv][cache_len][dv] with v_scale [B][hv]; a value
 * element is v_scale * e4m3(code), decoded like a key element. */
int oracle_atopn_run_e4m3kv(int B, int hq, int hk, int hv, int d, int dv, int64_t cache_len,
                            int T, const int64_t* ctx, double scale, int64_t top_n,
                            int64_t refresh_n, const uint16_t* q, const uint8_t* K8,
                            const float* k_scale, const uint8_t* V8, const float* v_scale,
                            double* out, double* tau, int64_t* count, unsigned char* sel,
                            double* logits, int nthreads)
{
    const kv_cache kc = {NULL, K8, k_scale}, vc = {NULL, V8, v_scale};
    return atopn_run_impl(B, hq, hk, hv, d, dv, cache_len, T, ctx, scale, top_n, refresh_n, q,
                          &kc, &vc, out, tau, count, sel, logits, nthreads);
}

/* One step with the selection given by the caller as a bitmap
 * [B][hq][ceil(cache_len/32)] (bit j%32 of word j/32 selects row j): the
 * "use the device's mask" mode that isolates softmax and PV from selection. */
static int masked_impl(int B, int hq, int hk, int hv, int d, int dv, int64_t cache_len, int64_t ctx,
                       double scale, const uint16_t* q, const kv_cache* K, const kv_cache* V,
                       const uint32_t* bitmap, double* out, int64_t* count, int nthreads)
{
    if (check_dims(B, hq, hk, hv, d, dv, cache_len) || ctx < 1 || ctx > cache_len) return 1;
    set_threads(nthreads);
    const int Gk = hq / hk, Gv = hq / hv;
    const int64_t words = (cache_len + 31) / 32;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
    for (int bi = 0; bi < B * hq; ++bi) {
        const int b = bi / hq, i = bi % hq;
        double* s = (double*)malloc(sizeof(double) * (size_t)ctx);
        unsigned char* S = (unsigned char*)malloc((size_t)ctx);
        if (!s || !S) { err = 1; free(s); free(S); continue; }
        const kv_head Kh = head_of(K, b, hk, i / Gk, cache_len, d);
        head_logits(q + (int64_t)bi * d, &Kh, d, ctx, scale, s);
        const uint32_t* bits = bitmap + (int64_t)bi * words;
        for (int64_t j = 0; j < ctx; ++j) S[j] = (bits[j / 32] >> (j % 32)) & 1u;
        const kv_head Vh = head_of(V, b, hv, i / Gv, cache_len, dv);
        count[bi] = attend_selected(s, S, ctx, &Vh, dv, out + (int64_t)bi * dv);
        free(s);
        free(S);
    }
    return err;
}

int oracle_masked(int B, int hq, int hk, int hv, int d, int dv, int64_t cache_len, int64_t ctx,
                  double scale, const uint16_t* q, const uint16_t* K, const uint16_t* V,
                  const uint32_t* bitmap, double* out, int64_t* count, int nthreads)
{
    const kv_cache kc = {K, NULL, NULL}, vc = {V, NULL, NULL};
    return masked_impl(B, hq, hk, hv, d, dv, cache_len, ctx, scale, q, &kc, &vc, bitmap, out, count,
                       nthreads);
}

/* One step over a caller-given bitmap with an E4M3 key cache. */
int oracle_masked_e4m3k(int B, int hq, int hk, int hv, int d, int dv, int64_t cache_len, int64_t ctx,
                        double scale, const uint16_t* q, const uint8_t* K8,
                        const float* k_scale, const uint16_t* V, const uint32_t* bitmap,
                        double* out, int64_t* count, int nthreads)
{
    const kv_cache kc = {NULL, K8, k_scale}, vc = {V, NULL, NULL};
    return masked_impl(B, hq, hk, hv, d, dv, cache_len, ctx, scale, q, &kc, &vc, bitmap, out, count,
                       nthreads);
}

/* One step over a caller-given bitmap with E4M3 key and value caches. */
int oracle_masked_e4m3kv(int B, int hq, int hk, int hv, int d, int dv, int64_t cache_len,
                         int64_t ctx, double scale, const uint16_t* q, const uint8_t* K8,
                         const float* k_scale, const uint8_t* V8, const float* v_scale,
                         const uint32_t* bitmap, double* out, int64_t* count, int nthreads)
{
    const kv_cache kc = {NULL, K8, k_scale}, vc = {NULL, V8, v_scale};
    return masked_impl(B, hq, hk, hv, d, dv, cache_len, ctx, scale, q, &kc, &vc, bitmap, out, count,
                       nthreads);
}

typedef struct { double s; int64_t j; } scored_index;

static int cmp_scored_desc(const void* a, const void* b)
{
    const scored_index* x = (const scored_index*)a;
    const scored_index* y = (const scored_index*)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->j > y->j) - (x->j < y->j);
}

/* Exact top-N attention of one step (a baseline the pages list, [P2]
 * Experimental setup): rank the indices by logit (descending, index breaks
 * ties), keep the first min(N, ctx), softmax over those and apply to V.
 * Written without thresholds, independently of oracle_atopn_run. */
int oracle_exact_topn(int B, int hq, int hk, int hv, int d, int dv, int64_t cache_len, int64_t ctx,
                      double scale, int64_t top_n, const uint16_t* q, const uint16_t* K,
                      const uint16_t* V, double* out, int nthreads)
{
    if (check_dims(B, hq, hk, hv, d, dv, cache_len) || ctx < 1 || ctx > cache_len || top_n < 1)
        return 1;
    set_threads(nthreads);
    const int Gk = hq / hk, Gv = hq / hv;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
    for (int bi = 0; bi < B * hq; ++bi) {
        const int b = bi / hq, i = bi % hq;
        const uint16_t* Kh = cache_head(K, b, hk, i / Gk, cache_len, d);
        const uint16_t* Vh = cache_head(V, b, hv, i / Gv, cache_len, dv);
        const uint16_t* qi = q + (int64_t)bi * d;
        scored_index* idx = (scored_index*)malloc(sizeof(scored_index) * (size_t)ctx);
        if (!idx) { err = 1; continue; }
        for (int64_t j = 0; j < ctx; ++j) {
            double acc = 0.0;
            for (int c = 0; c < d; ++c)
                acc += bf16_to_double(qi[c]) * bf16_to_double(Kh[j * d + c]);
            idx[j].s = scale * acc;
            idx[j].j = j;
        }
        qsort(idx, (size_t)ctx, sizeof(scored_index), cmp_scored_desc);
        const int64_t keep = top_n < ctx ? top_n : ctx;
        double* o = out + (int64_t)bi * dv;
        for (int c = 0; c < dv; ++c) o[c] = 0.0;
        double denom = 0.0;
        for (int64_t r = 0; r < keep; ++r) {
            double w = exp(idx[r].s - idx[0].s); /* idx[0] holds the maximum */
            denom += w;
            for (int c = 0; c < dv; ++c) o[c] += w * bf16_to_double(Vh[idx[r].j * dv + c]);
        }
        for (int c = 0; c < dv; ++c) o[c] /= denom;
        free(idx);
    }
    return err;
}

/* Full (dense) decode attention of one step: softmax over every attended row.
 * This is the full-attention GQA/SAGA baseline the pages time against
 * ([P1] Main Findings, end-to-end speedups and the flash-attention note). */
int oracle_full(int B, int hq, int hk, int hv, int d, int dv, int64_t cache_len, int64_t ctx,
                double scale, const uint16_t* q, const uint16_t* K, const uint16_t* V,
                double* out, int nthreads)
{
    if (check_dims(B, hq, hk, hv, d, dv, cache_len) || ctx < 1 || ctx > cache_len) return 1;
    set_threads(nthreads);
    const int Gk = hq / hk, Gv = hq / hv;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
    for (int bi = 0; bi < B * hq; ++bi) {
        const int b = bi / hq, i = bi % hq;
        const kv_cache kc = {K, NULL, NULL};
        const kv_head Kh = head_of(&kc, b, hk, i / Gk, cache_len, d);
        const uint16_t* Vh = cache_head(V, b, hv, i / Gv, cache_len, dv);
        double* s = (double*)malloc(sizeof(double) * (size_t)ctx);
        if (!s) { err = 1; continue; }
        head_logits(q + (int64_t)bi * d, &Kh, d, ctx, scale, s);
        double m = -INFINITY;
        for (int64_t j = 0; j < ctx; ++j) if (s[j] > m) m = s[j];
        double* o = out + (int64_t)bi * dv;
        for (int c = 0; c < dv; ++c) o[c] = 0.0;
        double denom = 0.0;
        for (int64_t j = 0; j < ctx; ++j) {
            double w = exp(s[j] - m);
            denom += w;
            for (int c = 0; c < dv; ++c) o[c] += w * bf16_to_double(Vh[j * dv + c]);
        }
        for (int c = 0; c < dv; ++c) o[c] /= denom;
        free(s);
    }
    return err;
}

/* Threads an OpenMP region of this library will use (for reporting). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

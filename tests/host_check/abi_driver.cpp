// abi_driver.cpp -- drives every entry point of include/saga.h through the
// library's own host code (api.hip), built for the CPU together with
// launch_stubs.cpp under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// Host heap buffers of exactly the documented sizes stand in for device
// memory (the host code never dereferences them; the stubs touch the extreme
// elements each kernel would).  Two parts:
//   * valid calls on a table of shapes (the benchmark shapes included), each
//     of which must return SAGA_OK and launch work;
//   * the error paths: each bad argument must return its documented status
//     and launch nothing.
// Exit status 0 when every check holds; a sanitizer report or a failed check
// aborts with a message.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "saga.h"

namespace saga {
extern int g_launches;
extern int g_fused_launches;
extern int g_tail_launches;
struct TouchedRange {
    const char* name;
    uintptr_t lo, hi;
};
extern std::vector<TouchedRange> g_ranges;
}

namespace {

int g_failures = 0;
int g_checks = 0;

#define CHECK(cond, ...)                                                      \
    do {                                                                      \
        ++g_checks;                                                           \
        if (!(cond)) {                                                        \
            ++g_failures;                                                     \
            fprintf(stderr, "FAIL %s:%d: %s -- ", __FILE__, __LINE__, #cond); \
            fprintf(stderr, __VA_ARGS__);                                     \
            fprintf(stderr, "\n");                                            \
        }                                                                     \
    } while (0)

// Exact-size, 256-byte-aligned host buffers, freed at scope end.
struct Arena {
    std::vector<void*> ptrs;
    void* get(size_t bytes)
    {
        if (bytes == 0) return nullptr;
        void* p = nullptr;
        if (posix_memalign(&p, 256, bytes) != 0) {
            fprintf(stderr, "out of host memory (%zu bytes)\n", bytes);
            abort();
        }
        ptrs.push_back(p);
        return p;
    }
    ~Arena()
    {
        for (void* p : ptrs) free(p);
    }
};

struct Shape {
    const char* name;
    int B, hq, hk, hv, dk, dv;   // dv: 0 = dk
    int64_t cache_len;
    int top_n;
};

// The named workspace regions the kernels of one call used: each inside the
// workspace, and no two different regions overlapping.
void check_regions(const void* ws, size_t wsb, const char* what)
{
    const uintptr_t w0 = reinterpret_cast<uintptr_t>(ws), w1 = w0 + wsb;
    const std::vector<saga::TouchedRange>& r = saga::g_ranges;
    for (size_t i = 0; i < r.size(); ++i) {
        if (r[i].hi <= w0 || r[i].lo >= w1) continue;      // not a workspace region
        CHECK(r[i].lo >= w0 && r[i].hi <= w1, "%s: %s leaves the workspace", what, r[i].name);
        for (size_t j = 0; j < r.size(); ++j) {
            if (strcmp(r[i].name, r[j].name) == 0) continue;
            const bool overlap = r[i].lo < r[j].hi && r[j].lo < r[i].hi;
            CHECK(!overlap, "%s: workspace regions %s and %s overlap", what, r[i].name, r[j].name);
        }
    }
    saga::g_ranges.clear();
}

saga_dims make_dims(const Shape& s, int64_t ctx)
{
    saga_dims d;
    memset(&d, 0, sizeof d);
    d.batch = s.B;
    d.h_q = s.hq;
    d.h_k = s.hk;
    d.h_v = s.hv;
    d.head_dim = s.dk;
    d.head_dim_v = s.dv;
    d.ctx_len = ctx;
    d.cache_len = s.cache_len;
    d.scale = 0.125f;
    return d;
}

// Each (query head -> value head) group of a key head's query heads spans at
// most 4 value heads with at most 8 query heads per value head (the dense
// kernel's limits, documented in saga.h).
bool full_supported(const Shape& s)
{
    const int Gk = s.hq / s.hk, Gv = s.hq / s.hv;
    int nv = 1, maxs = 1;
    for (int g = 0; g < s.hk; ++g) {
        const int i0 = g * Gk, v0 = i0 / Gv, v1 = (i0 + Gk - 1) / Gv;
        if (v1 - v0 + 1 > nv) nv = v1 - v0 + 1;
        for (int vh = v0; vh <= v1; ++vh) {
            const int lo = vh * Gv > i0 ? vh * Gv : i0;
            const int hi = (vh + 1) * Gv < i0 + Gk ? (vh + 1) * Gv : i0 + Gk;
            if (hi - lo > maxs) maxs = hi - lo;
        }
    }
    return nv <= 4 && maxs <= 8;
}

// Which path saga_decode_step takes: the small-batch path needs at most four
// (b, key head) groups and a plan of at least 64 workgroups whose worst case
// fits the LDS with the whole launch resident.  Otherwise the K stream gathers
// in its tail when V is contiguous bf16 with d_v = d_k of 64, or of 128 with
// chunks of at least 2048 rows, and the launch has at least 256 workgroups;
// else the list path (stream, gather, combine).
void plan_choices()
{
    struct Case {
        Shape s;
        int64_t ctx;
        bool fused;
        bool fp8k = false;   // the fp8 K call
        bool tail = false;   // the K stream gathers in its tail
        bool fp8kv = false;  // the fp8 K and V call
    };
    const Case cases[] = {
        {{"qwen_like_128k_b1", 1, 12, 1, 2, 128, 0, 131104, 1024}, 131104, true},
        {{"tiny_8k_b1", 1, 4, 1, 2, 64, 0, 8200, 64}, 8192, true},               // smoke(): 64
        {{"tiny_b1", 1, 4, 1, 2, 64, 0, 1032, 64}, 1024, false},                // smoke(): 8
        {{"tiny_b64", 64, 4, 1, 2, 64, 0, 1032, 64}, 1024, false, false, true}, // smoke(): 512
        {{"qwen_like_4k_b1", 1, 12, 1, 2, 128, 0, 4111, 1024}, 4111, false},     // 33 workgroups
        {{"qwen_like_8k_b1", 1, 12, 1, 2, 128, 0, 8207, 1024}, 8207, true},      // 65
        {{"qwen_like_16k_b1", 1, 12, 1, 2, 128, 0, 16399, 1024}, 16399, true},   // 129
        {{"llama_like_8k_b1", 1, 32, 4, 8, 64, 0, 8207, 512}, 8207, true},
        {{"llama_like_64k_b1", 1, 32, 4, 8, 64, 0, 65551, 1024}, 65551, true},
        {{"llama_like_128k_b1", 1, 32, 4, 8, 64, 0, 131104, 2048}, 131104, true},
        {{"llama_like_128k_b2", 2, 32, 4, 8, 64, 0, 131104, 2048}, 131104, false, false, true},  // 8 groups
        {{"qwen_like_40k_b1_fp8k", 1, 12, 1, 2, 128, 0, 40003, 500}, 40000, true, true},
        {{"qwen_like_3k_b2_fp8k", 2, 12, 1, 2, 128, 0, 3005, 100}, 3000, false, true},
        {{"dk64_dv128_40k_b1", 1, 12, 1, 2, 64, 128, 40003, 500}, 40000, true},
        {{"sigma_like_dk32_dv64_30k", 1, 16, 2, 8, 32, 64, 30003, 300}, 30000, true},
        // Large batches: the tail gather, or the list path where it does not apply.
        {{"llama_like_128k_b16", 16, 32, 4, 8, 64, 0, 131104, 2048}, 131104, false, false, true},
        {{"qwen_like_128k_b16", 16, 12, 1, 2, 128, 0, 131104, 1024}, 131104, false, false, true},
        {{"llama_like_128k_b16_fp8k", 16, 32, 4, 8, 64, 0, 131104, 2048}, 131104, false, true, true},
        {{"tail_llama_like_2k_b4", 4, 32, 4, 8, 64, 0, 2103, 100}, 2100, false, false, true},    // 272
        {{"qwen_like_4k_b16", 16, 12, 1, 2, 128, 0, 4103, 200}, 4100, false, false, false},  // 128-row chunks
        {{"qwen_like_32k_b16", 16, 12, 1, 2, 128, 0, 32771, 1024}, 32768, false, false, false},  // 1024
        {{"qwen_like_64k_b16", 16, 12, 1, 2, 128, 0, 65539, 1024}, 65536, false, false, true},   // 2048
        {{"tail_qwen_like_16k_b32", 32, 24, 2, 4, 128, 0, 16403, 200}, 16400, false, false, true},
        {{"tail_group16_d128_b32", 32, 32, 2, 8, 128, 0, 16403, 300}, 16400, false, false, true},
        {{"tail_fewer_value_heads_b8", 8, 8, 4, 2, 64, 0, 1103, 50}, 1100, false, false, true},
        {{"tail_mha_d64_b4", 4, 8, 8, 8, 64, 0, 1103, 40}, 1100, false, false, true},
        {{"tail_fp8k_llama_like_b4", 4, 32, 4, 8, 64, 0, 2503, 64}, 2500, false, true, true},
        {{"llama_like_128k_b16_fp8kv", 16, 32, 4, 8, 64, 0, 131104, 2048}, 131104, false, false, true, true},
        {{"tail_fp8kv_qwen_like_16k_b32", 32, 24, 2, 4, 128, 0, 16403, 200}, 16400, false, false, true, true},
        {{"qwen_like_4k_b16_fp8kv", 16, 12, 1, 2, 128, 0, 4103, 200}, 4100, false, false, false, true},
        {{"gqa_llama_small_b2", 2, 32, 8, 8, 64, 0, 2052, 64}, 2049, false, false, true},   // 272
        {{"tail_group16_d64_b16", 16, 16, 1, 4, 64, 0, 2103, 100}, 2100, false, false, true}, // 272
        {{"llama_like_1k_b4", 4, 32, 4, 8, 64, 0, 1024, 64}, 1000, false, false, false},    // 128
        {{"group16_d64_b16", 16, 16, 1, 4, 64, 0, 8200, 300}, 8192, false, false, true},    // G_k 16
        {{"dk64_dv128_b16", 16, 12, 1, 2, 64, 128, 8200, 300}, 8192, false, false, false},  // d_v != d_k
        {{"mha_d32_b16", 16, 8, 8, 8, 32, 0, 8200, 300}, 8192, false, false, false},        // d = 32
    };
    for (const Case& c : cases) {
        const Shape& s = c.s;
        const int dv = s.dv ? s.dv : s.dk;
        const int64_t bh = (int64_t)s.B * s.hq;
        Arena a;
        void* q = a.get(bh * s.dk * 2);
        void* k = a.get((size_t)s.B * s.hk * s.cache_len * s.dk * 2);
        void* v = a.get((size_t)s.B * s.hv * s.cache_len * dv * 2);
        float* ks = static_cast<float*>(a.get((size_t)s.B * s.hk * 4));
        float* vs = static_cast<float*>(a.get((size_t)s.B * s.hv * 4));
        float* tau = static_cast<float*>(a.get(bh * 4));
        void* out = a.get(bh * dv * 2);
        const saga_dims d = make_dims(s, c.ctx);
        const size_t wsb = saga_workspace_bytes(&d, s.top_n);
        void* ws = a.get(wsb);
        saga::g_launches = saga::g_fused_launches = saga::g_tail_launches = 0;
        const int st =
            c.fp8kv ? saga_decode_step_fp8kv(&d, q, k, ks, v, vs, tau, out, nullptr, nullptr, ws,
                                             wsb, nullptr)
            : c.fp8k ? saga_decode_step_fp8k(&d, q, k, ks, v, tau, out, nullptr, nullptr, ws, wsb,
                                             nullptr)
                     : saga_decode_step(&d, q, k, v, tau, out, nullptr, nullptr, ws, wsb, nullptr);
        CHECK(st == SAGA_OK, "%s: status %d", s.name, st);
        CHECK((saga::g_fused_launches > 0) == c.fused, "%s: small-batch path %s", s.name,
              c.fused ? "expected" : "not expected");
        CHECK((saga::g_tail_launches > 0) == c.tail, "%s: tail gather %s", s.name,
              c.tail ? "expected" : "not expected");
        saga::g_ranges.clear();
    }
    saga::g_launches = saga::g_fused_launches = saga::g_tail_launches = 0;
    fprintf(stderr, "plan choices checked\n");
}

void valid_calls(const Shape& s)
{
    const int dv = s.dv ? s.dv : s.dk;
    const int64_t bh = (int64_t)s.B * s.hq;
    const int64_t words = (s.cache_len + 31) / 32;
    Arena a;
    void* q = a.get(bh * s.dk * 2);
    void* k = a.get((size_t)s.B * s.hk * s.cache_len * s.dk * 2);
    void* v = a.get((size_t)s.B * s.hv * s.cache_len * dv * 2);
    void* k8 = s.dk >= 64 ? a.get((size_t)s.B * s.hk * s.cache_len * s.dk) : nullptr;
    void* v8 = s.dk >= 64 ? a.get((size_t)s.B * s.hv * s.cache_len * dv) : nullptr;
    float* ks = static_cast<float*>(a.get((size_t)s.B * s.hk * 4));
    float* vs = static_cast<float*>(a.get((size_t)s.B * s.hv * 4));
    float* tau = static_cast<float*>(a.get(bh * 4));
    void* out = a.get(bh * dv * 2);
    int32_t* cnt = static_cast<int32_t*>(a.get(bh * 4));
    uint32_t* bm = static_cast<uint32_t*>(a.get(bh * words * 4));
    const saga_dims d0 = make_dims(s, s.cache_len);
    const size_t wsb = saga_workspace_bytes(&d0, s.top_n);
    CHECK(wsb > 0, "%s: workspace size", s.name);
    void* ws = a.get(wsb);

    int64_t ctxs[4] = {s.cache_len, s.cache_len > 40 ? s.cache_len - 37 : 1,
                       s.cache_len < 17 ? s.cache_len : 17, 1};
    for (const int64_t ctx : ctxs) {
        const saga_dims d = make_dims(s, ctx);
        CHECK(saga_workspace_bytes(&d, s.top_n) == wsb, "%s: layout depends on ctx", s.name);
        Arena b;
        float* lg = static_cast<float*>(b.get(bh * ctx * 4));
        void* cur_ws = ws;
        size_t cur_wsb = wsb;
        auto ok = [&](int st, const char* call) {
            CHECK(st == SAGA_OK, "%s ctx=%lld %s: status %d", s.name, (long long)ctx, call, st);
            CHECK(saga::g_launches > 0, "%s ctx=%lld %s: nothing launched", s.name,
                  (long long)ctx, call);
            check_regions(cur_ws, cur_wsb, call);
            saga::g_launches = 0;
        };
        saga::g_launches = 0;
        ok(atopn_refresh_thresholds(&d, s.top_n, q, k, tau, lg, ws, wsb, nullptr), "refresh+logits");
        ok(atopn_refresh_thresholds(&d, s.top_n, q, k, tau, nullptr, ws, wsb, nullptr), "refresh");
        ok(saga_decode_step(&d, q, k, v, tau, out, cnt, bm, ws, wsb, nullptr), "decode+debug");
        ok(saga_decode_step(&d, q, k, v, tau, out, nullptr, nullptr, ws, wsb, nullptr), "decode");
        ok(atopn_refresh_decode_step(&d, s.top_n, q, k, v, tau, out, cnt, ws, wsb, nullptr),
           "refresh_decode");
        if (k8) {
            ok(atopn_refresh_thresholds_fp8k(&d, s.top_n, q, k8, ks, tau, lg, ws, wsb, nullptr),
               "refresh_fp8k");
            ok(saga_decode_step_fp8k(&d, q, k8, ks, v, tau, out, cnt, bm, ws, wsb, nullptr),
               "decode_fp8k");
            ok(atopn_refresh_decode_step_fp8k(&d, s.top_n, q, k8, ks, v, tau, out, cnt, ws, wsb,
                                              nullptr), "refresh_decode_fp8k");
            ok(saga_decode_step_fp8kv(&d, q, k8, ks, v8, vs, tau, out, cnt, bm, ws, wsb, nullptr),
               "decode_fp8kv");
            ok(atopn_refresh_decode_step_fp8kv(&d, s.top_n, q, k8, ks, v8, vs, tau, out, cnt, ws,
                                               wsb, nullptr), "refresh_decode_fp8kv");
        }
        if (full_supported(s)) {
            ok(saga_full_attention(&d, q, k, v, out, ws, wsb, nullptr), "full");
        } else {
            CHECK(saga_full_attention(&d, q, k, v, out, ws, wsb, nullptr) == SAGA_ERR_UNSUPPORTED,
                  "%s: dense head map", s.name);
            CHECK(saga::g_launches == 0, "%s: dense launched", s.name);
        }

        // Paged pools (pages of 256 rows) when the cache length allows.
        if (s.cache_len % 256 == 0) {
            const int P = 256, maxp = (int)(s.cache_len / P);
            const int64_t np = (int64_t)s.B * maxp + 1;
            void* kp = b.get((size_t)np * s.hk * P * s.dk * 2);
            void* vp = b.get((size_t)np * s.hv * P * dv * 2);
            int32_t* table = static_cast<int32_t*>(b.get((size_t)s.B * maxp * 4));
            int32_t* lens = static_cast<int32_t*>(b.get((size_t)s.B * 4));
            saga_paged pg;
            memset(&pg, 0, sizeof pg);
            pg.block_table_dev = table;
            pg.ctx_lens_dev = lens;
            pg.page_rows = P;
            pg.max_pages = maxp;
            pg.num_pages = np;
            // Every sequence at ctx_len; lengths from ctx_len down to 0 (the
            // kernels' work split follows them); every sequence empty.
            for (int pattern = 0; pattern < 3; ++pattern) {
                for (int bb = 0; bb < s.B; ++bb)
                    lens[bb] = pattern == 0 ? (int32_t)ctx
                             : pattern == 1 ? (int32_t)(ctx - ctx * bb / s.B)
                                            : 0;
                if (pattern == 1 && s.B > 1) lens[s.B - 1] = 0;
                ok(atopn_refresh_thresholds_paged(&d, &pg, s.top_n, q, kp, tau, ws, wsb, nullptr),
                   "refresh_paged");
                ok(saga_decode_step_paged(&d, &pg, q, kp, vp, tau, out, cnt, ws, wsb, nullptr),
                   "decode_paged");
                ok(atopn_refresh_decode_step_paged(&d, &pg, s.top_n, q, kp, vp, tau, out, cnt, ws,
                                                   wsb, nullptr), "refresh_decode_paged");
            }
        }

        // Two query tokens per step when the group allows it.
        if ((s.hq / s.hk) * 2 <= 16 && ctx >= 2) {
            const int lq = 2;
            saga_dims dv2 = d0;
            dv2.h_q = s.hq * lq;
            const size_t wsl = saga_workspace_bytes(&dv2, s.top_n);
            CHECK(wsl > 0, "%s: lq workspace", s.name);
            void* wl = b.get(wsl);
            cur_ws = wl;
            cur_wsb = wsl;
            void* ql = b.get(bh * lq * s.dk * 2);
            float* tl = static_cast<float*>(b.get(bh * lq * 4));
            void* ol = b.get(bh * lq * dv * 2);
            int32_t* cl = static_cast<int32_t*>(b.get(bh * lq * 4));
            ok(atopn_refresh_thresholds_lq(&d, lq, s.top_n, ql, k, tl, wl, wsl, nullptr),
               "refresh_lq");
            ok(saga_decode_step_lq(&d, lq, ql, k, v, tl, ol, cl, wl, wsl, nullptr), "decode_lq");
            ok(atopn_refresh_decode_step_lq(&d, lq, s.top_n, ql, k, v, tl, ol, cl, wl, wsl,
                                            nullptr), "refresh_decode_lq");
        }
    }
    fprintf(stderr, "valid calls: %s (workspace %zu bytes)\n", s.name, wsb);
}

void error_paths()
{
    const Shape s = {"errors", 2, 8, 2, 4, 64, 0, 4096, 100};
    Arena a;
    const int64_t bh = (int64_t)s.B * s.hq;
    void* q = a.get(bh * 64 * 2);
    void* k = a.get((size_t)s.B * s.hk * s.cache_len * 64 * 2);
    void* v = a.get((size_t)s.B * s.hv * s.cache_len * 64 * 2);
    float* tau = static_cast<float*>(a.get(bh * 4));
    void* out = a.get(bh * 64 * 2);
    float* ks = static_cast<float*>(a.get(s.B * s.hk * 4));
    const saga_dims good = make_dims(s, 3000);
    const size_t wsb = saga_workspace_bytes(&good, s.top_n);
    void* ws = a.get(wsb);
    char* qm = static_cast<char*>(q) + 2;                // misaligned by 2 bytes

    auto expect = [&](int st, int want, const char* what) {
        CHECK(st == want, "%s: status %d, expected %d", what, st, want);
        CHECK(saga::g_launches == 0, "%s: launched work on an error", what);
        saga::g_launches = 0;
        saga::g_ranges.clear();
    };
    saga::g_launches = 0;

    // Dimension checks (every entry point shares them; one call each here).
    struct DimCase { const char* what; void (*edit)(saga_dims*); int want; };
    const DimCase cases[] = {
        {"h_q not a multiple of h_k", [](saga_dims* d) { d->h_k = 3; }, SAGA_ERR_INVALID_ARGUMENT},
        {"h_q not a multiple of h_v", [](saga_dims* d) { d->h_v = 3; }, SAGA_ERR_INVALID_ARGUMENT},
        {"batch 0", [](saga_dims* d) { d->batch = 0; }, SAGA_ERR_INVALID_ARGUMENT},
        {"negative h_q", [](saga_dims* d) { d->h_q = -8; }, SAGA_ERR_INVALID_ARGUMENT},
        {"ctx 0", [](saga_dims* d) { d->ctx_len = 0; }, SAGA_ERR_INVALID_ARGUMENT},
        {"ctx > cache", [](saga_dims* d) { d->ctx_len = d->cache_len + 1; },
         SAGA_ERR_INVALID_ARGUMENT},
        {"cache 2^27", [](saga_dims* d) { d->cache_len = (int64_t)1 << 27; d->ctx_len = 10; },
         SAGA_ERR_INVALID_ARGUMENT},
        {"huge cache", [](saga_dims* d) { d->cache_len = INT64_MAX; d->ctx_len = 10; },
         SAGA_ERR_INVALID_ARGUMENT},
        {"NaN scale", [](saga_dims* d) { d->scale = NAN; }, SAGA_ERR_INVALID_ARGUMENT},
        {"inf scale", [](saga_dims* d) { d->scale = INFINITY; }, SAGA_ERR_INVALID_ARGUMENT},
        {"reserved2", [](saga_dims* d) { d->reserved2 = 1.0f; }, SAGA_ERR_INVALID_ARGUMENT},
        {"head_dim 48", [](saga_dims* d) { d->head_dim = 48; }, SAGA_ERR_UNSUPPORTED},
        {"head_dim_v 96", [](saga_dims* d) { d->head_dim_v = 96; }, SAGA_ERR_UNSUPPORTED},
        {"negative head_dim_v", [](saga_dims* d) { d->head_dim_v = -64; },
         SAGA_ERR_INVALID_ARGUMENT},
        {"32 query heads per key head", [](saga_dims* d) { d->h_q = 64; d->h_k = 2; },
         SAGA_ERR_UNSUPPORTED},
        {"batch * h_k > 65535", [](saga_dims* d) { d->batch = 40000; d->h_k = 2; },
         SAGA_ERR_UNSUPPORTED},
        {"head over 2 GiB", [](saga_dims* d) { d->cache_len = (int64_t)1 << 24; d->head_dim = 128; },
         SAGA_ERR_UNSUPPORTED},
        {"batch * h_q * cache_len > 2^40",
         [](saga_dims* d) { d->batch = 4095; d->h_q = 16; d->h_k = 16; d->h_v = 16;
                            d->cache_len = ((int64_t)1 << 24) + ((int64_t)1 << 22);
                            d->head_dim = 32; },
         SAGA_ERR_UNSUPPORTED},
    };
    for (const DimCase& c : cases) {
        saga_dims d = good;
        c.edit(&d);
        expect(saga_decode_step(&d, q, k, v, tau, out, nullptr, nullptr, ws, wsb, nullptr), c.want,
               c.what);
        expect(atopn_refresh_thresholds(&d, s.top_n, q, k, tau, nullptr, ws, wsb, nullptr), c.want,
               c.what);
        CHECK(saga_workspace_bytes(&d, s.top_n) == 0, "%s: workspace size of invalid dims", c.what);
    }
    expect(saga_decode_step(nullptr, q, k, v, tau, out, nullptr, nullptr, ws, wsb, nullptr),
           SAGA_ERR_INVALID_ARGUMENT, "null dims");
    CHECK(saga_workspace_bytes(nullptr, 1) == 0, "null dims workspace");

    // Pointer, alignment, N and workspace checks of each call family.
    const saga_dims* d = &good;
    expect(atopn_refresh_thresholds(d, 0, q, k, tau, nullptr, ws, wsb, nullptr),
           SAGA_ERR_INVALID_ARGUMENT, "top_n 0");
    expect(atopn_refresh_thresholds(d, -5, q, k, tau, nullptr, ws, wsb, nullptr),
           SAGA_ERR_INVALID_ARGUMENT, "top_n < 0");
    expect(atopn_refresh_thresholds(d, s.top_n, nullptr, k, tau, nullptr, ws, wsb, nullptr),
           SAGA_ERR_INVALID_ARGUMENT, "refresh null q");
    expect(atopn_refresh_thresholds(d, s.top_n, q, k, nullptr, nullptr, ws, wsb, nullptr),
           SAGA_ERR_INVALID_ARGUMENT, "refresh null tau");
    expect(atopn_refresh_thresholds(d, s.top_n, qm, k, tau, nullptr, ws, wsb, nullptr),
           SAGA_ERR_INVALID_ARGUMENT, "refresh misaligned q");
    expect(atopn_refresh_thresholds(d, s.top_n, q, k, tau, nullptr, ws, wsb - 1, nullptr),
           SAGA_ERR_WORKSPACE_TOO_SMALL, "refresh workspace");
    expect(atopn_refresh_thresholds(d, s.top_n, q, k, tau, nullptr, nullptr, wsb, nullptr),
           SAGA_ERR_INVALID_ARGUMENT, "refresh null workspace");
    expect(saga_decode_step(d, q, k, nullptr, tau, out, nullptr, nullptr, ws, wsb, nullptr),
           SAGA_ERR_INVALID_ARGUMENT, "decode null v");
    expect(saga_decode_step(d, q, k, v, nullptr, out, nullptr, nullptr, ws, wsb, nullptr),
           SAGA_ERR_INVALID_ARGUMENT, "decode null tau");
    expect(saga_decode_step(d, q, k, v, tau, nullptr, nullptr, nullptr, ws, wsb, nullptr),
           SAGA_ERR_INVALID_ARGUMENT, "decode null out");
    expect(saga_decode_step(d, q, static_cast<char*>(k) + 8, v, tau, out, nullptr, nullptr, ws,
                            wsb, nullptr), SAGA_ERR_INVALID_ARGUMENT, "decode misaligned k");
    expect(saga_decode_step(d, q, k, v, tau, out, reinterpret_cast<int32_t*>(qm), nullptr, ws,
                            wsb, nullptr), SAGA_ERR_INVALID_ARGUMENT, "decode misaligned counts");
    expect(saga_decode_step(d, q, k, v, tau, out, nullptr, nullptr, ws, wsb - 1, nullptr),
           SAGA_ERR_WORKSPACE_TOO_SMALL, "decode workspace");
    expect(atopn_refresh_decode_step(d, 0, q, k, v, tau, out, nullptr, ws, wsb, nullptr),
           SAGA_ERR_INVALID_ARGUMENT, "refresh_decode top_n 0");
    expect(atopn_refresh_decode_step(d, s.top_n, q, k, v, tau, out, nullptr, ws, 0, nullptr),
           SAGA_ERR_WORKSPACE_TOO_SMALL, "refresh_decode workspace");
    expect(saga_full_attention(d, q, k, v, nullptr, ws, wsb, nullptr), SAGA_ERR_INVALID_ARGUMENT,
           "full null out");
    expect(saga_full_attention(d, q, k, v, out, ws, 16, nullptr), SAGA_ERR_WORKSPACE_TOO_SMALL,
           "full workspace");
    {
        saga_dims wide = good;
        wide.h_q = 16;
        wide.h_k = 1;
        wide.h_v = 16;                                  // 16 value heads under one key head
        const size_t w2 = saga_workspace_bytes(&wide, 1);
        Arena b;
        void* ws2 = b.get(w2);
        void* q2 = b.get((size_t)s.B * 16 * 64 * 2);
        void* v2 = b.get((size_t)s.B * 16 * s.cache_len * 64 * 2);
        void* o2 = b.get((size_t)s.B * 16 * 64 * 2);
        expect(saga_full_attention(&wide, q2, k, v2, o2, ws2, w2, nullptr), SAGA_ERR_UNSUPPORTED,
               "full: 16 value heads per key head");
    }

    // Paged descriptions.
    int32_t* table = static_cast<int32_t*>(a.get((size_t)s.B * 16 * 4));
    int32_t* lens = static_cast<int32_t*>(a.get((size_t)s.B * 4));
    saga_paged pg;
    memset(&pg, 0, sizeof pg);
    pg.block_table_dev = table;
    pg.ctx_lens_dev = lens;
    pg.page_rows = 256;
    pg.max_pages = 16;                                  // 16 * 256 = cache_len
    pg.num_pages = 40;
    void* kp = a.get((size_t)40 * s.hk * 256 * 64 * 2);
    void* vp = a.get((size_t)40 * s.hv * 256 * 64 * 2);
    expect(saga_decode_step_paged(d, nullptr, q, kp, vp, tau, out, nullptr, ws, wsb, nullptr),
           SAGA_ERR_INVALID_ARGUMENT, "paged null description");
    struct PgCase { const char* what; void (*edit)(saga_paged*); };
    const PgCase pcases[] = {
        {"page_rows 100", [](saga_paged* p) { p->page_rows = 100; p->max_pages = 40; }},
        {"page_rows 384", [](saga_paged* p) { p->page_rows = 384; }},
        {"table rows * pages != cache_len", [](saga_paged* p) { p->max_pages = 15; }},
        {"no pages", [](saga_paged* p) { p->num_pages = 0; }},
        {"reserved", [](saga_paged* p) { p->reserved = 1; }},
        {"null table", [](saga_paged* p) { p->block_table_dev = nullptr; }},
        {"null lengths", [](saga_paged* p) { p->ctx_lens_dev = nullptr; }},
        {"misaligned table",
         [](saga_paged* p) { p->block_table_dev = reinterpret_cast<const int32_t*>(
                                 reinterpret_cast<const char*>(p->block_table_dev) + 2); }},
    };
    for (const PgCase& c : pcases) {
        saga_paged p2 = pg;
        c.edit(&p2);
        expect(saga_decode_step_paged(d, &p2, q, kp, vp, tau, out, nullptr, ws, wsb, nullptr),
               SAGA_ERR_INVALID_ARGUMENT, c.what);
        expect(atopn_refresh_thresholds_paged(d, &p2, s.top_n, q, kp, tau, ws, wsb, nullptr),
               SAGA_ERR_INVALID_ARGUMENT, c.what);
    }

    // Several query tokens.
    expect(saga_decode_step_lq(d, 0, q, k, v, tau, out, nullptr, ws, wsb, nullptr),
           SAGA_ERR_INVALID_ARGUMENT, "l_q 0");
    {
        saga_dims d2 = good;
        d2.ctx_len = 3;
        expect(saga_decode_step_lq(&d2, 4, q, k, v, tau, out, nullptr, ws, wsb, nullptr),
               SAGA_ERR_INVALID_ARGUMENT, "l_q > ctx");
    }
    expect(saga_decode_step_lq(d, 5, q, k, v, tau, out, nullptr, ws, wsb, nullptr),
           SAGA_ERR_UNSUPPORTED, "(h_q/h_k) * l_q > 16");

    // fp8 caches.
    expect(saga_decode_step_fp8k(d, q, k, nullptr, v, tau, out, nullptr, nullptr, ws, wsb, nullptr),
           SAGA_ERR_INVALID_ARGUMENT, "fp8k null scale");
    expect(saga_decode_step_fp8k(d, q, k, reinterpret_cast<float*>(qm), v, tau, out, nullptr,
                                 nullptr, ws, wsb, nullptr),
           SAGA_ERR_INVALID_ARGUMENT, "fp8k misaligned scale");
    expect(saga_decode_step_fp8kv(d, q, k, ks, v, nullptr, tau, out, nullptr, nullptr, ws, wsb,
                                  nullptr), SAGA_ERR_INVALID_ARGUMENT, "fp8kv null value scale");
    {
        saga_dims d32 = good;
        d32.head_dim = 32;
        const size_t w32 = saga_workspace_bytes(&d32, s.top_n);
        expect(saga_decode_step_fp8k(&d32, q, k, ks, v, tau, out, nullptr, nullptr, ws, w32,
                                     nullptr), SAGA_ERR_UNSUPPORTED, "fp8k head_dim 32");
        expect(atopn_refresh_thresholds_fp8k(&d32, s.top_n, q, k, ks, tau, nullptr, ws, w32,
                                             nullptr), SAGA_ERR_UNSUPPORTED, "fp8k refresh d 32");
    }

    // Status strings.
    for (int st = -1; st <= 5; ++st) {
        const char* m = saga_status_string(st);
        CHECK(m != nullptr && m[0] != 0, "status string %d", st);
    }
    CHECK(saga_version() > 0, "version");
    fprintf(stderr, "error paths checked\n");
}

}  // namespace

int main(int argc, char** argv)
{
    const bool big = argc > 1 && strcmp(argv[1], "--big") == 0;
    error_paths();
    if (big) plan_choices();
    const Shape shapes[] = {
        {"tiny", 1, 4, 1, 2, 64, 0, 1032, 64},
        {"llama_like_8k", 1, 32, 4, 8, 64, 0, 8224, 512},
        {"qwen_like_small", 2, 12, 1, 2, 128, 0, 3005, 100},
        {"group16_d64", 3, 16, 1, 4, 64, 0, 1504, 40},
        {"mha_d128", 2, 8, 8, 8, 128, 0, 703, 33},
        {"fewer_value_heads", 1, 8, 4, 2, 64, 0, 903, 20},
        {"short_ctx", 1, 4, 2, 4, 64, 0, 20, 5},
        {"one_row", 1, 4, 1, 1, 64, 0, 1, 1},
        {"sigma_dk32_dv64", 2, 32, 8, 8, 32, 64, 2048, 64},
        {"dk128_dv32", 1, 8, 2, 4, 128, 32, 1024, 50},
        {"paged_llama", 2, 32, 4, 8, 64, 0, 4096, 256},
        {"many_rows", 4200, 16, 1, 1, 64, 0, 256, 8},
    };
    for (const Shape& s : shapes) valid_calls(s);
    if (big) {
        // The benchmark shapes at 128K context, and the largest accepted head.
        const Shape bigs[] = {
            {"llama_like_128k_b16", 16, 32, 4, 8, 64, 0, 131104, 2048},
            {"qwen_like_128k_b1", 1, 12, 1, 2, 128, 0, 131104, 1024},
            {"llama_like_128k_b1", 1, 32, 4, 8, 64, 0, 131104, 2048},
            {"qwen_like_128k_b16", 16, 12, 1, 2, 128, 0, 131104, 1024},
            {"paged_128k", 2, 32, 4, 8, 64, 0, 131072, 2048},
            {"largest_head_d128", 1, 4, 1, 1, 128, 0, ((int64_t)1 << 23) - 1, 1024},
        };
        for (const Shape& s : bigs) valid_calls(s);
    }
    fprintf(stderr, "%d checks, %d failures\n", g_checks, g_failures);
    return g_failures == 0 ? 0 : 1;
}

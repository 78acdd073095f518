// api.hip -- the C ABI declared in include/saga.h: argument validation,
// workspace layout, chunk planning and kernel dispatch.  Host code only.
//
// Every entry point validates all of its arguments before it enqueues
// anything, never allocates, never copies between host and device and never
// synchronises, so a call can be captured into a hipGraph.
#include <math.h>
#include <string.h>

#include "saga.h"
#include "kernels.hpp"

#define SAGA_EXPORT extern "C" __attribute__((visibility("default")))

using namespace saga;

namespace {

constexpr int kTargetBlocks = 2048;       // workgroups per launch we aim for (256 CUs)
constexpr int64_t kMaxCacheLen = int64_t(1) << 27;

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int validate_dims(const saga_dims* d)
{
    if (!d) return SAGA_ERR_INVALID_ARGUMENT;
    if (d->batch < 1 || d->h_q < 1 || d->h_k < 1 || d->h_v < 1 || d->head_dim < 1)
        return SAGA_ERR_INVALID_ARGUMENT;
    if (d->reserved != 0 || d->reserved2 != 0.0f) return SAGA_ERR_INVALID_ARGUMENT;
    if (d->h_q % d->h_k != 0 || d->h_q % d->h_v != 0) return SAGA_ERR_INVALID_ARGUMENT;
    if (d->cache_len < 1 || d->cache_len >= kMaxCacheLen) return SAGA_ERR_INVALID_ARGUMENT;
    if (d->ctx_len < 1 || d->ctx_len > d->cache_len) return SAGA_ERR_INVALID_ARGUMENT;
    if (!isfinite(d->scale)) return SAGA_ERR_INVALID_ARGUMENT;
    if (d->head_dim != 64 && d->head_dim != 128) return SAGA_ERR_UNSUPPORTED;
    if (d->h_q / d->h_k > 16) return SAGA_ERR_UNSUPPORTED;
    if ((int64_t)d->batch * d->h_k > 65535) return SAGA_ERR_UNSUPPORTED;
    if ((int64_t)d->batch * d->h_q * d->cache_len > (int64_t(1) << 40)) return SAGA_ERR_UNSUPPORTED;
    return SAGA_OK;
}

bool misaligned(const void* p, size_t a) { return ((uintptr_t)p) % a != 0; }

// Workspace layout (byte offsets), identical for every ctx_len <= cache_len.
struct Layout {
    int64_t ld;           // row stride of logits / candidates (elements)
    int max_chunks;
    size_t pm, pl, pc, po, logits, cand, ghist, done, ccount, state, total;
};

Layout make_layout(const saga_dims* d)
{
    Layout L{};
    const size_t rows = (size_t)d->batch * d->h_q;
    L.ld = (int64_t)round_up((size_t)d->cache_len, 64);
    const int64_t want = kTargetBlocks / ((int64_t)d->batch * d->h_k);
    const int64_t by_len = (d->cache_len + 127) / 128;   // smallest block tile is 128 rows
    int64_t mc = want < by_len ? want : by_len;
    L.max_chunks = (int)(mc < 1 ? 1 : mc);
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off += round_up(bytes, 256); return o; };
    L.pm = take(rows * L.max_chunks * 4);
    L.pl = take(rows * L.max_chunks * 4);
    L.pc = take(rows * L.max_chunks * 4);
    L.po = take(rows * L.max_chunks * (size_t)d->head_dim * 4);
    L.logits = take(rows * (size_t)L.ld * 4);
    L.cand = take(rows * (size_t)L.ld * 4);
    L.ghist = take(rows * kHistBins * 4);
    L.done = take(rows * 4);
    L.ccount = take(rows * 4);
    L.state = take(rows * 16);
    L.total = off;
    return L;
}

struct Chunking {
    int chunks;
    int64_t rows;
};

// Split ctx rows into chunks of whole block tiles so that the launch has about
// kTargetBlocks workgroups and never more chunks than the workspace holds.
Chunking plan_chunks(int64_t ctx, int64_t pairs, int64_t block_rows, int max_chunks)
{
    int64_t want = kTargetBlocks / pairs;
    if (want < 1) want = 1;
    int64_t c = (ctx + block_rows - 1) / block_rows;
    if (c > want) c = want;
    if (c > max_chunks) c = max_chunks;
    if (c < 1) c = 1;
    int64_t rows = (ctx + c - 1) / c;
    rows = (rows + block_rows - 1) / block_rows * block_rows;
    return {(int)((ctx + rows - 1) / rows), rows};
}

Partials partials(void* ws, const Layout& L)
{
    unsigned char* w = static_cast<unsigned char*>(ws);
    Partials p;
    p.m = reinterpret_cast<float*>(w + L.pm);
    p.l = reinterpret_cast<float*>(w + L.pl);
    p.c = reinterpret_cast<int32_t*>(w + L.pc);
    p.o = reinterpret_cast<float*>(w + L.po);
    return p;
}

int hip_status(hipError_t e) { return e == hipSuccess ? SAGA_OK : SAGA_ERR_HIP; }

}  // namespace

SAGA_EXPORT size_t saga_workspace_bytes(const saga_dims* dims, int32_t top_n)
{
    (void)top_n;   // the layout does not depend on N
    if (validate_dims(dims) != SAGA_OK) return 0;
    return make_layout(dims).total;
}

SAGA_EXPORT int atopn_refresh_thresholds(const saga_dims* dims, int32_t top_n, const void* q_dev,
                                         const void* k_cache_dev, float* thresholds_dev,
                                         float* logits_debug_dev, void* workspace_dev,
                                         size_t workspace_bytes, void* stream)
{
    int st = validate_dims(dims);
    if (st != SAGA_OK) return st;
    if (top_n < 1 || !q_dev || !k_cache_dev || !thresholds_dev || !workspace_dev)
        return SAGA_ERR_INVALID_ARGUMENT;
    if (misaligned(q_dev, 16) || misaligned(k_cache_dev, 16) || misaligned(thresholds_dev, 4) ||
        misaligned(logits_debug_dev, 4) || misaligned(workspace_dev, 16))
        return SAGA_ERR_INVALID_ARGUMENT;
    const Layout L = make_layout(dims);
    if (workspace_bytes < L.total) return SAGA_ERR_WORKSPACE_TOO_SMALL;

    hipStream_t s = static_cast<hipStream_t>(stream);
    unsigned char* w = static_cast<unsigned char*>(workspace_dev);
    const int D = dims->head_dim;
    const int rows = dims->batch * dims->h_q;
    const int64_t ctx = dims->ctx_len;
    const Chunking ch = plan_chunks(ctx, (int64_t)dims->batch * dims->h_k, decode_block_rows(D),
                                    L.max_chunks);
    const bool need_select = (int64_t)top_n < ctx;

    if (need_select || logits_debug_dev) {
        LogitsArgs la{};
        la.q = static_cast<const uint16_t*>(q_dev);
        la.k = static_cast<const uint16_t*>(k_cache_dev);
        la.logits = reinterpret_cast<float*>(w + L.logits);
        la.debug = logits_debug_dev;
        la.ld = L.ld;
        la.B = dims->batch;
        la.hq = dims->h_q;
        la.hk = dims->h_k;
        la.Gk = dims->h_q / dims->h_k;
        la.ctx = ctx;
        la.cache_len = dims->cache_len;
        la.rows_per_chunk = ch.rows;
        la.scale = dims->scale;
        la.ghist = reinterpret_cast<uint32_t*>(w + L.ghist);
        la.done = reinterpret_cast<uint32_t*>(w + L.done);
        la.cand_count = reinterpret_cast<uint32_t*>(w + L.ccount);
        st = hip_status(launch_qk_logits(D, la, ch.chunks, s));
        if (st != SAGA_OK) return st;
    }
    if (!need_select) {
        // N >= ctx: every entry is kept, tau = -inf.
        return hip_status(launch_fill_u32(reinterpret_cast<uint32_t*>(thresholds_dev), rows,
                                          0xff800000u, s));
    }
    SelectArgs sa{};
    sa.logits = reinterpret_cast<const float*>(w + L.logits);
    sa.ld = L.ld;
    sa.ctx = ctx;
    sa.rows = rows;
    sa.segs = (int)((ctx + kSelectSeg - 1) / kSelectSeg);
    sa.top_n = (uint32_t)top_n;
    sa.ghist = reinterpret_cast<uint32_t*>(w + L.ghist);
    sa.done = reinterpret_cast<uint32_t*>(w + L.done);
    sa.state = reinterpret_cast<uint32_t*>(w + L.state);
    sa.cand = reinterpret_cast<uint32_t*>(w + L.cand);
    sa.cand_count = reinterpret_cast<uint32_t*>(w + L.ccount);
    sa.tau = thresholds_dev;
    return hip_status(launch_select(sa, s));
}

SAGA_EXPORT int saga_decode_step(const saga_dims* dims, const void* q_dev, const void* k_cache_dev,
                                 const void* v_cache_dev, const float* thresholds_dev,
                                 void* out_dev, int32_t* sel_counts_dev,
                                 uint32_t* sel_bitmap_debug_dev, void* workspace_dev,
                                 size_t workspace_bytes, void* stream)
{
    int st = validate_dims(dims);
    if (st != SAGA_OK) return st;
    if (!q_dev || !k_cache_dev || !v_cache_dev || !thresholds_dev || !out_dev || !workspace_dev)
        return SAGA_ERR_INVALID_ARGUMENT;
    if (misaligned(q_dev, 16) || misaligned(k_cache_dev, 16) || misaligned(v_cache_dev, 16) ||
        misaligned(thresholds_dev, 4) || misaligned(out_dev, 2) || misaligned(sel_counts_dev, 4) ||
        misaligned(sel_bitmap_debug_dev, 4) || misaligned(workspace_dev, 16))
        return SAGA_ERR_INVALID_ARGUMENT;
    const Layout L = make_layout(dims);
    if (workspace_bytes < L.total) return SAGA_ERR_WORKSPACE_TOO_SMALL;

    hipStream_t s = static_cast<hipStream_t>(stream);
    const int D = dims->head_dim;
    const int rows = dims->batch * dims->h_q;
    const int64_t words = (dims->cache_len + 31) / 32;
    if (sel_bitmap_debug_dev) {
        st = hip_status(launch_fill_u32(sel_bitmap_debug_dev, (int64_t)rows * words, 0u, s));
        if (st != SAGA_OK) return st;
    }
    const Chunking ch = plan_chunks(dims->ctx_len, (int64_t)dims->batch * dims->h_k,
                                    decode_block_rows(D), L.max_chunks);
    DecodeArgs a{};
    a.q = static_cast<const uint16_t*>(q_dev);
    a.k = static_cast<const uint16_t*>(k_cache_dev);
    a.v = static_cast<const uint16_t*>(v_cache_dev);
    a.tau = thresholds_dev;
    a.bitmap = sel_bitmap_debug_dev;
    a.bitmap_words = words;
    a.part = partials(workspace_dev, L);
    a.B = dims->batch;
    a.hq = dims->h_q;
    a.hk = dims->h_k;
    a.hv = dims->h_v;
    a.Gk = dims->h_q / dims->h_k;
    a.Gv = dims->h_q / dims->h_v;
    a.ctx = dims->ctx_len;
    a.cache_len = dims->cache_len;
    a.rows_per_chunk = ch.rows;
    a.chunks = ch.chunks;
    a.scale = dims->scale;
    a.wave_lds = decode_wave_lds_bytes(D, a.Gk);
    st = hip_status(launch_sparse_decode(D, a, s));
    if (st != SAGA_OK) return st;
    return hip_status(launch_combine(D, a.part, rows, ch.chunks, static_cast<uint16_t*>(out_dev),
                                     sel_counts_dev, s));
}

SAGA_EXPORT int saga_full_attention(const saga_dims* dims, const void* q_dev,
                                    const void* k_cache_dev, const void* v_cache_dev,
                                    void* out_dev, void* workspace_dev, size_t workspace_bytes,
                                    void* stream)
{
    int st = validate_dims(dims);
    if (st != SAGA_OK) return st;
    if (!q_dev || !k_cache_dev || !v_cache_dev || !out_dev || !workspace_dev)
        return SAGA_ERR_INVALID_ARGUMENT;
    if (misaligned(q_dev, 16) || misaligned(k_cache_dev, 16) || misaligned(v_cache_dev, 16) ||
        misaligned(out_dev, 2) || misaligned(workspace_dev, 16))
        return SAGA_ERR_INVALID_ARGUMENT;
    const Layout L = make_layout(dims);
    if (workspace_bytes < L.total) return SAGA_ERR_WORKSPACE_TOO_SMALL;

    const int D = dims->head_dim;
    const int Gk = dims->h_q / dims->h_k, Gv = dims->h_q / dims->h_v;
    // Value heads touched by one key head's query heads, and query heads per
    // (key head, value head) pair.
    int nv = 1, maxs = 1;
    for (int g = 0; g < dims->h_k; ++g) {
        const int i0 = g * Gk, vfirst = i0 / Gv, vlast = (i0 + Gk - 1) / Gv;
        if (vlast - vfirst + 1 > nv) nv = vlast - vfirst + 1;
        for (int vh = vfirst; vh <= vlast; ++vh) {
            const int lo = vh * Gv > i0 ? vh * Gv : i0;
            const int hi = (vh + 1) * Gv < i0 + Gk ? (vh + 1) * Gv : i0 + Gk;
            if (hi - lo > maxs) maxs = hi - lo;
        }
    }
    if (nv == 3) nv = 4;
    if (nv > 4 || maxs > 8) return SAGA_ERR_UNSUPPORTED;
    const int maxs_t = maxs <= 2 ? 2 : (maxs <= 4 ? 4 : 8);

    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t block_rows = (int64_t)kWavesPerBlock * 16 * full_unroll(D);
    const Chunking ch = plan_chunks(dims->ctx_len, (int64_t)dims->batch * dims->h_k, block_rows,
                                    L.max_chunks);
    FullArgs a{};
    a.q = static_cast<const uint16_t*>(q_dev);
    a.k = static_cast<const uint16_t*>(k_cache_dev);
    a.v = static_cast<const uint16_t*>(v_cache_dev);
    a.part = partials(workspace_dev, L);
    a.B = dims->batch;
    a.hq = dims->h_q;
    a.hk = dims->h_k;
    a.hv = dims->h_v;
    a.Gk = Gk;
    a.Gv = Gv;
    a.nv = nv;
    a.ctx = dims->ctx_len;
    a.cache_len = dims->cache_len;
    a.rows_per_chunk = ch.rows;
    a.chunks = ch.chunks;
    a.scale = dims->scale;
    a.wave_lds = full_wave_lds_bytes(D, maxs_t);
    st = hip_status(launch_full(D, maxs_t, a, s));
    if (st != SAGA_OK) return st;
    return hip_status(launch_combine(D, a.part, dims->batch * dims->h_q, ch.chunks,
                                     static_cast<uint16_t*>(out_dev), nullptr, s));
}

SAGA_EXPORT const char* saga_status_string(int status)
{
    switch (status) {
    case SAGA_OK: return "ok";
    case SAGA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case SAGA_ERR_UNSUPPORTED: return "unsupported shape";
    case SAGA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case SAGA_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
    }
}

SAGA_EXPORT int saga_version(void) { return 100; }

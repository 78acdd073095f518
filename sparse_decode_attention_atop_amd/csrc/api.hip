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

// Workgroups per K-stream launch.  Each workgroup streams one contiguous
// chunk; measured on MI355X, fewer concurrent streams per CU read faster as
// long as every CU gets the same count: three per CU (768) at head_dim 64,
// two (512) at head_dim 128, and four (1024) for the half-size rows of an fp8
// K cache at head_dim 64.
constexpr int64_t kFullTargetBlocks = SAGA_FULL_BLOCKS;   // dense kernel: workgroups per launch

int64_t target_blocks(int head_dim, bool k8 = false)
{
    if (k8) return head_dim == 128 ? SAGA_TARGET_BLOCKS128_K8 : SAGA_TARGET_BLOCKS64_K8;
    if (head_dim == 32) return SAGA_TARGET_BLOCKS32;
    return head_dim == 128 ? SAGA_TARGET_BLOCKS128 : SAGA_TARGET_BLOCKS64;
}
constexpr int64_t kMaxCacheLen = int64_t(1) << 27;

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Value / output head dimension (head_dim_v, or head_dim when that is 0).
int value_dim(const saga_dims* d) { return d->head_dim_v ? d->head_dim_v : d->head_dim; }

bool supported_dim(int x) { return x == 32 || x == 64 || x == 128; }

int validate_dims(const saga_dims* d)
{
    if (!d) return SAGA_ERR_INVALID_ARGUMENT;
    if (d->batch < 1 || d->h_q < 1 || d->h_k < 1 || d->h_v < 1 || d->head_dim < 1 ||
        d->head_dim_v < 0)
        return SAGA_ERR_INVALID_ARGUMENT;
    if (d->reserved2 != 0.0f) return SAGA_ERR_INVALID_ARGUMENT;
    if (d->h_q % d->h_k != 0 || d->h_q % d->h_v != 0) return SAGA_ERR_INVALID_ARGUMENT;
    if (d->cache_len < 1 || d->cache_len >= kMaxCacheLen) return SAGA_ERR_INVALID_ARGUMENT;
    if (d->ctx_len < 1 || d->ctx_len > d->cache_len) return SAGA_ERR_INVALID_ARGUMENT;
    if (!isfinite(d->scale)) return SAGA_ERR_INVALID_ARGUMENT;
    if (!supported_dim(d->head_dim) || !supported_dim(value_dim(d))) return SAGA_ERR_UNSUPPORTED;
    if (d->h_q / d->h_k > 16) return SAGA_ERR_UNSUPPORTED;
    if ((int64_t)d->batch * d->h_k > 65535) return SAGA_ERR_UNSUPPORTED;
    if ((int64_t)d->batch * d->h_q * d->cache_len > (int64_t(1) << 40)) return SAGA_ERR_UNSUPPORTED;
    // One cache head is addressed with 32-bit buffer offsets.
    const int64_t dmax = d->head_dim > value_dim(d) ? d->head_dim : value_dim(d);
    if (d->cache_len * dmax * 2 >= (int64_t(1) << 31)) return SAGA_ERR_UNSUPPORTED;
    return SAGA_OK;
}

bool misaligned(const void* p, size_t a) { return ((uintptr_t)p) % a != 0; }

struct Chunking {
    int chunks;
    int64_t rows;
};

// Split ctx rows into chunks of whole block tiles (block_rows each) so that the
// launch has about `target` workgroups and never more chunks than the
// workspace holds.
Chunking split_rows(int64_t ctx, int64_t pairs, int64_t block_rows, int64_t target,
                    int max_chunks)
{
    int64_t want = target / pairs;
    if (want < 1) want = 1;
    int64_t c = (ctx + block_rows - 1) / block_rows;
    if (c > want) c = want;
    if (c > max_chunks) c = max_chunks;
    if (c < 1) c = 1;
    int64_t rows = (ctx + c - 1) / c;
    rows = (rows + block_rows - 1) / block_rows * block_rows;
    return {(int)((ctx + rows - 1) / rows), rows};
}

// Chunking of the K stream (stream-select kernel) for one call.  The chunk
// count comes from a plan in whole tile pairs (the kernel streams pairs).
// Paged caches keep those pair-sized chunks, so with pages of kPageQuantum
// rows no pair starts in one page and ends in the next.  Contiguous caches
// keep the count but round the rows per chunk to whole tiles only: a pair's
// second tile past the chunk end reads zeros and selects nothing, and the
// last chunk is then about as long as the others (131073 rows in 12 chunks:
// 11 of 10944 rows and one of 10689, rather than 11 of 11008 and one of
// 9985).  Never more rows per chunk than the pair plan.
Chunking plan_chunks(int64_t ctx, int64_t pairs, int head_dim, int max_chunks, bool k8,
                     bool paged)
{
    const int64_t block = k8 ? decode_block_rows_k8(head_dim) : decode_block_rows(head_dim);
    Chunking c = split_rows(ctx, pairs, 2 * block, target_blocks(head_dim, k8), max_chunks);
    if (!paged) {
        int64_t rows = (ctx + c.chunks - 1) / c.chunks;
        rows = (rows + block - 1) / block * block;
        c = {(int)((ctx + rows - 1) / rows), rows};
    }
    return c;
}

// Workspace layout (byte offsets), identical for every ctx_len <= cache_len.
struct Layout {
    int max_chunks;
    int64_t entry_rows;   // selection-list capacity per (b, query head)
    int64_t top_rows;     // rows per chunk of the paged plan at cache_len
    size_t pm, pl, pc, po, entries, overflow, lcount, lmax, sample, pivot, flags, plan, total;
};

Layout make_layout(const saga_dims* d)
{
    Layout L{};
    const size_t rows = (size_t)d->batch * d->h_q;
    // Room for the largest launch any call makes: the bf16 and fp8 K streams
    // and the dense kernel.
    int64_t target = kFullTargetBlocks;
    for (const bool k8 : {false, true})
        if (target_blocks(d->head_dim, k8) > target) target = target_blocks(d->head_dim, k8);
    // Twice the chunks of the largest launch: paged calls with per-sequence
    // lengths give long sequences more chunks than a uniform split would.
    const int64_t want = 2 * target / ((int64_t)d->batch * d->h_k);
    const int64_t by_len = (d->cache_len + 127) / 128;   // smallest tile pair is 128 rows
    int64_t mc = want < by_len ? want : by_len;
    if (mc > kMaxListsPerRow / kWavesPerBlock) mc = kMaxListsPerRow / kWavesPerBlock;   // 512
    L.max_chunks = (int)(mc < 1 ? 1 : mc);
    // chunks * rows_per_chunk <= ctx + rows_per_chunk(ctx), and rows_per_chunk
    // never exceeds max(block rows, its value at ctx = cache_len).
    // The larger of the bf16 and fp8 K plans (one layout serves both).
    int64_t top_rows = 0;
    for (const bool k8 : {false, true}) {
        const int64_t br = 2 * (k8 ? decode_block_rows_k8(d->head_dim) : decode_block_rows(d->head_dim));
        // The paged plan: its chunks are at least as long as the contiguous one's.
        const Chunking top = plan_chunks(d->cache_len, (int64_t)d->batch * d->h_k, d->head_dim,
                                         L.max_chunks, k8, true);
        const int64_t r = top.rows > br ? top.rows : br;
        if (r > top_rows) top_rows = r;
    }
    L.top_rows = top_rows;
    L.entry_rows = d->cache_len + top_rows;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off += round_up(bytes, 256); return o; };
    L.pm = take(rows * L.max_chunks * 4);
    L.pl = take(rows * L.max_chunks * 4);
    L.pc = take(rows * L.max_chunks * 4);
    L.po = take(rows * L.max_chunks * (size_t)value_dim(d) * 4);
    L.entries = take(rows * L.max_chunks * kWavesPerBlock * (size_t)kListPrimary * 8);
    L.overflow = take(rows * (size_t)L.entry_rows * 8);
    L.lcount = take(rows * L.max_chunks * kWavesPerBlock * 4);
    L.lmax = take(rows * L.max_chunks * kWavesPerBlock * 4);
    L.sample = take(rows * kSampleMax * 4);
    L.pivot = take(rows * 4);
    L.flags = take((size_t)d->batch * d->h_k * 4);
    L.plan = take(((size_t)d->batch + 1) * 4);
    L.total = off;
    return L;
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

// What each (b, query head) row attends: paged caches and per-sequence
// lengths (pg), query tokens per step (lq; the call's h_q then counts
// virtual heads, one per token), and an fp8 e4m3 K cache with one scale per
// (b, key head) (k_scale; null for bf16 K).
struct RowModel {
    PagedKV pg{};
    int32_t lq = 1;
    const float* k_scale = nullptr;
    const float* v_scale = nullptr;   // non-null: fp8 e4m3 V cache, one scale per (b, value head)
};

// Chunking of a list-path call.  Paged caches: the launch has room for
// twice the chunks of the uniform plan at ctx_len (never more than the
// workspace holds) and the kernels take their rows per chunk from the
// sequence lengths on the device (PagedKV::plan_*), so that a batch of mixed
// lengths still spreads over about the stream's target of workgroups.
Chunking list_chunks(const saga_dims* dims, const Layout& L, void* ws, RowModel* rm)
{
    const int D = dims->head_dim;
    const bool k8 = rm->k_scale != nullptr, paged = rm->pg.block_table != nullptr;
    Chunking ch = plan_chunks(dims->ctx_len, (int64_t)dims->batch * dims->h_k, D, L.max_chunks,
                              k8, paged);
    if (!paged) return ch;
    const int64_t cap = 2 * (int64_t)ch.chunks < L.max_chunks ? 2 * (int64_t)ch.chunks : L.max_chunks;
    const int64_t target = target_blocks(D, k8), rows = (int64_t)dims->batch * dims->h_k;
    rm->pg.plan_cap = (int32_t)cap;
    rm->pg.plan_target = (int32_t)target;
    rm->pg.plan_quantum = 2 * (k8 ? decode_block_rows_k8(D) : decode_block_rows(D));
    rm->pg.plan_rows_max = L.top_rows;
    // Work items of the K stream: h_k * sum_b ceil(len_b / r) < h_k * sum / r
    // + B * h_k.  The device plan takes r >= h_k * sum / target unless that
    // exceeds top_rows, when r = top_rows and len_b <= ctx bound the count;
    // no sequence has more than cap chunks.
    int64_t grid = target + rows;
    const int64_t by_rows = rows * ((dims->ctx_len + L.top_rows - 1) / L.top_rows);
    if (by_rows > grid) grid = by_rows;
    if (rows * cap < grid) grid = rows * cap;
    rm->pg.plan_grid = grid;
    rm->pg.plan = reinterpret_cast<int32_t*>(static_cast<unsigned char*>(ws) + L.plan);
    return {(int)cap, L.top_rows};
}

// Arguments of the stream-select kernel for one call.
SelectStreamArgs stream_args(const saga_dims* dims, const Layout& L, const Chunking& ch,
                             const void* q, const void* k, const float* tau, void* ws,
                             const RowModel& rm)
{
    unsigned char* w = static_cast<unsigned char*>(ws);
    SelectStreamArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.tau = tau;
    a.entries = reinterpret_cast<uint2*>(w + L.entries);
    a.overflow_at = (int64_t)((L.overflow - L.entries) / 8);
    a.head_stride = L.entry_rows;
    a.list_count = reinterpret_cast<int32_t*>(w + L.lcount);
    a.list_max = reinterpret_cast<float*>(w + L.lmax);
    a.B = dims->batch;
    a.hq = dims->h_q;
    a.hk = dims->h_k;
    a.Gk = dims->h_q / dims->h_k;
    a.ctx = dims->ctx_len;
    a.cache_len = dims->cache_len;
    a.rows_per_chunk = ch.rows;
    a.chunks = ch.chunks;
    a.scale = dims->scale;
    a.pg = rm.pg;
    a.lq = rm.lq;
    a.k_scale = rm.k_scale;
    return a;
}

}  // namespace

SAGA_EXPORT size_t saga_workspace_bytes(const saga_dims* dims, int32_t top_n)
{
    (void)top_n;   // the layout does not depend on N
    if (validate_dims(dims) != SAGA_OK) return 0;
    return make_layout(dims).total;
}

namespace {

// Refresh steps 1-4 (see refresh.hip): sample, pivot, candidate lists, exact
// N-th largest.  Requires top_n < ctx.  With group_flags, key groups in which
// a row needed the recompute path are flagged (their lists are incomplete).
int enqueue_refresh(const saga_dims* dims, int32_t top_n, const void* q_dev,
                    const void* k_cache_dev, float* thresholds_dev, float* logits_debug_dev,
                    void* workspace_dev, const Layout& L, const Chunking& ch, hipStream_t s,
                    uint32_t* group_flags, const RowModel& rm)
{
    unsigned char* w = static_cast<unsigned char*>(workspace_dev);
    const int D = dims->head_dim;
    const int64_t ctx = dims->ctx_len;
    float* pivot = reinterpret_cast<float*>(w + L.pivot);

    // 1-2. Pivot from a sample of 16-row blocks, one every `stride` rows
    // (stride a multiple of 16), at most kSampleMax rows; the whole context
    // when it is that short, and then the pivot is tau itself.  Otherwise its
    // rank in the sample sits five standard deviations above the expected
    // number of sample logits >= tau, so at least N logits are >= pivot except
    // with negligible probability (and step 4 stays exact regardless).
    SampleArgs sa{};
    sa.q = static_cast<const uint16_t*>(q_dev);
    sa.k = static_cast<const uint16_t*>(k_cache_dev);
    sa.sample = reinterpret_cast<float*>(w + L.sample);
    sa.pivot = pivot;
    sa.group_flags = group_flags;
    sa.B = dims->batch;
    sa.hq = dims->h_q;
    sa.hk = dims->h_k;
    sa.Gk = dims->h_q / dims->h_k;
    sa.cache_len = dims->cache_len;
    const int64_t blocks_max = kSampleMax / 16;
    if (ctx <= kSampleMax) {
        sa.stride = 16;
        sa.m = (int)ctx;
    } else {
        sa.stride = (ctx / 16 + blocks_max - 1) / blocks_max * 16;   // every block fully inside ctx
        sa.m = (int)(ctx / sa.stride) * 16;
    }
    if (sa.m == ctx) {
        sa.rank = top_n;
    } else {
        const double mu = (double)top_n * sa.m / (double)ctx;
        double r = ceil(mu + 5.0 * sqrt(mu) + 5.0);
        if (r > sa.m) r = sa.m;
        sa.rank = (int)r;
    }
    sa.scale = dims->scale;
    sa.top_n = top_n;
    sa.ctx = dims->ctx_len;
    sa.pg = rm.pg;
    sa.lq = rm.lq;
    sa.k_scale = rm.k_scale;
    int st = hip_status(launch_sample(D, sa, s));
    if (st != SAGA_OK) return st;

    // 3. Candidate lists: every logit >= pivot.
    SelectStreamArgs a = stream_args(dims, L, ch, q_dev, k_cache_dev, pivot, workspace_dev, rm);
    a.logits_out = logits_debug_dev;
    st = hip_status(launch_select_stream(D, a, s));
    if (st != SAGA_OK) return st;

    // 4. Exact N-th largest per row.
    FinalArgs fa{};
    fa.q = sa.q;
    fa.k = sa.k;
    fa.entries = a.entries;
    fa.overflow_at = a.overflow_at;
    fa.head_stride = a.head_stride;
    fa.list_count = a.list_count;
    fa.tau = thresholds_dev;
    fa.group_flags = group_flags;
    fa.B = dims->batch;
    fa.hq = dims->h_q;
    fa.hk = dims->h_k;
    fa.Gk = sa.Gk;
    fa.ctx = ctx;
    fa.cache_len = dims->cache_len;
    fa.rows_per_chunk = ch.rows;
    fa.chunks = ch.chunks;
    fa.top_n = (uint32_t)top_n;
    fa.scale = dims->scale;
    fa.pg = rm.pg;
    fa.lq = rm.lq;
    fa.k_scale = rm.k_scale;
    return hip_status(launch_refresh_final(D, fa, s));
}

// Masked softmax + sparse gather over the lists in the workspace, then the
// combine into out.  With tau_filter, list entries below it are skipped.
int enqueue_gather_combine(const saga_dims* dims, const Layout& L, const Chunking& ch,
                           const void* v_cache_dev, const float* tau_filter, void* out_dev,
                           int32_t* sel_counts_dev, void* workspace_dev, hipStream_t s,
                           const RowModel& rm)
{
    unsigned char* w = static_cast<unsigned char*>(workspace_dev);
    const int D = value_dim(dims);                      // the gather reads V rows only
    const int rows = dims->batch * dims->h_q;
    // Each (b, query head) gets `segs` gather workgroups that split its selected
    // entries evenly: about gather_target_blocks(D) workgroups in all.
    GatherArgs ga{};
    ga.v = static_cast<const uint16_t*>(v_cache_dev);
    ga.entries = reinterpret_cast<const uint2*>(w + L.entries);
    ga.overflow_at = (int64_t)((L.overflow - L.entries) / 8);
    ga.head_stride = L.entry_rows;
    ga.list_count = reinterpret_cast<const int32_t*>(w + L.lcount);
    ga.list_max = reinterpret_cast<const float*>(w + L.lmax);
    ga.tau_filter = tau_filter;
    ga.v_scale = rm.v_scale;
    ga.part = partials(workspace_dev, L);
    ga.B = dims->batch;
    ga.hq = dims->h_q;
    ga.hk = dims->h_k;
    ga.hv = dims->h_v;
    ga.ctx = dims->ctx_len;
    ga.Gv = dims->h_q / dims->h_v;
    ga.cache_len = dims->cache_len;
    ga.rows_per_chunk = ch.rows;
    ga.chunks = ch.chunks;
    ga.pg = rm.pg;
    if (rm.pg.block_table) {
        const uint64_t pool = (uint64_t)rm.pg.num_pages * dims->h_v * rm.pg.page_rows * D * 2;
        ga.pool_bytes = pool + 16 * D <= (uint64_t)kPoolLimit ? (uint32_t)pool : 0u;
    }
    int64_t segs = (gather_target_blocks(D) + rows - 1) / rows;
    if (segs > kGatherMaxSegs) segs = kGatherMaxSegs;
    if (segs > L.max_chunks) segs = L.max_chunks;       // partials hold max_chunks per row
    ga.segs = (int)segs;
    int st = hip_status(launch_gather(D, ga, s));
    if (st != SAGA_OK) return st;
    return hip_status(launch_combine(D, ga.part, rows, ga.segs, static_cast<uint16_t*>(out_dev),
                                     sel_counts_dev, s));
}

// The small-batch path (fused.hip): with few (b, key head) groups a decode
// call is a chain of latency-bound launches, so the value gather runs inside
// the K-stream kernel, from entries kept in LDS.  The chunks are the pair
// plan of the stream (the same for paged and contiguous caches, so both give
// the same sums), shortened when needed so that a chunk's worst case (every
// row selected for every head slot) fits the LDS budget; never more chunks
// than the workspace's partials hold.  Launches of fewer than kFusedMinBlocks
// workgroups (short contexts) keep the list path: there a chunk's selected
// value rows are many for one workgroup to read, and the list path's gather
// spreads them over many.
constexpr int64_t kFusedMinBlocks = 64;

struct FusedPlan {
    bool use = false;
    Chunking ch{};
    int32_t scap = 0, unroll = 1;
    size_t lds = 0;
};

FusedPlan plan_fused(const saga_dims* dims, const Layout& L, const RowModel& rm)
{
    FusedPlan best;
    if (rm.v_scale) return best;                    // fp8 values: the list path
    const int64_t groups = (int64_t)dims->batch * dims->h_k;
    if (groups > SAGA_FUSED_MAX_GROUPS) return best;
    const int D = dims->head_dim, DV = value_dim(dims);
    const bool k8 = rm.k_scale != nullptr;
    const int Gk = dims->h_q / dims->h_k;
    // LDS bytes per row of a chunk: one 8-byte queue entry per head slot (a
    // wave's queue of a slot holds every row of its quarter of the chunk).
    const int64_t row_bytes = 8 * (int64_t)Gk;
    const int64_t R = kBlock / (Gk * (DV / 8));
    const size_t red = (size_t)(R * Gk * DV + R * Gk) * 4;
    auto lds_of = [&](int64_t rows) {
        const size_t lists = round_up((size_t)rows * row_bytes, 16);
        return lists > red ? lists : red;
    };
    // Tiles of two 16-row groups halve a long chunk's dependent round trips;
    // they are taken unless their longer pairs cost more than 30% of the chunks.
    for (const int U : {1, 2}) {
        const int64_t pair = 2 * fused_block_rows(U, k8);
        Chunking ch = split_rows(dims->ctx_len, groups, pair, target_blocks(D, k8), L.max_chunks);
        // Shorten the chunks until their worst case fits the LDS with every
        // workgroup of the launch resident at once.
        bool ok = false;
        for (;;) {
            const int64_t per_cu = (groups * ch.chunks + kComputeUnits - 1) / kComputeUnits;
            const size_t cap = (size_t)kLdsPerCu / (size_t)per_cu;
            if (lds_of(ch.rows) <= (cap < (size_t)kLdsPerGroup ? cap : (size_t)kLdsPerGroup)) {
                ok = true;
                break;
            }
            if (ch.rows <= pair) break;
            ch.rows -= pair;
            ch.chunks = (int)((dims->ctx_len + ch.rows - 1) / ch.rows);
            if (ch.chunks > L.max_chunks) break;
        }
        if (!ok || groups * ch.chunks < kFusedMinBlocks) continue;
        if (best.use && 10 * ch.chunks < 7 * best.ch.chunks) continue;
        FusedPlan f;
        f.use = true;
        f.unroll = U;
        f.ch = ch;
        f.scap = (int32_t)(ch.rows / kWavesPerBlock);
        f.lds = lds_of(ch.rows);
        best = f;
    }
    return best;
}

int enqueue_fused(const saga_dims* dims, const Layout& L, const FusedPlan& f, const void* q_dev,
                  const void* k_cache_dev, const void* v_cache_dev, const float* thresholds_dev,
                  void* out_dev, int32_t* sel_counts_dev, uint32_t* sel_bitmap_debug_dev,
                  int64_t words, void* workspace_dev, hipStream_t s, const RowModel& rm)
{
    FusedArgs a{};
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
    a.rows_per_chunk = f.ch.rows;
    a.chunks = f.ch.chunks;
    a.scap = f.scap;
    a.unroll = f.unroll;
    a.scale = dims->scale;
    a.lq = rm.lq;
    a.k_scale = rm.k_scale;
    a.pg = rm.pg;
    const int st = hip_status(launch_select_gather(dims->head_dim, value_dim(dims), a, f.lds, s));
    if (st != SAGA_OK) return st;
    return hip_status(launch_combine_parts(value_dim(dims), a.part, dims->batch * dims->h_q,
                                           f.ch.chunks, static_cast<uint16_t*>(out_dev),
                                           sel_counts_dev, s));
}

// Large-batch calls gather in the K stream's tail (decode.hip, tail_gather):
// contiguous V (bf16, or fp8 with an fp8 K cache) with d_v = d_k of 64 or
// 128, value heads of one key group addressable with 32-bit offsets, and
// a launch of at least kTailMinBlocks workgroups (fewer, longer chunks would
// leave each workgroup many value rows to read on its own, where the list
// path's gather spreads them).  At d = 128 the chunks must also be at least
// kTailMinRows128 rows: the workgroups then share a CU two at a time and keep
// half as many value rows in flight, and over shorter chunks (Qwen-like batch
// 16 at 32K context and below) the tail outlasts the stream it follows, so
// the list path is faster; at d = 64 the tail was faster at every length
// measured (8K to 128K).
constexpr int64_t kTailMinBlocks = 256;
constexpr int64_t kTailMinRows128 = 2048;

bool use_tail(const saga_dims* dims, const RowModel& rm, const Chunking& ch)
{
    if (!SAGA_TAIL_GATHER || rm.pg.block_table) return false;
    if (rm.v_scale && !rm.k_scale) return false;         // fp8 V comes with fp8 K
    const int D = dims->head_dim, Gk = dims->h_q / dims->h_k, Gv = dims->h_q / dims->h_v;
    if (value_dim(dims) != D || (D != 64 && D != 128) || Gk > 16) return false;
    if ((int64_t)dims->batch * dims->h_k * ch.chunks < kTailMinBlocks) return false;
    if (D == 128 && ch.rows < kTailMinRows128) return false;
    // Value heads one key group reads: ceil over its query heads' map.
    const int64_t nvh = (Gk + Gv - 1) / Gv + 1;
    return nvh * dims->cache_len * D * (rm.v_scale ? 1 : 2) < ((int64_t)1 << 31);
}

// Decode with kept thresholds: stream-select into the lists, then gather
// (or the small-batch path above, or the tail gather).
int enqueue_decode(const saga_dims* dims, const Layout& L, const void* q_dev,
                   const void* k_cache_dev, const void* v_cache_dev, const float* thresholds_dev,
                   void* out_dev, int32_t* sel_counts_dev, uint32_t* sel_bitmap_debug_dev,
                   void* workspace_dev, hipStream_t s, const RowModel& rm)
{
    const int D = dims->head_dim;
    const int rows = dims->batch * dims->h_q;
    const int64_t words = (dims->cache_len + 31) / 32;
    int st;
    if (sel_bitmap_debug_dev) {
        st = hip_status(launch_fill_u32(sel_bitmap_debug_dev, (int64_t)rows * words, 0u, s));
        if (st != SAGA_OK) return st;
    }
    const FusedPlan f = plan_fused(dims, L, rm);
    if (f.use)
        return enqueue_fused(dims, L, f, q_dev, k_cache_dev, v_cache_dev, thresholds_dev, out_dev,
                             sel_counts_dev, sel_bitmap_debug_dev, words, workspace_dev, s, rm);
    RowModel lrm = rm;
    const Chunking ch = list_chunks(dims, L, workspace_dev, &lrm);
    SelectStreamArgs a =
        stream_args(dims, L, ch, q_dev, k_cache_dev, thresholds_dev, workspace_dev, lrm);
    a.bitmap = sel_bitmap_debug_dev;
    a.bitmap_words = words;
    if (use_tail(dims, lrm, ch)) {
        a.v = static_cast<const uint16_t*>(v_cache_dev);
        a.part = partials(workspace_dev, L);
        a.hv = dims->h_v;
        a.Gv = dims->h_q / dims->h_v;
        a.v_scale = lrm.v_scale;
        st = hip_status(launch_select_stream(D, a, s));
        if (st != SAGA_OK) return st;
        return hip_status(launch_combine(D, a.part, rows, ch.chunks,
                                         static_cast<uint16_t*>(out_dev), sel_counts_dev, s));
    }
    st = hip_status(launch_select_stream(D, a, s));
    if (st != SAGA_OK) return st;
    return enqueue_gather_combine(dims, L, ch, v_cache_dev, nullptr, out_dev, sel_counts_dev,
                                  workspace_dev, s, lrm);
}

// Checks of a page description against the call's dims: pages of a multiple
// of kPageQuantum rows and cache_len = max_pages * page_rows.
int validate_paged(const saga_dims* d, const saga_paged* p, PagedKV* out)
{
    if (!p || !p->block_table_dev || !p->ctx_lens_dev) return SAGA_ERR_INVALID_ARGUMENT;
    if (misaligned(p->block_table_dev, 4) || misaligned(p->ctx_lens_dev, 4))
        return SAGA_ERR_INVALID_ARGUMENT;
    if (p->page_rows < kPageQuantum || p->page_rows % kPageQuantum != 0 || p->max_pages < 1 ||
        p->num_pages < 1 || p->reserved != 0)
        return SAGA_ERR_INVALID_ARGUMENT;
    if ((int64_t)p->max_pages * p->page_rows != d->cache_len) return SAGA_ERR_INVALID_ARGUMENT;
    out->block_table = p->block_table_dev;
    out->ctx_lens = p->ctx_lens_dev;
    out->page_rows = p->page_rows;
    out->max_pages = p->max_pages;
    out->num_pages = p->num_pages;
    return SAGA_OK;
}

int do_refresh(const saga_dims* dims, const RowModel& rm, int32_t top_n, const void* q_dev,
               const void* k_dev, float* thresholds_dev, float* logits_debug_dev,
               void* workspace_dev, size_t workspace_bytes, void* stream)
{
    if (top_n < 1 || !q_dev || !k_dev || !thresholds_dev || !workspace_dev)
        return SAGA_ERR_INVALID_ARGUMENT;
    if (misaligned(q_dev, 16) || misaligned(k_dev, 16) || misaligned(thresholds_dev, 4) ||
        misaligned(logits_debug_dev, 4) || misaligned(workspace_dev, 16))
        return SAGA_ERR_INVALID_ARGUMENT;
    const Layout L = make_layout(dims);
    if (workspace_bytes < L.total) return SAGA_ERR_WORKSPACE_TOO_SMALL;

    hipStream_t s = static_cast<hipStream_t>(stream);
    unsigned char* w = static_cast<unsigned char*>(workspace_dev);
    const int D = dims->head_dim;
    const int rows = dims->batch * dims->h_q;
    RowModel lrm = rm;
    const Chunking ch = list_chunks(dims, L, workspace_dev, &lrm);
    int st;
    if ((int64_t)top_n >= dims->ctx_len) {
        // N >= ctx (of every sequence): every entry is kept, tau = -inf.  The
        // logits are still produced when asked for (a pass that selects nothing).
        if (logits_debug_dev) {
            float* pivot = reinterpret_cast<float*>(w + L.pivot);
            st = hip_status(launch_fill_u32(reinterpret_cast<uint32_t*>(pivot), rows, 0x7f800000u, s));
            if (st != SAGA_OK) return st;
            SelectStreamArgs a = stream_args(dims, L, ch, q_dev, k_dev, pivot, workspace_dev, lrm);
            a.logits_out = logits_debug_dev;
            st = hip_status(launch_select_stream(D, a, s));
            if (st != SAGA_OK) return st;
        }
        return hip_status(launch_fill_u32(reinterpret_cast<uint32_t*>(thresholds_dev), rows,
                                          0xff800000u, s));
    }
    return enqueue_refresh(dims, top_n, q_dev, k_dev, thresholds_dev, logits_debug_dev,
                           workspace_dev, L, ch, s, nullptr, lrm);
}

int do_decode(const saga_dims* dims, const RowModel& rm, const void* q_dev, const void* k_dev,
              const void* v_dev, const float* thresholds_dev, void* out_dev,
              int32_t* sel_counts_dev, uint32_t* sel_bitmap_debug_dev, void* workspace_dev,
              size_t workspace_bytes, void* stream)
{
    if (!q_dev || !k_dev || !v_dev || !thresholds_dev || !out_dev || !workspace_dev)
        return SAGA_ERR_INVALID_ARGUMENT;
    if (misaligned(q_dev, 16) || misaligned(k_dev, 16) || misaligned(v_dev, 16) ||
        misaligned(thresholds_dev, 4) || misaligned(out_dev, 2) || misaligned(sel_counts_dev, 4) ||
        misaligned(sel_bitmap_debug_dev, 4) || misaligned(workspace_dev, 16))
        return SAGA_ERR_INVALID_ARGUMENT;
    const Layout L = make_layout(dims);
    if (workspace_bytes < L.total) return SAGA_ERR_WORKSPACE_TOO_SMALL;
    return enqueue_decode(dims, L, q_dev, k_dev, v_dev, thresholds_dev, out_dev, sel_counts_dev,
                          sel_bitmap_debug_dev, workspace_dev, static_cast<hipStream_t>(stream),
                          rm);
}

int do_refresh_decode(const saga_dims* dims, const RowModel& rm, int32_t top_n,
                      const void* q_dev, const void* k_dev, const void* v_dev,
                      float* thresholds_dev, void* out_dev, int32_t* sel_counts_dev,
                      void* workspace_dev, size_t workspace_bytes, void* stream)
{
    if (top_n < 1 || !q_dev || !k_dev || !v_dev || !thresholds_dev || !out_dev || !workspace_dev)
        return SAGA_ERR_INVALID_ARGUMENT;
    if (misaligned(q_dev, 16) || misaligned(k_dev, 16) || misaligned(v_dev, 16) ||
        misaligned(thresholds_dev, 4) || misaligned(out_dev, 2) || misaligned(sel_counts_dev, 4) ||
        misaligned(workspace_dev, 16))
        return SAGA_ERR_INVALID_ARGUMENT;
    const Layout L = make_layout(dims);
    if (workspace_bytes < L.total) return SAGA_ERR_WORKSPACE_TOO_SMALL;

    hipStream_t s = static_cast<hipStream_t>(stream);
    unsigned char* w = static_cast<unsigned char*>(workspace_dev);
    const int D = dims->head_dim;
    const int rows = dims->batch * dims->h_q;
    int st;
    if ((int64_t)top_n >= dims->ctx_len) {
        st = hip_status(launch_fill_u32(reinterpret_cast<uint32_t*>(thresholds_dev), rows,
                                        0xff800000u, s));
        if (st != SAGA_OK) return st;
        return enqueue_decode(dims, L, q_dev, k_dev, v_dev, thresholds_dev, out_dev,
                              sel_counts_dev, nullptr, workspace_dev, s, rm);
    }
    RowModel lrm = rm;
    const Chunking ch = list_chunks(dims, L, workspace_dev, &lrm);
    uint32_t* flags = reinterpret_cast<uint32_t*>(w + L.flags);
    st = enqueue_refresh(dims, top_n, q_dev, k_dev, thresholds_dev, nullptr, workspace_dev,
                         L, ch, s, flags, lrm);
    if (st != SAGA_OK) return st;
    // Key groups whose candidate lists miss selected entries (a row took the
    // recompute path) are streamed again with the fresh thresholds; every
    // other workgroup of this launch exits at once.
    SelectStreamArgs a = stream_args(dims, L, ch, q_dev, k_dev, thresholds_dev, workspace_dev, lrm);
    a.group_flags = flags;
    st = hip_status(launch_select_stream(D, a, s));
    if (st != SAGA_OK) return st;
    // The lists hold every logit >= tau (and more): keep those >= tau.
    return enqueue_gather_combine(dims, L, ch, v_dev, thresholds_dev, out_dev,
                                  sel_counts_dev, workspace_dev, s, lrm);
}

}  // namespace

namespace saga {

// saga_decode_step with the selection bitmap off, for the other source files
// of the library (declared in kernels.hpp).
size_t decode_workspace_bytes(const saga_dims* dims)
{
    return validate_dims(dims) == SAGA_OK ? make_layout(dims).total : 0;
}

int decode_step(const saga_dims* dims, const void* q_dev, const void* k_dev, const void* v_dev,
                const float* thresholds_dev, void* out_dev, int32_t* sel_counts_dev,
                void* workspace_dev, size_t workspace_bytes, void* stream)
{
    const int st = validate_dims(dims);
    if (st != SAGA_OK) return st;
    return do_decode(dims, RowModel{}, q_dev, k_dev, v_dev, thresholds_dev, out_dev,
                     sel_counts_dev, nullptr, workspace_dev, workspace_bytes, stream);
}

}  // namespace saga

SAGA_EXPORT int atopn_refresh_thresholds(const saga_dims* dims, int32_t top_n, const void* q_dev,
                                         const void* k_cache_dev, float* thresholds_dev,
                                         float* logits_debug_dev, void* workspace_dev,
                                         size_t workspace_bytes, void* stream)
{
    const int st = validate_dims(dims);
    if (st != SAGA_OK) return st;
    return do_refresh(dims, RowModel{}, top_n, q_dev, k_cache_dev, thresholds_dev, logits_debug_dev,
                      workspace_dev, workspace_bytes, stream);
}

SAGA_EXPORT int saga_decode_step(const saga_dims* dims, const void* q_dev, const void* k_cache_dev,
                                 const void* v_cache_dev, const float* thresholds_dev,
                                 void* out_dev, int32_t* sel_counts_dev,
                                 uint32_t* sel_bitmap_debug_dev, void* workspace_dev,
                                 size_t workspace_bytes, void* stream)
{
    const int st = validate_dims(dims);
    if (st != SAGA_OK) return st;
    return do_decode(dims, RowModel{}, q_dev, k_cache_dev, v_cache_dev, thresholds_dev, out_dev,
                     sel_counts_dev, sel_bitmap_debug_dev, workspace_dev, workspace_bytes, stream);
}

SAGA_EXPORT int atopn_refresh_decode_step(const saga_dims* dims, int32_t top_n, const void* q_dev,
                                          const void* k_cache_dev, const void* v_cache_dev,
                                          float* thresholds_dev, void* out_dev,
                                          int32_t* sel_counts_dev, void* workspace_dev,
                                          size_t workspace_bytes, void* stream)
{
    const int st = validate_dims(dims);
    if (st != SAGA_OK) return st;
    return do_refresh_decode(dims, RowModel{}, top_n, q_dev, k_cache_dev, v_cache_dev,
                             thresholds_dev, out_dev, sel_counts_dev, workspace_dev,
                             workspace_bytes, stream);
}

SAGA_EXPORT int atopn_refresh_thresholds_paged(const saga_dims* dims, const saga_paged* paged,
                                               int32_t top_n, const void* q_dev,
                                               const void* k_pages_dev, float* thresholds_dev,
                                               void* workspace_dev, size_t workspace_bytes,
                                               void* stream)
{
    int st = validate_dims(dims);
    if (st != SAGA_OK) return st;
    RowModel rm;
    st = validate_paged(dims, paged, &rm.pg);
    if (st != SAGA_OK) return st;
    return do_refresh(dims, rm, top_n, q_dev, k_pages_dev, thresholds_dev, nullptr, workspace_dev,
                      workspace_bytes, stream);
}

SAGA_EXPORT int saga_decode_step_paged(const saga_dims* dims, const saga_paged* paged,
                                       const void* q_dev, const void* k_pages_dev,
                                       const void* v_pages_dev, const float* thresholds_dev,
                                       void* out_dev, int32_t* sel_counts_dev, void* workspace_dev,
                                       size_t workspace_bytes, void* stream)
{
    int st = validate_dims(dims);
    if (st != SAGA_OK) return st;
    RowModel rm;
    st = validate_paged(dims, paged, &rm.pg);
    if (st != SAGA_OK) return st;
    return do_decode(dims, rm, q_dev, k_pages_dev, v_pages_dev, thresholds_dev, out_dev,
                     sel_counts_dev, nullptr, workspace_dev, workspace_bytes, stream);
}

SAGA_EXPORT int atopn_refresh_decode_step_paged(const saga_dims* dims, const saga_paged* paged,
                                                int32_t top_n, const void* q_dev,
                                                const void* k_pages_dev, const void* v_pages_dev,
                                                float* thresholds_dev, void* out_dev,
                                                int32_t* sel_counts_dev, void* workspace_dev,
                                                size_t workspace_bytes, void* stream)
{
    int st = validate_dims(dims);
    if (st != SAGA_OK) return st;
    RowModel rm;
    st = validate_paged(dims, paged, &rm.pg);
    if (st != SAGA_OK) return st;
    return do_refresh_decode(dims, rm, top_n, q_dev, k_pages_dev, v_pages_dev, thresholds_dev,
                             out_dev, sel_counts_dev, workspace_dev, workspace_bytes, stream);
}

namespace {

// The call's dims with one virtual query head per (query head, token).
int lq_dims(const saga_dims* dims, int32_t l_q, saga_dims* v)
{
    int st = validate_dims(dims);
    if (st != SAGA_OK) return st;
    if (l_q < 1 || (int64_t)l_q > dims->ctx_len) return SAGA_ERR_INVALID_ARGUMENT;
    *v = *dims;
    v->h_q = dims->h_q * l_q;
    return validate_dims(v);         // UNSUPPORTED past 16 query slots per key head
}

}  // namespace

SAGA_EXPORT int atopn_refresh_thresholds_lq(const saga_dims* dims, int32_t l_q, int32_t top_n,
                                            const void* q_dev, const void* k_cache_dev,
                                            float* thresholds_dev, void* workspace_dev,
                                            size_t workspace_bytes, void* stream)
{
    saga_dims v;
    const int st = lq_dims(dims, l_q, &v);
    if (st != SAGA_OK) return st;
    RowModel rm;
    rm.lq = l_q;
    return do_refresh(&v, rm, top_n, q_dev, k_cache_dev, thresholds_dev, nullptr, workspace_dev,
                      workspace_bytes, stream);
}

SAGA_EXPORT int saga_decode_step_lq(const saga_dims* dims, int32_t l_q, const void* q_dev,
                                    const void* k_cache_dev, const void* v_cache_dev,
                                    const float* thresholds_dev, void* out_dev,
                                    int32_t* sel_counts_dev, void* workspace_dev,
                                    size_t workspace_bytes, void* stream)
{
    saga_dims v;
    const int st = lq_dims(dims, l_q, &v);
    if (st != SAGA_OK) return st;
    RowModel rm;
    rm.lq = l_q;
    return do_decode(&v, rm, q_dev, k_cache_dev, v_cache_dev, thresholds_dev, out_dev,
                     sel_counts_dev, nullptr, workspace_dev, workspace_bytes, stream);
}

SAGA_EXPORT int atopn_refresh_decode_step_lq(const saga_dims* dims, int32_t l_q, int32_t top_n,
                                             const void* q_dev, const void* k_cache_dev,
                                             const void* v_cache_dev, float* thresholds_dev,
                                             void* out_dev, int32_t* sel_counts_dev,
                                             void* workspace_dev, size_t workspace_bytes,
                                             void* stream)
{
    saga_dims v;
    const int st = lq_dims(dims, l_q, &v);
    if (st != SAGA_OK) return st;
    RowModel rm;
    rm.lq = l_q;
    return do_refresh_decode(&v, rm, top_n, q_dev, k_cache_dev, v_cache_dev, thresholds_dev,
                             out_dev, sel_counts_dev, workspace_dev, workspace_bytes, stream);
}

namespace {

// An fp8 K cache: a scale pointer (4-byte aligned) per call.
int fp8k_model(const saga_dims* dims, const float* k_scale_dev, RowModel* rm)
{
    const int st = validate_dims(dims);
    if (st != SAGA_OK) return st;
    if (!k_scale_dev || misaligned(k_scale_dev, 4)) return SAGA_ERR_INVALID_ARGUMENT;
    if (dims->head_dim < 64) return SAGA_ERR_UNSUPPORTED;   // fp8 loads cover 64 bytes of a row
    rm->k_scale = k_scale_dev;
    return SAGA_OK;
}

}  // namespace

SAGA_EXPORT int atopn_refresh_thresholds_fp8k(const saga_dims* dims, int32_t top_n,
                                              const void* q_dev, const void* k8_cache_dev,
                                              const float* k_scale_dev, float* thresholds_dev,
                                              float* logits_debug_dev, void* workspace_dev,
                                              size_t workspace_bytes, void* stream)
{
    RowModel rm;
    const int st = fp8k_model(dims, k_scale_dev, &rm);
    if (st != SAGA_OK) return st;
    return do_refresh(dims, rm, top_n, q_dev, k8_cache_dev, thresholds_dev, logits_debug_dev,
                      workspace_dev, workspace_bytes, stream);
}

SAGA_EXPORT int saga_decode_step_fp8k(const saga_dims* dims, const void* q_dev,
                                      const void* k8_cache_dev, const float* k_scale_dev,
                                      const void* v_cache_dev, const float* thresholds_dev,
                                      void* out_dev, int32_t* sel_counts_dev,
                                      uint32_t* sel_bitmap_debug_dev, void* workspace_dev,
                                      size_t workspace_bytes, void* stream)
{
    RowModel rm;
    const int st = fp8k_model(dims, k_scale_dev, &rm);
    if (st != SAGA_OK) return st;
    return do_decode(dims, rm, q_dev, k8_cache_dev, v_cache_dev, thresholds_dev, out_dev,
                     sel_counts_dev, sel_bitmap_debug_dev, workspace_dev, workspace_bytes, stream);
}

SAGA_EXPORT int atopn_refresh_decode_step_fp8k(const saga_dims* dims, int32_t top_n,
                                               const void* q_dev, const void* k8_cache_dev,
                                               const float* k_scale_dev, const void* v_cache_dev,
                                               float* thresholds_dev, void* out_dev,
                                               int32_t* sel_counts_dev, void* workspace_dev,
                                               size_t workspace_bytes, void* stream)
{
    RowModel rm;
    const int st = fp8k_model(dims, k_scale_dev, &rm);
    if (st != SAGA_OK) return st;
    return do_refresh_decode(dims, rm, top_n, q_dev, k8_cache_dev, v_cache_dev, thresholds_dev,
                             out_dev, sel_counts_dev, workspace_dev, workspace_bytes, stream);
}

namespace {

// fp8 K and V caches: both scale pointers (4-byte aligned) per call.
int fp8kv_model(const saga_dims* dims, const float* k_scale_dev, const float* v_scale_dev,
                RowModel* rm)
{
    const int st = fp8k_model(dims, k_scale_dev, rm);
    if (st != SAGA_OK) return st;
    if (!v_scale_dev || misaligned(v_scale_dev, 4)) return SAGA_ERR_INVALID_ARGUMENT;
    rm->v_scale = v_scale_dev;
    return SAGA_OK;
}

}  // namespace

SAGA_EXPORT int saga_decode_step_fp8kv(const saga_dims* dims, const void* q_dev,
                                       const void* k8_cache_dev, const float* k_scale_dev,
                                       const void* v8_cache_dev, const float* v_scale_dev,
                                       const float* thresholds_dev, void* out_dev,
                                       int32_t* sel_counts_dev, uint32_t* sel_bitmap_debug_dev,
                                       void* workspace_dev, size_t workspace_bytes, void* stream)
{
    RowModel rm;
    const int st = fp8kv_model(dims, k_scale_dev, v_scale_dev, &rm);
    if (st != SAGA_OK) return st;
    return do_decode(dims, rm, q_dev, k8_cache_dev, v8_cache_dev, thresholds_dev, out_dev,
                     sel_counts_dev, sel_bitmap_debug_dev, workspace_dev, workspace_bytes, stream);
}

SAGA_EXPORT int atopn_refresh_decode_step_fp8kv(const saga_dims* dims, int32_t top_n,
                                                const void* q_dev, const void* k8_cache_dev,
                                                const float* k_scale_dev, const void* v8_cache_dev,
                                                const float* v_scale_dev, float* thresholds_dev,
                                                void* out_dev, int32_t* sel_counts_dev,
                                                void* workspace_dev, size_t workspace_bytes,
                                                void* stream)
{
    RowModel rm;
    const int st = fp8kv_model(dims, k_scale_dev, v_scale_dev, &rm);
    if (st != SAGA_OK) return st;
    return do_refresh_decode(dims, rm, top_n, q_dev, k8_cache_dev, v8_cache_dev, thresholds_dev,
                             out_dev, sel_counts_dev, workspace_dev, workspace_bytes, stream);
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

    const int D = dims->head_dim, DV = value_dim(dims);
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
    const int64_t block_rows = (int64_t)kWavesPerBlock * 16 * full_unroll(D, DV);
    const Chunking ch = split_rows(dims->ctx_len, (int64_t)dims->batch * dims->h_k, block_rows,
                                   kFullTargetBlocks, L.max_chunks);
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
    a.wave_lds = full_wave_lds_bytes(D, DV, maxs_t);
    st = hip_status(launch_full(D, DV, maxs_t, a, s));
    if (st != SAGA_OK) return st;
    return hip_status(launch_combine(DV, a.part, dims->batch * dims->h_q, ch.chunks,
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

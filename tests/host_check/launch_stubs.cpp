// launch_stubs.cpp -- host stand-ins for the kernel launchers of libsaga.so,
// for a CPU build of the C-ABI host code (api.hip) under AddressSanitizer and
// UndefinedBehaviorSanitizer.
//
// Each stub receives exactly the arguments the real launcher would, checks the
// launch shape the kernel assumes, and then reads or writes the first and the
// last element of every buffer region that the kernel indexes, at the largest
// index the kernel's own indexing can reach for those arguments.  The caller
// (abi_driver.cpp) passes host heap buffers of exactly the documented sizes in
// place of device memory, so a workspace region, a chunk plan or an output
// size that is too small for its kernel shows up as a heap-buffer-overflow.
// Regions that live inside the caller's workspace are also recorded by name
// with the extent the kernel uses ([lowest, highest] element touched), and
// the driver checks after each call that no two regions overlap: an overrun
// from one region into the next stays inside the workspace allocation, where
// the address sanitizer cannot see it.
// Nothing here computes attention.
#include <stdio.h>
#include <stdlib.h>

#include <type_traits>
#include <vector>

#include "kernels.hpp"

namespace saga {

int g_launches = 0;   // launches since the driver last cleared it
int g_fused_launches = 0;   // select_gather launches (the small-batch path), same
int g_tail_launches = 0;    // K-stream launches that gather in their tail, same

struct TouchedRange {
    const char* name;
    uintptr_t lo, hi;     // bytes [lo, hi)
};
std::vector<TouchedRange> g_ranges;   // cleared by the driver

namespace {

volatile unsigned char g_sink;

[[noreturn]] void fail(const char* what)
{
    fprintf(stderr, "launch stub: %s\n", what);
    abort();
}
#define EXPECT(c) do { if (!(c)) fail(#c); } while (0)

template <typename T>
void rd(const T* p, int64_t i)
{
    EXPECT(p != nullptr && i >= 0);
    const volatile unsigned char* b = reinterpret_cast<const volatile unsigned char*>(p + i);
    for (size_t k = 0; k < sizeof(T); ++k) g_sink = b[k];
}
template <typename T>
void wr(T* p, int64_t i)
{
    EXPECT(p != nullptr && i >= 0);
    volatile unsigned char* b = reinterpret_cast<volatile unsigned char*>(p + i);
    for (size_t k = 0; k < sizeof(T); ++k) b[k] = b[k];
}
// Records elements [i0, i1] of p as region `name`.
template <typename T>
void note(const char* name, const T* p, int64_t i0, int64_t i1)
{
    g_ranges.push_back({name, reinterpret_cast<uintptr_t>(p + i0), reinterpret_cast<uintptr_t>(p + i1 + 1)});
}
// First and last element of [0, n).
template <typename T> void rd_span(const T* p, int64_t n) { if (n > 0) { rd(p, 0); rd(p, n - 1); } }
template <typename T> void wr_span(T* p, int64_t n) { if (n > 0) { wr(p, 0); wr(p, n - 1); } }
// Same, recorded as a named region.
template <typename T>
void rd_span(const char* name, const T* p, int64_t n) { if (n > 0) { rd_span(p, n); note(name, p, 0, n - 1); } }
template <typename T>
void wr_span(const char* name, T* p, int64_t n) { if (n > 0) { wr_span(p, n); note(name, p, 0, n - 1); } }

// Selection-list entries: list `local` of row `head` holds at most capw
// entries (see list_index).
int64_t entry_index(int64_t head, int64_t local, int64_t E, int64_t capw, int64_t nl,
                    int64_t head_stride, int64_t overflow_at)
{
    return E < kListPrimary ? (head * nl + local) * kListPrimary + E
                            : overflow_at + head * head_stride + local * capw + (E - kListPrimary);
}

// The lists a call's kernels index: rows 0 .. heads-1, lists 0 .. used-1 of
// the nl per row, capw entries each.
struct ListUse {
    int64_t heads, nl, used, capw, head_stride, overflow_at;
};

// Host model of paged_rows_per_chunk / paged_chunks (kernels.hpp), from the
// lengths the driver passes in host memory: the rows per chunk and the most
// chunks any sequence uses and the K stream's work items.
void paged_plan(const PagedKV& pg, int B, int hk, int64_t ctx, int64_t* rpc, int64_t* most,
                int64_t* items)
{
    const int64_t cap = (int64_t)pg.max_pages * pg.page_rows;
    int64_t sum = 0, mx = 0;
    for (int b = 0; b < B; ++b) {
        int64_t c = pg.ctx_lens[b];
        c = c < 0 ? 0 : (c > cap ? cap : c);
        c = c < ctx ? c : ctx;
        sum += c;
        mx = c > mx ? c : mx;
    }
    const int64_t q = pg.plan_quantum;
    auto up = [q](int64_t x) { return (x + q - 1) / q * q; };
    int64_t r = up(((int64_t)hk * sum + pg.plan_target - 1) / pg.plan_target);
    r = r < pg.plan_rows_max ? r : pg.plan_rows_max;
    const int64_t need = up((mx + pg.plan_cap - 1) / pg.plan_cap);
    r = r > need ? r : need;
    r = r > q ? r : q;
    auto count = [&](int64_t rr) {
        int64_t n = 0;
        for (int b = 0; b < B; ++b) {
            int64_t c = pg.ctx_lens[b];
            c = c < 0 ? 0 : (c > cap ? cap : c);
            c = c < ctx ? c : ctx;
            n += (c + rr - 1) / rr * hk;
        }
        return n;
    };
    if (count(r) > pg.plan_target) {
        int64_t lo = r / q, hi = up(mx) / q;
        hi = hi < pg.plan_rows_max / q ? hi : pg.plan_rows_max / q;
        if (hi > lo) {
            while (hi - lo > 1) {
                const int64_t mid = lo + (hi - lo) / 2;
                if (count(mid * q) > pg.plan_target) lo = mid; else hi = mid;
            }
            r = hi * q;
        }
    }
    *rpc = r;
    *most = (mx + r - 1) / r;
    *items = count(r);
}

// Lists of one list-path call; checks the chunk plan the kernels follow.
ListUse list_use(int B, int hq, int hk, int64_t ctx, int chunks, int64_t rows_per_chunk,
                 const PagedKV& pg, int64_t head_stride, int64_t overflow_at)
{
    EXPECT(chunks >= 1 && rows_per_chunk >= 1);
    EXPECT((int64_t)chunks * kWavesPerBlock <= kMaxListsPerRow);
    int64_t rpc = rows_per_chunk, used_chunks = chunks;
    if (pg.block_table && pg.plan_cap) {
        EXPECT(pg.plan_cap == chunks);
        EXPECT(pg.plan_target >= 1 && pg.plan_quantum >= 64 && pg.plan_quantum % 64 == 0);
        EXPECT(pg.plan_rows_max >= pg.plan_quantum);
        int64_t items = 0;
        paged_plan(pg, B, hk, ctx, &rpc, &used_chunks, &items);
        EXPECT(used_chunks <= chunks);                    // every row of every sequence
        EXPECT(rpc <= pg.plan_rows_max);
        EXPECT(items <= pg.plan_grid);                    // one K-stream workgroup per item
        EXPECT(pg.plan_grid <= (int64_t)B * hk * chunks && pg.plan_grid <= 0x7fffffffLL);
    } else {
        EXPECT((int64_t)chunks * rows_per_chunk >= ctx);      // every row in a chunk
        EXPECT((int64_t)(chunks - 1) * rows_per_chunk < ctx); // no chunk entirely empty
    }
    EXPECT(rpc % 64 == 0);                                    // whole 4-wave tiles
    // A row's overflow entries (the last at used*rpc - kListPrimary - 1 past
    // the row's start) stay inside its head_stride slots.
    EXPECT(used_chunks * rpc <= head_stride + kListPrimary);
    return {(int64_t)B * hq, (int64_t)chunks * kWavesPerBlock, used_chunks * kWavesPerBlock,
            rpc / kWavesPerBlock, head_stride, overflow_at};
}

template <typename T>
void touch_lists(T* entries, const ListUse& u)
{
    EXPECT(u.capw >= 1 && u.heads >= 1 && u.used >= 0 && u.used <= u.nl);
    if (u.used == 0) return;                     // every sequence empty: no list is used
    const int64_t h1 = u.heads - 1, l1 = u.used - 1;
    const int64_t top = u.capw - 1 < kListPrimary ? u.capw - 1 : kListPrimary - 1;
    auto at = [&](int64_t h, int64_t l, int64_t E) {
        return entry_index(h, l, E, u.capw, u.nl, u.head_stride, u.overflow_at);
    };
    note("list entries (primary)", entries, 0, at(h1, l1, top));
    if (u.capw > kListPrimary)
        note("list entries (overflow)", entries, at(0, 0, kListPrimary), at(h1, l1, u.capw - 1));
    for (const int64_t h : {(int64_t)0, h1})
        for (const int64_t lid : {(int64_t)0, l1}) {
            const int64_t hi = u.capw - 1;
            const int64_t e1 = hi < kListPrimary ? hi : kListPrimary - 1;
            if constexpr (std::is_const_v<T>) {
                rd(entries, at(h, lid, 0));
                rd(entries, at(h, lid, e1));
                if (hi >= kListPrimary) {
                    rd(entries, at(h, lid, kListPrimary));
                    rd(entries, at(h, lid, hi));
                }
            } else {
                wr(entries, at(h, lid, 0));
                wr(entries, at(h, lid, e1));
                if (hi >= kListPrimary) {
                    wr(entries, at(h, lid, kListPrimary));
                    wr(entries, at(h, lid, hi));
                }
            }
        }
}

// Last K (or V) element a kernel reads for a contiguous cache of `heads`
// heads: row ctx - 1 of the last head.  esize: bytes per element.
void touch_cache(const void* c, int B, int heads, int64_t cache_len, int64_t ctx, int D, int esize)
{
    const unsigned char* p = static_cast<const unsigned char*>(c);
    rd(p, 0);
    rd(p, (((int64_t)B * heads - 1) * cache_len + ctx - 1) * D * esize + (int64_t)D * esize - 1);
}

void touch_paged(const PagedKV& pg, int B)
{
    rd(pg.ctx_lens, B - 1);
    rd(pg.block_table, (int64_t)B * pg.max_pages - 1);
}

void touch_partials(const Partials& p, int64_t parts, int D)
{
    wr_span("partials m", p.m, parts);
    wr_span("partials l", p.l, parts);
    wr_span("partials c", p.c, parts);
    wr_span("partials o", p.o, parts * D);
}

}  // namespace

hipError_t launch_select_stream(int D, const SelectStreamArgs& a, hipStream_t)
{
    ++g_launches;
    EXPECT(D == 32 || D == 64 || D == 128);
    EXPECT(a.B >= 1 && a.hk >= 1 && a.hq == a.hk * a.Gk && a.Gk <= 16);
    EXPECT((int64_t)a.B * a.hk <= 65535);                       // grid.y
    const ListUse u = list_use(a.B, a.hq, a.hk, a.ctx, a.chunks, a.rows_per_chunk, a.pg,
                               a.head_stride, a.overflow_at);
    const int64_t lists = (int64_t)a.B * a.hq * a.chunks * kWavesPerBlock;
    if (a.v) {
        // The tail gather: contiguous bf16 V with d_v = d_k, at most 16 head
        // slots, one partial per (b*h_q + i, chunk), the key group's value
        // heads under 2^31 bytes (32-bit buffer offsets).
        ++g_tail_launches;
        EXPECT(!a.pg.block_table && (D == 64 || D == 128) && a.Gk <= 16);
        EXPECT(a.hv >= 1 && a.Gv >= 1 && a.hq == a.hv * a.Gv);
        EXPECT(a.chunks >= 1 && (int64_t)a.chunks * a.rows_per_chunk >= a.ctx);
        const int64_t nvh = (int64_t)(a.Gk + a.Gv - 1) / a.Gv + 1;
        EXPECT(nvh * a.cache_len * D * (a.v_scale ? 1 : 2) < ((int64_t)1 << 31));
        EXPECT(!a.v_scale || a.k_scale);
        touch_partials(a.part, (int64_t)a.B * a.hq * a.chunks, D);
        touch_cache(a.v, a.B, a.hv, a.cache_len, a.ctx, D, a.v_scale ? 1 : 2);
        if (a.v_scale) rd_span(a.v_scale, (int64_t)a.B * a.hv);
    } else {
        wr_span("list counts", a.list_count, lists);
        wr_span("list maxima", a.list_max, lists);
    }
    touch_lists(a.entries, u);
    if (a.pg.block_table && a.pg.plan_cap) wr_span("paged plan", a.pg.plan, (int64_t)a.B + 1);
    rd_span(a.q, (int64_t)a.B * a.hq * D);
    rd_span(a.tau, (int64_t)a.B * a.hq);
    if (a.group_flags) rd_span("group flags", a.group_flags, (int64_t)a.B * a.hk);
    if (a.k_scale) rd_span(a.k_scale, (int64_t)a.B * a.hk);
    if (a.logits_out) wr_span(a.logits_out, (int64_t)a.B * a.hq * a.ctx);
    if (a.bitmap) {
        EXPECT(a.bitmap_words * 32 >= a.cache_len);
        wr(a.bitmap, 0);
        wr(a.bitmap, ((int64_t)a.B * a.hq - 1) * a.bitmap_words + (a.ctx - 1) / 32);
    }
    if (a.pg.block_table) touch_paged(a.pg, a.B);
    else touch_cache(a.k, a.B, a.hk, a.cache_len, a.ctx, D, a.k_scale ? 1 : 2);
    return hipSuccess;
}

hipError_t launch_gather(int D, const GatherArgs& a, hipStream_t)
{
    ++g_launches;
    EXPECT(D == 32 || D == 64 || D == 128);
    EXPECT(a.segs >= 1);
    EXPECT(a.hq == a.hv * a.Gv && a.hq % a.hk == 0);
    EXPECT((int64_t)a.segs * a.B * a.hq <= 0x7fffffffLL);      // 1-D grid
    const ListUse u = list_use(a.B, a.hq, a.hk, a.ctx, a.chunks, a.rows_per_chunk, a.pg,
                               a.head_stride, a.overflow_at);
    const int64_t lists = (int64_t)a.B * a.hq * a.chunks * kWavesPerBlock;
    rd_span("list counts", a.list_count, lists);
    rd_span("list maxima", a.list_max, lists);
    touch_lists(a.entries, u);
    if (a.pg.block_table && a.pg.plan_cap) rd_span("paged plan", a.pg.plan, (int64_t)a.B + 1);
    if (a.tau_filter) rd_span(a.tau_filter, (int64_t)a.B * a.hq);
    if (a.v_scale) rd_span(a.v_scale, (int64_t)a.B * a.hv);
    touch_partials(a.part, (int64_t)a.B * a.hq * a.segs, D);
    if (a.pg.block_table) touch_paged(a.pg, a.B);
    else touch_cache(a.v, a.B, a.hv, a.cache_len, a.cache_len, D, a.v_scale ? 1 : 2);
    return hipSuccess;
}

hipError_t launch_combine(int D, const Partials& p, int rows, int parts, uint16_t* out,
                          int32_t* counts, hipStream_t)
{
    ++g_launches;
    EXPECT(D == 32 || D == 64 || D == 128);
    EXPECT(rows >= 1 && parts >= 1);
    const int64_t n = (int64_t)rows * parts;
    rd_span("partials m", p.m, n);
    rd_span("partials l", p.l, n);
    rd_span("partials c", p.c, n);
    rd_span("partials o", p.o, n * D);
    wr_span(out, (int64_t)rows * D);
    if (counts) wr_span(counts, rows);
    return hipSuccess;
}

hipError_t launch_sample(int D, const SampleArgs& a, hipStream_t)
{
    ++g_launches;
    EXPECT(D == 32 || D == 64 || D == 128);
    EXPECT(a.m >= 1 && a.m <= kSampleMax && (a.m % 16 == 0 || a.m == a.ctx));
    EXPECT(a.stride % 16 == 0 && a.stride >= 16);
    EXPECT(a.rank >= 1 && a.rank <= a.m);
    const int64_t last_row = (int64_t)((a.m - 1) / 16) * a.stride + (a.m - 1) % 16;
    EXPECT(last_row < a.ctx);
    rd_span(a.q, (int64_t)a.B * a.hq * D);
    wr_span("sample logits", a.sample, ((int64_t)a.B * a.hq - 1) * kSampleMax + a.m);
    wr_span("pivots", a.pivot, (int64_t)a.B * a.hq);
    if (a.group_flags) wr_span("group flags", a.group_flags, (int64_t)a.B * a.hk);
    if (a.k_scale) rd_span(a.k_scale, (int64_t)a.B * a.hk);
    if (a.pg.block_table) touch_paged(a.pg, a.B);
    else touch_cache(a.k, a.B, a.hk, a.cache_len, last_row + 1, D, a.k_scale ? 1 : 2);
    return hipSuccess;
}

hipError_t launch_refresh_final(int D, const FinalArgs& a, hipStream_t)
{
    ++g_launches;
    EXPECT(D == 32 || D == 64 || D == 128);
    EXPECT(a.top_n >= 1 && (int64_t)a.top_n < a.ctx);
    const ListUse u = list_use(a.B, a.hq, a.hk, a.ctx, a.chunks, a.rows_per_chunk, a.pg,
                               a.head_stride, a.overflow_at);
    const int64_t lists = (int64_t)a.B * a.hq * a.chunks * kWavesPerBlock;
    rd_span("list counts", a.list_count, lists);
    touch_lists(a.entries, u);
    if (a.pg.block_table && a.pg.plan_cap) rd_span("paged plan", a.pg.plan, (int64_t)a.B + 1);
    wr_span(a.tau, (int64_t)a.B * a.hq);
    if (a.group_flags) wr_span("group flags", a.group_flags, (int64_t)a.B * a.hk);
    rd_span(a.q, (int64_t)a.B * a.hq * D);
    if (a.k_scale) rd_span(a.k_scale, (int64_t)a.B * a.hk);
    if (a.pg.block_table) touch_paged(a.pg, a.B);
    else touch_cache(a.k, a.B, a.hk, a.cache_len, a.ctx, D, a.k_scale ? 1 : 2);
    return hipSuccess;
}

hipError_t launch_full(int DK, int DV, int maxs, const FullArgs& a, hipStream_t)
{
    ++g_launches;
    EXPECT(maxs == 2 || maxs == 4 || maxs == 8);
    EXPECT(a.nv >= 1 && a.nv <= 4);
    EXPECT(a.chunks >= 1 && (int64_t)a.chunks * a.rows_per_chunk >= a.ctx);
    EXPECT((int64_t)(a.chunks - 1) * a.rows_per_chunk < a.ctx);
    EXPECT((int64_t)a.B * a.hk <= 65535);
    EXPECT(a.wave_lds * kWavesPerBlock <= 160 * 1024);
    touch_partials(a.part, (int64_t)a.B * a.hq * a.chunks, DV);
    rd_span(a.q, (int64_t)a.B * a.hq * DK);
    touch_cache(a.k, a.B, a.hk, a.cache_len, a.ctx, DK, 2);
    touch_cache(a.v, a.B, a.hv, a.cache_len, a.ctx, DV, 2);
    return hipSuccess;
}

hipError_t launch_select_gather(int D, int DV, const FusedArgs& a, size_t lds_bytes, hipStream_t)
{
    ++g_launches;
    ++g_fused_launches;
    EXPECT(D == 32 || D == 64 || D == 128);
    EXPECT(DV == 32 || DV == 64 || DV == 128);
    EXPECT(a.B >= 1 && a.hk >= 1 && a.hq == a.hk * a.Gk && a.Gk <= 16 && a.hq == a.hv * a.Gv);
    EXPECT((int64_t)a.B * a.hk <= 65535);
    EXPECT(a.chunks >= 1 && (int64_t)a.chunks * a.rows_per_chunk >= a.ctx);
    EXPECT((int64_t)(a.chunks - 1) * a.rows_per_chunk < a.ctx);
    EXPECT(a.unroll == 1 || a.unroll == 2);
    EXPECT(a.rows_per_chunk % (2 * fused_block_rows(a.unroll, a.k_scale != nullptr)) == 0);
    // Every row of a wave's share fits its queue of each head slot.
    EXPECT((int64_t)a.scap * kWavesPerBlock >= a.rows_per_chunk);
    EXPECT((int64_t)a.B * a.hk * a.chunks >= 64);               // the plan's smallest fused launch
    EXPECT(lds_bytes >= (size_t)kWavesPerBlock * a.Gk * a.scap * 8);
    EXPECT(lds_bytes <= (size_t)kLdsPerGroup);
    const int64_t per_cu = ((int64_t)a.B * a.hk * a.chunks + kComputeUnits - 1) / kComputeUnits;
    EXPECT((int64_t)lds_bytes * per_cu <= kLdsPerCu);           // every workgroup resident
    const int64_t P = (int64_t)a.Gk * (DV / 8), R = kBlock / P;
    EXPECT(R >= 1 && lds_bytes >= (size_t)(R * a.Gk * DV + R * a.Gk) * 4);
    touch_partials(a.part, (int64_t)a.B * a.hq * a.chunks, DV);
    rd_span(a.q, (int64_t)a.B * a.hq * D);
    rd_span(a.tau, (int64_t)a.B * a.hq);
    if (a.k_scale) rd_span(a.k_scale, (int64_t)a.B * a.hk);
    if (a.logits_out) wr_span(a.logits_out, (int64_t)a.B * a.hq * a.ctx);
    if (a.bitmap) {
        wr(a.bitmap, 0);
        wr(a.bitmap, ((int64_t)a.B * a.hq - 1) * a.bitmap_words + (a.ctx - 1) / 32);
    }
    if (a.pg.block_table) {
        touch_paged(a.pg, a.B);
    } else {
        touch_cache(a.k, a.B, a.hk, a.cache_len, a.ctx, D, a.k_scale ? 1 : 2);
        touch_cache(a.v, a.B, a.hv, a.cache_len, a.cache_len, DV, 2);
    }
    return hipSuccess;
}

hipError_t launch_combine_parts(int D, const Partials& p, int rows, int parts, uint16_t* out,
                                int32_t* counts, hipStream_t s)
{
    EXPECT(D % 16 == 0);
    return launch_combine(D, p, rows, parts, out, counts, s);   // same buffers, same extents
}

hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t, hipStream_t)
{
    ++g_launches;
    wr_span(p, n);
    return hipSuccess;
}

}  // namespace saga

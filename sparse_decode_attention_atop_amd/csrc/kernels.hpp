// kernels.hpp -- internal interface between the C-ABI host code (api.hip) and
// the kernel files.  Nothing here is exported from libsaga.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "device.hpp"

namespace saga {

// Rows of one workgroup tile (4 waves x 16*U rows) per kernel family and
// key head_dim; chunk lengths are multiples of these.
constexpr int decode_unroll(int D)
{
    return D == 32 ? SAGA_STREAM_U32 : (D == 64 ? SAGA_STREAM_U64 : SAGA_STREAM_U128);
}
constexpr int decode_block_rows(int D) { return kWavesPerBlock * 16 * decode_unroll(D); }
// fp8 K: tiles of SAGA_STREAM_K8_UMUL times the rows of bf16 tiles.
constexpr int decode_unroll_k8(int D) { return SAGA_STREAM_K8_UMUL * decode_unroll(D); }
constexpr int decode_block_rows_k8(int D) { return kWavesPerBlock * 16 * decode_unroll_k8(D); }
// MI355X: compute units, LDS per CU, and the LDS one workgroup may use.
constexpr int64_t kComputeUnits = 256;
constexpr int64_t kLdsPerCu = 160 * 1024;
constexpr int64_t kLdsPerGroup = 64 * 1024;

// Small-batch fused path: 16-row groups per wave tile, 1 or 2, chosen per call
// (2 halves the dependent round trips of a long chunk; a tile pair of 2 is
// 256 rows, which still never straddles a page).
constexpr int fused_block_rows(int U, bool k8)
{
    return kWavesPerBlock * 16 * U * (k8 ? SAGA_STREAM_K8_UMUL : 1);
}
// Dense kernel: 16-row groups per wave tile (the K tile and the V tile of the
// same rows are in registers together).
constexpr int full_unroll(int DK, int DV) { return (DK == 128 || DV == 128) ? 2 : 4; }

// LDS bytes of one wave in the full-attention kernel:
//   P[TR][16] fp32, alpha[16], m[16], l[16], o[MAXS][DV]
inline __host__ __device__ size_t full_wave_lds_bytes(int DK, int DV, int maxs)
{
    const int TR = 16 * full_unroll(DK, DV);
    size_t b = (size_t)TR * 16 * 4 + 3 * 16 * 4 + (size_t)maxs * DV * 4;
    return (b + 15) & ~(size_t)15;
}

// Radix select: 11 + 11 + 10 bits of the order-preserving key.
constexpr int kHistBins = 2048;

// Threshold refresh: sample size cap, candidates staged in LDS by the final
// select, and the most selection lists one row can have (4 per chunk).
constexpr int kSampleMax = 2048;
constexpr int kFinalStage = 8192;
constexpr int kMaxListsPerRow = 2048;

// Entries queued per (wave, head index) in the stream kernel before a flush.
constexpr int kQueueCap = 256;

// Gather: workgroups per launch we aim for, and the most per (b, query head).
#ifndef SAGA_GATHER_BLOCKS64
#define SAGA_GATHER_BLOCKS64 2048
#endif
#ifndef SAGA_GATHER_BLOCKS128
#define SAGA_GATHER_BLOCKS128 1536
#endif
constexpr int gather_target_blocks(int head_dim)
{
    return head_dim == 128 ? SAGA_GATHER_BLOCKS128 : SAGA_GATHER_BLOCKS64;
}
constexpr int kGatherMaxSegs = SAGA_GATHER_MAX_SEGS;
constexpr int kGatherStage = 1024;   // entries a gather workgroup stages per round

// Storage of selection list `local` (= chunk*4 + wave; nl lists per row) of
// row `head` (= b*h_q + i), at most capw = rows_per_chunk/4 entries: its first
// kListPrimary entries sit in a dense primary part at (head*nl + local) *
// kListPrimary + E, so one call's typical lists share a few tens of megabytes
// (few pages for the address translation); entries past those go to an
// overflow part sized for the worst case, head_stride entries per row
// starting at entry overflow_at (a row's chunks * rows_per_chunk never exceed
// head_stride).
constexpr int kListPrimary = 64;
__device__ __forceinline__ int64_t list_index(int64_t head, int64_t local, uint32_t E,
                                              int64_t capw, int64_t nl, int64_t head_stride,
                                              int64_t overflow_at)
{
    return E < (uint32_t)kListPrimary
               ? (head * nl + local) * kListPrimary + E
               : overflow_at + head * head_stride + local * capw + (E - kListPrimary);
}

// Paged caches.  Sequence b attends ctx_lens[b] rows; its logical row r sits
// in page block_table[b][r / P] of a pool laid out [num_pages][heads][P][d],
// at row r % P.  P is a multiple of kPageQuantum, so a pair of stream tiles, a
// 16-row sample block and a recompute tile never straddle two pages.  With
// block_table == nullptr the caches are contiguous [B][heads][cache_len][d]
// and every sequence attends the call's ctx rows.
constexpr int kPageQuantum = 256;
// Pools below this many bytes are read with 32-bit offsets; this offset (and
// any above it) reads zeros.
constexpr uint32_t kPoolLimit = 0xFFFFF000u;
struct PagedKV {
    const int32_t* block_table;   // [B][max_pages], nullptr: contiguous caches
    const int32_t* ctx_lens;      // [B]
    int32_t page_rows;            // P
    int32_t max_pages;
    int64_t num_pages;
    // Work split from the lengths (list path; plan_cap == 0: the host's rows).
    int32_t plan_cap;             // most chunks per sequence (the lists' chunks)
    int32_t plan_target;          // workgroups the batch's rows are spread over
    int64_t plan_quantum;         // rows per chunk: a multiple of this (a tile pair)
    int64_t plan_rows_max;        // and at most this
    int64_t plan_grid;            // K-stream workgroups: at least the call's work items
    int32_t* plan;                // workspace [1 + B]: rows per chunk, then each sequence's
                                  // chunks; written by the K stream for the kernels after it
};

// Rows attended by sequence b (ctx_lens[b] clamped to the table's capacity).
__device__ __forceinline__ int64_t seq_ctx(const PagedKV& pg, int b, int64_t ctx)
{
    if (!pg.block_table) return ctx;
    int64_t c = pg.ctx_lens[b];
    const int64_t cap = (int64_t)pg.max_pages * pg.page_rows;
    return c < 0 ? 0 : (c > cap ? cap : c);
}

// Length of sequence b as the work split of a paged call sees it: ctx_lens[b]
// clamped to the table and to the call's ctx (the bound the host planned
// with); 0 for b >= B.  Lengths and rows per chunk stay below 2^27.
__device__ __forceinline__ uint32_t plan_len(const PagedKV& pg, int b, int B, int64_t ctx)
{
    if (b >= B) return 0u;
    const int64_t c = seq_ctx(pg, b, ctx);
    return (uint32_t)(c < ctx ? c : ctx);
}

// Rows per chunk of a call on paged caches with per-sequence lengths, computed
// on the device from the lengths so that graph-captured calls follow them.
// Each sequence is cut into chunks of r rows (its last one shorter), h_k rows
// of chunks per sequence being the K stream's work items.  r is the smallest
// multiple of plan_quantum for which the items fit in plan_target workgroups
// (one round of resident streams on every CU), at most plan_rows_max (the
// list storage) and at least what keeps every sequence within plan_cap
// chunks.  The K stream computes it and stores it, with each sequence's chunk
// count, in PagedKV::plan for the gather and threshold kernels of the same
// call.  len0 = plan_len(threadIdx.x): thread t
// holds sequence t, so with B <= kBlock the search reads no memory.  All
// threads of the workgroup must call it (it synchronises); `red` is LDS for
// 8 int64 values followed by kBlock lengths (1088 bytes, 8-byte aligned).
__device__ __forceinline__ int64_t paged_rows_per_chunk(const PagedKV& pg, int B, int hk,
                                                        int64_t ctx, uint32_t len0, int64_t* red)
{
    uint32_t* lens = reinterpret_cast<uint32_t*>(red + 2 * kWavesPerBlock);
    lens[threadIdx.x] = len0;      // ordered before its reads by the barrier below
    int64_t sum = len0;
    uint32_t mx = len0;
    for (int b = threadIdx.x + kBlock; b < B; b += kBlock) {
        const uint32_t c = plan_len(pg, b, B, ctx);
        sum += c;
        mx = c > mx ? c : mx;
    }
    for (int off = kWave / 2; off > 0; off >>= 1) {
        sum += __shfl_xor(sum, off);
        const uint32_t o = __shfl_xor(mx, off);
        mx = o > mx ? o : mx;
    }
    if ((threadIdx.x & (kWave - 1)) == 0) {
        red[threadIdx.x / kWave] = sum;
        red[kWavesPerBlock + threadIdx.x / kWave] = mx;
    }
    __syncthreads();
    sum = 0;
    int64_t m = 0;
    for (int w = 0; w < kWavesPerBlock; ++w) {
        sum += red[w];
        m = red[kWavesPerBlock + w] > m ? red[kWavesPerBlock + w] : m;
    }
    __syncthreads();
    sum = wave_uniform(sum);       // the same in every lane: keep the search scalar
    m = wave_uniform(m);
    const int64_t q = pg.plan_quantum, target = pg.plan_target;
    auto up = [q](int64_t x) { return (x + q - 1) / q * q; };
    int64_t r = up(((int64_t)hk * sum + target - 1) / target);   // items >= h_k * sum / r
    r = r < pg.plan_rows_max ? r : pg.plan_rows_max;
    const int64_t need = up((m + pg.plan_cap - 1) / pg.plan_cap);   // chunks <= plan_cap
    r = r > need ? r : need;
    r = r > q ? r : q;
    // Work items for rows-per-chunk rr.
    auto items = [&](int64_t rr) {
        const uint32_t r32 = (uint32_t)rr;
        int64_t n = (len0 + r32 - 1) / r32;
        for (int b = threadIdx.x + kBlock; b < B; b += kBlock)
            n += (plan_len(pg, b, B, ctx) + r32 - 1) / r32;
        for (int off = kWave / 2; off > 0; off >>= 1) n += __shfl_xor(n, off);
        if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = n;
        __syncthreads();
        n = 0;
        for (int w = 0; w < kWavesPerBlock; ++w) n += red[w];
        __syncthreads();
        return wave_uniform(n) * hk;
    };
    // Rounding every sequence's last chunk up adds up to one item per (b, key
    // head): find the smallest r whose items fit.  r = up(longest) (one chunk
    // per sequence) is the most that can help; beyond plan_rows_max nothing
    // is allowed.  With every length in LDS, each thread tests one candidate
    // (r + t * plan_quantum) and the first that fits wins; otherwise, or past
    // those candidates, bisection.
    int64_t lo = r / q, hi = up(m) / q;              // in quanta
    hi = hi < pg.plan_rows_max / q ? hi : pg.plan_rows_max / q;
    if (hi <= lo) return r;
    bool bisect = true;
    if (B <= kBlock) {
        const int64_t cand = lo + threadIdx.x;
        bool ok = cand >= hi;
        if (!ok) {
            const uint32_t rc = (uint32_t)(cand * q);
            int64_t n = 0;
            for (int b = 0; b < B; ++b) n += (lens[b] + rc - 1) / rc;
            ok = n * hk <= target;
        }
        const uint64_t bal = __ballot(ok);
        if ((threadIdx.x & (kWave - 1)) == 0)
            red[threadIdx.x / kWave] = bal ? (threadIdx.x & ~(kWave - 1)) + __ffsll((unsigned long long)bal) - 1
                                           : kBlock;
        __syncthreads();
        int64_t first = kBlock;
        for (int w = 0; w < kWavesPerBlock; ++w) first = red[w] < first ? red[w] : first;
        __syncthreads();
        first = wave_uniform(first);
        if (first < kBlock) return (lo + first) * q;
        lo += kBlock - 1;                            // items(lo * q) > target
        bisect = hi > lo;
    } else {
        bisect = items(r) > target;
    }
    if (bisect) {
        while (hi - lo > 1) {                        // items(hi * q) is the best there is
            const int64_t mid = lo + (hi - lo) / 2;
            if (items(mid * q) > target) lo = mid; else hi = mid;
        }
        r = hi * q;
    }
    return r;
}

// The same plan computed by one wave on its own, for B <= kWave: lane l holds
// plan_len(l) in `len`; no LDS and no barrier (every wave of a workgroup
// gets the same result).  Candidates r + (base + lane) * plan_quantum are
// tested 64 at a time; the first that fits wins (the same r as the block
// version's search).
__device__ __forceinline__ int64_t readlane64(int64_t v, int l)
{
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, l);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)((uint64_t)v >> 32), l);
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ int64_t paged_rows_per_chunk_wave(const PagedKV& pg, int B, int hk,
                                                             uint32_t len)
{
    int64_t sum = len;
    uint32_t mx = len;
    for (int off = kWave / 2; off > 0; off >>= 1) {
        sum += __shfl_xor(sum, off);
        const uint32_t o = __shfl_xor(mx, off);
        mx = o > mx ? o : mx;
    }
    sum = wave_uniform(sum);
    const int64_t m = __builtin_amdgcn_readfirstlane(mx);
    const int64_t q = pg.plan_quantum, target = pg.plan_target;
    auto up = [q](int64_t x) { return (x + q - 1) / q * q; };
    int64_t r = up(((int64_t)hk * sum + target - 1) / target);
    r = r < pg.plan_rows_max ? r : pg.plan_rows_max;
    const int64_t need = up((m + pg.plan_cap - 1) / pg.plan_cap);
    r = r > need ? r : need;
    r = r > q ? r : q;
    const int64_t lo = r / q;
    int64_t hi = up(m) / q;
    hi = hi < pg.plan_rows_max / q ? hi : pg.plan_rows_max / q;
    if (hi <= lo) return r;
    const int lane = threadIdx.x & (kWave - 1);
    for (int64_t base = lo;; base += kWave) {     // ends: candidates >= hi always fit
        const int64_t cand = base + lane;
        bool ok = cand >= hi;
        if (!ok) {
            const uint32_t rc = (uint32_t)(cand * q);
            int64_t n = 0;
            for (int b = 0; b < B; ++b) {
                const uint32_t lb = __builtin_amdgcn_readlane(len, b);
                n += (lb + rc - 1) / rc;
            }
            ok = n * hk <= target;
        }
        const uint64_t bal = __ballot(ok);
        if (bal) return (base + __ffsll((unsigned long long)bal) - 1) * q;
    }
}

// paged_item for B <= kWave, one wave on its own (same inputs as
// paged_rows_per_chunk_wave).
__device__ __forceinline__ bool paged_item_wave(int hk, int64_t r, uint32_t len, int64_t item,
                                                int* b_out, int* g_out, int* chunk_out)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t n = (int64_t)((len + (uint32_t)r - 1) / (uint32_t)r) * hk;
    int64_t incl = n;
    for (int off = 1; off < kWave; off <<= 1) {
        const int64_t u = __shfl_up(incl, off);
        if (lane >= off) incl += u;
    }
    const int64_t lo = incl - n;
    const uint64_t bal = __ballot(n > 0 && item >= lo && item < lo + n);
    if (!bal) return false;
    const int lb = __ffsll((unsigned long long)bal) - 1;
    const int64_t off = item - readlane64(lo, lb);
    const int64_t nb = readlane64(n, lb) / hk;
    *b_out = lb;
    *g_out = (int)(off / nb);
    *chunk_out = (int)(off - off / nb * nb);
    return true;
}

// Chunks of sequence b for rows-per-chunk r (0 for an empty sequence).
__device__ __forceinline__ int64_t paged_chunks(const PagedKV& pg, int b, int64_t ctx, int64_t r)
{
    int64_t c = seq_ctx(pg, b, ctx);
    c = c < ctx ? c : ctx;
    return wave_uniform((c + r - 1) / r);
}

// The K stream of such a call is a 1-D launch of plan_grid workgroups over
// its work items: sequence by sequence, h_k key heads of paged_chunks(b)
// chunks each, chunk fastest.  Item `item` -> (b, g, chunk); false when the
// call has fewer items.  Consecutive workgroups take consecutive items, so the
// live ones are spread over the XCDs (which take workgroups round-robin) and
// the few idle ones sit at the end of the grid.  Block-wide, same calling
// rules and len0 as paged_rows_per_chunk; `red` is LDS for 8 values.
__device__ __forceinline__ bool paged_item(const PagedKV& pg, int B, int hk, int64_t ctx,
                                           int64_t r, uint32_t len0, int64_t item, int64_t* red,
                                           int* b_out, int* g_out, int* chunk_out)
{
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    int64_t base = 0;                           // items of the sequences before this pass
    bool found = false;
    for (int b0 = 0; b0 < B && !found; b0 += kBlock) {
        const int b = b0 + threadIdx.x;        // one sequence per thread (not wave-uniform)
        const uint32_t c = b0 == 0 ? len0 : plan_len(pg, b, B, ctx);
        const int64_t n = (int64_t)((c + (uint32_t)r - 1) / (uint32_t)r) * hk;
        int64_t incl = n;                       // inclusive scan over the block
        for (int off = 1; off < kWave; off <<= 1) {
            const int64_t u = __shfl_up(incl, off);
            if (lane >= off) incl += u;
        }
        if (lane == kWave - 1) red[w] = incl;
        if (threadIdx.x == 0) red[kWavesPerBlock] = -1;
        __syncthreads();
        int64_t total = 0;
        for (int k = 0; k < kWavesPerBlock; ++k) {
            incl += k < w ? red[k] : 0;
            total += red[k];
        }
        const int64_t lo = base + incl - n;
        if (n > 0 && item >= lo && item < lo + n) {
            red[kWavesPerBlock] = b;
            red[kWavesPerBlock + 1] = item - lo;
        }
        __syncthreads();
        found = red[kWavesPerBlock] >= 0;
        base += total;
        const int bf = (int)red[kWavesPerBlock];
        const int64_t off = red[kWavesPerBlock + 1];
        __syncthreads();                        // red is rewritten by the next pass
        if (found) {
            const int64_t nb = paged_chunks(pg, bf, ctx, r);
            *b_out = __builtin_amdgcn_readfirstlane(bf);
            *g_out = __builtin_amdgcn_readfirstlane((int)(off / nb));
            *chunk_out = __builtin_amdgcn_readfirstlane((int)(off - off / nb * nb));
        }
    }
    return found;
}

// Several query tokens per step (lq > 1): token j of query head i is the
// virtual query head i*lq + j (same key and value heads as i), and it attends
// the rows up to its own position, ctx - (lq - 1 - j), where ctx counts the
// step's tokens.  Rows attended by virtual head v of sequence b:
__device__ __forceinline__ int64_t head_ctx(const PagedKV& pg, int lq, int b, int v, int64_t ctx)
{
    return seq_ctx(pg, b, ctx) - (lq - 1 - v % lq);
}

// Element offset of the first row of the page that holds row r of (b, head h)
// in a pool with nh heads per page, or -1 when the table points outside the
// pool (the caller then reads nothing).
template <int D>
__device__ __forceinline__ int64_t page_base(const PagedKV& pg, int b, int h, int nh, int64_t r)
{
    const int64_t p = r / pg.page_rows;
    if (p >= pg.max_pages) return -1;
    const int32_t page = pg.block_table[(int64_t)b * pg.max_pages + p];
    if (page < 0 || page >= pg.num_pages) return -1;
    return (((int64_t)page * nh + h) * pg.page_rows) * D;
}

// Stream-select kernel: K stream, threshold mask, compaction into lists.
// List (b*h_q + i, chunk, wave) holds up to rows_per_chunk/4 entries
// (row - chunk_start, logit bits) at entries[list_index(list, ...)].
struct SelectStreamArgs {
    const uint16_t* q;
    const uint16_t* k;
    const float* tau;
    uint32_t* bitmap;        // nullable
    int64_t bitmap_words;    // words per (b, i) row of the bitmap
    uint2* entries;          // list storage (see list_index)
    int64_t overflow_at;
    int64_t head_stride;     // overflow entries per row (see list_index)
    int32_t* list_count;     // [B*hq][chunks][4]
    float* list_max;         // [B*hq][chunks][4]  largest selected logit (-inf if none)
    float* logits_out;       // nullable [B*hq][ctx]: every logit, for checking
    const uint32_t* group_flags;  // nullable [B*hk]: run only key groups flagged non-zero
    int32_t B, hq, hk, Gk;
    int64_t ctx, cache_len, rows_per_chunk;
    int32_t chunks;
    float scale;
    int32_t lq;              // query tokens per query head and step (1: one)
    const float* k_scale;    // non-null: fp8 e4m3 K, one scale per (b, key head)
    PagedKV pg;              // paged caches (block_table != nullptr)
    // Value gather in the stream's tail (v non-null; contiguous V, bf16 or fp8
    // with v_scale, d_v = d_k of 64 or 128): each workgroup gathers its own
    // chunk's selected value rows and writes one partial per (b*h_q + i, chunk)
    // instead of list lengths.
    const uint16_t* v;
    Partials part;
    int32_t hv, Gv;
    const float* v_scale;    // non-null: fp8 e4m3 V (d bytes per row), one scale per (b, value head)
};

// Gather kernel: softmax weights and the sparse value gather over the lists.
struct GatherArgs {
    const uint16_t* v;
    const uint2* entries;
    int64_t overflow_at;
    int64_t head_stride;     // overflow entries per row (see list_index)
    const int32_t* list_count;
    const float* list_max;
    const float* tau_filter; // nullable [B*hq]: keep only entries with logit >= tau_filter
    const float* v_scale;    // non-null: fp8 e4m3 V (d_v bytes per row), one scale per (b, value head)
    Partials part;           // one partial per (b*h_q + i, segment)
    uint32_t pool_bytes;     // paged: V pool bytes when below kPoolLimit (32-bit offsets), else 0
    int32_t B, hq, hk, hv, Gv;
    int64_t ctx, cache_len, rows_per_chunk;
    int32_t chunks, segs;    // segs: equal entry ranges per (b, query head)
    PagedKV pg;              // paged caches (block_table != nullptr)
};

// Refresh steps 1-2: sampled logits and the per-row pivot.
struct SampleArgs {
    const uint16_t* q;
    const uint16_t* k;
    float* sample;           // [B*hq][kSampleMax]
    float* pivot;            // [B*hq]
    uint32_t* group_flags;   // nullable [B*hk]: cleared here
    int32_t B, hq, hk, Gk;
    int64_t ctx;                 // rows attended (tokens > 1: by the last token)
    int64_t cache_len, stride;   // one 16-row sample block every `stride` rows
    int32_t m, rank;             // sample size, rank of the pivot within the sample
    int32_t top_n;               // paged: per-row rank from each sequence's length
    float scale;
    int32_t lq;              // query tokens per query head and step (1: one)
    const float* k_scale;    // non-null: fp8 e4m3 K, one scale per (b, key head)
    PagedKV pg;              // paged caches (block_table != nullptr)
};

// Refresh step 4: exact N-th largest from the candidate lists.
struct FinalArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint2* entries;
    int64_t overflow_at;
    int64_t head_stride;     // overflow entries per row (see list_index)
    const int32_t* list_count;
    float* tau;              // [B*hq] out
    uint32_t* group_flags;   // nullable [B*hk]: set when a row of the group used the recompute path
    int32_t B, hq, hk, Gk;
    int64_t ctx, cache_len, rows_per_chunk;
    int32_t chunks;
    uint32_t top_n;
    float scale;
    int32_t lq;              // query tokens per query head and step (1: one)
    const float* k_scale;    // non-null: fp8 e4m3 K, one scale per (b, key head)
    PagedKV pg;              // paged caches (block_table != nullptr)
};

struct FullArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    Partials part;
    int32_t B, hq, hk, hv, Gk, Gv, nv;
    int64_t ctx, cache_len, rows_per_chunk;
    int32_t chunks;
    float scale;
    size_t wave_lds;
};

// Small-batch path (fused.hip): K stream, mask, compaction and value gather
// in one kernel; one partial per (b*h_q + i, chunk).  The selected entries of
// a chunk stay in LDS: one queue per (wave, head slot) of scap 8-byte entries,
// enough for every row of the wave's share of the chunk (rows_per_chunk / 4).
struct FusedArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const float* tau;
    uint32_t* bitmap;        // nullable
    int64_t bitmap_words;
    float* logits_out;       // nullable [B*hq][ctx]
    Partials part;           // [B*hq][chunks]
    int32_t B, hq, hk, hv, Gk, Gv;
    int64_t ctx, cache_len, rows_per_chunk;
    int32_t chunks;
    int32_t scap;            // entries per (wave, head slot) queue
    int32_t unroll;          // 16-row groups per wave tile: 1 or 2
    float scale;
    int32_t lq;
    const float* k_scale;    // non-null: fp8 e4m3 K
    PagedKV pg;
};

hipError_t launch_select_gather(int D, int DV, const FusedArgs& a, size_t lds_bytes,
                                hipStream_t s);
hipError_t launch_combine_parts(int D, const Partials& p, int rows, int parts, uint16_t* out,
                                int32_t* counts, hipStream_t s);
hipError_t launch_select_stream(int D, const SelectStreamArgs& a, hipStream_t s);
hipError_t launch_gather(int D, const GatherArgs& a, hipStream_t s);
hipError_t launch_combine(int D, const Partials& p, int rows, int parts, uint16_t* out,
                          int32_t* counts, hipStream_t s);
hipError_t launch_sample(int D, const SampleArgs& a, hipStream_t s);
hipError_t launch_refresh_final(int D, const FinalArgs& a, hipStream_t s);
hipError_t launch_full(int DK, int DV, int maxs, const FullArgs& a, hipStream_t s);
hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s);

}  // namespace saga

// Host entry points of api.hip used by the other source files (not exported).
struct saga_dims;
namespace saga {
// Workspace bytes of a decode step for dims (0 if the dims are invalid).
size_t decode_workspace_bytes(const saga_dims* dims);
// saga_decode_step without the selection bitmap.
int decode_step(const saga_dims* dims, const void* q_dev, const void* k_dev, const void* v_dev,
                const float* thresholds_dev, void* out_dev, int32_t* sel_counts_dev,
                void* workspace_dev, size_t workspace_bytes, void* stream);
}  // namespace saga

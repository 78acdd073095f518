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

// Storage of selection list lid = (b*h_q + i) * nl + chunk*4 + wave (nl lists
// per row in this call, capw = rows_per_chunk/4 entries at most): its first
// kListPrimary entries sit in a dense primary part at lid * kListPrimary + E,
// so one call's typical lists share a few tens of megabytes (few pages for the
// address translation); entries past those go to an overflow part sized for
// the worst case, which starts at entry overflow_at.
constexpr int kListPrimary = 64;
__device__ __forceinline__ int64_t list_index(int64_t lid, uint32_t E, int64_t capw,
                                              int64_t overflow_at)
{
    return E < (uint32_t)kListPrimary ? lid * kListPrimary + E
                                      : overflow_at + lid * capw + (E - kListPrimary);
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
};

// Rows attended by sequence b (ctx_lens[b] clamped to the table's capacity).
__device__ __forceinline__ int64_t seq_ctx(const PagedKV& pg, int b, int64_t ctx)
{
    if (!pg.block_table) return ctx;
    int64_t c = pg.ctx_lens[b];
    const int64_t cap = (int64_t)pg.max_pages * pg.page_rows;
    return c < 0 ? 0 : (c > cap ? cap : c);
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
};

// Gather kernel: softmax weights and the sparse value gather over the lists.
struct GatherArgs {
    const uint16_t* v;
    const uint2* entries;
    int64_t overflow_at;
    const int32_t* list_count;
    const float* list_max;
    const float* tau_filter; // nullable [B*hq]: keep only entries with logit >= tau_filter
    const float* v_scale;    // non-null: fp8 e4m3 V (d_v bytes per row), one scale per (b, value head)
    Partials part;           // one partial per (b*h_q + i, segment)
    uint32_t pool_bytes;     // paged: V pool bytes when below kPoolLimit (32-bit offsets), else 0
    int32_t B, hq, hv, Gv;
    int64_t cache_len, rows_per_chunk;
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
// a chunk stay in LDS: qcap entries per (wave, queue), enough for every row
// of the wave's share of the chunk for the ceil(G_k/4) head slots of a queue,
// then G_k lists of hcap 16-bit entry indices, one per head slot.
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
    int32_t chunks, qcap;
    int32_t hcap;            // entries per head slot list (rows_per_chunk)
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

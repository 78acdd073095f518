// kernels.hpp -- internal interface between the C-ABI host code (api.hip) and
// the kernel files.  Nothing here is exported from libsaga.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "device.hpp"

namespace saga {

// Rows of one workgroup tile (4 waves x 16*U rows) per kernel family and
// head_dim; chunk lengths are multiples of these.
constexpr int decode_unroll(int D) { return D == 64 ? 8 : 4; }
constexpr int decode_block_rows(int D) { return kWavesPerBlock * 16 * decode_unroll(D); }
constexpr int full_unroll(int D) { return D == 64 ? 4 : 2; }

// Entry-queue capacity (entries per wave) of the sparse decode kernel.
constexpr int kQueueCap = 256;

// LDS bytes of one wave in the sparse decode kernel:
//   queue keys + logits, o[R][Gk][D], l[R][16], m_cur[16], m_new[16], count[16]
inline __host__ __device__ size_t decode_wave_lds_bytes(int D, int Gk)
{
    const int R = 128 / D;
    size_t b = (size_t)kQueueCap * 8 + (size_t)R * Gk * D * 4 + (size_t)R * 16 * 4 + 3 * 16 * 4;
    return (b + 15) & ~(size_t)15;
}
constexpr size_t kDecodeLdsHeader = 128;   // 16 value-head offsets (int64)

// LDS bytes of one wave in the full-attention kernel:
//   P[TR][16] fp32, alpha[16], m[16], l[16], o[MAXS][D]
inline __host__ __device__ size_t full_wave_lds_bytes(int D, int maxs)
{
    const int TR = 16 * full_unroll(D);
    size_t b = (size_t)TR * 16 * 4 + 3 * 16 * 4 + (size_t)maxs * D * 4;
    return (b + 15) & ~(size_t)15;
}

// Radix select geometry: 12 + 10 + 10 bits of the order-preserving key.
constexpr int kHistBins = 4096;
constexpr int kSelectSeg = 16384;          // logits per workgroup in the select passes

struct DecodeArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const float* tau;
    uint32_t* bitmap;        // nullable
    int64_t bitmap_words;    // words per (b, i) row of the bitmap
    Partials part;
    int32_t B, hq, hk, hv, Gk, Gv;
    int64_t ctx, cache_len, rows_per_chunk;
    int32_t chunks;
    float scale;
    size_t wave_lds;         // decode_wave_lds_bytes(D, Gk)
};

struct LogitsArgs {
    const uint16_t* q;
    const uint16_t* k;
    float* logits;           // [B*hq][ld]
    float* debug;            // nullable [B*hq][ctx]
    int64_t ld;
    int32_t B, hq, hk, Gk;
    int64_t ctx, cache_len, rows_per_chunk;
    float scale;
    // per-row select state cleared by the chunk-0 workgroups
    uint32_t* ghist;         // [B*hq][kHistBins]
    uint32_t* done;          // [B*hq]
    uint32_t* cand_count;    // [B*hq]
};

struct SelectArgs {
    const float* logits;     // [rows][ld]
    int64_t ld, ctx;
    int32_t rows, segs;
    uint32_t top_n;
    uint32_t* ghist;         // [rows][kHistBins]
    uint32_t* done;          // [rows]
    uint32_t* state;         // [rows][4]: bucket, rank within bucket, bucket size
    uint32_t* cand;          // [rows][ld]
    uint32_t* cand_count;    // [rows]
    float* tau;              // [rows]
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

hipError_t launch_sparse_decode(int D, const DecodeArgs& a, hipStream_t s);
hipError_t launch_combine(int D, const Partials& p, int rows, int chunks, uint16_t* out,
                          int32_t* counts, hipStream_t s);
hipError_t launch_qk_logits(int D, const LogitsArgs& a, int chunks, hipStream_t s);
hipError_t launch_select(const SelectArgs& a, hipStream_t s);
hipError_t launch_full(int D, int maxs, const FullArgs& a, hipStream_t s);
hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s);

}  // namespace saga

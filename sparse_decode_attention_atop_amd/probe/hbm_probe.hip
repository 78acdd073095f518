// hbm_probe.hip -- HBM measurement kernels (libsaga_probe.so; C ABI in
// include/saga_probe.h).  They calibrate the decode library's roofline: each
// reproduces one access pattern of the decode step with nothing else in the
// kernel, so its rate is what this GPU sustains for that pattern.
//
//   read_kernel   contiguous chunks, one per workgroup, 16-byte loads through a
//                 buffer resource, two batches of DEPTH loads per lane in
//                 flight (the K stream's pattern: every key row read once);
//   tiles_kernel  the same chunks read in the K stream's own lane mapping:
//                 each wave reads 16-row tiles of RB-byte rows, lane l loading
//                 16 bytes of row l % 16 at bytes 16 * (l / 16) + 64 m (an MFMA
//                 operand's layout: one load instruction covers 16 rows x 64
//                 bytes, half of each 128-byte line), TILES tiles per wave in
//                 each of two batches in flight;
//   rows_kernel   rows of RB bytes at pseudo-random places in the buffer,
//                 RB/16 lanes per row, DEPTH rows in flight per lane (the
//                 sparse value gather's pattern).
// Row k of a launch is hash(seed, k) mod rows, with the "lowbias32" 32-bit
// integer hash of C. Wellons (hash-prospector): two xor-shift-multiply
// rounds and a final xor-shift.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "saga_probe.h"

#define PROBE_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 256;

__device__ __forceinline__ uint32_t lowbias32(uint32_t x)
{
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

// XOR of one word per thread over the workgroup, written by thread 0.
__device__ __forceinline__ void fold_to_sink(u32x4 acc, uint32_t* sink)
{
    __shared__ uint32_t part[kBlock / 64];
    uint32_t v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    for (int off = 32; off > 0; off >>= 1) v ^= __shfl_xor(v, off);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

__device__ __forceinline__ u32x4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// Workgroup w reads bytes [w * chunk, (w + 1) * chunk).  Loads past the chunk
// (the last prefetch) read zero through the buffer resource without touching
// memory, so every prefetch is unconditional.
template <int DEPTH>
__global__ __launch_bounds__(kBlock) void read_kernel(const unsigned char* buf, uint32_t chunk,
                                                      uint32_t* sink)
{
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char*>(buf + (uint64_t)blockIdx.x * chunk), (short)0, (int)chunk,
        0x00020000);
    constexpr uint32_t kSlot = kBlock * 16;              // bytes of one load across the block
    constexpr uint32_t kBatch = kSlot * DEPTH;
    u32x4 acc = {0u, 0u, 0u, 0u};
    u32x4 a[DEPTH], b[DEPTH];
    uint32_t off = threadIdx.x * 16u;
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) a[d] = buf_ld16(r, off + d * kSlot);
    for (uint32_t base = 0; base < chunk; base += 2 * kBatch) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) b[d] = buf_ld16(r, off + kBatch + d * kSlot);
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) acc ^= a[d];
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) a[d] = buf_ld16(r, off + 2 * kBatch + d * kSlot);
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) acc ^= b[d];
        off += 2 * kBatch;
    }
    fold_to_sink(acc, sink);
}

// Workgroup w reads bytes [w * chunk, (w + 1) * chunk) as 16-row tiles: wave
// v takes tiles v, v + 4, ..., M = RB / 64 loads per lane and tile.
template <int RB, int TILES>
__global__ __launch_bounds__(kBlock) void tiles_kernel(const unsigned char* buf, uint32_t chunk,
                                                       uint32_t* sink)
{
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char*>(buf + (uint64_t)blockIdx.x * chunk), (short)0, (int)chunk,
        0x00020000);
    constexpr int M = RB / 64;
    constexpr uint32_t kTile = 16 * RB;                  // one wave's tile
    constexpr uint32_t kStep = 4 * kTile;                // one tile per wave
    constexpr uint32_t kBatch = TILES * kStep;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    u32x4 acc = {0u, 0u, 0u, 0u};
    u32x4 a[TILES][M], b[TILES][M];
    uint32_t off = w * kTile + (lane & 15) * RB + (lane >> 4) * 16;
#pragma unroll
    for (int t = 0; t < TILES; ++t)
#pragma unroll
        for (int m = 0; m < M; ++m) a[t][m] = buf_ld16(r, off + t * kStep + 64 * m);
    for (uint32_t base = 0; base < chunk; base += 2 * kBatch) {
#pragma unroll
        for (int t = 0; t < TILES; ++t)
#pragma unroll
            for (int m = 0; m < M; ++m) b[t][m] = buf_ld16(r, off + kBatch + t * kStep + 64 * m);
#pragma unroll
        for (int t = 0; t < TILES; ++t)
#pragma unroll
            for (int m = 0; m < M; ++m) acc ^= a[t][m];
#pragma unroll
        for (int t = 0; t < TILES; ++t)
#pragma unroll
            for (int m = 0; m < M; ++m) a[t][m] = buf_ld16(r, off + 2 * kBatch + t * kStep + 64 * m);
#pragma unroll
        for (int t = 0; t < TILES; ++t)
#pragma unroll
            for (int m = 0; m < M; ++m) acc ^= b[t][m];
        off += 2 * kBatch;
    }
    fold_to_sink(acc, sink);
}

// Rows k = first .. first + per - 1 of the launch for workgroup w; lane group
// `slot` (RB/16 lanes) reads rows first + slot, first + slot + SLOTS, ...
template <int RB, int DEPTH>
__global__ __launch_bounds__(kBlock) void rows_kernel(const unsigned char* buf, uint32_t nrows,
                                                      uint64_t rows, uint32_t seed, uint32_t* sink)
{
    constexpr int LPR = RB / 16;                // lanes per row
    constexpr int SLOTS = kBlock / LPR;         // rows per load instruction of the workgroup
    const int slot = threadIdx.x / LPR, lc = threadIdx.x - slot * LPR;
    const uint64_t per = (rows + gridDim.x - 1) / gridDim.x;
    const uint64_t k_begin = (uint64_t)blockIdx.x * per;
    const uint64_t k_end = k_begin + per < rows ? k_begin + per : rows;
    const uint32_t mix = seed * 0x9e3779b9u;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (uint64_t k0 = k_begin + slot; k0 < k_end; k0 += (uint64_t)SLOTS * DEPTH) {
        u32x4 v[DEPTH];
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            const uint64_t k = k0 + (uint64_t)d * SLOTS;
            const uint32_t row = lowbias32((uint32_t)k ^ mix) % nrows;
            // Always a row of the buffer, so the load needs no branch; rows
            // past this workgroup's share are read and then dropped.
            const u32x4 x = *reinterpret_cast<const u32x4*>(buf + (uint64_t)row * RB + 16 * lc);
            v[d] = k < k_end ? x : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) acc ^= v[d];
    }
    fold_to_sink(acc, sink);
}

bool aligned256(const void* p) { return ((uintptr_t)p & 255u) == 0; }

}  // namespace

PROBE_EXPORT int saga_probe_read(const void* buf_dev, size_t bytes, int32_t workgroups,
                                 int32_t depth, uint32_t* sink_dev, void* stream)
{
    if (!buf_dev || !sink_dev || !aligned256(buf_dev) || ((uintptr_t)sink_dev & 3u))
        return 1;
    if (workgroups < 1 || workgroups > 65535 || bytes == 0 || bytes >= (size_t(1) << 40))
        return 1;
    if (bytes % ((size_t)workgroups * 4096) != 0) return 1;
    const size_t chunk = bytes / workgroups;
    if (chunk >= (size_t(1) << 31)) return 1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const unsigned char* b = static_cast<const unsigned char*>(buf_dev);
    const dim3 grid((unsigned)workgroups);
    switch (depth) {
    case 1: hipLaunchKernelGGL(read_kernel<1>, grid, dim3(kBlock), 0, s, b, (uint32_t)chunk, sink_dev); break;
    case 2: hipLaunchKernelGGL(read_kernel<2>, grid, dim3(kBlock), 0, s, b, (uint32_t)chunk, sink_dev); break;
    case 4: hipLaunchKernelGGL(read_kernel<4>, grid, dim3(kBlock), 0, s, b, (uint32_t)chunk, sink_dev); break;
    case 8: hipLaunchKernelGGL(read_kernel<8>, grid, dim3(kBlock), 0, s, b, (uint32_t)chunk, sink_dev); break;
    default: return 1;
    }
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

PROBE_EXPORT int saga_probe_read_tiles(const void* buf_dev, size_t bytes, int32_t row_bytes,
                                       int32_t workgroups, int32_t tiles, uint32_t* sink_dev,
                                       void* stream)
{
    if (!buf_dev || !sink_dev || !aligned256(buf_dev) || ((uintptr_t)sink_dev & 3u))
        return 1;
    if (row_bytes != 128 && row_bytes != 256) return 1;
    if (tiles != 1 && tiles != 2) return 1;
    if (workgroups < 1 || workgroups > 65535 || bytes == 0 || bytes >= (size_t(1) << 40))
        return 1;
    if (bytes % ((size_t)workgroups * 16384) != 0) return 1;
    const size_t chunk = bytes / workgroups;
    if (chunk >= (size_t(1) << 31)) return 1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const unsigned char* b = static_cast<const unsigned char*>(buf_dev);
    const dim3 grid((unsigned)workgroups);
    const uint32_t c = (uint32_t)chunk;
    if (row_bytes == 128) {
        if (tiles == 1) hipLaunchKernelGGL((tiles_kernel<128, 1>), grid, dim3(kBlock), 0, s, b, c, sink_dev);
        else hipLaunchKernelGGL((tiles_kernel<128, 2>), grid, dim3(kBlock), 0, s, b, c, sink_dev);
    } else {
        if (tiles == 1) hipLaunchKernelGGL((tiles_kernel<256, 1>), grid, dim3(kBlock), 0, s, b, c, sink_dev);
        else hipLaunchKernelGGL((tiles_kernel<256, 2>), grid, dim3(kBlock), 0, s, b, c, sink_dev);
    }
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

PROBE_EXPORT int saga_probe_rows(const void* buf_dev, size_t buf_bytes, int32_t row_bytes,
                                 int64_t rows, uint32_t seed, int32_t workgroups, int32_t depth,
                                 uint32_t* sink_dev, void* stream)
{
    if (!buf_dev || !sink_dev || !aligned256(buf_dev) || ((uintptr_t)sink_dev & 3u))
        return 1;
    if (row_bytes != 64 && row_bytes != 128 && row_bytes != 256) return 1;
    if (buf_bytes == 0 || buf_bytes >= (size_t(1) << 40) || buf_bytes % row_bytes != 0) return 1;
    const size_t nrows = buf_bytes / row_bytes;
    if (nrows >= (size_t(1) << 32)) return 1;
    if (rows < 1 || workgroups < 1 || workgroups > (1 << 20)) return 1;
    if (depth != 1 && depth != 2 && depth != 4 && depth != 8) return 1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const unsigned char* b = static_cast<const unsigned char*>(buf_dev);
    const dim3 grid((unsigned)workgroups);
    const uint32_t n = (uint32_t)nrows;
#define PROBE_ROWS(RB, DP) \
    hipLaunchKernelGGL((rows_kernel<RB, DP>), grid, dim3(kBlock), 0, s, b, n, (uint64_t)rows, seed, sink_dev)
#define PROBE_ROWS_RB(RB)                                      \
    switch (depth) {                                           \
    case 1: PROBE_ROWS(RB, 1); break;                          \
    case 2: PROBE_ROWS(RB, 2); break;                          \
    case 4: PROBE_ROWS(RB, 4); break;                          \
    default: PROBE_ROWS(RB, 8); break;                         \
    }
    if (row_bytes == 64) { PROBE_ROWS_RB(64) }
    else if (row_bytes == 128) { PROBE_ROWS_RB(128) }
    else { PROBE_ROWS_RB(256) }
#undef PROBE_ROWS_RB
#undef PROBE_ROWS
    return hipGetLastError() == hipSuccess ? 0 : 4;
}

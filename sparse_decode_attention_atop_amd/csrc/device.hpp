// device.hpp -- gfx950 device helpers shared by the SAGA / Atop-N kernels.
//
// The one piece of arithmetic that every kernel must do identically is the
// QK tile (qk_tile below): the threshold refresh ranks the logits it produces
// and the decode step compares the logits it produces against that rank, so
// both must be the same fp32 values bit for bit.  Both call this one routine,
// which fixes the MFMA sequence and the accumulation order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tuning.hpp"

namespace saga {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kBlock = 256;            // 4 waves per workgroup
constexpr int kWavesPerBlock = kBlock / kWave;

// ------------------------------------------------------------ conversions
__device__ __forceinline__ float bf16lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16hi(uint32_t packed) { return __uint_as_float(packed & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest, ties to even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Order-preserving map of fp32 bit patterns to unsigned keys: a > b as floats
// iff key(a) > key(b).  -0.0 is first folded onto +0.0 so that the key order
// and the float comparison agree on zeros.
__device__ __forceinline__ uint32_t float_key(float f)
{
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k)
{
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// ------------------------------------------------------------ memory
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
// Streaming load for data read exactly once per call (the K cache).
__device__ __forceinline__ u32x4 ld16_stream(const void* p)
{
#if SAGA_K_NONTEMPORAL
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#else
    return *reinterpret_cast<const u32x4*>(p);
#endif
}

// Raw buffer resources (gfx9 family, word 3 = 0x00020000): 32-bit offsets from
// an SGPR base, and loads past `bytes` return zero instead of touching memory.
constexpr int kBufferWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             kBufferWord3);
}
__device__ __forceinline__ u32x4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// s_waitcnt immediate (gfx9 encoding) that waits for vmcnt = 0 only:
// vmcnt bits [3:0] and [15:14] zero, expcnt [6:4] = 7, lgkmcnt [11:8] = 15.
constexpr int kWaitVmcnt0 = 0x0F70;

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
// Eight fp8 e4m3 (OCP: bias 7, max 448, no infinities) values, in byte order,
// widened to eight bf16 (exact: 3 mantissa bits fit bf16's 7).
__device__ __forceinline__ u32x4 fp8x8_to_bf16x8(u32x2 x)
{
    u32x4 r;
    r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[0], 1.0f, false));
    r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[0], 1.0f, true));
    r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[1], 1.0f, false));
    r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[1], 1.0f, true));
    return r;
}

// ------------------------------------------------------------ wave utilities
// Orders LDS traffic between lanes of one wave (no workgroup barrier).
__device__ __forceinline__ void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// A value the caller knows is the same in every lane, moved to scalar
// registers so that branches on it stay scalar.
__device__ __forceinline__ int64_t wave_uniform(int64_t v)
{
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Number of set bits of `mask` in lanes below this one.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Block-wide (256 threads) reductions and scan.  `red` holds one value per wave.
__device__ __forceinline__ float block_max(float v, float* red)
{
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    if (lane_id() == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    v = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    return v;
}

__device__ __forceinline__ int32_t block_sum(int32_t v, int32_t* red)
{
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    if (lane_id() == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    v = red[0] + red[1] + red[2] + red[3];
    __syncthreads();
    return v;
}

// Inclusive prefix sum over the block in thread order.
__device__ __forceinline__ int32_t block_scan(int32_t v, int32_t* red)
{
    const int lane = lane_id();
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int32_t u = __shfl_up(v, off);
        if (lane >= off) v += u;
    }
    if (lane == kWave - 1) red[threadIdx.x >> 6] = v;
    __syncthreads();
    const int w = threadIdx.x >> 6;
    int32_t add = 0;
#pragma unroll
    for (int k = 0; k < kWavesPerBlock - 1; ++k) add += k < w ? red[k] : 0;
    __syncthreads();
    return v + add;
}

// Max / sum over the 16 lanes that share lane>>4 (one MFMA row group).
__device__ __forceinline__ float group16_max(float v)
{
    v = fmaxf(v, __shfl_xor(v, 1));
    v = fmaxf(v, __shfl_xor(v, 2));
    v = fmaxf(v, __shfl_xor(v, 4));
    v = fmaxf(v, __shfl_xor(v, 8));
    return v;
}
__device__ __forceinline__ float group16_sum(float v)
{
    v += __shfl_xor(v, 1);
    v += __shfl_xor(v, 2);
    v += __shfl_xor(v, 4);
    v += __shfl_xor(v, 8);
    return v;
}

// ------------------------------------------------------------ the QK tile
//
// One wave computes logits for 16*U consecutive cache rows and up to 16 query
// heads of one key-head group with v_mfma_f32_16x16x32_bf16:
//   A (16 x 32)  = query heads x a 32-wide slab of head_dim   (q fragment)
//   B (32 x 16)  = the same slab x 16 cache rows               (K fragment)
//   D (16 x 16)  = logits[head][row]
// Lane l supplies A row l%16 / B column l%16 with the 8 slab elements
// 8*(l/16) .. 8*(l/16)+7, i.e. one 16-byte load per lane per slab; the 64
// lanes of one load instruction cover 16 rows x 64 contiguous bytes.
// Lane l receives D[4*(l/16)+i][l%16], i = 0..3: the logits of row l%16 for
// the head slots 4*(l/16)+i.
template <int D>
struct QFrag {
    u32x4 v[D / 32];
};

// q_head: row of query head slot (lane%16) or nullptr for an unused slot.
template <int D>
__device__ __forceinline__ QFrag<D> load_qfrag(const uint16_t* q_head)
{
    QFrag<D> f;
    const int grp = lane_id() >> 4;
#pragma unroll
    for (int m = 0; m < D / 32; ++m) {
        if (q_head) f.v[m] = ld16(q_head + 32 * m + 8 * grp);
        else f.v[m] = u32x4{0u, 0u, 0u, 0u};
    }
    return f;
}

// Rows row0 + 16u + (lane%16) for u < U; rows at or past `row_end` are read
// from row_end-1 instead (always a valid row) and must be masked by the caller.
template <int D, int U>
struct KTile {
    u32x4 v[U][D / 32];
};

template <int D, int U>
__device__ __forceinline__ void load_ktile(KTile<D, U>& t, const uint16_t* k_head, int64_t row0,
                                           int64_t row_end)
{
    const int col = lane_id() & 15, grp = lane_id() >> 4;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        int64_t r = row0 + 16 * u + col;
        r = r < row_end ? r : row_end - 1;
        const uint16_t* p = k_head + r * D + 8 * grp;
#pragma unroll
        for (int m = 0; m < D / 32; ++m) t.v[u][m] = ld16_stream(p + 32 * m);
    }
}

// Logits of one 16-row group: s[i] = scale * sum_c q[slot 4*(lane/16)+i][c] *
// K[row lane%16][c].  Every kernel that produces logits goes through here.
template <int D>
__device__ __forceinline__ void qk_group(const QFrag<D>& qf, const u32x4 (&kv)[D / 32], float scale,
                                         float (&s)[4])
{
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < D / 32; ++m)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, qf.v[m]), __builtin_bit_cast(bf16x8, kv[m]), acc, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = acc[i] * scale;
}

// Same tile through a buffer resource over one key head's first `rows` rows:
// row indices past the resource read as zero rows (the caller masks them).
// Offsets are 32-bit: a key head must be smaller than 2 GiB.
template <int D, int U>
__device__ __forceinline__ void load_ktile_buf(KTile<D, U>& t, __amdgpu_buffer_rsrc_t k_head,
                                               uint32_t row0)
{
    const int col = lane_id() & 15, grp = lane_id() >> 4;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t off = (row0 + 16 * u + col) * (uint32_t)(D * 2) + 16 * grp;
#pragma unroll
        for (int m = 0; m < D / 32; ++m) t.v[u][m] = buf_ld16(k_head, off + 64 * m);
    }
}

// Same tile, given this lane's byte offset of its first 16 bytes in the tile
// (row0 + lane%16) * 2D + 16*(lane/16): the U x D/32 loads then differ by
// compile-time constants that fit the instruction's immediate offset field, so
// a tile costs no per-load address arithmetic.
template <int D, int U>
__device__ __forceinline__ void load_ktile_at(KTile<D, U>& t, __amdgpu_buffer_rsrc_t k_head,
                                              uint32_t lane_off)
{
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int m = 0; m < D / 32; ++m)
            t.v[u][m] = buf_ld16(k_head, lane_off + (uint32_t)(16 * u * D * 2 + 64 * m));
}

// fp8 K (one byte per element).  A lane loads 16 bytes per load: load j of
// lane group g (= lane/16) holds elements 64j + 16g .. 64j + 16g + 15 of its
// row, and MFMA slab m = 2j + h takes the h-th 8 of them.  The dot product is
// the same sum in another order; q is loaded in that same order
// (load_qfrag_k8), so every fp8 kernel computes identical logits.
template <int D>
__device__ __forceinline__ QFrag<D> load_qfrag_k8(const uint16_t* q_head)
{
    QFrag<D> f;
    const int grp = lane_id() >> 4;
#pragma unroll
    for (int m = 0; m < D / 32; ++m) {
        if (q_head) f.v[m] = ld16(q_head + 64 * (m >> 1) + 16 * grp + 8 * (m & 1));
        else f.v[m] = u32x4{0u, 0u, 0u, 0u};
    }
    return f;
}

// One 16-row group of fp8 K: D/64 loads of 16 bytes per lane.
template <int D>
struct K8Group {
    u32x4 v[D / 64];
};

// The group widened (exactly) to the bf16 operand layout of qk_group.
template <int D>
__device__ __forceinline__ void widen_k8group(const K8Group<D>& x, u32x4 (&kv)[D / 32])
{
#pragma unroll
    for (int j = 0; j < D / 64; ++j) {
        kv[2 * j] = fp8x8_to_bf16x8(u32x2{x.v[j][0], x.v[j][1]});
        kv[2 * j + 1] = fp8x8_to_bf16x8(u32x2{x.v[j][2], x.v[j][3]});
    }
}

template <int D, int U>
struct K8Tile {
    K8Group<D> g[U];
};

// Lane byte offset (row0 + lane%16) * D + 16*(lane/16); the loads differ by
// compile-time constants.
template <int D, int U>
__device__ __forceinline__ void load_k8tile_at(K8Tile<D, U>& t, __amdgpu_buffer_rsrc_t k_head,
                                               uint32_t lane_off)
{
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int j = 0; j < D / 64; ++j)
            t.g[u].v[j] = buf_ld16(k_head, lane_off + (uint32_t)(16 * u * D + 64 * j));
}

// Plain global loads of one group at row pointer p8 (= row * D bytes + 16*(lane/16)).
template <int D>
__device__ __forceinline__ K8Group<D> load_k8group(const uint8_t* p8)
{
    K8Group<D> x;
#pragma unroll
    for (int j = 0; j < D / 64; ++j) x.v[j] = ld16(p8 + 64 * j);
    return x;
}

// logits[u][i] = scale * sum_c q[slot 4*(lane/16)+i][c] * K[row0+16u+lane%16][c]
template <int D, int U>
__device__ __forceinline__ void qk_tile(const QFrag<D>& qf, const KTile<D, U>& kt, float scale,
                                        float (&s)[U][4])
{
#pragma unroll
    for (int u = 0; u < U; ++u) qk_group<D>(qf, kt.v[u], scale, s[u]);
}

// ------------------------------------------------------------ partials
// Per (b, query head, chunk) partial softmax state written by the decode and
// full-attention kernels and merged by combine_kernel.
struct Partials {
    float* m;      // [B*h_q][chunks]  reference max (or -inf: nothing selected)
    float* l;      // [B*h_q][chunks]  sum of exp(s - m)
    int32_t* c;    // [B*h_q][chunks]  number of selected rows
    float* o;      // [B*h_q][chunks][D] sum of exp(s - m) * v
};

}  // namespace saga

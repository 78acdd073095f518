// decode.hip -- SAGA Atop-N decode step: (1) K stream with the threshold
// mask and wave-ballot compaction, (2) masked softmax with the sparse value
// gather, (3) split-sequence combine (shared with the full-attention path).
//
// Method: "More Value per Key: Asymmetric Sparse Attention for Faster LLM
// Decoding" (ai.info AI summary): entries are selected by comparing each
// logit with a reused exact top-N threshold instead of sorting (Key
// Contributions 2, Methodology), and the probability-value product reads only
// the selected value vectors, h_q * N of them per step whatever the number of
// key/value heads (Main Findings, first item).  Key heads are decoupled from
// value heads (Key Contributions 3).
//
// select_stream_kernel: grid.y = (b, key head g), grid.x = a chunk of rows.
//   Each wave streams 16*U-row K tiles once for all h_q/h_k query heads of the
//   group (MFMA QK tile from device.hpp), compares every logit with its head's
//   threshold, and compacts the hits with ballot + popcount straight into a
//   per-(b, query head, chunk, wave) list of (row, logit) in the workspace,
//   together with the list length and the list's largest logit.  No LDS, no
//   waiting on anything but the K stream.
// gather_kernel: grid.y = (b, query head), grid.x = a segment of chunks.
//   Reads its lists' lengths and maxima, stages the entries in LDS with their
//   softmax weights exp(s - M) (M = the segment's largest selected logit),
//   then gathers the selected rows of the query head's value head with
//   16-byte loads, many rows in flight per lane, accumulating in fp32.
//   One (M, l, count, o) partial per (b, query head, segment).
// combine_kernel merges the partials in segment order.
// Every sum runs in a fixed order and no float atomics are used, so results
// are bit-identical run to run.
#include "kernels.hpp"

namespace saga {

namespace {

template <int D, int U>
__global__ __launch_bounds__(kBlock) void select_stream_kernel(SelectStreamArgs a)
{
    // Hits are staged per (wave, head slot) in LDS and written to the global
    // lists in runs of up to kStageCap entries, so the lists are written with
    // whole cache lines instead of scattered 8-byte stores.
    __shared__ uint2 stage[kWavesPerBlock][16][kStageCap];
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int chunk = blockIdx.x;
    const int b = blockIdx.y / a.hk, g = blockIdx.y - b * a.hk;
    const int Gk = a.Gk;
    const int64_t r0 = (int64_t)chunk * a.rows_per_chunk;
    const int64_t r1 = min(r0 + a.rows_per_chunk, a.ctx);
    const int64_t capw = a.rows_per_chunk / kWavesPerBlock;
    const int qh0 = b * a.hq + g * Gk;
    uint2 (*st)[kStageCap] = stage[wave];

    const QFrag<D> qf = load_qfrag<D>(col < Gk ? a.q + (int64_t)(qh0 + col) * D : nullptr);
    float tau[4], mx[4];
    int32_t hits[4], flushed[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int slot = 4 * grp + i;
        tau[i] = slot < Gk ? a.tau[qh0 + slot] : INFINITY;
        mx[i] = -INFINITY;
        hits[i] = 0;
        flushed[i] = 0;
    }
    const uint32_t below = (1u << col) - 1u;

    // Write the staged entries of slots 4*gf + i (gf = 0..3) to their lists.
    auto flush = [&](int i) {
        wave_sync();
#pragma unroll
        for (int gf = 0; gf < 4; ++gf) {
            const int slot = 4 * gf + i;
            if (slot >= Gk) break;
            const int n = __shfl(hits[i] - flushed[i], 16 * gf);
            const int done = __shfl(flushed[i], 16 * gf);
            if (n > 0 && lane < n) {
                const int64_t list = ((int64_t)(qh0 + slot) * a.chunks + chunk) * kWavesPerBlock + wave;
                a.entries[list * capw + done + lane] = st[slot][lane];
            }
        }
        flushed[i] = hits[i];
        wave_sync();
    };

    const uint16_t* khead = a.k + ((int64_t)(b * a.hk + g) * a.cache_len) * D;
    for (int64_t t0 = r0 + wave * 16 * U; t0 < r1; t0 += kWavesPerBlock * 16 * U) {
        KTile<D, U> kt;
        load_ktile<D, U>(kt, khead, t0, r1);
        float s[U][4];
        qk_tile<D, U>(qf, kt, a.scale, s);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t row = t0 + 16 * u + col;
            const bool valid = row < r1;
            if (a.logits_out && valid) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (4 * grp + i < Gk) a.logits_out[(int64_t)(qh0 + 4 * grp + i) * a.ctx + row] = s[u][i];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool pred = valid && s[u][i] >= tau[i];
                const uint64_t mask = __ballot(pred);
                if (mask == 0) continue;                         // wave-uniform
                const uint32_t mine = (uint32_t)(mask >> (16 * grp)) & 0xffffu;
                if (pred) {
                    mx[i] = fmaxf(mx[i], s[u][i]);
                    const int pos = hits[i] - flushed[i] + __popc(mine & below);
                    st[4 * grp + i][pos] = make_uint2((uint32_t)(row - r0), __float_as_uint(s[u][i]));
                }
                hits[i] += __popc(mine);
                if (a.bitmap && col == 0 && mine) {
                    const int64_t row0 = t0 + 16 * u;             // multiple of 16
                    atomicOr(a.bitmap + (int64_t)(qh0 + 4 * grp + i) * a.bitmap_words + row0 / 32,
                             mine << (row0 & 31));
                }
                // A slot gains at most 16 entries per ballot: flush before overflow.
                if (__ballot(hits[i] - flushed[i] > kStageCap - 16)) flush(i);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (__ballot(hits[i] > flushed[i])) flush(i);
        const float m = group16_max(mx[i]);
        if (col == 0 && 4 * grp + i < Gk) {
            const int64_t list = ((int64_t)(qh0 + 4 * grp + i) * a.chunks + chunk) * kWavesPerBlock + wave;
            a.list_count[list] = hits[i];
            a.list_max[list] = m;
        }
    }
}

// Block-wide (256 threads) max and exclusive prefix sum.
__device__ float block_max(float v, float* red)
{
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    if (lane_id() == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    v = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    return v;
}

template <int D>
__global__ __launch_bounds__(kBlock) void gather_kernel(GatherArgs a)
{
    constexpr int LPR = D / 8;             // lanes per value row (16 bytes each)
    constexpr int SLOTS = kBlock / LPR;    // rows per workgroup load instruction
    constexpr int CAPL = 2048;             // entries staged per round
    constexpr int NB = 8;                  // rows in flight per lane
    static_assert(SLOTS * D <= CAPL, "reduction scratch reuses the staging buffer");
    __shared__ int32_t pre[kBlock + 1];
    __shared__ float red[kWavesPerBlock];
    __shared__ uint32_t erow[CAPL];
    __shared__ float ew[CAPL];

    const int seg = blockIdx.x;
    const int bi = blockIdx.y;
    const int b = bi / a.hq, i = bi - b * a.hq;
    const int t = threadIdx.x;
    const int c0 = seg * a.chunks_per_seg;
    const int c1 = min(c0 + a.chunks_per_seg, a.chunks);
    const int nl = (c1 - c0) * kWavesPerBlock;
    const int64_t capw = a.rows_per_chunk / kWavesPerBlock;
    const int64_t lbase = ((int64_t)bi * a.chunks + c0) * kWavesPerBlock;

    int32_t cnt = 0;
    float mx = -INFINITY;
    if (t < nl) {
        cnt = a.list_count[lbase + t];
        mx = a.list_max[lbase + t];
    }
    const float M = block_max(mx, red);
    // exclusive prefix of list lengths
    pre[t] = cnt;
    __syncthreads();
    for (int off = 1; off < kBlock; off <<= 1) {
        const int32_t v = t >= off ? pre[t - off] : 0;
        __syncthreads();
        pre[t] += v;
        __syncthreads();
    }
    const int32_t incl = pre[t];
    __syncthreads();
    pre[t + 1] = incl;
    if (t == 0) pre[0] = 0;
    __syncthreads();
    const int32_t total = pre[nl];

    const uint16_t* vh = a.v + ((int64_t)(b * a.hv + i / a.Gv) * a.cache_len) * D;
    const int slot = t / LPR, lc = t - slot * LPR;
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.f;
    float lsum = 0.f;

    for (int32_t base = 0; base < total; base += CAPL) {
        const int n = min(CAPL, total - base);
        for (int e = t; e < n; e += kBlock) {
            const int32_t E = base + e;
            int lo = 0, hi = nl - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (pre[mid] <= E) lo = mid;
                else hi = mid - 1;
            }
            const int chunk = c0 + lo / kWavesPerBlock;
            const uint2 ent = a.entries[(lbase + lo) * capw + (E - pre[lo])];
            erow[e] = (uint32_t)(chunk * a.rows_per_chunk + ent.x);
            ew[e] = __expf(__uint_as_float(ent.y) - M);
        }
        __syncthreads();
        for (int e0 = slot; e0 < n; e0 += SLOTS * NB) {
            u32x4 vv[NB];
            float w[NB];
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                const int e = e0 + k * SLOTS;
                if (e < n) {
                    vv[k] = ld16(vh + (int64_t)erow[e] * D + 8 * lc);
                    w[k] = ew[e];
                } else {
                    vv[k] = u32x4{0u, 0u, 0u, 0u};
                    w[k] = 0.f;
                }
            }
#pragma unroll
            for (int k = 0; k < NB; ++k) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    acc[2 * j] += w[k] * bf16lo(vv[k][j]);
                    acc[2 * j + 1] += w[k] * bf16hi(vv[k][j]);
                }
                lsum += w[k];
            }
        }
        __syncthreads();
    }

    // Reduce the slots in slot order.
    float* ored = reinterpret_cast<float*>(erow);       // [SLOTS][D]
#pragma unroll
    for (int j = 0; j < 8; ++j) ored[slot * D + 8 * lc + j] = acc[j];
    if (lc == 0) ew[slot] = lsum;
    __syncthreads();
    float l = 0.f;
    for (int s = 0; s < SLOTS; ++s) l += ew[s];
    const int64_t idx = (int64_t)bi * a.segs + seg;
    for (int p = t; p < D; p += kBlock) {
        float o = 0.f;
        for (int s = 0; s < SLOTS; ++s) o += ored[s * D + p];
        a.part.o[idx * D + p] = o;
    }
    if (t == 0) {
        a.part.m[idx] = M;
        a.part.l[idx] = l;
        a.part.c[idx] = total;
    }
}

// Merge the per-segment partials of one (b, query head) in order:
//   M = max m_c, l = sum e^(m_c - M) l_c, o = sum e^(m_c - M) o_c, out = o / l
// (zero when nothing was selected), rounded to bf16.
template <int D>
__global__ __launch_bounds__(D) void combine_kernel(Partials p, int parts, uint16_t* out,
                                                    int32_t* counts)
{
    const int64_t bh = blockIdx.x;
    const int e = threadIdx.x;
    const float* pm = p.m + bh * parts;
    const float* pl = p.l + bh * parts;
    const int32_t* pc = p.c + bh * parts;
    const float* po = p.o + bh * parts * D;
    float M = -INFINITY;
    for (int c = 0; c < parts; ++c) M = fmaxf(M, pm[c]);
    float acc = 0.f, l = 0.f;
    int32_t n = 0;
    for (int c = 0; c < parts; ++c) {
        const float m = pm[c];
        if (m > -INFINITY) {
            const float alpha = __expf(m - M);
            acc += alpha * po[(int64_t)c * D + e];
            l += alpha * pl[c];
        }
        n += pc[c];
    }
    out[bh * D + e] = f32_to_bf16_rne(l > 0.f ? acc / l : 0.f);
    if (counts && e == 0) counts[bh] = n;
}

__global__ void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t v)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

}  // namespace

hipError_t launch_select_stream(int D, const SelectStreamArgs& a, hipStream_t s)
{
    const dim3 grid(a.chunks, a.B * a.hk);
    if (D == 64)
        hipLaunchKernelGGL((select_stream_kernel<64, decode_unroll(64)>), grid, dim3(kBlock), 0, s, a);
    else
        hipLaunchKernelGGL((select_stream_kernel<128, decode_unroll(128)>), grid, dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_gather(int D, const GatherArgs& a, hipStream_t s)
{
    const dim3 grid(a.segs, a.B * a.hq);
    if (D == 64)
        hipLaunchKernelGGL(gather_kernel<64>, grid, dim3(kBlock), 0, s, a);
    else
        hipLaunchKernelGGL(gather_kernel<128>, grid, dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_combine(int D, const Partials& p, int rows, int parts, uint16_t* out,
                          int32_t* counts, hipStream_t s)
{
    if (D == 64)
        hipLaunchKernelGGL(combine_kernel<64>, dim3(rows), dim3(64), 0, s, p, parts, out, counts);
    else
        hipLaunchKernelGGL(combine_kernel<128>, dim3(rows), dim3(128), 0, s, p, parts, out, counts);
    return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n, v);
    return hipGetLastError();
}

}  // namespace saga

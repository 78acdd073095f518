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
    // Hits are staged per (wave, head slot) in LDS (stage_cap(U) entries each)
    // and written to the global lists in whole runs, never as scattered
    // 8-byte stores.  A slot gains at most 16*U entries per tile, so one flush
    // check per tile suffices.
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int CAPS = stage_cap(U);
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int chunk = blockIdx.x;
    const int b = blockIdx.y / a.hk, g = blockIdx.y - b * a.hk;
    const int Gk = a.Gk;
    const int64_t r0 = (int64_t)chunk * a.rows_per_chunk;
    const int64_t r1 = min(r0 + a.rows_per_chunk, a.ctx);
    const int64_t capw = a.rows_per_chunk / kWavesPerBlock;
    const int qh0 = b * a.hq + g * Gk;
    uint2* st = reinterpret_cast<uint2*>(smem) + (size_t)wave * Gk * CAPS;

    const QFrag<D> qf = load_qfrag<D>(col < Gk ? a.q + (int64_t)(qh0 + col) * D : nullptr);
    // Per lane: head slot 4*grp + i.  staged = entries waiting in LDS,
    // written = entries already in the global list.
    float tau[4], mx[4];
    int32_t staged[4], written[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int slot = 4 * grp + i;
        tau[i] = slot < Gk ? a.tau[qh0 + slot] : INFINITY;
        mx[i] = -INFINITY;
        staged[i] = 0;
        written[i] = 0;
    }
    const uint32_t below = (1u << col) - 1u;
    const int64_t list0 = (int64_t)qh0 * a.chunks * kWavesPerBlock + chunk * kWavesPerBlock + wave;
    const int64_t list_stride = (int64_t)a.chunks * kWavesPerBlock;   // between head slots

    auto pick = [](const int32_t (&v)[4], int i) {
        return i == 0 ? v[0] : (i == 1 ? v[1] : (i == 2 ? v[2] : v[3]));
    };
    auto flush_all = [&]() {
        wave_sync();
#pragma unroll 1
        for (int h = 0; h < Gk; ++h) {
            const int n = __shfl(pick(staged, h & 3), 16 * (h >> 2));
            const int off = __shfl(pick(written, h & 3), 16 * (h >> 2));
            uint2* dst = a.entries + (list0 + h * list_stride) * capw + off;
            for (int k = lane; k < n; k += kWave) dst[k] = st[h * CAPS + k];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            written[i] += staged[i];
            staged[i] = 0;
        }
        wave_sync();
    };

    auto process = [&](const KTile<D, U>& kt, int64_t t0) {
        bool full = false;
#pragma unroll
        for (int i = 0; i < 4; ++i) full |= staged[i] > CAPS - 16 * U;
        if (__ballot(full)) flush_all();
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float s[4];
            qk_group<D>(qf, kt.v[u], a.scale, s);
            const int64_t row = t0 + 16 * u + col;
            const bool valid = row < r1;
            if (a.logits_out && valid) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (4 * grp + i < Gk) a.logits_out[(int64_t)(qh0 + 4 * grp + i) * a.ctx + row] = s[i];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool pred = valid && s[i] >= tau[i];
                const uint64_t mask = __ballot(pred);
                if (mask == 0) continue;                         // wave-uniform
                const uint32_t mine = (uint32_t)(mask >> (16 * grp)) & 0xffffu;
                if (pred) {
                    mx[i] = fmaxf(mx[i], s[i]);
                    st[(4 * grp + i) * CAPS + staged[i] + __popc(mine & below)] =
                        make_uint2((uint32_t)(row - r0), __float_as_uint(s[i]));
                }
                staged[i] += __popc(mine);
                if (a.bitmap && col == 0 && mine) {
                    const int64_t row0 = t0 + 16 * u;             // multiple of 16
                    atomicOr(a.bitmap + (int64_t)(qh0 + 4 * grp + i) * a.bitmap_words + row0 / 32,
                             mine << (row0 & 31));
                }
            }
        }
    };

    // Software-pipelined stream: the next tile's loads are issued before the
    // current tile is processed, so every wave keeps a tile in flight.
    const uint16_t* khead = a.k + ((int64_t)(b * a.hk + g) * a.cache_len) * D;
    constexpr int64_t kStep = kWavesPerBlock * 16 * U;
    int64_t t0 = r0 + wave * 16 * U;
    if (t0 < r1) {
        KTile<D, U> ka, kb;
        load_ktile<D, U>(ka, khead, t0, r1);
        while (true) {
            const int64_t t1 = t0 + kStep;
            if (t1 < r1) load_ktile<D, U>(kb, khead, t1, r1);
            process(ka, t0);
            if (t1 >= r1) break;
            const int64_t t2 = t1 + kStep;
            if (t2 < r1) load_ktile<D, U>(ka, khead, t2, r1);
            process(kb, t1);
            if (t2 >= r1) break;
            t0 = t2;
        }
    }
    flush_all();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float m = group16_max(mx[i]);
        if (col == 0 && 4 * grp + i < Gk) {
            const int64_t list = list0 + (4 * grp + i) * list_stride;
            a.list_count[list] = written[i];
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
    constexpr int NB = 16;                 // rows in flight per lane
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

// Merge the per-segment partials of one (b, query head) in a fixed order:
//   M = max m_c, l = sum e^(m_c - M) l_c, o = sum e^(m_c - M) o_c, out = o / l
// (zero when nothing was selected), rounded to bf16.  256 threads: PL part
// lanes x D elements; part lane p takes partials p, p + PL, ...; the part
// lanes are then summed in order.
template <int D>
__global__ __launch_bounds__(kBlock) void combine_kernel(Partials p, int parts, uint16_t* out,
                                                         int32_t* counts)
{
    constexpr int PL = kBlock / D;
    __shared__ float red[kBlock];
    __shared__ float lsh[PL];
    __shared__ int32_t csh[kBlock];
    const int64_t bh = blockIdx.x;
    const int t = threadIdx.x, pl = t / D, e = t - pl * D;
    const float* pm = p.m + bh * parts;
    const float* pl_ = p.l + bh * parts;
    const int32_t* pc = p.c + bh * parts;
    const float* po = p.o + bh * parts * D;

    float M = -INFINITY;
    int32_t n = 0;
    for (int c = t; c < parts; c += kBlock) {
        M = fmaxf(M, pm[c]);
        n += pc[c];
    }
    red[t] = M;
    csh[t] = n;
    __syncthreads();
    for (int off = kBlock / 2; off > 0; off >>= 1) {
        if (t < off) {
            red[t] = fmaxf(red[t], red[t + off]);
            csh[t] += csh[t + off];
        }
        __syncthreads();
    }
    M = red[0];
    n = csh[0];
    __syncthreads();
    if (M == -INFINITY) {                                  // nothing selected anywhere
        if (t < D) out[bh * D + t] = 0;
        if (counts && t == 0) counts[bh] = n;
        return;
    }
    float acc = 0.f, l = 0.f;
    int c = pl;
    for (; c + 3 * PL < parts; c += 4 * PL) {
        float w[4], ov[4], lv[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            w[k] = pm[c + k * PL];
            ov[k] = po[(int64_t)(c + k * PL) * D + e];
            lv[k] = pl_[c + k * PL];
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float a = __expf(w[k] - M);              // -inf partials weigh 0
            acc += a * ov[k];
            l += a * lv[k];
        }
    }
    for (; c < parts; c += PL) {
        const float a = __expf(pm[c] - M);
        acc += a * po[(int64_t)c * D + e];
        l += a * pl_[c];
    }
    red[t] = acc;
    if (e == 0) lsh[pl] = l;
    __syncthreads();
    if (t < D) {
        float o = 0.f, L = 0.f;
        for (int k = 0; k < PL; ++k) {
            o += red[k * D + t];
            L += lsh[k];
        }
        out[bh * D + t] = f32_to_bf16_rne(L > 0.f ? o / L : 0.f);
        if (counts && t == 0) counts[bh] = n;
    }
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
    const size_t lds = (size_t)kWavesPerBlock * a.Gk * stage_cap(decode_unroll(D)) * sizeof(uint2);
    if (D == 64)
        hipLaunchKernelGGL((select_stream_kernel<64, decode_unroll(64)>), grid, dim3(kBlock), lds, s, a);
    else
        hipLaunchKernelGGL((select_stream_kernel<128, decode_unroll(128)>), grid, dim3(kBlock), lds, s, a);
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
        hipLaunchKernelGGL(combine_kernel<64>, dim3(rows), dim3(kBlock), 0, s, p, parts, out, counts);
    else
        hipLaunchKernelGGL(combine_kernel<128>, dim3(rows), dim3(kBlock), 0, s, p, parts, out, counts);
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

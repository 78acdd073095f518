// decode.hip -- SAGA Atop-N decode step: fused K stream, threshold mask,
// wave-ballot compaction, masked online softmax and sparse value gather; plus
// the split-sequence combine shared with the full-attention path.
//
// Method: "More Value per Key: Asymmetric Sparse Attention for Faster LLM
// Decoding" (ai.info AI summary): entries are selected by comparing each
// logit with a reused exact top-N threshold instead of sorting (Key
// Contributions 2, Methodology), and the probability-value product reads only
// the selected value vectors, h_q * N of them per step whatever the number of
// key/value heads (Main Findings, first item).  Key heads are decoupled from
// value heads (Key Contributions 3).
//
// Work decomposition (one launch):
//   grid.y = (b, key head g), grid.x = a chunk of context rows;
//   each of the 4 waves streams 16*U-row tiles of K[b][g] (once for all
//   h_q/h_k query heads of the group: MFMA QK tile from device.hpp), compares
//   each logit with its head's threshold, compacts the hits into a wave-private
//   LDS queue with ballot + mbcnt, and when the queue fills (or the chunk
//   ends) drains it: rescale the running softmax state to the new reference
//   max, gather the selected V rows of each query head's value head and
//   accumulate exp(s - m) * v into wave-private fp32 LDS accumulators.
//   Waves are merged in a fixed order at the end and one (m, l, count, o)
//   partial per (b, query head, chunk) goes to the workspace; combine_kernel
//   merges chunks in chunk order.  No float atomics: results are
//   deterministic run to run.
#include "kernels.hpp"

namespace saga {

namespace {

template <int D>
struct WaveState {
    static constexpr int R = 128 / D;      // value rows gathered per wave instruction
    static constexpr int LPR = kWave / R;  // lanes per gathered row, 2 elements each
    uint32_t* qkey;   // [kQueueCap] (row - chunk_start) << 4 | head slot
    float* qs;        // [kQueueCap] logit of the entry
    float* o;         // [R][Gk][D]
    float* l;         // [R][16]
    float* m_cur;     // [16]
    float* m_new;     // [16]
    int32_t* cnt;     // [16]

    __device__ void carve(unsigned char* base, int Gk)
    {
        qkey = reinterpret_cast<uint32_t*>(base);
        qs = reinterpret_cast<float*>(qkey + kQueueCap);
        o = qs + kQueueCap;
        l = o + R * Gk * D;
        m_cur = l + R * 16;
        m_new = m_cur + 16;
        cnt = reinterpret_cast<int32_t*>(m_new + 16);
    }
};

// Drain the wave's queue of `qn` entries into its softmax accumulators.
// mx[i]: this lane's running max over selected logits of slot 4*(lane/16)+i
// (cumulative over the chunk, so it bounds every queued entry).
template <int D>
__device__ void drain_queue(const WaveState<D>& w, int qn, const float (&mx)[4], int Gk,
                            const uint16_t* __restrict__ v, const int64_t* voff, int64_t r0)
{
    constexpr int R = WaveState<D>::R, LPR = WaveState<D>::LPR, NB = 8;
    const int lane = lane_id(), col = lane & 15, grp = lane >> 4;

    // 1. New reference max per head slot.
    float mg[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) mg[i] = group16_max(mx[i]);
    if (col == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) w.m_new[4 * grp + i] = mg[i];
    }
    wave_sync();

    // 2. Rescale the accumulators of slots whose max moved.
    const int r = lane / LPR, e0 = 2 * (lane % LPR);
    for (int h = 0; h < Gk; ++h) {
        const float mo = w.m_cur[h], mn = w.m_new[h];
        if (mn > mo) {                                   // wave-uniform
            const float alpha = __expf(mo - mn);         // mo = -inf gives 0
            float2* po = reinterpret_cast<float2*>(w.o + (r * Gk + h) * D + e0);
            float2 t = *po;
            t.x *= alpha;
            t.y *= alpha;
            *po = t;
            if ((lane % LPR) == 0) w.l[r * 16 + h] *= alpha;
        }
    }
    wave_sync();
    if (col == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) w.m_cur[4 * grp + i] = mg[i];
    }
    wave_sync();

    // 3. Gather the selected value rows, NB entries per lane slot in flight.
    for (int base = 0; base < qn; base += NB * R) {
        uint32_t vv[NB];
        uint32_t key[NB];
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            const int idx = base + k * R + r;
            key[k] = idx < qn ? w.qkey[idx] : 0xffffffffu;
            if (key[k] != 0xffffffffu) {
                const int h = key[k] & 15;
                const int64_t row = r0 + (key[k] >> 4);
                vv[k] = *reinterpret_cast<const uint32_t*>(v + voff[h] + row * D + e0);
            } else {
                vv[k] = 0u;
            }
        }
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            if (key[k] == 0xffffffffu) continue;
            const int idx = base + k * R + r;
            const int h = key[k] & 15;
            const float wgt = __expf(w.qs[idx] - w.m_cur[h]);
            float2* po = reinterpret_cast<float2*>(w.o + (r * Gk + h) * D + e0);
            float2 t = *po;
            t.x += wgt * bf16lo(vv[k]);
            t.y += wgt * bf16hi(vv[k]);
            *po = t;
            if ((lane % LPR) == 0) w.l[r * 16 + h] += wgt;
        }
    }
    wave_sync();
}

template <int D, int U>
__global__ __launch_bounds__(kBlock) void sparse_decode_kernel(DecodeArgs a)
{
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int R = WaveState<D>::R;
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int chunk = blockIdx.x;
    const int b = blockIdx.y / a.hk, g = blockIdx.y - b * a.hk;
    const int Gk = a.Gk;
    const int64_t r0 = (int64_t)chunk * a.rows_per_chunk;
    const int64_t r1 = min(r0 + a.rows_per_chunk, a.ctx);
    const int qh0 = b * a.hq + g * Gk;                  // flat index of slot 0

    int64_t* voff = reinterpret_cast<int64_t*>(smem);
    WaveState<D> ws;
    ws.carve(smem + kDecodeLdsHeader + wave * a.wave_lds, Gk);

    if (threadIdx.x < 16) {
        const int slot = threadIdx.x;
        const int vh = (g * Gk + slot) / a.Gv;
        voff[slot] = slot < Gk ? ((int64_t)(b * a.hv + vh) * a.cache_len) * D : 0;
    }
    for (int t = lane; t < R * Gk * D; t += kWave) ws.o[t] = 0.f;
    if (lane < 16) {
        ws.m_cur[lane] = -INFINITY;
        ws.cnt[lane] = 0;
        for (int r = 0; r < R; ++r) ws.l[r * 16 + lane] = 0.f;
    }
    __syncthreads();

    const QFrag<D> qf = load_qfrag<D>(col < Gk ? a.q + (int64_t)(qh0 + col) * D : nullptr);
    float tau[4], mx[4];
    int32_t hits[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int slot = 4 * grp + i;
        tau[i] = slot < Gk ? a.tau[qh0 + slot] : INFINITY;
        mx[i] = -INFINITY;
        hits[i] = 0;
    }

    const uint16_t* khead = a.k + ((int64_t)(b * a.hk + g) * a.cache_len) * D;
    int qn = 0;                                          // queued entries (wave-uniform)
    for (int64_t t0 = r0 + wave * 16 * U; t0 < r1; t0 += kWavesPerBlock * 16 * U) {
        KTile<D, U> kt;
        load_ktile<D, U>(kt, khead, t0, r1);
        float s[U][4];
        qk_tile<D, U>(qf, kt, a.scale, s);
        bool pred[U][4];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool valid = t0 + 16 * u + col < r1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pred[u][i] = valid && s[u][i] >= tau[i];
                if (pred[u][i]) mx[i] = fmaxf(mx[i], s[u][i]);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint64_t mask = __ballot(pred[u][i]);
                if (mask == 0) continue;                 // wave-uniform
                const uint32_t mine = (uint32_t)(mask >> (16 * grp)) & 0xffffu;
                hits[i] += __popc(mine);
                if (a.bitmap && col == 0 && mine) {
                    const int64_t row = t0 + 16 * u;     // multiple of 16
                    atomicOr(a.bitmap + (int64_t)(qh0 + 4 * grp + i) * a.bitmap_words + row / 32,
                             mine << (row & 31));
                }
                const int nsel = __popcll(mask);
                if (qn + nsel > kQueueCap) {
                    drain_queue<D>(ws, qn, mx, Gk, a.v, voff, r0);
                    qn = 0;
                }
                if (pred[u][i]) {
                    const int pos = qn + (int)lanes_below(mask);
                    ws.qkey[pos] = (uint32_t)((t0 + 16 * u + col - r0) << 4) | (uint32_t)(4 * grp + i);
                    ws.qs[pos] = s[u][i];
                }
                qn += nsel;
            }
        }
    }
    if (qn > 0) drain_queue<D>(ws, qn, mx, Gk, a.v, voff, r0);
    if (col == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) ws.cnt[4 * grp + i] = hits[i];
    }
    __syncthreads();

    // Merge the 4 waves (fixed order) into this chunk's partial.
    for (int p = threadIdx.x; p < Gk * D; p += kBlock) {
        const int h = p / D, e = p - h * D;
        float M = -INFINITY;
        for (int wv = 0; wv < kWavesPerBlock; ++wv) {
            WaveState<D> o;
            o.carve(smem + kDecodeLdsHeader + wv * a.wave_lds, Gk);
            M = fmaxf(M, o.m_cur[h]);
        }
        float acc = 0.f, l = 0.f;
        int32_t c = 0;
        for (int wv = 0; wv < kWavesPerBlock; ++wv) {
            WaveState<D> o;
            o.carve(smem + kDecodeLdsHeader + wv * a.wave_lds, Gk);
            const float mw = o.m_cur[h];
            if (mw > -INFINITY) {
                const float alpha = __expf(mw - M);
                for (int r = 0; r < R; ++r) {
                    acc += alpha * o.o[(r * Gk + h) * D + e];
                    l += alpha * o.l[r * 16 + h];
                }
            }
            c += o.cnt[h];
        }
        const int64_t idx = (int64_t)(qh0 + h) * a.chunks + chunk;
        a.part.o[idx * D + e] = acc;
        if (e == 0) {
            a.part.m[idx] = M;
            a.part.l[idx] = l;
            a.part.c[idx] = c;
        }
    }
}

// Merge the per-chunk partials of one (b, query head) in chunk order:
//   M = max m_c, l = sum e^(m_c - M) l_c, o = sum e^(m_c - M) o_c, out = o / l
// (zero when nothing was selected), rounded to bf16.
template <int D>
__global__ __launch_bounds__(D) void combine_kernel(Partials p, int chunks, uint16_t* out,
                                                    int32_t* counts)
{
    const int64_t bh = blockIdx.x;
    const int e = threadIdx.x;
    const float* pm = p.m + bh * chunks;
    const float* pl = p.l + bh * chunks;
    const int32_t* pc = p.c + bh * chunks;
    const float* po = p.o + bh * chunks * D;
    float M = -INFINITY;
    for (int c = 0; c < chunks; ++c) M = fmaxf(M, pm[c]);
    float acc = 0.f, l = 0.f;
    int32_t n = 0;
    for (int c = 0; c < chunks; ++c) {
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

hipError_t launch_sparse_decode(int D, const DecodeArgs& a, hipStream_t s)
{
    const dim3 grid(a.chunks, a.B * a.hk);
    const size_t lds = kDecodeLdsHeader + kWavesPerBlock * a.wave_lds;
    if (D == 64)
        hipLaunchKernelGGL((sparse_decode_kernel<64, decode_unroll(64)>), grid, dim3(kBlock), lds, s, a);
    else
        hipLaunchKernelGGL((sparse_decode_kernel<128, decode_unroll(128)>), grid, dim3(kBlock), lds, s, a);
    return hipGetLastError();
}

hipError_t launch_combine(int D, const Partials& p, int rows, int chunks, uint16_t* out,
                          int32_t* counts, hipStream_t s)
{
    if (D == 64)
        hipLaunchKernelGGL(combine_kernel<64>, dim3(rows), dim3(64), 0, s, p, chunks, out, counts);
    else
        hipLaunchKernelGGL(combine_kernel<128>, dim3(rows), dim3(128), 0, s, p, chunks, out, counts);
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

// fused.hip -- the small-batch decode path: K stream, threshold mask,
// ballot compaction and the sparse value gather in one kernel, then a
// combine over many chunks.
//
// Same method as decode.hip ("More Value per Key: Asymmetric Sparse Attention
// for Faster LLM Decoding", ai.info AI summary: selection by per-element
// comparison with a kept exact top-N threshold, Key Contributions 2 and
// Methodology; only the selected value rows are read, Main Findings first
// item).  What differs is where the work runs.  With few (batch row, key
// head) groups, a call is a chain of latency-bound launches: the separate
// gather spends two dependent round trips (list lengths, then entries) before
// its first value row, and one more launch.  Here each workgroup keeps the
// entries its chunk selects in LDS (sized on the host for the worst case, every
// row selected, so nothing spills) and, right after its own K stream, reads
// the value rows of those entries and writes one softmax partial per
// (b, query head, chunk).  combine_parts_kernel merges the chunk partials.
//
// select_gather_kernel: grid (chunks, B * h_k), 256 threads.
//   Stream: as select_stream_kernel, except that each wave compacts its hits
//   straight into one LDS queue per head slot, sized for every row of the
//   wave's share of the chunk, so the queues are never flushed.  Slot s's
//   entries are then in a fixed order: waves in order, then row order.
//   Gather: thread t serves value-row chunk c (16 bytes), head slot h and
//   replica r.  It takes entries r, r + R, ... of slot h (the four waves'
//   queues of slot h, concatenated), NB value rows in flight, and accumulates
//   exp(s - m_h) * v with m_h the slot's largest selected logit in this
//   chunk.  Replicas are then added in replica order, so every sum has a
//   fixed order and results are bit-reproducible.
// combine_parts_kernel: grid (B*h_q rows) x (D / 16 slices); thread t takes
//   partials t, t + 256, ...; M = max m, then sum e^(m - M) (l, o) in a fixed
//   reduction tree; out = o / l in bf16 (zero when nothing was selected).
#include "kernels.hpp"

namespace saga {

namespace {

template <int D, int DV, int U, bool DEBUG, bool PAGED, bool FP8>
__global__ __launch_bounds__(kBlock) SAGA_STREAM_ATTR void select_gather_kernel(FusedArgs a)
{
    extern __shared__ uint2 fq[];                  // [4 waves][G_k head slots][scap]
    __shared__ float hmax[kWavesPerBlock][16];
    const int lane = lane_id(), wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15, grp = lane >> 4;
    const int chunk = blockIdx.x;
    const int b = blockIdx.y / a.hk, g = blockIdx.y - b * a.hk;
    const int Gk = a.Gk;
    const int64_t r0 = (int64_t)chunk * a.rows_per_chunk;
    const int64_t ctx_b = PAGED ? seq_ctx(a.pg, b, a.ctx) : a.ctx;
    const int64_t r1 = wave_uniform(min(r0 + a.rows_per_chunk, ctx_b));
    const int qh0 = b * a.hq + g * Gk;
    const int scap = a.scap;
    uint2* qw = fq + (int64_t)wave * Gk * scap;    // this wave's head-slot queues
    // This lane's group in a ballot: the hits below this lane in it are its
    // group-mates' (rows of the same head slot).
    const uint64_t grp_bits = 0xffffull << (16 * grp);

    const uint16_t* qrow = col < Gk ? a.q + (int64_t)(qh0 + col) * D : nullptr;
    const QFrag<D> qf = FP8 ? load_qfrag_k8<D>(qrow) : load_qfrag<D>(qrow);
    const float sc = FP8 ? a.scale * a.k_scale[blockIdx.y] : a.scale;
    float tau[4], mx[4];
    int64_t lim[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int slot = 4 * grp + i;
        tau[i] = slot < Gk ? a.tau[qh0 + slot] : INFINITY;
        mx[i] = -INFINITY;
        const int64_t hc = a.lq > 1 ? head_ctx(a.pg, a.lq, b, g * Gk + slot, a.ctx) : r1;
        lim[i] = hc < r1 ? hc : r1;
    }
    // Entries so far in the queue of this lane's head slot 4*grp + i (the
    // same in the 16 lanes of a group).
    uint32_t qn[4] = {0u, 0u, 0u, 0u};

    // One 16-row group at row g0: logits, mask, compaction into the queues.
    auto process_group = [&](const u32x4 (&kv)[D / 32], int64_t g0) {
        float s[4];
        qk_group<D>(qf, kv, sc, s);
        const int64_t row = g0 + col;
        const uint32_t tag = (uint32_t)(row - r0);
        if constexpr (DEBUG) {
            if (a.logits_out && row < r1) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (4 * grp + i < Gk)
                        a.logits_out[(int64_t)(qh0 + 4 * grp + i) * a.ctx + row] = s[i];
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool pred = row < lim[i] && s[i] >= tau[i];
            // The hits of this lane's group (head slot 4*grp + i) go to that
            // slot's queue, after its earlier entries, in row order.
            const uint64_t mask = __ballot(pred), ours = mask & grp_bits;
            const uint32_t at = __builtin_amdgcn_mbcnt_hi(
                (uint32_t)(ours >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)ours, qn[i]));
            if (pred)
                qw[(4 * grp + i) * scap + (int)at] = make_uint2(tag, __float_as_uint(s[i]));
            qn[i] += (uint32_t)__popcll(ours);
            mx[i] = fmaxf(mx[i], pred ? s[i] : -INFINITY);
            if constexpr (DEBUG) {
                const uint32_t mine = (uint32_t)(mask >> (16 * grp)) & 0xffffu;
                if (a.bitmap && col == 0 && mine)
                    atomicOr(a.bitmap + (int64_t)(qh0 + 4 * grp + i) * a.bitmap_words + g0 / 32,
                             mine << (g0 & 31));
            }
        }
    };
    auto process = [&](const KTile<D, U>& kt, int64_t t0) {
#pragma unroll
        for (int u = 0; u < U; ++u) process_group(kt.v[u], t0 + 16 * u);
    };
    auto process8 = [&](const K8Tile<D, U>& kt, int64_t t0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            u32x4 kv[D / 32];
            widen_k8group<D>(kt.g[u], kv);
            process_group(kv, t0 + 16 * u);
        }
    };

    // The K stream: software-pipelined tile pairs, buffer resources ending at
    // r1 (prefetches past it read zeros), exactly as in select_stream_kernel.
    constexpr int64_t kStep = kWavesPerBlock * 16 * U;
    if constexpr (PAGED) {
        static_assert(kPageQuantum % (2 * kStep) == 0, "a tile pair must not straddle pages");
        const int64_t P = a.pg.page_rows;
        const uint32_t page_bytes = (uint32_t)(P * D * 2);
        auto lookup = [&](int64_t p) -> int64_t {
            if (p >= a.pg.max_pages) return -1;
            const int32_t page = a.pg.block_table[(int64_t)b * a.pg.max_pages + p];
            if (page < 0 || page >= a.pg.num_pages) return -1;
            return (((int64_t)page * a.hk + g) * P) * D;
        };
        auto page_rsrc = [&](int64_t p, int64_t base) {
            int64_t n = r1 - p * P;
            n = n > P ? P : n;
            if (n < 0 || base < 0) n = 0;
            return make_rsrc(a.k + (base < 0 ? 0 : base), (uint32_t)(n * D * 2));
        };
        constexpr uint32_t kStepBytes = (uint32_t)(kStep * D * 2);
        const uint32_t lane_off = (uint32_t)(wave * 16 * U + col) * (uint32_t)(D * 2) + 16u * grp;
        int64_t tp = r0;
        if (tp < r1) {
            int64_t pi = tp / P;
            uint32_t in = (uint32_t)(tp - pi * P) * (uint32_t)(D * 2);
            __amdgpu_buffer_rsrc_t ra = page_rsrc(pi, lookup(pi));
            int64_t base_n = lookup(pi + 1);
            KTile<D, U> ka, kb;
            load_ktile_at<D, U>(ka, ra, lane_off + in);
            do {
                load_ktile_at<D, U>(kb, ra, lane_off + in + kStepBytes);
                process(ka, tp + wave * 16 * U);
                in += 2 * kStepBytes;
                if (in == page_bytes) {
                    in = 0;
                    ++pi;
                    ra = page_rsrc(pi, base_n);
                    base_n = lookup(pi + 1);
                }
                load_ktile_at<D, U>(ka, ra, lane_off + in);
                process(kb, tp + kStep + wave * 16 * U);
                tp += 2 * kStep;
            } while (tp < r1);
        }
    } else if constexpr (FP8) {
        const uint8_t* k8 = reinterpret_cast<const uint8_t*>(a.k);
        const __amdgpu_buffer_rsrc_t khead =
            make_rsrc(k8 + ((int64_t)(b * a.hk + g) * a.cache_len) * D, (uint32_t)(r1 * D));
        int64_t t0 = r0 + wave * 16 * U;
        if (t0 < r1) {
            constexpr uint32_t kStepBytes = (uint32_t)(kStep * D);
            uint32_t koff = (uint32_t)(t0 + col) * (uint32_t)D + 16u * grp;
            K8Tile<D, U> ka, kb;
            load_k8tile_at<D, U>(ka, khead, koff);
            do {
                load_k8tile_at<D, U>(kb, khead, koff + kStepBytes);
                process8(ka, t0);
                load_k8tile_at<D, U>(ka, khead, koff + 2 * kStepBytes);
                process8(kb, t0 + kStep);
                t0 += 2 * kStep;
                koff += 2 * kStepBytes;
            } while (t0 < r1);
        }
    } else {
        const __amdgpu_buffer_rsrc_t khead =
            make_rsrc(a.k + ((int64_t)(b * a.hk + g) * a.cache_len) * D, (uint32_t)(r1 * D * 2));
        int64_t t0 = r0 + wave * 16 * U;
        if (t0 < r1) {
            constexpr uint32_t kStepBytes = (uint32_t)(kStep * D * 2);
            uint32_t koff = (uint32_t)(t0 + col) * (uint32_t)(D * 2) + 16u * grp;
            KTile<D, U> ka, kb;
            load_ktile_at<D, U>(ka, khead, koff);
            do {
                load_ktile_at<D, U>(kb, khead, koff + kStepBytes);
                process(ka, t0);
                load_ktile_at<D, U>(ka, khead, koff + 2 * kStepBytes);
                process(kb, t0 + kStep);
                t0 += 2 * kStep;
                koff += 2 * kStepBytes;
            } while (t0 < r1);
        }
    }

    // Per-slot largest selected logit and entry count of this wave.
    __shared__ int32_t hcnt[kWavesPerBlock][16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float m = group16_max(mx[i]);
        if (col == 0) hmax[wave][4 * grp + i] = m;
    }
    if (col == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) hcnt[wave][4 * grp + i] = (int32_t)qn[i];
    }
    __syncthreads();

    // Gather.  Thread t: 16-byte chunk c of the value row, head slot h, replica
    // `rep`; it takes entries rep, rep + R, ... of its slot, NB at a time.
    constexpr int C = DV / 8;
    const int P = Gk * C;
    const int R = kBlock / P;                  // >= 1 (Gk <= 16, C <= 16)
    const int t = threadIdx.x;
    const int c = t % C, h = (t / C) % Gk, rep = t / P;
    const bool active = rep < R;
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.f;
    float lsum = 0.f;
    int32_t nsel = 0;
    float M = -INFINITY;
    // Slot h's k-th entry sits in wave w's queue of slot h, w the last wave
    // whose entries start at or below k (c1, c2, c3 for waves 1-3): LDS index
    // k + o_w, with o_w = (w*G_k + h)*scap minus the entries of the waves
    // before w.  Named values, not arrays: an array indexed by a compare
    // would be kept in scratch memory.
    static_assert(kWavesPerBlock == 4, "the wave lookup below covers four waves");
    int32_t c1 = 0, c2 = 0, c3 = 0, o0 = 0, o1 = 0, o2 = 0, o3 = 0;
    if (active) {
        const int32_t n0 = hcnt[0][h], n1 = hcnt[1][h], n2 = hcnt[2][h], n3 = hcnt[3][h];
        M = fmaxf(fmaxf(hmax[0][h], hmax[1][h]), fmaxf(hmax[2][h], hmax[3][h]));
        c1 = n0;
        c2 = c1 + n1;
        c3 = c2 + n2;
        nsel = c3 + n3;
        o0 = h * scap;
        o1 = (Gk + h) * scap - c1;
        o2 = (2 * Gk + h) * scap - c2;
        o3 = (3 * Gk + h) * scap - c3;
    }
    if (active && rep < nsel) {
        const int vi = g * Gk + h;                  // query head (virtual when lq > 1)
        const int nu = vi / a.Gv;
        constexpr int NB = 8;                       // value rows in flight per thread
        // Plain 64-bit loads: the value head differs between the threads of a
        // wave.  Slots past the head's count re-read its entry `rep` with
        // weight zero, so the loads carry no branch.
        const uint16_t* vh = a.v + ((int64_t)(b * a.hv + nu) * a.cache_len) * DV + 8 * c;
        for (int k0 = rep; k0 < nsel; k0 += NB * R) {
            u32x4 vv[NB];
            float wj[NB];
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int k = k0 + j * R;
                const bool valid = k < nsel;
                const int kk = valid ? k : rep;
                const int o = kk >= c3 ? o3 : kk >= c2 ? o2 : kk >= c1 ? o1 : o0;
                const uint2 e = fq[kk + o];
                const uint32_t row = (uint32_t)(r0 + e.x);
                wj[j] = valid ? __expf(__uint_as_float(e.y) - M) : 0.f;
                if constexpr (PAGED) {
                    // A page outside the pool reads as zero.
                    const int64_t pidx = (int64_t)row / a.pg.page_rows;
                    const int32_t page = pidx < a.pg.max_pages
                        ? a.pg.block_table[(int64_t)b * a.pg.max_pages + pidx] : -1;
                    const bool ok = page >= 0 && page < a.pg.num_pages;
                    const u32x4 x = ld16(a.v + ((((int64_t)(ok ? page : 0) * a.hv + nu) *
                                                 a.pg.page_rows + row % a.pg.page_rows) * DV + 8 * c));
                    vv[j] = ok ? x : u32x4{0u, 0u, 0u, 0u};
                } else {
                    vv[j] = ld16(vh + (int64_t)row * DV);
                }
            }
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                lsum += wj[j];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    acc[2 * k] += wj[j] * bf16lo(vv[j][k]);
                    acc[2 * k + 1] += wj[j] * bf16hi(vv[j][k]);
                }
            }
        }
    }
    __syncthreads();                                // queues no longer read

    // Replica sums in replica order; the queues' LDS holds them.
    float* red = reinterpret_cast<float*>(fq);      // [R][Gk][DV], then l [R][Gk]
    float* lred = red + (int64_t)R * Gk * DV;
    if (active) {
#pragma unroll
        for (int j = 0; j < 8; ++j) red[((int64_t)rep * Gk + h) * DV + 8 * c + j] = acc[j];
        if (c == 0) lred[rep * Gk + h] = lsum;
    }
    __syncthreads();
    const int64_t prow0 = (int64_t)qh0 * a.chunks + chunk;   // partial of slot 0
    for (int idx = t; idx < Gk * DV; idx += kBlock) {
        const int hh = idx / DV, p = idx - hh * DV;
        float o = 0.f;
        for (int rr = 0; rr < R; ++rr) o += red[((int64_t)rr * Gk + hh) * DV + p];
        a.part.o[(prow0 + (int64_t)hh * a.chunks) * DV + p] = o;
    }
    if (active && c == 0 && rep == 0) {
        float l = 0.f;
        for (int rr = 0; rr < R; ++rr) l += lred[rr * Gk + h];
        const int64_t pi = prow0 + (int64_t)h * a.chunks;
        a.part.m[pi] = nsel > 0 ? M : -INFINITY;
        a.part.l[pi] = l;
        a.part.c[pi] = nsel;
    }
}

// Merge P partials of one (b, query head) over dims [16 s, 16 s + 16).
template <int D>
__global__ __launch_bounds__(kBlock) void combine_parts_kernel(Partials p, int parts,
                                                               uint16_t* out, int32_t* counts)
{
    constexpr int SL = 16;                          // dims per workgroup
    constexpr int KP = 4;                           // partials per thread held in registers
    __shared__ float wred[kWavesPerBlock];
    __shared__ int32_t cred[kWavesPerBlock];
    __shared__ float ored[kWavesPerBlock][SL + 1];
    const int64_t bh = blockIdx.x / (D / SL);
    const int s = blockIdx.x - (int)(bh * (D / SL));
    const int t = threadIdx.x;
    const float* pm = p.m + bh * parts;
    const float* pl = p.l + bh * parts;
    const int32_t* pc = p.c + bh * parts;
    const float* po = p.o + bh * parts * D + SL * s;

    // Loads for the first KP partials of this thread, all in flight at once.
    float m[KP], l[KP];
    u32x4 o[KP][SL / 4];
    float M = -INFINITY;
    int32_t n = 0;
#pragma unroll
    for (int k = 0; k < KP; ++k) {
        const int cp = t + k * kBlock;
        const int ci = cp < parts ? cp : parts - 1;
        m[k] = pm[ci];
        l[k] = pl[ci];
        const int32_t cc = pc[ci];
#pragma unroll
        for (int q = 0; q < SL / 4; ++q) o[k][q] = ld16(po + (int64_t)ci * D + 4 * q);
        const bool in = cp < parts;
        m[k] = in ? m[k] : -INFINITY;
        M = fmaxf(M, m[k]);
        n += in ? cc : 0;
    }
    for (int cp = t + KP * kBlock; cp < parts; cp += kBlock) {       // many partials: loop
        M = fmaxf(M, pm[cp]);
        n += pc[cp];
    }
    M = block_max(M, wred);
    n = block_sum(n, cred);
    if (M == -INFINITY) {                                  // nothing selected anywhere
        if (t < SL) out[bh * D + SL * s + t] = 0;
        if (counts && s == 0 && t == 0) counts[bh] = n;
        return;
    }
    float acc[SL], L = 0.f;
#pragma unroll
    for (int j = 0; j < SL; ++j) acc[j] = 0.f;
#pragma unroll
    for (int k = 0; k < KP; ++k) {
        const float w = __expf(m[k] - M);                  // -inf partials weigh 0
        L += w * l[k];
#pragma unroll
        for (int q = 0; q < SL / 4; ++q) {
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[4 * q + e] += w * __uint_as_float(o[k][q][e]);
        }
    }
    for (int cp = t + KP * kBlock; cp < parts; cp += kBlock) {
        const float w = __expf(pm[cp] - M);
        L += w * pl[cp];
#pragma unroll
        for (int j = 0; j < SL; ++j) acc[j] += w * po[(int64_t)cp * D + j];
    }
    // Fixed-order reduction: butterfly within the wave, then waves in order.
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) {
        L += __shfl_xor(L, off);
#pragma unroll
        for (int j = 0; j < SL; ++j) acc[j] += __shfl_xor(acc[j], off);
    }
    const int w = t >> 6;
    if ((t & 63) == 0) {
#pragma unroll
        for (int j = 0; j < SL; ++j) ored[w][j] = acc[j];
        ored[w][SL] = L;
    }
    __syncthreads();
    if (t < SL) {
        float os = 0.f, ls = 0.f;
#pragma unroll
        for (int ww = 0; ww < kWavesPerBlock; ++ww) {
            os += ored[ww][t];
            ls += ored[ww][SL];
        }
        out[bh * D + SL * s + t] = f32_to_bf16_rne(ls > 0.f ? os / ls : 0.f);
    }
    if (counts && s == 0 && t == 0) counts[bh] = n;
}

}  // namespace

hipError_t launch_select_gather(int D, int DV, const FusedArgs& a, size_t lds_bytes, hipStream_t s)
{
    const dim3 grid(a.chunks, a.B * a.hk);
    const bool dbg = a.bitmap != nullptr || a.logits_out != nullptr;
    const bool paged = a.pg.block_table != nullptr;
    const bool k8 = a.k_scale != nullptr;
    if (k8 && (paged || D == 32)) return hipErrorInvalidValue;
    if (a.unroll != 1 && a.unroll != 2) return hipErrorInvalidValue;
#define SAGA_FUSED(DD, DDV, UU, DBG, PG, F8)                                                    \
    hipLaunchKernelGGL((select_gather_kernel<DD, DDV, (F8 ? SAGA_STREAM_K8_UMUL : 1) * UU, DBG,   \
                                             PG, F8>),                                             \
                       grid, dim3(kBlock), lds_bytes, s, a)
#define SAGA_FUSED_U(DD, DDV, DBG, PG, F8)                                                      \
    if (a.unroll == 2) SAGA_FUSED(DD, DDV, 2, DBG, PG, F8); else SAGA_FUSED(DD, DDV, 1, DBG, PG, F8);
#define SAGA_FUSED_DBG(DD, DDV, PG, F8)                                                         \
    if (dbg) { SAGA_FUSED_U(DD, DDV, true, PG, F8) } else { SAGA_FUSED_U(DD, DDV, false, PG, F8) }
#define SAGA_FUSED_MODE(DD, DDV)                                                                \
    if (k8) { SAGA_FUSED_DBG(DD, DDV, false, true) }                                            \
    else if (paged) { SAGA_FUSED_DBG(DD, DDV, true, false) }                                    \
    else { SAGA_FUSED_DBG(DD, DDV, false, false) }
#define SAGA_FUSED_MODE_BF(DD, DDV)                                                             \
    if (paged) { SAGA_FUSED_DBG(DD, DDV, true, false) }                                         \
    else { SAGA_FUSED_DBG(DD, DDV, false, false) }
    if (D == 32) {
        if (DV == 32) { SAGA_FUSED_MODE_BF(32, 32) }
        else if (DV == 64) { SAGA_FUSED_MODE_BF(32, 64) }
        else { SAGA_FUSED_MODE_BF(32, 128) }
    } else if (D == 64) {
        if (DV == 32) { SAGA_FUSED_MODE(64, 32) }
        else if (DV == 64) { SAGA_FUSED_MODE(64, 64) }
        else { SAGA_FUSED_MODE(64, 128) }
    } else {
        if (DV == 32) { SAGA_FUSED_MODE(128, 32) }
        else if (DV == 64) { SAGA_FUSED_MODE(128, 64) }
        else { SAGA_FUSED_MODE(128, 128) }
    }
#undef SAGA_FUSED_MODE_BF
#undef SAGA_FUSED_MODE
#undef SAGA_FUSED_DBG
#undef SAGA_FUSED_U
#undef SAGA_FUSED
    return hipGetLastError();
}

hipError_t launch_combine_parts(int D, const Partials& p, int rows, int parts, uint16_t* out,
                                int32_t* counts, hipStream_t s)
{
    const dim3 grid((unsigned)rows * (unsigned)(D / 16));
    if (D == 32)
        hipLaunchKernelGGL(combine_parts_kernel<32>, grid, dim3(kBlock), 0, s, p, parts, out, counts);
    else if (D == 64)
        hipLaunchKernelGGL(combine_parts_kernel<64>, grid, dim3(kBlock), 0, s, p, parts, out, counts);
    else
        hipLaunchKernelGGL(combine_parts_kernel<128>, grid, dim3(kBlock), 0, s, p, parts, out, counts);
    return hipGetLastError();
}

}  // namespace saga

// full.hip -- dense decode attention over every attended row (the full-
// attention GQA baseline when h_k == h_v, "SAGA full attention" when
// h_k < h_v).  "More Value per Key: Asymmetric Sparse Attention for Faster
// LLM Decoding" (ai.info AI summary, Main Findings): the pages time SAGA +
// Atop-N against full-attention GQA, and SAGA's fewer key heads alone against
// the GQA baseline; decode attention is a matrix-vector product, so the
// baseline is plain (non-flash) attention.
//
// Decomposition: grid.y = (b, key head g), grid.x = context chunk.  The query
// heads of key head g read nv value heads (1, 2 or 4); the 4 waves are split
// into (4/nv row sets) x (nv value heads).  Every wave streams the K tile of
// its rows (waves of one row set read the same K lines, served from cache),
// runs the shared MFMA QK tile, keeps an online softmax per head slot, and
// accumulates p * v for the query heads of its own value head on the VALU
// from 16-byte V loads.  Row sets are merged in a fixed order into one
// partial per (b, query head, chunk), then combine_kernel (decode.hip)
// merges chunks.
#include "kernels.hpp"

namespace saga {

namespace {

template <int DK, int DV, int U, int MAXS>
__global__ __launch_bounds__(kBlock) void full_attn_kernel(FullArgs a)
{
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int TR = 16 * U;            // rows per wave tile
    constexpr int LPRV = DV / 8;          // lanes per V row (16 bytes each)
    constexpr int RPI = kWave / LPRV;     // V rows per load instruction
    constexpr int NV = TR / RPI;          // V loads per lane per tile
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int chunk = blockIdx.x;
    const int b = blockIdx.y / a.hk, g = blockIdx.y - b * a.hk;
    const int Gk = a.Gk, Gv = a.Gv, nv = a.nv;
    const int rowsets = kWavesPerBlock / nv;
    const int rs = wave / nv, vsel = wave - rs * nv;
    const int i0 = g * Gk;
    const int vh = i0 / Gv + vsel;                      // this wave's value head
    int slo = max(vh * Gv, i0) - i0;
    int ns = min((vh + 1) * Gv, i0 + Gk) - i0 - slo;    // its query-head slots
    if (vh >= a.hv || ns < 0) ns = 0;
    const int64_t r0 = (int64_t)chunk * a.rows_per_chunk;
    const int64_t r1 = min(r0 + a.rows_per_chunk, a.ctx);
    const int qh0 = b * a.hq + i0;

    unsigned char* wb = smem + wave * a.wave_lds;
    float* P = reinterpret_cast<float*>(wb);             // [TR][16]
    float* alpha_l = P + TR * 16;                        // [16]
    float* m_l = alpha_l + 16;                           // [16]
    float* l_l = m_l + 16;                               // [16]
    float* o_l = l_l + 16;                               // [MAXS][DV]

    const QFrag<DK> qf = load_qfrag<DK>(col < Gk ? a.q + (int64_t)(qh0 + col) * DK : nullptr);
    const uint16_t* khead = a.k + ((int64_t)(b * a.hk + g) * a.cache_len) * DK;
    const uint16_t* vhead = a.v + ((int64_t)(b * a.hv + (ns > 0 ? vh : 0)) * a.cache_len) * DV;
    const int vrow = lane / LPRV, vcol = 8 * (lane % LPRV);

    float m_run[4], l_part[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        m_run[i] = -INFINITY;
        l_part[i] = 0.f;
    }
    float oacc[MAXS][8];
#pragma unroll
    for (int k = 0; k < MAXS; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e) oacc[k][e] = 0.f;

    for (int64_t t0 = r0 + rs * TR; t0 < r1; t0 += rowsets * TR) {
        KTile<DK, U> kt;
        load_ktile<DK, U>(kt, khead, t0, r1);
        u32x4 vt[NV];
        if (ns > 0) {
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                int64_t row = t0 + k * RPI + vrow;
                row = row < r1 ? row : r1 - 1;
                vt[k] = ld16(vhead + row * DV + vcol);
            }
        }
        float s[U][4];
        qk_tile<DK, U>(qf, kt, a.scale, s);

        float alpha[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float tm = -INFINITY;
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (t0 + 16 * u + col < r1) tm = fmaxf(tm, s[u][i]);
            tm = group16_max(tm);
            const float mn = fmaxf(m_run[i], tm);
            alpha[i] = __expf(m_run[i] - mn);
            float psum = 0.f;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float p = (t0 + 16 * u + col < r1) ? __expf(s[u][i] - mn) : 0.f;
                s[u][i] = p;
                psum += p;
            }
            l_part[i] = alpha[i] * l_part[i] + psum;
            m_run[i] = mn;
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            *reinterpret_cast<float4*>(P + (16 * u + col) * 16 + 4 * grp) =
                make_float4(s[u][0], s[u][1], s[u][2], s[u][3]);
        if (col == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) alpha_l[4 * grp + i] = alpha[i];
        }
        wave_sync();
        if (ns > 0) {
#pragma unroll
            for (int k = 0; k < MAXS; ++k) {
                if (k < ns) {
                    const float al = alpha_l[slo + k];
#pragma unroll
                    for (int e = 0; e < 8; ++e) oacc[k][e] *= al;
                }
            }
#pragma unroll
            for (int kk = 0; kk < NV; ++kk) {
                float vf[8];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    vf[2 * j] = bf16lo(vt[kk][j]);
                    vf[2 * j + 1] = bf16hi(vt[kk][j]);
                }
                const float* prow = P + (kk * RPI + vrow) * 16 + slo;
#pragma unroll
                for (int k = 0; k < MAXS; ++k) {
                    if (k < ns) {
                        const float pk = prow[k];
#pragma unroll
                        for (int e = 0; e < 8; ++e) oacc[k][e] += pk * vf[e];
                    }
                }
            }
        }
        wave_sync();
    }

    // Wave results: m and l per slot (MFMA layout), o for this wave's slots.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float lsum = group16_sum(l_part[i]);
        if (col == 0) {
            m_l[4 * grp + i] = m_run[i];
            l_l[4 * grp + i] = lsum;
        }
    }
#pragma unroll
    for (int k = 0; k < MAXS; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float v = oacc[k][e];
            for (int off = LPRV; off < kWave; off <<= 1) v += __shfl_xor(v, off);
            oacc[k][e] = v;
        }
    if (lane < LPRV) {
#pragma unroll
        for (int k = 0; k < MAXS; ++k)
            if (k < ns) {
#pragma unroll
                for (int e = 0; e < 8; ++e) o_l[k * DV + vcol + e] = oacc[k][e];
            }
    }
    __syncthreads();

    // Merge row sets in a fixed order.
    for (int p = threadIdx.x; p < Gk * DV; p += kBlock) {
        const int h = p / DV, e = p - h * DV;
        const int vh_h = (i0 + h) / Gv;
        const int vsel_h = vh_h - i0 / Gv;
        const int k_h = h - (max(vh_h * Gv, i0) - i0);
        float M = -INFINITY;
        for (int r = 0; r < rowsets; ++r) {
            const float* mw = reinterpret_cast<const float*>(
                smem + (r * nv + vsel_h) * a.wave_lds) + TR * 16 + 16;
            M = fmaxf(M, mw[h]);
        }
        float acc = 0.f, l = 0.f;
        for (int r = 0; r < rowsets; ++r) {
            const float* base = reinterpret_cast<const float*>(smem + (r * nv + vsel_h) * a.wave_lds);
            const float mw = base[TR * 16 + 16 + h];
            if (mw > -INFINITY) {
                const float al = __expf(mw - M);
                acc += al * base[TR * 16 + 48 + k_h * DV + e];
                l += al * base[TR * 16 + 32 + h];
            }
        }
        const int64_t idx = (int64_t)(qh0 + h) * a.chunks + chunk;
        a.part.o[idx * DV + e] = acc;
        if (e == 0) {
            a.part.m[idx] = M;
            a.part.l[idx] = l;
            a.part.c[idx] = (int32_t)(r1 - r0);
        }
    }
}

template <int DK, int DV>
hipError_t launch_full_d(int maxs, const FullArgs& a, hipStream_t s)
{
    const dim3 grid(a.chunks, a.B * a.hk);
    const size_t lds = kWavesPerBlock * a.wave_lds;
    constexpr int U = full_unroll(DK, DV);
    if (maxs <= 2)
        hipLaunchKernelGGL((full_attn_kernel<DK, DV, U, 2>), grid, dim3(kBlock), lds, s, a);
    else if (maxs <= 4)
        hipLaunchKernelGGL((full_attn_kernel<DK, DV, U, 4>), grid, dim3(kBlock), lds, s, a);
    else
        hipLaunchKernelGGL((full_attn_kernel<DK, DV, U, 8>), grid, dim3(kBlock), lds, s, a);
    return hipGetLastError();
}

template <int DK>
hipError_t launch_full_dk(int DV, int maxs, const FullArgs& a, hipStream_t s)
{
    if (DV == 32) return launch_full_d<DK, 32>(maxs, a, s);
    if (DV == 64) return launch_full_d<DK, 64>(maxs, a, s);
    return launch_full_d<DK, 128>(maxs, a, s);
}

}  // namespace

hipError_t launch_full(int DK, int DV, int maxs, const FullArgs& a, hipStream_t s)
{
    if (DK == 32) return launch_full_dk<32>(DV, maxs, a, s);
    if (DK == 64) return launch_full_dk<64>(DV, maxs, a, s);
    return launch_full_dk<128>(DV, maxs, a, s);
}

}  // namespace saga

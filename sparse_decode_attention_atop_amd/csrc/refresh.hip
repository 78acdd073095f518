// refresh.hip -- Atop-N exact top-N threshold refresh.
//
// "More Value per Key: Asymmetric Sparse Attention for Faster LLM Decoding"
// (ai.info AI summary, Key Contributions 2 and Methodology): every n decode
// steps the thresholds are recomputed exactly, then reused in between.  Here
// "exact" means: tau[b][i] is bit for bit the N-th largest of the fp32 logits
// that the decode kernel computes for the same inputs (one shared QK tile
// routine), so s >= tau keeps exactly N entries when there are no ties.
//
// Pipeline (4 launches, all on the caller's stream):
//   1. qk_logits_kernel   stream K once per (b, key head), write fp32 logits
//                         [B*h_q][ld] to the workspace; chunk-0 workgroups
//                         also clear the per-row select state.
//   2. radix_hist_kernel  per (row, segment): LDS histogram of the top 12 bits
//                         of the order-preserving key, merged into a global
//                         per-row histogram with integer atomics; the last
//                         segment of a row to finish scans it and records the
//                         bucket holding rank N and the rank inside it.
//   3. radix_compact_kernel per (row, segment): append the keys of that bucket
//                         to a per-row candidate list (wave-aggregated atomics).
//   4. radix_final_kernel per row: two 10-bit LDS histogram passes over the
//                         candidates fix the remaining 20 key bits.
// Integer counting only, so the result does not depend on scheduling.
#include "kernels.hpp"

namespace saga {

namespace {

template <int D, int U>
__global__ __launch_bounds__(kBlock) void qk_logits_kernel(LogitsArgs a)
{
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int chunk = blockIdx.x;
    const int b = blockIdx.y / a.hk, g = blockIdx.y - b * a.hk;
    const int Gk = a.Gk;
    const int64_t r0 = (int64_t)chunk * a.rows_per_chunk;
    const int64_t r1 = min(r0 + a.rows_per_chunk, a.ctx);
    const int qh0 = b * a.hq + g * Gk;

    if (chunk == 0) {
        for (int t = threadIdx.x; t < Gk * kHistBins; t += kBlock)
            a.ghist[(int64_t)qh0 * kHistBins + t] = 0u;
        if (threadIdx.x < Gk) {
            a.done[qh0 + threadIdx.x] = 0u;
            a.cand_count[qh0 + threadIdx.x] = 0u;
        }
    }

    const QFrag<D> qf = load_qfrag<D>(col < Gk ? a.q + (int64_t)(qh0 + col) * D : nullptr);
    const uint16_t* khead = a.k + ((int64_t)(b * a.hk + g) * a.cache_len) * D;
    for (int64_t t0 = r0 + wave * 16 * U; t0 < r1; t0 += kWavesPerBlock * 16 * U) {
        KTile<D, U> kt;
        load_ktile<D, U>(kt, khead, t0, r1);
        float s[U][4];
        qk_tile<D, U>(qf, kt, a.scale, s);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t row = t0 + 16 * u + col;
            if (row >= r1) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int slot = 4 * grp + i;
                if (slot >= Gk) continue;
                a.logits[(int64_t)(qh0 + slot) * a.ld + row] = s[u][i];
                if (a.debug) a.debug[(int64_t)(qh0 + slot) * a.ctx + row] = s[u][i];
            }
        }
    }
}

// Block-wide search of a histogram held in LDS for the bucket containing
// rank `rank` (1-based, counted from the largest key).  Thread t owns the
// BINS/256 consecutive buckets starting from the top.  Returns the bucket in
// *bin and the rank inside it in *rank_in; all threads see the result.
template <int BINS>
__device__ void find_rank_bucket(const uint32_t* hist, uint32_t rank, uint32_t* scan,
                                 uint32_t* result, uint32_t* bin, uint32_t* rank_in,
                                 uint32_t* bin_count)
{
    constexpr int PER = BINS / kBlock;
    const int t = threadIdx.x;
    uint32_t c[PER], sum = 0;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        c[k] = hist[BINS - 1 - PER * t - k];
        sum += c[k];
    }
    scan[t] = sum;
    __syncthreads();
    for (int off = 1; off < kBlock; off <<= 1) {
        const uint32_t v = t >= off ? scan[t - off] : 0u;
        __syncthreads();
        scan[t] += v;
        __syncthreads();
    }
    uint32_t above = scan[t] - sum;
    if (above < rank && above + sum >= rank) {
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            if (above + c[k] >= rank) {
                result[0] = (uint32_t)(BINS - 1 - PER * t - k);
                result[1] = rank - above;
                result[2] = c[k];
                break;
            }
            above += c[k];
        }
    }
    __syncthreads();
    *bin = result[0];
    *rank_in = result[1];
    *bin_count = result[2];
    __syncthreads();
}

__global__ __launch_bounds__(kBlock) void radix_hist_kernel(SelectArgs a)
{
    __shared__ uint32_t hist[kHistBins];
    __shared__ uint32_t scan[kBlock];
    __shared__ uint32_t result[3];
    __shared__ int last;
    const int row = blockIdx.y, seg = blockIdx.x, t = threadIdx.x;
    for (int k = t; k < kHistBins; k += kBlock) hist[k] = 0u;
    __syncthreads();
    const float* s = a.logits + (int64_t)row * a.ld;
    const int64_t j0 = (int64_t)seg * kSelectSeg;
    const int64_t j1 = min(j0 + (int64_t)kSelectSeg, a.ctx);
    for (int64_t j = j0 + t; j < j1; j += kBlock) atomicAdd(&hist[float_key(s[j]) >> 20], 1u);
    __syncthreads();
    uint32_t* gh = a.ghist + (int64_t)row * kHistBins;
    for (int k = t; k < kHistBins; k += kBlock)
        if (hist[k]) atomicAdd(&gh[k], hist[k]);
    __threadfence();
    __syncthreads();
    if (t == 0) last = atomicAdd(&a.done[row], 1u) == (uint32_t)(a.segs - 1);
    __syncthreads();
    if (!last) return;
    __threadfence();
    for (int k = t; k < kHistBins; k += kBlock)
        hist[k] = __hip_atomic_load(&gh[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    uint32_t bin, rank_in, cnt;
    find_rank_bucket<kHistBins>(hist, a.top_n, scan, result, &bin, &rank_in, &cnt);
    if (t == 0) {
        a.state[row * 4 + 0] = bin;
        a.state[row * 4 + 1] = rank_in;
        a.state[row * 4 + 2] = cnt;
    }
}

__global__ __launch_bounds__(kBlock) void radix_compact_kernel(SelectArgs a)
{
    const int row = blockIdx.y, seg = blockIdx.x, t = threadIdx.x;
    const uint32_t bucket = a.state[row * 4 + 0];
    const float* s = a.logits + (int64_t)row * a.ld;
    uint32_t* cand = a.cand + (int64_t)row * a.ld;
    const int64_t j0 = (int64_t)seg * kSelectSeg;
    const int64_t j1 = min(j0 + (int64_t)kSelectSeg, a.ctx);
    for (int64_t jb = j0; jb < j1; jb += kBlock) {
        const int64_t j = jb + t;
        uint32_t key = 0u;
        bool hit = false;
        if (j < j1) {
            key = float_key(s[j]);
            hit = (key >> 20) == bucket;
        }
        const uint64_t mask = __ballot(hit);
        if (mask == 0) continue;
        const int leader = __ffsll((unsigned long long)mask) - 1;
        uint32_t base = 0u;
        if (lane_id() == leader) base = atomicAdd(&a.cand_count[row], (uint32_t)__popcll(mask));
        base = __shfl(base, leader);
        if (hit) cand[base + lanes_below(mask)] = key;
    }
}

__global__ __launch_bounds__(kBlock) void radix_final_kernel(SelectArgs a)
{
    constexpr int BINS = 1024;
    __shared__ uint32_t hist[BINS];
    __shared__ uint32_t scan[kBlock];
    __shared__ uint32_t result[3];
    const int row = blockIdx.x, t = threadIdx.x;
    const uint32_t bucket = a.state[row * 4 + 0];
    const uint32_t rank = a.state[row * 4 + 1];
    const uint32_t n = a.cand_count[row];
    const uint32_t* cand = a.cand + (int64_t)row * a.ld;

    // Pass A: key bits 19..10.
    for (int k = t; k < BINS; k += kBlock) hist[k] = 0u;
    __syncthreads();
    for (uint32_t k = t; k < n; k += kBlock) atomicAdd(&hist[(cand[k] >> 10) & 1023u], 1u);
    __syncthreads();
    uint32_t binA, rankA, cntA;
    find_rank_bucket<BINS>(hist, rank, scan, result, &binA, &rankA, &cntA);

    // Pass B: key bits 9..0 among keys that share bits 19..10.
    for (int k = t; k < BINS; k += kBlock) hist[k] = 0u;
    __syncthreads();
    for (uint32_t k = t; k < n; k += kBlock) {
        const uint32_t key = cand[k];
        if (((key >> 10) & 1023u) == binA) atomicAdd(&hist[key & 1023u], 1u);
    }
    __syncthreads();
    uint32_t binB, rankB, cntB;
    find_rank_bucket<BINS>(hist, rankA, scan, result, &binB, &rankB, &cntB);
    if (t == 0) a.tau[row] = key_float((bucket << 20) | (binA << 10) | binB);
}

}  // namespace

hipError_t launch_qk_logits(int D, const LogitsArgs& a, int chunks, hipStream_t s)
{
    const dim3 grid(chunks, a.B * a.hk);
    if (D == 64)
        hipLaunchKernelGGL((qk_logits_kernel<64, decode_unroll(64)>), grid, dim3(kBlock), 0, s, a);
    else
        hipLaunchKernelGGL((qk_logits_kernel<128, decode_unroll(128)>), grid, dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_select(const SelectArgs& a, hipStream_t s)
{
    const dim3 grid(a.segs, a.rows);
    hipLaunchKernelGGL(radix_hist_kernel, grid, dim3(kBlock), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(radix_compact_kernel, grid, dim3(kBlock), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(radix_final_kernel, dim3(a.rows), dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

}  // namespace saga

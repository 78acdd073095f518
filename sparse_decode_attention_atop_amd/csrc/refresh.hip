// refresh.hip -- Atop-N exact top-N threshold refresh.
//
// "More Value per Key: Asymmetric Sparse Attention for Faster LLM Decoding"
// (ai.info AI summary, Key Contributions 2 and Methodology): every n decode
// steps the thresholds are recomputed exactly, then reused in between.  Here
// "exact" means: tau[b][i] is bit for bit the N-th largest of the fp32 logits
// that the decode kernel computes for the same inputs (one shared QK tile
// routine), so s >= tau keeps exactly N entries when there are no ties.
//
// Pipeline (all on the caller's stream; one pass over the K cache):
//   1. sample_logits_kernel  logits of a sample of at most kSampleMax rows per
//                            (b, query head): evenly spaced 16-row blocks.
//   2. pivot_kernel          per row: the k-th largest sample logit (radix
//                            select on keys held in registers), with k chosen
//                            so that the pivot p lies below tau with
//                            overwhelming probability.
//   3. select_stream_kernel  (decode.hip) with p as the threshold: every logit
//                            >= p goes to the per-(row, chunk, wave) lists.
//   4. refresh_final_kernel  per row: if the lists hold at least N entries,
//                            tau is the N-th largest of them (then every entry
//                            >= tau is in the lists; radix select on the
//                            candidates held in registers).
//                            Otherwise -- or if they are too many to stage --
//                            the workgroup recomputes the row's logits with the
//                            same QK tile and radix-selects over all of them.
// Steps 1-2 only decide how much work step 4 has; they never change tau.
// Integer counting on order-preserving keys throughout: the result does not
// depend on scheduling.
#include "kernels.hpp"

namespace saga {

namespace {

// Block-wide search of a histogram held in LDS for the bucket containing
// rank `rank` (1-based, counted from the largest key).  Thread t owns the
// BINS/256 consecutive buckets starting from the top.  All threads receive
// the bucket, the rank inside it and its size.
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
    // Counts of one row stay below 2^31, so the signed scan is exact.
    uint32_t above = (uint32_t)block_scan((int32_t)sum, reinterpret_cast<int32_t*>(scan)) - sum;
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

// Radix digits of the 32-bit key, most significant first: 11, 11, 10 bits.
__device__ __forceinline__ int digit_shift(int pass) { return pass == 0 ? 21 : (pass == 1 ? 10 : 0); }
__device__ __forceinline__ uint32_t digit_mask(int pass) { return pass == 2 ? 1023u : 2047u; }
// Bits above the digit of `pass` (they must match the prefix found so far).
__device__ __forceinline__ uint32_t prefix_mask(int pass)
{
    return pass == 0 ? 0u : (pass == 1 ? 0xffe00000u : 0xfffffc00u);
}

// Exclusive max-scan over the block in thread order (0 before thread 0).
__device__ __forceinline__ uint32_t block_scan_max_excl(uint32_t v, uint32_t* red)
{
    const int lane = lane_id();
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t u = __shfl_up(v, off);
        if (lane >= off) v = v > u ? v : u;
    }
    if (lane == kWave - 1) red[threadIdx.x >> 6] = v;
    const uint32_t below = __shfl_up(v, 1);
    __syncthreads();
    const int w = threadIdx.x >> 6;
    uint32_t x = lane > 0 ? below : 0u;
#pragma unroll
    for (int k = 0; k < kWavesPerBlock - 1; ++k)
        if (k < w && red[k] > x) x = red[k];
    __syncthreads();
    return x;
}

// Histogram width of the register-resident select: 12-bit digits.
constexpr int kRegDigit = 12;
constexpr int kRegBins = 1 << kRegDigit;
static_assert(kRegBins >= kHistBins, "one histogram serves both selects");

struct SelectLds {
    alignas(16) uint32_t hist[kRegBins];
    uint32_t scan[kBlock];
    uint32_t result[3];
};

// The rank-th largest (1 <= rank <= n) of n keys held in registers by the
// block: key j of thread t is item t + j * kBlock, valid below n.  A radix
// select on u = key - (smallest key), in digits of up to 12 bits from the top
// bit of the largest u down.  Counting from the range rather than from the
// key's sign and exponent spreads the keys over the bins from the first pass
// (few LDS atomics on one bin), and a range below 2^24 takes two passes.
template <int KPT>
__device__ uint32_t reg_radix_select(const uint32_t (&kv)[KPT], uint32_t n, uint32_t rank,
                                     SelectLds& w)
{
    const int t = threadIdx.x;
    uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        if (j * kBlock >= n) break;                   // block-uniform: no key left
        if (t + j * kBlock < n) {
            lo = kv[j] < lo ? kv[j] : lo;
            hi = kv[j] > hi ? kv[j] : hi;
        }
    }
    for (int off = kWave / 2; off > 0; off >>= 1) {
        const uint32_t a = __shfl_xor(lo, off), b = __shfl_xor(hi, off);
        lo = a < lo ? a : lo;
        hi = b > hi ? b : hi;
    }
    if (lane_id() == 0) {
        w.scan[t / kWave] = lo;
        w.scan[kWavesPerBlock + t / kWave] = hi;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kWavesPerBlock; ++k) {
        lo = w.scan[k] < lo ? w.scan[k] : lo;
        hi = w.scan[kWavesPerBlock + k] > hi ? w.scan[kWavesPerBlock + k] : hi;
    }
    __syncthreads();
    const uint32_t range = hi - lo;
    if (range == 0u) return lo;                       // every key is the same
    const int bits = 32 - __clz(range);
    int s = bits > kRegDigit ? bits - kRegDigit : 0;  // lowest bit of this pass's digit
    int d = bits - s;                                 // its width (1..12)
    int sp = 0;                                       // lowest bit of the digits already chosen
    bool first = true;
    uint32_t sel = 0u;                                // u >> sp of the answer, once chosen
    for (;;) {
#pragma unroll
        for (int k = 0; k < kRegBins / (4 * kBlock); ++k)
            reinterpret_cast<uint4*>(w.hist)[t + k * kBlock] = make_uint4(0u, 0u, 0u, 0u);
        __syncthreads();
        const uint32_t dm = (1u << d) - 1u;
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            if (j * kBlock >= n) break;               // block-uniform: no key left
            const uint32_t u = kv[j] - lo;
            if (t + j * kBlock < n && (first || (u >> sp) == sel))
                atomicAdd(&w.hist[(u >> s) & dm], 1u);
        }
        __syncthreads();
        uint32_t bin, rin, cnt;
        find_rank_bucket<kRegBins>(w.hist, rank, w.scan, w.result, &bin, &rin, &cnt);
        sel = first ? bin : (sel << d) | bin;
        rank = rin;
        if (s == 0) break;
        first = false;
        sp = s;
        d = s > kRegDigit ? kRegDigit : s;
        s -= d;
    }
    return lo + sel;
}

// Logits of sampled rows for every query head of key head g.  The sample is
// made of 16-row blocks (one MFMA group each, contiguous in memory): sample
// index k covers row (k/16)*stride + k%16, k < m.  Output sample[b*hq + i][k]
// (row stride kSampleMax).
template <int D, int U, bool PAGED, bool FP8>
__global__ __launch_bounds__(kBlock) void sample_logits_kernel(SampleArgs a)
{
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int b = blockIdx.y / a.hk, g = blockIdx.y - b * a.hk;
    const int Gk = a.Gk;
    const int qh0 = b * a.hq + g * Gk;
    const int k0 = (blockIdx.x * kWavesPerBlock + wave) * 16 * U;   // first sample index
    if (k0 >= a.m) return;                                          // whole wave idle
    const uint16_t* qrow = col < Gk ? a.q + (int64_t)(qh0 + col) * D : nullptr;
    const QFrag<D> qf = FP8 ? load_qfrag_k8<D>(qrow) : load_qfrag<D>(qrow);
    const uint16_t* khead = a.k + ((int64_t)(b * a.hk + g) * a.cache_len) * D;
    const int64_t ctx_b = PAGED ? seq_ctx(a.pg, b, 0) : (a.lq > 1 ? a.ctx : INT64_MAX);
    KTile<D, U> kt;
    // Paged: every page-table read is issued before any K load (an index past
    // the table reads its last entry and the row is then dropped).
    int32_t page[U];
    if constexpr (PAGED) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int k = k0 + 16 * u + col;
            k = k < a.m ? k : a.m - 1;
            const int64_t pi = ((int64_t)(k >> 4) * a.stride + (k & 15)) / a.pg.page_rows;
            page[u] = a.pg.block_table[(int64_t)b * a.pg.max_pages +
                                       (pi < a.pg.max_pages ? pi : a.pg.max_pages - 1)];
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        int k = k0 + 16 * u + col;
        k = k < a.m ? k : a.m - 1;
        const int64_t row = (int64_t)(k >> 4) * a.stride + (k & 15);
        const uint16_t* p;
        bool ok = true;
        if constexpr (PAGED) {
            // Rows past the sequence, past the table or on a page outside the
            // pool load row 0 of page 0 (the pool holds at least one page)
            // and are zeroed.
            const int64_t P = a.pg.page_rows;
            ok = row < ctx_b && row / P < a.pg.max_pages && page[u] >= 0 && page[u] < a.pg.num_pages;
            p = (ok ? a.k + (((int64_t)page[u] * a.hk + g) * P + row % P) * D : a.k) + 8 * grp;
        } else if constexpr (FP8) {
            p = nullptr;
            const uint8_t* p8 = reinterpret_cast<const uint8_t*>(a.k) +
                                ((int64_t)(b * a.hk + g) * a.cache_len + row) * D + 16 * grp;
            widen_k8group<D>(load_k8group<D>(p8), kt.v[u]);
        } else {
            p = khead + row * D + 8 * grp;
        }
        if constexpr (!FP8) {
            // Loads without a branch: all of them in flight before the first wait.
#pragma unroll
            for (int mm = 0; mm < D / 32; ++mm) {
                const u32x4 x = ld16(p + 32 * mm);
                kt.v[u][mm] = ok ? x : u32x4{0u, 0u, 0u, 0u};
            }
        }
    }
    float s[U][4];
    qk_tile<D, U>(qf, kt, FP8 ? a.scale * a.k_scale[blockIdx.y] : a.scale, s);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int k = k0 + 16 * u + col;
        if (k >= a.m) continue;
        const int64_t row = (int64_t)(k >> 4) * a.stride + (k & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int slot = 4 * grp + i;
            // Rows past the sequence (paged) or past a later token's own
            // position (lq > 1) rank below every real logit.
            const int64_t lim = a.lq > 1 ? ctx_b - (a.lq - 1 - (g * Gk + slot) % a.lq) : ctx_b;
            if (slot < Gk)
                a.sample[(int64_t)(qh0 + slot) * kSampleMax + k] = row < lim ? s[u][i] : -INFINITY;
        }
    }
}

// pivot[row] = the k-th largest of the row's m sample logits.
__global__ __launch_bounds__(kBlock) void pivot_kernel(SampleArgs a)
{
    __shared__ SelectLds w;
    const int row = blockIdx.x;
    const float* s = a.sample + (int64_t)row * kSampleMax;
    int rank = a.rank;
    bool all = false;                                  // pivot -inf: every row is a candidate
    if (a.pg.block_table || a.lq > 1) {
        // Paged or several tokens: the sample and the rank follow this row's
        // own length.  The sample rows past it hold -inf, below every row
        // that counts.
        const int64_t cb = head_ctx(a.pg, a.lq, row / a.hq, row % a.hq, a.ctx);
        // Sampled rows below cb: block j holds samples 16j .. min(16j+16, m)-1
        // at rows j*stride + 0..15; one block per thread, then a block sum.
        int32_t part = 0;
        for (int j = threadIdx.x; 16 * j < a.m; j += kBlock) {
            const int64_t in_block = a.m - 16 * j < 16 ? a.m - 16 * j : 16;
            const int64_t v = cb - (int64_t)j * a.stride;
            part += (int32_t)(v < 0 ? 0 : (v > in_block ? in_block : v));
        }
        for (int off = kWave / 2; off > 0; off >>= 1) part += __shfl_xor(part, off);
        if (lane_id() == 0) w.scan[threadIdx.x / kWave] = (uint32_t)part;
        __syncthreads();
        int64_t mb = 0;
        for (int k = 0; k < kWavesPerBlock; ++k) mb += w.scan[k];
        __syncthreads();
        if ((int64_t)a.top_n >= cb || mb == 0) {
            all = true;
        } else if (mb == cb) {
            rank = a.top_n;
        } else {
            const double mu = (double)a.top_n * (double)mb / (double)cb;
            const double r = ceil(mu + 5.0 * sqrt(mu) + 5.0);
            rank = (int)(r < (double)mb ? r : (double)mb);
        }
    }
    // Unconditional loads (slots past m read sample 0 or m-1 again and are
    // masked by the select), all in flight before the first wait.
    constexpr int KPT = kSampleMax / kBlock;
    uint32_t kv[KPT];
    const int last = a.m > 0 ? a.m - 1 : 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const int k = threadIdx.x + j * kBlock;
        kv[j] = float_key(s[k < a.m ? k : last]);
    }
    const uint32_t key = reg_radix_select<KPT>(kv, (uint32_t)a.m, (uint32_t)rank, w);
    if (threadIdx.x == 0) {
        a.pivot[row] = all ? -INFINITY : key_float(key);
        if (a.group_flags) {
            const int b = row / a.hq;
            a.group_flags[b * a.hk + (row - b * a.hq) / a.Gk] = 0u;
        }
    }
}

// Exact N-th largest of one row by recomputing its logits (three radix passes
// over the row's key head, each with the shared QK tile).  Used when the
// candidate lists cannot answer.
template <int D, int U, bool PAGED, bool FP8>
__device__ uint32_t select_by_recompute(const FinalArgs& a, int row, int64_t ctx, SelectLds& w)
{
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int b = row / a.hq, i = row - b * a.hq;
    const int g = i / a.Gk, slot = i - g * a.Gk;
    const int qh0 = b * a.hq + g * a.Gk;
    const uint16_t* qrow = col < a.Gk ? a.q + (int64_t)(qh0 + col) * D : nullptr;
    const QFrag<D> qf = FP8 ? load_qfrag_k8<D>(qrow) : load_qfrag<D>(qrow);
    const uint16_t* khead = a.k + ((int64_t)(b * a.hk + g) * a.cache_len) * D;
    const uint8_t* khead8 = reinterpret_cast<const uint8_t*>(a.k) + ((int64_t)(b * a.hk + g) * a.cache_len) * D;
    const float sc = FP8 ? a.scale * a.k_scale[b * a.hk + g] : a.scale;
    uint32_t prefix = 0u, rank = a.top_n;
    for (int pass = 0; pass < 3; ++pass) {
        const int sh = digit_shift(pass);
        const uint32_t dm = digit_mask(pass), pm = prefix_mask(pass);
        for (int k = threadIdx.x; k < kHistBins; k += kBlock) w.hist[k] = 0u;
        __syncthreads();
        for (int64_t t0 = wave * 16 * U; t0 < ctx; t0 += kWavesPerBlock * 16 * U) {
            KTile<D, U> kt;
            if constexpr (PAGED) {
                // The tile lies in one page; a page outside the pool reads zeros.
                const int64_t base = page_base<D>(a.pg, b, g, a.hk, t0);
                const uint16_t* p = base < 0 ? nullptr
                                             : a.k + base + (t0 % a.pg.page_rows + col) * D + 8 * grp;
#pragma unroll
                for (int u = 0; u < U; ++u)
#pragma unroll
                    for (int m = 0; m < D / 32; ++m)
                        kt.v[u][m] = p ? ld16_stream(p + 16 * u * D + 32 * m) : u32x4{0u, 0u, 0u, 0u};
            } else if constexpr (FP8) {
                // Rows past ctx re-read the last row; they are skipped below.
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    int64_t r = t0 + 16 * u + col;
                    r = r < ctx ? r : ctx - 1;
                    widen_k8group<D>(load_k8group<D>(khead8 + r * D + 16 * grp), kt.v[u]);
                }
            } else {
                load_ktile<D, U>(kt, khead, t0, ctx);
            }
            float s[U][4];
            qk_tile<D, U>(qf, kt, sc, s);
            if (grp == (slot >> 2)) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    if (t0 + 16 * u + col >= ctx) continue;
                    float v = s[u][0];
#pragma unroll
                    for (int ii = 1; ii < 4; ++ii)
                        if ((slot & 3) == ii) v = s[u][ii];
                    const uint32_t key = float_key(v);
                    if ((key & pm) == prefix) atomicAdd(&w.hist[(key >> sh) & dm], 1u);
                }
            }
        }
        __syncthreads();
        uint32_t bin, rin, cnt;
        find_rank_bucket<kHistBins>(w.hist, rank, w.scan, w.result, &bin, &rin, &cnt);
        prefix |= bin << sh;
        rank = rin;
    }
    return prefix;
}

// Exact N-th largest of one row from candidate lists too long to stage
// (more than kFinalStage entries, at least N of them): three radix passes
// (11, 11, 10 bits) over the keys of every list entry, read from the lists
// on each pass.  `pre` holds the lists' entry offsets (pre[l] = entries before
// list l, pre[kMaxListsPerRow] = total).  Thread t takes EPT consecutive
// entries per round: one binary search over the offsets for the first, a
// forward walk for the rest.
template <int EPT>
__device__ uint32_t select_from_lists(const FinalArgs& a, int row, int nl, int64_t capw,
                                      const int32_t* pre, uint32_t total, SelectLds& w)
{
    uint32_t prefix = 0u, rank = a.top_n;
    for (int pass = 0; pass < 3; ++pass) {
        const int sh = digit_shift(pass);
        const uint32_t dm = digit_mask(pass), pm = prefix_mask(pass);
        for (int k = threadIdx.x; k < kHistBins; k += kBlock) w.hist[k] = 0u;
        __syncthreads();
        for (uint32_t base = 0; base < total; base += kBlock * EPT) {
            const uint32_t E0 = base + threadIdx.x * EPT;
            if (E0 < total) {
                int l0 = 0, hi = kMaxListsPerRow - 1;     // the last list starting at or before E0
                while (l0 < hi) {
                    const int mid = (l0 + hi + 1) >> 1;
                    if ((uint32_t)pre[mid] <= E0) l0 = mid;
                    else hi = mid - 1;
                }
                uint32_t kv[EPT];
#pragma unroll
                for (int k = 0; k < EPT; ++k) {
                    const uint32_t E = E0 + k < total ? E0 + k : total - 1;
                    while ((uint32_t)pre[l0 + 1] <= E) ++l0;   // skips empty lists; stops below the last
                    kv[k] = a.entries[list_index(row, l0, E - (uint32_t)pre[l0], capw, nl,
                                                 a.head_stride, a.overflow_at)].y;
                }
#pragma unroll
                for (int k = 0; k < EPT; ++k) {
                    const uint32_t key = float_key(__uint_as_float(kv[k]));
                    if (E0 + k < total && (key & pm) == prefix)
                        atomicAdd(&w.hist[(key >> sh) & dm], 1u);
                }
            }
        }
        __syncthreads();
        uint32_t bin, rin, cnt;
        find_rank_bucket<kHistBins>(w.hist, rank, w.scan, w.result, &bin, &rin, &cnt);
        prefix |= bin << sh;
        rank = rin;
    }
    return prefix;
}

template <int D, int U, bool PAGED, bool FP8>
__global__ __launch_bounds__(kBlock) void refresh_final_kernel(FinalArgs a)
{
    __shared__ int32_t pre[kMaxListsPerRow + 1];
    __shared__ uint32_t own[kFinalStage];
    __shared__ SelectLds w;
    const int row = blockIdx.x, t = threadIdx.x;
    const int64_t ctx = head_ctx(a.pg, a.lq, row / a.hq, row % a.hq, a.ctx);
    // Paged caches with a work split from the lengths: the lists of this
    // sequence's chunks only, from the K stream's plan.
    const bool plan = PAGED && a.pg.plan_cap != 0;
    const int64_t rpc = plan ? a.pg.plan[0] : a.rows_per_chunk;
    const int nl = a.chunks * kWavesPerBlock;
    const int nlv = plan ? a.pg.plan[1 + row / a.hq] * kWavesPerBlock : nl;
    if ((int64_t)a.top_n >= ctx) {                     // N covers the row: keep everything
        if (t == 0) a.tau[row] = -INFINITY;
        return;
    }
    const int64_t capw = rpc / kWavesPerBlock;

    // Prefix of list lengths: thread t sums a contiguous run of lists.
    constexpr int PER = kMaxListsPerRow / kBlock;
    int32_t c[PER], sum = 0;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int l = t * PER + k;
        c[k] = l < nlv ? a.list_count[(int64_t)row * nl + l] : 0;
        sum += c[k];
    }
    int32_t run = block_scan(sum, reinterpret_cast<int32_t*>(w.scan)) - sum;
    int32_t first[PER];                  // first entry of each of this thread's lists
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        first[k] = run;
        pre[t * PER + k] = run;
        run += c[k];
    }
    if (t == kBlock - 1) pre[kMaxListsPerRow] = run;
    __syncthreads();
    const uint32_t total = (uint32_t)pre[kMaxListsPerRow];

    uint32_t key;
    if (total >= a.top_n && total <= (uint32_t)kFinalStage) {
        // The list of every entry, with no search: each non-empty list marks
        // its first entry with its index, and an inclusive max-scan over the
        // marks (runs of `per` entries per thread) carries it to the entries
        // that follow.
        for (uint32_t E = t; E < total; E += kBlock) own[E] = 0u;
        __syncthreads();
#pragma unroll
        for (int k = 0; k < PER; ++k)
            if (c[k] > 0) own[first[k]] = (uint32_t)(t * PER + k);
        __syncthreads();
        constexpr int KPT = kFinalStage / kBlock;
        const uint32_t per = (total + kBlock - 1) / kBlock;   // <= KPT
        const uint32_t r0 = min(t * per, total), r1 = min(r0 + per, total);
        uint32_t mk[KPT];
        uint32_t m = 0u;
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            if ((uint32_t)j >= per) break;                   // block-uniform
            mk[j] = r0 + j < r1 ? own[r0 + j] : 0u;
            m = max(m, mk[j]);
        }
        uint32_t runmax = block_scan_max_excl(m, w.scan);
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            if ((uint32_t)j >= per) break;
            runmax = max(runmax, mk[j]);
            if (r0 + j < r1) own[r0 + j] = runmax;
        }
        __syncthreads();
        // Load the candidates into registers (coalesced: entry t + k * kBlock
        // of thread t).  No branches: a slot past the end reads the last
        // entry again and is masked by the select, so every LDS read and
        // load is issued before any of them is waited for.
        uint32_t l[KPT], off[KPT], kv[KPT];
#pragma unroll
        for (int k = 0; k < KPT; ++k) {
            if (k * kBlock >= (int)total) break;             // block-uniform
            const uint32_t E = t + k * kBlock;
            off[k] = E < total ? E : total - 1;
            l[k] = own[off[k]];
        }
#pragma unroll
        for (int k = 0; k < KPT; ++k)
            if (k * kBlock < (int)total) off[k] -= (uint32_t)pre[l[k]];
#pragma unroll
        for (int k = 0; k < KPT; ++k)
            if (k * kBlock < (int)total)
                kv[k] = a.entries[list_index(row, l[k], off[k], capw, nl, a.head_stride,
                                             a.overflow_at)].y;
#pragma unroll
        for (int k = 0; k < KPT; ++k)
            if (k * kBlock < (int)total) kv[k] = float_key(__uint_as_float(kv[k]));
        key = reg_radix_select<KPT>(kv, total, a.top_n, w);
    } else if (total >= a.top_n) {
        // The lists are complete (every logit >= the pivot) but too long to
        // stage: select over them in place, no K traffic.
        key = select_from_lists<8>(a, row, nl, capw, pre, total, w);
    } else {
        key = select_by_recompute<D, U, PAGED, FP8>(a, row, ctx, w);
        // The lists miss entries of this row: a fused decode must re-stream its group.
        if (t == 0 && a.group_flags) {
            const int b = row / a.hq;
            a.group_flags[b * a.hk + (row - b * a.hq) / a.Gk] = 1u;
        }
    }
    if (t == 0) a.tau[row] = key_float(key);
}

}  // namespace

hipError_t launch_sample(int D, const SampleArgs& a, hipStream_t s)
{
    constexpr int U = 4;
    const int per_block = kWavesPerBlock * 16 * U;
    const dim3 grid((a.m + per_block - 1) / per_block, a.B * a.hk);
    const int kind = a.pg.block_table != nullptr ? 1 : (a.k_scale != nullptr ? 2 : 0);
#define SAGA_LAUNCH_SAMPLE(DD, PG, F8)                                                            \
    hipLaunchKernelGGL((sample_logits_kernel<DD, U, PG, F8>), grid, dim3(kBlock), 0, s, a)
    if (D == 32) {
        if (kind == 2) return hipErrorInvalidValue;      // no fp8 K at head_dim 32 (the API rejects it)
        if (kind == 1) SAGA_LAUNCH_SAMPLE(32, true, false);
        else SAGA_LAUNCH_SAMPLE(32, false, false);
    } else if (D == 64) {
        if (kind == 1) SAGA_LAUNCH_SAMPLE(64, true, false);
        else if (kind == 2) SAGA_LAUNCH_SAMPLE(64, false, true);
        else SAGA_LAUNCH_SAMPLE(64, false, false);
    } else {
        if (kind == 1) SAGA_LAUNCH_SAMPLE(128, true, false);
        else if (kind == 2) SAGA_LAUNCH_SAMPLE(128, false, true);
        else SAGA_LAUNCH_SAMPLE(128, false, false);
    }
#undef SAGA_LAUNCH_SAMPLE
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(pivot_kernel, dim3(a.B * a.hq), dim3(kBlock), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_refresh_final(int D, const FinalArgs& a, hipStream_t s)
{
    const int kind = a.pg.block_table != nullptr ? 1 : (a.k_scale != nullptr ? 2 : 0);
#define SAGA_LAUNCH_FINAL(DD, PG, F8)                                                             \
    hipLaunchKernelGGL((refresh_final_kernel<DD, decode_unroll(DD), PG, F8>), dim3(a.B * a.hq),    \
                       dim3(kBlock), 0, s, a)
    if (D == 32) {
        if (kind == 2) return hipErrorInvalidValue;      // no fp8 K at head_dim 32 (the API rejects it)
        if (kind == 1) SAGA_LAUNCH_FINAL(32, true, false);
        else SAGA_LAUNCH_FINAL(32, false, false);
    } else if (D == 64) {
        if (kind == 1) SAGA_LAUNCH_FINAL(64, true, false);
        else if (kind == 2) SAGA_LAUNCH_FINAL(64, false, true);
        else SAGA_LAUNCH_FINAL(64, false, false);
    } else {
        if (kind == 1) SAGA_LAUNCH_FINAL(128, true, false);
        else if (kind == 2) SAGA_LAUNCH_FINAL(128, false, true);
        else SAGA_LAUNCH_FINAL(128, false, false);
    }
#undef SAGA_LAUNCH_FINAL
    return hipGetLastError();
}

}  // namespace saga

// decode.hip -- SAGA Atop-N decode step: (1) K stream with the threshold
// mask and wave-ballot compaction, (2) masked softmax with the sparse value
// gather, either in the K stream's tail (large batches) or as a kernel of its
// own over the selection lists, (3) split-sequence combine (shared with the
// full-attention path).
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
//   threshold, and compacts the hits with ballot + mbcnt into wave-private
//   LDS queues, flushed when full to per-(b, query head, chunk, wave) lists
//   of (row, logit) in the workspace.  The list path then writes each list's
//   length and largest logit for gather_kernel; with GKT > 0 the workgroup
//   instead gathers its own chunk's value rows in its tail (tail_gather) and
//   writes one partial per (b, query head, chunk).
// gather_kernel: one workgroup per (b, query head, segment of its entries).
//   Reads its lists' lengths and maxima, stages the entries in LDS with their
//   softmax weights exp(s - M) (M = the segment's largest selected logit),
//   then gathers the selected rows of the query head's value head with
//   16-byte loads, many rows in flight per lane, accumulating in fp32.
//   One (M, l, count, o) partial per (b, query head, segment).
// combine_kernel merges the partials in segment (or chunk) order.
// Every sum runs in a fixed order and no float atomics are used, so results
// are bit-identical run to run.
#include "kernels.hpp"

namespace saga {

namespace {

// Value gather in the K stream's tail (large batches; contiguous bf16 V with
// d_v = d_k).  The workgroup has just written its chunk's selected entries
// to its lists (one per head slot and wave) and knows each wave's counts and
// largest logits, so it gathers their value rows itself: no gather launch,
// no list-length prologue, and workgroups whose stream ends early gather
// while the others still stream.
//   Order: the chunk's entries are taken in one flat order, head slot first,
//   then wave, then list position, and staged in LDS (byte offset of the
//   value row in the group's value heads with the head slot in its low four
//   bits, weight exp(s - M_h), M_h the slot's largest selected logit in this
//   chunk), at most CAPL per round.  Wave w takes the w-th quarter of each
//   round in order, C lanes per value row, NB rows in flight per lane, and
//   keeps one running sum for the head slot it is in; where the slot changes
//   it sums its lanes' rows (fixed butterfly) and adds them to its own
//   (wave, slot) partial in LDS.  So a head slot that selected many rows is
//   spread over all four waves, every sum has a fixed order, and results are
//   bit-reproducible.  The four waves' partials are added in wave order into
//   one partial per (b, query head, chunk), merged by combine_kernel.
// GKT: most head slots a key group may have (8 or 16; at 16 the (wave, slot)
// partials fill half of the queues' 32 KB at d = 64 and all of it at d = 128).
// V8: an fp8 E4M3 value cache (d bytes per row, one scale per (b, value
// head)): each lane loads 16 codes and widens them exactly, and a head slot's
// partial is multiplied by its value head's scale once.
template <int D, int GKT, bool V8>
// qe/qp: the wave's last queue entries (block k of queue i in lane order,
// x = ~0u where the queue ends) and their list positions; `flushed`: the wave
// wrote entries to its lists earlier in the stream.
__device__ __forceinline__ void tail_gather(const SelectStreamArgs& a, unsigned char* qlds,
                                            const int (&written)[16],
                                            const uint2 (&qe)[4][4], const int (&qp)[4][4],
                                            bool flushed, const float (&mx)[4], int b, int g,
                                            int chunk, int64_t r0, int qh0, int64_t capw,
                                            int64_t nl, int wave, int lane)
{
    constexpr int VB = V8 ? 1 : 2;            // bytes per value element
    constexpr int EPL = 16 / VB;              // elements per lane load (16 bytes)
    constexpr int C = D / EPL;                // 16-byte pieces of a value row
    constexpr int SLW = kWave / C;            // value rows per wave load instruction
    // Value rows in flight per lane.  An fp8 row is half as wide, so a wave
    // load covers twice the rows; the fp8 count keeps the kernel within the
    // 128 VGPRs that the four workgroups per CU of the fp8 K launch need.
    constexpr int NB = V8 ? SAGA_TAIL_NB_V8 : (D == 128 ? SAGA_TAIL_NB128 : SAGA_TAIL_NB);
    constexpr uint32_t kNoRow = 0x80000000u;  // past the value heads (< 2^31 bytes, host-checked)
    constexpr size_t kPartFloats = (size_t)kWavesPerBlock * GKT * D;
    constexpr size_t kPartBytes = kPartFloats * 4;
    constexpr size_t kQueueBytes = sizeof(uint2) * kWavesPerBlock * 4 * kQueueCap;
    // Entries staged per round: the queues' LDS left after the partials (3072
    // at d = 64 with 8 head slots, 2048 with 16), else 2048 in LDS of their own.
    constexpr int kLeft = (int)((kQueueBytes - kPartBytes) / 8 / kBlock * kBlock);
    constexpr int CAPL = kLeft >= 2048 ? kLeft : 2048;
    constexpr int EPT = CAPL / kBlock;
    static_assert(kPartBytes <= kQueueBytes, "the (wave, slot) partials live in the queues' LDS");
    __shared__ int32_t tcnt[kWavesPerBlock][16];
    __shared__ float tmx[kWavesPerBlock][16];
    __shared__ int32_t tpre[4 * 16 + 1];      // flat start of list (head slot, wave)
    __shared__ float tM[16];
    __shared__ float wl[kWavesPerBlock * GKT];   // (wave, slot) weight sums
    __shared__ int32_t tfl[kWavesPerBlock + 1];  // waves that flushed; [4]: stage directly
    // The stream's queues (no longer used) hold the (wave, slot) partials and,
    // when they fit, the staged entries too.
    constexpr bool kStageInQueue = kPartBytes + CAPL * 8 <= kQueueBytes;
    __shared__ uint2 extra[kStageInQueue ? 1 : CAPL];
    float* wpart = reinterpret_cast<float*>(qlds);          // [wave][GKT][D]
    uint2* stage = kStageInQueue ? reinterpret_cast<uint2*>(qlds + kPartBytes) : extra;
    const int Gk = a.Gk;
    const int col = lane & 15, grp = lane >> 4;

#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float m = group16_max(mx[i]);
        if (col == 0) tmx[wave][4 * grp + i] = m;
    }
    if (lane < 16) {
        int32_t c = 0;
#pragma unroll
        for (int h = 0; h < 16; ++h) c = lane == h ? written[h] : c;
        tcnt[wave][lane] = c;
    }
    if (lane == 0) tfl[wave] = flushed ? 1 : 0;
    __syncthreads();                           // every wave's queue is in its registers
    for (int i = threadIdx.x; i < (int)kPartFloats; i += kBlock) wpart[i] = 0.f;
    if (threadIdx.x < kWavesPerBlock * GKT) wl[threadIdx.x] = 0.f;
    if (wave == 0) {
        const int h = lane >> 2, w = lane & 3;
        const int32_t n = h < Gk ? tcnt[w][h] : 0;
        int32_t incl = n;
        for (int off = 1; off < kWave; off <<= 1) {
            const int32_t u = __shfl_up(incl, off);
            if (lane >= off) incl += u;
        }
        tpre[lane] = incl - n;
        if (lane == kWave - 1) {
            tpre[64] = incl;
            // The whole chunk's entries are still in the waves' registers and
            // fit one staging round: stage them from there.
            tfl[kWavesPerBlock] = (tfl[0] | tfl[1] | tfl[2] | tfl[3]) == 0 && incl <= CAPL;
        }
        if (lane < 16)
            tM[lane] = fmaxf(fmaxf(tmx[0][lane], tmx[1][lane]), fmaxf(tmx[2][lane], tmx[3][lane]));
    }
    __syncthreads();
    const int32_t total = tpre[64];
    const bool direct = tfl[kWavesPerBlock] != 0;

    // Value heads of this key group's query heads (virtual heads when lq > 1).
    const int vi0 = g * Gk;
    const int nu0 = vi0 / a.Gv;
    const int nvh = (vi0 + Gk - 1) / a.Gv - nu0 + 1;
    const unsigned char* vb = reinterpret_cast<const unsigned char*>(a.v);
    const __amdgpu_buffer_rsrc_t vrs =
        make_rsrc(vb + ((int64_t)(b * a.hv + nu0) * a.cache_len) * D * VB,
                  (uint32_t)((int64_t)nvh * a.cache_len * D * VB));
    const int t = threadIdx.x, c = lane % C, sl = lane / C;
    float cur[EPL], ls = 0.f;
#pragma unroll
    for (int j = 0; j < EPL; ++j) cur[j] = 0.f;
    int hc = -1;                               // the wave's current head slot
    auto flush = [&](int h) {
#pragma unroll
        for (int off = C; off < kWave; off <<= 1) {
#pragma unroll
            for (int j = 0; j < EPL; ++j) cur[j] += __shfl_xor(cur[j], off);
            ls += __shfl_xor(ls, off);
        }
        if (sl == 0) {
            float* dst = wpart + (wave * GKT + h) * D + EPL * c;
#pragma unroll
            for (int j = 0; j < EPL; ++j) dst[j] += cur[j];
            if (c == 0) wl[wave * GKT + h] += ls;
        }
#pragma unroll
        for (int j = 0; j < EPL; ++j) cur[j] = 0.f;
        ls = 0.f;
    };

    const int64_t local0 = (int64_t)chunk * kWavesPerBlock + wave;   // this wave's lists
    if (direct) {
        // Each lane stages its own entries at their flat places.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint2 e = qe[i][k];
                if (e.x != ~0u) {
                    const int h = 4 * (int)((e.x & 15u) >> 2) + i;
                    const int f = tpre[4 * h + wave] + qp[i][k];
                    const uint32_t nrel = (uint32_t)((vi0 + h) / a.Gv - nu0);
                    const uint32_t row = (uint32_t)(r0 + (e.x >> 4));
                    const uint32_t off = (nrel * (uint32_t)a.cache_len + row) * (uint32_t)(D * VB);
                    stage[f] = make_uint2(off | (uint32_t)h,
                                          __float_as_uint(__expf(__uint_as_float(e.y) - tM[h])));
                }
            }
        }
    } else {
        // Store them to the lists, after the entries flushed earlier.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint2 e = qe[i][k];
                if (e.x != ~0u)
                    a.entries[list_index(qh0 + 4 * (int)((e.x & 15u) >> 2) + i, local0,
                                         (uint32_t)qp[i][k], capw, nl, a.head_stride,
                                         a.overflow_at)] = make_uint2(e.x >> 4, e.y);
            }
        }
        __syncthreads();                       // every wave's lists are complete
    }
    for (int32_t base = 0; base < total; base += CAPL) {
        const int n = min(CAPL, total - base);
        // Stage entries t, t + 256, ...: list by binary search over the flat
        // starts, all loads in flight before any is used.
        if (!direct) {
        uint2 ent[EPT];
        int lst[EPT];
#pragma unroll
        for (int k = 0; k < EPT; ++k) {
            const int32_t f = base + min(t + k * kBlock, n - 1);
            int l = 0;
#pragma unroll
            for (int st = 32; st > 0; st >>= 1) l = tpre[l + st] <= f ? l + st : l;
            lst[k] = l;
            ent[k] = a.entries[list_index(qh0 + (l >> 2), (int64_t)chunk * kWavesPerBlock + (l & 3),
                                          (uint32_t)(f - tpre[l]), capw, nl, a.head_stride,
                                          a.overflow_at)];
        }
#pragma unroll
        for (int k = 0; k < EPT; ++k) {
            const int e = t + k * kBlock;
            if (e < n) {
                const int h = lst[k] >> 2;
                const uint32_t nrel = (uint32_t)((vi0 + h) / a.Gv - nu0);
                const uint32_t row = (uint32_t)(r0 + ent[k].x);
                const uint32_t off = (nrel * (uint32_t)a.cache_len + row) * (uint32_t)(D * VB);
                stage[e] = make_uint2(off | (uint32_t)h,
                                      __float_as_uint(__expf(__uint_as_float(ent[k].y) - tM[h])));
            }
        }
        }
        __syncthreads();
        const int e_lo = wave * n / kWavesPerBlock, e_hi = (wave + 1) * n / kWavesPerBlock;
        for (int e0 = e_lo; e0 < e_hi; e0 += SLW * NB) {
            const int e_last = min(e0 + SLW * NB, e_hi) - 1;
            const int h_first = __builtin_amdgcn_readfirstlane((int)(stage[e0].x & 15u));
            const int h_last = __builtin_amdgcn_readfirstlane((int)(stage[e_last].x & 15u));
            u32x4 vv[NB];
            float w[NB];
            int hh[NB];
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                const int e = e0 + k * SLW + sl;
                const bool in = e <= e_last;
                const uint2 st = stage[in ? e : e_last];
                hh[k] = (int)(st.x & 15u);
                w[k] = in ? __uint_as_float(st.y) : 0.f;
                vv[k] = buf_ld16(vrs, (in ? (st.x & ~15u) : kNoRow) + 16u * c);
            }
            for (int h = h_first; h <= h_last; ++h) {
                if (h != hc) {
                    if (hc >= 0) flush(hc);
                    hc = h;
                }
#pragma unroll
                for (int k = 0; k < NB; ++k) {
                    const bool m = hh[k] == h;
                    ls += m ? w[k] : 0.f;
                    if constexpr (V8) {
                        // Codes 0-7 then 8-15 of the lane's 16, widened in order.
                        const u32x4 x0 = fp8x8_to_bf16x8(u32x2{vv[k][0], vv[k][1]});
                        const u32x4 x1 = fp8x8_to_bf16x8(u32x2{vv[k][2], vv[k][3]});
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            cur[2 * q] = m ? fmaf(w[k], bf16lo(x0[q]), cur[2 * q]) : cur[2 * q];
                            cur[2 * q + 1] = m ? fmaf(w[k], bf16hi(x0[q]), cur[2 * q + 1]) : cur[2 * q + 1];
                            cur[8 + 2 * q] = m ? fmaf(w[k], bf16lo(x1[q]), cur[8 + 2 * q]) : cur[8 + 2 * q];
                            cur[9 + 2 * q] = m ? fmaf(w[k], bf16hi(x1[q]), cur[9 + 2 * q]) : cur[9 + 2 * q];
                        }
                    } else {
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            cur[2 * q] = m ? fmaf(w[k], bf16lo(vv[k][q]), cur[2 * q]) : cur[2 * q];
                            cur[2 * q + 1] = m ? fmaf(w[k], bf16hi(vv[k][q]), cur[2 * q + 1]) : cur[2 * q + 1];
                        }
                    }
                }
            }
        }
        __syncthreads();                       // the stage is rewritten by the next round
    }
    if (hc >= 0) flush(hc);
    __syncthreads();

    const int64_t prow0 = (int64_t)qh0 * a.chunks + chunk;   // partial of head slot 0
    for (int idx = t; idx < Gk * D; idx += kBlock) {
        const int h = idx / D, p = idx - h * D;
        float o = 0.f;
#pragma unroll
        for (int w = 0; w < kWavesPerBlock; ++w) o += wpart[(w * GKT + h) * D + p];
        if constexpr (V8) o *= a.v_scale[b * a.hv + (vi0 + h) / a.Gv];
        a.part.o[(prow0 + (int64_t)h * a.chunks) * D + p] = o;
    }
    if (t < Gk) {
        float l = 0.f;
#pragma unroll
        for (int w = 0; w < kWavesPerBlock; ++w) l += wl[w * GKT + t];
        const int32_t nh = tpre[4 * t + 4] - tpre[4 * t];
        const int64_t pi = prow0 + (int64_t)t * a.chunks;
        a.part.m[pi] = nh > 0 ? tM[t] : -INFINITY;
        a.part.l[pi] = l;
        a.part.c[pi] = nh;
    }
}

// Stream-select kernel.  Hits are compacted with one ballot per (16-row
// group u, head index i): the four lane groups' hits for head slots 4*g + i
// go to one wave-private LDS queue per i in ballot order, so the queue length
// stays wave-uniform (scalar registers) and each hit costs one mbcnt.  When a
// queue could overflow, it is split by head slot and appended to the global
// per-(head, chunk, wave) lists in order.  DEBUG adds the optional logits and
// selection-bitmap outputs.
template <int D, int U, bool DEBUG, bool PAGED, bool FP8, int GKT, bool V8>
__global__ __launch_bounds__(kBlock) SAGA_STREAM_ATTR void select_stream_kernel(SelectStreamArgs a)
{
    __shared__ uint2 queue[kWavesPerBlock][4][kQueueCap];
    // The wave index is uniform within a wave; saying so keeps the row
    // bookkeeping and the loop exit scalar (a vector loop exit makes the
    // compiler wait for every K load in flight on each trip).
    const int lane = lane_id(), wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15, grp = lane >> 4;
    int chunk = blockIdx.x;
    int b = blockIdx.y / a.hk, g = blockIdx.y - b * a.hk;
    const int Gk = a.Gk;
    // Paged caches with a work split from the lengths: this call's rows per
    // chunk (the same in every kernel of the call) and this workgroup's work
    // item (a 1-D launch, see paged_item); the LDS of the queues, not yet in
    // use, serves the block reductions.
    int64_t rpc = a.rows_per_chunk;
    if constexpr (PAGED) {
        if (a.pg.plan_cap && a.B <= kWave) {
            // Every wave computes the plan on its own (no LDS, no barrier).
            const uint32_t len = plan_len(a.pg, lane, a.B, a.ctx);
            rpc = paged_rows_per_chunk_wave(a.pg, a.B, a.hk, len);
            if (blockIdx.x == 0 && wave == 0) {   // the plan, for the kernels after this one
                if (lane < a.B) a.pg.plan[1 + lane] = (int32_t)((len + (uint32_t)rpc - 1) / (uint32_t)rpc);
                if (lane == 0) a.pg.plan[0] = (int32_t)rpc;
            }
            if (!paged_item_wave(a.hk, rpc, len, blockIdx.x, &b, &g, &chunk))
                return;                                                // whole workgroup
        } else if (a.pg.plan_cap) {
            int64_t* red = reinterpret_cast<int64_t*>(&queue[0][0][0]);
            const uint32_t len0 = plan_len(a.pg, threadIdx.x, a.B, a.ctx);
            rpc = paged_rows_per_chunk(a.pg, a.B, a.hk, a.ctx, len0, red);
            if (blockIdx.x == 0) {           // the plan, for the gather and threshold kernels
                const uint32_t r32 = (uint32_t)rpc;
                for (int s = threadIdx.x; s < a.B; s += kBlock) {
                    const uint32_t c = s < kBlock ? len0 : plan_len(a.pg, s, a.B, a.ctx);
                    a.pg.plan[1 + s] = (int32_t)((c + r32 - 1) / r32);
                }
                if (threadIdx.x == 0) a.pg.plan[0] = (int32_t)rpc;
            }
            if (!paged_item(a.pg, a.B, a.hk, a.ctx, rpc, len0, blockIdx.x, red, &b, &g, &chunk))
                return;                                                // whole workgroup
        }
    }
    const int bg = b * a.hk + g;
    const int64_t r0 = (int64_t)chunk * rpc;
    const int64_t ctx_b = PAGED ? seq_ctx(a.pg, b, a.ctx) : a.ctx;
    const int64_t r1 = wave_uniform(min(r0 + rpc, ctx_b));
    const int64_t capw = rpc / kWavesPerBlock;
    const int qh0 = b * a.hq + g * Gk;
    uint2 (*q4)[kQueueCap] = queue[wave];
    if (a.group_flags && a.group_flags[bg] == 0u) return;   // whole workgroup

    const uint16_t* qrow = col < Gk ? a.q + (int64_t)(qh0 + col) * D : nullptr;
    const QFrag<D> qf = FP8 ? load_qfrag_k8<D>(qrow) : load_qfrag<D>(qrow);
    // Logit scale; an fp8 K cache adds its (b, key head) scale.
    const float sc = FP8 ? a.scale * a.k_scale[bg] : a.scale;
    float tau[4], mx[4];
    int64_t lim[4];          // rows of this lane's head slots: r1, or less for later tokens
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int slot = 4 * grp + i;
        tau[i] = slot < Gk ? a.tau[qh0 + slot] : INFINITY;
        mx[i] = -INFINITY;
        const int64_t hc = a.lq > 1 ? head_ctx(a.pg, a.lq, b, g * Gk + slot, a.ctx) : r1;
        lim[i] = hc < r1 ? hc : r1;
    }
    // Wave-uniform bookkeeping: entries waiting in queue i, entries already in
    // the global list of head slot h.
    int qn[4] = {0, 0, 0, 0};
    int written[16];
#pragma unroll
    for (int h = 0; h < 16; ++h) written[h] = 0;
    const int64_t nl = (int64_t)a.chunks * kWavesPerBlock;          // lists per row
    const int64_t local = chunk * kWavesPerBlock + wave;               // this wave's list
    const int64_t list0 = (int64_t)qh0 * nl + local;
    const int64_t list_stride = nl;                                    // between head slots

    // Split every queue by head slot (4*gs + i) and append to the global lists.
    auto flush_all = [&]() {
        wave_sync();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            for (int base = 0; base < qn[i]; base += kWave) {
                const bool have = base + lane < qn[i];
                const uint2 e = have ? q4[i][base + lane] : make_uint2(0u, 0u);
                const int gs = (e.x & 15) >> 2;                 // head slot 4*gs + i
                // Each lane finds its own list and position, so one store
                // writes the whole batch whatever the mix of head slots.
                int pos = 0;
#pragma unroll
                for (int g2 = 0; g2 < 4; ++g2) {
                    const uint64_t m = __ballot(have && gs == g2);
                    if (gs == g2) pos = written[4 * g2 + i] + (int)lanes_below(m);
                    written[4 * g2 + i] += __popcll(m);
                }
                if (have)
                    a.entries[list_index(qh0 + 4 * gs + i, local, (uint32_t)pos, capw, nl,
                                         a.head_stride, a.overflow_at)] = make_uint2(e.x >> 4, e.y);
            }
            qn[i] = 0;
        }
        wave_sync();
        // Let the stores finish (vmcnt(0)) before leaving this rare path: the
        // code after it then starts from a known-empty store state, and the
        // compiler needs no full wait on the common path where the merged
        // state would otherwise be unknown (it would drain the K prefetch).
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    };

    // A tile adds at most 64*U entries to a queue: flush before one can overflow.
    auto maybe_flush = [&]() {
        // Four scalar compares: no vector temporaries that could alias the
        // registers of a K tile still in flight (that would force a wait).
        constexpr int lim = kQueueCap - kWave * U;
        if (((lim - qn[0]) | (lim - qn[1]) | (lim - qn[2]) | (lim - qn[3])) < 0) flush_all();
    };

    // One 16-row group starting at row g0 (a multiple of 16).
    auto process_group = [&](const u32x4 (&kv)[D / 32], int64_t g0) {
        {
            float s[4];
            qk_group<D>(qf, kv, sc, s);
            const int64_t row = g0 + col;
            const bool valid = row < r1;
            const uint32_t tag = (uint32_t)(row - r0) << 4;
            if constexpr (DEBUG) {
                if (a.logits_out && valid) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (4 * grp + i < Gk)
                            a.logits_out[(int64_t)(qh0 + 4 * grp + i) * a.ctx + row] = s[i];
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool pred = row < lim[i] && s[i] >= tau[i];
                const uint64_t mask = __ballot(pred);
                if (pred)
                    q4[i][qn[i] + lanes_below(mask)] =
                        make_uint2(tag | (uint32_t)(4 * grp + i), __float_as_uint(s[i]));
                qn[i] += __popcll(mask);
                mx[i] = fmaxf(mx[i], pred ? s[i] : -INFINITY);
                if constexpr (DEBUG) {
                    const uint32_t mine = (uint32_t)(mask >> (16 * grp)) & 0xffffu;
                    if (a.bitmap && col == 0 && mine)
                        atomicOr(a.bitmap + (int64_t)(qh0 + 4 * grp + i) * a.bitmap_words + g0 / 32,
                                 mine << (g0 & 31));
                }
            }
        }
    };
    auto process = [&](const KTile<D, U>& kt, int64_t t0) {
#pragma unroll
        for (int u = 0; u < U; ++u) process_group(kt.v[u], t0 + 16 * u);
    };
    // fp8 tile: each group is widened to bf16 just before its MFMA.
    auto process8 = [&](const K8Tile<D, U>& kt, int64_t t0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            u32x4 kv[D / 32];
            widen_k8group<D>(kt.g[u], kv);
            process_group(kv, t0 + 16 * u);
        }
    };

    // Software-pipelined stream: the next tile's loads are issued before the
    // current tile is processed, so every wave keeps a tile in flight.  The
    // buffer resource ends at this chunk's last row r1: prefetches past it
    // return zeros without touching memory, so every prefetch is issued
    // unconditionally and the load counters stay the same on every path (a
    // conditional prefetch makes the compiler wait for it before the current
    // tile).  Queue flushes (the only global stores) happen before a prefetch.
    constexpr int64_t kStep = kWavesPerBlock * 16 * U;
    if constexpr (PAGED) {
        // Paged K: a tile pair (2 * kStep rows, pair starts aligned to it) lies
        // in one page (page_rows is a multiple of the pair).  The page and the
        // pair's byte offset in it advance incrementally (one division per
        // workgroup), each page gets a buffer resource that ends at r1 or at
        // the page end, a table entry outside the pool gives an empty resource
        // (zeros), and the next page's table entry is read one page ahead.
        static_assert(kPageQuantum % (2 * kStep) == 0, "a tile pair must not straddle pages");
        const int64_t P = a.pg.page_rows;
        const uint32_t page_bytes = (uint32_t)(P * D * 2);   // < 2^31 (checked on the host)
        auto lookup = [&](int64_t p) -> int64_t {             // element offset, or -1
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
        int64_t tp = r0;                                // first row of the current pair
        if (tp < r1) {
            int64_t pi = tp / P;                        // page of the current pair
            uint32_t in = (uint32_t)(tp - pi * P) * (uint32_t)(D * 2);   // its byte offset there
            __amdgpu_buffer_rsrc_t ra = page_rsrc(pi, lookup(pi));
            int64_t base_n = lookup(pi + 1);
            KTile<D, U> ka, kb;
            load_ktile_at<D, U>(ka, ra, lane_off + in);
            do {
                maybe_flush();
                load_ktile_at<D, U>(kb, ra, lane_off + in + kStepBytes);
                process(ka, tp + wave * 16 * U);
                in += 2 * kStepBytes;
                if (in == page_bytes) {                 // the next pair opens a new page
                    in = 0;
                    ++pi;
                    ra = page_rsrc(pi, base_n);
                    base_n = lookup(pi + 1);
                }
                maybe_flush();
                load_ktile_at<D, U>(ka, ra, lane_off + in);
                process(kb, tp + kStep + wave * 16 * U);
                tp += 2 * kStep;
            } while (tp < r1);
        }
    } else if constexpr (FP8) {
        // fp8 K (one byte per element): the same pipeline on half the bytes,
        // 16-byte loads in the permuted order of the fp8 helpers, each group
        // widened to bf16 just before its MFMA.
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
                maybe_flush();
                load_k8tile_at<D, U>(kb, khead, koff + kStepBytes);
                process8(ka, t0);
                maybe_flush();
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
        // This lane's byte offset in tile t0, advanced one tile pair per trip.
        constexpr uint32_t kStepBytes = (uint32_t)(kStep * D * 2);
        uint32_t koff = (uint32_t)(t0 + col) * (uint32_t)(D * 2) + 16u * grp;
        // Tiles go in pairs and the loop leaves only at the bottom: a second
        // tile past r1 reads zeros and all its rows are masked, which costs at
        // most one tile per wave and keeps a single, scalar loop exit (an exit
        // between the tiles makes the compiler drain the prefetch every trip).
        KTile<D, U> ka, kb;
        load_ktile_at<D, U>(ka, khead, koff);
        do {
            maybe_flush();
            load_ktile_at<D, U>(kb, khead, koff + kStepBytes);
            process(ka, t0);
            maybe_flush();
            load_ktile_at<D, U>(ka, khead, koff + 2 * kStepBytes);
            process(kb, t0 + kStep);
            t0 += 2 * kStep;
            koff += 2 * kStepBytes;
        } while (t0 < r1);
    }
    }
    if constexpr (GKT > 0) {
        static_assert(!PAGED, "the tail gather reads contiguous value caches");
        // The queues' last entries go to registers with the list positions
        // flush_all would give them: the tail stages them from there, or
        // stores them to the lists when it must read the lists anyway.
        bool flushed = false;
#pragma unroll
        for (int h = 0; h < 16; ++h) flushed |= written[h] != 0;
        uint2 qe[4][4];
        int qp[4][4];
        wave_sync();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const bool have = kWave * k + lane < qn[i];
                const uint2 e = have ? q4[i][kWave * k + lane] : make_uint2(~0u, 0u);
                const int gs = (e.x & 15) >> 2;
                int pos = 0;
#pragma unroll
                for (int g2 = 0; g2 < 4; ++g2) {
                    const uint64_t m = __ballot(have && gs == g2);
                    if (gs == g2) pos = written[4 * g2 + i] + (int)lanes_below(m);
                    written[4 * g2 + i] += __popcll(m);
                }
                qe[i][k] = e;
                qp[i][k] = pos;
            }
        }
        static_assert(sizeof(queue) == sizeof(uint2) * kWavesPerBlock * 4 * kQueueCap,
                      "tail_gather reuses the queues' LDS");
        tail_gather<D, GKT, V8>(a, reinterpret_cast<unsigned char*>(&queue[0][0][0]), written,
                                qe, qp, flushed, mx, b, g, chunk, r0, qh0, capw, nl, wave, lane);
        return;
    }
    flush_all();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float m = group16_max(mx[i]);
        if (col == 0 && 4 * grp + i < Gk) {
            const int64_t list = list0 + (4 * grp + i) * list_stride;
            int cnt = written[i];
#pragma unroll
            for (int gs = 1; gs < 4; ++gs)
                if (grp == gs) cnt = written[4 * gs + i];
            a.list_count[list] = cnt;
            a.list_max[list] = m;
        }
    }
}

// Gather kernel: a 1-D grid, workgroup (b*h_q + i) * segs + segment (1-D so
// that b*h_q may exceed the 65535 limit of a grid's y dimension).  The segments of
// a head split its selected entries (the concatenation of all its lists, in
// list order) into equal ranges, so a head whose selection grew between
// refreshes is spread evenly over its workgroups.  M is the head's largest
// selected logit (from the list maxima), the same in every segment.
//
// Value rows are read with buffer loads at 32-bit byte offsets inside one
// value head (under 2 GiB); entries that carry no weight get an offset past
// the resource's end, which reads zero without touching memory, so the loads
// need no branch.
// PAGED: 0 contiguous caches; 1 paged, V pool under 4 GiB (32-bit offsets into
// the pool, same load path as contiguous); 2 paged, 64-bit addresses.
// V8 (contiguous caches only): an fp8 E4M3 value cache, d bytes per row, one
// scale per (b, value head).  Each lane loads 16 codes, widens them exactly
// to bf16, and the segment's sum is multiplied by the head's scale once.
template <int D, int PAGED, bool V8>
__global__ __launch_bounds__(kBlock) SAGA_GATHER_ATTR void gather_kernel(GatherArgs a)
{
    static_assert(!V8 || PAGED == 0, "fp8 values: contiguous caches only");
    constexpr int VB = V8 ? 1 : 2;         // bytes per value element
    constexpr int EPL = 16 / VB;           // elements per lane load (16 bytes)
    constexpr int LPR = D / EPL;           // lanes per value row
    constexpr int SLOTS = kBlock / LPR;    // rows per workgroup load instruction
    constexpr int RED = V8 ? SLOTS / 2 : SLOTS;   // slot sums held at once in the reduction
    constexpr int CAPL = kGatherStage;     // entries staged per round
    constexpr int EPT = CAPL / kBlock;     // staged entries per thread
    constexpr int NB = SAGA_GATHER_NB;     // rows in flight per lane
    constexpr int PER = kMaxListsPerRow / kBlock;
    constexpr uint32_t kNoRow = 0x80000000u;   // past any value head (< 2^31 bytes)
    constexpr uint32_t kNoRowPool = kPoolLimit;  // past any 32-bit-addressed pool
    static_assert(RED * D <= kMaxListsPerRow, "slot reduction reuses the prefix array");
    static_assert(CAPL % kBlock == 0, "staging rounds are whole threads");
    __shared__ int32_t pre[kMaxListsPerRow + 1];
    __shared__ int32_t red[kWavesPerBlock];
    __shared__ uint32_t eoff[CAPL];     // byte offset in the value head; paged: row in page
    __shared__ float ew[CAPL];
    __shared__ int32_t eps[PAGED == 2 ? CAPL : 1];   // page * h_v + value head, -1 if none

    const int bi = blockIdx.x / a.segs;
    const int seg = blockIdx.x - bi * a.segs;
    const int b = bi / a.hq, i = bi - b * a.hq;
    const int t = threadIdx.x;
    const int nl = a.chunks * kWavesPerBlock;
    const int64_t lbase = (int64_t)bi * nl;

    // List lengths (prefix) and the head's largest selected logit.  The
    // loads are unconditional (lists past nl read the last list again and are
    // masked after), so all of them are in flight before the first wait.
    // Paged caches with a work split from the lengths: the K stream's plan
    // (rows per chunk, this sequence's chunks), loaded with the list lengths.
    const bool plan = PAGED != 0 && a.pg.plan_cap != 0;
    const int32_t plan_rows = plan ? a.pg.plan[0] : 0;
    const int32_t plan_chunks = plan ? a.pg.plan[1 + b] : 0;
    int32_t c[PER], sum = 0;
    float lm[PER], mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int l = t * PER + k < nl ? t * PER + k : nl - 1;
        c[k] = a.list_count[lbase + l];
        lm[k] = a.list_max[lbase + l];
    }
    // Then the lists of this sequence's chunks only.
    const int64_t rpc = plan ? plan_rows : a.rows_per_chunk;
    const int nlv = plan ? plan_chunks * kWavesPerBlock : nl;
    const int64_t capw = rpc / kWavesPerBlock;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const bool in = t * PER + k < nlv;
        c[k] = in ? c[k] : 0;
        sum += c[k];
        mx = fmaxf(mx, in ? lm[k] : -INFINITY);
    }
    const float M = block_max(mx, reinterpret_cast<float*>(red));
    int32_t run = block_scan(sum, red) - sum;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        pre[t * PER + k] = run;
        run += c[k];
    }
    if (t == kBlock - 1) pre[kMaxListsPerRow] = run;
    __syncthreads();
    const int32_t total = pre[kMaxListsPerRow];
    const int32_t e_begin = (int32_t)((int64_t)total * seg / a.segs);
    const int32_t e_end = (int32_t)((int64_t)total * (seg + 1) / a.segs);

    const int nu = i / a.Gv;
    const unsigned char* vh = reinterpret_cast<const unsigned char*>(a.v) +
                              ((int64_t)(b * a.hv + nu) * a.cache_len) * D * VB;
    // Contiguous: the value head; paged (32-bit): the whole pool.
    const __amdgpu_buffer_rsrc_t vrs =
        PAGED == 1 ? make_rsrc(a.v, a.pool_bytes)
                   : make_rsrc(vh, (uint32_t)(PAGED ? 0 : a.cache_len * D * VB));
    const int slot = t / LPR, lc = t - slot * LPR;
    const float tf = a.tau_filter ? a.tau_filter[bi] : -INFINITY;
    float acc[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) acc[j] = 0.f;
    float lsum = 0.f;
    int32_t kept = 0;                                   // entries with logit >= tf

    for (int32_t base = e_begin; base < e_end; base += CAPL) {
        const int n = min(CAPL, e_end - base);
        // Thread t stages entries EPT*t .. EPT*t + EPT-1 of this round: one
        // binary search over the list offsets for the first, a forward walk
        // for the rest.  Slots past n take entry n-1 again (masked below), so
        // the loads carry no branch and all are in flight before any is used.
        int lo[EPT];
        uint32_t in_list[EPT];
        {
            const int32_t E0 = base + min(EPT * t, n - 1);
            int l0 = 0, hi = nl - 1;
            while (l0 < hi) {
                const int mid = (l0 + hi + 1) >> 1;
                if (pre[mid] <= E0) l0 = mid;
                else hi = mid - 1;
            }
#pragma unroll
            for (int k = 0; k < EPT; ++k) {
                const int32_t E = base + min(EPT * t + k, n - 1);
                while (pre[l0 + 1] <= E) ++l0;          // skips empty lists; stops below nl
                lo[k] = l0;
                in_list[k] = (uint32_t)(E - pre[l0]);
            }
        }
        uint2 ent[EPT];
#pragma unroll
        for (int k = 0; k < EPT; ++k)
            ent[k] = a.entries[list_index(bi, lo[k], in_list[k], capw, nl, a.head_stride,
                                          a.overflow_at)];
        if constexpr (PAGED) {
            // The value row's page: every table read issued before any use.
            int32_t page[EPT];
#pragma unroll
            for (int k = 0; k < EPT; ++k) {
                const int64_t r = (int64_t)(lo[k] / kWavesPerBlock) * rpc + ent[k].x;
                const int64_t pi = r / a.pg.page_rows;
                page[k] = (EPT * t + k < n && pi < a.pg.max_pages)
                              ? a.pg.block_table[(int64_t)b * a.pg.max_pages + pi] : -1;
            }
#pragma unroll
            for (int k = 0; k < EPT; ++k) {
                const int e = EPT * t + k;
                if (e < n) {
                    const float sv = __uint_as_float(ent[k].y);
                    const bool keep = sv >= tf;
                    kept += keep;
                    const int64_t r = (int64_t)(lo[k] / kWavesPerBlock) * rpc + ent[k].x;
                    const bool ok = page[k] >= 0 && page[k] < a.pg.num_pages;   // else reads nothing
                    if constexpr (PAGED == 1) {
                        eoff[e] = keep && ok ? (uint32_t)((((int64_t)page[k] * a.hv + nu) *
                                                           a.pg.page_rows + r % a.pg.page_rows) * (D * 2))
                                             : kNoRowPool;
                    } else {
                        eoff[e] = (uint32_t)(r % a.pg.page_rows);
                        eps[e] = ok ? page[k] * a.hv + nu : -1;
                    }
                    ew[e] = keep && ok ? __expf(sv - M) : 0.f;
                }
            }
        } else {
#pragma unroll
        for (int k = 0; k < EPT; ++k) {
            const int e = EPT * t + k;
            if (e < n) {
                const float sv = __uint_as_float(ent[k].y);
                const bool keep = sv >= tf;
                kept += keep;
                const uint32_t r = (uint32_t)((lo[k] / kWavesPerBlock) * rpc) + ent[k].x;
                eoff[e] = keep ? r * (uint32_t)(D * VB) : kNoRow;
                ew[e] = keep ? __expf(sv - M) : 0.f;
            }
        }
        }
        __syncthreads();
        for (int e0 = slot; e0 < n; e0 += SLOTS * NB) {
            u32x4 vv[NB];
            float w[NB];
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                const int e = e0 + k * SLOTS;
                const bool in = e < n;
                w[k] = in ? ew[e] : 0.f;
                if constexpr (PAGED == 2) {
                    if (w[k] > 0.f)                     // weight zero: no row (or no page)
                        vv[k] = ld16(a.v + ((int64_t)eps[e] * a.pg.page_rows + eoff[e]) * D + 8 * lc);
                    else
                        vv[k] = u32x4{0u, 0u, 0u, 0u};
                } else if constexpr (PAGED == 1) {
                    vv[k] = buf_ld16(vrs, (in ? eoff[e] : kNoRowPool) + 16u * lc);
                } else {
                    vv[k] = buf_ld16(vrs, (in ? eoff[e] : kNoRow) + 16u * lc);
                }
            }
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                if constexpr (V8) {
                    // Codes 0-7 then 8-15 of the lane's 16, widened in order.
                    const u32x4 h0 = fp8x8_to_bf16x8(u32x2{vv[k][0], vv[k][1]});
                    const u32x4 h1 = fp8x8_to_bf16x8(u32x2{vv[k][2], vv[k][3]});
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        acc[2 * j] += w[k] * bf16lo(h0[j]);
                        acc[2 * j + 1] += w[k] * bf16hi(h0[j]);
                        acc[8 + 2 * j] += w[k] * bf16lo(h1[j]);
                        acc[8 + 2 * j + 1] += w[k] * bf16hi(h1[j]);
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        acc[2 * j] += w[k] * bf16lo(vv[k][j]);
                        acc[2 * j + 1] += w[k] * bf16hi(vv[k][j]);
                    }
                }
                lsum += w[k];
            }
        }
        __syncthreads();
    }

    // Reduce the slots in slot order.  fp8 values: the slots' sums take twice
    // the prefix array, so slot s + SLOTS/2 is first added to slot s.
    float* ored = reinterpret_cast<float*>(pre);        // [RED][D]
    if constexpr (V8) {
        if (slot < RED) {
#pragma unroll
            for (int j = 0; j < EPL; ++j) ored[slot * D + EPL * lc + j] = acc[j];
        }
        __syncthreads();
        if (slot >= RED) {
#pragma unroll
            for (int j = 0; j < EPL; ++j) ored[(slot - RED) * D + EPL * lc + j] += acc[j];
        }
    } else {
#pragma unroll
        for (int j = 0; j < EPL; ++j) ored[slot * D + EPL * lc + j] = acc[j];
    }
    if (lc == 0) ew[slot] = lsum;
    const int32_t nkept = block_sum(kept, red);         // its barrier orders the stores above
    const int64_t idx = (int64_t)bi * a.segs + seg;
    const float vscale = V8 ? a.v_scale[b * a.hv + nu] : 1.f;
    for (int p = t; p < D; p += kBlock) {
        float o = 0.f;
        for (int s = 0; s < RED; ++s) o += ored[s * D + p];
        a.part.o[idx * D + p] = V8 ? o * vscale : o;
    }
    if (t == 0) {
        float l = 0.f;
        for (int s = 0; s < SLOTS; ++s) l += ew[s];
        a.part.m[idx] = nkept > 0 ? M : -INFINITY;
        a.part.l[idx] = l;
        a.part.c[idx] = nkept;
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
    __shared__ float wred[kWavesPerBlock];
    __shared__ int32_t cred[kWavesPerBlock];
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
    // This thread's first partial, loaded before the reductions need M.
    const bool have0 = pl < parts;
    const float w0 = have0 ? pm[pl] : -INFINITY;
    const float o0 = have0 ? po[(int64_t)pl * D + e] : 0.f;
    const float l0 = have0 ? pl_[pl] : 0.f;
    M = block_max(M, wred);
    n = block_sum(n, cred);
    if (M == -INFINITY) {                                  // nothing selected anywhere
        if (t < D) out[bh * D + t] = 0;
        if (counts && t == 0) counts[bh] = n;
        return;
    }
    float acc = 0.f, l = 0.f;
    if (have0) {
        const float a = __expf(w0 - M);                    // -inf partials weigh 0
        acc += a * o0;
        l += a * l0;
    }
    int c = pl + PL;
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
    // Paged calls with the work split from the lengths: a 1-D launch over the
    // work items (paged_item).
    const dim3 grid = a.pg.plan_cap ? dim3((unsigned)a.pg.plan_grid, 1)
                                    : dim3(a.chunks, a.B * a.hk);
    const bool dbg = a.bitmap != nullptr || a.logits_out != nullptr;
    const int kind = a.pg.block_table != nullptr ? 1 : (a.k_scale != nullptr ? 2 : 0);
#define SAGA_LAUNCH_STREAM(DD, DBG, PG, F8)                                                      \
    hipLaunchKernelGGL((select_stream_kernel<DD, F8 ? decode_unroll_k8(DD) : decode_unroll(DD),  \
                                             DBG, PG, F8, 0, false>), grid, dim3(kBlock), 0, s, a)
#define SAGA_LAUNCH_TAIL(DD, DBG, F8, GG)                                                        \
    if (a.v_scale) hipLaunchKernelGGL((select_stream_kernel<DD, F8 ? decode_unroll_k8(DD) :       \
                                                            decode_unroll(DD), DBG, false, F8, GG, F8>), \
                                      grid, dim3(kBlock), 0, s, a);                              \
    else hipLaunchKernelGGL((select_stream_kernel<DD, F8 ? decode_unroll_k8(DD) : decode_unroll(DD), \
                                                  DBG, false, F8, GG, false>),                   \
                            grid, dim3(kBlock), 0, s, a)
    if (a.v) {
        // The tail gather: contiguous caches, d = 64 or 128, at most 16 head
        // slots; an fp8 V cache comes with an fp8 K cache.  With bf16 K at
        // d = 64, key groups of at most 8 query heads get 8 slots and the
        // larger stage that leaves (128 VGPRs, three workgroups per CU, which
        // the bf16 launch of 768 has); the fp8 K launch needs four per CU.
        if (a.pg.block_table || (D != 64 && D != 128) || a.Gk > 16 || (a.v_scale && kind != 2))
            return hipErrorInvalidValue;
        if (D == 64) {
            if (kind == 2) { if (dbg) SAGA_LAUNCH_TAIL(64, true, true, 16); else SAGA_LAUNCH_TAIL(64, false, true, 16); }
            else if (a.Gk <= 8) { if (dbg) SAGA_LAUNCH_TAIL(64, true, false, 8); else SAGA_LAUNCH_TAIL(64, false, false, 8); }
            else { if (dbg) SAGA_LAUNCH_TAIL(64, true, false, 16); else SAGA_LAUNCH_TAIL(64, false, false, 16); }
        } else {
            if (kind == 2) { if (dbg) SAGA_LAUNCH_TAIL(128, true, true, 16); else SAGA_LAUNCH_TAIL(128, false, true, 16); }
            else { if (dbg) SAGA_LAUNCH_TAIL(128, true, false, 16); else SAGA_LAUNCH_TAIL(128, false, false, 16); }
        }
#undef SAGA_LAUNCH_TAIL
        return hipGetLastError();
    }
#define SAGA_LAUNCH_STREAM_BF(DD)                                                                \
    if (kind == 1) { if (dbg) SAGA_LAUNCH_STREAM(DD, true, true, false); else SAGA_LAUNCH_STREAM(DD, false, true, false); } \
    else { if (dbg) SAGA_LAUNCH_STREAM(DD, true, false, false); else SAGA_LAUNCH_STREAM(DD, false, false, false); }
#define SAGA_LAUNCH_STREAM_D(DD)                                                                 \
    if (kind == 2) { if (dbg) SAGA_LAUNCH_STREAM(DD, true, false, true); else SAGA_LAUNCH_STREAM(DD, false, false, true); } \
    else { SAGA_LAUNCH_STREAM_BF(DD) }
    if (D == 32) {
        if (kind == 2) return hipErrorInvalidValue;      // no fp8 K at head_dim 32 (the API rejects it)
        SAGA_LAUNCH_STREAM_BF(32)
    } else if (D == 64) {
        SAGA_LAUNCH_STREAM_D(64)
    } else {
        SAGA_LAUNCH_STREAM_D(128)
    }
#undef SAGA_LAUNCH_STREAM_D
#undef SAGA_LAUNCH_STREAM_BF
#undef SAGA_LAUNCH_STREAM
    return hipGetLastError();
}

hipError_t launch_gather(int D, const GatherArgs& a, hipStream_t s)
{
    const dim3 grid((unsigned)a.segs * (unsigned)(a.B * a.hq));
    const int mode = a.pg.block_table == nullptr ? 0 : (a.pool_bytes != 0 ? 1 : 2);
    if (a.v_scale && mode != 0) return hipErrorInvalidValue;   // fp8 values: contiguous only
#define SAGA_LAUNCH_GATHER(DD, M, V8) \
    hipLaunchKernelGGL((gather_kernel<DD, M, V8>), grid, dim3(kBlock), 0, s, a)
#define SAGA_LAUNCH_GATHER_D(DD)                                                   \
    if (a.v_scale) SAGA_LAUNCH_GATHER(DD, 0, true);                                \
    else if (mode == 0) SAGA_LAUNCH_GATHER(DD, 0, false);                          \
    else if (mode == 1) SAGA_LAUNCH_GATHER(DD, 1, false);                          \
    else SAGA_LAUNCH_GATHER(DD, 2, false);
    if (D == 32) {
        SAGA_LAUNCH_GATHER_D(32)
    } else if (D == 64) {
        SAGA_LAUNCH_GATHER_D(64)
    } else {
        SAGA_LAUNCH_GATHER_D(128)
    }
#undef SAGA_LAUNCH_GATHER_D
#undef SAGA_LAUNCH_GATHER
    return hipGetLastError();
}

hipError_t launch_combine(int D, const Partials& p, int rows, int parts, uint16_t* out,
                          int32_t* counts, hipStream_t s)
{
    if (D == 32)
        hipLaunchKernelGGL(combine_kernel<32>, dim3(rows), dim3(kBlock), 0, s, p, parts, out, counts);
    else if (D == 64)
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

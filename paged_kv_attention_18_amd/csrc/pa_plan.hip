// pa_plan.hip -- the device-side work planner.
//
// The planner plays the role of the task-list generator that the
// SparseAttnSharedkvMetadata README describes (function section: a list of
// start/end points -- batch, head, Q block, K block -- for every core,
// consumed by the attention operator, and reduction tasks for split rows).
// Here it runs on the GPU and reads only the lengths: it sanitises them,
// numbers the (sequence, KV head, row tile, KV chunk) items, cuts them into
// N equal pieces, lists the units that a piece boundary cuts (the reduction
// tasks) and resets the counter the attention kernels use to hand out
// pieces.  Every workgroup numbers the items (a scan over the batch); each
// then places kPlanPieces of the pieces, and workgroup 0 alone writes the
// per-sequence arrays, the header and the error bits.  The pieces depend on the lengths alone, so the partial
// sums that make up an output row, and the order they are merged in, do not
// depend on which workgroup ran which piece.
//
// The merge combines the fp32 partials of rows whose KV range was split over
// several pieces: with per-part running max m_p (log2 domain), sum l_p and
// unnormalised output acc_p,
//     M = max_p m_p,  L = sum_p l_p 2^(m_p - M),  o = sum_p 2^(m_p - M) acc_p / L,
// which is the softmax over the union of the parts exactly (the "FlashDecode
// reduction" tasks of the same README's metadata output).
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kPlanThreads = 1024;
constexpr int kPlanLdsB = 2048;   // sequences kept in LDS for the piece phase
// pieces per workgroup: placing a piece walks its sequence's row tiles on
// one thread, so one wave of pieces per workgroup keeps each CU's walk short
constexpr int kPlanPieces = 64;
// row tiles whose leading item counts are kept in LDS, so that placing a
// piece bisects its sequence's tiles instead of walking them
constexpr int kPlanLdsT = 8192;

// The whole-tile queues (workgroup 0 of the plan kernel, every thread).
// Sequences are ranked by their longest row tile (then their work); the
// (sequence, KV head) groups in that order are dealt to the XCDs in snake
// order (0..7, 7..0, ...), which balances the XCDs' work; each XCD's queue
// lists its groups in order, every group's row tiles together (last tile,
// the longest under the causal mask, first).  Workers of one XCD take
// consecutive tasks (tile_first_task, tile_claim), so the tiles of a group
// start close together and read their sequence's KV from that XCD's L2.  The
// queues' claim counters start at 0.
// s_key[b]: the sequence's longest row tile in chunks (the first phase of the
// plan kernel leaves it there).
__device__ void build_tile_queues(const Params &p, int *s_order, const int *s_key, int *s_xtot, const int *s_ipg,
                                  const int *s_ql)
{
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int B = p.batch, Hkv = p.kv_head_num;
    // rank: the longest row tile (a queue then runs roughly longest task
    // first), then the work, then the index; one wave per sequence counts
    // the sequences ahead of it, 64 at a time
    for (int b = wv; b < B; b += kPlanThreads / 64) {
        const int m = s_key[b], w = s_ipg[b];
        int r = 0;
        for (int b0 = 0; b0 < B; b0 += 64) {
            const int b2 = b0 + lane;
            bool ahead = false;
            if (b2 < B) {
                const int m2 = s_key[b2], w2 = s_ipg[b2];
                ahead = m2 > m || (m2 == m && (w2 > w || (w2 == w && b2 < b)));
            }
            r += __popcll(__ballot(ahead));
        }
        if (lane == 0)
            s_order[r] = b;
    }
    __syncthreads();
    const int NG = B * Hkv;
    // group k of the order sits on XCD x = snake(k); the r-th group of XCD x
    // is k = 8 r + (r even ? x : 7 - x)
    auto tiles_of = [&](int x, int r, int &b, int &g) {
        const int k = kXcds * r + ((r & 1) ? kXcds - 1 - x : x);
        if (k >= NG)
            return 0;
        b = s_order[k / Hkv];
        g = k % Hkv;
        return seq_tiles(p, s_ql[b]);
    };
    if (wv < kXcds) {
        int tot = 0;
        for (int r0 = 0; kXcds * r0 < NG; r0 += 64) {
            int b = 0, g = 0;
            const int nt = tiles_of(wv, r0 + lane, b, g);
            tot += __shfl(wave_scan(nt, lane), 63);
        }
        if (lane == 0)
            s_xtot[wv] = tot;
    }
    __syncthreads();
    if (wv < kXcds) {
        int start = 0;
        for (int x = 0; x < wv; ++x)
            start += s_xtot[x];
        int run = 0;
        for (int r0 = 0; kXcds * r0 < NG; r0 += 64) {
            int b = 0, g = 0;
            const int nt = tiles_of(wv, r0 + lane, b, g);
            const int inc = wave_scan(nt, lane);
            int32_t *e = p.ws.tq + kTqHeader + 2 * (size_t)(start + run + inc - nt);
            for (int t = 0; t < nt; ++t) {
                e[2 * t] = b;
                e[2 * t + 1] = (g << 16) | (nt - 1 - t);
            }
            run += __shfl(inc, 63);
        }
        if (lane == 0) {
            p.ws.tq[kTqLength + wv] = s_xtot[wv];
            p.ws.tq[kTqStart + wv] = start;
            __hip_atomic_store(p.ws.tq + kTqCounter + kTqCounterStride * wv, 0, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_SYSTEM);
        }
    }
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(Params p)
{
    constexpr int NWV = kPlanThreads / 64;
    __shared__ int s_wq[NWV], s_wt[NWV], s_ww[NWV];
    // per-sequence data for the piece phase (global arrays past kPlanLdsB)
    __shared__ int s_wsb[kPlanLdsB + 1], s_kv[kPlanLdsB], s_ql[kPlanLdsB], s_ipg[kPlanLdsB], s_t0[kPlanLdsB];
    // each sequence's first row tile in s_tp, and per row tile the items per
    // KV head of its sequence before it
    __shared__ int s_toff[kPlanLdsB], s_tp[kPlanLdsT];
    __shared__ int s_carry_q, s_carry_t, s_carry_w, s_lmax;
    __shared__ uint32_t s_err;
    // whole-tile mode: the sequences in order of decreasing work, and the
    // tiles each XCD's queue holds
    __shared__ int s_order[kTileOrderMaxBatch], s_key[kTileOrderMaxBatch], s_xtot[kXcds];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const bool lead = blockIdx.x == 0;
    if (tid == 0) {
        s_carry_q = 0;
        s_carry_t = 0;
        s_carry_w = 0;
        s_lmax = 0;
        s_err = 0;
    }
    __syncthreads();
    const int cap = seq_cap(p);
    for (int base = 0; base < p.batch; base += kPlanThreads) {
        const int b = base + tid;
        int ql = 0, kv = 0, nt = 0;
        uint32_t err = 0;
        if (b < p.batch) {
            kv = p.context_lens[b];
            ql = p.q_seq_lens ? p.q_seq_lens[b] : 1;
            err = sanitize_seq(p, cap, kv, ql);
            nt = seq_tiles(p, ql);
        }
        if (err)
            atomicOr(&s_err, err);
        // exclusive prefix sums (wave scans, then the wave totals) of the
        // query tokens and row tiles, then of the items
        const int iq = wave_scan(ql, lane), it = wave_scan(nt, lane);
        if (lane == 63) {
            s_wq[wv] = iq;
            s_wt[wv] = it;
        }
        __syncthreads();
        if (tid == 0) {
            int aq = s_carry_q, at = s_carry_t;
            for (int w = 0; w < NWV; ++w) {
                const int tq = s_wq[w], tt = s_wt[w];
                s_wq[w] = aq;
                s_wt[w] = at;
                aq += tq;
                at += tt;
            }
            s_carry_q = aq;
            s_carry_t = at;
        }
        __syncthreads();
        const int t0 = s_wq[wv] + iq - ql;
        const int toff = s_wt[wv] + it - nt;
        int ipg = 0, lmax = 0;
        for (int qt = 0; qt < nt; ++qt) {
            if (toff + qt < kPlanLdsT)
                s_tp[toff + qt] = ipg;
            const int n = unit_chunks(p, kv, ql, qt);
            ipg += n;
            lmax = n > lmax ? n : lmax;
        }
        if (lmax > 0)
            atomicMax(&s_lmax, lmax);
        if (b < p.batch && b < kTileOrderMaxBatch)
            s_key[b] = lmax;   // whole-tile mode: the rank key
        const int items = ipg * p.kv_head_num;
        if (lead && b < p.batch) {
            p.ws.qlen[b] = ql;
            p.ws.kvlen[b] = kv;
            p.ws.ipg[b] = ipg;
        }
        const int iw = wave_scan(items, lane);
        if (lane == 63)
            s_ww[wv] = iw;
        __syncthreads();
        if (tid == 0) {
            int aw = s_carry_w;
            for (int w = 0; w < NWV; ++w) {
                const int tw = s_ww[w];
                s_ww[w] = aw;
                aw += tw;
            }
            s_carry_w = aw;
        }
        __syncthreads();
        const int wsb = s_ww[wv] + iw - items;
        if (b < p.batch) {
            if (lead) {
                p.ws.cu_q[b] = t0;
                p.ws.wsb[b] = wsb;
            }
            if (b < kPlanLdsB) {
                s_wsb[b] = wsb;
                s_kv[b] = kv;
                s_ql[b] = ql;
                s_ipg[b] = ipg;
                s_t0[b] = t0;
                s_toff[b] = toff;
            }
        }
        __syncthreads();
    }
    const int W = s_carry_w;
    const int per = p.no_split ? 0 : (W + p.pieces - 1) / p.pieces;
    // Whole row tiles from per-XCD queues instead of pieces, where there are
    // enough tiles for the workers and the longest is at most half a
    // worker's share of the chunks (every workgroup decides alike, from the
    // lengths).
    const long long tiles = (long long)s_carry_t * p.kv_head_num;
    const bool ordered = p.tile_order && !p.no_split && p.batch <= kTileOrderMaxBatch && W > 0 &&
                         tiles >= 2LL * p.partitions && 2LL * s_lmax * p.partitions <= (long long)W;
    if (lead && tid == 0) {
        p.ws.cu_q[p.batch] = s_carry_q;
        p.ws.wsb[p.batch] = W;
        p.ws.hdr[0] = W;
        p.ws.hdr[1] = per > 0 ? per : (p.no_split ? 0 : 1);
        p.ws.hdr[2] = p.no_split ? 0 : p.pieces;
        p.ws.hdr[3] = 0;
        p.ws.hdr[4] = p.no_split ? 0 : p.pieces;   // all pieces alike: no tail
        p.ws.hdr[5] = 0;
        p.ws.hdr[6] = p.partitions;
        p.ws.hdr[7] = 0;
        if (s_carry_q != p.num_q_tokens)
            s_err |= PA_DEVERR_TOKENS;
    }
    if (!p.no_split) {
        const int pe = per > 0 ? per : 1;
        const bool lds = p.batch <= kPlanLdsB;
        if (tid == 0 && lds)
            s_wsb[p.batch] = W;
        __syncthreads();
        // Past kPlanLdsB sequences the piece phase reads the per-sequence
        // arrays back from memory, where only workgroup 0's writes are
        // ready for it: then workgroup 0 places every piece.
        const bool spread = lds && gridDim.x > 1;
        if (!spread && !lead)
            return;
        const int k0 = spread ? blockIdx.x * kPlanPieces : 0;
        const int k1 = spread ? min(k0 + kPlanPieces, p.pieces) : p.pieces;
        const bool table = lds && s_carry_t <= kPlanLdsT;
        // Piece k starts at item k * pe, in the last sequence b with
        // wsb[b] <= k * pe.  Its split entry (entry k - 1) records the unit
        // that boundary k cuts, if it falls strictly inside one.
        const int nk = ordered ? 0 : ((W + pe - 1) / pe < p.pieces ? (W + pe - 1) / pe : p.pieces);
        for (int k = k0 + tid; k < k1 && k < nk; k += kPlanThreads) {
            const int s = k * pe;
            // (LDS and global reads on separate paths: a pointer that may be
            // either compiles to flat loads, each waited for)
            int lo = 0, hi = p.batch - 1;
            if (lds) {
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (s_wsb[mid] <= s)
                        lo = mid;
                    else
                        hi = mid - 1;
                }
            } else {
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (p.ws.wsb[mid] <= s)
                        lo = mid;
                    else
                        hi = mid - 1;
                }
            }
            const int b = lo;
            p.ws.wg_b[k] = b;
            if (k == 0)
                continue;
            int kv, ql, ipg, t0, wb;
            if (lds) {
                kv = s_kv[b];
                ql = s_ql[b];
                ipg = s_ipg[b];
                t0 = s_t0[b];
                wb = s_wsb[b];
            } else {
                kv = p.ws.kvlen[b];
                ql = p.ws.qlen[b];
                ipg = p.ws.ipg[b];
                t0 = p.ws.cu_q[b];
                wb = p.ws.wsb[b];
            }
            (void)piece_start(p, k, s, s - pe, b, kv, ql, ipg, wb, t0, true, table ? s_tp + s_toff[b] : nullptr);
        }
        // boundaries past the last item (every boundary in whole-tile mode)
        for (int k = max(nk, k0) + tid; k < k1; k += kPlanThreads)
            if (k > 0)
                p.ws.splits[(size_t)(k - 1) * 8] = -1;
    }
    if (lead && p.tile_order) {
        if (ordered)
            build_tile_queues(p, s_order, s_key, s_xtot, s_ipg, s_ql);
        if (tid == 0)
            p.ws.tq[kTqMode] = ordered ? 1 : 0;
    }
    if (lead && tid == 0 && s_err)
        set_error(p.ws.err, s_err);
}

// Rows per merge workgroup: enough to give every thread ~4 outputs, or ~16
// for narrow rows (Dv <= 128), where a workgroup's dependent reads of the
// header and its split entry cost more than its few outputs.
__host__ __device__ inline int merge_rows_per_wg(int dv)
{
    const int r = ((dv <= 128 ? 16 : 4) * kThreads) / dv;
    return r < 1 ? 1 : (r > 64 ? 64 : r);
}

// One workgroup per (split entry, group of rows), for as many entries as a
// pass can have (their number is known on the device only).
// Piece k's partial of a unit is in slot 0 if the unit started at or before
// the piece, else in slot 1: slot 1 only for the first piece of the unit.
// Workgroup 0 also resets the piece counter for the next pass, which the
// attention kernel has finished with (the self-planning kernel does not
// reset it: its workers claim pieces from the moment they start).
// Each thread owns four consecutive outputs of one row and combines the
// parts online (running max, rescaled sum and accumulator), reading a part's
// m, l and its four accumulator values together: the loads of KB parts
// (4, or 8 with a claimed tail) are issued before any is used, so each batch of parts costs one
// memory round trip and the row statistics need no pass of their own.
// TAIL: the pass may have a claimed tail (PieceMap); else its pieces are
// all alike and every entry of the grid belongs to the pass.
template <int DT, bool TAIL>
__device__ __forceinline__ void merge_body(const Params &p, int row_groups)
{
    constexpr int KB = TAIL ? 8 : 4;   // a claimed tail cuts units into more parts
    const int entry = blockIdx.x / row_groups;
    const int32_t *d = p.ws.splits + (size_t)entry * 8;
    int first, last, slot_first;
    int us, ue;
    if constexpr (TAIL) {
        const PieceMap pm = header_piece_map(p.ws.hdr);
        // entries past the pass's last boundary are left over from other passes
        if (d[0] < 0 || pm.per <= 0 || entry >= piece_count(pm) - 1)
            return;
        us = d[3];
        ue = d[4];
        first = piece_of(pm, us);
        last = piece_of(pm, ue - 1);
        int f0, f1;
        piece_range(pm, first, f0, f1);
        slot_first = 2 * first + (f0 >= us ? 0 : 1);
    } else {
        const int per = p.ws.hdr[1];
        if (d[0] < 0 || per <= 0)
            return;
        us = d[3];
        ue = d[4];
        first = us / per;
        last = (ue - 1) / per;
        slot_first = 2 * first + (first * per >= us ? 0 : 1);
    }
    const int g = d[1], qt = d[2], t0 = d[5], rows = d[6];
    const int rgp = blockIdx.x % row_groups;
    const int G = p.group;
    const int R = p.rows_per_tile;
    const int DV = p.head_size_v;
    const int RPW = merge_rows_per_wg(DV);
    const int r0 = rgp * RPW;
    if (r0 >= rows)
        return;
    const int nr = rows - r0 < RPW ? rows - r0 : RPW;
    auto part_of = [&](int k) -> const float * {
        k = k < last ? k : last;
        return p.ws.partials + (size_t)(k == first ? slot_first : 2 * k) * p.partial_stride;
    };
    uint16_t *out = (uint16_t *)p.out;
    // four consecutive outputs per thread and step (DV is a multiple of 4)
    for (int idx = 4 * threadIdx.x; idx < nr * DV; idx += 4 * kThreads) {
        const int rr = idx / DV;
        const int e = idx - rr * DV;
        const int r = r0 + rr;
        float M = -INFINITY, L = 0.f;
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        for (int k0 = first; k0 <= last; k0 += KB) {
            float mk[KB], lk[KB];
            float4 a[KB];
#pragma unroll
            for (int i = 0; i < KB; ++i) {
                const float *pt = part_of(k0 + i);
                mk[i] = pt[R * DV + r];
                lk[i] = pt[R * DV + R + r];
                a[i] = *(const float4 *)(pt + r * DV + e);
            }
#pragma unroll
            for (int i = 0; i < KB; ++i) {
                if (k0 + i > last || mk[i] == -INFINITY)
                    continue;
                if (mk[i] > M) {
                    const float sc = exp2f(M - mk[i]);   // 0 while M is -inf
                    L = L * sc + lk[i];
                    acc[0] = acc[0] * sc + a[i].x;
                    acc[1] = acc[1] * sc + a[i].y;
                    acc[2] = acc[2] * sc + a[i].z;
                    acc[3] = acc[3] * sc + a[i].w;
                    M = mk[i];
                } else {
                    const float w = exp2f(mk[i] - M);
                    L += lk[i] * w;
                    acc[0] += w * a[i].x;
                    acc[1] += w * a[i].y;
                    acc[2] += w * a[i].z;
                    acc[3] += w * a[i].w;
                }
            }
        }
        const int rg = qt * R + r;
        const int t = t0 + rg / G;
        if (t < p.num_q_tokens) {
            const float inv = L > 0.f ? 1.f / L : 0.f;
            const uint32_t w0 = (uint32_t)to_bits<DT>(acc[0] * inv) | ((uint32_t)to_bits<DT>(acc[1] * inv) << 16);
            const uint32_t w1 = (uint32_t)to_bits<DT>(acc[2] * inv) | ((uint32_t)to_bits<DT>(acc[3] * inv) << 16);
            *(uint2 *)(out + ((size_t)t * p.head_num + g * G + rg % G) * DV + e) = uint2{w0, w1};
            if (e == 0 && p.lse)
                p.lse[(size_t)t * p.head_num + g * G + rg % G] =
                    L > 0.f ? (M + log2f(L)) * 0.69314718055994531f : -INFINITY;
        }
    }
}

template <int DT, bool TAIL>
__global__ __launch_bounds__(kThreads) void merge_kernel(Params p, int row_groups)
{
    merge_body<DT, TAIL>(p, row_groups);
    // after every load of the header (a store ahead of them would keep them
    // off the scalar cache)
    if (blockIdx.x == 0 && threadIdx.x == 0)
        p.ws.hdr[3] = 0;
}

}  // namespace

hipError_t launch_plan(const Params &p, hipStream_t s, hipEvent_t e0, hipEvent_t e1)
{
    // one workgroup when the piece phase cannot keep the sequences in LDS
    const int wgs = (p.no_split || p.batch > kPlanLdsB) ? 1 : (p.pieces + kPlanPieces - 1) / kPlanPieces;
    Params pc = p;
    void *args[] = {(void *)&pc};
    return launch_kernel((const void *)&plan_kernel, dim3(wgs > 0 ? wgs : 1), dim3(kPlanThreads), args, s, e0, e1);
}

hipError_t launch_merge(const Params &p, int dtype, hipStream_t s, hipEvent_t e0, hipEvent_t e1, bool *launched)
{
    if (launched)
        *launched = false;
    // row groups of the largest unit this pass can have (a decode unit has
    // only its query heads' rows, fewer than the tile's)
    const long long max_rows = (long long)p.max_q * p.group;
    const int rows = max_rows < p.rows_per_tile ? (int)max_rows : p.rows_per_tile;
    const int row_groups = (rows + merge_rows_per_wg(p.head_size_v) - 1) / merge_rows_per_wg(p.head_size_v);
    // the self-planning kernel's claimed tail makes up to kTailRounds rounds
    // of pieces more; workgroups past the pass's split entries return at once
    const long long max_pieces = (p.self_plan && p.tail_min > 0) ? (long long)(1 + kTailRounds) * p.partitions
                                                                 : (long long)p.pieces;
    long long grid = (max_pieces - 1) * row_groups;
    if (grid <= 0 || p.no_split)
        return hipSuccess;
    if (grid > 0x7fffffff)
        return hipErrorInvalidValue;
    const bool tail = p.self_plan && p.tail_min > 0;
    void (*k)(Params, int) = dtype == 0 ? (tail ? merge_kernel<0, true> : merge_kernel<0, false>)
                                        : (tail ? merge_kernel<1, true> : merge_kernel<1, false>);
    Params pc = p;
    int rg = row_groups;
    void *args[] = {(void *)&pc, (void *)&rg};
    const hipError_t e = launch_kernel((const void *)k, dim3((unsigned)grid), dim3(kThreads), args, s, e0, e1);
    if (launched)
        *launched = e == hipSuccess;
    return e;
}

}  // namespace pa

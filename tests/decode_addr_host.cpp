// Host-side bounds check of the VALU decode kernel (pa_decode.hip) and of the
// planning it runs on, in causal and no-mask mode.
//
// The planner's arithmetic (length clamping, item counts, piece starts and
// split entries, the cursor a worker walks) and the kernel's addressing
// (head_row, bt_column, kv_row_elem, lane_col) are the library's own
// functions from pa_internal.h, compiled here for the host.  This file
// repeats only the kernel's control flow: workers, segments, the chunk loop
// with its block-id prefetch one and two chunks ahead, the final output or
// partial writes, and the merge kernel's reads of the partials.  Every
// element index of every lane is checked against the size of the buffer it
// reads or writes: query, key and value caches, block table, output, lse,
// partial slots and split entries.
//
// Cases: the shape whose GPU run once ended in a memory fault (kv 50 / 9 /
// 200, q 4 / 3 / 1, H 8 / Hkv 4, D 128, block size 16), then a seeded
// sweep over batch, lengths, group size, head size, block size, worker
// count, mask and malformed inputs (bad block ids, short tables, q_seq_lens
// above context_lens, negative lengths), which the kernels must clamp.
// Prints "ok <cases> <accesses>" or the first violation.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <string>
#include <vector>

#include "pa_internal.h"

namespace {

struct Case {
    std::vector<int> kv, ql;          // as passed to the kernel (may be malformed)
    int H, Hkv, D, bs, P;             // P: workers (= pieces on the VALU path)
    bool causal;
    int max_q;                        // the call's max_q_seq_len
    int mb;                           // block-table row length
    long long nb;                     // physical blocks
    std::vector<int> table;           // [B, mb]
    std::string name;
};

long long g_accesses = 0;

[[noreturn]] void fail(const Case &c, const std::string &what)
{
    std::printf("FAIL %s: %s\n", c.name.c_str(), what.c_str());
    std::exit(1);
}

void check(const Case &c, const char *buf, long long idx, long long count, long long size, const std::string &where)
{
    ++g_accesses;
    if (idx < 0 || idx + count > size)
        fail(c, std::string(buf) + " index " + std::to_string(idx) + " (+" + std::to_string(count) + ") outside [0, " +
                    std::to_string(size) + ") at " + where);
}

int next_pow2(int x)
{
    int p = 1;
    while (p < x)
        p <<= 1;
    return p;
}

// One case: plan on the host, then every worker of the kernel and the merge.
void run(const Case &c)
{
    const int B = (int)c.kv.size();
    const int G = c.H / c.Hkv;
    const int D = c.D;
    const int RP = next_pow2(c.max_q * G);
    if (RP > 8)
        fail(c, "case has more than 8 rows per unit");
    const int L = D / 16, NG = 64 / L, TL = RP <= 4 ? 4 : 2, CT = TL * NG;
    const int NQ = RP * 16, PER = NQ / NG;
    long long T = 0;   // query tokens as the caller counts them: the sum of the clamped-at-0 lengths
    for (int q : c.ql)
        T += q > 0 ? q : 0;

    pa::Params p{};
    p.batch = B;
    p.num_q_tokens = (int)T;
    p.head_num = c.H;
    p.kv_head_num = c.Hkv;
    p.group = G;
    p.head_size_k = p.head_size_v = D;
    p.block_size = c.bs;
    p.bs_shift = (c.bs & (c.bs - 1)) == 0 ? __builtin_ctz(c.bs) : -1;
    p.max_blocks = c.mb;
    p.num_blocks = c.nb;
    p.max_q = c.max_q;
    p.causal = c.causal ? 1 : 0;
    p.rows_per_tile = RP;
    p.chunk = CT;
    auto l2 = [](int x) { return (x > 0 && (x & (x - 1)) == 0) ? __builtin_ctz((unsigned)x) : -1; };
    p.chunk_shift = l2(CT);
    p.group_shift = l2(G);
    p.tile_shift = l2(RP);
    p.max_tiles = (c.max_q * G + RP - 1) / RP;
    p.partitions = c.P;
    p.pieces = c.P;
    p.partial_stride = (int)(((size_t)RP * (D + 2) + 3) & ~(size_t)3);

    // workspace as pa_create sizes it for this variant: P pieces, 2 slots each
    std::vector<int32_t> hdr(8), cu_q(B + 1), wsb(B + 1), ipg(B), qlen(B), kvlen(B), wg_b(c.P), splits(8 * c.P);
    p.ws.hdr = hdr.data();
    p.ws.cu_q = cu_q.data();
    p.ws.wsb = wsb.data();
    p.ws.ipg = ipg.data();
    p.ws.qlen = qlen.data();
    p.ws.kvlen = kvlen.data();
    p.ws.wg_b = wg_b.data();
    p.ws.splits = splits.data();
    const long long part_size = 2LL * c.P * p.partial_stride;

    // ---- the plan kernel's reading of the lengths and its cut
    const int cap = pa::seq_cap(p);
    long long W = 0, tq = 0;
    for (int b = 0; b < B; ++b) {
        int kv = c.kv[b], ql = c.ql[b];
        (void)pa::sanitize_seq(p, cap, kv, ql);
        const int items = pa::seq_items_per_group(p, kv, ql) * c.Hkv;
        qlen[b] = ql;
        kvlen[b] = kv;
        ipg[b] = pa::seq_items_per_group(p, kv, ql);
        cu_q[b] = (int)tq;
        wsb[b] = (int)W;
        tq += ql;
        W += items;
    }
    cu_q[B] = (int)tq;
    wsb[B] = (int)W;
    const int per = (int)((W + p.pieces - 1) / p.pieces);
    hdr[0] = (int)W;
    hdr[1] = per > 0 ? per : 1;
    hdr[2] = p.pieces;
    const int pe = per > 0 ? per : 1;
    const int nk = (int)((W + pe - 1) / pe) < p.pieces ? (int)((W + pe - 1) / pe) : p.pieces;
    for (int k = 0; k < nk; ++k) {
        const int s = k * pe;
        int lo = 0, hi = B - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (wsb[mid] <= s)
                lo = mid;
            else
                hi = mid - 1;
        }
        wg_b[k] = lo;
        if (k == 0)
            continue;
        check(c, "split entry", (long long)(k - 1) * 8, 8, (long long)splits.size(), "plan");
        (void)pa::piece_start(p, k, s, s - pe, lo, kvlen[lo], qlen[lo], ipg[lo], wsb[lo], cu_q[lo], true);
    }
    for (int k = (int)((W + pe - 1) / pe); k < p.pieces; ++k)
        if (k > 0)
            splits[(size_t)(k - 1) * 8] = -1;

    // ---- the attention kernel: every worker, as the grid runs them
    const long long q_size = T * c.H * D, out_size = T * c.H * D, lse_size = T * c.H;
    const long long cache_size = c.nb * c.bs * c.Hkv * D;
    const long long bt_size = (long long)B * c.mb;
    const size_t row_stride = (size_t)c.Hkv * D;
    const int grid = (c.P + 3) / 4;
    std::vector<int> written(2 * c.P, 0);   // partial slots written
    for (int bid = 0; bid < grid; ++bid) {
        for (int wave = 0; wave < 4; ++wave) {
            int piece = pa::xcd_logical_index(bid, grid) * 4 + wave;
            pa::Cursor cu{};
            int end = 0;
            if (piece >= p.partitions || !pa::wg_range(p, piece, cu, end))
                continue;
            bool first_seg = true;
            int guard = 0;
            while (true) {
                if (++guard > 1 << 22)
                    fail(c, "worker does not finish");
                const int b = cu.b, g = cu.g;
                check(c, "sequence", b, 1, B, "segment");
                const int c0 = cu.c;
                const int c1 = cu.nch < c0 + (end - cu.item) ? cu.nch : c0 + (end - cu.item);
                if (c1 <= c0)
                    fail(c, "empty segment");
                const bool whole = (c0 == 0 && c1 == cu.nch);
                const int kv = kvlen[b], ql = qlen[b], rows = ql * G, t0 = cu_q[b];
                const int nvis = pa::tile_nvis(p, kv, ql, rows - 1);
                const size_t head_off = (size_t)g * D;
                for (int lane = 0; lane < 64; ++lane) {
                    const int kq = lane % L, grp = lane / L;
                    const int d0 = 8 * kq, d1 = D / 2 + 8 * kq;
                    // q of every row
                    for (int r = 0; r < RP; ++r) {
                        const int t = t0 + r / G;
                        if (r < rows && t < p.num_q_tokens) {
                            const long long src = (long long)pa::head_row(p, t, g, r) * D;
                            check(c, "query", src + d0, 8, q_size, "q load");
                            check(c, "query", src + d1, 8, q_size, "q load");
                        }
                    }
                    const int nblk = nvis > 0 ? pa::div_bs(nvis - 1, c.bs, p.bs_shift) + 1 : 1;
                    // block ids are fetched for c0, c0 + 1, ..., up to two chunks past
                    // the last computed one; chunks c0 .. c1 - 1 are loaded
                    for (int ch = c0; ch < c1 + 2; ++ch) {
                        for (int t = 0; t < TL; ++t) {
                            const int j = ch * CT + t * NG + grp;
                            const int col = pa::bt_column(j, c.bs, p.bs_shift, nblk);
                            check(c, "block table column", col, 1, c.mb, "id prefetch");
                            const long long bti = (long long)b * c.mb + col;
                            check(c, "block table", bti, 1, bt_size, "id prefetch");
                            if (ch >= c1)
                                continue;
                            const int blk = c.table[bti];
                            const bool inb = (unsigned)blk < (unsigned long long)c.nb;
                            const bool ok = j < nvis && inb;
                            const long long off =
                                (long long)pa::kv_row_elem(ok, blk, j, c.bs, p.bs_shift, row_stride, head_off);
                            check(c, "key cache", off + d0, 8, cache_size, "K load");
                            check(c, "key cache", off + d1, 8, cache_size, "K load");
                            check(c, "value cache", off + d0, 8, cache_size, "V load");
                            check(c, "value cache", off + d1, 8, cache_size, "V load");
                        }
                    }
                    if (whole) {
                        const int Wc = PER >= 8 ? 8 : PER;
                        for (int k0 = 0; k0 < PER; k0 += Wc) {
                            const int q = PER * grp + k0;
                            const int r = q / 16, e = q % 16;
                            const int t = t0 + r / G;
                            if (r < rows && t < p.num_q_tokens) {
                                const long long dst = (long long)pa::head_row(p, t, g, r) * D + pa::lane_col(e, d0, d1);
                                check(c, "output", dst, Wc, out_size, "output store");
                                if (e == 0 && kq == 0)
                                    check(c, "lse", (long long)pa::head_row(p, t, g, r), 1, lse_size, "lse store");
                            }
                        }
                    } else {
                        const int slot = first_seg ? 0 : 1;
                        const long long base = (long long)(2 * piece + slot) * p.partial_stride;
                        for (int k = 0; k < PER; ++k) {
                            const int q = PER * grp + k;
                            const int r = q / 16, e = q % 16;
                            const long long at = base + (long long)r * D + pa::lane_col(e, d0, d1);
                            if (at - base >= p.partial_stride)
                                fail(c, "partial store past its slot");
                            check(c, "partials", at, 1, part_size, "partial store");
                        }
                        if (lane < RP) {
                            check(c, "partials", base + RP * D + lane, 1, part_size, "partial max");
                            check(c, "partials", base + RP * D + RP + lane, 1, part_size, "partial sum");
                            if (RP * D + RP + lane >= p.partial_stride)
                                fail(c, "partial statistics past their slot");
                        }
                        written[2 * piece + slot] = 1;
                    }
                }
                first_seg = false;
                cu.item += c1 - c0;
                bool more = cu.item < end;
                if (more) {
                    pa::cursor_next_unit(p, cu);
                    more = cu.b < p.batch;
                }
                if (!more)
                    break;   // one piece per worker on this path
            }
        }
    }

    // ---- the merge kernel: the parts of every split entry
    for (int entry = 0; entry < p.pieces - 1; ++entry) {
        const int32_t *d = splits.data() + (size_t)entry * 8;
        if (d[0] < 0 || per <= 0)
            continue;
        const int us = d[3], ue = d[4];
        const int first = us / per, last = (ue - 1) / per;
        if (first < 0 || last >= p.pieces || first > last)
            fail(c, "split entry pieces out of range");
        const int slot_first = 2 * first + (first * per >= us ? 0 : 1);
        const int g = d[1], qt = d[2], t0 = d[5], rows = d[6];
        if (g < 0 || g >= c.Hkv || rows < 1 || rows > RP)
            fail(c, "split entry fields out of range");
        for (int k = first; k <= last; ++k) {
            const int slot = k == first ? slot_first : 2 * k;
            check(c, "partial slot", slot, 1, 2LL * c.P, "merge");
            if (!written[slot])
                fail(c, "merge reads a partial slot no worker wrote (piece " + std::to_string(k) + ")");
            for (int r = 0; r < rows; ++r) {
                const long long base = (long long)slot * p.partial_stride;
                check(c, "partials", base + (long long)RP * D + r, 1, part_size, "merge max");
                check(c, "partials", base + (long long)RP * D + RP + r, 1, part_size, "merge sum");
                check(c, "partials", base + (long long)r * D, D, part_size, "merge acc");
            }
        }
        for (int r = 0; r < rows; ++r) {
            const int rg = qt * RP + r;
            const int t = t0 + rg / G;
            if (t < p.num_q_tokens) {
                const long long o = ((long long)t * c.H + g * G + rg % G) * D;
                check(c, "output", o, D, out_size, "merge store");
                check(c, "lse", (long long)t * c.H + g * G + rg % G, 1, lse_size, "merge lse");
            }
        }
    }
}

// The tables of a well-formed case: sequences take consecutive ids of a
// shuffled block list, unused entries 0.
void fill_tables(Case &c, std::mt19937 &rng, int slack)
{
    const int B = (int)c.kv.size();
    int need = 0, mx = 1;
    for (int k : c.kv) {
        const int n = k > 0 ? (k + c.bs - 1) / c.bs : 0;
        need += n;
        mx = n > mx ? n : mx;
    }
    c.mb = mx;
    c.nb = need + slack > 0 ? need + slack : 1;
    std::vector<int> ids(c.nb);
    for (int i = 0; i < c.nb; ++i)
        ids[i] = i;
    std::shuffle(ids.begin(), ids.end(), rng);
    c.table.assign((size_t)B * c.mb, 0);
    int at = 0;
    for (int b = 0; b < B; ++b) {
        const int n = c.kv[b] > 0 ? (c.kv[b] + c.bs - 1) / c.bs : 0;
        for (int j = 0; j < n; ++j)
            c.table[(size_t)b * c.mb + j] = ids[at++];
    }
}

}  // namespace

int main()
{
    int cases = 0;
    std::mt19937 rng(20261203);
    // the recorded case, at several worker counts (the GPU ran 1024 workers)
    for (int P : {1024, 4096, 256, 8, 7, 1}) {
        Case c;
        c.kv = {50, 9, 200};
        c.ql = {4, 3, 1};
        c.H = 8;
        c.Hkv = 4;
        c.D = 128;
        c.bs = 16;
        c.P = P;
        c.causal = true;
        c.max_q = 4;
        std::mt19937 r2(12);
        fill_tables(c, r2, 5);
        c.name = "recorded causal case P=" + std::to_string(P);
        run(c);
        ++cases;
    }
    // the sweep
    const int Ds[] = {64, 128, 256};
    const int bss[] = {16, 32, 48, 64, 128, 256};
    const int Ps[] = {1, 3, 8, 64, 256, 1024, 2048, 4096};
    for (int it = 0; it < 1500; ++it) {
        Case c;
        const int G = 1 << (rng() % 4);            // 1, 2, 4, 8
        c.Hkv = 1 + rng() % 4;
        c.H = c.Hkv * G;
        c.D = Ds[rng() % 3];
        c.bs = bss[rng() % 6];
        c.P = Ps[rng() % 8];
        c.causal = rng() % 4 != 0;
        c.max_q = 1;
        while (c.max_q * 2 * G <= 8 && rng() % 2)
            c.max_q *= 2;
        c.max_q = c.max_q * G > 8 ? 8 / G : c.max_q;
        if (c.max_q < 1)
            c.max_q = 1;
        const int B = 1 + rng() % 40;
        for (int b = 0; b < B; ++b) {
            const int q = 1 + rng() % c.max_q;
            int k = (int)(rng() % (rng() % 3 == 0 ? 40 : 3000));
            if (c.causal && k < q)
                k = q;
            c.kv.push_back(k);
            c.ql.push_back(c.causal ? q : 1 + rng() % c.max_q);
        }
        fill_tables(c, rng, (int)(rng() % 10));
        // malformed inputs, which the kernels clamp and flag
        const int bad = rng() % 8;
        if (bad == 0 && !c.table.empty())
            c.table[rng() % c.table.size()] = (rng() % 2) ? -1 : 0x7fffffff;   // bad block id
        if (bad == 1)
            c.kv[rng() % B] += c.bs * (1 + rng() % 4);                         // table too short
        if (bad == 2)
            c.ql[rng() % B] = c.max_q + 3;                                      // q_seq_len too large
        if (bad == 3)
            c.kv[rng() % B] = -5;                                               // negative length
        if (bad == 4) {
            const int b = rng() % B;
            c.ql[b] = c.kv[b] + 1 <= c.max_q ? c.kv[b] + 1 : c.ql[b];          // q_seq_len above kv
        }
        c.name = "sweep " + std::to_string(it) + " B=" + std::to_string(B) + " G=" + std::to_string(G) +
                 " D=" + std::to_string(c.D) + " bs=" + std::to_string(c.bs) + " P=" + std::to_string(c.P) +
                 (c.causal ? " causal" : " none") + " bad=" + std::to_string(bad);
        run(c);
        ++cases;
    }
    std::printf("ok %d %lld\n", cases, g_accesses);
    return 0;
}

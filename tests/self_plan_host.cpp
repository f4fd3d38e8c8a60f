// Host-side check that the 576/512 tile kernel's own plan (pa_tile_kernels.h,
// tile_kernel with SELF) walks the same segments and writes the same split
// entries as the plan kernel's arrays do (plan_kernel, then wg_range and
// cursor_next_unit in the tile kernel without SELF).
//
// The planner's arithmetic (length clamping, item counts, piece starts and
// split entries, the plan-path cursor) is the library's own, from
// pa_internal.h compiled for the host.  This file repeats the control flow of
// both: the plan kernel's per-sequence arrays and cut, and the SELF prologue
// (one pass over the lengths with running sums, pieces of ceil(W / pieces)
// items, the bisection for the sequence holding a piece's first item, the
// whole-unit mode, and the step to the next unit that skips sequences without
// query rows).  For every worker it compares the list of segments (sequence,
// KV head, row tile, first chunk, chunks) and every split entry.
//
// Cases: seeded passes of one row tile per (sequence, KV head), as the host
// takes the kernel's own plan for them: group sizes 8 to 64 at 64 rows per
// tile, no mask, causal and band masks, sparse lists, empty and
// malformed lengths, 1 to 256 sequences, 1 to 600 workers, split and whole
// units.  Prints "ok <cases> <segments>" or the first difference.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <string>
#include <vector>

#include "pa_internal.h"

namespace {

struct Seg {
    int b, g, qt, c, n;
    bool operator==(const Seg &o) const { return b == o.b && g == o.g && qt == o.qt && c == o.c && n == o.n; }
};

long long g_segments = 0;

[[noreturn]] void fail(const std::string &name, const std::string &what)
{
    std::printf("FAIL %s: %s\n", name.c_str(), what.c_str());
    std::exit(1);
}

int l2(int x)
{
    return (x > 0 && (x & (x - 1)) == 0) ? __builtin_ctz((unsigned)x) : -1;
}

// A worker's segments from its cursor to `end`, stepping with `next`.
template <class Next>
std::vector<Seg> walk(const pa::Params &p, pa::Cursor cu, int end, Next next)
{
    std::vector<Seg> out;
    for (;;) {
        const int nseg = cu.nch < cu.c + (end - cu.item) ? cu.nch - cu.c : end - cu.item;
        out.push_back({cu.b, cu.g, cu.qt, cu.c, nseg});
        cu.item += nseg;
        if (cu.item >= end)
            break;
        next(cu);
        if (cu.b >= p.batch)
            break;
        if (out.size() > 1000000)
            return out;
    }
    return out;
}

std::string seg_str(const std::vector<Seg> &v)
{
    std::string s;
    for (const Seg &x : v)
        s += "(" + std::to_string(x.b) + "," + std::to_string(x.g) + "," + std::to_string(x.qt) + "," +
             std::to_string(x.c) + "," + std::to_string(x.n) + ")";
    return s.substr(0, 400);
}

void run(const std::string &name, const std::vector<int> &kv_in, const std::vector<int> &ql_in, int G, int Hkv,
         int chunk, int mask, int win_l, int win_r, int topk, int mb, int bs, int P, bool no_split)
{
    const int B = (int)kv_in.size();
    pa::Params p{};
    p.batch = B;
    p.head_num = G * Hkv;
    p.kv_head_num = Hkv;
    p.group = G;
    p.head_size_k = 576;
    p.head_size_v = 512;
    p.block_size = bs;
    p.bs_shift = l2(bs);
    p.max_blocks = mb;
    p.num_blocks = 1 << 20;
    int max_q = 1;
    for (int q : ql_in)
        max_q = std::max(max_q, q);
    p.max_q = max_q;
    p.causal = (mask == 1 || mask == 2) ? 1 : 0;
    p.band = mask == 2 ? 1 : 0;
    p.win_left = win_l;
    p.win_right = win_r;
    p.sparse = mask == 4 ? 1 : 0;
    p.topk = topk;
    p.rows_per_tile = 64;
    p.chunk = chunk;
    p.chunk_shift = l2(chunk);
    p.group_shift = l2(G);
    p.tile_shift = l2(64);
    p.max_tiles = (max_q * G + 63) / 64;
    if (p.max_tiles != 1)
        fail(name, "case has more than one row tile per unit");
    p.no_split = no_split ? 1 : 0;
    p.partitions = no_split ? B * Hkv : P;
    p.pieces = no_split ? 0 : P;
    const int cap = pa::seq_cap(p);

    // ---- the plan kernel's arrays and cut (plan path)
    std::vector<int32_t> hdr(8), cu_q(B + 1), wsb(B + 1), ipg(B), qlen(B), kvlen(B), wg_b(std::max(1, P)),
        splits_plan(8 * std::max(1, P), 12345), splits_self(8 * std::max(1, P), 12345);
    p.ws.hdr = hdr.data();
    p.ws.cu_q = cu_q.data();
    p.ws.wsb = wsb.data();
    p.ws.ipg = ipg.data();
    p.ws.qlen = qlen.data();
    p.ws.kvlen = kvlen.data();
    p.ws.wg_b = wg_b.data();
    long long W = 0, tq = 0;
    for (int b = 0; b < B; ++b) {
        int kv = kv_in[b], ql = ql_in[b];
        (void)pa::sanitize_seq(p, cap, kv, ql);
        qlen[b] = ql;
        kvlen[b] = kv;
        ipg[b] = pa::seq_items_per_group(p, kv, ql);
        cu_q[b] = (int)tq;
        wsb[b] = (int)W;
        tq += ql;
        W += (long long)ipg[b] * Hkv;
    }
    cu_q[B] = (int)tq;
    wsb[B] = (int)W;
    const int per = no_split ? 0 : (int)((W + p.pieces - 1) / p.pieces);
    hdr[0] = (int)W;
    hdr[1] = per > 0 ? per : (no_split ? 0 : 1);
    if (!no_split) {
        p.ws.splits = splits_plan.data();
        const int pe = per > 0 ? per : 1;
        const int nk = std::min((int)((W + pe - 1) / pe), p.pieces);
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
            if (k > 0)
                (void)pa::piece_start(p, k, s, s - pe, lo, kvlen[lo], qlen[lo], ipg[lo], wsb[lo], cu_q[lo], true);
        }
        for (int k = std::max(nk, 1); k < p.pieces; ++k)
            splits_plan[(size_t)(k - 1) * 8] = -1;
    }

    // ---- the kernel's own plan (SELF): one pass with running sums
    std::vector<int> s_kv(B), s_ql(B), s_t0(B), s_wsb(B + 1);
    {
        int lq = 0, lw = 0;
        for (int b = 0; b < B; ++b) {
            int kv = kv_in[b], ql = ql_in[b];
            (void)pa::sanitize_seq(p, cap, kv, ql);
            s_kv[b] = kv;
            s_ql[b] = ql;
            s_t0[b] = lq;
            s_wsb[b] = lw;
            lq += ql;
            lw += pa::seq_items_per_group(p, kv, ql) * Hkv;
        }
        s_wsb[B] = lw;
    }
    const int Ws = s_wsb[B];
    if (Ws != (int)W)
        fail(name, "item totals differ");
    auto self_next = [&](pa::Cursor &cu) {
        cu.c = 0;
        if (++cu.g >= Hkv) {
            cu.g = 0;
            do {
                ++cu.b;
            } while (cu.b < B && s_ql[cu.b] <= 0);
        }
        if (cu.b < B)
            cu.nch = pa::unit_chunks(p, s_kv[cu.b], s_ql[cu.b], 0);
    };
    auto plan_next = [&](pa::Cursor &cu) { pa::cursor_next_unit(p, cu); };

    for (int piece = 0; piece < p.partitions; ++piece) {
        // plan path
        pa::Cursor pc{};
        int pend = 0;
        const bool phave = pa::wg_range(p, piece, pc, pend);
        // own plan
        pa::Cursor sc{};
        int send = 0;
        bool shave = true;
        if (no_split) {
            const int b = piece / Hkv;
            shave = b < B && s_ql[b] > 0;
            if (shave) {
                sc.b = b;
                sc.g = piece - b * Hkv;
                sc.qt = 0;
                sc.c = 0;
                sc.ntile = pa::seq_tiles(p, s_ql[b]);
                sc.nch = pa::unit_chunks(p, s_kv[b], s_ql[b], 0);
                sc.item = s_wsb[b] + sc.g * sc.nch;
                send = sc.item + sc.nch;
            }
        } else {
            p.ws.splits = splits_self.data();
            const int sper = (Ws + p.pieces - 1) / p.pieces;
            const int s0 = piece * sper;
            if (sper <= 0 || s0 >= Ws) {
                if (piece > 0)
                    splits_self[(size_t)(piece - 1) * 8] = -1;
                shave = false;
            } else {
                send = std::min(s0 + sper, Ws);
                int lo = 0, hi = B - 1;
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (s_wsb[mid] <= s0)
                        lo = mid;
                    else
                        hi = mid - 1;
                }
                sc = pa::piece_start(p, piece, s0, s0 - sper, lo, s_kv[lo], s_ql[lo],
                                     pa::seq_items_per_group(p, s_kv[lo], s_ql[lo]), s_wsb[lo], s_t0[lo], true);
            }
        }
        if (phave != shave)
            fail(name, "worker " + std::to_string(piece) + ": has a piece on one path only");
        if (!phave)
            continue;
        if (pend != send)
            fail(name, "worker " + std::to_string(piece) + ": end items differ");
        const std::vector<Seg> a = walk(p, pc, pend, plan_next), s = walk(p, sc, send, self_next);
        if (!(a == s))
            fail(name, "worker " + std::to_string(piece) + ": plan " + seg_str(a) + " own " + seg_str(s));
        for (const Seg &x : s) {
            if (x.b < 0 || x.b >= B || x.g < 0 || x.g >= Hkv || x.qt != 0 || x.n <= 0 || x.c < 0)
                fail(name, "worker " + std::to_string(piece) + ": segment out of range " + seg_str(s));
            if (s_t0[x.b] != cu_q[x.b])
                fail(name, "first query rows differ");
        }
        g_segments += (long long)s.size();
    }
    if (!no_split)
        for (int e = 0; e + 1 < p.pieces; ++e)
            for (int j = 0; j < 7; ++j)
                if (splits_plan[(size_t)e * 8 + j] != splits_self[(size_t)e * 8 + j] &&
                    !(splits_plan[(size_t)e * 8] < 0 && splits_self[(size_t)e * 8] < 0))
                    fail(name, "split entry " + std::to_string(e) + " differs");
}

}  // namespace

int main()
{
    int cases = 0;
    std::mt19937 rng(2024);
    auto uni = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
    for (int it = 0; it < 3000; ++it) {
        const int G = 8 << uni(0, 3);                 // 8, 16, 32, 64
        const int Hkv = uni(1, 3) == 1 ? 2 : 1;
        const int mask = std::vector<int>{0, 0, 1, 2, 4}[uni(0, 4)];
        const int chunk = (mask == 4 || uni(0, 1)) ? 16 : 32;
        const int bs = std::vector<int>{16, 32, 64, 128}[uni(0, 3)];
        const int B = uni(0, 4) == 0 ? uni(200, 256) : uni(1, 40);
        const int qmax = std::max(1, 64 / G);         // one 64-row tile per unit
        const int mb = uni(1, 40);
        std::vector<int> kv(B), ql(B);
        for (int b = 0; b < B; ++b) {
            kv[b] = uni(0, 9) == 0 ? 0 : uni(1, mb * bs + (uni(0, 19) == 0 ? 300 : 0));   // some too long
            if (uni(0, 49) == 0)
                kv[b] = -uni(1, 5);                    // negative: clamped to 0
            ql[b] = mask == 0 && uni(0, 1) ? 1 : uni(0, qmax);
            if (mask == 1 || mask == 2)
                ql[b] = std::min(ql[b], std::max(0, kv[b]));
        }
        if (mask == 4)
            std::fill(ql.begin(), ql.end(), 1);
        const int P = uni(0, 3) == 0 ? uni(1, 8) : uni(9, 600);
        const bool no_split = uni(0, 5) == 0;
        const std::string name = "case" + std::to_string(it) + " G" + std::to_string(G) + " Hkv" +
                                 std::to_string(Hkv) + " mask" + std::to_string(mask) + " B" + std::to_string(B) +
                                 " P" + std::to_string(P) + (no_split ? " whole" : "");
        run(name, kv, ql, G, Hkv, chunk, mask, uni(0, 300), uni(0, 8), mask == 4 ? 16 * uni(1, 40) : 0, mb, bs, P,
            no_split);
        ++cases;
    }
    std::printf("ok %d %lld\n", cases, g_segments);
    return 0;
}

// Host-side check of the piece map the self-planning streaming kernel and the
// merge kernel share (pa::PieceMap): over a sweep of item counts, worker
// counts and tail minimums, the pieces tile [0, W) in index order without
// gaps or overlap, every claimed piece holds at least m items (the kernel
// claims a piece that many chunks ahead of its use), piece_of inverts
// piece_range, the static pieces and the claims cover every piece exactly
// once with the claims' sizes never growing, and the count stays within the
// (1 + kTailRounds) * P pieces the workspace holds.  Prints "ok <maps
// checked>" or the first violation.
#include <cstdio>
#include <vector>

#include "pa_internal.h"

using pa::PieceMap;

static int fail(const char *what, const PieceMap &pm, int k)
{
    std::printf("FAIL %s: W=%d per=%d a=%d m=%d P=%d nr=%d k=%d\n", what, pm.W, pm.per, pm.a, pm.m, pm.P, pm.nr, k);
    return 1;
}

static int check(const PieceMap &pm)
{
    const int n = pa::piece_count(pm);
    if (pm.m > 0 && (pm.nr < 1 || pm.nr > pa::kTailRounds))
        return fail("rounds out of range", pm, n);
    int expect = 0;
    std::vector<int> size(n);
    for (int k = 0; k < n; ++k) {
        int s0, s1;
        pa::piece_range(pm, k, s0, s1);
        if (s0 != expect)
            return fail("gap or overlap", pm, k);
        if (s1 < s0 || (pm.m > 0 && s1 == s0))
            return fail("empty piece", pm, k);
        for (int it : {s0, (s0 + s1) / 2, s1 - 1})
            if (s1 > s0 && pa::piece_of(pm, it) != k)
                return fail("piece_of", pm, k);
        size[k] = s1 - s0;
        expect = s1;
    }
    if (expect != pm.W)
        return fail("pieces do not end at W", pm, n);
    int a, b;
    pa::piece_range(pm, n, a, b);
    if (a != pm.W || b != pm.W)
        return fail("piece past the last is not empty", pm, n);
    if (pm.m <= 0)
        return 0;
    // every piece is a worker's static piece or exactly one claim
    std::vector<int> seen(n, 0);
    for (int w = 0; w < pm.P; ++w) {
        const int k = pa::static_piece(pm, w);
        if (k < 0 || k >= n || seen[k]++)
            return fail("static piece", pm, k);
        if (size[k] < 4 * pm.m - 1 || size[k] > pm.a + 1)
            return fail("static piece size", pm, k);
    }
    int prev = 1 << 30;
    for (int c = 0;; ++c) {
        const int k = pa::claimed_piece(pm, c);
        if (k < 0) {
            if (c != pm.nr * pm.P)
                return fail("claims end early", pm, c);
            break;
        }
        if (k >= n || seen[k]++)
            return fail("claimed piece twice or out of range", pm, k);
        if (size[k] < pm.m)
            return fail("claimed piece below the minimum", pm, k);
        // claims go round by round: sizes never grow, except in the last
        // round, whose pieces take what their tail has left (less than m
        // more than a piece of the round before)
        const bool last_round = (k + 1) % (1 + pm.nr) == 0;
        if (size[k] > prev && (!last_round || size[k] - prev >= pm.m))
            return fail("claimed pieces grow", pm, k);
        if (!last_round)
            prev = size[k];
    }
    for (int k = 0; k < n; ++k)
        if (seen[k] != 1)
            return fail("piece not covered", pm, k);
    return 0;
}

int main()
{
    long checked = 0;
    unsigned seed = 12345;
    auto rnd = [&](int lo, int hi) {   // uniform in [lo, hi]
        seed = seed * 1103515245u + 12345u;
        return lo + (int)((seed >> 8) % (unsigned)(hi - lo + 1));
    };
    const int Ps[] = {1, 8, 17, 256, 512, 768, 1024};
    const int ms[] = {5, 8, 16};
    for (int P : Ps) {
        for (int m : ms) {
            pa::Params p{};
            p.partitions = P;
            p.pieces = P;
            p.tail_min = m;
            // the self-planning map as the kernel builds it (a tail iff
            // W >= kTailMinShare m P)
            const int lo = pa::kTailMinShare * m * P;
            for (int t = 0; t < 300; ++t) {
                const int W = t < 100 ? rnd(lo, lo + m * P) : rnd(lo, t < 290 ? 4000 * P : 200000 * P);
                const PieceMap pm = pa::self_piece_map(p, W);
                if (pm.m != m)
                    return fail("no tail where one is due", pm, 0);
                if (check(pm))
                    return 1;
                ++checked;
            }
            // below the threshold: one piece per worker
            const PieceMap pm = pa::self_piece_map(p, lo - 1);
            if (pm.m != 0 || check(pm))
                return fail("short pass", pm, 0);
            ++checked;
        }
        // uniform maps (plan kernel): N pieces of ceil(W / N), some empty at the end
        for (int W : {1, 7, 1000, 123457}) {
            const int per = (W + P - 1) / P;
            const PieceMap pm{W, per, P, 0, P, 0};
            int expect = 0;
            for (int k = 0; k < P; ++k) {
                int s0, s1;
                pa::piece_range(pm, k, s0, s1);
                if (s0 != expect || s1 < s0)
                    return fail("uniform map", pm, k);
                if (s1 > s0 && pa::piece_of(pm, s0) != k)
                    return fail("uniform piece_of", pm, k);
                if (pa::static_piece(pm, k) != k || pa::claimed_piece(pm, 0) != -1)
                    return fail("uniform map has claims", pm, k);
                expect = s1;
            }
            if (expect != W)
                return fail("uniform map does not end at W", pm, P);
            ++checked;
        }
    }
    std::printf("ok %ld\n", checked);
    return 0;
}

// Host enumeration of the LDS loads of the matrix-core kernels
// (pa_tile_kernels.h): every global_load_lds instruction that the tile
// kernel and the one-wave streaming kernel issue for a list of problems,
// with the address of each of its 64 lanes computed as the kernels compute
// it (same planner helpers from pa_internal.h, same per-lane piece offsets,
// same zero-page, junk-slot, shared-K/V, sparse and mask-slab choices).
//
// Checks, per lane: the address lies inside the buffer it reads (query, K
// cache, V source, zero page, mask matrix, sparse lists, block table), the
// 16-byte piece lies inside its token row and head, and the LDS bytes it
// fills lie inside their stage.  A violation prints FAIL and exits 1.
//
// Reports, per instruction, how its 64 addresses split into one
// wave-uniform 64-bit base and a 32-bit unsigned per-lane offset, the form
// of the LDS load with a scalar base register:
//   group  base = the lane-independent part of the kernel's own address
//          expression (the 16-token group's row in the head, or the zero
//          page; for sparse loads the head's column of the cache); counted:
//          instructions whose base differs between lanes, and offsets
//          outside [0, 2^32);
//   head   base = the head's column of the cache (offset = token row times
//          row stride + piece): the largest offset, and the instructions
//          with an offset at or above 2^31 and 2^32;
//   span   lanes in more than one allocation (no common base exists), and
//          the largest spread between the lowest and highest lane address.
//
// The cases come from a text file (argument 1) that the test writes from
// the seeded input generators; the kernel shapes come from the library's own
// selection functions (linked from libpa.so), every variant that exists for
// a case's head sizes, mask kind and K/V sharing.
#include <algorithm>
#include <array>
#include <atomic>
#include <cinttypes>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <fstream>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "pa_internal.h"

namespace {

enum Buf { BQ = 0, BK, BV, BZ, BM, NBUF };
const char *kBufName[NBUF] = {"query", "key cache", "value source", "zero page", "mask matrix"};

enum { M_NONE = 0, M_CAUSAL, M_BAND, M_TENSOR, M_SPARSE };

struct Case {
    std::string name;
    int B, H, Hkv, DK, DV, bs, mb, mode, wl, wr, shared, topk;
    long long nb;
    std::vector<int> kv, ql, table, lists;
};

struct Stats {
    long long instr = 0, lanes = 0;
    long long group_nonuniform = 0, group_off_range = 0;
    uint64_t group_max = 0;
    uint64_t head_max = 0;
    long long head_ge31 = 0, head_ge32 = 0;
    long long multi_buf = 0;
    uint64_t span_max = 0;
    void add(const Stats &o)
    {
        instr += o.instr;
        lanes += o.lanes;
        group_nonuniform += o.group_nonuniform;
        group_off_range += o.group_off_range;
        group_max = group_max > o.group_max ? group_max : o.group_max;
        head_max = head_max > o.head_max ? head_max : o.head_max;
        head_ge31 += o.head_ge31;
        head_ge32 += o.head_ge32;
        multi_buf += o.multi_buf;
        span_max = span_max > o.span_max ? span_max : o.span_max;
    }
};

// one lane of one instruction
struct Lane {
    int buf;
    long long addr;    // byte offset from the start of buffer `buf`
    long long gbase;   // the kernel's lane-independent part (same buffer)
    long long hbase;   // the head's column of the cache (-1: not a cache read)
};

std::string g_case;
std::atomic<long long> g_checks{0};
thread_local long long t_checks = 0;

// where the enumeration is (printed with a violation only)
struct Pos {
    std::string kernel;
    int b = -1, g = -1, qt = -1, ch = -1;
    const char *load = "";
};
thread_local Pos g_pos;

[[noreturn]] void fail(const std::string &what)
{
    static std::mutex mu;
    std::lock_guard<std::mutex> lock(mu);
    std::printf("FAIL %s: %s at %s b %d g %d qt %d chunk %d %s\n", g_case.c_str(), what.c_str(),
                g_pos.kernel.c_str(), g_pos.b, g_pos.g, g_pos.qt, g_pos.ch, g_pos.load);
    std::fflush(stdout);
    std::_Exit(1);
}

void check_index(const char *what, long long i, long long n)
{
    ++t_checks;
    if (i < 0 || i >= n)
        fail(std::string(what) + " index " + std::to_string(i) + " outside [0, " + std::to_string(n) + ")");
}

// One instruction: bounds of every lane, then the scalar-base splits.
void instr(Stats &st, const Lane *ln, int width, const long long *bufsize, const char *load)
{
    g_pos.load = load;
    ++st.instr;
    st.lanes += 64;
    bool multi = false, nonuni = false, grange = false;
    long long lo = ln[0].addr, hi = ln[0].addr;
    for (int l = 0; l < 64; ++l) {
        const Lane &x = ln[l];
        ++t_checks;
        if (x.addr < 0 || x.addr + width > bufsize[x.buf])
            fail(std::string(kBufName[x.buf]) + " byte " + std::to_string(x.addr) + " (+" + std::to_string(width) +
                 ") outside [0, " + std::to_string(bufsize[x.buf]) + ") lane " + std::to_string(l));
        if (x.buf != ln[0].buf)
            multi = true;
        if (x.buf != ln[0].buf || x.gbase != ln[0].gbase)
            nonuni = true;
        const long long goff = x.addr - x.gbase;
        if (goff < 0 || goff >= (1LL << 32))
            grange = true;
        if ((uint64_t)goff > st.group_max && goff >= 0)
            st.group_max = (uint64_t)goff;
        if (x.hbase >= 0) {
            const long long hoff = x.addr - x.hbase;
            if (hoff < 0)
                fail("head offset below the head's column");
            if ((uint64_t)hoff > st.head_max)
                st.head_max = (uint64_t)hoff;
        }
        if (x.buf == ln[0].buf) {
            lo = x.addr < lo ? x.addr : lo;
            hi = x.addr > hi ? x.addr : hi;
        }
    }
    // an instruction counts once for the head thresholds (its largest offset)
    long long hmax = -1;
    for (int l = 0; l < 64; ++l)
        if (ln[l].hbase >= 0 && ln[l].addr - ln[l].hbase > hmax)
            hmax = ln[l].addr - ln[l].hbase;
    if (hmax >= (1LL << 31))
        ++st.head_ge31;
    if (hmax >= (1LL << 32))
        ++st.head_ge32;
    if (multi)
        ++st.multi_buf;
    if (nonuni)
        ++st.group_nonuniform;
    if (grange)
        ++st.group_off_range;
    if (!multi && (uint64_t)(hi - lo) > st.span_max)
        st.span_max = (uint64_t)(hi - lo);
}

int vswz(int rb, int r)
{
    return rb % 256 == 0 ? 2 * (r & 7) : (r & 7);
}

int l2(int x)
{
    return (x > 0 && (x & (x - 1)) == 0) ? __builtin_ctz((unsigned)x) : -1;
}

struct Shape {
    bool stream;
    int mb, kt, nw, cs, s;
    bool sh;   // V read out of the K tile in LDS
    int hp;    // KV heads per unit (2: the streaming kernel on head pairs)
};

// Every load of one kernel shape over one case.  st[0]: K/V loads, st[1]:
// Q tile loads (streaming kernel), st[2]: mask slab loads.
void run(const Case &c, const Shape &sh, Stats stv[3])
{
    // (head pairs: the pass runs with G and Hkv taken per pair of KV heads)
    const int HP = sh.hp, Hkv = c.Hkv / HP;
    const int B = c.B, G = c.H / c.Hkv * HP, DK = c.DK, DV = c.DV;
    const bool BAND = c.mode == M_BAND, TMASK = c.mode == M_TENSOR, SPARSE = c.mode == M_SPARSE;
    const int R = sh.stream ? 16 : 16 * sh.mb * (sh.nw / sh.cs);
    const int KT = sh.kt, NTT = KT / 16, NW = sh.stream ? 1 : sh.nw;
    const int RBK = 2 * DK * HP, RBV = 2 * DV * HP, RBQ = 2 * DK;
    const int IPGK = RBK / 64, IPGV = sh.sh ? 0 : RBV / 64, IPGQ = RBQ / 64;
    const int MK = sh.stream ? IPGK : (IPGK + NW - 1) / NW;
    const int MV = sh.stream ? IPGV : (IPGV + NW - 1) / NW;
    const bool PAD = !sh.stream && (MK * NW != IPGK || MV * NW != IPGV);
    const int SDW = (KT + 2) / 2;
    const int SLB = ((R * SDW + 63) / 64) * 256;
    const long long STK = (long long)KT * RBK, STV = (long long)KT * RBV;
    if (c.bs % 16 != 0)
        fail("block size not a multiple of 16 on a matrix-core path");

    long long T = 0;
    for (int q : c.ql)
        T += q > 0 ? q : 0;
    pa::Params p{};
    p.batch = B;
    p.num_q_tokens = (int)T;
    p.head_num = c.H;
    p.kv_head_num = Hkv;
    p.group = G;
    p.head_size_k = DK;
    p.head_size_v = DV;
    p.block_size = c.bs;
    p.bs_shift = l2(c.bs);
    p.max_blocks = c.mb;
    p.num_blocks = c.nb;
    int maxq = 1;
    for (int q : c.ql)
        maxq = q > maxq ? q : maxq;
    p.max_q = maxq;
    p.causal = (c.mode == M_CAUSAL || c.mode == M_BAND) ? 1 : 0;
    p.band = BAND ? 1 : 0;
    p.win_left = BAND ? c.wl : 0;
    p.win_right = BAND ? c.wr : 0;
    p.sparse = SPARSE ? 1 : 0;
    p.topk = SPARSE ? c.topk : 0;
    p.rows_per_tile = R;
    p.chunk = KT;
    p.chunk_shift = l2(KT);
    p.group_shift = l2(G);
    p.tile_shift = l2(R);

    // buffers, in bytes, as the library sizes or takes them
    const long long rsk = (long long)Hkv * RBK;                                     // K token row
    const long long rsv = (long long)c.Hkv * 2 * (c.shared ? DK : DV);              // V source token row
    const long long vhead = 2LL * (c.shared ? DK : DV) * HP;                        // V source head stride
    long long bufsize[NBUF];
    bufsize[BQ] = T * c.H * DK * 2;
    bufsize[BK] = c.nb * c.bs * rsk;
    bufsize[BV] = c.nb * c.bs * rsv;
    bufsize[BZ] = 16LL * c.Hkv * (DK > DV ? DK : DV) * 2;
    bufsize[BM] = 2048LL * 2048 * 2;
    const int vbuf = c.shared ? BK : BV;   // the V source is the K cache itself
    if (c.shared)
        bufsize[BV] = bufsize[BK];

    // the plan kernel's reading of the lengths
    const int cap = pa::seq_cap(p);
    std::vector<int> kvl(B), qll(B), cu(B + 1);
    long long tq = 0;
    for (int b = 0; b < B; ++b) {
        int kv = c.kv[b], ql = c.ql[b];
        (void)pa::sanitize_seq(p, cap, kv, ql);
        kvl[b] = kv;
        qll[b] = ql;
        cu[b] = (int)tq;
        tq += ql;
    }

    // sequences are independent: a pool of threads takes them in turn, each
    // with statistics of its own
    const std::string kname = sh.stream ? "stream" : ("tile MB" + std::to_string(sh.mb) + " KT" + std::to_string(KT));
    std::atomic<int> next_b{0};
    const int nthr = std::max(1, std::min(8, (int)std::thread::hardware_concurrency()));
    std::vector<std::array<Stats, 3>> tst(nthr);
    auto worker = [&](int ti) {
        Stats *st = tst[ti].data();
        Lane ln[64];
        g_pos.kernel = kname;
        std::vector<int> rows;   // sparse: cache row of each list entry of the unit (-1: skipped)
        for (int b = next_b++; b < B; b = next_b++) {
            const int kv = kvl[b], ql = qll[b];
            const int ntile = pa::seq_tiles(p, ql);
            const int prefix = pa::seq_prefix(kv, ql);
            const int t0 = cu[b];
            for (int g = 0; g < Hkv; ++g) {
                const long long kgh = (long long)g * RBK;      // head column, K cache
                const long long vgh = (long long)g * vhead;    // head column, V source
                for (int qt = 0; qt < ntile; ++qt) {
                    const int nch = pa::unit_chunks(p, kv, ql, qt);
                    const int cb = BAND ? pa::unit_first_chunk(p, kv, ql, qt) : 0;
                    int rows_tile = ql * G - qt * R;
                    rows_tile = rows_tile < R ? rows_tile : R;
                    const int nvis = SPARSE ? kv
                                            : (BAND ? pa::row_hi_t<true>(p, kv, prefix, (qt * R + rows_tile - 1) / G)
                                                    : pa::row_hi_t<false>(p, kv, prefix, (qt * R + rows_tile - 1) / G));
                    const int nblk = nvis > 0 ? pa::div_bs(nvis - 1, c.bs, p.bs_shift) + 1 : 1;
                    const int lo_tile = BAND ? pa::row_lo_t<true>(p, prefix, (qt * R) / G) : 0;
                    g_pos.b = b;
                    g_pos.g = g;
                    g_pos.qt = qt;
                    g_pos.ch = -1;
                    if (nch < 1)
                        fail("unit without chunks");

                    // sparse: the unit's list entries resolved to cache rows
                    if (SPARSE) {
                        const int itok = (qt * R) / G;
                        const bool lst_ok = t0 + itok < p.num_q_tokens;
                        const int lim_c = prefix + itok + 1 < kv ? prefix + itok + 1 : kv;
                        rows.assign((size_t)nch * 16, -1);
                        for (int k = 0; k < nch * 16; ++k) {
                            if (!(lst_ok && k < p.topk))
                                continue;
                            const long long li = ((long long)(t0 + itok) * c.Hkv + g) * c.topk + k;
                            check_index("sparse list", li, (long long)c.lists.size());
                            const int ci = c.lists[li];
                            if (ci >= 0 && ci < lim_c) {
                                const int col = pa::div_bs(ci, c.bs, p.bs_shift);
                                check_index("block table column", col, c.mb);
                                const int blk = c.table[(size_t)b * c.mb + col];
                                if ((unsigned)blk < (unsigned)(c.nb < 0x7fffffff ? c.nb : 0x7fffffff)) {
                                    const uint32_t r = (uint32_t)blk * (uint32_t)c.bs + (uint32_t)pa::mod_bs(ci, c.bs, p.bs_shift);
                                    if (r > 0x7fffffffu)
                                        fail("sparse cache row above 2^31 - 1");
                                    rows[k] = (int)r;
                                }
                            }
                        }
                    }

                    // streaming kernel: the unit's Q tile, loaded with its first
                    // chunk (rows past the unit read the zero page)
                    if (sh.stream) {
                        for (int m = 0; m < IPGQ; ++m) {
                            for (int l = 0; l < 64; ++l) {
                                const int x = m * 1024 + 16 * l;
                                const int qrow = x / RBQ;
                                const int qlp = ((x % RBQ) >> 4) ^ (qrow & 7);
                                if (16 * qlp + 16 > RBQ)
                                    fail("Q piece past its row");
                                const int rg = qt * 16 + qrow;
                                const int t = t0 + rg / G;
                                const bool ok = qrow < rows_tile && t < p.num_q_tokens;
                                if (ok) {
                                    const long long a = (((long long)t * c.H + g * G + rg % G) * DK + 8 * qlp) * 2;
                                    ln[l] = Lane{BQ, a, 0, -1};
                                } else {
                                    ln[l] = Lane{BZ, 16LL * qlp, 0, -1};
                                }
                                if (m * 1024 + 16 * l + 16 > 16 * RBQ)
                                    fail("Q tile LDS write past its stage");
                            }
                            instr(st[1], ln, 16, bufsize, "Q");
                        }
                    }

                    for (int ch = cb; ch < cb + nch; ++ch) {
                        g_pos.ch = ch;
                        // tensor mask slab of the chunk
                        if (TMASK) {
                            const int c0m = ch * KT - prefix;
                            const int i0 = (qt * R) / G;
                            int i1 = (qt * R + rows_tile - 1) / G;
                            i1 = i1 < 2047 ? i1 : 2047;
                            int nim = i1 - i0 + 1;
                            nim = nim > 0 ? nim : 0;
                            if (c0m < 2048 && c0m + KT > 0 && nim > 0) {
                                int cs = c0m & ~1;
                                cs = cs < 0 ? 0 : (cs > 2048 - 2 * SDW ? 2048 - 2 * SDW : cs);
                                const int ntot = nim * SDW;
                                const int nin = (ntot + 63) / 64;
                                for (int m = 0; m < nin; ++m) {
                                    for (int l = 0; l < 64; ++l) {
                                        const int x = m * 64 + l;
                                        const int r = x / SDW;
                                        const long long a = x < ntot ? ((long long)(i0 + r) * 2048 + cs) * 2 + 4 * (x - r * SDW) : 0;
                                        ln[l] = Lane{BM, a, 0, -1};
                                    }
                                    if ((long long)m * 256 + 256 > SLB)
                                        fail("mask slab LDS write past its stage");
                                    instr(st[2], ln, 4, bufsize, "mask");
                                }
                            }
                        }
                        // K and V of each 16-token group of the chunk
                        for (int q = 0; q < NTT; ++q) {
                            const int j0 = ch * KT + 16 * q;
                            int gbuf_k = BZ, gbuf_v = BZ;
                            long long gk = 0, gv = 0;
                            if (!SPARSE) {
                                const bool vis = j0 < nvis && (!BAND || j0 + 16 > lo_tile);
                                int col = pa::div_bs(j0, c.bs, p.bs_shift);
                                col = col < nblk ? col : nblk - 1;
                                check_index("block table column", col, c.mb);
                                const int bid = c.table[(size_t)b * c.mb + col];
                                const bool inb = (unsigned)bid < (unsigned)(c.nb < 0x7fffffff ? c.nb : 0x7fffffff);
                                const long long trow = (long long)(uint32_t)bid * c.bs + pa::mod_bs(j0, c.bs, p.bs_shift);
                                if (vis && inb) {
                                    gbuf_k = BK;
                                    gk = kgh + trow * rsk;
                                    gbuf_v = vbuf;
                                    gv = vgh + trow * rsv;
                                }
                            }
                            for (int w = 0; w < NW; ++w) {
                                for (int m = 0; m < MK; ++m) {
                                    const int i = sh.stream ? m : w + NW * m;
                                    const bool real = !PAD || i < IPGK;
                                    for (int l = 0; l < 64; ++l) {
                                        const int x = i * 1024 + 16 * l;
                                        const int row = x / RBK;
                                        const int piece = ((x % RBK) >> 4) ^ (row & 7);
                                        if (real && 16 * piece + 16 > RBK)
                                            fail("K piece past its row");
                                        const long long vo = real ? (long long)(SPARSE ? 0 : row * rsk) + 16 * piece : 16LL * l;
                                        if (SPARSE) {
                                            const int rv = rows[(size_t)(ch - cb) * 16 + row];
                                            const long long rl = rv >= 0 ? rv : 0;
                                            ln[l] = real ? Lane{BK, kgh + rl * rsk + vo, kgh, kgh} : Lane{BZ, vo, 0, -1};
                                        } else if (real && gbuf_k == BK) {
                                            ln[l] = Lane{BK, gk + vo, gk, kgh};
                                        } else {
                                            ln[l] = Lane{BZ, vo, 0, -1};
                                        }
                                        const long long dst = real ? (long long)(q * IPGK + i) * 1024 + 16 * l : 16LL * l;
                                        if (dst + 16 > (real ? STK : 1024))
                                            fail("K LDS write past its stage");
                                    }
                                    instr(st[0], ln, 16, bufsize, "K");
                                }
                                for (int m = 0; m < MV; ++m) {
                                    const int i = sh.stream ? m : w + NW * m;
                                    const bool real = !PAD || i < IPGV;
                                    for (int l = 0; l < 64; ++l) {
                                        const int x = i * 1024 + 16 * l;
                                        const int row = x / RBV;
                                        const int piece = ((x % RBV) >> 4) ^ vswz(RBV, row);
                                        if (real && 16 * piece + 16 > RBV)
                                            fail("V piece past its row");
                                        const long long vo = real ? (long long)(SPARSE ? 0 : row * rsv) + 16 * piece : 16LL * l;
                                        if (SPARSE) {
                                            const int rv = rows[(size_t)(ch - cb) * 16 + row];
                                            const long long rl = rv >= 0 ? rv : 0;
                                            ln[l] = real ? Lane{vbuf, vgh + rl * rsv + vo, vgh, vgh} : Lane{BZ, vo, 0, -1};
                                        } else if (real && gbuf_v != BZ) {
                                            ln[l] = Lane{vbuf, gv + vo, gv, vgh};
                                        } else {
                                            ln[l] = Lane{BZ, vo, 0, -1};
                                        }
                                        const long long dst = real ? (long long)(q * IPGV + i) * 1024 + 16 * l : 16LL * l;
                                        if (dst + 16 > (real ? STV : 1024))
                                            fail("V LDS write past its stage");
                                    }
                                    instr(st[0], ln, 16, bufsize, "V");
                                }
                            }
                        }
                    }
                }
            }
        }
        g_checks += t_checks;
        t_checks = 0;
    };
    std::vector<std::thread> pool;
    for (int ti = 0; ti < nthr; ++ti)
        pool.emplace_back(worker, ti);
    for (auto &t : pool)
        t.join();
    for (auto &a : tst)
        for (int i = 0; i < 3; ++i)
            stv[i].add(a[i]);
}

bool read_ints(std::ifstream &in, std::vector<int> &v, size_t n)
{
    v.resize(n);
    for (size_t i = 0; i < n; ++i)
        if (!(in >> v[i]))
            return false;
    return true;
}

void print_stats(const char *what, const Stats &s)
{
    std::printf(" %s instr %lld group_nonuniform %lld group_off_range %lld group_max %" PRIu64
                " head_max %" PRIu64 " head_ge31 %lld head_ge32 %lld multi_buf %lld span_max %" PRIu64,
                what, s.instr, s.group_nonuniform, s.group_off_range, s.group_max, s.head_max, s.head_ge31,
                s.head_ge32, s.multi_buf, s.span_max);
}

}  // namespace

int main(int argc, char **argv)
{
    if (argc < 2) {
        std::printf("usage: lds_load_addr_host CASES\n");
        return 2;
    }
    std::ifstream in(argv[1]);
    std::string tag;
    int ncases = 0;
    Stats total[3];
    while (in >> tag) {
        if (tag != "case")
            fail("bad case file near '" + tag + "'");
        Case c;
        in >> c.name >> c.B >> c.H >> c.Hkv >> c.DK >> c.DV >> c.bs >> c.nb >> c.mb >> c.mode >> c.wl >> c.wr >>
            c.shared >> c.topk;
        g_case = c.name;
        if (!read_ints(in, c.kv, c.B) || !read_ints(in, c.ql, c.B) || !read_ints(in, c.table, (size_t)c.B * c.mb))
            fail("truncated case");
        long long tt = 0;
        for (int q : c.ql)
            tt += q > 0 ? q : 0;
        if (c.mode == M_SPARSE && !read_ints(in, c.lists, (size_t)tt * c.Hkv * c.topk))
            fail("truncated lists");
        // every kernel shape the library has for this case
        const int mode = c.mode == M_BAND ? 1 : c.mode == M_TENSOR ? 2 : c.mode == M_SPARSE ? 3 : 0;
        std::vector<Shape> shapes;
        for (int v = 0; v <= 7; ++v) {
            pa::TileShape t{};
            const void *k = mode == 1 ? pa::tile_kernel_band(0, c.DK, c.DV, v, c.shared != 0, &t)
                          : mode == 2 ? pa::tile_kernel_tensor(0, c.DK, c.DV, v, c.shared != 0, &t)
                          : mode == 3 ? pa::tile_kernel_sparse(0, c.DK, c.DV, v, c.shared != 0, &t)
                                      : pa::tile_kernel_plain(0, c.DK, c.DV, v, c.shared != 0, &t);
            if (!k)
                continue;
            // variants 5 to 7: the streaming kernel on head pairs (the library
            // takes them for an even number of KV heads)
            const int hp = v >= 5 ? 2 : 1;
            if (hp == 2 && c.Hkv % 2 != 0)
                continue;
            Shape s{pa::tile_streaming(c.DK, c.DV, v), t.mb, t.kt, t.nw, t.cs, t.s,
                    c.shared != 0 && c.DK > 256,   // only the 576/512 instances read V out of the K tile
                    hp};
            if (!s.stream && pa::tile_rows(c.DK, c.DV, v, c.shared != 0, mode) != 16 * t.mb * (t.nw / t.cs))
                fail("tile rows disagree with the shape of variant " + std::to_string(v));
            bool dup = false;
            for (const Shape &o : shapes)
                dup |= o.stream == s.stream && o.mb == s.mb && o.kt == s.kt && o.nw == s.nw && o.cs == s.cs &&
                       o.sh == s.sh && o.hp == s.hp;
            if (!dup)
                shapes.push_back(s);
        }
        if (shapes.empty())
            fail("no matrix-core kernel for the case");
        for (const Shape &s : shapes) {
            Stats st[3];
            run(c, s, st);
            std::printf("case %s kernel %s%s_MB%d_KT%d_NW%d", c.name.c_str(), s.stream ? "stream" : "tile",
                        s.hp > 1 ? "_pairs" : "", s.mb, s.kt, s.nw);
            print_stats("kv", st[0]);
            print_stats("q", st[1]);
            print_stats("mask", st[2]);
            std::printf("\n");
            for (int i = 0; i < 3; ++i)
                total[i].add(st[i]);
        }
        ++ncases;
    }
    std::printf("total");
    print_stats("kv", total[0]);
    print_stats("q", total[1]);
    print_stats("mask", total[2]);
    std::printf("\nok %d %lld\n", ncases, g_checks.load());
    return 0;
}

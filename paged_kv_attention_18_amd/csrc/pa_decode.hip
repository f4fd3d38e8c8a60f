// pa_decode.hip -- split-KV paged-attention decode on the vector ALUs (gfx950).
//
// For units of at most 4 rows (rows = query tokens x query heads of one GQA
// group) by default, where the contraction is too thin for the matrix cores;
// built for up to 8.  (From 5 rows on the MFMA kernel with one padded 16-row
// block streams faster: this kernel keeps its chunks in registers, and the
// accumulators of more rows leave room for fewer bytes in flight.)
//
// Every wave is an independent worker: the planner hands it a contiguous
// range of (sequence, KV head, chunk) items and it streams them with its own
// online-softmax state, so the chunk loop has no LDS traffic and no barriers;
// latency is hidden by the other waves resident on the CU.
//
// Lane layout: the L = D / 16 lanes of a "token group" share one KV token;
// lane kq of the group owns head dimensions [8 kq, 8 kq + 8) and
// [D/2 + 8 kq, D/2 + 8 kq + 8), for K (in QK) and for V / the output (in PV),
// so each 128-bit load instruction of the wave reads 64 / L whole half-rows of
// D/2 contiguous elements.  A chunk is CT = TL * (64 / L) tokens: every lane
// handles TL of them (4 for up to 4 rows, 2 for 8 rows, to bound the
// registers).
//
//   gather  token j -> block_tables[b][j / block_size], slot j % block_size
//           (Ascend ATB PagedAttentionOperation, Constraints); block ids are
//           fetched one chunk ahead; tokens past the visible range are never
//           loaded (their registers are zeroed).
//   QK      v_dot2_f32_{f16,bf16} over the lane's 16 dims for every row, then
//           a DPP all-reduce over the token group: every lane holds the whole
//           scores of its tokens.
//   softmax the chunk max of each row over the wave's tokens (3 cross-lane
//           steps), running max / sum in the log2 domain; masked positions
//           are set to -inf by select and get weight exactly 0.
//   PV      fp32 FMA of p into the lane's 16 output columns for every row.
//
// At the end of a unit's range the wave sums its lanes' accumulators
// (transposing reduction over the token groups) and writes either the
// normalised output (whole unit) or an fp32 partial (acc, m, l) for the
// merge kernel.
#include "pa_internal.h"

namespace pa {

namespace {

template <int DT>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
{
    if constexpr (DT == 0) {
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, a), __builtin_bit_cast(h2, b), c, false);
    } else {
        typedef __bf16 b2 __attribute__((ext_vector_type(2)));
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, a), __builtin_bit_cast(b2, b), c,
                                               false);
    }
}

// Value of lane ^ D exactly (D = 8: DPP row_ror:8, which is lane ^ 8 inside
// each row of 16 lanes; otherwise a lane permute).
template <int D>
__device__ __forceinline__ float xor_swap(float v)
{
    const int x = __builtin_bit_cast(int, v);
    int r;
    if constexpr (D == 8)
        r = __builtin_amdgcn_mov_dpp(x, 0x128, 0xf, 0xf, false);   // row_ror:8
    else
        r = __shfl_xor(x, D);
    return __builtin_bit_cast(float, r);
}

// Transposing reduction across the token groups of a wave.  Lanes l and
// l ^ D (D = L .. 32) hold partial sums of the same NV quantities; on exit
// lane l holds the full sums of quantities (NV / G) * (l / L) + k,
// k < NV / G, where G = 64 / L is the number of token groups.
template <int NV, int D, int L, int N>
__device__ __forceinline__ void slot_treduce(float (&v)[N], int lane)
{
    if constexpr (D >= L) {
        const bool upper = (lane & D) != 0;
#pragma unroll
        for (int k = 0; k < NV / 2; ++k) {
            const float keep = upper ? v[k + NV / 2] : v[k];
            const float send = upper ? v[k] : v[k + NV / 2];
            v[k] = keep + xor_swap<D>(send);
        }
        slot_treduce<NV / 2, D / 2, L>(v, lane);
    }
}

// Max / sum over the token groups: lanes l ^ D for D = L .. 32, i.e. the
// lanes that hold the same row slot in the other token groups.
template <int L>
__device__ __forceinline__ float slots_max(float v)
{
    if constexpr (L <= 32)
        v = fmaxf(v, xor_swap<32>(v));
    if constexpr (L <= 16)
        v = fmaxf(v, xor_swap<16>(v));
    if constexpr (L <= 8)
        v = fmaxf(v, xor_swap<8>(v));
    if constexpr (L <= 4)
        v = fmaxf(v, xor_swap<4>(v));
    return v;
}

template <int L>
__device__ __forceinline__ float slots_sum(float v)
{
    if constexpr (L <= 32)
        v += xor_swap<32>(v);
    if constexpr (L <= 16)
        v += xor_swap<16>(v);
    if constexpr (L <= 8)
        v += xor_swap<8>(v);
    if constexpr (L <= 4)
        v += xor_swap<4>(v);
    return v;
}

// Two 16-bit values packed as (lo, hi) with round to nearest even.
template <int DT>
__device__ __forceinline__ uint32_t pack_pair(float lo, float hi)
{
    if constexpr (DT == 0) {
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        const h2 v = {(_Float16)lo, (_Float16)hi};
        return __builtin_bit_cast(uint32_t, v);
    } else {
        typedef __bf16 b2 __attribute__((ext_vector_type(2)));
        const b2 v = {(__bf16)lo, (__bf16)hi};
        return __builtin_bit_cast(uint32_t, v);
    }
}

template <int DT, int D, int RP>
__global__ __launch_bounds__(kThreads) void decode_kernel(Params p)
{
    constexpr int L = D / 16;          // lanes per token group
    constexpr int NG = 64 / L;         // token groups per wave
    constexpr int TL = RP <= 4 ? 4 : 2;   // tokens per lane per chunk
    static_assert(RP <= 8, "more than 8 rows per unit take the MFMA kernel");
    constexpr int CT = TL * NG;        // tokens per chunk
    constexpr int NQ = RP * 16;        // accumulator values per lane
    constexpr int NRL = RP >= L ? RP / L : 1;   // rows a lane holds after the QK reduction
    static_assert(L >= 4 && L <= 16 && (L & (L - 1)) == 0, "D must be 64, 128 or 256");
    static_assert(TL % 2 == 0, "PV pairs tokens");

    const int lane = threadIdx.x & 63;
    const int kq = lane % L;
    const int grp = lane / L;
    const int wave = threadIdx.x >> 6;
    int piece = xcd_logical_index(blockIdx.x, gridDim.x) * (kThreads / 64) + wave;
    Cursor cu;
    int end;
    if (piece >= p.partitions || !wg_range(p, piece, cu, end))
        return;

    const uint16_t *__restrict__ qg = (const uint16_t *)p.query;
    const uint16_t *__restrict__ kg = (const uint16_t *)p.key_cache;
    const uint16_t *__restrict__ vg = (const uint16_t *)p.value_cache;
    uint16_t *__restrict__ og = (uint16_t *)p.out;
    const int G = p.group;
    const int bs = p.block_size;
    const int bsh = p.bs_shift;
    const size_t row_stride = (size_t)p.kv_head_num * D;
    const int d0 = 8 * kq, d1 = D / 2 + 8 * kq;   // this lane's two 8-element pieces
    const int gbase = grp * L;                    // first lane of this token group
    // After the transposing QK reduction lane kq of a group holds the score of
    // row own_row(k) (k < NRL); row r lives in lane holder(r), slot r % NRL.
    auto own_row = [&](int k) __attribute__((always_inline)) {
        return RP >= L ? NRL * kq + k : kq / (L / RP);
    };
    auto holder = [](int r) { return RP >= L ? r / NRL : r * (L / RP); };
    uint32_t err = 0;
    bool first_seg = true;

    while (true) {
        // ----------------------------------------------------------- segment
        const int b = cu.b, g = cu.g;
        const int c0 = cu.c;
        const int c1 = cu.nch < c0 + (end - cu.item) ? cu.nch : c0 + (end - cu.item);
        const bool whole = (c0 == 0 && c1 == cu.nch);
        const int kv = p.ws.kvlen[b];
        const int ql = p.ws.qlen[b];
        const int rows = ql * G;
        const int t0 = p.ws.cu_q[b];
        const int prefix = kv - ql > 0 ? kv - ql : 0;
        const int nvis = tile_nvis(p, kv, ql, rows - 1);   // (no band mask: the host never picks this kernel for it)
        const int32_t *bt = p.block_tables + (size_t)b * p.max_blocks;
        const size_t head_off = (size_t)g * D;

        // q: this lane's 16 dims of every row (zero for padding rows)
        uint32_t qr[RP][8];
#pragma unroll
        for (int r = 0; r < RP; ++r) {
            const int t = t0 + r / G;
            if (r < rows && t < p.num_q_tokens) {
                const uint16_t *src = qg + head_row(p, t, g, r) * D;
                const u32x4 a = *(const u32x4 *)(src + d0), c = *(const u32x4 *)(src + d1);
                qr[r][0] = a.x; qr[r][1] = a.y; qr[r][2] = a.z; qr[r][3] = a.w;
                qr[r][4] = c.x; qr[r][5] = c.y; qr[r][6] = c.z; qr[r][7] = c.w;
            } else {
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    qr[r][k] = 0;
            }
        }

        float acc[RP][16];
#pragma unroll
        for (int r = 0; r < RP; ++r)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[r][e] = 0.f;
        // softmax state of the rows this lane holds after the QK reduction
        float m_run[NRL], l_part[NRL];
        int lim_own[NRL];
#pragma unroll
        for (int k = 0; k < NRL; ++k) {
            m_run[k] = -INFINITY;
            l_part[k] = 0.f;
            const int r = own_row(k);
            lim_own[k] = row_hi(p, kv, prefix, r / G);
        }

        // Two register buffers: while the wave computes chunk c from one, the
        // loads of chunk c + 1 are in flight into the other.  Block ids are
        // read one chunk before their loads, from a clamped (always valid)
        // table index and without branches; they are checked when used.
        // Loads of tokens that are not visible (or whose block id is out of
        // range) read row 0 of block 0 and become zeros.
        const int nblk = nvis > 0 ? div_bs(nvis - 1, bs, bsh) + 1 : 1;
        int bid[TL];
        u32x4 kA[TL][2], vA[TL][2], kB[TL][2], vB[TL][2];
        int okA = 0, okB = 0;   // bit t: token t of the buffered chunk is visible and readable
#define PA_FETCH_BIDS(c_)                                                         \
        _Pragma("unroll") for (int t = 0; t < TL; ++t) {                          \
            bid[t] = bt[bt_column((c_) * CT + t * NG + grp, bs, bsh, nblk)];      \
        }
#define PA_LOAD_CHUNK(kregs_, vregs_, okm_, c_)                                   \
        okm_ = 0;                                                                 \
        _Pragma("unroll") for (int t = 0; t < TL; ++t) {                          \
            const int j = (c_) * CT + t * NG + grp;                               \
            const bool inb = (unsigned)bid[t] < (unsigned long long)p.num_blocks; \
            const bool ok = j < nvis && inb;                                      \
            err |= (j < nvis && !inb) ? (uint32_t)PA_DEVERR_BLOCK_ID : 0u;        \
            okm_ |= ok ? (1 << t) : 0;                                            \
            const size_t off = kv_row_elem(ok, bid[t], j, bs, bsh, row_stride, head_off); \
            kregs_[t][0] = *(const u32x4 *)(kg + off + d0);                       \
            kregs_[t][1] = *(const u32x4 *)(kg + off + d1);                       \
            vregs_[t][0] = *(const u32x4 *)(vg + off + d0);                       \
            vregs_[t][1] = *(const u32x4 *)(vg + off + d1);                       \
        }

        // one chunk: QK, mask, online softmax, PV
        // (the loaded words of tokens that are not visible are whatever row 0 of
        // block 0 holds: their scores are replaced by -inf and their V words by
        // zeros before use, never multiplied away)
        auto compute = [&](const u32x4 (&kr)[TL][2], u32x4 (&vr)[TL][2], int okm, int c)
                           __attribute__((always_inline)) {
            const int jb = c * CT;
            // QK: partial dots over the lane's 16 dims, then a transposing
            // reduction over the token group
            float d[TL][RP];
#pragma unroll
            for (int t = 0; t < TL; ++t) {
                const uint32_t kw[8] = {kr[t][0].x, kr[t][0].y, kr[t][0].z, kr[t][0].w,
                                        kr[t][1].x, kr[t][1].y, kr[t][1].z, kr[t][1].w};
#pragma unroll
                for (int r = 0; r < RP; ++r) {
                    float a = 0.f;
#pragma unroll
                    for (int k = 0; k < 8; ++k)
                        a = dot2<DT>(qr[r][k], kw[k], a);
                    d[t][r] = a;
                }
                treduce<RP, L>(d[t], lane);
            }
            // softmax of the lane's rows (scores in d[t][k], k < NRL)
            float alpha[NRL];
            bool rescale = false;
#pragma unroll
            for (int k = 0; k < NRL; ++k) {
                float mx = -INFINITY;
#pragma unroll
                for (int t = 0; t < TL; ++t) {
                    const int j = jb + t * NG + grp;
                    const float v = (j < lim_own[k] && ((okm >> t) & 1)) ? d[t][k] * p.scale_log2 : -INFINITY;
                    d[t][k] = v;
                    mx = fmaxf(mx, v);
                }
                mx = slots_max<L>(mx);
                const float m_new = fmaxf(m_run[k], mx);
                alpha[k] = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run[k] - m_new);
                rescale |= alpha[k] != 1.f;
                float ps = 0.f;
#pragma unroll
                for (int t = 0; t < TL; ++t) {
                    const float pv = d[t][k] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(d[t][k] - m_new);
                    d[t][k] = pv;
                    ps += pv;
                }
                l_part[k] = l_part[k] * alpha[k] + ps;
                m_run[k] = m_new;
            }
            if (__any(rescale)) {
#pragma unroll
                for (int r = 0; r < RP; ++r) {
                    const float a = __shfl(alpha[r % NRL], gbase + holder(r));
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        acc[r][e] *= a;
                }
            }
            if (__any(okm != (1 << TL) - 1)) {
#pragma unroll
                for (int t = 0; t < TL; ++t) {
                    const u32x4 z = {0u, 0u, 0u, 0u};
                    vr[t][0] = ((okm >> t) & 1) ? vr[t][0] : z;
                    vr[t][1] = ((okm >> t) & 1) ? vr[t][1] : z;
                }
            }
            // PV on token pairs: p of both tokens packed to 16 bits, V words of
            // both tokens interleaved, v_dot2 into fp32
#pragma unroll
            for (int u = 0; u < TL / 2; ++u) {
                uint32_t pk[RP];
#pragma unroll
                for (int r = 0; r < RP; ++r) {
                    const float pa = __shfl(d[2 * u][r % NRL], gbase + holder(r));
                    const float pb = __shfl(d[2 * u + 1][r % NRL], gbase + holder(r));
                    pk[r] = pack_pair<DT>(pa, pb);
                }
                const uint32_t w0[8] = {vr[2 * u][0].x, vr[2 * u][0].y, vr[2 * u][0].z, vr[2 * u][0].w,
                                        vr[2 * u][1].x, vr[2 * u][1].y, vr[2 * u][1].z, vr[2 * u][1].w};
                const uint32_t w1[8] = {vr[2 * u + 1][0].x, vr[2 * u + 1][0].y, vr[2 * u + 1][0].z,
                                        vr[2 * u + 1][0].w, vr[2 * u + 1][1].x, vr[2 * u + 1][1].y,
                                        vr[2 * u + 1][1].z, vr[2 * u + 1][1].w};
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    const uint32_t vlo = __builtin_amdgcn_perm(w1[m], w0[m], 0x05040100u);
                    const uint32_t vhi = __builtin_amdgcn_perm(w1[m], w0[m], 0x07060302u);
#pragma unroll
                    for (int r = 0; r < RP; ++r) {
                        acc[r][2 * m] = dot2<DT>(pk[r], vlo, acc[r][2 * m]);
                        acc[r][2 * m + 1] = dot2<DT>(pk[r], vhi, acc[r][2 * m + 1]);
                    }
                }
            }
        };

        PA_FETCH_BIDS(c0)
        PA_LOAD_CHUNK(kA, vA, okA, c0)
        PA_FETCH_BIDS(c0 + 1)
        for (int c = c0; c < c1; c += 2) {
            if (c + 1 < c1) {
                PA_LOAD_CHUNK(kB, vB, okB, c + 1)
                PA_FETCH_BIDS(c + 2)
            }
            compute(kA, vA, okA, c);
            if (c + 1 >= c1)
                break;
            if (c + 2 < c1) {
                PA_LOAD_CHUNK(kA, vA, okA, c + 2)
                PA_FETCH_BIDS(c + 3)
            }
            compute(kB, vB, okB, c + 1);
        }

#undef PA_FETCH_BIDS
#undef PA_LOAD_CHUNK
        // ---------------------------------------------------------- finalise
        float l_tot[RP], m_all[RP];
        {
            float l_own[NRL];
#pragma unroll
            for (int k = 0; k < NRL; ++k)
                l_own[k] = slots_sum<L>(l_part[k]);
#pragma unroll
            for (int r = 0; r < RP; ++r) {
                l_tot[r] = __shfl(l_own[r % NRL], gbase + holder(r));
                m_all[r] = __shfl(m_run[r % NRL], gbase + holder(r));
            }
        }
        float flat[NQ];
#pragma unroll
        for (int r = 0; r < RP; ++r)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                flat[r * 16 + e] = acc[r][e];
        slot_treduce<NQ, 32, L>(flat, lane);
        // lane holds quantities q = (NQ / NG) * grp + k: row q / 16, element q % 16
        constexpr int PER = NQ / NG;
        // row statistics of row r (wave-uniform values, lane-dependent r)
        auto row_stat = [&](int r, float &Mr, float &Lr) __attribute__((always_inline)) {
            Mr = m_all[0];
            Lr = l_tot[0];
#pragma unroll
            for (int rr = 1; rr < RP; ++rr) {
                Mr = r == rr ? m_all[rr] : Mr;
                Lr = r == rr ? l_tot[rr] : Lr;
            }
        };
        if (whole) {
#pragma unroll
            for (int k0 = 0; k0 < PER; k0 += (PER >= 8 ? 8 : PER)) {
                constexpr int W = PER >= 8 ? 8 : PER;   // contiguous columns held
                const int q = PER * grp + k0;
                const int r = q / 16, e = q % 16;
                const int t = t0 + r / G;
                if (r < rows && t < p.num_q_tokens) {
                    float Mr, Lr;
                    row_stat(r, Mr, Lr);
                    const float inv = Lr > 0.f ? 1.f / Lr : 0.f;
                    const int col = lane_col(e, d0, d1);
                    uint16_t *dst = og + head_row(p, t, g, r) * D + col;
                    if constexpr (W == 8) {
                        uint4 o;
                        o.x = (uint32_t)to_bits<DT>(flat[k0] * inv) | ((uint32_t)to_bits<DT>(flat[k0 + 1] * inv) << 16);
                        o.y = (uint32_t)to_bits<DT>(flat[k0 + 2] * inv) | ((uint32_t)to_bits<DT>(flat[k0 + 3] * inv) << 16);
                        o.z = (uint32_t)to_bits<DT>(flat[k0 + 4] * inv) | ((uint32_t)to_bits<DT>(flat[k0 + 5] * inv) << 16);
                        o.w = (uint32_t)to_bits<DT>(flat[k0 + 6] * inv) | ((uint32_t)to_bits<DT>(flat[k0 + 7] * inv) << 16);
                        *(uint4 *)dst = o;
                    } else {
#pragma unroll
                        for (int k = 0; k < W; ++k)
                            dst[k] = to_bits<DT>(flat[k0 + k] * inv);
                    }
                    if (e == 0 && kq == 0 && p.lse)
                        p.lse[head_row(p, t, g, r)] =
                            Lr > 0.f ? (Mr + log2f(Lr)) * 0.69314718055994531f : -INFINITY;
                }
            }
        } else {
            const int slot = first_seg ? 0 : 1;
            float *part = p.ws.partials + (size_t)(2 * piece + slot) * p.partial_stride;
#pragma unroll
            for (int k = 0; k < PER; ++k) {
                const int q = PER * grp + k;
                const int r = q / 16, e = q % 16;
                part[r * D + lane_col(e, d0, d1)] = flat[k];
            }
            if (lane < RP) {
                float Mr, Lr;
                row_stat(lane, Mr, Lr);
                part[RP * D + lane] = Mr;
                part[RP * D + RP + lane] = Lr;
            }
        }

        first_seg = false;
        cu.item += c1 - c0;
        bool more = cu.item < end;
        if (more) {
            cursor_next_unit(p, cu);
            more = cu.b < p.batch;
        }
        if (!more) {
            // this piece is done: take the next one, if any
            if (p.no_split || p.pieces <= p.partitions)
                break;
            int nxt = 0;
            if (lane == 0)
                nxt = grab_piece(p);
            piece = __shfl(nxt, 0);
            if (!wg_range(p, piece, cu, end))
                break;
            first_seg = true;
        }
    }
    if (err)
        set_error(p.ws.err, err);
}

template <int DT, int D>
const void *kernel_rp(int rp)
{
    switch (rp) {
    case 1: return (const void *)&decode_kernel<DT, D, 1>;
    case 2: return (const void *)&decode_kernel<DT, D, 2>;
    case 4: return (const void *)&decode_kernel<DT, D, 4>;
    case 8: return (const void *)&decode_kernel<DT, D, 8>;
    default: return nullptr;
    }
}

template <int DT>
const void *kernel_dt(int dk, int dv, int rp)
{
    if (dk != dv)
        return nullptr;
    if (dk == 64)
        return kernel_rp<DT, 64>(rp);
    if (dk == 128)
        return kernel_rp<DT, 128>(rp);
    if (dk == 256)
        return kernel_rp<DT, 256>(rp);
    return nullptr;
}

const void *decode_kernel_ptr(int dtype, int dk, int dv, int rp)
{
    return dtype == 0 ? kernel_dt<0>(dk, dv, rp) : kernel_dt<1>(dk, dv, rp);
}

}  // namespace

bool decode_supported(int dk, int dv)
{
    return dk == dv && (dk == 64 || dk == 128 || dk == 256);
}

int decode_chunk(int dk, int rows_pad)
{
    const int tl = rows_pad <= 4 ? 4 : 2;
    return tl * (64 / (dk / 16));
}

int decode_workers_per_cu(int dtype, int dk, int dv, int rows_pad)
{
    const void *k = decode_kernel_ptr(dtype, dk, dv, rows_pad);
    int n = 0;
    if (!k || hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k, kThreads, 0) != hipSuccess || n < 1)
        n = 1;
    return n * (kThreads / 64);
}

hipError_t launch_decode(const Params &p, int dtype, int rows_pad, hipStream_t s, hipEvent_t e0, hipEvent_t e1)
{
    const void *k = decode_kernel_ptr(dtype, p.head_size_k, p.head_size_v, rows_pad);
    if (!k)
        return hipErrorInvalidValue;
    const int per_wg = kThreads / 64;
    const int grid = (p.partitions + per_wg - 1) / per_wg;
    void *args[] = {(void *)&p};
    return launch_kernel(k, dim3(grid), dim3(kThreads), args, s, e0, e1);
}

}  // namespace pa

// pa_decode.hip -- split-KV paged-attention decode on the vector ALUs (gfx950).
//
// For units with fewer than 16 rows (rows = query tokens x query heads of one
// GQA group), where the contraction is too thin for the matrix cores.  One
// 256-thread workgroup walks a contiguous range of (sequence, KV head, chunk)
// items handed out by the planner.  Per 64-token chunk:
//
//   stage   K and V rows of KV head g are gathered through the block table
//           (token j -> block_tables[b][j / block_size], slot j % block_size;
//           Ascend ATB PagedAttentionOperation, Constraints) with 128-bit
//           loads into registers one chunk ahead, then stored to LDS (double
//           buffer).  Tokens past the visible range are stored as zeros, so
//           tail slots and unreferenced blocks are never read.
//   QK      every thread holds 16 head dimensions of all rows of q and dots
//           them with one K row at a time (v_dot2 fp16/bf16 -> fp32); the
//           per-row partial sums of the Dk/16 threads that share a token are
//           combined with a transposing DPP reduction, so each thread ends
//           with whole scores for its share of the rows.
//   softmax running max / sum per row (log2 domain); masked positions are
//           set to -inf by select and get weight exactly 0.
//   PV      every thread accumulates 8 output columns of all rows over its
//           share of the chunk's tokens in fp32.
//
// At the end of a unit's range the per-thread accumulators are summed
// through LDS and either normalised into the output (the unit is whole) or
// written as an fp32 partial (acc, m, l) for the merge kernel.
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

template <int DK, int DV>
struct DecodeShape {
    static constexpr int NT = kThreads;
    static constexpr int CT = kDecodeChunk;
    static constexpr int KP = DK + 8;           // LDS row pitch of K (elements)
    static constexpr int VP = DV + 8;
    static constexpr int TPT = DK / 16;         // threads per token in QK
    static constexpr int TPP = NT / TPT;        // tokens per QK pass
    static constexpr int QK_PASSES = CT / TPP;
    static constexpr int ECH = DV / 8;          // 8-column groups in PV
    static constexpr int NTS = NT / ECH;        // token subsets in PV
    static constexpr int TPS = CT / NTS;        // tokens per subset and chunk
    static constexpr int NK = CT * DK / 8 / NT; // 128-bit K pieces per thread per chunk
    static constexpr int NV = CT * DV / 8 / NT;
    static constexpr int KBUF = CT * KP;        // elements per K buffer
    static constexpr int VBUF = CT * VP;
    static_assert(DK % 16 == 0 && DV % 8 == 0, "head sizes");
    static_assert(TPT >= 1 && TPT <= 16 && (TPT & (TPT - 1)) == 0, "Dk/16 must be a power of two <= 16");
    static_assert(QK_PASSES >= 1 && NTS >= 1 && TPS >= 1, "shape");
    static_assert((CT * DK / 8) % NT == 0 && (CT * DV / 8) % NT == 0, "staging");
};

template <int DT, int DK, int DV, int RP>
__global__ __launch_bounds__(kThreads) void decode_kernel(Params p)
{
    using S = DecodeShape<DK, DV>;
    constexpr int NT = S::NT, CT = S::CT, KP = S::KP, VP = S::VP, TPT = S::TPT, TPP = S::TPP;
    constexpr int ECH = S::ECH, NTS = S::NTS, TPS = S::TPS, NK = S::NK, NV = S::NV;
    constexpr int TR = (NT / RP) < 64 ? (NT / RP) : 64;  // softmax threads per row
    constexpr int TOKR = CT / TR;                        // tokens per softmax thread
    constexpr int RED_ROWS_MAX = (2 * S::KBUF * 2) / (NTS * DV * 4);
    constexpr int RED_ROWS = RED_ROWS_MAX < RP ? RED_ROWS_MAX : RP;
    static_assert(RED_ROWS >= 1, "reduction buffer");

    __shared__ __attribute__((aligned(16))) uint16_t sK[2 * S::KBUF];
    __shared__ __attribute__((aligned(16))) uint16_t sV[2 * S::VBUF];
    __shared__ __attribute__((aligned(16))) float sS[CT * RP];
    __shared__ float sAlpha[RP], sM[RP], sL[RP];
    __shared__ int32_t sBT[kBtWindow];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int kq = tid % TPT;            // QK: which 16 head dims
    const int tq = tid / TPT;            // QK: token within a pass
    const int srow = tid / TR;           // softmax: row
    const int sl = tid % TR;             // softmax: lane within the row group
    const int ec = tid % ECH;            // PV: 8-column group
    const int ts = tid / ECH;            // PV: token subset

    const int w = xcd_logical_index(blockIdx.x, gridDim.x);
    Cursor cu;
    int end;
    if (!wg_range(p, w, cu, end))
        return;

    const uint16_t *__restrict__ qg = (const uint16_t *)p.query;
    const uint16_t *__restrict__ kg = (const uint16_t *)p.key_cache;
    const uint16_t *__restrict__ vg = (const uint16_t *)p.value_cache;
    uint16_t *__restrict__ og = (uint16_t *)p.out;
    const int G = p.group;
    const int H = p.head_num;
    const int Hkv = p.kv_head_num;
    const int bs = p.block_size;
    const int bsh = p.bs_shift;
    uint32_t err = 0;
    bool first_seg = true;

    while (true) {
        // ---------------------------------------------------------- segment
        const int b = cu.b, g = cu.g;
        const int c0 = cu.c;
        const int c1 = cu.nch < c0 + (end - cu.item) ? cu.nch : c0 + (end - cu.item);
        const bool whole = (c0 == 0 && c1 == cu.nch);
        const int kv = p.ws.kvlen[b];
        const int ql = p.ws.qlen[b];
        const int rows = ql * G;
        const int t0 = p.ws.cu_q[b];
        const int prefix = kv - ql > 0 ? kv - ql : 0;
        const int nvis = tile_nvis(kv, ql, G, rows - 1, p.causal);
        const int nblk = nvis > 0 ? div_bs(nvis - 1, bs, bsh) + 1 : 0;
        const int64_t row_stride_k = (int64_t)Hkv * DK;
        const int64_t row_stride_v = (int64_t)Hkv * DV;

        // q: this thread's 16 head dims of every row (zero for padding rows)
        uint32_t qr[RP][8];
#pragma unroll
        for (int r = 0; r < RP; ++r) {
            const int t = t0 + r / G;
            if (r < rows && t < p.num_q_tokens) {
                const uint4 *src = (const uint4 *)(qg + ((size_t)t * H + g * G + r % G) * DK + kq * 16);
                const uint4 a = src[0], c = src[1];
                qr[r][0] = a.x; qr[r][1] = a.y; qr[r][2] = a.z; qr[r][3] = a.w;
                qr[r][4] = c.x; qr[r][5] = c.y; qr[r][6] = c.z; qr[r][7] = c.w;
            } else {
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    qr[r][k] = 0;
            }
        }

        float acc[RP][8];
#pragma unroll
        for (int r = 0; r < RP; ++r)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                acc[r][e] = 0.f;
        float m_run = -INFINITY, l_run = 0.f;

        // block-table window
        int win0 = div_bs(c0 * CT, bs, bsh);
        auto load_window = [&](int first_blk) {
            __syncthreads();
            for (int k = tid; k < kBtWindow; k += NT) {
                const int blk = first_blk + k;
                sBT[k] = blk < nblk ? p.block_tables[(size_t)b * p.max_blocks + blk] : 0;
            }
            __syncthreads();
        };
        load_window(win0);

        uint4 kreg[NK], vreg[NV];
        auto issue = [&](int c) {
            const int jb = c * CT;
#pragma unroll
            for (int k = 0; k < NK; ++k) {
                const int piece = tid + NT * k;
                const int row = piece / (DK / 8);
                const int col = (piece % (DK / 8)) * 8;
                const int j = jb + row;
                uint4 v = make_uint4(0, 0, 0, 0);
                if (j < nvis) {
                    const int phys = sBT[div_bs(j, bs, bsh) - win0];
                    if ((unsigned)phys < (unsigned long long)p.num_blocks) {
                        const size_t off = ((size_t)phys * bs + mod_bs(j, bs, bsh)) * row_stride_k +
                                           (size_t)g * DK + col;
                        v = *(const uint4 *)(kg + off);
                    } else {
                        err |= PA_DEVERR_BLOCK_ID;
                    }
                }
                kreg[k] = v;
            }
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                const int piece = tid + NT * k;
                const int row = piece / (DV / 8);
                const int col = (piece % (DV / 8)) * 8;
                const int j = jb + row;
                uint4 v = make_uint4(0, 0, 0, 0);
                if (j < nvis) {
                    const int phys = sBT[div_bs(j, bs, bsh) - win0];
                    if ((unsigned)phys < (unsigned long long)p.num_blocks) {
                        const size_t off = ((size_t)phys * bs + mod_bs(j, bs, bsh)) * row_stride_v +
                                           (size_t)g * DV + col;
                        v = *(const uint4 *)(vg + off);
                    }
                }
                vreg[k] = v;
            }
        };
        auto store = [&](int buf) {
#pragma unroll
            for (int k = 0; k < NK; ++k) {
                const int piece = tid + NT * k;
                const int row = piece / (DK / 8);
                const int col = (piece % (DK / 8)) * 8;
                *(uint4 *)(sK + buf * S::KBUF + row * KP + col) = kreg[k];
            }
#pragma unroll
            for (int k = 0; k < NV; ++k) {
                const int piece = tid + NT * k;
                const int row = piece / (DV / 8);
                const int col = (piece % (DV / 8)) * 8;
                *(uint4 *)(sV + buf * S::VBUF + row * VP + col) = vreg[k];
            }
        };
        // blocks of chunk c lie in [first, last]; make sure the window holds them
        auto ensure_window = [&](int c) {
            const int jb = c * CT;
            int jl = jb + CT - 1;
            jl = jl < nvis - 1 ? jl : nvis - 1;
            if (jl < jb)
                return;
            const int lastb = div_bs(jl, bs, bsh);
            if (lastb >= win0 + kBtWindow) {
                win0 = div_bs(jb, bs, bsh);
                load_window(win0);
            }
        };

        issue(c0);
        store(0);
        __syncthreads();

        for (int c = c0; c < c1; ++c) {
            const int buf = (c - c0) & 1;
            const bool has_next = c + 1 < c1;
            if (has_next) {
                ensure_window(c + 1);
                issue(c + 1);
            }
            const uint16_t *kb = sK + buf * S::KBUF;
            const uint16_t *vb = sV + buf * S::VBUF;
            const int jb = c * CT;

            // ------------------------------------------------------- QK
#pragma unroll
            for (int pass = 0; pass < S::QK_PASSES; ++pass) {
                const int tok = tq + pass * TPP;
                const uint4 k0 = *(const uint4 *)(kb + tok * KP + kq * 16);
                const uint4 k1 = *(const uint4 *)(kb + tok * KP + kq * 16 + 8);
                const uint32_t kw[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
                float d[RP];
#pragma unroll
                for (int r = 0; r < RP; ++r) {
                    float s = 0.f;
#pragma unroll
                    for (int k = 0; k < 8; ++k)
                        s = dot2<DT>(qr[r][k], kw[k], s);
                    d[r] = s;
                }
                treduce<RP, TPT>(d, lane);
                const int j = jb + tok;
                if constexpr (RP >= TPT) {
#pragma unroll
                    for (int k = 0; k < RP / TPT; ++k) {
                        const int r = (RP / TPT) * kq + k;
                        const int lim = p.causal ? prefix + r / G + 1 : kv;
                        const bool vis = j < kv && j < lim;
                        sS[tok * RP + r] = vis ? d[k] * p.scale_log2 : -INFINITY;
                    }
                } else {
                    if (kq % (TPT / RP) == 0) {
                        const int r = kq / (TPT / RP);
                        const int lim = p.causal ? prefix + r / G + 1 : kv;
                        const bool vis = j < kv && j < lim;
                        sS[tok * RP + r] = vis ? d[0] * p.scale_log2 : -INFINITY;
                    }
                }
            }
            __syncthreads();

            // -------------------------------------------------- softmax
            if (srow < RP) {
                float sv[TOKR];
                float mx = -INFINITY;
#pragma unroll
                for (int k = 0; k < TOKR; ++k) {
                    sv[k] = sS[(sl + TR * k) * RP + srow];
                    mx = fmaxf(mx, sv[k]);
                }
                mx = group_max<TR>(mx);
                const float m_new = fmaxf(m_run, mx);
                const float alpha = m_new == -INFINITY ? 1.f : exp2f(m_run - m_new);
                float ps = 0.f;
#pragma unroll
                for (int k = 0; k < TOKR; ++k) {
                    const float pk = sv[k] == -INFINITY ? 0.f : exp2f(sv[k] - m_new);
                    sS[(sl + TR * k) * RP + srow] = pk;
                    ps += pk;
                }
                ps = group_sum<TR>(ps);
                l_run = l_run * alpha + ps;
                m_run = m_new;
                if (sl == 0)
                    sAlpha[srow] = alpha;
            }
            __syncthreads();

            // ------------------------------------------------------- PV
            {
                float al[RP];
                bool rescale = false;
#pragma unroll
                for (int r = 0; r < RP; ++r) {
                    al[r] = sAlpha[r];
                    rescale |= al[r] != 1.f;
                }
                if (rescale) {
#pragma unroll
                    for (int r = 0; r < RP; ++r)
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            acc[r][e] *= al[r];
                }
#pragma unroll
                for (int k = 0; k < TPS; ++k) {
                    const int tok = ts + NTS * k;
                    const uint4 vv = *(const uint4 *)(vb + tok * VP + ec * 8);
                    const uint32_t vw[4] = {vv.x, vv.y, vv.z, vv.w};
                    float vf[8];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        vf[2 * e] = lo_f32<DT>(vw[e]);
                        vf[2 * e + 1] = hi_f32<DT>(vw[e]);
                    }
                    float pr[RP];
                    if constexpr (RP % 4 == 0) {
#pragma unroll
                        for (int r = 0; r < RP; r += 4) {
                            const float4 q4 = *(const float4 *)(sS + tok * RP + r);
                            pr[r] = q4.x; pr[r + 1] = q4.y; pr[r + 2] = q4.z; pr[r + 3] = q4.w;
                        }
                    } else {
#pragma unroll
                        for (int r = 0; r < RP; ++r)
                            pr[r] = sS[tok * RP + r];
                    }
#pragma unroll
                    for (int r = 0; r < RP; ++r)
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            acc[r][e] = fmaf(pr[r], vf[e], acc[r][e]);
                }
            }
            if (has_next)
                store(buf ^ 1);
            __syncthreads();
        }

        // ---------------------------------------------------- finalise
        if (srow < RP && sl == 0) {
            sM[srow] = m_run;
            sL[srow] = l_run;
        }
        float *red = (float *)sK;   // reused: NTS x RED_ROWS x DV floats
        const int slot = first_seg ? 0 : 1;
        float *part = p.ws.partials + (size_t)(2 * w + slot) * p.partial_stride;
#pragma unroll
        for (int r0 = 0; r0 < RP; r0 += RED_ROWS) {
            __syncthreads();
#pragma unroll
            for (int rr = 0; rr < RED_ROWS; ++rr) {
                if (r0 + rr < RP) {
                    float4 *dst = (float4 *)(red + ((size_t)rr * NTS + ts) * DV + ec * 8);
                    dst[0] = make_float4(acc[r0 + rr][0], acc[r0 + rr][1], acc[r0 + rr][2], acc[r0 + rr][3]);
                    dst[1] = make_float4(acc[r0 + rr][4], acc[r0 + rr][5], acc[r0 + rr][6], acc[r0 + rr][7]);
                }
            }
            __syncthreads();
            for (int idx = tid; idx < RED_ROWS * DV; idx += NT) {
                const int rr = idx / DV;
                const int e = idx - rr * DV;
                const int r = r0 + rr;
                if (r >= RP || r >= rows)
                    continue;
                float sum = 0.f;
#pragma unroll 4
                for (int t2 = 0; t2 < NTS; ++t2)
                    sum += red[((size_t)rr * NTS + t2) * DV + e];
                if (whole) {
                    const int t = t0 + r / G;
                    if (t >= p.num_q_tokens)
                        continue;
                    const int h = g * G + r % G;
                    const float L = sL[r];
                    og[((size_t)t * H + h) * DV + e] = to_bits<DT>(L > 0.f ? sum / L : 0.f);
                    if (e == 0 && p.lse)
                        p.lse[(size_t)t * H + h] =
                            L > 0.f ? (sM[r] + log2f(L)) * 0.69314718055994531f : -INFINITY;
                } else {
                    part[r * DV + e] = sum;
                    if (e == 0) {
                        part[RP * DV + r] = sM[r];
                        part[RP * DV + RP + r] = sL[r];
                    }
                }
            }
        }
        __syncthreads();

        first_seg = false;
        cu.item += c1 - c0;
        if (cu.item >= end)
            break;
        cursor_next_unit(p, cu);
        if (cu.b >= p.batch)
            break;
    }
    if (err)
        set_error(p.ws.err, err);
}

template <int DT, int DK, int DV>
const void *kernel_rp(int rp)
{
    switch (rp) {
    case 1: return (const void *)&decode_kernel<DT, DK, DV, 1>;
    case 2: return (const void *)&decode_kernel<DT, DK, DV, 2>;
    case 4: return (const void *)&decode_kernel<DT, DK, DV, 4>;
    case 8: return (const void *)&decode_kernel<DT, DK, DV, 8>;
    case 16: return (const void *)&decode_kernel<DT, DK, DV, 16>;
    default: return nullptr;
    }
}

template <int DT>
const void *kernel_dt(int dk, int dv, int rp)
{
    if (dk == 64 && dv == 64)
        return kernel_rp<DT, 64, 64>(rp);
    if (dk == 128 && dv == 128)
        return kernel_rp<DT, 128, 128>(rp);
    if (dk == 256 && dv == 256)
        return kernel_rp<DT, 256, 256>(rp);
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

int decode_wgs_per_cu(int dtype, int dk, int dv, int rows_pad)
{
    const void *k = decode_kernel_ptr(dtype, dk, dv, rows_pad);
    int n = 0;
    if (!k || hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k, kThreads, 0) != hipSuccess || n < 1)
        return 1;
    return n;
}

hipError_t launch_decode(const Params &p, int dtype, int rows_pad, hipStream_t s)
{
    const void *k = decode_kernel_ptr(dtype, p.head_size_k, p.head_size_v, rows_pad);
    if (!k)
        return hipErrorInvalidValue;
    void *args[] = {(void *)&p};
    return hipLaunchKernel(k, dim3(p.partitions), dim3(kThreads), args, 0, s);
}

}  // namespace pa

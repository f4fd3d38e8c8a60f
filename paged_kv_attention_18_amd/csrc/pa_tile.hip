// pa_tile.hip -- paged attention on the matrix cores (gfx950 MFMA).
//
// For units with 16 or more rows: parallel decoding / splitfuse chunks with
// the prefix-aligned causal mask (Ascend ATB PagedAttentionOperation,
// Constraints, mask type 5 list) and decode with a wide GQA group (e.g. 64
// query heads on one KV head with 576/512 key/value head sizes, which the
// same Constraints allow at block_size <= 128).
//
// A workgroup of NW waves owns a tile of rows of one (sequence, KV head).  The
// waves form NW / CS row groups of 16 * MB rows; the CS waves of a row group
// share its rows and split the Dv output columns (CS = 2 halves the output
// accumulator per wave for Dv = 512).  Per KT-token chunk:
//
//   stage  K rows are copied to LDS as they are ([token][Dk], padded pitch);
//          V rows are transposed in registers (4 tokens x 8 columns at a
//          time) and stored as [column][token] with an XOR swizzle of the
//          4-token groups, so both the stores and the MFMA operand reads are
//          free of bank conflicts.  Loads run one chunk ahead (double buffer).
//   S^T    = K . Q^T with v_mfma_f32_16x16x32_{f16,bf16}: K is the A operand
//          (16 tokens x 32 dims per lane group), Q^T the B operand, held in
//          registers for the whole unit.  The accumulator gives every lane
//          one query row and 4 + 4 tokens, which is exactly the A-operand
//          layout P needs for the next product, so P never leaves registers.
//   mask   select -inf where j >= kv or (causal) j > prefix + i; chunks that
//          lie wholly inside every row's visible range skip the test, and
//          chunks wholly outside are never planned.
//   PV     O += P . V with the same instruction; V^T read from LDS.
//
// Row statistics (running max and sum, log2 domain) stay per wave; at the end
// of a unit's range O is normalised into the output, or written as an fp32
// partial for the merge kernel.
#include "pa_internal.h"

namespace pa {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int DT>
struct Mfma;

template <>
struct Mfma<0> {
    typedef _Float16 v8 __attribute__((ext_vector_type(8)));
    static __device__ __forceinline__ f32x4 run(u32x4 a, u32x4 b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8, a), __builtin_bit_cast(v8, b), c,
                                                      0, 0, 0);
    }
};

template <>
struct Mfma<1> {
    typedef __bf16 v8 __attribute__((ext_vector_type(8)));
    static __device__ __forceinline__ f32x4 run(u32x4 a, u32x4 b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8, a), __builtin_bit_cast(v8, b), c,
                                                       0, 0, 0);
    }
};

// Position of 4-token group q in LDS column `col` of the transposed V tile.
template <int KT>
__device__ __forceinline__ int vt_group(int q, int col)
{
    if constexpr (KT == 32)
        return q ^ ((((col >> 4) * 5) ^ (col >> 5)) & 7);
    else
        return q ^ ((col ^ (col >> 2)) & 15);
}

template <int KT>
constexpr int vt_pitch()
{
    return KT == 32 ? 36 : 64;
}

template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi)
{
    return (uint32_t)to_bits<DT>(lo) | ((uint32_t)to_bits<DT>(hi) << 16);
}

template <int DT, int DK, int DV, int MB, int KT, int NW, int CS>
__global__ __launch_bounds__(64 * NW) void tile_kernel(Params p)
{
    constexpr int NT = 64 * NW;
    constexpr int RGS = NW / CS;                  // row groups
    constexpr int R = 16 * MB * RGS;              // rows per tile
    constexpr int KP = DK + 8;
    constexpr int VTP = vt_pitch<KT>();
    constexpr int KS = DK / 32;
    constexpr int NTT = KT / 16;
    constexpr int ND = DV / 16 / CS;              // output column tiles per wave
    constexpr int PVK = KT / 32;
    constexpr int NKP_T = KT * DK / 8;            // 128-bit K pieces per chunk
    constexpr int NKP = (NKP_T + NT - 1) / NT;
    constexpr int NVP_T = (KT / 4) * (DV / 8);    // 4-token x 8-column V pieces per chunk
    constexpr int NVP = (NVP_T + NT - 1) / NT;
    constexpr int KBUF = KT * KP;
    constexpr int VBUF = DV * VTP;
    static_assert(DK % 32 == 0 && DV % 64 == 0 && (KT == 32 || KT == 64), "shape");
    static_assert(NW % CS == 0 && (DV / 16) % CS == 0, "split");

    __shared__ __attribute__((aligned(16))) uint16_t sK[2 * KBUF];
    __shared__ __attribute__((aligned(16))) uint16_t sVt[2 * VBUF];
    __shared__ int32_t sBT[kBtWindow];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int rgi = wave / CS;          // row group
    const int csl = wave % CS;          // column slice
    const int col0 = csl * (DV / CS);
    const int lr = lane & 15;
    const int lg = lane >> 4;

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
        const int b = cu.b, g = cu.g, qt = cu.qt;
        const int c0 = cu.c;
        const int c1 = cu.nch < c0 + (end - cu.item) ? cu.nch : c0 + (end - cu.item);
        const bool whole = (c0 == 0 && c1 == cu.nch);
        const int kv = p.ws.kvlen[b];
        const int ql = p.ws.qlen[b];
        const int rows = ql * G;
        int rows_tile = rows - qt * R;
        rows_tile = rows_tile < R ? rows_tile : R;
        const int t0 = p.ws.cu_q[b];
        const int prefix = kv - ql > 0 ? kv - ql : 0;
        const int nvis = tile_nvis(kv, ql, G, qt * R + rows_tile - 1, p.causal);
        const int nblk = nvis > 0 ? div_bs(nvis - 1, bs, bsh) + 1 : 0;
        // the fewest visible tokens of any row of the tile (masking threshold)
        const int min_lim = p.causal ? tile_nvis(kv, ql, G, qt * R, 1) : kv;
        const int wr0 = rgi * 16 * MB;
        const bool wave_active = wr0 < rows_tile;
        const int64_t row_stride_k = (int64_t)Hkv * DK;
        const int64_t row_stride_v = (int64_t)Hkv * DV;

        // Q^T operand and the visible limit of this lane's rows
        u32x4 qb[MB][KS];
        int lim[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int row_t = wr0 + 16 * mb + lr;
            const int rg = qt * R + row_t;
            const int t = t0 + rg / G;
            const bool ok = row_t < rows_tile && t < p.num_q_tokens;
            lim[mb] = p.causal ? (prefix + rg / G + 1 < kv ? prefix + rg / G + 1 : kv) : kv;
            const uint16_t *src = qg + ((size_t)t * H + g * G + rg % G) * DK + 8 * lg;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qb[mb][ks] = ok ? *(const u32x4 *)(src + 32 * ks) : u32x4{0u, 0u, 0u, 0u};
        }

        f32x4 oacc[MB][ND];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nd = 0; nd < ND; ++nd)
                oacc[mb][nd] = f32x4{0.f, 0.f, 0.f, 0.f};
        float m_run[MB], lsum[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            m_run[mb] = -INFINITY;
            lsum[mb] = 0.f;
        }

        int win0 = div_bs(c0 * KT, bs, bsh);
        auto load_window = [&](int first_blk) {
            __syncthreads();
            for (int k = tid; k < kBtWindow; k += NT) {
                const int blk = first_blk + k;
                sBT[k] = blk < nblk ? p.block_tables[(size_t)b * p.max_blocks + blk] : 0;
            }
            __syncthreads();
        };
        load_window(win0);

        uint4 kreg[NKP];
        uint4 vreg[NVP][4];
        auto row_offset = [&](int j, int64_t stride, int d, bool &ok) -> size_t {
            const int phys = sBT[div_bs(j, bs, bsh) - win0];
            ok = (unsigned)phys < (unsigned long long)p.num_blocks;
            return ((size_t)phys * bs + mod_bs(j, bs, bsh)) * stride + (size_t)g * d;
        };
        auto issue = [&](int c) {
            const int jb = c * KT;
#pragma unroll
            for (int k = 0; k < NKP; ++k) {
                const int piece = tid + NT * k;
                const int row = piece / (DK / 8);
                const int col = (piece % (DK / 8)) * 8;
                const int j = jb + row;
                uint4 v = make_uint4(0, 0, 0, 0);
                if (piece < NKP_T && j < nvis) {
                    bool ok;
                    const size_t off = row_offset(j, row_stride_k, DK, ok);
                    if (ok)
                        v = *(const uint4 *)(kg + off + col);
                    else
                        err |= PA_DEVERR_BLOCK_ID;
                }
                kreg[k] = v;
            }
#pragma unroll
            for (int k = 0; k < NVP; ++k) {
                const int piece = tid + NT * k;
                const int x = piece & 63, y = piece >> 6;
                const int col8 = (x & 7) + 8 * (y % (DV / 64));
                const int tg = (x >> 3) + 8 * (y / (DV / 64));
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int j = jb + 4 * tg + q;
                    uint4 v = make_uint4(0, 0, 0, 0);
                    if (piece < NVP_T && j < nvis) {
                        bool ok;
                        const size_t off = row_offset(j, row_stride_v, DV, ok);
                        if (ok)
                            v = *(const uint4 *)(vg + off + col8 * 8);
                    }
                    vreg[k][q] = v;
                }
            }
        };
        auto store = [&](int buf) {
#pragma unroll
            for (int k = 0; k < NKP; ++k) {
                const int piece = tid + NT * k;
                if (piece < NKP_T) {
                    const int row = piece / (DK / 8);
                    const int col = (piece % (DK / 8)) * 8;
                    *(uint4 *)(sK + buf * KBUF + row * KP + col) = kreg[k];
                }
            }
#pragma unroll
            for (int k = 0; k < NVP; ++k) {
                const int piece = tid + NT * k;
                if (piece < NVP_T) {
                    const int x = piece & 63, y = piece >> 6;
                    const int col8 = (x & 7) + 8 * (y % (DV / 64));
                    const int tg = (x >> 3) + 8 * (y / (DV / 64));
                    const uint32_t w0[4] = {vreg[k][0].x, vreg[k][0].y, vreg[k][0].z, vreg[k][0].w};
                    const uint32_t w1[4] = {vreg[k][1].x, vreg[k][1].y, vreg[k][1].z, vreg[k][1].w};
                    const uint32_t w2[4] = {vreg[k][2].x, vreg[k][2].y, vreg[k][2].z, vreg[k][2].w};
                    const uint32_t w3[4] = {vreg[k][3].x, vreg[k][3].y, vreg[k][3].z, vreg[k][3].w};
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const int colA = col8 * 8 + 2 * m, colB = colA + 1;
                        const uint2 lo = make_uint2(__builtin_amdgcn_perm(w1[m], w0[m], 0x05040100u),
                                                    __builtin_amdgcn_perm(w3[m], w2[m], 0x05040100u));
                        const uint2 hi = make_uint2(__builtin_amdgcn_perm(w1[m], w0[m], 0x07060302u),
                                                    __builtin_amdgcn_perm(w3[m], w2[m], 0x07060302u));
                        *(uint2 *)(sVt + buf * VBUF + colA * VTP + 4 * vt_group<KT>(tg, colA)) = lo;
                        *(uint2 *)(sVt + buf * VBUF + colB * VTP + 4 * vt_group<KT>(tg, colB)) = hi;
                    }
                }
            }
        };
        auto ensure_window = [&](int c) {
            const int jb = c * KT;
            int jl = jb + KT - 1;
            jl = jl < nvis - 1 ? jl : nvis - 1;
            if (jl < jb)
                return;
            if (div_bs(jl, bs, bsh) >= win0 + kBtWindow) {
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
            if (wave_active) {
                const uint16_t *kb = sK + buf * KBUF;
                const uint16_t *vb = sVt + buf * VBUF;
                const int jb = c * KT;
                // ---------------------------------------- S^T = K . Q^T
                f32x4 sacc[MB][NTT];
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int n = 0; n < NTT; ++n)
                        sacc[mb][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                    for (int n = 0; n < NTT; ++n) {
                        const u32x4 a = *(const u32x4 *)(kb + (16 * n + lr) * KP + 32 * ks + 8 * lg);
#pragma unroll
                        for (int mb = 0; mb < MB; ++mb)
                            sacc[mb][n] = Mfma<DT>::run(a, qb[mb][ks], sacc[mb][n]);
                    }
                }
                // ------------------------------------- mask, softmax
                const bool need_mask = jb + KT > min_lim;
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    float mx = -INFINITY;
#pragma unroll
                    for (int n = 0; n < NTT; ++n) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            float s = sacc[mb][n][r] * p.scale_log2;
                            if (need_mask) {
                                const int j = jb + 16 * n + 4 * lg + r;
                                s = j < lim[mb] ? s : -INFINITY;
                            }
                            sacc[mb][n][r] = s;
                            mx = fmaxf(mx, s);
                        }
                    }
                    mx = fmaxf(mx, pair_swap<16>(mx));
                    mx = fmaxf(mx, pair_swap<32>(mx));
                    const float m_new = fmaxf(m_run[mb], mx);
                    const float alpha = m_new == -INFINITY ? 1.f : exp2f(m_run[mb] - m_new);
                    float ps = 0.f;
#pragma unroll
                    for (int n = 0; n < NTT; ++n) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float s = sacc[mb][n][r];
                            const float pv = s == -INFINITY ? 0.f : exp2f(s - m_new);
                            sacc[mb][n][r] = pv;
                            ps += pv;
                        }
                    }
                    lsum[mb] = lsum[mb] * alpha + ps;
                    m_run[mb] = m_new;
                    // O rows 4 lg + r take the factor of the lane holding that row
                    if (__ballot(alpha != 1.f) != 0) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float ar = __shfl(alpha, 4 * lg + r);
#pragma unroll
                            for (int nd = 0; nd < ND; ++nd)
                                oacc[mb][nd][r] *= ar;
                        }
                    }
                }
                // --------------------------------------------- O += P V
#pragma unroll
                for (int kk = 0; kk < PVK; ++kk) {
                    u32x4 pa[MB];
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) {
                        const f32x4 s0 = sacc[mb][2 * kk], s1 = sacc[mb][2 * kk + 1];
                        pa[mb] = u32x4{pack2<DT>(s0[0], s0[1]), pack2<DT>(s0[2], s0[3]),
                                       pack2<DT>(s1[0], s1[1]), pack2<DT>(s1[2], s1[3])};
                    }
#pragma unroll
                    for (int nd = 0; nd < ND; ++nd) {
                        const int col = col0 + 16 * nd + lr;
                        const uint16_t *vrow = vb + col * VTP;
                        const uint2 v0 = *(const uint2 *)(vrow + 4 * vt_group<KT>(8 * kk + lg, col));
                        const uint2 v1 = *(const uint2 *)(vrow + 4 * vt_group<KT>(8 * kk + 4 + lg, col));
                        const u32x4 bv = {v0.x, v0.y, v1.x, v1.y};
#pragma unroll
                        for (int mb = 0; mb < MB; ++mb)
                            oacc[mb][nd] = Mfma<DT>::run(pa[mb], bv, oacc[mb][nd]);
                    }
                }
            }
            if (has_next)
                store(buf ^ 1);
            __syncthreads();
        }

        // -------------------------------------------------------- finalise
        if (wave_active) {
            const int slot = first_seg ? 0 : 1;
            float *part = p.ws.partials + (size_t)(2 * w + slot) * p.partial_stride;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                float L = lsum[mb] + pair_swap<16>(lsum[mb]);
                L += pair_swap<32>(L);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float Lr = __shfl(L, 4 * lg + r);
                    const float Mr = __shfl(m_run[mb], 4 * lg + r);
                    const int row_t = wr0 + 16 * mb + 4 * lg + r;
                    if (row_t >= rows_tile)
                        continue;
                    const int rg = qt * R + row_t;
                    const int t = t0 + rg / G;
                    const int h = g * G + rg % G;
                    if (whole) {
                        if (t >= p.num_q_tokens)
                            continue;
                        const float inv = Lr > 0.f ? 1.f / Lr : 0.f;
                        uint16_t *dst = og + ((size_t)t * H + h) * DV;
#pragma unroll
                        for (int nd = 0; nd < ND; ++nd)
                            dst[col0 + 16 * nd + lr] = to_bits<DT>(oacc[mb][nd][r] * inv);
                        if (lr == 0 && csl == 0 && p.lse)
                            p.lse[(size_t)t * H + h] =
                                Lr > 0.f ? (Mr + log2f(Lr)) * 0.69314718055994531f : -INFINITY;
                    } else {
#pragma unroll
                        for (int nd = 0; nd < ND; ++nd)
                            part[row_t * DV + col0 + 16 * nd + lr] = oacc[mb][nd][r];
                        if (lr == 0 && csl == 0) {
                            part[R * DV + row_t] = Mr;
                            part[R * DV + R + row_t] = Lr;
                        }
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

// Kernel variants: (Dk, Dv) -> chunk KT, waves NW, column split CS.
template <int DK, int DV>
struct TileCfg {
    static constexpr int KT = (DK <= 128 && DV <= 128) ? 64 : 32;
    static constexpr int NW = DV > 256 ? 8 : 4;
    static constexpr int CS = DV > 256 ? 2 : 1;
    static constexpr int MB2 = DV > 256 ? 1 : 2;   // the larger row block count built
};

template <int DT, int DK, int DV>
const void *kernel_for(int mb)
{
    using C = TileCfg<DK, DV>;
    if (mb == 1)
        return (const void *)&tile_kernel<DT, DK, DV, 1, C::KT, C::NW, C::CS>;
    if (mb == 2 && C::MB2 == 2)
        return (const void *)&tile_kernel<DT, DK, DV, C::MB2, C::KT, C::NW, C::CS>;
    return nullptr;
}

template <int DT>
const void *kernel_dt(int dk, int dv, int mb, int *threads)
{
    if (dk == 64 && dv == 64) {
        *threads = 64 * TileCfg<64, 64>::NW;
        return kernel_for<DT, 64, 64>(mb);
    }
    if (dk == 128 && dv == 128) {
        *threads = 64 * TileCfg<128, 128>::NW;
        return kernel_for<DT, 128, 128>(mb);
    }
    if (dk == 256 && dv == 256) {
        *threads = 64 * TileCfg<256, 256>::NW;
        return kernel_for<DT, 256, 256>(mb);
    }
    if (dk == 576 && dv == 512) {
        *threads = 64 * TileCfg<576, 512>::NW;
        return kernel_for<DT, 576, 512>(mb);
    }
    return nullptr;
}

const void *tile_kernel_ptr(int dtype, int dk, int dv, int mb, int *threads)
{
    return dtype == 0 ? kernel_dt<0>(dk, dv, mb, threads) : kernel_dt<1>(dk, dv, mb, threads);
}

}  // namespace

int tile_chunk(int dk, int dv)
{
    return (dk <= 128 && dv <= 128) ? 64 : 32;
}

bool tile_supported(int dk, int dv, int row_blocks)
{
    int threads = 0;
    return tile_kernel_ptr(0, dk, dv, row_blocks, &threads) != nullptr;
}

int tile_rows(int dk, int dv, int row_blocks)
{
    const int nw = dv > 256 ? 8 : 4, cs = dv > 256 ? 2 : 1;
    return 16 * row_blocks * (nw / cs);
}

int tile_workers_per_cu(int dtype, int dk, int dv, int row_blocks)
{
    int threads = 0;
    const void *k = tile_kernel_ptr(dtype, dk, dv, row_blocks, &threads);
    int n = 0;
    if (!k || hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k, threads, 0) != hipSuccess || n < 1)
        return 1;
    return n;
}

hipError_t launch_tile(const Params &p, int dtype, int row_blocks, hipStream_t s)
{
    int threads = 0;
    const void *k = tile_kernel_ptr(dtype, p.head_size_k, p.head_size_v, row_blocks, &threads);
    if (!k)
        return hipErrorInvalidValue;
    void *args[] = {(void *)&p};
    return hipLaunchKernel(k, dim3(p.partitions), dim3(threads), args, 0, s);
}

}  // namespace pa

// pa_tile_kernels.h -- paged attention on the matrix cores (gfx950 MFMA):
// the kernel templates and their shape selection, included by the
// translation units that instantiate them (pa_tile.hip without the band
// mask, pa_tile_band.hip with it).
//
// For units of 5 rows or more: parallel decoding / splitfuse chunks with the
// prefix-aligned causal mask (Ascend ATB PagedAttentionOperation,
// Constraints, mask type 5 list), decode with GQA groups of 8 or more, and a
// wide GQA group on one KV head with 576/512 key/value head sizes (which the
// same Constraints allow at block_size <= 128).  Rows are padded to 16.
//
// A workgroup of NW waves owns a tile of rows of one (sequence, KV head).  The
// waves form NW / CS row groups of 16 * MB rows; the CS waves of a row group
// share its rows and split the Dv output columns (CS = 2 halves the output
// accumulator per wave for Dv = 512).  Per KT-token chunk:
//
//   stage  K and V rows are copied from the paged cache straight into LDS
//          with global_load_lds_dwordx4 (no registers, no ALU work) into a
//          ring of S stages, S - 1 chunks ahead of the one computed.  Each
//          lane picks the global 16-byte piece that lands at its LDS slot,
//          which realises an XOR swizzle of the pieces within a row (K:
//          piece ^ (row & 7); V: piece ^ 2(row & 7), or ^ (row & 7) for
//          128-byte rows), so the operand reads below are free of bank
//          conflicts.  A block id out of range reads
//          a zero page (and is flagged); rows past the visible range are
//          masked (P = 0, and their V operand halves are zeroed).
//   S^T    = K . Q^T with v_mfma_f32_16x16x32_{f16,bf16}: K is the A operand
//          (ds_read_b128), Q^T the B operand, held in registers for the whole
//          unit.  The accumulator gives every lane one query row and 4 + 4
//          tokens, which is exactly the A-operand layout P needs for the next
//          product, so P never leaves registers.
//   mask   select -inf where j >= kv or (causal) j > prefix + i; chunks that
//          lie wholly inside every row's visible range skip the test, and
//          chunks wholly outside are never planned.
//   PV     O += P . V with the same instruction (16x16x16 for 16-token
//          chunks); the V operand is read from the row-major tile with
//          ds_read_b64_tr_b16 (a transposing LDS read: within each 16-lane
//          group, lane i receives element i % 4 of the 8-byte chunks
//          addressed by lanes i / 4, 4 + i / 4, 8 + i / 4 and 12 + i / 4).
//
// Every wave issues the same number of LDS loads per chunk, so the wait for
// chunk c is an exact vmcnt count, followed by one barrier.  Row statistics
// (running max and sum, log2 domain) stay per wave; at the end of a unit's
// range O is normalised into the output, or written as an fp32 partial for
// the merge kernel.
#ifndef PA_TILE_KERNELS_H_
#define PA_TILE_KERNELS_H_

#include "pa_internal.h"

#include <type_traits>

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

// Two 16-bit values packed as (lo, hi), round to nearest even.
template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi)
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

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) void lds_void;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
// 16 bytes per lane from global memory straight into LDS: lane l's bytes
// land at dst + 16 l (global_load_lds_dwordx4, LDS base in M0).  Issued from
// inline assembly so that the compiler does not add waits of its own for
// these stores; the kernel waits for them explicitly (vmcnt + barrier)
// before it reads the LDS they fill.
__device__ __forceinline__ void lds_load16(const void *src, lds_u8 *dst)
{
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(m0) : "memory", "m0");
}

// 4 bytes per lane from global memory into LDS (lane l -> dst + 4 l); the
// source must be 4-byte aligned.  Waited for like lds_load16.
__device__ __forceinline__ void lds_load4(const void *src, lds_u8 *dst)
{
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" : : "v"(src), "s"(m0) : "memory", "m0");
}

// Kernel modes: the mask kinds that need code of their own.
enum { MODE_PLAIN = 0, MODE_BAND = 1, MODE_TENSOR = 2, MODE_SPARSE = 3 };
constexpr int kMaskDim = 2048;   // side of the shared mask matrix (tensor mask)
constexpr int kSparseMaxTopk = 2048;   // list entries a segment stages in LDS (sparse lists)

// Tensor mask: per chunk, the slice of the shared matrix a tile needs is
// staged in LDS next to the K/V tiles, one row per query index of the tile
// (at most R), KT + 2 columns from an even start (dword-aligned loads).
template <int KT>
constexpr int slab_row_dwords()
{
    return (KT + 2) / 2;
}
template <int R, int KT>
constexpr int slab_bytes()
{
    return ((R * slab_row_dwords<KT>() + 63) / 64) * 256;
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t h)
{
    return (float)__builtin_bit_cast(_Float16, h);
}

template <int DT>
struct Mfma16;   // 16 x 16 x 16 products (PV over 16-token chunks)

template <>
struct Mfma16<0> {
    typedef _Float16 v4 __attribute__((ext_vector_type(4)));
    static __device__ __forceinline__ f32x4 run(uint2 a, uint2 b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(v4, a), __builtin_bit_cast(v4, b), c, 0, 0, 0);
    }
};

template <>
struct Mfma16<1> {
    static __device__ __forceinline__ f32x4 run(uint2 a, uint2 b, f32x4 c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(v4i16, a), __builtin_bit_cast(v4i16, b), c,
                                                         0, 0, 0);
    }
};

// s_waitcnt with vmcnt(n) only (gfx9 encoding: vmcnt in bits 3:0 and 15:14).
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt lgkmcnt(0) only.
__device__ __forceinline__ void wait_lgkm0()
{
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
}

// Wait until at most LW * min(ahead, A) vector memory instructions of this
// wave are outstanding.
template <int LW, int A>
__device__ __forceinline__ void wait_ahead(int ahead)
{
    if constexpr (A == 0) {
        wait_vm<0>();
    } else {
        if (ahead >= A)
            wait_vm<LW * A>();
        else
            wait_ahead<LW, A - 1>(ahead);
    }
}

// XOR swizzle of the 16-byte pieces of V tile row r.  The PV operand is
// read with ds_read_b64_tr_b16, whose 32-lane passes touch pieces 2 nd and
// 2 nd + 1 of rows 8 i .. 8 i + 7; the swizzle spreads those 16 pieces over
// all 64 banks: rows of a multiple of 256 bytes move by 2 (r % 8) pieces,
// 128-byte rows (which alternate between the two bank halves) by r % 8.
template <int RB>
__device__ __forceinline__ int v_swz(int r)
{
    return RB % 256 == 0 ? 2 * (r & 7) : (r & 7);
}
// Per-lane read offsets the swizzle needs: one per nd % NVO.
template <int RB>
constexpr int v_offsets()
{
    return RB % 256 == 0 ? 8 : 4;
}

// Workgroups per CU the register budget is cut for: as many as fit in LDS
// (at most 4; at most 2 with two 16-row blocks per wave, 1 at head sizes
// above 128).  SH: no V tiles in LDS.  TM: a tensor-mask slab per stage.
template <int DK, int DV, int MB, int KT, int S, int NW, int CS, bool SH, bool TM>
constexpr int tile_min_wgs()
{
    constexpr int lds = S * KT * 2 * (DK + (SH ? 0 : DV)) + 2048 +
                        (TM ? S * slab_bytes<16 * MB * (NW / CS), KT>() : 0);
    constexpr int fit = (160 * 1024) / lds;
    // waves per SIMD the registers allow: 2 with two 16-row blocks (1 at
    // head sizes above 128), 2 at head sizes above 128, else 4
    constexpr int waves = MB == 2 ? ((DK > 128 || DV > 128) ? 1 : 2) : (DK > 128 || DV > 128 ? 2 : 4);
    constexpr int cap = 4 * waves / NW > 0 ? 4 * waves / NW : 1;
    return fit < 1 ? 1 : (fit > cap ? cap : fit);
}

// DT: 0 f16 / 1 bf16.  MB: 16-row blocks per wave.  KT: tokens per chunk
// (16, 32 or 64).  NW: waves.  CS: waves sharing a row group (column split).
// S: LDS stages (chunks c + 1 .. c + S - 1 are in flight while c is
// computed).  SH: shared K/V cache -- V is the leading Dv elements of each
// K row, so only K tiles are loaded and the PV product reads its operand
// from the K tile (the K swizzle keeps those transposing reads free of
// bank conflicts as well).  MODE_BAND: band mask (rows also have a lower
// visibility bound, and a unit starts at the chunk of its lowest visible
// token); otherwise the lower bounds are the constant 0.  MODE_TENSOR: the
// shared mask matrix is added to the scaled scores (row i, token j: element
// [i][j - prefix]; history visible with nothing added; the causal rule
// outside the matrix); the matrix slice of each chunk is staged in LDS with
// the chunk, and the online softmax runs on scaled log2-domain scores.
// MODE_SPARSE: the KV tokens of a unit are the entries of its query token's
// list (all rows of a tile belong to one query token): chunk c holds list
// entries 16 c .. 16 c + 15.  At the start of a segment the workgroup
// resolves all its entries to cache rows (list entry, then block id) into
// LDS, so the chunk loop never waits for a lookup; each lane's LDS-load
// piece comes from the cache row of its entry's token (the rows of a chunk
// sit one per lane and each lane takes its own with ds_bpermute), and a
// per-chunk bit mask marks the entries that select a visible token.
template <int DT, int DK, int DV, int MB, int KT, int NW, int CS, int S, bool SH, int MODE, bool SELF = false>
__global__ __launch_bounds__(64 * NW, (tile_min_wgs<DK, DV, MB, KT, S, NW, CS, SH, MODE == MODE_TENSOR>()))
void tile_kernel(Params p)
{
    constexpr bool BAND = MODE == MODE_BAND, TMASK = MODE == MODE_TENSOR, SPARSE = MODE == MODE_SPARSE;
    static_assert(!SPARSE || KT == 16, "sparse lists are taken 16 entries per chunk");
    constexpr int RGS = NW / CS;                  // row groups
    constexpr int R = 16 * MB * RGS;              // rows per tile
    constexpr int RBK = 2 * DK, RBV = 2 * DV;     // LDS row bytes
    constexpr int RBVL = SH ? RBK : RBV;          // LDS row bytes of the tile the V operand is read from
    constexpr int KS = DK / 32;
    constexpr int NTT = KT / 16;
    constexpr int ND = DV / 16 / CS;              // output column tiles per wave
    constexpr int IPGK = RBK / 64;                // 1 KiB LDS-load instructions per 16-token group (K)
    constexpr int IPGV = SH ? 0 : RBV / 64;
    constexpr int MK = (IPGK + NW - 1) / NW;      // ... per wave per group
    constexpr int MV = (IPGV + NW - 1) / NW;
    constexpr int LW = NTT * (MK + MV);           // load instructions per wave per chunk, all waves alike
    constexpr bool PAD = MK * NW != IPGK || MV * NW != IPGV;
    constexpr int VTB = SH ? 16 : KT * RBV;       // bytes of a V stage buffer
    constexpr int SDW = slab_row_dwords<KT>();
    constexpr int SLB = TMASK ? slab_bytes<R, KT>() : 16;   // bytes of a mask slab stage
    static_assert(DK % 32 == 0 && DV % 64 == 0 && (KT == 16 || KT == 32 || KT == 64), "shape");
    static_assert(NW % CS == 0 && ND % 4 == 0 && S >= 2 && S <= 4, "split");
    static_assert(LW * (S - 2) < 64, "vmcnt range");
    static_assert(!SH || DV <= DK, "V inside the K row");
    // explicit interleave of operand reads and MFMAs (128-row tiles)
    constexpr bool SCHED = MB == 2;
    // the same for the 576/512 tiles, a few fragments ahead (one 16-row
    // block per wave, registers for a short ring only)
    constexpr bool PIPE = MB == 1 && DK > 256;
    constexpr int PFK = 2, PFV = 3;

    // the S stages of the ring, each a K tile, a V tile (none with one K/V
    // cache) and a mask slab (tensor mask only)
    constexpr int VSB = SH ? 0 : VTB;
    constexpr int MSB = TMASK ? SLB : 0;
    __shared__ __attribute__((aligned(1024))) uint8_t sK[S * KT * RBK];
    __shared__ __attribute__((aligned(1024))) uint8_t sV[SH ? 16 : S * VSB];
    __shared__ __attribute__((aligned(256))) uint8_t sM[TMASK ? S * MSB : 16];
    // destination of the padding loads that keep every wave's count at LW
    __shared__ __attribute__((aligned(1024))) uint8_t sJunk[PAD ? 1024 : 16];
    // sparse: the cache row of every list entry of the segment (-1: skipped)
    __shared__ int s_rows[SPARSE ? kSparseMaxTopk : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rgi = wave / CS;          // row group
    const int csl = wave % CS;          // column slice
    const int col0 = csl * (DV / CS);
    const int lr = lane & 15;
    const int lg = lane >> 4;

    int piece = xcd_logical_index(blockIdx.x, gridDim.x);
    Cursor cu;
    int end;
    __shared__ int s_piece;
    // SELF (the kernel plans for itself): context length, query length,
    // first packed query row and first item of each sequence
    __shared__ int s_skv[SELF ? kSelfPlanMaxBatch : 1], s_sql[SELF ? kSelfPlanMaxBatch : 1];
    __shared__ int s_st0[SELF ? kSelfPlanMaxBatch : 1], s_swsb[SELF ? kSelfPlanMaxBatch + 1 : 1];
    auto seq_kv = [&](int b) __attribute__((always_inline)) {
        if constexpr (SELF)
            return (int)__builtin_amdgcn_readfirstlane(s_skv[b]);
        else
            return sload(p.ws.kvlen, b);
    };
    auto seq_ql = [&](int b) __attribute__((always_inline)) {
        if constexpr (SELF)
            return (int)__builtin_amdgcn_readfirstlane(s_sql[b]);
        else
            return sload(p.ws.qlen, b);
    };
    auto seq_t0 = [&](int b) __attribute__((always_inline)) {
        if constexpr (SELF)
            return (int)__builtin_amdgcn_readfirstlane(s_st0[b]);
        else
            return sload(p.ws.cu_q, b);
    };
    auto seq_wsb = [&](int b) __attribute__((always_inline)) {
        return (int)__builtin_amdgcn_readfirstlane(s_swsb[b]);
    };
    // Whole-tile mode (the planner's choice for this pass): tasks come from
    // the queue of this workgroup's XCD (the dispatcher deals workgroups
    // round-robin over the XCDs), one whole row tile each: the first at a
    // fixed position, the others claimed (tile_claim) when kClaimAhead chunks
    // of the current one are left, by thread 0, whose claim returns while
    // those chunks are computed.
    const bool ordered = !SELF && tile_whole_tasks(DK, SH) && p.tile_order && sload(p.ws.tq, kTqMode) != 0;
    const int xq = blockIdx.x % kXcds;   // whole-tile mode: this workgroup's queue
    constexpr int kClaimAhead = 3;
    int nxt = 0;   // whole-tile mode, lane 0 of wave 0: the position claimed for the next task
    if constexpr (SELF) {
        // The kernel's own plan, for at most kSelfPlanMaxBatch sequences of
        // one row tile per (sequence, KV head), one piece per workgroup or
        // (no split) one unit: wave 0 reads the lengths, up to four
        // consecutive sequences per lane, and keeps each sequence's lengths,
        // first packed query row and first item in LDS; then every wave
        // finds its piece there and cuts it as the plan kernel would.
        // Workgroup 0 writes the header and the error bits, every
        // workgroup the split entry its piece starts.
        if (piece >= p.partitions)
            return;
        if (wave == 0) {
            const int cap = seq_cap(p);
            const int spl = (p.batch + 63) >> 6;
            int kvr[4] = {0, 0, 0, 0}, qlr[4] = {0, 0, 0, 0};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int b = spl * lane + i;
                if (i < spl && b < p.batch) {
                    kvr[i] = p.context_lens[b];
                    qlr[i] = p.q_seq_lens ? p.q_seq_lens[b] : 1;
                }
            }
            uint32_t serr = 0;
            int t0r[4], wsbr[4];
            int lq = 0, lw = 0;   // the lane's running sums
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int b = spl * lane + i;
                int ipg = 0;
                if (i < spl && b < p.batch) {
                    serr |= sanitize_seq(p, cap, kvr[i], qlr[i]);
                    ipg = seq_items_per_group(p, kvr[i], qlr[i]);
                }
                t0r[i] = lq;
                wsbr[i] = lw;
                lq += qlr[i];
                lw += ipg * p.kv_head_num;
            }
            const int iq = wave_scan(lq, lane), iw = wave_scan(lw, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int b = spl * lane + i;
                if (i < spl && b < p.batch) {
                    s_skv[b] = kvr[i];
                    s_sql[b] = qlr[i];
                    s_st0[b] = t0r[i] + iq - lq;
                    s_swsb[b] = wsbr[i] + iw - lw;
                }
            }
            const int cq = __builtin_amdgcn_readlane(iq, 63), W = __builtin_amdgcn_readlane(iw, 63);
            if (lane == 0)
                s_swsb[p.batch] = W;
            if (piece == 0) {
#pragma unroll
                for (int d = 1; d < 64; d <<= 1)
                    serr |= __shfl_xor(serr, d);
                if (cq != p.num_q_tokens)
                    serr |= PA_DEVERR_TOKENS;
                if (lane == 0) {
                    // the header as the plan kernel writes it (the piece
                    // counter, hdr[3], is the merge kernel's to reset)
                    const int per = p.no_split ? 0 : (W + p.pieces - 1) / p.pieces;
                    p.ws.hdr[0] = W;
                    p.ws.hdr[1] = per > 0 ? per : (p.no_split ? 0 : 1);
                    p.ws.hdr[2] = p.no_split ? 0 : p.pieces;
                    p.ws.hdr[4] = p.no_split ? 0 : p.pieces;
                    p.ws.hdr[5] = 0;
                    p.ws.hdr[6] = p.partitions;
                    p.ws.hdr[7] = 0;
                    if (serr)
                        set_error(p.ws.err, serr);
                }
            }
        }
        __syncthreads();
        const int W = seq_wsb(p.batch);
        if (p.no_split) {
            // workgroup w: unit (w / Hkv, w % Hkv), if its sequence has rows
            const int b = piece / p.kv_head_num;
            if (b >= p.batch)
                return;
            const int ql = seq_ql(b);
            if (ql <= 0)
                return;
            const int kv = seq_kv(b);
            cu.b = b;
            cu.g = piece - b * p.kv_head_num;
            cu.qt = 0;
            cu.c = 0;
            cu.ntile = seq_tiles(p, ql);
            cu.nch = unit_chunks(p, kv, ql, 0);
            cu.item = seq_wsb(b) + cu.g * cu.nch;
            end = cu.item + cu.nch;
        } else {
            // pieces of per items (one per workgroup: pieces == partitions)
            const int per = (W + p.pieces - 1) / p.pieces;
            const int s0 = piece * per;
            if (per <= 0 || s0 >= W) {
                // a boundary past the last item cuts nothing
                if (piece > 0 && wave == 0 && lane == 0)
                    p.ws.splits[(size_t)(piece - 1) * 8] = -1;
                return;
            }
            end = s0 + per < W ? s0 + per : W;
            // the sequence holding item s0: the last one whose first item is <= s0
            int lo = 0, hi = p.batch - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (seq_wsb(mid) <= s0)
                    lo = mid;
                else
                    hi = mid - 1;
            }
            const int kv = seq_kv(lo), ql = seq_ql(lo);
            cu = piece_start(p, piece, s0, s0 - per, lo, kv, ql, seq_items_per_group(p, kv, ql), seq_wsb(lo),
                             seq_t0(lo), wave == 0 && lane == 0);
        }
    } else if (ordered) {
        piece = tile_first_task(p, blockIdx.x);
        if (piece < 0)
            return;
        tile_task_cursor(p, piece, cu, end);
    } else if (piece >= p.partitions || !wg_range(p, piece, cu, end)) {
        return;
    }

    const uint16_t *__restrict__ qg = (const uint16_t *)p.query;
    const char *__restrict__ kg = (const char *)p.key_cache;
    const char *__restrict__ vg = (const char *)p.value_cache;
    const char *__restrict__ zg = (const char *)p.ws.zeros;
    const char *__restrict__ mg = (const char *)p.mask_tensor;
    uint16_t *__restrict__ og = (uint16_t *)p.out;
    const int G = p.group;
    const int H = p.head_num;
    const int bs = p.block_size;
    const int bsh = p.bs_shift;
    const uint32_t rsk = (uint32_t)p.kv_head_num * RBK;   // bytes per token row of the cache
    const uint32_t rsv = p.v_row_bytes;
    const uint32_t nb32 = p.num_blocks < 0x7fffffff ? (uint32_t)p.num_blocks : 0x7fffffffu;
    // every KT-token chunk lies in one cache block
    const bool chunk_in_block = bs % KT == 0;
    // Scores are kept raw (q . k) and scaled on the way into exp2 by
    // sc = |scale| log2(e); a negative scale is folded into Q.
    const bool neg_scale = p.scale_log2 < 0.f;
    const float scq = fmaxf(fabsf(p.scale_log2), 1e-30f);   // scale 0: every visible token weighs 1
    // Softmax domain: raw scores scaled by sc on the way into exp2 (with the
    // tensor mask the scores are scaled first, and sc is 1).
    const float sc = TMASK ? 1.f : scq;
    // The running max used as exp2 reference is only moved when a row's
    // max grows by more than 2^8 (P stays below 256, exact in the
    // 16-bit operand types); a moved reference rescales O and the sum.
    const float grow_raw = 8.f / sc;
    uint32_t err = 0;
    bool bad_id = false;   // a visible group's block id was out of range (wave-uniform)
    bool first_seg = true;

    // Per-lane byte offset, inside a 16-token group of the cache, of the piece
    // that load instruction wave + NW m of the group moves; the piece is the
    // one whose LDS slot holds the swizzled layout.
    // (sparse: the row part is per token -- tK / tV name the token of the
    // group the piece belongs to, voK / voV keep only the piece offset)
    uint32_t voK[MK], voV[MV > 0 ? MV : 1];
    int tK[MK], tV[MV > 0 ? MV : 1];
#pragma unroll
    for (int m = 0; m < MK; ++m) {
        const int x = (wave + NW * m) * 1024 + 16 * lane;
        const int row = x / RBK;
        tK[m] = row;
        voK[m] = (wave + NW * m) < IPGK ? (SPARSE ? 0u : row * rsk) + 16 * (((x % RBK) >> 4) ^ (row & 7)) : 16 * lane;
    }
#pragma unroll
    for (int m = 0; m < MV; ++m) {
        const int x = (wave + NW * m) * 1024 + 16 * lane;
        const int row = x / RBV;
        tV[m] = row;
        voV[m] = (wave + NW * m) < IPGV ? (SPARSE ? 0u : row * rsv) + 16 * (((x % RBV) >> 4) ^ v_swz<RBV>(row))
                                        : 16 * lane;
    }
    // LDS read offsets.  K (A operand): row 16 n + lr, piece 4 ks + lg, which
    // the swizzle moves by +-64 bytes depending on bit 2 of the row.
    const int kq = 16 * (lg ^ (lr & 3));
    const int kb2 = 64 * ((lr >> 2) & 1);
    const int koE = lr * RBK + kq + kb2, koO = lr * RBK + kq - kb2;
    // V (B operand, transposing read): row 4 lg + lr / 4 (+ 16 n),
    // columns col0 + 16 nd + 4 (lr % 4) .. + 3, i.e. 16-byte piece
    // col0 / 8 + 2 nd + (lr % 4) / 2 of the row, moved by the tile's swizzle
    // (the K swizzle when V is read from the K tile).  Column tile nd reads
    // at vo[nd % NVO] + (nd / NVO) NVO 32 bytes.
    constexpr int NVO = SH ? 4 : v_offsets<RBV>();
    int vo[NVO];
#pragma unroll
    for (int m = 0; m < NVO; ++m) {
        const int vrow = 4 * lg + (lr >> 2);
        const int vpiece = (2 * m + ((lr & 3) >> 1)) ^ (SH ? (vrow & 7) : v_swz<RBV>(vrow));
        vo[m] = vrow * RBVL + 16 * vpiece + 8 * (lr & 1) + 2 * col0;
    }

    while (true) {
        const int b = cu.b, g = cu.g, qt = cu.qt;
        const int kv = seq_kv(b);
        const int ql = seq_ql(b);
        // chunks [c0, c1) of the segment, counted from the sequence start (a
        // unit starts at the chunk holding its lowest visible token)
        const int cb = BAND ? unit_first_chunk(p, kv, ql, qt) : 0;
        const int nseg = cu.nch < cu.c + (end - cu.item) ? cu.nch - cu.c : end - cu.item;
        const bool whole = (cu.c == 0 && nseg == cu.nch);
        const int c0 = cb + cu.c;
        const int c1 = c0 + nseg;
        const int rows = ql * G;
        int rows_tile = rows - qt * R;
        rows_tile = rows_tile < R ? rows_tile : R;
        const int t0 = seq_t0(b);
        const int prefix = seq_prefix(kv, ql);
        // tokens [lo_tile, nvis) are seen by some row of the tile; every row
        // sees [max_lo, min_lim) (the thresholds below which, and from which
        // on, a chunk needs the per-element mask)
        const int nvis = SPARSE ? kv : row_hi_t<BAND>(p, kv, prefix, (qt * R + rows_tile - 1) / G);
        const int nblk = nvis > 0 ? div_bs(nvis - 1, bs, bsh) + 1 : 1;
        const int min_lim = row_hi_t<BAND>(p, kv, prefix, (qt * R) / G);
        const int lo_tile = row_lo_t<BAND>(p, prefix, (qt * R) / G);
        const int max_lo = row_lo_t<BAND>(p, prefix, (qt * R + rows_tile - 1) / G);
        // tensor mask: query indices [i0, i0 + nim) of the tile have matrix rows
        const int i0 = (qt * R) / G;
        int nim = 0;
        if constexpr (TMASK) {
            const int i1 = (qt * R + rows_tile - 1) / G;
            nim = (i1 < kMaskDim - 1 ? i1 : kMaskDim - 1) - i0 + 1;
            nim = nim > 0 ? nim : 0;
        }
        const int wr0 = rgi * 16 * MB;
        const bool wave_active = wr0 < rows_tile;
        const int32_t *bt = p.block_tables + (size_t)b * p.max_blocks;
        const char *kgh = kg + (size_t)g * RBK;
        const char *vgh = vg + (size_t)g * p.v_head_bytes;

        // Q^T operand and the visible range [lo_r, lim) of this lane's rows
        u32x4 qb[MB][KS];
        int lim[MB], lo_r[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const int row_t = wr0 + 16 * mb + lr;
            const int rg = qt * R + row_t;
            const int t = t0 + rg / G;
            const bool ok = row_t < rows_tile && t < p.num_q_tokens;
            lim[mb] = row_hi_t<BAND>(p, kv, prefix, rg / G);
            lo_r[mb] = row_lo_t<BAND>(p, prefix, rg / G);
            const uint16_t *src = qg + ((size_t)t * H + g * G + rg % G) * DK + 8 * lg;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                qb[mb][ks] = ok ? *(const u32x4 *)(src + 32 * ks) : u32x4{0u, 0u, 0u, 0u};
                if (neg_scale)   // exact: softmax(c s) = softmax(|c| (-s)) with -s = (-q) . k
                    qb[mb][ks] ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
            }
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

        // Block id and slot of each 16-token group of the chunk fetched last
        // (clamped table index; the id is range-checked when used).  Chunks
        // are fetched in order, so the block and slot of the next fetch
        // (f_blk, f_slot) advance by additions; a 16-token group never
        // crosses a block (block_size % 16 == 0).
        int bid[NTT], bslot[NTT];
        int f_blk = 0, f_slot = 0;
        // sparse: the tile's query token, its list, the tokens it may see
        // (c < lim_c), and for the fetched chunk the cache row of entry t in
        // lane t (srow) and the entries that select a visible token (sbits)
        const int itok = (qt * R) / G;
        const bool lst_ok = SPARSE && t0 + itok < p.num_q_tokens;
        const int lim_c = prefix + itok + 1 < kv ? prefix + itok + 1 : kv;
        const int32_t *lst = SPARSE ? p.topk_idx + ((size_t)(t0 + itok) * p.kv_head_num + g) * p.topk : nullptr;
        int srow = 0;
        uint32_t sbits = 0;
        // sparse: the visible-entry bits of the chunks issued and not yet
        // computed, oldest first
        uint32_t smask[S];
        auto fetch_bids = [&](int c) __attribute__((always_inline)) {
            if constexpr (SPARSE) {
                // entry 16 c + lane's row from the segment's table (lanes < 16)
                const int rv = lane < 16 ? s_rows[(c - c0) * 16 + lane] : -1;
                sbits = (uint32_t)__ballot(rv >= 0);
                srow = rv >= 0 ? rv : 0;
            } else {
                (void)c;
                // (wave-uniform: read once into scalar registers)
                int blk = __builtin_amdgcn_readfirstlane(f_blk), slot = __builtin_amdgcn_readfirstlane(f_slot);
                if (chunk_in_block) {
                    // the chunk lies in one block: one id for its groups
                    const int b0 = sload(bt, blk < nblk ? blk : nblk - 1);
#pragma unroll
                    for (int q = 0; q < NTT; ++q) {
                        bid[q] = b0;
                        bslot[q] = slot + 16 * q;
                    }
                    slot += KT;
                    if (slot == bs) {
                        slot = 0;
                        ++blk;
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < NTT; ++q) {
                        bid[q] = sload(bt, blk < nblk ? blk : nblk - 1);
                        bslot[q] = slot;
                        slot += 16;
                        if (slot == bs) {
                            slot = 0;
                            ++blk;
                        }
                    }
                }
                f_blk = blk;
                f_slot = slot;
            }
        };
        // Issue the LDS loads of chunk c: exactly LW instructions per wave.
        // Groups wholly outside the tile's visible range read the zero page
        // (their block-table entries are not used); their rows are masked in
        // compute anyway.
        auto issue = [&](int c, lds_u8 *kb, lds_u8 *vb, lds_u8 *mb_) __attribute__((always_inline)) {
            if constexpr (TMASK) {
                // the matrix slice of chunk c (beyond the fixed LW loads per
                // wave; extra loads only make the waits for later chunks
                // wait longer)
                const int c0m = c * KT - prefix;
                if (c0m < kMaskDim && c0m + KT > 0 && nim > 0) {
                    int cs = c0m & ~1;
                    cs = cs < 0 ? 0 : (cs > kMaskDim - 2 * SDW ? kMaskDim - 2 * SDW : cs);
                    const int ntot = nim * SDW;
                    const int nin = (ntot + 63) / 64;
                    for (int m = wave; m < nin; m += NW) {
                        const int x = m * 64 + lane;
                        const int r = x / SDW;
                        const char *src = x < ntot ? mg + ((size_t)(i0 + r) * kMaskDim + cs) * 2 + 4 * (x - r * SDW) : mg;
                        lds_load4(src, mb_ + m * 256);
                    }
                }
            }
            if constexpr (SPARSE) {
                // one 16-entry group: each lane's piece from its entry's row
                // (invalid entries read row 0 of block 0 and are masked)
#pragma unroll
                for (int m = 0; m < MK; ++m) {
                    const int i = wave + NW * m;
                    const bool real = !PAD || i < IPGK;
                    lds_u8 *dst = real ? kb + i * 1024 : (lds_u8 *)sJunk;
                    const uint32_t rl = (uint32_t)__builtin_amdgcn_ds_bpermute(tK[m] * 4, srow);
                    const char *src = real ? kgh + (size_t)rl * rsk + voK[m] : zg + voK[m];
                    lds_load16(src, dst);
                }
#pragma unroll
                for (int m = 0; m < MV; ++m) {
                    const int i = wave + NW * m;
                    const bool real = !PAD || i < IPGV;
                    lds_u8 *dst = real ? vb + i * 1024 : (lds_u8 *)sJunk;
                    const uint32_t rl = (uint32_t)__builtin_amdgcn_ds_bpermute(tV[m] * 4, srow);
                    const char *src = real ? vgh + (size_t)rl * rsv + voV[m] : zg + voV[m];
                    lds_load16(src, dst);
                }
                return;
            }
#pragma unroll
            for (int q = 0; q < NTT; ++q) {
                const int j0 = c * KT + 16 * q;
                const bool vis = j0 < nvis && (!BAND || j0 + 16 > lo_tile);
                const bool inb = (unsigned)bid[q] < nb32;
                bad_id |= vis && !inb;
                const size_t trow = (size_t)(uint32_t)bid[q] * (uint32_t)bs + (uint32_t)bslot[q];
                // (a bit select, which stays on the scalar unit)
                const uint64_t sel = (vis && inb) ? ~0ull : 0ull;
                const char *kbase = (const char *)((((uint64_t)kgh + trow * rsk) & sel) | ((uint64_t)zg & ~sel));
                const char *vbase = (const char *)((((uint64_t)vgh + trow * rsv) & sel) | ((uint64_t)zg & ~sel));
                // (the empty asm hides each 32-bit offset from loop-invariant
                // hoisting: otherwise the 64-bit forms of all of a chunk's
                // offsets stay live across the chunk loop, and where the
                // registers run out one is spilled and reloaded behind the
                // next chunk's first load, which then waits for that load;
                // with one K and one V offset per wave the two 64-bit forms
                // fit, and keeping them saves a copy per load)
#pragma unroll
                for (int m = 0; m < MK; ++m) {
                    const int i = wave + NW * m;
                    lds_u8 *dst = (!PAD || i < IPGK) ? kb + (q * IPGK + i) * 1024 : (lds_u8 *)sJunk;
                    const char *src = (!PAD || i < IPGK) ? kbase : zg;
                    uint32_t off = voK[m];
                    if constexpr (MK + MV > 2)
                        asm volatile("" : "+v"(off));
                    lds_load16(src + off, dst);
                }
#pragma unroll
                for (int m = 0; m < MV; ++m) {
                    const int i = wave + NW * m;
                    lds_u8 *dst = (!PAD || i < IPGV) ? vb + (q * IPGV + i) * 1024 : (lds_u8 *)sJunk;
                    const char *src = (!PAD || i < IPGV) ? vbase : zg;
                    uint32_t off = voV[m];
                    if constexpr (MK + MV > 2)
                        asm volatile("" : "+v"(off));
                    lds_load16(src + off, dst);
                }
            }
        };

        // one chunk from (kb, vb): S^T, mask, online softmax, PV.  NM: the
        // chunk needs the per-element mask (it reaches past the visible range
        // of some row of the tile); the other chunks take an instance
        // without any mask or tail code.
        auto compute = [&](auto nm, const lds_u8 *kb, const lds_u8 *vb, const lds_u8 *mb_, int c, uint32_t vbits)
                           __attribute__((always_inline)) {
            constexpr bool NM = decltype(nm)::value;
            if (!wave_active)
                return;
            const int jb = c * KT;
            f32x4 sacc[MB][NTT];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int n = 0; n < NTT; ++n)
                    sacc[mb][n] = f32x4{0.f, 0.f, 0.f, 0.f};
            if constexpr (SCHED) {
                // the K fragments of slice ks + 1 are read while slice ks is
                // multiplied (the scheduler, left alone, waits for each read)
                u32x4 ka[2][NTT];
#pragma unroll
                for (int n = 0; n < NTT; ++n)
                    ka[0][n] = *(const lds_u32x4 *)(kb + koE + 16 * n * RBK);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    if (ks + 1 < KS) {
#pragma unroll
                        for (int n = 0; n < NTT; ++n)
                            ka[(ks + 1) & 1][n] =
                                *(const lds_u32x4 *)(kb + (((ks + 1) & 1) ? koO : koE) + 16 * n * RBK + 64 * (ks + 1));
                    }
#pragma unroll
                    for (int n = 0; n < NTT; ++n)
#pragma unroll
                        for (int mb = 0; mb < MB; ++mb)
                            sacc[mb][n] = Mfma<DT>::run(ka[ks & 1][n], qb[mb][ks], sacc[mb][n]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else if constexpr (PIPE) {
                // fragment i + PFK is read while fragment i is multiplied
                constexpr int NR = KS * NTT;
                auto kread = [&](int i) __attribute__((always_inline)) -> u32x4 {
                    const int ks = i / NTT, n = i % NTT;
                    return *(const lds_u32x4 *)(kb + ((ks & 1) ? koO : koE) + 16 * n * RBK + 64 * ks);
                };
                u32x4 kr[PFK + 1];
#pragma unroll
                for (int i = 0; i < PFK && i < NR; ++i)
                    kr[i] = kread(i);
#pragma unroll
                for (int i = 0; i < NR; ++i) {
                    if (i + PFK < NR)
                        kr[(i + PFK) % (PFK + 1)] = kread(i + PFK);
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
                        sacc[mb][i % NTT] = Mfma<DT>::run(kr[i % (PFK + 1)], qb[mb][i / NTT], sacc[mb][i % NTT]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                    for (int n = 0; n < NTT; ++n) {
                        const u32x4 a = *(const lds_u32x4 *)(kb + ((ks & 1) ? koO : koE) + 16 * n * RBK + 64 * ks);
#pragma unroll
                        for (int mb = 0; mb < MB; ++mb)
                            sacc[mb][n] = Mfma<DT>::run(a, qb[mb][ks], sacc[mb][n]);
                    }
                }
            }
            if constexpr (TMASK) {
                // scaled log2-domain scores plus the matrix (log2 e times
                // its value); outside the matrix the causal rule
                const int c0m = jb - prefix;
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int n = 0; n < NTT; ++n)
                        sacc[mb][n] *= scq;
                if (c0m + KT > 0) {
                    int cs = c0m & ~1;
                    cs = cs < 0 ? 0 : (cs > kMaskDim - 2 * SDW ? kMaskDim - 2 * SDW : cs);
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) {
                        const int i = (qt * R + wr0 + 16 * mb + lr) / G;
                        const lds_u8 *row = mb_ + (i - i0) * (4 * SDW);
#pragma unroll
                        for (int n = 0; n < NTT; ++n) {
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                const int cj = c0m + 16 * n + 4 * lg + r;
                                if ((unsigned)cj < (unsigned)kMaskDim && i < kMaskDim) {
                                    const uint16_t hb = *(const __attribute__((address_space(3))) uint16_t *)(row + 2 * (cj - cs));
                                    sacc[mb][n][r] = __builtin_fmaf(f16_bits_to_f32(hb), 1.4426950408889634f, sacc[mb][n][r]);
                                } else if (cj > i) {
                                    sacc[mb][n][r] = -INFINITY;
                                }
                            }
                        }
                    }
                }
            }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                float mx = -INFINITY;
#pragma unroll
                for (int n = 0; n < NTT; ++n) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        if constexpr (NM) {
                            const int j = jb + 16 * n + 4 * lg + r;
                            const bool vis = SPARSE ? ((vbits >> (16 * n + 4 * lg + r)) & 1u) != 0
                                                    : (j < lim[mb] && (!BAND || j >= lo_r[mb]));
                            sacc[mb][n][r] = vis ? sacc[mb][n][r] : -INFINITY;
                        }
                        mx = fmaxf(mx, sacc[mb][n][r]);
                    }
                }
                mx = xor_max<16>(mx);
                mx = xor_max<32>(mx);
                if (__any(mx > m_run[mb] + grow_raw)) {
                    const float m_new = fmaxf(m_run[mb], mx);
                    const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f((m_run[mb] - m_new) * sc);
                    lsum[mb] *= alpha;
                    m_run[mb] = m_new;
                    // O rows 4 lg + r take the factor of the lane holding that row
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float ar = __shfl(alpha, 4 * lg + r);
#pragma unroll
                        for (int nd = 0; nd < ND; ++nd)
                            oacc[mb][nd][r] *= ar;
                    }
                }
                const float mref = m_run[mb] == -INFINITY ? 0.f : m_run[mb] * sc;
                float ps = 0.f;
#pragma unroll
                for (int n = 0; n < NTT; ++n) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[mb][n][r], sc, -mref));
                        sacc[mb][n][r] = pv;
                        ps += pv;
                    }
                }
                lsum[mb] += ps;
            }
            // V rows of tokens outside [lo_tile, nvis) may be stale or
            // unwritten cache slots: zero their operand halves (P is 0 there).
            // (Such a chunk always takes the masked instance: nvis and lo_tile
            // bound the visible range of every row.)
            const bool tail = NM && (SPARSE || jb + KT > nvis || (BAND && jb < lo_tile));
            auto tok_ok = [&](int t) __attribute__((always_inline)) {
                if constexpr (SPARSE)
                    return ((vbits >> (t - jb)) & 1u) != 0;
                else
                    return BAND ? (unsigned)(t - lo_tile) < (unsigned)(nvis - lo_tile) : t < nvis;
            };
            if constexpr (KT == 16) {
                uint2 pa[MB];
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    pa[mb] = uint2{pack2<DT>(sacc[mb][0][0], sacc[mb][0][1]), pack2<DT>(sacc[mb][0][2], sacc[mb][0][3])};
                uint2 vm = {~0u, ~0u};
                if (tail) {
                    const int tb = jb + 4 * lg;
                    vm.x = (tok_ok(tb) ? 0xffffu : 0u) | (tok_ok(tb + 1) ? 0xffff0000u : 0u);
                    vm.y = (tok_ok(tb + 2) ? 0xffffu : 0u) | (tok_ok(tb + 3) ? 0xffff0000u : 0u);
                }
                auto vread = [&](int nd) __attribute__((always_inline)) -> uint2 {
                    const v4i16 b0 =
                        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(vb + vo[nd % NVO] + 32 * NVO * (nd / NVO)));
                    return __builtin_bit_cast(uint2, b0);
                };
                if constexpr (PIPE) {
                    // column tile nd + PFV is read while tile nd is multiplied
                    uint2 vr[PFV + 1];
#pragma unroll
                    for (int i = 0; i < PFV && i < ND; ++i)
                        vr[i] = vread(i);
#pragma unroll
                    for (int nd = 0; nd < ND; ++nd) {
                        if (nd + PFV < ND)
                            vr[(nd + PFV) % (PFV + 1)] = vread(nd + PFV);
                        uint2 bv = vr[nd % (PFV + 1)];
                        if (tail) {
                            bv.x &= vm.x;
                            bv.y &= vm.y;
                        }
#pragma unroll
                        for (int mb = 0; mb < MB; ++mb)
                            oacc[mb][nd] = Mfma16<DT>::run(pa[mb], bv, oacc[mb][nd]);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                } else {
#pragma unroll
                    for (int nd = 0; nd < ND; ++nd) {
                        uint2 bv = vread(nd);
                        if (tail) {
                            bv.x &= vm.x;
                            bv.y &= vm.y;
                        }
#pragma unroll
                        for (int mb = 0; mb < MB; ++mb)
                            oacc[mb][nd] = Mfma16<DT>::run(pa[mb], bv, oacc[mb][nd]);
                    }
                }
            } else {
#pragma unroll
                for (int kk = 0; kk < KT / 32; ++kk) {
                    u32x4 pa[MB];
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) {
                        const f32x4 s0 = sacc[mb][2 * kk], s1 = sacc[mb][2 * kk + 1];
                        pa[mb] = u32x4{pack2<DT>(s0[0], s0[1]), pack2<DT>(s0[2], s0[3]),
                                       pack2<DT>(s1[0], s1[1]), pack2<DT>(s1[2], s1[3])};
                    }
                    u32x4 vm = {~0u, ~0u, ~0u, ~0u};
                    if (tail) {
                        const int tb = jb + 32 * kk + 4 * lg;
#pragma unroll
                        for (int h = 0; h < 2; ++h)
#pragma unroll
                            for (int e = 0; e < 2; ++e)
                                vm[2 * h + e] = (tok_ok(tb + 16 * h + 2 * e) ? 0xffffu : 0u) |
                                                (tok_ok(tb + 16 * h + 2 * e + 1) ? 0xffff0000u : 0u);
                    }
                    auto vread = [&](int nd) __attribute__((always_inline)) -> u32x4 {
                        const int off = 32 * kk * RBVL + 32 * NVO * (nd / NVO);
                        const v4i16 b0 =
                            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(vb + vo[nd % NVO] + off));
                        const v4i16 b1 =
                            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(vb + vo[nd % NVO] + off + 16 * RBVL));
                        const uint2 lo = __builtin_bit_cast(uint2, b0), hi = __builtin_bit_cast(uint2, b1);
                        return u32x4{lo.x, lo.y, hi.x, hi.y};
                    };
                    if constexpr (SCHED && ND % 4 == 0) {
                        // the V fragments of 4 column tiles are read while the
                        // previous 4 are multiplied
                        u32x4 vf[2][4];
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            vf[0][i] = vread(i);
#pragma unroll
                        for (int q = 0; q < ND / 4; ++q) {
                            if (q + 1 < ND / 4) {
#pragma unroll
                                for (int i = 0; i < 4; ++i)
                                    vf[(q + 1) & 1][i] = vread(4 * (q + 1) + i);
                            }
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                u32x4 bv = vf[q & 1][i];
                                if (tail)
                                    bv &= vm;
#pragma unroll
                                for (int mb = 0; mb < MB; ++mb)
                                    oacc[mb][4 * q + i] = Mfma<DT>::run(pa[mb], bv, oacc[mb][4 * q + i]);
                            }
                            __builtin_amdgcn_sched_barrier(0);
                        }
                    } else {
#pragma unroll
                        for (int nd = 0; nd < ND; ++nd) {
                            u32x4 bv = vread(nd);
                            if (tail)
                                bv &= vm;
#pragma unroll
                            for (int mb = 0; mb < MB; ++mb)
                                oacc[mb][nd] = Mfma<DT>::run(pa[mb], bv, oacc[mb][nd]);
                        }
                    }
                }
            }
        };

        auto kbuf = [&](int st) __attribute__((always_inline)) -> lds_u8 * {
            return (lds_u8 *)sK + st * (KT * RBK);
        };
        auto vbuf = [&](int st) __attribute__((always_inline)) -> lds_u8 * {
            if constexpr (SH)
                return kbuf(st);
            else
                return (lds_u8 *)sV + st * VSB;
        };
        auto mbuf = [&](int st) __attribute__((always_inline)) -> lds_u8 * {
            return (lds_u8 *)sM + st * MSB;
        };
        // one pipeline step: chunk c sits in stage st (NM: the chunk takes
        // the masked instance of compute)
        auto step = [&](auto nm, int st, int c) __attribute__((always_inline)) {
            const int nx = st == 0 ? S - 1 : st - 1;   // stage of chunk c + S - 1
            wait_ahead<LW, S - 2>(c1 - 1 - c);     // this wave's loads of chunk c are in LDS
            __builtin_amdgcn_s_barrier();          // ... and every wave's; stage nx is free
            if (c + S - 1 < c1) {
                issue(c + S - 1, kbuf(nx), vbuf(nx), mbuf(nx));
                if constexpr (SPARSE)
                    smask[S - 1] = sbits;
            }
            compute(nm, kbuf(st), vbuf(st), mbuf(st), c, smask[0]);
            if constexpr (SPARSE) {
#pragma unroll
                for (int i = 0; i + 1 < S; ++i)
                    smask[i] = smask[i + 1];
            }
            if (c + S < c1)
                fetch_bids(c + S);                 // scalar loads land during the next wait
        };

        // Q in registers before the LDS loads start: the vector memory
        // counter then covers only those loads.  All waves are done reading
        // every stage (previous segment).
        wait_vm<0>();
        __syncthreads();
        if constexpr (SPARSE) {
            // resolve the segment's list entries to cache rows (two dependent
            // loads each, all entries at once), before any LDS load is issued
            for (int k = c0 * 16 + tid; k < c1 * 16; k += 64 * NW) {
                int row = -1;
                if (lst_ok && k < p.topk) {
                    const int ci = lst[k];
                    if (ci >= 0 && ci < lim_c) {
                        const int blk = bt[div_bs(ci, bs, bsh)];
                        if ((unsigned)blk < nb32)
                            row = (int)((uint32_t)blk * (uint32_t)bs + (uint32_t)mod_bs(ci, bs, bsh));
                        else
                            err |= (uint32_t)PA_DEVERR_BLOCK_ID;
                    }
                }
                s_rows[k - c0 * 16] = row;
            }
            wait_vm<0>();
            __syncthreads();
        }
        if constexpr (!SPARSE) {
            f_blk = div_bs(c0 * KT, bs, bsh);
            f_slot = c0 * KT - f_blk * bs;
        }
        fetch_bids(c0);
        issue(c0, kbuf(0), vbuf(0), mbuf(0));
        smask[0] = sbits;
#pragma unroll
        for (int i = 1; i + 1 < S; ++i) {
            if (c0 + i < c1) {
                fetch_bids(c0 + i);
                issue(c0 + i, kbuf(i), vbuf(i), mbuf(i));
                smask[i] = sbits;
            }
        }
        if (c0 + S - 1 < c1)
            fetch_bids(c0 + S - 1);
        // A chunk needs the per-element mask where it reaches past the
        // visible range of the tile's first row (c KT + KT > min_lim: the
        // causal diagonal and the tail of the context) or, with the band
        // mask, before the start of its last row's window (c KT < max_lo).
        // Those chunks are a leading and a trailing run of the segment; the
        // chunks between take the unmasked instance.  Three loops, each with
        // one instance of compute, keep the register pressure of one.  In
        // whole-tile mode the trailing run is at least kClaimAhead chunks
        // long, and the next task is claimed before it.
        int cu0 = c0, cu1 = c0;   // the unmasked run [cu0, cu1)
        if constexpr (!SPARSE) {
            cu0 = BAND ? (max_lo + KT - 1) / KT : c0;
            cu0 = cu0 < c0 ? c0 : (cu0 > c1 ? c1 : cu0);
            cu1 = min_lim > 0 ? min_lim / KT : 0;
            if (ordered && cu1 > c1 - kClaimAhead)
                cu1 = c1 - kClaimAhead;
            cu1 = cu1 < cu0 ? cu0 : (cu1 > c1 ? c1 : cu1);
        }
        int c = c0, st = 0;
        for (; c < cu0; ++c, st = st + 1 == S ? 0 : st + 1)
            step(std::true_type{}, st, c);
        for (; c < cu1; ++c, st = st + 1 == S ? 0 : st + 1)
            step(std::false_type{}, st, c);
        if (ordered && threadIdx.x == 0)
            nxt = tile_claim(p, xq, gridDim.x);
        for (; c < c1; ++c, st = st + 1 == S ? 0 : st + 1)
            step(std::true_type{}, st, c);

        // -------------------------------------------------------- finalise
        if (wave_active) {
            // One-cache 576/512 tiles (at the register limit): the lane's
            // row and column taken afresh, so that the store indices derived
            // from them are computed here instead of being kept (spilled)
            // through the chunk loop
            constexpr bool FRESH = SH && !SPARSE && DK > 256;
            int lane_f = lane;
            if constexpr (FRESH)
                asm volatile("" : "+v"(lane_f));
            const int lr_f = FRESH ? (lane_f & 15) : lr, lg_f = FRESH ? (lane_f >> 4) : lg;
            const int slot = first_seg ? 0 : 1;
            float *part = p.ws.partials + (size_t)(2 * piece + slot) * p.partial_stride;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const float L = xor_sum<32>(xor_sum<16>(lsum[mb]));
                const float Ms = m_run[mb] * sc;   // log2 domain
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float Lr = __shfl(L, 4 * lg_f + r);
                    const float Mr = __shfl(Ms, 4 * lg_f + r);
                    const int row_t = wr0 + 16 * mb + 4 * lg_f + r;
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
                            dst[col0 + 16 * nd + lr_f] = to_bits<DT>(oacc[mb][nd][r] * inv);
                        if (lr_f == 0 && csl == 0 && p.lse)
                            p.lse[(size_t)t * H + h] =
                                Lr > 0.f ? (Mr + log2f(Lr)) * 0.69314718055994531f : -INFINITY;
                    } else {
#pragma unroll
                        for (int nd = 0; nd < ND; ++nd)
                            part[row_t * DV + col0 + 16 * nd + lr_f] = oacc[mb][nd][r];
                        if (lr_f == 0 && csl == 0) {
                            part[R * DV + row_t] = Mr;
                            part[R * DV + R + row_t] = Lr;
                        }
                    }
                }
            }
        }

        first_seg = false;
        cu.item += nseg;
        bool more = cu.item < end;
        if (more) {
            if constexpr (SELF) {
                // the next unit: one row tile per (sequence, KV head)
                cu.c = 0;
                if (++cu.g >= p.kv_head_num) {
                    cu.g = 0;
                    do {
                        ++cu.b;
                    } while (cu.b < p.batch && seq_ql(cu.b) <= 0);
                }
                if (cu.b < p.batch)
                    cu.nch = unit_chunks(p, seq_kv(cu.b), seq_ql(cu.b), 0);
            } else {
                cursor_next_unit(p, cu);
            }
            more = cu.b < p.batch;
        }
        if (!more) {
            if (ordered) {
                // the next whole tile, if any
                if (threadIdx.x == 0)
                    s_piece = tile_next_task(p, xq, gridDim.x, nxt);
                __syncthreads();
                piece = s_piece;
                if (piece < 0)
                    break;
                tile_task_cursor(p, piece, cu, end);
                first_seg = true;
                continue;
            }
            // this piece is done: take the next one, if any
            if (SELF || p.no_split || p.pieces <= p.partitions)
                break;
            if (threadIdx.x == 0)
                s_piece = grab_piece(p);
            __syncthreads();
            piece = s_piece;
            if (!wg_range(p, piece, cu, end))
                break;
            first_seg = true;
        }
    }
    if (bad_id)
        err |= (uint32_t)PA_DEVERR_BLOCK_ID;
    if (err)
        set_error(p.ws.err, err);
}

// ---------------------------------------------------------------------------
// Streaming kernel for units of at most 16 rows (decode).  A workgroup of
// two waves is a worker with an S-stage LDS ring: wave 0 issues the loads
// (chunk k + S - 1 of its stream, whatever unit or piece it belongs to),
// wave 1 computes chunk k, and one barrier per chunk hands a landed stage
// to wave 1 and the stage wave 1 has finished back to wave 0.  The ring does
// not drain between units, and the compute side's latencies (softmax, the
// start and end of a segment, its output stores) never hold back a load:
// the stores sit on the other wave's memory counter.  The first chunk of
// every segment also carries the segment's 16 x Dk Q tile into its stage,
// and each stage carries the chunk's segment parameters in a small LDS
// record, so the compute side never waits for a lookup.  MODE as for the
// tile kernel.
// SELF: the kernel plans for itself (no plan kernel, at most
// kSelfPlanMaxBatch sequences): the issuing wave reads and sums the lengths
// as the plan kernel does, finds its piece, writes the header (worker 0)
// and its piece's split entry, and keeps the sequences' lengths and first
// items in LDS, so neither the start nor a move to the next unit waits for
// plan data in memory.  With a claimed tail (PieceMap), a worker goes on
// from its static piece to pieces it claims from the shared counter.  The
// computing wave claims: the atomic's return would make the issuing wave
// wait on its in-order memory counter, behind every KV load in flight,
// while the computing wave's counter holds only its few stores.  It sends
// the atomic kClaimAhead chunks before it must know the answer and puts the
// claimed piece (or -1: none left) into LDS before the barrier after which
// the issuing wave issues the last chunk of the current piece; the issuing
// wave then moves straight on to the claimed piece and the ring never
// drains.  Every stage record carries the chunks left in its piece, and the
// last chunk of a worker's stream is flagged, so the two waves agree on the
// number of barriers.
template <int DT, int DK, int DV, int KT, int S, int MODE, bool SELF, bool TAIL, int HP>
__global__ __launch_bounds__(128, DK * HP > 128 ? (HP > 1 ? 2 : 1) : 3) void stream_kernel(Params p)
{
    static_assert(SELF || !TAIL, "a claimed tail needs the kernel's own plan");
    constexpr bool BAND = MODE == MODE_BAND, TMASK = MODE == MODE_TENSOR;
    constexpr int SDW = slab_row_dwords<KT>();
    constexpr int SLB = TMASK ? slab_bytes<16, KT>() : 0;   // bytes of a mask slab stage
    // HP KV heads per unit (head pairs: HP = 2): their K (V) rows sit side by
    // side in the cache, so a unit reads HP * Dk contiguous elements of each
    // token row and stages them as one wide row; each query row takes the
    // products with its own head's half (Q is zero in the other) and its
    // output from its own head's half of the wide PV product.
    constexpr int DKE = HP * DK, DVE = HP * DV;   // staged row elements
    constexpr int RBK = 2 * DKE, RBV = 2 * DVE;   // LDS row bytes
    constexpr int RBQ = 2 * DK;                   // Q tile row bytes (one query head)
    constexpr int KS = DKE / 32;
    constexpr int KSQ = DK / 32;                  // Q slices of one head
    constexpr int NTT = KT / 16;
    constexpr int ND = DVE / 16;
    constexpr int NDO = DV / 16;                  // output column tiles of one head
    constexpr int IPGK = RBK / 64;                // 1 KiB loads per 16 rows of K
    constexpr int IPGV = RBV / 64;
    constexpr int IPGQ = RBQ / 64;                // ... of the Q tile
    constexpr int LW = NTT * (IPGK + IPGV);       // loads per chunk (plus IPGQ for a Q tile)
    constexpr int STK = KT * RBK, STV = KT * RBV, STQ = 16 * RBQ;
    constexpr int MW = TAIL ? 13 : 12;            // ints per stage record
    constexpr int kClaimAhead = 4;                // chunks between a claim and its deadline
    static_assert(DKE <= 256 && DVE <= 256 && DK % 32 == 0 && DV % 64 == 0 && (KT == 16 || KT == 32), "shape");
    static_assert(HP == 1 || (HP == 2 && DK == DV), "head pairs");
    static_assert(S >= 2 && S <= 4 && LW * (S - 2) + IPGQ < 64, "ring");

    __shared__ __attribute__((aligned(1024))) uint8_t sK[S * STK];
    __shared__ __attribute__((aligned(1024))) uint8_t sV[S * STV];
    __shared__ __attribute__((aligned(1024))) uint8_t sQ[S * STQ];
    __shared__ __attribute__((aligned(256))) uint8_t sMk[TMASK ? S * SLB : 16];
    __shared__ int s_meta[S * MW];
    // SELF: context length, first packed query row and query length
    // (at most 16 here) of each sequence
    __shared__ int s_skv[SELF ? kSelfPlanMaxBatch : 1], s_st0[SELF ? kSelfPlanMaxBatch : 1];
    __shared__ uint8_t s_sql[SELF ? kSelfPlanMaxBatch : 4];
    // SELF: first item of each sequence; the piece claimed next (index, or
    // -1: none; then its cursor and end item)
    __shared__ int s_wsb[TAIL ? kSelfPlanMaxBatch : 1];
    __shared__ int s_claim[TAIL ? 9 : 1];

    __shared__ int s_n, s_dyn;   // chunks of the first piece, claimed tail
    __shared__ PieceMap s_pm;    // TAIL: the pass's piece map
    const int lane = threadIdx.x & 63;
    const int lr = lane & 15;
    const int lg = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);   // 0 issues, 1 computes
    const int worker = xcd_logical_index(blockIdx.x, gridDim.x);

    const uint16_t *__restrict__ qg = (const uint16_t *)p.query;
    const char *__restrict__ kg = (const char *)p.key_cache;
    const char *__restrict__ vg = (const char *)p.value_cache;
    const char *__restrict__ zg = (const char *)p.ws.zeros;
    const char *__restrict__ mg = (const char *)p.mask_tensor;
    uint16_t *__restrict__ og = (uint16_t *)p.out;
    const int G = p.group;
    const int H = p.head_num;
    const int bs = p.block_size;
    const int bsh = p.bs_shift;
    const uint32_t rsk = (uint32_t)p.kv_head_num * RBK;
    const uint32_t rsv = p.v_row_bytes;
    const uint32_t nb32 = p.num_blocks < 0x7fffffff ? (uint32_t)p.num_blocks : 0x7fffffffu;
    const bool neg_scale = p.scale_log2 < 0.f;
    const float scq = fmaxf(fabsf(p.scale_log2), 1e-30f);   // scale 0: every visible token weighs 1
    const float sc = TMASK ? 1.f : scq;   // scores already scaled with the tensor mask
    const float grow_raw = 8.f / sc;
    uint32_t err = 0;

    // per-lane offsets of the loads (inside a 16-token group / the Q tile)
    uint32_t voK[IPGK], voV[IPGV];
    int qrow[IPGQ], qlp[IPGQ];
#pragma unroll
    for (int m = 0; m < IPGK; ++m) {
        const int x = m * 1024 + 16 * lane;
        const int row = x / RBK;
        voK[m] = row * rsk + 16 * (((x % RBK) >> 4) ^ (row & 7));
    }
#pragma unroll
    for (int m = 0; m < IPGQ; ++m) {
        const int x = m * 1024 + 16 * lane;
        const int row = x / RBQ;
        qrow[m] = row;
        qlp[m] = ((x % RBQ) >> 4) ^ (row & 7);
    }
#pragma unroll
    for (int m = 0; m < IPGV; ++m) {
        const int x = m * 1024 + 16 * lane;
        const int row = x / RBV;
        voV[m] = row * rsv + 16 * (((x % RBV) >> 4) ^ v_swz<RBV>(row));
    }
    // LDS read offsets (K and Q: row lr, piece 4 ks + lg; V: transposing read)
    const int kq = 16 * (lg ^ (lr & 3));
    const int kb2 = 64 * ((lr >> 2) & 1);
    const int koE = lr * RBK + kq + kb2, koO = lr * RBK + kq - kb2;
    const int qoE = lr * RBQ + kq + kb2, qoO = lr * RBQ + kq - kb2;
    constexpr int NVO = v_offsets<RBV>();
    int vo[NVO];
#pragma unroll
    for (int m = 0; m < NVO; ++m) {
        const int vrow = 4 * lg + (lr >> 2);
        vo[m] = vrow * RBV + 16 * ((2 * m + ((lr & 3) >> 1)) ^ v_swz<RBV>(vrow)) + 8 * (lr & 1);
    }

    // ------------------------------------------------------------ the piece
    // Sequence lengths: the plan kernel's arrays, or (SELF) this wave's LDS.
    auto lds_int = [&](const int *a, int b) __attribute__((always_inline)) {
        return __builtin_amdgcn_readfirstlane(a[b]);
    };
    auto seq_kv = [&](int b) __attribute__((always_inline)) {
        if constexpr (SELF)
            return lds_int(s_skv, b);
        else
            return sload(p.ws.kvlen, b);
    };
    auto seq_ql = [&](int b) __attribute__((always_inline)) {
        if constexpr (SELF)
            return (int)__builtin_amdgcn_readfirstlane((int)s_sql[b]);
        else
            return sload(p.ws.qlen, b);
    };
    auto seq_t0 = [&](int b) __attribute__((always_inline)) {
        if constexpr (SELF)
            return lds_int(s_st0, b);
        else
            return sload(p.ws.cu_q, b);
    };
    auto seq_has_items = [&](int b) __attribute__((always_inline)) {
        if constexpr (SELF)   // a sequence has items iff it has query rows
            return seq_ql(b) > 0;
        else
            return sload(p.ws.ipg, b) > 0;
    };

    int ipiece = worker;
    Cursor ic{};
    int iend = 0;
    if (ipiece >= p.partitions)
        return;
    if (wave == 0) {
    bool have = true;
    int dyn = 0;
    if constexpr (SELF) {
        // up to four consecutive sequences per lane: b = spl * lane + i,
        // summed in the lane first and then over the wave (one scan each for
        // query tokens and items, whatever the batch)
        const int cap = seq_cap(p);
        const int spl = (p.batch + 63) >> 6;
        int kvr[4] = {0, 0, 0, 0}, qlr[4] = {0, 0, 0, 0}, ipr[4] = {0, 0, 0, 0}, t0r[4] = {0, 0, 0, 0};
        int wsbr[4] = {0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int b = spl * lane + i;
            if (i < spl && b < p.batch) {
                kvr[i] = p.context_lens[b];
                qlr[i] = p.q_seq_lens ? p.q_seq_lens[b] : 1;
            }
        }
        uint32_t serr = 0;
        int lq = 0, lw = 0;   // the lane's running sums
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int b = spl * lane + i;
            if (i < spl && b < p.batch) {
                serr |= sanitize_seq(p, cap, kvr[i], qlr[i]);
                ipr[i] = seq_items_per_group(p, kvr[i], qlr[i]);
            }
            t0r[i] = lq;
            wsbr[i] = lw;
            lq += qlr[i];
            lw += ipr[i] * p.kv_head_num;
        }
        const int iq = wave_scan(lq, lane), iw = wave_scan(lw, lane);
        const int cq = __builtin_amdgcn_readlane(iq, 63), cw = __builtin_amdgcn_readlane(iw, 63);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int b = spl * lane + i;
            t0r[i] += iq - lq;
            wsbr[i] += iw - lw;
            if (i < spl && b < p.batch) {
                s_skv[b] = kvr[i];
                s_st0[b] = t0r[i];
                s_sql[b] = (uint8_t)qlr[i];
                if constexpr (TAIL)
                    s_wsb[b] = wsbr[i];
            }
        }
        const int W = cw;
        if (p.no_split) {
            // Whole units (short passes): workgroup w runs unit (b, g) =
            // (w / Hkv, w % Hkv) at once, so the pass writes no partials
            // and launches no merge.
            const int b = worker / p.kv_head_num, g = worker - b * p.kv_head_num;
            have = b < p.batch;
            if (have) {
                const int l0 = b / spl, i0 = b - l0 * spl;   // the lane and slot holding b
                auto pick4 = [&](const int(&r)[4]) __attribute__((always_inline)) {
                    return __builtin_amdgcn_readlane(i0 == 0 ? r[0] : (i0 == 1 ? r[1] : (i0 == 2 ? r[2] : r[3])), l0);
                };
                const int ipg = pick4(ipr), kv = pick4(kvr), ql = pick4(qlr);
                have = ipg > 0;
                if (have) {
                    ic.b = b;
                    ic.g = g;
                    ic.qt = 0;
                    ic.c = 0;
                    ic.ntile = seq_tiles(p, ql);
                    ic.nch = unit_chunks(p, kv, ql, 0);
                    ic.item = pick4(wsbr) + g * ipg;
                    iend = ic.item + ipg;
                }
            }
            if (worker == 0) {
#pragma unroll
                for (int d = 1; d < 64; d <<= 1)
                    serr |= __shfl_xor(serr, d);
                if (cq != p.num_q_tokens)
                    serr |= PA_DEVERR_TOKENS;
                if (lane == 0 && serr)
                    set_error(p.ws.err, serr);
            }
        } else {
        const PieceMap ipm = self_piece_map(p, W);
        if (TAIL && lane == 0)
            s_pm = ipm;
        dyn = ipm.m > 0 ? 1 : 0;
        ipiece = static_piece(ipm, worker);
        if (worker == 0) {
            // the header and the error word, as the plan kernel writes them
#pragma unroll
            for (int d = 1; d < 64; d <<= 1)
                serr |= __shfl_xor(serr, d);
            if (cq != p.num_q_tokens)
                serr |= PA_DEVERR_TOKENS;
            if (lane == 0) {
                // (the piece counter, hdr[3], is reset by the merge kernel)
                p.ws.hdr[0] = W;
                p.ws.hdr[1] = ipm.per;
                p.ws.hdr[2] = piece_count(ipm);
                p.ws.hdr[4] = ipm.a;
                p.ws.hdr[5] = ipm.m;
                p.ws.hdr[6] = ipm.P;
                p.ws.hdr[7] = ipm.nr;
                if (serr)
                    set_error(p.ws.err, serr);
            }
        }
        int s0, s1, sp0, sp1;
        piece_range(ipm, ipiece, s0, s1);
        piece_range(ipm, ipiece - 1, sp0, sp1);
        have = s0 < s1;
        // a boundary past the last item cuts nothing
        if (!have && ipiece > 0 && lane == 0)
            p.ws.splits[(size_t)(ipiece - 1) * 8] = -1;
        if (have) {
        // the sequence holding item s0: the last one whose first item is
        // <= s0 (first items grow with b, so a lane's qualifying sequences
        // are a prefix of its own)
        int nle = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            nle += (i < spl && spl * lane + i < p.batch && wsbr[i] <= s0) ? 1 : 0;
        const uint64_t m = __ballot(nle > 0);   // lane 0 always qualifies (b = 0)
        const int l0 = 63 - __builtin_clzll(m);
        const int i0 = __builtin_amdgcn_readlane(nle, l0) - 1;
        const int b0 = spl * l0 + i0;
        auto pick4 = [&](const int(&r)[4]) __attribute__((always_inline)) {
            return __builtin_amdgcn_readlane(i0 == 0 ? r[0] : (i0 == 1 ? r[1] : (i0 == 2 ? r[2] : r[3])), l0);
        };
        ic = piece_start(p, ipiece, s0, sp0, b0, pick4(kvr), pick4(qlr), pick4(ipr), pick4(wsbr), pick4(t0r),
                         lane == 0);
        iend = s1;
        }
        }
    } else {
        have = wg_range(p, ipiece, ic, iend);
    }
    if (lane == 0) {
        s_n = have ? iend - ic.item : 0;
        s_dyn = dyn;
        s_claim[0] = -1;
    }
    }
    // both waves learn the piece's length (0: no work) from wave 0
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    const int n = __builtin_amdgcn_readfirstlane(s_n);
    if (n <= 0)
        return;
    const bool cdyn = TAIL && __builtin_amdgcn_readfirstlane(s_dyn) != 0;
    // the first chunk of the next unit (skipping sequences without rows);
    // the caller has already advanced ic.item past the current unit
    auto next_unit = [&]() __attribute__((always_inline)) {
        ic.c = 0;
        if (++ic.qt >= ic.ntile) {
            ic.qt = 0;
            if (++ic.g >= p.kv_head_num) {
                ic.g = 0;
                do {
                    ++ic.b;
                } while (ic.b < p.batch && !seq_has_items(ic.b));
                if (ic.b >= p.batch)
                    return;
                ic.ntile = seq_tiles(p, seq_ql(ic.b));
            }
        }
        ic.nch = unit_chunks(p, seq_kv(ic.b), seq_ql(ic.b), ic.qt);
    };

    // ------------------------------------------------------------ issue side
    int idone = 0, ifirst = 1;
    int ic1 = 0, icb = 0, invis = 0, inblk = 1, ikv = 0, iql = 0, it0 = 0, irows = 0;
    int icf = 0, ilo = 0;   // first chunk of the unit (from the sequence start), lowest visible token
    const int32_t *ibt = p.block_tables;
    const char *ikg = kg, *ivg = vg;
    auto iseg = [&]() __attribute__((always_inline)) {
        icb = ic.c;
        ic1 = ic.nch < ic.c + (iend - ic.item) ? ic.nch : ic.c + (iend - ic.item);
        ikv = seq_kv(ic.b);
        iql = seq_ql(ic.b);
        it0 = seq_t0(ic.b);
        irows = iql * G - ic.qt * 16;
        irows = irows < 16 ? irows : 16;
        invis = row_hi_t<BAND>(p, ikv, seq_prefix(ikv, iql), (ic.qt * 16 + irows - 1) / G);
        icf = BAND ? unit_first_chunk(p, ikv, iql, ic.qt) : 0;
        ilo = row_lo_t<BAND>(p, seq_prefix(ikv, iql), (ic.qt * 16) / G);
        inblk = invis > 0 ? div_bs(invis - 1, bs, bsh) + 1 : 1;
        ibt = p.block_tables + (size_t)ic.b * p.max_blocks;
        ikg = kg + (size_t)ic.g * RBK;
        ivg = vg + (size_t)ic.g * p.v_head_bytes;
    };
    int ibid[NTT];
    auto ifetch = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < NTT; ++q) {
            const int blk = div_bs((icf + ic.c) * KT + 16 * q, bs, bsh);
            ibid[q] = sload(ibt, blk < inblk ? blk : inblk - 1);
        }
    };
    // SELF: the cursor at the start of piece k and its end, as the computing
    // wave resolved them (see resolve_piece)
    auto goto_piece = [&](int k) __attribute__((always_inline)) {
        if constexpr (TAIL) {
            ic.b = lds_int(s_claim, 1);
            ic.g = lds_int(s_claim, 2);
            ic.qt = lds_int(s_claim, 3);
            ic.c = lds_int(s_claim, 4);
            ic.nch = lds_int(s_claim, 5);
            ic.ntile = lds_int(s_claim, 6);
            ic.item = lds_int(s_claim, 7);
            iend = lds_int(s_claim, 8);
            ipiece = k;
        }
    };
    // SELF (computing wave): the claimed piece k, resolved for the issuing
    // wave -- the sequence holding its first item (the last one whose first
    // item is <= it; lane 0 always qualifies), the cursor there, and the
    // piece's split entry (entry k - 1) -- so that the issuing wave's loop
    // carries none of this arithmetic
    auto resolve_piece = [&](int k) __attribute__((always_inline)) {
        if constexpr (TAIL) {
            const PieceMap pm{lds_int(&s_pm.W, 0), lds_int(&s_pm.per, 0), lds_int(&s_pm.a, 0),
                              lds_int(&s_pm.m, 0), lds_int(&s_pm.P, 0), lds_int(&s_pm.nr, 0)};
            int s0, s1, sp0, sp1;
            piece_range(pm, k, s0, s1);
            piece_range(pm, k - 1, sp0, sp1);
            const int spl = (p.batch + 63) >> 6;
            int nle = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int b = spl * lane + i;
                nle += (i < spl && b < p.batch && s_wsb[b] <= s0) ? 1 : 0;
            }
            const uint64_t m = __ballot(nle > 0);
            const int l0 = 63 - __builtin_clzll(m);
            const int b0 = spl * l0 + __builtin_amdgcn_readlane(nle, l0) - 1;
            const int kv0 = lds_int(s_skv, b0), ql0 = seq_ql(b0);
            const Cursor cu = piece_start(p, k, s0, sp0, b0, kv0, ql0, seq_items_per_group(p, kv0, ql0),
                                          lds_int(s_wsb, b0), lds_int(s_st0, b0), lane == 0);
            if (lane == 0) {
                s_claim[1] = cu.b;
                s_claim[2] = cu.g;
                s_claim[3] = cu.qt;
                s_claim[4] = cu.c;
                s_claim[5] = cu.nch;
                s_claim[6] = cu.ntile;
                s_claim[7] = cu.item;
                s_claim[8] = s1;
            }
        }
    };
    int n_issued = 0;
    // Issue the next chunk of the stream into stage st (nothing once done).
    auto issue = [&](int st) __attribute__((always_inline)) {
        if (idone)
            return;
        if constexpr (TMASK) {
            // the matrix slice of the chunk: rows of the unit's query
            // indices, KT + 2 columns from an even start (extra loads, see
            // the tile kernel)
            const int c0m = (icf + ic.c) * KT - seq_prefix(ikv, iql);
            const int i0 = (ic.qt * 16) / G;
            int i1 = (ic.qt * 16 + irows - 1) / G;
            i1 = i1 < kMaskDim - 1 ? i1 : kMaskDim - 1;
            const int nim = i1 - i0 + 1;
            if (c0m < kMaskDim && c0m + KT > 0 && nim > 0) {
                int cs = c0m & ~1;
                cs = cs < 0 ? 0 : (cs > kMaskDim - 2 * SDW ? kMaskDim - 2 * SDW : cs);
                const int ntot = nim * SDW;
                const int nin = (ntot + 63) / 64;
                for (int m = 0; m < nin; ++m) {
                    const int x = m * 64 + lane;
                    const int r = x / SDW;
                    const char *src = x < ntot ? mg + ((size_t)(i0 + r) * kMaskDim + cs) * 2 + 4 * (x - r * SDW) : mg;
                    lds_load4(src, (lds_u8 *)sMk + st * SLB + m * 256);
                }
            }
        }
        const bool seg_begin = ic.c == icb;
        if (seg_begin) {
            // Q tile of the segment (rows past the unit read the zero page)
#pragma unroll
            for (int m = 0; m < IPGQ; ++m) {
                const int rg = ic.qt * 16 + qrow[m];
                const int t = it0 + rg / G;
                const bool ok = qrow[m] < irows && t < p.num_q_tokens;
                const char *src = ok ? (const char *)(qg + ((size_t)t * H + ic.g * G + rg % G) * DK + 8 * qlp[m])
                                     : zg + 16 * qlp[m];
                lds_load16(src, (lds_u8 *)sQ + st * STQ + m * 1024);
            }
        }
#pragma unroll
        for (int q = 0; q < NTT; ++q) {
            const int j0 = (icf + ic.c) * KT + 16 * q;
            const bool vis = j0 < invis && (!BAND || j0 + 16 > ilo);
            const bool inb = (unsigned)ibid[q] < nb32;
            err |= (vis && !inb) ? (uint32_t)PA_DEVERR_BLOCK_ID : 0u;
            const size_t trow = (size_t)ibid[q] * bs + mod_bs(j0, bs, bsh);
            const char *kbase = (vis && inb) ? ikg + trow * rsk : zg;
            const char *vbase = (vis && inb) ? ivg + trow * rsv : zg;
#pragma unroll
            for (int m = 0; m < IPGK; ++m)
                lds_load16(kbase + voK[m], (lds_u8 *)sK + st * STK + (q * IPGK + m) * 1024);
#pragma unroll
            for (int m = 0; m < IPGV; ++m)
                lds_load16(vbase + voV[m], (lds_u8 *)sV + st * STV + (q * IPGV + m) * 1024);
        }
        const bool seg_end = ic.c + 1 == ic1;
        // the last chunk of the piece: the piece the computing wave claimed
        // to follow it is in LDS by now (-1: none, the stream ends here)
        const bool piece_end = ic.item + 1 == iend;
        int nxt = -1;
        if constexpr (TAIL) {
            if (piece_end && cdyn)
                nxt = __builtin_amdgcn_readfirstlane(*(volatile int *)&s_claim[0]);
        }
        if (lane == 0) {
            int *md = s_meta + st * MW;
            md[0] = ic.b;
            md[1] = ic.g;
            md[2] = ic.qt;
            md[3] = icf + ic.c;
            md[4] = (seg_begin ? 1 : 0) | (seg_end ? 2 : 0) | ((icb == 0 && ic1 == ic.nch) ? 4 : 0) | (ifirst ? 8 : 0);
            md[5] = ipiece;
            md[6] = invis;
            md[7] = ikv;
            md[8] = iql;
            md[9] = it0;
            md[10] = irows;
            md[11] = ilo;
            if constexpr (TAIL)   // chunks of the piece after this one (no claims: many)
                md[12] = cdyn ? iend - ic.item - 1 : 0x7fffffff;
        }
        ++n_issued;
        // advance the issue position by one chunk
        ++ic.c;
        ++ic.item;
        if (ic.c == ic1) {
            ifirst = 0;
            bool more = ic.item < iend;
            if (more) {
                next_unit();
                more = ic.b < p.batch;
            } else if (TAIL && nxt >= 0) {
                goto_piece(nxt);
                ifirst = 1;
                more = true;
            }
            idone = more ? 0 : 1;
            if (!idone)
                iseg();
        }
        if (TAIL && idone && lane == 0)   // the last chunk of the stream: the computing wave stops after it
            s_meta[st * MW + 4] |= 16;
        if (!idone)
            ifetch();
    };

    // ---------------------------------------------------------- compute side
    u32x4 qb[KS];
    f32x4 oacc[ND];
    float m_run = -INFINITY, lsum = 0.f;
    int lim = 0, min_lim = 0, nvis = 0, seg_prefix = 0;
    int lo_r = 0, max_lo = 0, lo_tile = 0;

    if (wave == 0) {
        // the issuing wave: one barrier per chunk of the stream, as the
        // computing wave (the stream's length is known once it has ended)
        iseg();
        ifetch();
#pragma unroll
        for (int k = 0; k < S - 1; ++k)
            issue(k);
        for (int k = 0; k < (TAIL ? n_issued : n); ++k) {
            wait_ahead<LW, S - 2>((TAIL ? n_issued : n) - 1 - k);   // chunk k (and any earlier Q tile) is in LDS
            wait_lgkm0();                       // and its stage record
            __builtin_amdgcn_s_barrier();       // wave 1 has finished chunk k - 1 ...
            issue((k + S - 1) % S);             // ... whose stage this load fills
        }
        if (err)
            set_error(p.ws.err, err);
        return;
    }

    // claim state for the successor of the current piece: 0 (not yet), 1
    // (atomic sent), 2 (answer in LDS)
    int cstate = 0, cval = 0;
    for (int k = 0; TAIL || k < n; ++k) {
        const int st = k % S;
        wait_lgkm0();                  // this wave's reads of chunk k - 1 are done
        __builtin_amdgcn_s_barrier();  // chunk k has landed
        // the record: what every chunk needs (the segment's lengths are
        // read at its first chunk only)
        int md[MW];
#pragma unroll
        for (int i = 0; i < 6; ++i)
            md[i] = __builtin_amdgcn_readfirstlane(s_meta[st * MW + i]);
        const int g = md[1], qt = md[2], c = md[3], fl = md[4];
        if constexpr (TAIL) {
            md[12] = __builtin_amdgcn_readfirstlane(s_meta[st * MW + 12]);
            if ((fl & 9) == 9)   // the first chunk of a piece
                cstate = 0;
            if (cstate == 0 && md[12] <= S + kClaimAhead) {   // (never without claims)
                if (lane == 0)
                    cval = __hip_atomic_fetch_add(p.ws.hdr + 3, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                cstate = 1;
            }
        }
        const lds_u8 *kb = (const lds_u8 *)sK + st * STK;
        const lds_u8 *vb = (const lds_u8 *)sV + st * STV;
        if (fl & 1) {
            // first chunk of a segment: its Q tile and row limits
#pragma unroll
            for (int i = 6; i < 12; ++i)
                md[i] = __builtin_amdgcn_readfirstlane(s_meta[st * MW + i]);
            nvis = md[6];
            const int kv = md[7], ql = md[8], rows = md[10];
            const lds_u8 *qs = (const lds_u8 *)sQ + st * STQ;
            // (head pairs: this lane's row belongs to head hh of the pair;
            // its Q is zero in the other head's slices)
            const int hh = HP > 1 ? ((qt * 16 + lr) % G) / (G / HP) : 0;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int kq_ = ks % KSQ;
                u32x4 q = *(const lds_u32x4 *)(qs + ((kq_ & 1) ? qoO : qoE) + 64 * kq_);
                if (neg_scale)   // exact: softmax(c s) = softmax(|c| (-s)) with -s = (-q) . k
                    q ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
                qb[ks] = (HP == 1 || ks / KSQ == hh) ? q : u32x4{0u, 0u, 0u, 0u};
            }
            lo_tile = md[11];
            const int prefix = seq_prefix(kv, ql);
            seg_prefix = prefix;
            const int rg = qt * 16 + lr;
            lim = row_hi_t<BAND>(p, kv, prefix, rg / G);
            lo_r = row_lo_t<BAND>(p, prefix, rg / G);
            min_lim = row_hi_t<BAND>(p, kv, prefix, (qt * 16) / G);
            max_lo = row_lo_t<BAND>(p, prefix, (qt * 16 + rows - 1) / G);
#pragma unroll
            for (int nd = 0; nd < ND; ++nd)
                oacc[nd] = f32x4{0.f, 0.f, 0.f, 0.f};
            m_run = -INFINITY;
            lsum = 0.f;
        }

        // S^T = K . Q^T
        const int jb = c * KT;
        f32x4 sacc[NTT];
#pragma unroll
        for (int n = 0; n < NTT; ++n)
            sacc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int n = 0; n < NTT; ++n) {
                const u32x4 a = *(const lds_u32x4 *)(kb + ((ks & 1) ? koO : koE) + 16 * n * RBK + 64 * ks);
                sacc[n] = Mfma<DT>::run(a, qb[ks], sacc[n]);
            }
        }
        if constexpr (TMASK) {
            // scaled log2-domain scores plus the matrix; the causal rule
            // outside it
            const int c0m = jb - seg_prefix;
#pragma unroll
            for (int n = 0; n < NTT; ++n)
                sacc[n] *= scq;
            if (c0m + KT > 0) {
                int cs = c0m & ~1;
                cs = cs < 0 ? 0 : (cs > kMaskDim - 2 * SDW ? kMaskDim - 2 * SDW : cs);
                const int i = (qt * 16 + lr) / G;
                const lds_u8 *row = (const lds_u8 *)sMk + st * SLB + (i - (qt * 16) / G) * (4 * SDW);
#pragma unroll
                for (int n = 0; n < NTT; ++n) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int cj = c0m + 16 * n + 4 * lg + r;
                        if ((unsigned)cj < (unsigned)kMaskDim && i < kMaskDim) {
                            const uint16_t hb = *(const __attribute__((address_space(3))) uint16_t *)(row + 2 * (cj - cs));
                            sacc[n][r] = __builtin_fmaf(f16_bits_to_f32(hb), 1.4426950408889634f, sacc[n][r]);
                        } else if (cj > i) {
                            sacc[n][r] = -INFINITY;
                        }
                    }
                }
            }
        }
        // mask, online softmax (raw scores, lazy reference)
        float mx = -INFINITY;
        const bool need_mask = jb + KT > min_lim || (BAND && jb < max_lo);
#pragma unroll
        for (int n = 0; n < NTT; ++n) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (need_mask) {
                    const int j = jb + 16 * n + 4 * lg + r;
                    sacc[n][r] = (j < lim && (!BAND || j >= lo_r)) ? sacc[n][r] : -INFINITY;
                }
                mx = fmaxf(mx, sacc[n][r]);
            }
        }
        mx = xor_max<16>(mx);
        mx = xor_max<32>(mx);
        if (__any(mx > m_run + grow_raw)) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f((m_run - m_new) * sc);
            lsum *= alpha;
            m_run = m_new;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float ar = __shfl(alpha, 4 * lg + r);
#pragma unroll
                for (int nd = 0; nd < ND; ++nd)
                    oacc[nd][r] *= ar;
            }
        }
        const float mref = m_run == -INFINITY ? 0.f : m_run * sc;
        float ps = 0.f;
#pragma unroll
        for (int n = 0; n < NTT; ++n) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[n][r], sc, -mref));
                sacc[n][r] = pv;
                ps += pv;
            }
        }
        lsum += ps;
        // PV (V halves of tokens outside [lo_tile, nvis) zeroed)
        const bool tail = jb + KT > nvis || (BAND && jb < lo_tile);
        auto tok_ok = [&](int t) __attribute__((always_inline)) {
            return BAND ? (unsigned)(t - lo_tile) < (unsigned)(nvis - lo_tile) : t < nvis;
        };
        if constexpr (KT == 16) {
            const uint2 pa = uint2{pack2<DT>(sacc[0][0], sacc[0][1]), pack2<DT>(sacc[0][2], sacc[0][3])};
            uint2 vm = {~0u, ~0u};
            if (tail) {
                const int tb = jb + 4 * lg;
                vm.x = (tok_ok(tb) ? 0xffffu : 0u) | (tok_ok(tb + 1) ? 0xffff0000u : 0u);
                vm.y = (tok_ok(tb + 2) ? 0xffffu : 0u) | (tok_ok(tb + 3) ? 0xffff0000u : 0u);
            }
#pragma unroll
            for (int nd = 0; nd < ND; ++nd) {
                const v4i16 b0 =
                    __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(vb + vo[nd % NVO] + 32 * NVO * (nd / NVO)));
                uint2 bv = __builtin_bit_cast(uint2, b0);
                if (tail) {
                    bv.x &= vm.x;
                    bv.y &= vm.y;
                }
                oacc[nd] = Mfma16<DT>::run(pa, bv, oacc[nd]);
            }
        } else {
            const u32x4 pa = u32x4{pack2<DT>(sacc[0][0], sacc[0][1]), pack2<DT>(sacc[0][2], sacc[0][3]),
                                   pack2<DT>(sacc[1][0], sacc[1][1]), pack2<DT>(sacc[1][2], sacc[1][3])};
            u32x4 vm = {~0u, ~0u, ~0u, ~0u};
            if (tail) {
                const int tb = jb + 4 * lg;
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                    for (int e = 0; e < 2; ++e)
                        vm[2 * h2 + e] = (tok_ok(tb + 16 * h2 + 2 * e) ? 0xffffu : 0u) |
                                         (tok_ok(tb + 16 * h2 + 2 * e + 1) ? 0xffff0000u : 0u);
            }
#pragma unroll
            for (int nd = 0; nd < ND; ++nd) {
                const int off = 32 * NVO * (nd / NVO);
                const v4i16 b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(vb + vo[nd % NVO] + off));
                const v4i16 b1 =
                    __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(vb + vo[nd % NVO] + off + 16 * RBV));
                const uint2 lo = __builtin_bit_cast(uint2, b0), hi = __builtin_bit_cast(uint2, b1);
                u32x4 bv = {lo.x, lo.y, hi.x, hi.y};
                if (tail)
                    bv &= vm;
                oacc[nd] = Mfma<DT>::run(pa, bv, oacc[nd]);
            }
        }

        if (TAIL && cstate == 1 && md[12] <= S) {
            // the deadline: the issuing wave reads the answer after the next
            // barrier, when it issues the piece's last chunk
            const int nx = claimed_piece(PieceMap{0, 0, 0, 1, p.partitions, lds_int(&s_pm.nr, 0)},
                                         __builtin_amdgcn_readlane(cval, 0));
            if (nx >= 0)
                resolve_piece(nx);
            if (lane == 0)
                s_claim[0] = nx;
            cstate = 2;
        }
        if (fl & 2) {
            // last chunk of the segment: output or partial (its first
            // query row and row count are in this chunk's record too)
            const bool whole = fl & 4;
            const int piece = md[5];
            const int t0 = __builtin_amdgcn_readfirstlane(s_meta[st * MW + 9]);
            const int rows = __builtin_amdgcn_readfirstlane(s_meta[st * MW + 10]);
            float *part = p.ws.partials + (size_t)(2 * piece + ((fl & 8) ? 0 : 1)) * p.partial_stride;
            const float L = xor_sum<32>(xor_sum<16>(lsum));
            const float Ms = m_run * sc;   // log2 domain
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float Lr = __shfl(L, 4 * lg + r);
                const float Mr = __shfl(Ms, 4 * lg + r);
                const int row_t = 4 * lg + r;
                if (row_t >= rows)
                    continue;
                const int rg = qt * 16 + row_t;
                const int t = t0 + rg / G;
                const int h = g * G + rg % G;
                // (head pairs: the row's own head's half of the output)
                const int hr = HP > 1 ? (rg % G) / (G / HP) : 0;
                auto out_col = [&](int nd) __attribute__((always_inline)) -> float {
                    if constexpr (HP == 1)
                        return oacc[nd][r];
                    else
                        return hr ? oacc[NDO + nd][r] : oacc[nd][r];
                };
                if (whole) {
                    if (t >= p.num_q_tokens)
                        continue;
                    const float inv = Lr > 0.f ? 1.f / Lr : 0.f;
                    uint16_t *dst = og + ((size_t)t * H + h) * DV;
#pragma unroll
                    for (int nd = 0; nd < NDO; ++nd)
                        dst[16 * nd + lr] = to_bits<DT>(out_col(nd) * inv);
                    if (lr == 0 && p.lse)
                        p.lse[(size_t)t * H + h] = Lr > 0.f ? (Mr + log2f(Lr)) * 0.69314718055994531f : -INFINITY;
                } else {
#pragma unroll
                    for (int nd = 0; nd < NDO; ++nd)
                        part[row_t * DV + 16 * nd + lr] = out_col(nd);
                    if (lr == 0) {
                        part[16 * DV + row_t] = Mr;
                        part[16 * DV + 16 + row_t] = Lr;
                    }
                }
            }
        }
        if (TAIL && (fl & 16))   // the last chunk of the stream
            break;
    }
    if (err)
        set_error(p.ws.err, err);
}

// Variants per (Dk, Dv).  0: units of at most 16 rows (decode), memory-bound:
// the streaming kernel (one wave, 16-token chunks, four stages).  1: up to
// 64 rows.  2: more rows, two 16-row blocks per wave.  Dk = 576 has variant
// 0 only: 4 waves of 16 rows each own all 512 output columns (no duplicated
// K . Q^T work): 16-token chunks in three stages (104 KB of LDS, one
// workgroup per CU; two stages with the tensor mask), or with a shared K/V
// cache, where only K tiles are staged, 32-token chunks in two stages
// (74 KB, two workgroups per CU).

template <int DT, int DK, int DV, int MB, int KT, int NW, int CS, int S, bool SH, int MODE, bool SELF = false>
const void *pick(TileShape *t)
{
    *t = TileShape{MB, KT, NW, CS, S, 64 * NW};
    return (const void *)&tile_kernel<DT, DK, DV, MB, KT, NW, CS, S, SH, MODE, SELF>;
}

// The tensor mask takes 32-token chunks in variants 1 and 2 (LDS room for
// the matrix slices); variant 2 (128-row tiles) at head sizes up to 128.
template <int DT, int DK, int DV, int MODE>
const void *kernel_for(int variant, bool shared, TileShape *t)
{
    if constexpr (DK > 256) {
        // variant 8: variant 0 planning for itself (not with the tensor mask)
        if (variant == 8) {
            if constexpr (MODE != MODE_TENSOR) {
                if (shared) {
                    if constexpr (MODE == MODE_SPARSE)
                        return pick<DT, DK, DV, 1, 16, 4, 1, 2, true, MODE, true>(t);
                    else
                        return pick<DT, DK, DV, 1, 32, 4, 1, 2, true, MODE, true>(t);
                }
                return pick<DT, DK, DV, 1, 16, 4, 1, 3, false, MODE, true>(t);
            }
            return nullptr;
        }
        if (variant != 0)
            return nullptr;
        if (shared) {
            if constexpr (MODE == MODE_TENSOR || MODE == MODE_SPARSE)
                return pick<DT, DK, DV, 1, 16, 4, 1, 2, true, MODE>(t);
            else
                return pick<DT, DK, DV, 1, 32, 4, 1, 2, true, MODE>(t);
        }
        // separate K and V tiles: three stages in one workgroup per CU (two
        // chunks of 34 KB in flight; the mask slabs of the tensor mask leave
        // room for two)
        if constexpr (MODE == MODE_TENSOR)
            return pick<DT, DK, DV, 1, 16, 4, 1, 2, false, MODE>(t);
        else
            return pick<DT, DK, DV, 1, 16, 4, 1, 3, false, MODE>(t);
    } else {
        constexpr int KT = DK <= 128 ? 64 : 32;
        if constexpr (MODE == MODE_SPARSE) {
            // 64-row tiles of 16-entry chunks only (no streaming kernel)
            if (variant == 1)
                return pick<DT, DK, DV, 1, 16, 4, 1, 2, false, MODE>(t);
        } else {
            if (variant == 0) {   // one wave per workgroup, streaming across units
                *t = TileShape{1, 16, 1, 1, 4, 128};
                return (const void *)&stream_kernel<DT, DK, DV, 16, 4, MODE, false, false, 1>;
            }
            if (variant == 3) {   // the same, planning for itself
                *t = TileShape{1, 16, 1, 1, 4, 128};
                return (const void *)&stream_kernel<DT, DK, DV, 16, 4, MODE, true, false, 1>;
            }
            if (variant == 4) {   // the same, with a claimed tail of pieces
                *t = TileShape{1, 16, 1, 1, 4, 128};
                return (const void *)&stream_kernel<DT, DK, DV, 16, 4, MODE, true, true, 1>;
            }
            if constexpr (DK == 128 && DV == 128) {
                // 5, 6, 7: variants 0, 3, 4 on head pairs (three stages:
                // two workgroups per CU)
                if (variant == 5) {
                    *t = TileShape{1, 16, 1, 1, 3, 128};
                    return (const void *)&stream_kernel<DT, DK, DV, 16, 3, MODE, false, false, 2>;
                }
                if (variant == 6) {
                    *t = TileShape{1, 16, 1, 1, 3, 128};
                    return (const void *)&stream_kernel<DT, DK, DV, 16, 3, MODE, true, false, 2>;
                }
                if (variant == 7) {
                    *t = TileShape{1, 16, 1, 1, 3, 128};
                    return (const void *)&stream_kernel<DT, DK, DV, 16, 3, MODE, true, true, 2>;
                }
            }
            if constexpr (MODE == MODE_TENSOR) {
                // 32-token chunks: the mask slabs of two stages fit beside
                // the K/V tiles of two workgroups per CU
                if (variant == 1)
                    return pick<DT, DK, DV, 1, 32, 4, 1, 2, false, MODE>(t);
                if constexpr (DK <= 128 && DV <= 128) {
                    if (variant == 2)
                        return pick<DT, DK, DV, 2, 32, 4, 1, 2, false, MODE>(t);
                }
            } else {
                if (variant == 1)
                    return pick<DT, DK, DV, 1, KT, 4, 1, 2, false, MODE>(t);
                if (variant == 2)
                    return pick<DT, DK, DV, 2, KT, 4, 1, 2, false, MODE>(t);
            }
        }
        return nullptr;
    }
}

template <int DT, int MODE>
const void *kernel_dt(int dk, int dv, int variant, bool shared, TileShape *t)
{
    if (dk == 64 && dv == 64)
        return kernel_for<DT, 64, 64, MODE>(variant, shared, t);
    if (dk == 128 && dv == 128)
        return kernel_for<DT, 128, 128, MODE>(variant, shared, t);
    if (dk == 256 && dv == 256)
        return kernel_for<DT, 256, 256, MODE>(variant, shared, t);
    if (dk == 576 && dv == 512)
        return kernel_for<DT, 576, 512, MODE>(variant, shared, t);
    return nullptr;
}

// The kernel (and its shape) for a configuration, from this translation
// unit's instantiations.
template <int MODE>
const void *kernel_select(int dtype, int dk, int dv, int variant, bool shared, TileShape *t)
{
    return dtype == 0 ? kernel_dt<0, MODE>(dk, dv, variant, shared, t) : kernel_dt<1, MODE>(dk, dv, variant, shared, t);
}

}  // namespace

}  // namespace pa

#endif  // PA_TILE_KERNELS_H_

// pa_internal.h -- launch parameters, workspace layout and shared device code
// of the paged-attention library (gfx950).  Internal: not part of the C ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

// Work decomposition (shared by the plan, attention and merge kernels).
//
//  unit  = (sequence b, KV head g, row tile qt).  A row is one (query token i,
//          query head h of group g); the rows of (b, g) are ordered i-major,
//          r = i * G + (h - g * G), and cut into tiles of R rows.
//  item  = (unit, chunk c): the KV tokens [c * CT, (c + 1) * CT) of the unit,
//          CT tokens per chunk.  A unit has nch = max(1, ceil(nvis / CT))
//          items, nvis being the KV tokens its rows can see.
//  Items are numbered b-major, then g, then qt, then c.  In balanced mode the
//  items are cut into N pieces of `per` consecutive items; the grid of P
//  persistent workers (workgroups of the MFMA kernel, waves of the VALU
//  kernel) takes piece w first, then further pieces from a shared counter
//  (pieces P, P + 1, ...) until none is left, so the workers finish
//  together even when they stream at different rates.  The pieces are
//  either all alike, or (the self-planning streaming kernel, PieceMap) P
//  static pieces holding about nine tenths of the items followed by rounds
//  of smaller pieces that workers claim as they run out.  In no-split mode
//  (per = 0) every workgroup is one unit.  A unit whose items lie in more
//  than one piece is split: each of its pieces leaves an fp32 partial
//  (acc, m, l) in its slot (2k if the unit is the first of piece k, 2k + 1
//  if it is the last), and the merge kernel combines them.

struct Workspace {
    int32_t *hdr;        // [8]: W (total items), per, N (pieces), next piece counter, and
                         //      the rest of the PieceMap: a, m, P, nr
    int32_t *cu_q;       // [max_batch + 1]: first packed query row of each sequence
    int32_t *wsb;        // [max_batch + 1]: first item of each sequence
    int32_t *ipg;        // [max_batch]: items of each (b, g) (equal for all g of b)
    int32_t *qlen;       // [max_batch]: sanitised q_seq_lens
    int32_t *kvlen;      // [max_batch]: sanitised context_lens
    int32_t *wg_b;       // [N]: sequence holding the first item of each piece
    int32_t *splits;     // [N][8]: split units (b, g, qt, first item, end item, first query row, rows; b < 0: none)
    float *partials;     // [2 * N][R * (DV + 2)]
    const void *zeros;   // 16 token rows of zeros (K or V), read in place of a bad block
    uint32_t *err;       // device error word
    int32_t *tq;         // whole-tile task queues (Params::tile_order): kTqHeader ints, then
                         // 2 ints per task (b, g << 16 | qt), max_batch * Hkv * max_tiles tasks
};

// Whether the tile kernel instance for head size dk runs whole-tile tasks
// (Params::tile_order): all but the 576/512 instances that read V out of the
// K tile (one K/V cache), which sit at the register limit and run pieces
// only.
__host__ __device__ constexpr bool tile_whole_tasks(int dk, bool shared)
{
    return !(shared && dk > 256);
}

// Whole-tile task queues, one per XCD (see plan_kernel): the header holds the
// length and first task of each XCD's queue, the mode, then each queue's
// claim counter in a 128-byte line of its own.
constexpr int kXcds = 8;
constexpr int kTqLength = 8, kTqStart = 16, kTqMode = 24;
constexpr int kTqCounter = 32, kTqCounterStride = 32;
constexpr int kTqHeader = kTqCounter + kXcds * kTqCounterStride;
// Largest batch the planner builds the queues for (it ranks the sequences
// by their work with one comparison per pair).
constexpr int kTileOrderMaxBatch = 512;

struct Params {
    const void *query;
    const void *key_cache;
    const void *value_cache;
    const int32_t *block_tables;
    const int32_t *context_lens;
    const int32_t *q_seq_lens;   // may be null: one query token per sequence
    void *out;
    float *lse;                  // may be null
    int64_t num_blocks;
    int32_t batch, num_q_tokens, head_num, kv_head_num, group;
    int32_t head_size_k, head_size_v;
    int32_t block_size, bs_shift;      // bs_shift = log2(block_size) or -1
    int32_t max_blocks;                // block_tables row length
    int32_t max_q;                     // bound on q_seq_lens for this call
    int32_t causal;                    // row-dependent upper limit (causal or band mask)
    int32_t band;                      // band mask: row-dependent lower limit as well
    int32_t win_left, win_right;       // band mask window (0, 0 otherwise)
    int32_t tmask;                     // tensor mask: the shared matrix is added to the scores
    const uint16_t *mask_tensor;       // fp16 [2048, 2048] (tensor mask only)
    int32_t sparse;                    // sparse lists: a unit's tokens are its query token's list entries
    int32_t topk;                      // entries per list
    const int32_t *topk_idx;           // [num_q_tokens, kv_head_num, topk] (sparse only)
    float scale_log2;                  // scale * log2(e)
    int32_t rows_per_tile;             // R
    int32_t chunk;                     // CT
    // log2 of CT, of the group and of R where they are powers of 2, else -1
    int32_t chunk_shift, group_shift, tile_shift;
    int32_t partitions;                // P: workers in the grid (no-split mode: units)
    int32_t pieces;                    // N: pieces of the item range (balanced mode)
    int32_t no_split;
    int32_t max_tiles;                 // ceil(max_q * G / R)
    int32_t partial_stride;            // floats per partial slot = R * (DV + 2)
    // V source: value_cache, or (shared K/V) the key cache itself, whose
    // rows hold V as their leading Dv elements
    int32_t shared_kv;
    uint32_t v_row_bytes;              // bytes from one token row of the V source to the next
    uint32_t v_head_bytes;             // bytes from one KV head to the next within a token row
    // The streaming kernel plans for itself (no plan kernel): every wave
    // reads the lengths and cuts the pieces as the plan kernel would, and
    // writes the header and the split entry of its own piece.
    int32_t self_plan;
    // Self-planning launches: smallest piece of the claimed tail in items
    // (0: one piece per worker, no tail).
    int32_t tail_min;
    // The planner may run the pass as whole row tiles from per-XCD task
    // queues instead of pieces (tile kernel, ws.tq sized for the pass).
    int32_t tile_order;
    Workspace ws;
};

// Largest batch a self-planning launch takes (four sequences per lane).
constexpr int kSelfPlanMaxBatch = 256;

// Claimed pieces per worker share, at most: a launch with a claimed tail
// has at most (1 + kTailRounds) * workers pieces.
constexpr int kTailRounds = 8;
// Smallest claimed piece of the streaming kernel, in chunks: a worker claims
// its next piece when S + 4 chunks of the current one are left (S, the ring
// depth, is at most 4), and the answer must be in LDS before its issuing side
// needs it; and every piece beyond the first of a unit costs a partial write
// and its merge.  (16 chunks took 4-6 us longer per pass on the long skewed
// decode with head pairs: more small pieces in the merge.)
constexpr int kTailMinChunks = 8;
// Shares of fewer chunks per worker keep one piece each: balancing short
// streams gains less than the merge work the extra pieces cost.
constexpr int kTailMinShare = 40;   // in units of the tail minimum (320 chunks)

// Launches kernel k.  With events (timed passes) the start and stop events
// take the kernel's own start and end timestamps (hipExtLaunchKernel): no
// marker packets between the kernels of a pass, which slowed the
// compute-bound kernels by 3-5 % when markers were recorded around them.
inline hipError_t launch_kernel(const void *k, dim3 grid, dim3 block, void **args, hipStream_t s, hipEvent_t e0,
                                hipEvent_t e1)
{
    if (e0 || e1)
        return hipExtLaunchKernel(k, grid, block, args, 0, s, e0, e1, 0);
    return hipLaunchKernel(k, grid, block, args, 0, s);
}

// Launchers (defined in the .hip files); e0, e1: optional timing events.
hipError_t launch_plan(const Params &p, hipStream_t s, hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr);
// *launched (if given): whether a kernel was enqueued (passes without split
// entries have nothing to merge)
hipError_t launch_merge(const Params &p, int dtype, hipStream_t s, hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr,
                        bool *launched = nullptr);
// Returns hipErrorInvalidValue when no kernel exists for the shape.
hipError_t launch_decode(const Params &p, int dtype, int rows_pad, hipStream_t s, hipEvent_t e0 = nullptr,
                         hipEvent_t e1 = nullptr);
hipError_t launch_tile(const Params &p, int dtype, int variant, hipStream_t s, hipEvent_t e0 = nullptr,
                       hipEvent_t e1 = nullptr);
// Allocation-free passes (pa_forward_noalloc).  validate_config applies
// pa_create's checks.  forward_in_buffer runs one pass of pa_forward for cfg
// without a handle: it lays the pass's workspace out in `base` (device
// memory of `capacity` bytes), clears the words that must start at zero with
// launch_zero_words on the stream, and enqueues the pass; PA_ERR_SCRATCH when
// the pass needs more than `capacity` bytes.  Nothing is allocated.
pa_status validate_config(const pa_config *cfg);
pa_status forward_in_buffer(const pa_config *cfg, int num_cus, void *base, size_t capacity, const void *query,
                            const void *key_cache, const void *value_cache, const int32_t *block_tables,
                            const int32_t *context_lens, const int32_t *q_seq_lens, int32_t batch,
                            int32_t num_q_tokens, int32_t max_q_seq_len, void *out, float *lse, void *stream);
hipError_t launch_zero_words(uint32_t *p, long long n, hipStream_t s);
// Measurement: a plain streaming read of `bytes` (a multiple of 16) by `workgroups`
// workgroups, one word per workgroup written to sink.
hipError_t launch_read_probe(const void *src, long long bytes, uint32_t *sink, int workgroups, hipStream_t s);
// Shapes and occupancy used by the host to pick kernels and size the grid.
bool decode_supported(int dk, int dv);
// MFMA tile kernel variants: 0 for units of at most 16 rows, 1 for up to
// tile_rows(.., 1) rows, 2 above, 3 as 0 but planning for itself
// (Params::self_plan); tile_supported says which exist.
// `shared` selects the kernels that read V out of the K tile already in LDS
// (shared K/V cache) where such kernels exist; `mode` the kernels of a mask
// kind with code of its own (0 none / causal, 1 band, 2 tensor, 3 sparse).
bool tile_supported(int dk, int dv, int variant);
int tile_workers_per_cu(int dtype, int dk, int dv, int variant, bool shared, int mode);   // resident workgroups per CU
int tile_chunk(int dk, int dv, int variant, bool shared, int mode);
int tile_rows(int dk, int dv, int variant, bool shared, int mode);
bool tile_streaming(int dk, int dv, int variant);   // served by the one-wave streaming kernel
int decode_chunk(int dk, int rows_pad);
int decode_workers_per_cu(int dtype, int dk, int dv, int rows_pad);   // resident waves per CU

// Shape of a matrix-core kernel instance.
struct TileShape {
    int mb, kt, nw, cs, s;   // 16-row blocks per wave, tokens per chunk, waves owning rows,
                             // waves sharing a row group, LDS stages
    int threads;             // workgroup size
};
// Kernel instances without / with the band mask (nullptr: none for the shape).
const void *tile_kernel_plain(int dtype, int dk, int dv, int variant, bool shared, TileShape *t);
const void *tile_kernel_band(int dtype, int dk, int dv, int variant, bool shared, TileShape *t);
const void *tile_kernel_tensor(int dtype, int dk, int dv, int variant, bool shared, TileShape *t);
const void *tile_kernel_sparse(int dtype, int dk, int dv, int variant, bool shared, TileShape *t);

constexpr int kThreads = 256;        // threads per attention workgroup
constexpr int kBtWindow = 256;       // block-table entries staged in LDS at a time

#ifdef __HIPCC__
// ------------------------------------------------------------ device side

// 128-bit register data as a native vector (HIP's uint4 is a struct, and a
// select between two structs is lowered through memory).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Visible KV tokens of query row i (0-based in its sequence; the row sits at
// position prefix + i, prefix = max(0, kv - qlen)): j in [row_lo, row_hi).
// No mask: [0, kv); causal: j <= prefix + i; band: prefix + i - win_left <=
// j <= prefix + i + win_right (win_right = 0 in causal mode).
__host__ __device__ __forceinline__ int row_hi(const Params &p, int kv, int prefix, int i)
{
    if (!p.causal)
        return kv;
    const int lim = prefix + i + 1 + p.win_right;
    return lim < kv ? lim : kv;
}

__host__ __device__ __forceinline__ int row_lo(const Params &p, int prefix, int i)
{
    if (!p.band)
        return 0;
    const int lo = prefix + i - p.win_left;
    return lo > 0 ? lo : 0;
}

// The same with the mask kind fixed at compile time (BAND false: no lower
// bound, and the upper one of the causal mask).
template <bool BAND>
__host__ __device__ __forceinline__ int row_hi_t(const Params &p, int kv, int prefix, int i)
{
    if (!p.causal)
        return kv;
    const int lim = prefix + i + 1 + (BAND ? p.win_right : 0);
    return lim < kv ? lim : kv;
}

template <bool BAND>
__host__ __device__ __forceinline__ int row_lo_t(const Params &p, int prefix, int i)
{
    if constexpr (!BAND)
        return 0;
    const int lo = prefix + i - p.win_left;
    return lo > 0 ? lo : 0;
}

__host__ __device__ __forceinline__ int seq_prefix(int kv, int qlen)
{
    return kv - qlen > 0 ? kv - qlen : 0;
}

// Tokens up to which some row of rows [.., r1] of (b, g) looks (exclusive):
// the limit of row r1, the largest.
// Quotients the planner takes many times per piece, as shifts where the
// divisor is a power of 2 (x >= 0 there; the divisions otherwise).
__host__ __device__ __forceinline__ int div_group(const Params &p, int x)
{
    return (p.group_shift >= 0 && x >= 0) ? x >> p.group_shift : x / p.group;
}

__host__ __device__ __forceinline__ int div_chunk(const Params &p, int x)
{
    return (p.chunk_shift >= 0 && x >= 0) ? x >> p.chunk_shift : x / p.chunk;
}

__host__ __device__ __forceinline__ int tile_nvis(const Params &p, int kv, int qlen, int r1)
{
    return row_hi(p, kv, seq_prefix(kv, qlen), div_group(p, r1));
}

// The row tile qt of (b, g) covers chunks [first, first + count) of its
// sequence: from the chunk holding the lowest visible token of its first
// row (0 unless banded) to the one holding the last token its last row sees.
__host__ __device__ __forceinline__ int unit_first_chunk(const Params &p, int kv, int qlen, int qt)
{
    return div_chunk(p, row_lo(p, seq_prefix(kv, qlen), div_group(p, qt * p.rows_per_tile)));
}

__host__ __device__ __forceinline__ int unit_chunks(const Params &p, int kv, int qlen, int qt)
{
    if (p.sparse)   // the entries of the query token's list
        return div_chunk(p, p.topk + p.chunk - 1);
    const int rows = qlen * p.group;
    int r1 = (qt + 1) * p.rows_per_tile;
    r1 = (r1 < rows ? r1 : rows) - 1;
    const int n = tile_nvis(p, kv, qlen, r1);
    const int c = div_chunk(p, n + p.chunk - 1) - unit_first_chunk(p, kv, qlen, qt);
    return c > 1 ? c : 1;
}

__device__ __forceinline__ void set_error(uint32_t *err, uint32_t bit)
{
    atomicOr(err, bit);
}

// fp32 -> fp16 / bf16 bit patterns, round to nearest even.
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f)
{
    _Float16 h = (_Float16)f;
    return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f)
{
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x40u);   // quiet NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

template <int DT>
__device__ __forceinline__ uint16_t to_bits(float f)
{
    if constexpr (DT == 0)
        return f32_to_f16_bits(f);
    else
        return f32_to_bf16_bits(f);
}

// Low / high 16-bit element of a packed pair, widened to fp32.
template <int DT>
__device__ __forceinline__ float lo_f32(uint32_t w)
{
    if constexpr (DT == 0)
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
    else
        return __builtin_bit_cast(float, w << 16);
}

template <int DT>
__device__ __forceinline__ float hi_f32(uint32_t w)
{
    if constexpr (DT == 0)
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
    else
        return __builtin_bit_cast(float, w & 0xffff0000u);
}

__host__ __device__ __forceinline__ int div_bs(int j, int bs, int shift)
{
    return shift >= 0 ? (j >> shift) : (j / bs);
}

__host__ __device__ __forceinline__ int mod_bs(int j, int bs, int shift)
{
    return shift >= 0 ? (j & (bs - 1)) : (j % bs);
}

// Addressing of the VALU decode kernel, shared with a host check of its
// bounds.  Row r of unit (b, g) is query head g * G + r % G of packed token
// t = t0 + r / G; head_row is its row index in the [T, H] query, output and
// lse layouts.
__host__ __device__ __forceinline__ size_t head_row(const Params &p, int t, int g, int r)
{
    return (size_t)t * p.head_num + (size_t)g * p.group + (size_t)(r % p.group);
}

// Block-table column read for token j, clamped to the nblk blocks the unit's
// rows see (always a valid column, whatever j).
__host__ __device__ __forceinline__ int bt_column(int j, int bs, int bsh, int nblk)
{
    const int blk = div_bs(j, bs, bsh);
    return blk < nblk ? blk : nblk - 1;
}

// Element offset of token j's row of the KV head at head_off in a
// [num_blocks, bs, Hkv, D] cache (row_stride = Hkv * D); 0 (block 0, slot 0)
// for a token that is not loaded (not visible, or a bad block id).
__host__ __device__ __forceinline__ size_t kv_row_elem(bool ok, int bid, int j, int bs, int bsh, size_t row_stride,
                                                       size_t head_off)
{
    return ok ? ((size_t)bid * bs + mod_bs(j, bs, bsh)) * row_stride + head_off : 0;
}

// Output column of accumulator element e (< 16) of a lane whose two 8-element
// pieces start at d0 and d1.
__host__ __device__ __forceinline__ int lane_col(int e, int d0, int d1)
{
    return e < 8 ? d0 + e : d1 + e - 8;
}

// Cross-lane moves.  pair_swap<D>: the value of the partner lane in the
// other half of this lane's aligned group of 2D lanes.  For D < 16 the
// partner is the mirror image (DPP row_mirror / row_half_mirror / quad_perm),
// for D >= 16 it is lane ^ D.
template <int D>
__device__ __forceinline__ float pair_swap(float v)
{
    const int x = __builtin_bit_cast(int, v);
    int r;
    if constexpr (D == 8)
        r = __builtin_amdgcn_mov_dpp(x, 0x140, 0xf, 0xf, false);   // row_mirror
    else if constexpr (D == 4)
        r = __builtin_amdgcn_mov_dpp(x, 0x141, 0xf, 0xf, false);   // row_half_mirror
    else if constexpr (D == 2)
        r = __builtin_amdgcn_mov_dpp(x, 0x4e, 0xf, 0xf, false);    // quad_perm 2,3,0,1
    else if constexpr (D == 1)
        r = __builtin_amdgcn_mov_dpp(x, 0xb1, 0xf, 0xf, false);    // quad_perm 1,0,3,2
    else
        r = __shfl_xor(x, D);
    return __builtin_bit_cast(float, r);
}

// For D = 16 or 32: {this lane's v, lane (l ^ D)'s v}, in an order that
// depends on the lane (gfx950 v_permlane16_swap / v_permlane32_swap, no LDS
// round trip).  Enough for symmetric combinations such as max and sum.
template <int D>
__device__ __forceinline__ float xor_max(float v)
{
    const unsigned x = __builtin_bit_cast(unsigned, v);
    unsigned a, b;
    if constexpr (D == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
        a = r[0];
        b = r[1];
    } else {
        static_assert(D == 32, "D");
        const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        a = r[0];
        b = r[1];
    }
    return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}

template <int D>
__device__ __forceinline__ float xor_sum(float v)
{
    const unsigned x = __builtin_bit_cast(unsigned, v);
    unsigned a, b;
    if constexpr (D == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
        a = r[0];
        b = r[1];
    } else {
        static_assert(D == 32, "D");
        const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        a = r[0];
        b = r[1];
    }
    return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

// Transposing reduction.  On entry every lane of an aligned group of W lanes
// holds NV partial sums v[0..NV) of the same NV quantities.  On exit lane l
// holds complete sums: if NV >= W, v[0..NV/W) are quantities
// (NV/W) * (l % W) + k; otherwise v[0] is quantity (l % W) / (W / NV).
template <int NV, int W, int N>
__device__ __forceinline__ void treduce(float (&v)[N], int lane)
{
    if constexpr (W > 1) {
        constexpr int D = W / 2;
        const bool upper = (lane & D) != 0;
        if constexpr (NV >= 2) {
#pragma unroll
            for (int k = 0; k < NV / 2; ++k) {
                const float keep = upper ? v[k + NV / 2] : v[k];
                const float send = upper ? v[k] : v[k + NV / 2];
                v[k] = keep + pair_swap<D>(send);
            }
            treduce<NV / 2, D>(v, lane);
        } else {
            v[0] += pair_swap<D>(v[0]);
            treduce<1, D>(v, lane);
        }
    }
}

// Max over an aligned group of W lanes (every lane gets the result).
template <int W>
__device__ __forceinline__ float group_max(float v)
{
    if constexpr (W >= 64)
        v = fmaxf(v, pair_swap<32>(v));
    if constexpr (W >= 32)
        v = fmaxf(v, pair_swap<16>(v));
    if constexpr (W >= 16)
        v = fmaxf(v, pair_swap<8>(v));
    if constexpr (W >= 8)
        v = fmaxf(v, pair_swap<4>(v));
    if constexpr (W >= 4)
        v = fmaxf(v, pair_swap<2>(v));
    if constexpr (W >= 2)
        v = fmaxf(v, pair_swap<1>(v));
    return v;
}

template <int W>
__device__ __forceinline__ float group_sum(float v)
{
    if constexpr (W >= 64)
        v += pair_swap<32>(v);
    if constexpr (W >= 32)
        v += pair_swap<16>(v);
    if constexpr (W >= 16)
        v += pair_swap<8>(v);
    if constexpr (W >= 8)
        v += pair_swap<4>(v);
    if constexpr (W >= 4)
        v += pair_swap<2>(v);
    if constexpr (W >= 2)
        v += pair_swap<1>(v);
    return v;
}

// Workgroup index with consecutive logical indices on the same XCD: the
// dispatcher deals workgroups round-robin over the 8 XCDs.
__host__ __device__ __forceinline__ int xcd_logical_index(int bid, int nwg)
{
    if (nwg % 8 != 0)
        return bid;
    return (bid % 8) * (nwg / 8) + bid / 8;
}

// The cursor a workgroup walks its item range with.
// Loads of plan data and block tables at wave-uniform addresses, as scalar
// loads: the data is read-only for the whole launch (address space 4), and
// scalar loads do not share the vector memory counter with KV loads in
// flight, so waiting for them never waits for those.
typedef __attribute__((address_space(4))) const int32_t c_i32;

__host__ __device__ __forceinline__ int sload(const int32_t *ptr, size_t i)
{
#if defined(__HIP_DEVICE_COMPILE__)
    const uint64_t a = (uint64_t)(uintptr_t)(ptr + i);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return *(const c_i32 *)(uintptr_t)(((uint64_t)hi << 32) | lo);
#else
    return ptr[i];   // host builds of the planning code (bounds checks)
#endif
}

struct Cursor {
    int b, g, qt, c;     // current unit and chunk
    int nch;             // chunks of the current unit
    int ntile;           // row tiles of sequence b
    int item;            // global index of (unit, c)
};

__host__ __device__ __forceinline__ int seq_tiles(const Params &p, int qlen)
{
    const int x = qlen * p.group + p.rows_per_tile - 1;
    return (p.tile_shift >= 0 && x >= 0) ? x >> p.tile_shift : x / p.rows_per_tile;
}

// Position the cursor at item `item`, which lies in sequence b.
__host__ __device__ __forceinline__ void cursor_seek(const Params &p, Cursor &cu, int b, int item)
{
    const int kv = sload(p.ws.kvlen, b);
    const int ql = sload(p.ws.qlen, b);
    const int ipg = sload(p.ws.ipg, b);
    int local = item - sload(p.ws.wsb, b);
    cu.b = b;
    cu.g = local / ipg;
    local -= cu.g * ipg;
    cu.ntile = seq_tiles(p, ql);
    int qt = 0;
    int n = unit_chunks(p, kv, ql, 0);
    while (local >= n) {
        local -= n;
        ++qt;
        n = unit_chunks(p, kv, ql, qt);
    }
    cu.qt = qt;
    cu.c = local;
    cu.nch = n;
    cu.item = item;
}

// Move to the first chunk of the next unit (skipping sequences without
// rows); the caller has already advanced cu.item past the current unit.
__host__ __device__ __forceinline__ void cursor_next_unit(const Params &p, Cursor &cu)
{
    cu.c = 0;
    if (++cu.qt >= cu.ntile) {
        cu.qt = 0;
        if (++cu.g >= p.kv_head_num) {
            cu.g = 0;
            do {
                ++cu.b;
            } while (cu.b < p.batch && sload(p.ws.ipg, cu.b) == 0);
            if (cu.b >= p.batch)
                return;
            cu.ntile = seq_tiles(p, sload(p.ws.qlen, cu.b));
        }
    }
    cu.nch = unit_chunks(p, sload(p.ws.kvlen, cu.b), sload(p.ws.qlen, cu.b), cu.qt);
}

// The item range of piece w (balanced mode) or of the unit of workgroup w
// (no-split mode); returns false if it has none.
__host__ __device__ __forceinline__ bool wg_range(const Params &p, int w, Cursor &cu, int &end)
{
    const int W = sload(p.ws.hdr, 0);
    const int per = sload(p.ws.hdr, 1);
    if (per > 0) {
        const int s = w * per;
        if (w >= p.pieces || s >= W)
            return false;
        end = s + per < W ? s + per : W;
        cursor_seek(p, cu, sload(p.ws.wg_b, w), s);
        return true;
    }
    // no-split: workgroup w is unit (b, g, qt) with qt < max_tiles
    const int per_b = p.kv_head_num * p.max_tiles;
    const int b = w / per_b;
    if (b >= p.batch)
        return false;
    const int g = (w % per_b) / p.max_tiles;
    const int qt = w % p.max_tiles;
    const int ql = sload(p.ws.qlen, b);
    if (qt >= seq_tiles(p, ql))
        return false;
    const int kv = sload(p.ws.kvlen, b);
    int start = sload(p.ws.wsb, b) + g * sload(p.ws.ipg, b);
    for (int t = 0; t < qt; ++t)
        start += unit_chunks(p, kv, ql, t);
    cu.b = b;
    cu.g = g;
    cu.qt = qt;
    cu.c = 0;
    cu.ntile = seq_tiles(p, ql);
    cu.nch = unit_chunks(p, kv, ql, qt);
    cu.item = start;
    end = start + cu.nch;
    return true;
}

// ------------------------------------------------------------ planning
// The planner's reading of the lengths and its cut into pieces, shared by the
// plan kernel and the self-planning streaming kernel so both cut alike.

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_scan(int v, int lane)
{
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int t = __shfl_up(v, d);
        v += lane >= d ? t : 0;
    }
    return v;
}

// Longest context the block table can address.
__host__ __device__ __forceinline__ int seq_cap(const Params &p)
{
    const int64_t cap64 = (int64_t)p.max_blocks * p.block_size;
    return cap64 > 0x7fffffff ? 0x7fffffff : (int)cap64;
}

// Clamps one sequence's lengths into range; returns the error bits of what
// was out of range.
__host__ __device__ __forceinline__ uint32_t sanitize_seq(const Params &p, int cap, int &kv, int &ql)
{
    uint32_t err = 0;
    if (kv < 0) {
        err |= PA_DEVERR_CTX;
        kv = 0;
    }
    if (kv > cap) {
        err |= PA_DEVERR_TABLE_SHORT;
        kv = cap;
    }
    if (ql < 0) {
        err |= PA_DEVERR_QLEN;
        ql = 0;
    }
    if (ql > p.max_q) {
        err |= PA_DEVERR_QLEN;
        ql = p.max_q;
    }
    if (p.causal && ql > kv)   // causal and band rows sit at positions kv - ql .. kv - 1
        err |= PA_DEVERR_QLEN;
    return err;
}

// Items of one (sequence, KV head): the chunks of all its row tiles.
__host__ __device__ __forceinline__ int seq_items_per_group(const Params &p, int kv, int ql)
{
    const int ntile = seq_tiles(p, ql);
    int ipg = 0;
    for (int qt = 0; qt < ntile; ++qt)
        ipg += unit_chunks(p, kv, ql, qt);
    return ipg;
}

// Piece k begins at item s, inside sequence b (first item wsb, items per KV
// head ipg, first packed query row t0); piece k - 1 began at item s_prev.
// Returns the cursor at s and, when `write` and k > 0, writes split entry
// k - 1: the unit that boundary k cuts, if s falls strictly inside it and
// the unit began in piece k - 1 (a unit cut several times is listed once).
// With `tp` (the sequence's items per KV head before each of its row tiles,
// tp[0] = 0) the row tile is found by bisection, else by walking the tiles.
__host__ __device__ __forceinline__ Cursor piece_start(const Params &p, int k, int s, int s_prev, int b, int kv, int ql,
                                              int ipg, int wsb, int t0, bool write, const int *tp = nullptr)
{
    int local = s - wsb;
    const int gg = local / ipg;
    local -= gg * ipg;
    int u0 = wsb + gg * ipg;
    int t = 0, n;
    if (tp) {
        // every tile has at least one chunk: tp rises strictly
        int hi = seq_tiles(p, ql) - 1;
        while (t < hi) {
            const int mid = (t + hi + 1) >> 1;
            if (tp[mid] <= local)
                t = mid;
            else
                hi = mid - 1;
        }
        local -= tp[t];
        u0 += tp[t];
        n = unit_chunks(p, kv, ql, t);
    } else {
        n = unit_chunks(p, kv, ql, 0);
        while (local >= n) {
            local -= n;
            u0 += n;
            ++t;
            n = unit_chunks(p, kv, ql, t);
        }
    }
    if (write && k > 0) {
        int32_t *d = p.ws.splits + (size_t)(k - 1) * 8;
        const bool split = s > u0 && s_prev <= u0;
        int rows = ql * p.group - t * p.rows_per_tile;
        rows = rows < p.rows_per_tile ? rows : p.rows_per_tile;
        d[0] = split ? b : -1;
        d[1] = gg;
        d[2] = t;
        d[3] = u0;
        d[4] = u0 + n;
        d[5] = t0;
        d[6] = rows;
    }
    Cursor cu;
    cu.b = b;
    cu.g = gg;
    cu.qt = t;
    cu.c = local;
    cu.nch = n;
    cu.ntile = seq_tiles(p, ql);
    cu.item = s;
    return cu;
}

// ------------------------------------------------------------ piece map
// Where the pieces of an item range lie; pieces are numbered in item order.
// Uniform map (m = 0): pieces of `per` items, cut short at W (N = a pieces).
// Map with a claimed tail (m > 0, the self-planning streaming kernel): the
// range is cut into P shares of `per` items (the first W - P * per shares
// hold one item more, in their static piece); a share is its worker's
// static piece of `a` items followed by nr smaller pieces, of about half the share's remaining
// tail each, down to m items, the last taking what is left (at least m; at
// most kTailRounds of them).  Workers take their static piece first, then
// claim the tail pieces round by round over all shares (the largest first:
// the guided scheme known as factoring), so fast workers take more; and
// since every share keeps its own tail, a unit of the range is cut into at
// most about nr + 1 pieces per share it spans.  The map depends on the
// lengths alone, like the pieces themselves.
struct PieceMap {
    int W, per, a, m, P, nr;
};

// First item of share w (the first L = W - P * per shares hold per + 1).
__host__ __device__ __forceinline__ int share_start(const PieceMap &pm, int w)
{
    const int L = pm.W - pm.P * pm.per;
    return w * pm.per + (w < L ? w : L);
}

// Items of round r's piece in every share's tail (tail = per - a items).
__host__ __device__ __forceinline__ int tail_piece_size(const PieceMap &pm, int r, int &left)
{
    int s = left / 2;
    s = s > pm.m ? s : pm.m;
    if (left - s < pm.m || r == kTailRounds - 1)
        s = left;
    left -= s;
    return s;
}

// Pieces of the map.
__host__ __device__ __forceinline__ int piece_count(const PieceMap &pm)
{
    return pm.m > 0 ? pm.P * (1 + pm.nr) : pm.a;
}

// The piece a worker starts with, and the piece a claim (0, 1, ...: round
// by round, share by share) stands for (-1: none left).
__host__ __device__ __forceinline__ int static_piece(const PieceMap &pm, int w)
{
    return pm.m > 0 ? w * (1 + pm.nr) : w;
}

__host__ __device__ __forceinline__ int claimed_piece(const PieceMap &pm, int c)
{
    if (pm.m <= 0 || c < 0 || c >= pm.nr * pm.P)
        return -1;
    return (c % pm.P) * (1 + pm.nr) + 1 + c / pm.P;
}

// Items [s0, s1) of piece k (empty past the last piece).
__host__ __device__ __forceinline__ void piece_range(const PieceMap &pm, int k, int &s0, int &s1)
{
    if (pm.m <= 0) {
        const int64_t x = (int64_t)k * pm.per, y = x + pm.per;
        s0 = x < pm.W ? (int)x : pm.W;
        s1 = y < pm.W ? (int)y : pm.W;
        return;
    }
    if (k < 0 || k >= piece_count(pm)) {
        s0 = s1 = k < 0 ? 0 : pm.W;
        return;
    }
    const int w = k / (1 + pm.nr), j = k - w * (1 + pm.nr);
    const int a = pm.a + (share_start(pm, w + 1) - share_start(pm, w) - pm.per);   // static piece
    s0 = share_start(pm, w);
    if (j == 0) {
        s1 = s0 + a;
        return;
    }
    s0 += a;
    int left = pm.per - pm.a, sz = 0;
    for (int r = 0; r < j; ++r) {
        s0 += sz;
        sz = tail_piece_size(pm, r, left);
    }
    s1 = s0 + sz;
}

// The piece holding item `item` (0 <= item < W).
__host__ __device__ __forceinline__ int piece_of(const PieceMap &pm, int item)
{
    if (pm.m <= 0)
        return item / pm.per;
    const int L = pm.W - pm.P * pm.per;
    const int w = item < L * (pm.per + 1) ? item / (pm.per + 1) : L + (item - L * (pm.per + 1)) / pm.per;
    int off = item - share_start(pm, w) - pm.a - (w < L ? 1 : 0);
    if (off < 0)
        return w * (1 + pm.nr);
    int left = pm.per - pm.a;
    for (int r = 0; r < pm.nr; ++r) {
        const int sz = tail_piece_size(pm, r, left);
        if (off < sz || r == pm.nr - 1)
            return w * (1 + pm.nr) + 1 + r;
        off -= sz;
    }
    return w * (1 + pm.nr) + pm.nr;
}

// The map as written in the workspace header.
__device__ __forceinline__ PieceMap header_piece_map(const int32_t *hdr)
{
    return PieceMap{hdr[0], hdr[1], hdr[4], hdr[5], hdr[6], hdr[7]};
}

// The self-planning streaming kernel's map of W items: with a claimed tail
// when the launch asks for one and every share holds at least
// kTailMinShare * m items (static pieces of 9/10 of a share, so a tail holds
// at least 2 m), else one uniform piece per worker.  (Static pieces of 4/5
// took 5 us longer per pass on the long skewed decode with head pairs, 19/20
// 20 us longer.)
__host__ __device__ __forceinline__ PieceMap self_piece_map(const Params &p, int W)
{
    const int P = p.partitions, m = p.tail_min;
    if (m > 0 && (int64_t)W >= (int64_t)kTailMinShare * m * P) {
        PieceMap pm{W, W / P, 0, m, P, 0};
        pm.a = (int)(((int64_t)9 * pm.per) / 10);
        int left = pm.per - pm.a;
        while (left > 0)
            (void)tail_piece_size(pm, pm.nr++, left);
        return pm;
    }
    const int per = (W + p.pieces - 1) / p.pieces;
    return PieceMap{W, per > 0 ? per : 1, p.pieces, 0, P, 0};
}

// Next piece for a worker that finished its current one (one lane calls).
// The counter is updated at system scope, so workgroups on every XCD see one
// sequence of values.
__device__ __forceinline__ int grab_piece(const Params &p)
{
    return p.partitions + __hip_atomic_fetch_add(p.ws.hdr + 3, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Whole-tile mode.  The workgroups w with w % 8 == x (those the dispatcher
// deals to XCD x, Lx of them) take the tasks of queue x.  Each takes its first
// task at position w / 8; every later position (Lx, Lx + 1, ...) is claimed
// from the queue's counter by a workgroup a few chunks before its current task
// ends, so a worker that runs slow takes fewer tasks.  Consecutive positions
// -- the row tiles of one (sequence, KV head) -- start close together on one
// XCD and read their sequence's KV from its L2.  A workgroup whose queue is
// empty claims from the other queues in turn.
__device__ __forceinline__ int tile_queue_workers(int x, int nwg)
{
    return (nwg - x + kXcds - 1) / kXcds;
}

// The first task of workgroup w (index in the task array), or -1.
__device__ __forceinline__ int tile_first_task(const Params &p, int w)
{
    const int x = w % kXcds, l = w / kXcds;
    return l < sload(p.ws.tq, kTqLength + x) ? sload(p.ws.tq, kTqStart + x) + l : -1;
}

// One lane: the next unclaimed position of queue x (possibly past its end).
// System scope, as the piece counter: workgroups on every XCD see one
// sequence of values.
__device__ __forceinline__ int tile_claim(const Params &p, int x, int nwg)
{
    return tile_queue_workers(x, nwg) + __hip_atomic_fetch_add(p.ws.tq + kTqCounter + kTqCounterStride * x, 1,
                                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// One lane: the task at position pos of queue x, claimed earlier, or else one
// claimed from the other queues in turn; -1 when every queue is exhausted.
__device__ __forceinline__ int tile_next_task(const Params &p, int x, int nwg, int pos)
{
    for (int k = 0; k < kXcds; ++k) {
        const int y = (x + k) & (kXcds - 1);
        if (k > 0)
            pos = tile_claim(p, y, nwg);
        if (pos < p.ws.tq[kTqLength + y])
            return p.ws.tq[kTqStart + y] + pos;
    }
    return -1;
}

// The cursor of whole-tile task t: all chunks of row tile (b, g, qt).
__device__ __forceinline__ void tile_task_cursor(const Params &p, int t, Cursor &cu, int &end)
{
    const int32_t *e = p.ws.tq + kTqHeader + 2 * (size_t)t;
    const int b = sload(e, 0), gq = sload(e, 1);
    const int kv = sload(p.ws.kvlen, b), ql = sload(p.ws.qlen, b);
    cu.b = b;
    cu.g = gq >> 16;
    cu.qt = gq & 0xffff;
    cu.c = 0;
    cu.ntile = seq_tiles(p, ql);
    cu.nch = unit_chunks(p, kv, ql, cu.qt);
    cu.item = 0;
    end = cu.nch;
}

#endif  // __HIPCC__

}  // namespace pa

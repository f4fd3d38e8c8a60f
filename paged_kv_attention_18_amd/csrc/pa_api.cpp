// pa_api.cpp -- host side of the C ABI declared in include/pa.h: argument
// checks, kernel selection, workspace, launches and timing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "pa.h"
#include "pa_internal.h"

namespace {

constexpr int kMaxTimedPasses = 1024;
constexpr int kEventsPerPass = 6;   // start and stop of the plan, attention and merge kernels
// Pieces of the item range per worker in balanced mode.  With more pieces
// than workers, workers that finish early take the remaining pieces, which
// evens out end times; it pays where a chunk is long (many rows on the
// matrix cores).  The decode streaming kernel keeps one static piece per
// worker (the plan kernel's pieces), or, planning for itself on a long
// pass, adds the claimed tail of pa::PieceMap (variant 4): there the
// computing wave claims, since waiting for an atomic's return on the
// issuing wave would drain its load pipeline (one in-order vector memory
// counter per wave).
constexpr int kMaxPiecesPerWorker = 2;

struct Variant {
    int path;        // 0 = VALU decode, 1 = MFMA tile
    int rows_pad;    // VALU: padded rows per unit
    int tile_variant;  // MFMA: kernel variant (pa::tile_supported)
    int rows_per_tile;
    int chunk;
    int partitions;  // balanced-mode workers (waves for the VALU kernel, workgroups for MFMA)
    int pieces_per_worker;
    bool claimed_tail;   // self-planning launches cut a claimed tail (up to pa::kTailRounds rounds)
    bool streaming;      // MFMA: the one-wave streaming kernel (units of at most 16 rows)
    int hp;              // KV heads per unit (2: head pairs, streaming kernel)
    int self_variant, tail_variant;   // the self-planning variants (streaming: without, with claims; 576/512: 8)
    bool tile_self;      // 576/512 tile kernel: its self-planning twin serves this mode at full occupancy
    int max_pieces() const { return partitions * (claimed_tail ? 1 + pa::kTailRounds : pieces_per_worker); }
};

int next_pow2(int x)
{
    int p = 1;
    while (p < x)
        p <<= 1;
    return p;
}

// Floats per partial slot: R x Dv outputs, then R maxima and R sums, rounded
// up to a multiple of 4 so every slot starts 16-byte aligned.
size_t partial_floats(int rows, int dv)
{
    return ((size_t)rows * (dv + 2) + 3) & ~(size_t)3;
}

bool valid_dtype(int d) { return d == PA_F16 || d == PA_BF16; }
bool valid_mask(int m)
{
    return m == PA_MASK_NONE || m == PA_MASK_CAUSAL || m == PA_MASK_BAND || m == PA_MASK_TENSOR || m == PA_MASK_SPARSE;
}

int kernel_mode(int mask)
{
    return mask == PA_MASK_BAND ? 1 : (mask == PA_MASK_TENSOR ? 2 : (mask == PA_MASK_SPARSE ? 3 : 0));
}

// Sparse lists: every 64-row tile must hold the rows of one query token.
constexpr int kSparseTileRows = 64;

// Kernel variants of the streaming kernel that plan for themselves: one
// static piece per worker, and the same with a claimed tail of pieces.
constexpr int kSelfPlanVariant = 3;
constexpr int kSelfPlanTailVariant = 4;
// The streaming kernel on head pairs (variants 0, 3, 4 with two KV heads per
// unit): a unit reads 512-byte runs of each token row instead of 256-byte
// ones, which the memory system serves faster.
constexpr bool kHeadPairs = true;
constexpr int kPairVariant = 5, kPairSelfPlanVariant = 6, kPairSelfPlanTailVariant = 7;
// The 576/512 tile kernel (variant 0) planning for itself, for passes of one
// row tile per (sequence, KV head) and one piece per worker
constexpr int kTileSelfPlanVariant = 8;
// band units of at most this many KV chunks run whole (no split, no merge)
constexpr int kBandWholeUnitChunks = 8;
// decode passes whose units have at most this many chunks (by the block
// tables' capacity) run every unit whole on the streaming kernel
constexpr int kStreamWholeUnitChunks = 8;

}  // namespace

struct pa_handle {
    pa_config cfg;
    int device = 0;
    int num_cus = 256;
    void *ws_base = nullptr;
    size_t ws_bytes = 0;
    pa::Workspace ws{};
    int max_partitions = 0;
    size_t max_partial_floats = 0;
    size_t max_pieces = 0;   // pieces of a pass, at most (split entries and partial slot pairs)
    // timing
    bool timing = false;
    std::vector<hipEvent_t> events;   // per pass: start and stop of plan, attention, merge
    std::vector<char> planned;        // per timed pass: the plan kernel was launched
    std::vector<char> merged;         // ... the merge kernel was launched
    int timed = 0;

    Variant choose(int max_q) const
    {
        Variant v{};
        v.hp = 1;
        const int G = cfg.head_num / cfg.kv_head_num;
        const int rows = max_q * G;
        const bool dec_ok = pa::decode_supported(cfg.head_size_k, cfg.head_size_v);
        // The matrix-core kernels by default, also for thin decode units
        // (one padded 16-row block): the streaming kernel keeps a ring of
        // KV chunks in flight through LDS across units, which the VALU
        // kernel (chunks held in registers) cannot match in bytes in flight.
        // The VALU kernel stays available for up to 8 rows.
        const bool valu = (cfg.flags & PA_FLAG_FORCE_VALU) && dec_ok && rows <= 8;
        if (valu) {
            v.path = 0;
            v.rows_pad = next_pow2(rows < 1 ? 1 : rows);
            v.rows_per_tile = v.rows_pad;
            v.chunk = pa::decode_chunk(cfg.head_size_k, v.rows_pad);
            v.partitions = num_cus * pa::decode_workers_per_cu(cfg.dtype, cfg.head_size_k, cfg.head_size_v, v.rows_pad);
            v.pieces_per_worker = 1;
        } else {
            v.path = 1;
            const int dk = cfg.head_size_k, dv = cfg.head_size_v;
            const bool sh = (cfg.flags & PA_FLAG_SHARED_KV) != 0;
            const int mode = kernel_mode(cfg.mask);   // the kernels' shapes depend on the mode
            int var = 0;
            // (variant 2 with the tensor mask at head sizes up to 128 only;
            // sparse lists: variant 1 below 576, the one 576/512 variant
            // above)
            if ((rows > 16 || cfg.mask == PA_MASK_SPARSE) && pa::tile_supported(dk, dv, 1))
                var = (rows > pa::tile_rows(dk, dv, 1, sh, mode) && pa::tile_supported(dk, dv, 2) &&
                       cfg.mask != PA_MASK_SPARSE &&
                       (cfg.mask != PA_MASK_TENSOR || pa::tile_rows(dk, dv, 2, sh, mode) > 0)) ? 2 : 1;
            v.streaming = pa::tile_streaming(dk, dv, var);
            v.hp = 1;
            v.self_variant = kSelfPlanVariant;
            v.tail_variant = kSelfPlanTailVariant;
            // head pairs where both heads' rows still fit one 16-row block
            if (kHeadPairs && v.streaming && cfg.kv_head_num % 2 == 0 && 2 * rows <= 16 &&
                pa::tile_supported(dk, dv, kPairVariant)) {
                var = kPairVariant;
                v.hp = 2;
                v.self_variant = kPairSelfPlanVariant;
                v.tail_variant = kPairSelfPlanTailVariant;
            }
            v.tile_variant = var;
            v.rows_per_tile = pa::tile_rows(dk, dv, var, sh, mode);
            v.chunk = pa::tile_chunk(dk, dv, var, sh, mode);
            v.partitions = num_cus * pa::tile_workers_per_cu(cfg.dtype, dk, dv, var, sh, mode);
            // the self-planning twin of the 576/512 kernel, where it keeps
            // the same workgroups per CU
            v.tile_self = !v.streaming && var == 0 &&
                          pa::tile_chunk(dk, dv, kTileSelfPlanVariant, sh, mode) == v.chunk &&
                          num_cus * pa::tile_workers_per_cu(cfg.dtype, dk, dv, kTileSelfPlanVariant, sh, mode) >=
                              v.partitions;
            if (v.tile_self)
                v.self_variant = kTileSelfPlanVariant;
            if (v.streaming && pa::tile_supported(dk, dv, v.self_variant)) {
                // the self-planning twins of the streaming kernel run the same grid
                for (int sv : {v.self_variant, v.tail_variant}) {
                    const int w3 = num_cus * pa::tile_workers_per_cu(cfg.dtype, dk, dv, sv, sh, mode);
                    v.partitions = w3 < v.partitions ? w3 : v.partitions;
                }
            }
            // one piece per worker for the streaming kernel and for the one
            // kernel above head size 256 (variant 0: 64-row tiles whose fp32
            // partials, 131 KB per piece at 576/512, outweigh finer pieces)
            v.pieces_per_worker = (v.streaming || var == 0) ? 1 : kMaxPiecesPerWorker;
            // the self-planning streaming kernel may add rounds of claimed
            // pieces (pa::PieceMap)
            v.claimed_tail = v.streaming && pa::tile_supported(dk, dv, v.tail_variant) &&
                             !(cfg.flags & PA_FLAG_STATIC_PIECES);
        }
        if (cfg.num_partitions > 0)
            v.partitions = cfg.num_partitions;
        return v;
    }
};

extern "C" {

const char *pa_status_string(pa_status s)
{
    switch (s) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_HIP: return "HIP runtime error";
    case PA_ERR_OOM: return "out of device memory";
    case PA_ERR_SCRATCH: return "the pass needs more workspace than pa_forward_noalloc's static device array";
    }
    return "unknown status";
}

static pa_status check_config(const pa_config *c)
{
    if (!c)
        return PA_ERR_INVALID_ARG;
    if (c->head_num <= 0 || c->kv_head_num <= 0 || c->head_num % c->kv_head_num != 0)
        return PA_ERR_INVALID_ARG;
    if (c->head_size_k <= 0 || c->head_size_k > 576 || c->head_size_v <= 0 || c->head_size_v > 576)
        return PA_ERR_INVALID_ARG;
    if (c->block_size <= 0 || c->block_size % 16 != 0 || c->block_size > 256)
        return PA_ERR_INVALID_ARG;
    if ((c->mask == PA_MASK_CAUSAL || c->head_size_k > 256 || c->head_size_v > 256) && c->block_size > 128)
        return PA_ERR_INVALID_ARG;
    if (c->num_blocks <= 0 || c->max_batch <= 0 || c->max_num_blocks_per_seq <= 0 || c->max_q_seq_len <= 0)
        return PA_ERR_INVALID_ARG;
    if (!valid_dtype(c->dtype) || !valid_mask(c->mask) || !std::isfinite(c->scale) || c->num_partitions < 0)
        return PA_ERR_INVALID_ARG;
    if ((c->flags & PA_FLAG_FORCE_VALU) && (c->flags & PA_FLAG_FORCE_MFMA))
        return PA_ERR_INVALID_ARG;
    if (c->flags & ~(uint32_t)(PA_FLAG_FORCE_VALU | PA_FLAG_FORCE_MFMA | PA_FLAG_NO_SPLIT | PA_FLAG_SHARED_KV |
                               PA_FLAG_STATIC_PIECES | PA_FLAG_PLAN_KERNEL))
        return PA_ERR_INVALID_ARG;
    if ((c->flags & PA_FLAG_SHARED_KV) && c->head_size_v > c->head_size_k)
        return PA_ERR_INVALID_ARG;   // V must fit inside the K row
    if (c->mask == PA_MASK_BAND && (c->window_left < 0 || c->window_left > (1 << 30) || c->window_right < 0 ||
                                    c->window_right > (1 << 30)))
        return PA_ERR_INVALID_ARG;
    if (c->mask == PA_MASK_TENSOR && !c->mask_tensor)
        return PA_ERR_INVALID_ARG;
    if (c->mask == PA_MASK_SPARSE && c->topk <= 0)
        return PA_ERR_INVALID_ARG;
    // Item indices are int32 on the device: bound the largest possible count.
    const int G = c->head_num / c->kv_head_num;
    const double tiles = std::ceil((double)c->max_q_seq_len * G / 16.0);
    const double chunks = std::ceil((double)c->max_num_blocks_per_seq * c->block_size / 16.0) + 1.0;
    if ((double)c->max_batch * c->kv_head_num * tiles * chunks > 2.0e9)
        return PA_ERR_INVALID_ARG;
    if ((double)c->max_num_blocks_per_seq * c->block_size > 2.0e9)
        return PA_ERR_INVALID_ARG;
    // Shapes with kernels in this build.
    const bool dec = pa::decode_supported(c->head_size_k, c->head_size_v);
    const bool til = pa::tile_supported(c->head_size_k, c->head_size_v, 0);
    if (!dec && !til)
        return PA_ERR_UNSUPPORTED;
    // The VALU kernel serves decode without a mask only: it has neither a
    // lower visibility bound nor the matrix, and its causal mode is switched
    // off (a GPU memory fault was seen once in a causal run, cause not found).
    if ((c->flags & PA_FLAG_FORCE_VALU) && (!dec || c->mask != PA_MASK_NONE))
        return PA_ERR_UNSUPPORTED;
    if ((c->flags & PA_FLAG_FORCE_MFMA) && !til)
        return PA_ERR_UNSUPPORTED;
    if (c->mask == PA_MASK_SPARSE && (!til || G % kSparseTileRows != 0 || c->topk > 2048))
        return PA_ERR_UNSUPPORTED;   // a tile's rows share one query token's list, staged whole in LDS
    if (!til && (int64_t)c->max_q_seq_len * G > 8)
        return PA_ERR_UNSUPPORTED;   // only the VALU kernel exists for this shape
    if ((c->flags & PA_FLAG_FORCE_VALU) && (int64_t)c->max_q_seq_len * G > 8)
        return PA_ERR_UNSUPPORTED;   // the VALU kernel takes at most 8 rows per unit
    return PA_OK;
}

pa_status pa_create(const pa_config *cfg, pa_handle **out)
{
    if (!out)
        return PA_ERR_INVALID_ARG;
    *out = nullptr;
    pa_status st = check_config(cfg);
    if (st != PA_OK)
        return st;

    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return PA_ERR_HIP;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
        return PA_ERR_HIP;
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return PA_ERR_UNSUPPORTED;

    pa_handle *h = new (std::nothrow) pa_handle;
    if (!h)
        return PA_ERR_OOM;
    h->cfg = *cfg;
    h->device = dev;
    h->num_cus = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256;

    // Largest grid and partial slot over every call this handle may see.
    size_t max_floats = 0, max_pieces = 1, max_slot_floats = 0;   // slot floats: pieces x floats per slot
    int max_p = 8;
    // The variant depends on max_q * G only through thresholds at or below 65
    // rows, so the calls with max_q <= 65 and max_q = cfg->max_q_seq_len
    // cover every case.
    const int qmax = cfg->max_q_seq_len;
    std::vector<int> qs;
    for (int q = 1; q <= qmax && q <= 65; ++q)
        qs.push_back(q);
    if (qmax > 65)
        qs.push_back(qmax);
    int max_tiles = 1;
    const int G = cfg->head_num / cfg->kv_head_num;
    for (int q : qs) {
        const Variant v = h->choose(q);
        const size_t f = partial_floats(v.rows_per_tile, cfg->head_size_v);
        if (f > max_floats)
            max_floats = f;
        if (v.partitions > max_p)
            max_p = v.partitions;
        if ((size_t)v.max_pieces() > max_pieces)
            max_pieces = (size_t)v.max_pieces();
        if ((size_t)v.max_pieces() * f > max_slot_floats)
            max_slot_floats = (size_t)v.max_pieces() * f;
        const int tiles = (int)(((int64_t)q * G * v.hp + v.rows_per_tile - 1) / v.rows_per_tile);
        if (tiles > max_tiles)
            max_tiles = tiles;
    }
    h->max_partitions = max_p;
    h->max_partial_floats = max_floats;
    h->max_pieces = max_pieces;

    const int B = cfg->max_batch;
    auto align = [](size_t x) { return (x + 255) & ~(size_t)255; };
    size_t off = 0;
    const size_t o_hdr = off; off = align(off + 8 * sizeof(int32_t));
    const size_t o_cuq = off; off = align(off + (B + 1) * sizeof(int32_t));
    const size_t o_wsb = off; off = align(off + (B + 1) * sizeof(int32_t));
    const size_t o_ipg = off; off = align(off + B * sizeof(int32_t));
    const size_t o_ql = off; off = align(off + B * sizeof(int32_t));
    const size_t o_kv = off; off = align(off + B * sizeof(int32_t));
    const size_t o_wgb = off; off = align(off + max_pieces * sizeof(int32_t));
    const size_t o_spl = off; off = align(off + max_pieces * 8 * sizeof(int32_t));
    const size_t o_err = off; off = align(off + sizeof(uint32_t));
    const size_t zero_bytes = 16 * (size_t)cfg->kv_head_num * (size_t)(cfg->head_size_k > cfg->head_size_v ? cfg->head_size_k : cfg->head_size_v) * 2;
    const size_t o_zero = off; off = align(off + zero_bytes);
    const size_t o_part = off; off = align(off + 2 * max_slot_floats * sizeof(float));
    const size_t o_tq = off;
    off = align(off + (pa::kTqHeader + 2 * (size_t)B * cfg->kv_head_num * max_tiles) * sizeof(int32_t));
    h->ws_bytes = off;
    if (hipMalloc(&h->ws_base, h->ws_bytes) != hipSuccess) {
        delete h;
        return PA_ERR_OOM;
    }
    if (hipMemset(h->ws_base, 0, h->ws_bytes) != hipSuccess) {
        (void)hipFree(h->ws_base);
        delete h;
        return PA_ERR_HIP;
    }
    char *base = (char *)h->ws_base;
    h->ws.hdr = (int32_t *)(base + o_hdr);
    h->ws.cu_q = (int32_t *)(base + o_cuq);
    h->ws.wsb = (int32_t *)(base + o_wsb);
    h->ws.ipg = (int32_t *)(base + o_ipg);
    h->ws.qlen = (int32_t *)(base + o_ql);
    h->ws.kvlen = (int32_t *)(base + o_kv);
    h->ws.wg_b = (int32_t *)(base + o_wgb);
    h->ws.splits = (int32_t *)(base + o_spl);
    h->ws.err = (uint32_t *)(base + o_err);
    h->ws.zeros = base + o_zero;
    h->ws.partials = (float *)(base + o_part);
    h->ws.tq = (int32_t *)(base + o_tq);
    *out = h;
    return PA_OK;
}

pa_status pa_destroy(pa_handle *h)
{
    if (!h)
        return PA_OK;
    pa_status st = PA_OK;
    if (hipDeviceSynchronize() != hipSuccess)
        st = PA_ERR_HIP;
    for (hipEvent_t e : h->events)
        (void)hipEventDestroy(e);
    if (h->ws_base && hipFree(h->ws_base) != hipSuccess)
        st = PA_ERR_HIP;
    delete h;
    return st;
}

pa_status pa_describe(const pa_handle *h, int32_t max_q_seq_len, int32_t *path, int32_t *rows_per_tile,
                      int32_t *tokens_per_chunk, int32_t *partitions)
{
    if (!h || max_q_seq_len < 1 || max_q_seq_len > h->cfg.max_q_seq_len)
        return PA_ERR_INVALID_ARG;
    const Variant v = h->choose(max_q_seq_len);
    if (path)   // 2: the streaming variant of the matrix-core kernel
        *path = v.path == 1 && pa::tile_streaming(h->cfg.head_size_k, h->cfg.head_size_v, v.tile_variant) ? 2 : v.path;
    if (rows_per_tile)
        *rows_per_tile = v.rows_per_tile;
    if (tokens_per_chunk)
        *tokens_per_chunk = v.chunk;
    if (partitions)
        *partitions = v.partitions;
    return PA_OK;
}

// Checks the arguments of one pass and fills its launch parameters (all but
// the workspace pointers).  *empty: nothing to launch (no sequence or no
// query token).
static pa_status setup_params(const pa_handle *h, const void *query, const void *key_cache, const void *value_cache,
                              const int32_t *block_tables, const int32_t *context_lens, const int32_t *q_seq_lens,
                              const int32_t *topk_indices, int32_t batch, int32_t num_q_tokens, int32_t max_q_seq_len,
                              void *out, float *lse, pa::Params &p, Variant &v, bool *empty)
{
    *empty = true;
    if (!h || !query || !key_cache || !block_tables || !context_lens || !out)
        return PA_ERR_INVALID_ARG;
    const pa_config &c = h->cfg;
    // the sparse mode takes its lists through pa_forward_sparse only
    if ((c.mask == PA_MASK_SPARSE) != (topk_indices != nullptr))
        return PA_ERR_INVALID_ARG;
    const bool shared = (c.flags & PA_FLAG_SHARED_KV) != 0;
    // shared K/V: value_cache is NULL or the key cache itself
    if (shared ? (value_cache && value_cache != key_cache) : !value_cache)
        return PA_ERR_INVALID_ARG;
    if (batch < 0 || batch > c.max_batch || num_q_tokens < 0)
        return PA_ERR_INVALID_ARG;
    if (!q_seq_lens) {
        if (num_q_tokens != batch || max_q_seq_len != 1)
            return PA_ERR_INVALID_ARG;
    }
    if (max_q_seq_len < 1 || max_q_seq_len > c.max_q_seq_len)
        return PA_ERR_INVALID_ARG;
    if (batch == 0 || num_q_tokens == 0)
        return PA_OK;
    *empty = false;
    v = h->choose(max_q_seq_len);
    // (head pairs: a unit is two KV heads and their 2 G query heads; the
    // row -> (token, query head) map is the same with G and Hkv so taken)
    const int G = c.head_num / c.kv_head_num * v.hp;

    p = pa::Params{};
    p.query = query;
    p.key_cache = key_cache;
    p.value_cache = shared ? key_cache : value_cache;
    p.shared_kv = shared ? 1 : 0;
    p.v_row_bytes = (uint32_t)c.kv_head_num * (uint32_t)(shared ? c.head_size_k : c.head_size_v) * 2u;
    p.v_head_bytes = (uint32_t)(shared ? c.head_size_k : c.head_size_v) * 2u * (uint32_t)v.hp;
    p.block_tables = block_tables;
    p.context_lens = context_lens;
    p.q_seq_lens = q_seq_lens;
    p.out = out;
    p.lse = lse;
    p.num_blocks = c.num_blocks;
    p.batch = batch;
    p.num_q_tokens = num_q_tokens;
    p.head_num = c.head_num;
    p.kv_head_num = c.kv_head_num / v.hp;
    p.group = G;
    p.head_size_k = c.head_size_k;
    p.head_size_v = c.head_size_v;
    p.block_size = c.block_size;
    p.bs_shift = (c.block_size & (c.block_size - 1)) == 0 ? __builtin_ctz(c.block_size) : -1;
    p.max_blocks = c.max_num_blocks_per_seq;
    p.max_q = max_q_seq_len;
    p.causal = c.mask == PA_MASK_CAUSAL || c.mask == PA_MASK_BAND;
    p.band = c.mask == PA_MASK_BAND;
    p.win_left = p.band ? c.window_left : 0;
    p.win_right = p.band ? c.window_right : 0;
    p.tmask = c.mask == PA_MASK_TENSOR;
    p.mask_tensor = p.tmask ? (const uint16_t *)c.mask_tensor : nullptr;
    p.sparse = c.mask == PA_MASK_SPARSE;
    p.topk = p.sparse ? c.topk : 0;
    p.topk_idx = p.sparse ? topk_indices : nullptr;
    p.scale_log2 = c.scale * 1.4426950408889634f;
    p.rows_per_tile = v.rows_per_tile;
    p.chunk = v.chunk;
    auto log2_or_none = [](int x) { return (x > 0 && (x & (x - 1)) == 0) ? __builtin_ctz((unsigned)x) : -1; };
    p.chunk_shift = log2_or_none(v.chunk);
    p.group_shift = log2_or_none(G);
    p.tile_shift = log2_or_none(v.rows_per_tile);
    p.max_tiles = (max_q_seq_len * G + v.rows_per_tile - 1) / v.rows_per_tile;
    p.no_split = (c.flags & PA_FLAG_NO_SPLIT) ? 1 : 0;
    // A band unit's keys lie within its query tokens plus the window.  When
    // that is a few chunks and there are no more units than workers (so
    // that pieces would cut nearly every unit), the fp32 partials and the
    // merge cost more than the parallelism they buy: each unit then runs
    // whole on one workgroup.  With more units, pieces that stream through
    // several units stay faster; the streaming kernel always keeps its
    // pieces.
    if (!p.no_split && c.mask == PA_MASK_BAND && v.path == 1 &&
        !pa::tile_streaming(c.head_size_k, c.head_size_v, v.tile_variant)) {
        const int64_t rows = std::min<int64_t>((int64_t)max_q_seq_len * G, v.rows_per_tile);
        const int64_t keys = (rows + G - 1) / G + 1 + (int64_t)c.window_left + c.window_right;
        const int64_t units = (int64_t)batch * p.kv_head_num * p.max_tiles;
        if ((keys + v.chunk - 1) / v.chunk + 1 <= kBandWholeUnitChunks &&
            units <= std::min(v.partitions, h->max_partitions))
            p.no_split = 1;
    }
    // Short decode passes (no unit longer than kStreamWholeUnitChunks
    // chunks, no more units than workers): the self-planning streaming
    // kernel runs every unit whole, so the pass has no partials and no merge
    // launch (the merge's launch and round trips outweigh splitting units of
    // a few chunks).
    if (!p.no_split && v.path == 1 && v.streaming && batch <= pa::kSelfPlanMaxBatch && max_q_seq_len <= 16) {
        const int64_t units = (int64_t)batch * p.kv_head_num * p.max_tiles;
        const int64_t cap = (int64_t)c.max_num_blocks_per_seq * c.block_size;
        if ((cap + v.chunk - 1) / v.chunk <= kStreamWholeUnitChunks &&
            units <= std::min(v.partitions, h->max_partitions))
            p.no_split = 1;
    }
    p.partitions = p.no_split ? batch * p.kv_head_num * p.max_tiles
                              : (v.partitions < h->max_partitions ? v.partitions : h->max_partitions);
    // Sparse lists: every unit holds the same ceil(topk / 16) chunks.  Cut
    // into more than two pieces each, its fp32 partials (131 KB per piece at
    // 576/512) cost more than the extra workers gain: at most two workers
    // per unit, and at least one per CU.
    if (!p.no_split && c.mask == PA_MASK_SPARSE) {
        const int64_t units = (int64_t)batch * p.kv_head_num * p.max_tiles;
        const int64_t cap = std::max<int64_t>(h->num_cus, 2 * units);
        if (p.partitions > cap)
            p.partitions = (int32_t)cap;
    }
    p.pieces = p.no_split ? 0 : p.partitions * v.pieces_per_worker;
    p.partial_stride = (int32_t)partial_floats(v.rows_per_tile, c.head_size_v);
    p.tail_min = 0;
    // The tile kernel may run the pass as whole row tiles from per-XCD
    // queues; the planner decides from the lengths.
    p.tile_order = (v.path == 1 && !p.no_split && !pa::tile_streaming(c.head_size_k, c.head_size_v, v.tile_variant) &&
                    pa::tile_whole_tasks(c.head_size_k, shared))
                       ? 1
                       : 0;
    // The streaming kernel cuts its own pieces when the lengths fit in a
    // wave's registers: one launch fewer, and no wait on plan data when a
    // worker starts or moves to the next unit.  So does the 576/512 tile
    // kernel for passes of one row tile per (sequence, KV head) (decode,
    // sparse lists), whose pieces are then cut in the same way.
    const bool stream_self = v.streaming && max_q_seq_len <= 16 &&
                             pa::tile_supported(c.head_size_k, c.head_size_v, v.self_variant);
    const bool tile_self = v.tile_self && p.max_tiles == 1;
    p.self_plan = (v.path == 1 && (stream_self || tile_self) && batch <= pa::kSelfPlanMaxBatch &&
                   (p.no_split || p.pieces == p.partitions) && !(c.flags & PA_FLAG_PLAN_KERNEL))
                      ? 1
                      : 0;
    if (p.self_plan)
        p.tile_order = 0;
    // self-planning: claimed pieces after the static ones, in rounds that
    // shrink down to kTailMinChunks chunks, where the block tables can hold
    // a pass long enough for them (the kernel decides from the lengths);
    // shorter passes take the kernel without the claiming code
    if (p.self_plan && v.claimed_tail && !p.no_split) {
        const int64_t cap = (int64_t)c.max_num_blocks_per_seq * c.block_size;
        const int64_t w_max = (int64_t)batch * p.kv_head_num * ((cap + v.chunk - 1) / v.chunk);
        if (w_max >= (int64_t)pa::kTailMinShare * pa::kTailMinChunks * p.partitions)
            p.tail_min = pa::kTailMinChunks;
    }
    return PA_OK;
}

// Pieces a pass cuts (split entries and partial slot pairs it may use).
static int64_t pass_pieces(const pa::Params &p)
{
    if (p.no_split)
        return 0;
    return (p.self_plan && p.tail_min > 0) ? (int64_t)(1 + pa::kTailRounds) * p.partitions : (int64_t)p.pieces;
}

// Enqueues the kernels of one pass whose parameters (workspace included) are set.
static pa_status launch_pass(pa_handle *h, const pa::Params &p, const Variant &v, hipStream_t s)
{
    const pa_config &c = h->cfg;
    // timed passes: each kernel's own start and end (events on the launch)
    const bool timed = h->timing && h->timed < kMaxTimedPasses;
    hipEvent_t *ev = timed ? &h->events[kEventsPerPass * h->timed] : nullptr;
    hipEvent_t none = nullptr;
    if (!p.self_plan && pa::launch_plan(p, s, timed ? ev[0] : none, timed ? ev[1] : none) != hipSuccess)
        return PA_ERR_HIP;
    hipError_t e = v.path == 0 ? pa::launch_decode(p, c.dtype, v.rows_pad, s, timed ? ev[2] : none,
                                                   timed ? ev[3] : none)
                               : pa::launch_tile(p, c.dtype,
                                                 p.self_plan ? (p.tail_min > 0 ? v.tail_variant : v.self_variant)
                                                             : v.tile_variant,
                                                 s, timed ? ev[2] : none, timed ? ev[3] : none);
    if (e != hipSuccess)
        return PA_ERR_HIP;
    bool merged = false;
    if (pa::launch_merge(p, c.dtype, s, timed ? ev[4] : none, timed ? ev[5] : none, &merged) != hipSuccess)
        return PA_ERR_HIP;
    if (timed) {
        h->planned[h->timed] = p.self_plan ? 0 : 1;
        h->merged[h->timed] = merged ? 1 : 0;
        ++h->timed;
    }
    return PA_OK;
}

static pa_status forward_impl(pa_handle *h, const void *query, const void *key_cache, const void *value_cache,
                              const int32_t *block_tables, const int32_t *context_lens, const int32_t *q_seq_lens,
                              const int32_t *topk_indices, int32_t batch, int32_t num_q_tokens, int32_t max_q_seq_len,
                              void *out, float *lse, void *stream)
{
    pa::Params p;
    Variant v;
    bool empty = true;
    const pa_status st = setup_params(h, query, key_cache, value_cache, block_tables, context_lens, q_seq_lens,
                                      topk_indices, batch, num_q_tokens, max_q_seq_len, out, lse, p, v, &empty);
    if (st != PA_OK || empty)
        return st;
    p.ws = h->ws;
    return launch_pass(h, p, v, (hipStream_t)stream);
}

pa_status pa_forward(pa_handle *h, const void *query, const void *key_cache, const void *value_cache,
                     const int32_t *block_tables, const int32_t *context_lens, const int32_t *q_seq_lens,
                     int32_t batch, int32_t num_q_tokens, int32_t max_q_seq_len, void *out, float *lse,
                     void *stream)
{
    return forward_impl(h, query, key_cache, value_cache, block_tables, context_lens, q_seq_lens, nullptr, batch,
                        num_q_tokens, max_q_seq_len, out, lse, stream);
}

pa_status pa_forward_sparse(pa_handle *h, const void *query, const void *key_cache, const void *value_cache,
                            const int32_t *block_tables, const int32_t *context_lens, const int32_t *q_seq_lens,
                            const int32_t *topk_indices, int32_t batch, int32_t num_q_tokens, int32_t max_q_seq_len,
                            void *out, float *lse, void *stream)
{
    if (!topk_indices)
        return PA_ERR_INVALID_ARG;
    return forward_impl(h, query, key_cache, value_cache, block_tables, context_lens, q_seq_lens, topk_indices,
                        batch, num_q_tokens, max_q_seq_len, out, lse, stream);
}

pa_status pa_get_device_error(pa_handle *h, uint32_t *code, int32_t clear)
{
    if (!h || !code)
        return PA_ERR_INVALID_ARG;
    if (hipDeviceSynchronize() != hipSuccess)
        return PA_ERR_HIP;
    if (hipMemcpy(code, h->ws.err, sizeof(uint32_t), hipMemcpyDeviceToHost) != hipSuccess)
        return PA_ERR_HIP;
    if (clear && hipMemset(h->ws.err, 0, sizeof(uint32_t)) != hipSuccess)
        return PA_ERR_HIP;
    if (clear && hipDeviceSynchronize() != hipSuccess)
        return PA_ERR_HIP;
    return PA_OK;
}

pa_status pa_set_timing(pa_handle *h, int32_t enable)
{
    if (!h)
        return PA_ERR_INVALID_ARG;
    if (enable && h->events.empty()) {
        h->events.resize(kEventsPerPass * kMaxTimedPasses);
        h->planned.assign(kMaxTimedPasses, 0);
        h->merged.assign(kMaxTimedPasses, 0);
        for (auto &e : h->events)
            if (hipEventCreate(&e) != hipSuccess)
                return PA_ERR_HIP;
    }
    h->timing = enable != 0;
    h->timed = 0;
    return PA_OK;
}

pa_status pa_read_timing(pa_handle *h, double ms[3], int32_t *count, int32_t *plan_launches, double *per_pass_ms,
                         int32_t per_pass_cap)
{
    if (!h || !ms || !count || per_pass_cap < 0 || (per_pass_cap > 0 && !per_pass_ms))
        return PA_ERR_INVALID_ARG;
    ms[0] = ms[1] = ms[2] = 0.0;
    *count = h->timed;
    int planned = 0;
    if (h->timed > 0) {
        const int last = h->timed - 1;
        if (hipEventSynchronize(h->events[kEventsPerPass * last + (h->merged[last] ? 5 : 3)]) != hipSuccess)
            return PA_ERR_HIP;
        for (int k = 0; k < h->timed; ++k) {
            for (int j = 0; j < 3; ++j) {
                // passes whose kernel planned for itself launched no plan
                // kernel (-1); passes without split entries, no merge (0)
                const bool none = (j == 0 && !h->planned[k]) || (j == 2 && !h->merged[k]);
                float t = 0.f;
                if (!none && hipEventElapsedTime(&t, h->events[kEventsPerPass * k + 2 * j],
                                                 h->events[kEventsPerPass * k + 2 * j + 1]) != hipSuccess)
                    return PA_ERR_HIP;
                ms[j] += t;
                if (k < per_pass_cap)
                    per_pass_ms[3 * k + j] = (j == 0 && !h->planned[k]) ? -1.0 : (double)t;
            }
            planned += h->planned[k] ? 1 : 0;
        }
    }
    if (plan_launches)
        *plan_launches = planned;
    h->timed = 0;
    return PA_OK;
}

pa_status pa_read_probe(const void *src, int64_t bytes, uint32_t *sink, int32_t workgroups, void *stream)
{
    if (!src || !sink || bytes <= 0 || bytes % 16 != 0 || workgroups <= 0)
        return PA_ERR_INVALID_ARG;
    return pa::launch_read_probe(src, (long long)bytes, sink, workgroups, (hipStream_t)stream) == hipSuccess
               ? PA_OK
               : PA_ERR_HIP;
}

}  // extern "C"

namespace pa {

pa_status validate_config(const pa_config *cfg)
{
    return check_config(cfg);
}

pa_status forward_in_buffer(const pa_config *cfg, int num_cus, void *base, size_t capacity, const void *query,
                            const void *key_cache, const void *value_cache, const int32_t *block_tables,
                            const int32_t *context_lens, const int32_t *q_seq_lens, int32_t batch,
                            int32_t num_q_tokens, int32_t max_q_seq_len, void *out, float *lse, void *stream)
{
    const pa_status cst = check_config(cfg);
    if (cst != PA_OK)
        return cst;
    if (!base || max_q_seq_len < 1 || max_q_seq_len > cfg->max_q_seq_len)
        return PA_ERR_INVALID_ARG;
    // a handle on the stack: the configuration and the grid bound pa_create
    // would give this call (its partitions), no workspace, no events
    pa_handle h;
    h.cfg = *cfg;
    h.num_cus = num_cus > 0 ? num_cus : 256;
    h.max_partitions = h.choose(max_q_seq_len).partitions;
    Params p;
    Variant v;
    bool empty = true;
    const pa_status st = setup_params(&h, query, key_cache, value_cache, block_tables, context_lens, q_seq_lens,
                                      nullptr, batch, num_q_tokens, max_q_seq_len, out, lse, p, v, &empty);
    if (st != PA_OK || empty)
        return st;
    // Layout for this pass only: the words that must start at zero (header
    // with the piece counter, error word, zero page) first, then the plan
    // arrays of `batch` sequences, the split entries and the partial slot
    // pairs of the pass's pieces.
    const size_t N = (size_t)pass_pieces(p);
    const size_t ent = N > 0 ? N : 1;
    const size_t B = (size_t)batch;
    const size_t zero_bytes = 16 * (size_t)cfg->kv_head_num *
                              (size_t)(cfg->head_size_k > cfg->head_size_v ? cfg->head_size_k : cfg->head_size_v) * 2;
    size_t off = 0;
    auto take = [&off](size_t bytes) {
        const size_t o = off;
        off = (off + bytes + 255) & ~(size_t)255;
        return o;
    };
    const size_t o_hdr = take(8 * sizeof(int32_t));
    const size_t o_err = take(sizeof(uint32_t));
    const size_t o_zero = take(zero_bytes);
    const size_t cleared = off;
    const size_t o_cuq = take((B + 1) * sizeof(int32_t));
    const size_t o_wsb = take((B + 1) * sizeof(int32_t));
    const size_t o_ipg = take(B * sizeof(int32_t));
    const size_t o_ql = take(B * sizeof(int32_t));
    const size_t o_kv = take(B * sizeof(int32_t));
    const size_t o_wgb = take(ent * sizeof(int32_t));
    const size_t o_spl = take(ent * 8 * sizeof(int32_t));
    const size_t o_part = take(2 * N * (size_t)p.partial_stride * sizeof(float));
    const size_t o_tq = take((kTqHeader + 2 * B * (size_t)cfg->kv_head_num * (size_t)p.max_tiles) * sizeof(int32_t));
    if (off > capacity)
        return PA_ERR_SCRATCH;
    char *b = (char *)base;
    p.ws.hdr = (int32_t *)(b + o_hdr);
    p.ws.err = (uint32_t *)(b + o_err);
    p.ws.zeros = b + o_zero;
    p.ws.cu_q = (int32_t *)(b + o_cuq);
    p.ws.wsb = (int32_t *)(b + o_wsb);
    p.ws.ipg = (int32_t *)(b + o_ipg);
    p.ws.qlen = (int32_t *)(b + o_ql);
    p.ws.kvlen = (int32_t *)(b + o_kv);
    p.ws.wg_b = (int32_t *)(b + o_wgb);
    p.ws.splits = (int32_t *)(b + o_spl);
    p.ws.partials = (float *)(b + o_part);
    p.ws.tq = (int32_t *)(b + o_tq);
    // earlier calls leave other contents here: clear what must start at
    // zero with a fill kernel (no memset node if the caller captures a graph)
    const hipStream_t s = (hipStream_t)stream;
    if (launch_zero_words((uint32_t *)b, (long long)(cleared / sizeof(uint32_t)), s) != hipSuccess)
        return PA_ERR_HIP;
    return launch_pass(&h, p, v, s);
}

}  // namespace pa

/*
 * pa.h -- C ABI of the MI355X (gfx950) paged-attention forward library.
 *
 * The operation (Ascend ATB "PagedAttentionOperation", Constraints; the pages
 * give the operator's tensors and constraints, the formula is the usual
 * attention): for every sequence b, query token i of b and query head h,
 *
 *     out[t0+i][h] = softmax_j( scale * q[t0+i][h] . K_j + mask(i, j) ) . V_j
 *
 * over the KV tokens j < context_lens[b] of sequence b, where
 *   - token j sits in physical block block_tables[b][j / block_size], slot
 *     j % block_size; every table entry is in [0, num_blocks) and each row
 *     holds at least ceil(context_lens[b] / block_size) ids (Constraints);
 *   - query head h reads KV head h / (head_num / kv_head_num) (GQA requires
 *     head_num % kv_head_num == 0, Constraints);
 *   - scale is one scalar (scaleType TOR, Constraints, mask type 5 list);
 *   - PA_MASK_NONE: every row sees all context_lens[b] tokens (maskType
 *     UNDEFINED, Constraints); PA_MASK_CAUSAL: parallel decoding / splitfuse
 *     (mask type 5), context_lens[b] counts history plus the current query
 *     tokens, prefix = max(0, context_lens[b] - q_seq_lens[b]), and row i
 *     sees tokens j <= prefix + i (the causal mask with its upper triangle,
 *     diagonal excluded, invisible; Constraints, mask type 5 list);
 *     PA_MASK_BAND: a sliding window (mask mode 4 of the
 *     SparseAttnSharedkvMetadata README, parameter table, with window_left
 *     past and window_right future tokens; the page fixes 127 and 0): row i
 *     sits at position prefix + i as in the causal mode and sees tokens
 *     prefix + i - window_left <= j <= prefix + i + window_right.  Masked
 *     tokens get weight exactly 0, and the chunks of KV blocks that no row
 *     of a tile sees are neither planned nor read (block-table entries of
 *     blocks wholly before a band are never used); PA_MASK_TENSOR: the
 *     shared compressed mask of mask type 5 (Constraints, mask type 5
 *     list: one fp16 [2048, 2048] matrix for all sequences and heads, 0 where
 *     visible, a large negative value such as -10000 above the diagonal,
 *     aligned by the prefix, longer sequences handled) is added to the
 *     scaled scores: row i against token j adds element [i][j - prefix];
 *     history tokens (j < prefix) are visible with nothing added; outside
 *     the matrix (i >= 2048 or j - prefix >= 2048) token j is visible with
 *     nothing added if j - prefix <= i and invisible otherwise.  Every
 *     token j < context_lens[b] is computed (the matrix decides its weight);
 *   - query and output rows are packed (TND): sequence b's rows start at
 *     t0 = q_seq_lens[0] + ... + q_seq_lens[b-1] (the cu_seqlens_q prefix-sum
 *     convention of the SparseAttnSharedkvMetadata README, parameter table);
 *   - key and value head sizes may differ, each in (0, 576]
 *     (Constraints: head sizes; block_size <= 128 when either exceeds 256).
 *
 * Accumulation is fp32; out has the query's dtype (round to nearest even);
 * the optional lse output is fp32, natural log: lse = max_j z_j + ln sum_j
 * exp(z_j - max_j z_j) with z_j = scale * q . K_j.  A row with no visible
 * token gets out = 0 and lse = -inf.
 *
 * Ownership: every tensor argument of pa_forward is a device pointer owned by
 * the caller.  The handle owns its workspace (work plan, split partials, a
 * piece counter, an error word), allocated once by pa_create and freed by
 * pa_destroy; it is sized for the largest pass the configuration allows,
 * including, for decode shapes whose passes may be long, the pieces the
 * streaming kernel claims at run time (up to 9 per worker; none with
 * PA_FLAG_STATIC_PIECES).  pa_forward allocates nothing, does not
 * synchronise, and enqueues all of its work on the given stream, so it may be
 * captured in a HIP graph; every pass leaves the piece counter reset for the
 * next one.  One handle must not be used by two streams at once (the
 * workspace is shared).
 *
 * Errors: functions return a pa_status synchronously.  Argument and shape
 * errors are reported before any device work is queued.  Problems that can
 * only be seen in device data (a block id outside [0, num_blocks), a table
 * too short for context_lens, q_seq_lens > context_lens in causal or band mode,
 * q_seq_lens that do not sum to num_q_tokens, negative lengths) never cause an
 * out-of-bounds access: the kernels clamp them and set a device error word
 * that pa_get_device_error reads back.
 */
#ifndef PA_H_
#define PA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PA_OK = 0,
    PA_ERR_INVALID_ARG = 1,   /* NULL pointer, bad size, shape outside the documented limits */
    PA_ERR_UNSUPPORTED = 2,   /* valid by the operator's rules but not built here (see pa_create) */
    PA_ERR_HIP = 3,           /* a HIP runtime call failed */
    PA_ERR_OOM = 4,           /* workspace allocation failed */
    PA_ERR_SCRATCH = 5        /* pa_forward_noalloc: the pass needs more workspace than its static array */
} pa_status;

typedef enum { PA_F16 = 0, PA_BF16 = 1 } pa_dtype;

typedef enum {
    PA_MASK_NONE = 0,    /* maskType UNDEFINED: all context_lens[b] tokens visible */
    PA_MASK_CAUSAL = 1,  /* mask type 5 (parallel decoding / splitfuse), prefix-aligned */
    PA_MASK_BAND = 2,    /* sliding window (band mask mode 4), prefix-aligned like CAUSAL */
    PA_MASK_TENSOR = 3,  /* the shared compressed mask matrix (mask type 5), see pa_config.mask_tensor */
    PA_MASK_SPARSE = 4   /* per-query-token lists of selected tokens (compressed-KV top-k), see
                            pa_forward_sparse */
} pa_mask;

/* pa_config.flags */
enum {
    PA_FLAG_FORCE_VALU = 1u << 0,  /* testing: require the VALU decode path (at most 8 rows per unit,
                                      i.e. max_q_seq_len * head_num / kv_head_num <= 8) */
    PA_FLAG_FORCE_MFMA = 1u << 1,  /* testing: take the MFMA tile path always */
    PA_FLAG_NO_SPLIT = 1u << 2,    /* testing: one worker per (sequence, KV head, row tile); no merge.
                                      Without the flag the library takes this path by itself for a
                                      band mask whose units reach at most 8 KV chunks when there are
                                      no more units than workers (pa_describe's partitions is then
                                      the split count it would otherwise use) */
    PA_FLAG_SHARED_KV = 1u << 3,   /* one cache for K and V: the V row of a token is the leading
                                      head_size_v elements of its K row (requires Dv <= Dk); see
                                      pa_forward's value_cache */
    PA_FLAG_STATIC_PIECES = 1u << 4, /* measurement: the decode streaming kernel keeps one piece per
                                        worker (no pieces claimed at run time); results agree with
                                        the default to the usual tolerance, not bit for bit */
    PA_FLAG_PLAN_KERNEL = 1u << 5    /* testing: every pass runs the plan kernel (no attention kernel
                                        cuts its own pieces).  Without a claimed tail (short passes,
                                        or with PA_FLAG_STATIC_PIECES) the pieces are the same and so
                                        are the results, bit for bit */
};

/* Device error word bits (pa_get_device_error). */
enum {
    PA_DEVERR_BLOCK_ID = 1u << 0,     /* a block id outside [0, num_blocks): read as zeros */
    PA_DEVERR_TABLE_SHORT = 1u << 1,  /* ceil(context_lens / block_size) > max_num_blocks_per_seq: clamped */
    PA_DEVERR_QLEN = 1u << 2,         /* q_seq_lens < 0, > max_q_seq_len, or > context_lens (causal): clamped */
    PA_DEVERR_TOKENS = 1u << 3,       /* sum of q_seq_lens != num_q_tokens: rows past the end not written */
    PA_DEVERR_CTX = 1u << 4           /* context_lens < 0: treated as 0 */
};

typedef struct {
    int32_t head_num;                /* query heads H */
    int32_t kv_head_num;             /* KV heads Hkv; H % Hkv == 0 */
    int32_t head_size_k;             /* key / query head size Dk, 0 < Dk <= 576 */
    int32_t head_size_v;             /* value / output head size Dv, 0 < Dv <= 576 */
    int32_t block_size;              /* tokens per KV block; % 16 == 0; <= 256, <= 128 in causal
                                        mode or when Dk or Dv > 256 */
    int64_t num_blocks;              /* physical blocks in each cache */
    int32_t max_batch;               /* largest batch pa_forward will be given */
    int32_t max_num_blocks_per_seq;  /* block_tables row length (its stride, in int32) */
    int32_t max_q_seq_len;           /* largest q_seq_lens[b] pa_forward will be given (1 for decode) */
    pa_dtype dtype;                  /* query, caches and output */
    float scale;                     /* the TOR scale, e.g. 1/sqrt(Dk) */
    pa_mask mask;
    uint32_t flags;                  /* PA_FLAG_* */
    int32_t num_partitions;          /* workgroups of the attention launch; 0 = chosen from the CU count */
    int32_t window_left;             /* PA_MASK_BAND: tokens before a row's position it sees, in [0, 2^30];
                                        ignored otherwise */
    int32_t window_right;            /* PA_MASK_BAND: tokens after it, in [0, 2^30]; ignored otherwise */
    const void *mask_tensor;         /* PA_MASK_TENSOR: device pointer to the shared fp16 [2048, 2048]
                                        mask matrix, owned by the caller and kept alive and unchanged
                                        while the handle is used; ignored otherwise */
    int32_t topk;                    /* PA_MASK_SPARSE: entries per list (> 0); ignored otherwise */
} pa_config;

typedef struct pa_handle pa_handle;

/*
 * Validates cfg, selects the kernels, and allocates the workspace on the
 * current HIP device.  Rules checked before any HIP call (PA_ERR_INVALID_ARG):
 * H, Hkv > 0 and H % Hkv == 0; 0 < Dk, Dv <= 576; block_size > 0,
 * block_size % 16 == 0, block_size <= 256, and block_size <= 128 in causal
 * mode or when Dk or Dv > 256; window sizes in [0, 2^30] in band mode;
 * a non-NULL mask_tensor in tensor mode; topk > 0 in sparse mode; num_blocks > 0; max_batch > 0;
 * max_num_blocks_per_seq > 0; max_q_seq_len > 0; dtype and mask in range;
 * scale finite; num_partitions >= 0; only PA_FLAG_* bits, not FORCE_VALU
 * with FORCE_MFMA; Dv <= Dk with PA_FLAG_SHARED_KV.  PA_ERR_UNSUPPORTED: a (Dk, Dv) pair this
 * build has no kernels for (64/64, 128/128, 256/256, 576/512 are built),
 * PA_FLAG_FORCE_VALU with any mask other than PA_MASK_NONE, sparse mode
 * unless head_num / kv_head_num is a multiple of 64 (the matrix-core tiles
 * of 64 rows must each hold one query token) and topk <= 2048 (a list is
 * resolved to cache rows in LDS), or a device that is not gfx950.  On success *out receives the handle.
 */
pa_status pa_create(const pa_config *cfg, pa_handle **out);

/*
 * One forward pass, enqueued on `stream` (a hipStream_t; NULL = the null
 * stream).  All tensors are device pointers, row-major, contiguous:
 *   query        [num_q_tokens, H, Dk]  dtype   (TND, rows of sequence b contiguous)
 *   key_cache    [num_blocks, block_size, Hkv, Dk]  dtype
 *   value_cache  [num_blocks, block_size, Hkv, Dv]  dtype; with PA_FLAG_SHARED_KV it must be
 *                NULL or equal to key_cache, and V_j is elements [0, Dv) of key_cache's row
 *                for token j (the single K/V cache of the SparseAttnSharedkvMetadata page,
 *                function and parameter sections, with the MLA head sizes 576 / 512 of the
 *                PagedAttentionOperation Constraints: V is the leading part of the K row)
 *   block_tables [batch, max_num_blocks_per_seq]  int32
 *   context_lens [batch]  int32   (kvSeqLen: history + current query tokens)
 *   q_seq_lens   [batch]  int32, or NULL for one query token per sequence
 *   out          [num_q_tokens, H, Dv]  dtype   (written)
 *   lse          [num_q_tokens, H]  float32, or NULL   (written)
 * batch in [0, max_batch]; max_q_seq_len in [1, cfg.max_q_seq_len] bounds
 * q_seq_lens (1 when q_seq_lens is NULL); num_q_tokens >= 0 equals the sum of
 * q_seq_lens (batch when NULL).  Returns PA_ERR_INVALID_ARG for a NULL
 * handle or tensor (q_seq_lens, lse, and value_cache under PA_FLAG_SHARED_KV
 * excepted), a value_cache other than NULL or key_cache under
 * PA_FLAG_SHARED_KV, a NULL q_seq_lens with
 * num_q_tokens != batch, or sizes out of range; PA_ERR_HIP if a launch fails.
 */
pa_status pa_forward(pa_handle *h, const void *query, const void *key_cache,
                     const void *value_cache, const int32_t *block_tables,
                     const int32_t *context_lens, const int32_t *q_seq_lens, int32_t batch,
                     int32_t num_q_tokens, int32_t max_q_seq_len, void *out, float *lse,
                     void *stream);

/*
 * The sparse mode (PA_MASK_SPARSE handles only; pa_forward refuses them and
 * this call refuses other handles, PA_ERR_INVALID_ARG).  The compressed-KV
 * stream of the SparseAttnSharedkvMetadata README (parameter table: cmp_kv,
 * cmp_topk selected tokens -- 512 there -- under mask mode 3,
 * rightDownCausal): the caches hold the compressed tokens and context_lens
 * counts them; every query token t and KV head g carries a list
 *   topk_indices [num_q_tokens, Hkv, cfg.topk]  int32 (device)
 * of token indices.  Row i of sequence b (query head h, KV head g) attends
 * over the listed tokens c with 0 <= c < context_lens[b] and c <= prefix + i
 * (prefix = max(0, context_lens[b] - q_seq_lens[b]): the causal mask aligned
 * at the bottom right of the query x compressed-token matrix); other
 * entries (such as -1 padding of a short list) are skipped, and each
 * remaining entry contributes once (lists from a selector hold distinct
 * indices).  A row without a remaining entry gets out = 0, lse = -inf.
 * Every other argument and rule is pa_forward's.
 */
pa_status pa_forward_sparse(pa_handle *h, const void *query, const void *key_cache, const void *value_cache,
                            const int32_t *block_tables, const int32_t *context_lens, const int32_t *q_seq_lens,
                            const int32_t *topk_indices, int32_t batch, int32_t num_q_tokens, int32_t max_q_seq_len,
                            void *out, float *lse, void *stream);

/* Bytes of the static device array that holds pa_forward_noalloc's workspace on each GPU. */
#define PA_NOALLOC_SCRATCH_BYTES ((int64_t)64 << 20)

/*
 * For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: pa_forward
 * without a handle.  cfg is checked as pa_create checks it (same statuses,
 * before any HIP call); the other arguments are pa_forward's.  The pass runs
 * the kernels, pieces and merge order that pa_forward runs on a handle
 * created from cfg, so the outputs agree bit for bit.  Sparse-list
 * configurations are refused (PA_ERR_INVALID_ARG), as pa_forward refuses
 * them.
 *
 * The workspace (plan arrays, split entries, fp32 partials, piece counter,
 * error word, zero page) is laid out for this pass in a static device array
 * of PA_NOALLOC_SCRATCH_BYTES that each GPU the library runs on holds until
 * the process ends; nothing is allocated or freed.  The first call on a
 * device looks up that device's array and properties; later calls do no
 * set-up.  Each call clears the piece counter, the error word and the zero
 * page with a small fill kernel on `stream` (no memset), then enqueues the
 * pass; it does not synchronise.  PA_ERR_SCRATCH: the pass needs more than
 * the array holds (the partials grow with the partitions, the rows per tile
 * and Dv, the plan arrays with the batch); a smaller cfg.num_partitions or
 * PA_FLAG_STATIC_PIECES (no claimed tail) makes the pass smaller.  Device-data
 * errors are clamped as in pa_forward; the error word is not reported.
 *
 * Every call on one GPU uses that GPU's one array, which keeps the last
 * call's contents: calls that overlap in time on the same GPU (two streams,
 * or two host threads) race on it, and the caller must order them.
 */
pa_status pa_forward_noalloc(const pa_config *cfg, const void *query, const void *key_cache,
                             const void *value_cache, const int32_t *block_tables, const int32_t *context_lens,
                             const int32_t *q_seq_lens, int32_t batch, int32_t num_q_tokens, int32_t max_q_seq_len,
                             void *out, float *lse, void *stream);

/* Frees the workspace and the handle (synchronises the device first).  NULL is a no-op. */
pa_status pa_destroy(pa_handle *h);

/* A static English description of a status code. */
const char *pa_status_string(pa_status s);

/*
 * Reads the device error word (PA_DEVERR_* bits accumulated since the last
 * clear) into *code, then clears it if `clear` is non-zero.  Synchronises the
 * device.
 */
pa_status pa_get_device_error(pa_handle *h, uint32_t *code, int32_t clear);

/*
 * Per-kernel timing for measurement.  While enabled, pa_forward launches
 * each of its kernels (plan, attention, merge) with a pair of HIP events on
 * its stream that take the kernel's own start and end timestamps
 * (hipExtLaunchKernel; no marker packets are added between the kernels).
 * pa_read_timing synchronises, adds up the elapsed times of all recorded
 * passes since the last read into ms[3] (plan, attention, merge) and the
 * number of passes into *count, and resets the totals.  A pass whose
 * attention kernel planned for itself launches no plan kernel: ms[0] sums
 * the passes that launched one, and *plan_launches (if not NULL) receives
 * their number; a pass without split entries launches no merge kernel and
 * counts 0 for it.  If per_pass_cap > 0, per_pass_ms (host, 3 * per_pass_cap
 * doubles) receives (plan, attention, merge) of each of the first
 * per_pass_cap passes, plan = -1 for a pass without a plan kernel.  At most
 * 1024 passes are kept between reads; later ones are not timed.
 */
pa_status pa_set_timing(pa_handle *h, int32_t enable);
pa_status pa_read_timing(pa_handle *h, double ms[3], int32_t *count, int32_t *plan_launches, double *per_pass_ms,
                         int32_t per_pass_cap);

/*
 * Measurement support, not part of the forward pass: a plain streaming read
 * of `bytes` (> 0, a multiple of 16) at the device address src, enqueued on
 * `stream`.  Each of `workgroups` workgroups reads one contiguous share with
 * 16-byte loads and writes one word of sink (device, uint32 [workgroups]).
 * The rate it reaches is the device's read ceiling for whole-buffer
 * streaming, which the attention kernels' HBM bandwidth is set beside.
 * PA_ERR_INVALID_ARG for a NULL pointer or a bad size; PA_ERR_HIP if the
 * launch fails.
 */
pa_status pa_read_probe(const void *src, int64_t bytes, uint32_t *sink, int32_t workgroups, void *stream);

/*
 * What pa_create chose, for logging and tests: *path is 0 for the VALU decode
 * kernel, 1 for the MFMA tile kernel, 2 for the MFMA streaming kernel (units
 * of at most 16 rows), for a call with that max_q_seq_len (at most
 * cfg.max_q_seq_len); *rows_per_tile and *tokens_per_chunk describe its work
 * unit; *partitions is the number of workers a split pass launches.  A pass
 * may launch fewer: a sparse-list pass at most max(CUs, two per (sequence,
 * KV head, row tile)), and a pass whose units run whole (band units of a few
 * chunks, decode passes whose block tables hold at most 8 chunks per
 * sequence, PA_FLAG_NO_SPLIT) one workgroup per unit.
 */
pa_status pa_describe(const pa_handle *h, int32_t max_q_seq_len, int32_t *path,
                      int32_t *rows_per_tile, int32_t *tokens_per_chunk, int32_t *partitions);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */

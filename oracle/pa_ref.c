/*
 * pa_ref.c -- the oracle for the paged-attention forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark use it.  It shares no code, header, table or helper with
 * the HIP library; it converts fp16/bf16 bit patterns itself and computes
 * every row in double precision, in the plainest order: gather, dot
 * products, max, exponentials, sum, weighted sum of V.
 *
 * What it computes (one row = one query token i of sequence b, one query
 * head h):
 *
 *   out[t0+i][h][e] = sum_j w_j * V_j[e] / sum_j w_j,
 *   w_j = exp(z_j - max_j z_j),   z_j = scale * <q[t0+i][h], K_j>,
 *   lse[t0+i][h]    = max_j z_j + log(sum_j w_j)
 *
 * over the visible KV tokens j of sequence b.  Sources for each step:
 *
 *  - Token j of sequence b lives in physical block block_tables[b][j / bs],
 *    slot j % bs.  Every block-table entry lies in [0, num_blocks), and
 *    max_num_blocks_per_seq >= ceil(max(contextLens) / block_size)
 *    (Ascend ATB "PagedAttentionOperation", Constraints).  The caches are
 *    [num_blocks, block_size, kvHeadNum, head_size] (the BSND/ND layout named
 *    in the same list and the PA_ND kv layout of the SparseAttnSharedkvMetadata
 *    README, parameter table).
 *  - GQA: headNum > kvHeadNum and headNum % kvHeadNum == 0 (PagedAttention
 *    Constraints; SelfAttentionOperation Restrictions).  The pages give only
 *    the divisibility; query head h reads KV head h / (headNum / kvHeadNum)
 *    (contiguous groups), which is the reading this oracle takes.
 *  - scale is one scalar multiplying q.k (scaleType TOR, PagedAttention
 *    Constraints, mask type 5 list).
 *  - Mask "none" (maskType UNDEFINED): every row sees all contextLens[b]
 *    tokens (PagedAttention Constraints, mask-type selection).
 *  - Mask "causal" (parallel decoding / splitfuse, mask type 5): contextLens
 *    counts history plus the current query tokens, prefix =
 *    max(0, kvSeqLen - qSeqLen), and the mask is the standard causal mask --
 *    upper triangle without the diagonal invisible -- aligned at prefix, so
 *    row i sees tokens j <= prefix + i (PagedAttention Constraints, mask
 *    type 5 list).  Invisible tokens get weight exactly 0; with the pages'
 *    suggested fill of -10000 the additive form underflows to the same 0.
 *  - Mask "band" (mask mode 4 of the SparseAttnSharedkvMetadata README,
 *    parameter table, with win_left past tokens and win_right future tokens
 *    per query; the page fixes 127 and 0): the query row i sits at position
 *    prefix + i of its sequence, aligned as in the causal rule, and sees
 *    tokens prefix + i - win_left <= j <= prefix + i + win_right, j < kv.
 *    win_left counts the tokens before the query's own position, which is
 *    itself visible (the page is silent on the query's own token; this is
 *    the plain reading of a count of past tokens).
 *  - Mask "tensor" (the shared compressed mask of mask type 5: one fp16
 *    [2048, 2048] matrix for all sequences and heads, 0 where visible and a
 *    large negative value such as -10000 above the diagonal; the operator
 *    aligns it with prefix = max(0, kvSeqLen - qSeqLen) and adapts to
 *    sequences longer than 2048 -- PagedAttention Constraints, mask type 5
 *    list): the matrix is added to the scaled scores, row i of a sequence
 *    against token j reading element [i][j - prefix].  History tokens
 *    (j < prefix) are visible with nothing added.  Outside the matrix
 *    (i >= 2048 or j - prefix >= 2048) the causal rule holds: visible with
 *    nothing added if j - prefix <= i, invisible otherwise.  (The reading
 *    of the alignment: the prefix shifts the columns, so the matrix covers
 *    the current query tokens whatever the history length; for the pages'
 *    triangular matrix every alignment gives the causal mask.)
 *  - Mask "sparse" (the compressed-KV stream of the SparseAttnSharedkvMetadata
 *    README, parameter table: cmp_kv, the compression of ori_kv, from which
 *    an index selector keeps cmp_topk tokens, 512 there, under mask mode 3,
 *    rightDownCausal): the cache holds the compressed tokens, contextLens
 *    counts them, and every query token t of sequence b carries, per KV
 *    head g, a list of topk indices into them.  Row i of b (query head h,
 *    KV head g) attends over the listed tokens c with 0 <= c < kv and
 *    c <= prefix + i -- the causal mask aligned at the bottom right of the
 *    (query, compressed token) matrix, as rightDownCausal reads.  Entries
 *    outside that range (e.g. -1 padding of a short list) are skipped; every
 *    other entry contributes once (a selector's list holds distinct
 *    indices; a repeated entry would count twice).  The selector itself
 *    is not described on the page; its lists are inputs here.
 *  - Query/output rows are packed (TND): sequence b's rows start at
 *    t0 = q_seq_lens[0] + ... + q_seq_lens[b-1], the prefix-sum convention of
 *    cu_seqlens_q (SparseAttnSharedkvMetadata README, parameter table).
 *  - A row with no visible token gets out = 0 and lse = -inf (the pages are
 *    silent; this is the limit of an empty softmax taken here).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { REF_F16 = 0, REF_BF16 = 1 };
enum { REF_MASK_NONE = 0, REF_MASK_CAUSAL = 1, REF_MASK_BAND = 2, REF_MASK_TENSOR = 3, REF_MASK_SPARSE = 4 };
enum { REF_MASK_DIM = 2048 };   /* the shared mask matrix is REF_MASK_DIM x REF_MASK_DIM */
enum { REF_OK = 0, REF_BAD_ARG = -1, REF_BAD_BLOCK = -2, REF_BAD_LEN = -3, REF_NO_MEM = -4 };

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double from_f16_bits(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 31;
    int frac = h & 1023;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24);              /* subnormal: frac * 2^-24 */
    else if (expo == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + frac), expo - 25); /* (1 + frac/2^10) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16: the upper 16 bits of an IEEE binary32. */
static double from_bf16_bits(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* The value of every fp16 bit pattern, filled once from from_f16_bits (the
 * decoding stays that function; the table only saves recomputing it, which
 * with two ldexp calls per element made fp16 problems ~8x slower than bf16). */
static double f16_value[65536];
static pthread_once_t f16_value_once = PTHREAD_ONCE_INIT;

static void fill_f16_values(void)
{
    for (uint32_t u = 0; u < 65536u; ++u)
        f16_value[u] = from_f16_bits((uint16_t)u);
}

static double elem(const uint16_t *p, int64_t i, int dtype)
{
    return dtype == REF_F16 ? f16_value[p[i]] : from_bf16_bits(p[i]);
}

typedef struct {
    const uint16_t *query, *key_cache, *value_cache;
    const int32_t *block_tables, *context_lens, *q_seq_lens;
    int32_t batch, num_q_tokens, head_num, kv_head_num, head_size_k, head_size_v;
    int32_t block_size, max_num_blocks_per_seq;
    int64_t num_blocks;
    int32_t dtype, mask;
    double scale;
    int32_t win_left, win_right;   /* band mask only */
    const uint16_t *mask_tensor;   /* tensor mask only: fp16 [REF_MASK_DIM][REF_MASK_DIM] */
    const int32_t *topk_idx;       /* sparse only: [num_q_tokens][kv_head_num][topk] */
    int32_t topk;
    int64_t *row_start;  /* [batch + 1]: first packed query row of each sequence */
} problem;

/* One output row: sequence b, query position i, query head h; the result
 * goes to o[0 .. head_size_v) and *lse. */
static int one_row(const problem *P, int b, int i, int h, double *z, double *o, double *lse)
{
    const int H = P->head_num, Hkv = P->kv_head_num, Dk = P->head_size_k, Dv = P->head_size_v;
    const int bs = P->block_size;
    const int group = H / Hkv;
    const int g = h / group;
    const int64_t t = P->row_start[b] + i;
    const int qlen = P->q_seq_lens ? P->q_seq_lens[b] : 1;
    const int kv = P->context_lens[b];
    const int prefix = kv - qlen > 0 ? kv - qlen : 0;
    /* the visible tokens are lo, lo + 1, ..., hi - 1 */
    int64_t lo = 0, hi = kv;
    if (P->mask == REF_MASK_CAUSAL && prefix + i + 1 < hi)
        hi = prefix + i + 1;
    if (P->mask == REF_MASK_BAND) {
        const int64_t pos = (int64_t)prefix + i;    /* the query's own position */
        if (pos - P->win_left > lo)
            lo = pos - P->win_left;
        if (pos + 1 + P->win_right < hi)
            hi = pos + 1 + P->win_right;
    }
    int n = hi > lo ? (int)(hi - lo) : 0;
    /* sparse: the entries of the row's list instead of a token range */
    const int32_t *list = NULL;
    if (P->mask == REF_MASK_SPARSE) {
        list = P->topk_idx + (t * Hkv + g) * (int64_t)P->topk;
        n = P->topk;
    }

    const uint16_t *q = P->query + (t * H + h) * (int64_t)Dk;
    for (int j = 0; j < n; ++j) {
        const int tok = list ? list[j] : (int)lo + j;
        if (list && (tok < 0 || tok >= kv || tok > prefix + i)) {   /* skipped entry */
            z[j] = -INFINITY;
            continue;
        }
        int32_t phys = P->block_tables[(int64_t)b * P->max_num_blocks_per_seq + tok / bs];
        if (phys < 0 || phys >= P->num_blocks)
            return REF_BAD_BLOCK;
        int slot = tok % bs;
        const int64_t krow = (((int64_t)phys * bs + slot) * Hkv + g) * Dk;
        double dot = 0.0;
        for (int d = 0; d < Dk; ++d)
            dot += elem(q, d, P->dtype) * elem(P->key_cache, krow + d, P->dtype);
        z[j] = P->scale * dot;
        if (P->mask == REF_MASK_TENSOR) {
            const int64_t c = (int64_t)tok - prefix;   /* column of the shifted mask */
            if (c >= 0 && c < REF_MASK_DIM && i < REF_MASK_DIM)
                z[j] += from_f16_bits(P->mask_tensor[(int64_t)i * REF_MASK_DIM + c]);
            else if (c > i)
                z[j] = -INFINITY;                     /* causal rule outside the matrix */
        }
    }

    double zmax = -INFINITY;
    for (int j = 0; j < n; ++j)
        if (z[j] > zmax)
            zmax = z[j];
    if (n == 0 || zmax == -INFINITY) {   /* no visible token */
        for (int e = 0; e < Dv; ++e)
            o[e] = 0.0;
        *lse = -INFINITY;
        return REF_OK;
    }
    double wsum = 0.0;
    for (int j = 0; j < n; ++j) {
        z[j] = exp(z[j] - zmax);    /* z now holds the unnormalised weight */
        wsum += z[j];
    }
    for (int e = 0; e < Dv; ++e)
        o[e] = 0.0;
    /* V row of token j: its own tensor, or (no value_cache) the first Dv
     * elements of the token's K row.  The SparseAttnSharedkvMetadata page
     * (function and parameter sections) feeds an attention whose K and V are
     * one cache with one head count; with the MLA head sizes (576 for K, 512
     * for V) the plain reading is that V is the leading part of the K row. */
    const uint16_t *vsrc = P->value_cache ? P->value_cache : P->key_cache;
    const int vstride = P->value_cache ? Dv : Dk;
    for (int j = 0; j < n; ++j) {
        const int tok = list ? list[j] : (int)lo + j;
        if (list && (tok < 0 || tok >= kv || tok > prefix + i))    /* skipped entry */
            continue;
        int32_t phys = P->block_tables[(int64_t)b * P->max_num_blocks_per_seq + tok / bs];
        int slot = tok % bs;
        const int64_t vrow = (((int64_t)phys * bs + slot) * Hkv + g) * vstride;
        for (int e = 0; e < Dv; ++e)
            o[e] += z[j] * elem(vsrc, vrow + e, P->dtype);
    }
    for (int e = 0; e < Dv; ++e)
        o[e] /= wsum;
    *lse = zmax + log(wsum);
    return REF_OK;
}

/* Work list shared by the threads: rows are claimed in order by index;
 * item k writes out[out_index[k] * head_size_v ...] and lse[out_index[k]]. */
typedef struct {
    const problem *P;
    const int32_t *row_seq, *row_pos, *row_head;  /* per work item */
    const int64_t *out_index;
    int64_t n_items;
    double *out, *lse;
    int64_t next;
    int status;
    pthread_mutex_t lock;
    int max_kv;
} work;

static void *worker(void *arg)
{
    work *W = (work *)arg;
    double *z = (double *)malloc(sizeof(double) * (size_t)(W->max_kv > 0 ? W->max_kv : 1));
    if (!z) {
        pthread_mutex_lock(&W->lock);
        W->status = REF_NO_MEM;
        pthread_mutex_unlock(&W->lock);
        return NULL;
    }
    for (;;) {
        pthread_mutex_lock(&W->lock);
        int64_t k = W->next++;
        int stop = W->status != REF_OK;
        pthread_mutex_unlock(&W->lock);
        if (stop || k >= W->n_items)
            break;
        int64_t slot = W->out_index[k];
        int rc = one_row(W->P, W->row_seq[k], W->row_pos[k], W->row_head[k], z,
                         W->out + slot * W->P->head_size_v, W->lse + slot);
        if (rc != REF_OK) {
            pthread_mutex_lock(&W->lock);
            W->status = rc;
            pthread_mutex_unlock(&W->lock);
        }
    }
    free(z);
    return NULL;
}

static int run_items(const problem *P, const int32_t *seq, const int32_t *pos, const int32_t *head,
                     const int64_t *out_index, int64_t n_items, double *out, double *lse,
                     int num_threads)
{
    int max_kv = 0;
    for (int b = 0; b < P->batch; ++b)
        if (P->context_lens[b] > max_kv)
            max_kv = P->context_lens[b];
    work W;
    memset(&W, 0, sizeof W);
    W.P = P;
    W.row_seq = seq;
    W.row_pos = pos;
    W.row_head = head;
    W.out_index = out_index;
    W.n_items = n_items;
    W.out = out;
    W.lse = lse;
    W.max_kv = P->mask == REF_MASK_SPARSE && P->topk > max_kv ? P->topk : max_kv;
    pthread_mutex_init(&W.lock, NULL);
    if (num_threads < 1)
        num_threads = 1;
    if (num_threads > 512)
        num_threads = 512;
    pthread_t tid[512];
    int started = 0;
    for (int k = 1; k < num_threads; ++k)
        if (pthread_create(&tid[started], NULL, worker, &W) == 0)
            ++started;
    worker(&W);
    for (int k = 0; k < started; ++k)
        pthread_join(tid[k], NULL);
    pthread_mutex_destroy(&W.lock);
    return W.status;
}

/* Checks the problem description; fills P->row_start (caller frees). */
static int setup(problem *P)
{
    pthread_once(&f16_value_once, fill_f16_values);
    if (!P->query || !P->key_cache || !P->block_tables || !P->context_lens)
        return REF_BAD_ARG;
    if (!P->value_cache && P->head_size_v > P->head_size_k)   /* V rows inside K rows */
        return REF_BAD_ARG;
    if (P->batch < 0 || P->head_num <= 0 || P->kv_head_num <= 0 || P->head_size_k <= 0 ||
        P->head_size_v <= 0 || P->block_size <= 0 || P->max_num_blocks_per_seq < 0 ||
        P->num_blocks < 0 || P->head_num % P->kv_head_num != 0 ||
        (P->dtype != REF_F16 && P->dtype != REF_BF16) ||
        (P->mask != REF_MASK_NONE && P->mask != REF_MASK_CAUSAL && P->mask != REF_MASK_BAND &&
         P->mask != REF_MASK_TENSOR && P->mask != REF_MASK_SPARSE) ||
        P->win_left < 0 || P->win_right < 0 || (P->mask == REF_MASK_TENSOR && !P->mask_tensor) ||
        (P->mask == REF_MASK_SPARSE && (!P->topk_idx || P->topk <= 0)))
        return REF_BAD_ARG;
    P->row_start = (int64_t *)malloc(sizeof(int64_t) * (size_t)(P->batch + 1));
    if (!P->row_start)
        return REF_NO_MEM;
    P->row_start[0] = 0;
    for (int b = 0; b < P->batch; ++b) {
        int qlen = P->q_seq_lens ? P->q_seq_lens[b] : 1;
        int kv = P->context_lens[b];
        if (qlen < 0 || kv < 0 || (int64_t)(kv + P->block_size - 1) / P->block_size >
                                      P->max_num_blocks_per_seq) {
            free(P->row_start);
            return REF_BAD_LEN;
        }
        P->row_start[b + 1] = P->row_start[b] + qlen;
    }
    if (P->row_start[P->batch] != P->num_q_tokens) {
        free(P->row_start);
        return REF_BAD_LEN;
    }
    return REF_OK;
}

#define PROBLEM_ARGS                                                                           \
    const uint16_t *query, const uint16_t *key_cache, const uint16_t *value_cache,             \
        const int32_t *block_tables, const int32_t *context_lens, const int32_t *q_seq_lens,   \
        int32_t batch, int32_t num_q_tokens, int32_t head_num, int32_t kv_head_num,            \
        int32_t head_size_k, int32_t head_size_v, int32_t block_size, int64_t num_blocks,      \
        int32_t max_num_blocks_per_seq, int32_t dtype, int32_t mask, double scale,            \
        int32_t win_left, int32_t win_right, const uint16_t *mask_tensor,                      \
        const int32_t *topk_idx, int32_t topk

#define FILL_PROBLEM(P)                                                                        \
    do {                                                                                       \
        memset(&(P), 0, sizeof(P));                                                            \
        (P).query = query; (P).key_cache = key_cache; (P).value_cache = value_cache;           \
        (P).block_tables = block_tables; (P).context_lens = context_lens;                      \
        (P).q_seq_lens = q_seq_lens; (P).batch = batch; (P).num_q_tokens = num_q_tokens;       \
        (P).head_num = head_num; (P).kv_head_num = kv_head_num;                                \
        (P).head_size_k = head_size_k; (P).head_size_v = head_size_v;                          \
        (P).block_size = block_size; (P).num_blocks = num_blocks;                              \
        (P).max_num_blocks_per_seq = max_num_blocks_per_seq; (P).dtype = dtype;                \
        (P).mask = mask; (P).scale = scale;                                                    \
        (P).win_left = win_left; (P).win_right = win_right;                                    \
        (P).mask_tensor = mask_tensor; (P).topk_idx = topk_idx; (P).topk = topk;               \
    } while (0)

/*
 * All rows.  out: [num_q_tokens, head_num, head_size_v] doubles; lse:
 * [num_q_tokens, head_num] doubles.  q_seq_lens NULL means one query token
 * per sequence.  Returns 0, or a negative REF_* code on bad input (nothing
 * is read out of bounds).
 */
int pa_ref_forward(PROBLEM_ARGS, double *out, double *lse, int num_threads)
{
    problem P;
    FILL_PROBLEM(P);
    int rc = setup(&P);
    if (rc != REF_OK)
        return rc;
    int64_t n_items = (int64_t)num_q_tokens * head_num;
    int32_t *seq = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n_items + 1));
    int32_t *pos = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n_items + 1));
    int32_t *head = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n_items + 1));
    int64_t *slot = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n_items + 1));
    if (!seq || !pos || !head || !slot) {
        free(seq); free(pos); free(head); free(slot); free(P.row_start);
        return REF_NO_MEM;
    }
    int64_t k = 0;
    for (int b = 0; b < batch; ++b)
        for (int64_t t = P.row_start[b]; t < P.row_start[b + 1]; ++t)
            for (int h = 0; h < head_num; ++h) {
                seq[k] = b;
                pos[k] = (int32_t)(t - P.row_start[b]);
                head[k] = h;
                slot[k] = t * head_num + h;
                ++k;
            }
    rc = run_items(&P, seq, pos, head, slot, n_items, out, lse, num_threads);
    free(seq); free(pos); free(head); free(slot); free(P.row_start);
    return rc;
}

/*
 * Selected rows only: row k is (packed query token row_token[k], query head
 * row_head[k]); its result goes to out[k * head_size_v ...] and lse[k].
 */
int pa_ref_rows(PROBLEM_ARGS, int64_t n_rows, const int32_t *row_token, const int32_t *row_head,
                double *out, double *lse, int num_threads)
{
    problem P;
    FILL_PROBLEM(P);
    int rc = setup(&P);
    if (rc != REF_OK)
        return rc;
    int32_t *seq = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n_rows + 1));
    int32_t *pos = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n_rows + 1));
    int64_t *slot = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n_rows + 1));
    if (!seq || !pos || !slot) {
        free(seq); free(pos); free(slot); free(P.row_start);
        return REF_NO_MEM;
    }
    for (int64_t k = 0; k < n_rows; ++k) {
        int32_t t = row_token[k];
        if (t < 0 || t >= num_q_tokens || row_head[k] < 0 || row_head[k] >= head_num) {
            free(seq); free(pos); free(slot); free(P.row_start);
            return REF_BAD_ARG;
        }
        int lo = 0, hi = batch - 1;   /* the last b with row_start[b] <= t owns row t */
        while (lo < hi) {
            int mid = (lo + hi + 1) / 2;
            if (P.row_start[mid] <= t)
                lo = mid;
            else
                hi = mid - 1;
        }
        seq[k] = lo;
        pos[k] = (int32_t)(t - P.row_start[lo]);
        slot[k] = k;
    }
    rc = run_items(&P, seq, pos, row_head, slot, n_rows, out, lse, num_threads);
    free(seq); free(pos); free(slot); free(P.row_start);
    return rc;
}

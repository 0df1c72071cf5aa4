/*
 * pkv_oracle.c -- plain, slow, obviously-correct CPU oracle for paged-KV
 * grouped-query attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or
 * calls this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg do.  It shares no code, header, table or helper with the HIP
 * library: it is written from the pages' text alone.
 *
 * Sources (cited by page title and the part of the page):
 *   [P1] "nx_f32_attn_paged.nx source" -- header comment (offset-causal rule
 *        q_pos = total_k - n_q + i, GQA grouping, the output scatter, the
 *        ensure/append/advance caller contract), the error constants, and the
 *        body of nx_f32_attn_with_paged (argument checks, append, total_k,
 *        per-head gather through the page table, multi-query core, scatter).
 *   [P2] "nx_f32_gqa_attention.nx source" -- header comment (Qwen3-4B 32:8
 *        head sharing, kv head = h / group), nx_f32_gqa_attention and its
 *        inline self-test (Q = 0 worked example, bad grouping).
 *   [P3] "nx_f32_llama_v4b.nx source" -- batched decode: ensure_append for
 *        every sequence before any layer, one row per sequence with n_q = 1
 *        and causal = 1, advance for every sequence after all layers.
 *   [P4] "nx_paged_kv_gate.nx source" -- the gate: pool known-answer test,
 *        paged == contiguous, fork with copy-on-append, truncate rewind.
 *
 * Arithmetic: every score, exponential and weighted sum is carried in
 * double precision; each output element is rounded once to float at the
 * end.  The products of two floats are exact in double.
 *
 * Readings of what the pages leave open (the pool module itself is not on
 * the pages) are listed beside the functions that make them.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Status codes.  0..3 are the four constants of [P1]; 4..6 extend them for
 * failures the pages do not name. */
enum {
    O_OK = 0,
    O_BAD_DIM = 1,
    O_BAD_GQA = 2,
    O_ERR_SEQ = 3,
    O_OOM = 4,
    O_CAPACITY = 5,
    O_BAD_ARG = 6
};

/* ------------------------------------------------------------------------ */
/* The attention definition.                                                  */
/* ------------------------------------------------------------------------ */

/*
 * attend -- softmax(Q K^T * scale) V for every query head, written into the
 * [n_q, n_heads * head_dim] output ([P1] scatter; [P2] same layout).
 *
 * krow[j] / vrow[j] point at key/value row j (j < total_k) of width
 * n_kv_heads * head_dim: kv head c occupies elements [c*head_dim, (c+1)*head_dim).
 * Query head h reads kv head h / (n_heads / n_kv_heads) ([P1] body, [P2]).
 * Query i sits at position total_k - n_q + i ([P1] header); with causal set
 * it sees keys 0..q_pos, otherwise all total_k keys.
 */
static void attend(const float *Q, const float *const *krow,
                   const float *const *vrow, int n_q, int total_k,
                   int n_heads, int n_kv_heads, int head_dim, int causal,
                   float scale, float *out)
{
    const int group = n_heads / n_kv_heads;
    const int q_dim = n_heads * head_dim;
    double *s = (double *)malloc(sizeof(double) * (size_t)total_k);
    double *acc = (double *)malloc(sizeof(double) * (size_t)head_dim);

    for (int h = 0; h < n_heads; h++) {
        const int kvh = h / group;
        for (int i = 0; i < n_q; i++) {
            const int q_pos = total_k - n_q + i;
            const int vis = causal ? q_pos + 1 : total_k;
            const float *q = Q + (size_t)i * q_dim + (size_t)h * head_dim;

            /* scores: (q . k_j) * scale */
            double m = -INFINITY;
            for (int j = 0; j < vis; j++) {
                const float *k = krow[j] + (size_t)kvh * head_dim;
                double dot = 0.0;
                for (int d = 0; d < head_dim; d++)
                    dot += (double)q[d] * (double)k[d];
                s[j] = dot * (double)scale;
                if (s[j] > m)
                    m = s[j];
            }

            /* softmax weights e_j = exp(s_j - max), normaliser l = sum e_j */
            double l = 0.0;
            for (int j = 0; j < vis; j++) {
                s[j] = exp(s[j] - m);
                l += s[j];
            }

            /* weighted sum of values, divided by l, rounded once to float */
            for (int d = 0; d < head_dim; d++)
                acc[d] = 0.0;
            for (int j = 0; j < vis; j++) {
                const float *v = vrow[j] + (size_t)kvh * head_dim;
                for (int d = 0; d < head_dim; d++)
                    acc[d] += s[j] * (double)v[d];
            }
            float *o = out + (size_t)i * q_dim + (size_t)h * head_dim;
            for (int d = 0; d < head_dim; d++)
                o[d] = (float)(acc[d] / l);
        }
    }
    free(s);
    free(acc);
}

/*
 * pkvo_attn_contig -- the definition over explicit contiguous histories.
 * K, V: [total_k, n_kv_heads * head_dim]; Q, out: [n_q, n_heads * head_dim].
 * Argument checks follow [P1]'s order: dims, then grouping.
 */
int pkvo_attn_contig(const float *Q, const float *K, const float *V, int n_q,
                     int total_k, int n_heads, int n_kv_heads, int head_dim,
                     int causal, float scale, float *out)
{
    if (n_q <= 0 || n_heads <= 0 || n_kv_heads <= 0 || head_dim <= 0)
        return O_BAD_DIM;
    if (n_heads % n_kv_heads != 0)
        return O_BAD_GQA;
    if (total_k < n_q)
        return O_BAD_DIM;
    const int kv_dim = n_kv_heads * head_dim;
    const float **kr = (const float **)malloc(sizeof(float *) * (size_t)total_k);
    const float **vr = (const float **)malloc(sizeof(float *) * (size_t)total_k);
    for (int j = 0; j < total_k; j++) {
        kr[j] = K + (size_t)j * kv_dim;
        vr[j] = V + (size_t)j * kv_dim;
    }
    attend(Q, kr, vr, n_q, total_k, n_heads, n_kv_heads, head_dim, causal,
           scale, out);
    free(kr);
    free(vr);
    return O_OK;
}

/*
 * pkvo_gqa_attention -- [P2]'s nx_f32_gqa_attention: one chunk of n_tokens
 * rows attending to itself with no mask and no cache.  Its only failure is
 * a kv-head count that is non-positive or does not divide the query heads,
 * reported as 1.
 */
int pkvo_gqa_attention(const float *Q, const float *K, const float *V,
                       int n_tokens, int n_q_heads, int n_kv_heads,
                       int head_dim, float scale, float *out)
{
    if (n_kv_heads <= 0)
        return 1;
    if (n_q_heads % n_kv_heads != 0)
        return 1;
    if (n_tokens <= 0 || n_q_heads <= 0 || head_dim <= 0)
        return 1;
    return pkvo_attn_contig(Q, K, V, n_tokens, n_tokens, n_q_heads,
                            n_kv_heads, head_dim, 0, scale, out) == O_OK ? 0 : 1;
}

/* ------------------------------------------------------------------------ */
/* Rotary position embedding applied before the append and the attention.   */
/* ------------------------------------------------------------------------ */

/*
 * pkvo_rope -- [P3] (nx_f32_llama_block_forward_v4b, the RoPE step before
 * attention): when rotary embedding is on, every query head and every kv
 * head of the new rows is rotated in the "neox" form at the row's position
 * (the sequence's current length for a decode row, that length + t for
 * token t of a chunk) before K is appended and Q attends.  The page names
 * the form and passes a "log base" but does not spell out the rotation; the
 * reading taken is the standard neox rotary embedding with log_base the
 * natural logarithm of the rotary base: with half = D / 2 and frequency
 * inv_i = exp(-(2 i / D) * log_base), the pair (x_i, x_{i+half}) turns by
 * the angle pos * inv_i,
 *   x_i'        = x_i cos - x_{i+half} sin
 *   x_{i+half}' = x_i sin + x_{i+half} cos,
 * evaluated in double and rounded once to float.  x: [n_rows, n_heads *
 * head_dim], rotated in place; positions[r] is row r's position (>= 0).
 */
int pkvo_rope(float *x, int n_rows, int n_heads, int head_dim,
              const int *positions, double log_base)
{
    if (n_rows <= 0 || n_heads <= 0 || head_dim <= 0 || head_dim % 2 != 0)
        return O_BAD_DIM;
    if (!(log_base > 0.0))
        return O_BAD_ARG;
    for (int r = 0; r < n_rows; r++)
        if (positions[r] < 0)
            return O_BAD_ARG;
    const int half = head_dim / 2;
    for (int r = 0; r < n_rows; r++) {
        for (int h = 0; h < n_heads; h++) {
            float *v = x + ((size_t)r * n_heads + h) * head_dim;
            for (int i = 0; i < half; i++) {
                const double inv = exp(-((double)(2 * i) / head_dim) * log_base);
                const double ang = (double)positions[r] * inv;
                const double c = cos(ang), s = sin(ang);
                const double a = v[i], b = v[i + half];
                v[i] = (float)(a * c - b * s);
                v[i + half] = (float)(a * s + b * c);
            }
        }
    }
    return O_OK;
}

/* ------------------------------------------------------------------------ */
/* Contiguous cache: the twin that [P1] and [P4] compare the pool against.   */
/* ------------------------------------------------------------------------ */

typedef struct {
    int n_layers, n_kv_heads, max_seq, head_dim;
    int seq_len;
    float *k, *v; /* [layer][pos][kv_dim] */
} OCache;

OCache *pkvo_cache_new(int n_layers, int n_kv_heads, int max_seq, int head_dim)
{
    if (n_layers <= 0 || n_kv_heads <= 0 || max_seq <= 0 || head_dim <= 0)
        return NULL;
    OCache *c = (OCache *)calloc(1, sizeof(OCache));
    c->n_layers = n_layers;
    c->n_kv_heads = n_kv_heads;
    c->max_seq = max_seq;
    c->head_dim = head_dim;
    size_t n = (size_t)n_layers * max_seq * n_kv_heads * head_dim;
    c->k = (float *)calloc(n, sizeof(float));
    c->v = (float *)calloc(n, sizeof(float));
    return c;
}

void pkvo_cache_free(OCache *c)
{
    if (!c)
        return;
    free(c->k);
    free(c->v);
    free(c);
}

int pkvo_cache_len(const OCache *c) { return c ? c->seq_len : -1; }

/* seq_len += n once per step, after all layers ([P1] caller contract). */
int pkvo_cache_advance(OCache *c, int n)
{
    if (!c)
        return O_ERR_SEQ;
    if (n <= 0)
        return O_BAD_DIM;
    if (c->seq_len + n > c->max_seq)
        return O_CAPACITY;
    c->seq_len += n;
    return O_OK;
}

/*
 * pkvo_attn_with_cache -- per layer: write the n new K/V rows at positions
 * seq_len.. of that layer, then attend over seq_len + n keys.
 */
int pkvo_attn_with_cache(const float *Q, const float *K_new,
                         const float *V_new, int n_tokens, int n_heads,
                         int n_kv_heads, int head_dim, OCache *c, int layer,
                         int causal, float scale, float *out)
{
    if (n_tokens <= 0 || n_heads <= 0 || n_kv_heads <= 0 || head_dim <= 0)
        return O_BAD_DIM;
    if (n_heads % n_kv_heads != 0)
        return O_BAD_GQA;
    if (!c)
        return O_ERR_SEQ;
    if (n_kv_heads != c->n_kv_heads || head_dim != c->head_dim)
        return O_BAD_DIM;
    if (layer < 0 || layer >= c->n_layers)
        return O_BAD_ARG;
    if (c->seq_len + n_tokens > c->max_seq)
        return O_ERR_SEQ;
    const int kv_dim = n_kv_heads * head_dim;
    float *kl = c->k + (size_t)layer * c->max_seq * kv_dim;
    float *vl = c->v + (size_t)layer * c->max_seq * kv_dim;
    memcpy(kl + (size_t)c->seq_len * kv_dim, K_new,
           sizeof(float) * (size_t)n_tokens * kv_dim);
    memcpy(vl + (size_t)c->seq_len * kv_dim, V_new,
           sizeof(float) * (size_t)n_tokens * kv_dim);
    return pkvo_attn_contig(Q, kl, vl, n_tokens, c->seq_len + n_tokens,
                            n_heads, n_kv_heads, head_dim, causal, scale, out);
}

/* ------------------------------------------------------------------------ */
/* The paged pool.                                                            */
/*                                                                            */
/* The pool module is only named on the pages; what they show of it is:     */
/*  - pool_new(n_blocks, n_layers, kv_dim); a fresh pool hands out block ids */
/*    0, 1, 2, ..., -1 once exhausted, and a released id is handed out again  */
/*    ([P4] known-answer test);                                               */
/*  - a per-block reference count; forking a sequence shares its blocks and  */
/*    raises their count to 2; after both forks append, the block written by */
/*    each is private again with count 1 ([P4] fork part);                   */
/*  - truncation back to an earlier length releases references ([P4] header */
/*    "truncate unref"), and appending after it reproduces the other fork    */
/*    bit for bit ([P4] rewind part);                                         */
/*  - ensure_append reserves room and privatises shared blocks before any   */
/*    layer appends ([P1] caller contract, [P3] stack function).            */
/* Readings taken where the pages are silent:                                */
/*  - the block size is a pool parameter;                                    */
/*  - free ids form a LIFO stack, initially ordered so pops give 0,1,2,...;   */
/*  - only a shared block that the next append will write is copied (copy   */
/*    on append); copies happen in ensure_append, per sequence in batch      */
/*    order, ascending page index, before that sequence's new pages;         */
/*  - ensure_append pre-counts the ids it will take over the whole batch and */
/*    fails with OOM before changing anything if the free stack is short;    */
/*  - truncate and free release pages from the last page backwards;          */
/*  - fork shares exactly ceil(seq_len / block_size) pages;                  */
/*  - sequence ids are small integers; the lowest unused id is taken.        */
/* ------------------------------------------------------------------------ */

typedef struct {
    int alive;
    int seq_len;
    int max_tokens;
    int n_pages;
    int64_t *pt; /* capacity ceil(max_tokens / block_size) */
} OSeq;

typedef struct {
    int n_blocks, block_size, n_layers, n_kv_heads, head_dim, max_seqs;
    int *refcnt;
    int64_t *free_stack; /* top of stack at index n_free - 1 */
    int n_free;
    float *k, *v; /* NULL for a metadata-only pool; [block][layer][slot][kv_dim] */
    OSeq *seqs;
} OPool;

static int ceil_div(int a, int b) { return (a + b - 1) / b; }

static size_t block_floats(const OPool *p)
{
    return (size_t)p->n_layers * p->block_size * p->n_kv_heads * p->head_dim;
}

OPool *pkvo_pool_new(int n_blocks, int block_size, int n_layers,
                     int n_kv_heads, int head_dim, int max_seqs,
                     int with_storage)
{
    if (n_blocks <= 0 || block_size <= 0 || n_layers <= 0 || n_kv_heads <= 0 ||
        head_dim <= 0 || max_seqs <= 0)
        return NULL;
    OPool *p = (OPool *)calloc(1, sizeof(OPool));
    p->n_blocks = n_blocks;
    p->block_size = block_size;
    p->n_layers = n_layers;
    p->n_kv_heads = n_kv_heads;
    p->head_dim = head_dim;
    p->max_seqs = max_seqs;
    p->refcnt = (int *)calloc((size_t)n_blocks, sizeof(int));
    p->free_stack = (int64_t *)calloc((size_t)n_blocks, sizeof(int64_t));
    for (int i = 0; i < n_blocks; i++)
        p->free_stack[i] = n_blocks - 1 - i; /* pops yield 0, 1, 2, ... */
    p->n_free = n_blocks;
    p->seqs = (OSeq *)calloc((size_t)max_seqs, sizeof(OSeq));
    if (with_storage) {
        size_t n = (size_t)n_blocks * block_floats(p);
        p->k = (float *)calloc(n, sizeof(float));
        p->v = (float *)calloc(n, sizeof(float));
        if (!p->k || !p->v) {
            free(p->k);
            free(p->v);
            free(p->refcnt);
            free(p->free_stack);
            free(p->seqs);
            free(p);
            return NULL;
        }
    }
    return p;
}

void pkvo_pool_free(OPool *p)
{
    if (!p)
        return;
    for (int s = 0; s < p->max_seqs; s++)
        free(p->seqs[s].pt);
    free(p->seqs);
    free(p->refcnt);
    free(p->free_stack);
    free(p->k);
    free(p->v);
    free(p);
}

/* Pop a free id and give it one reference; -1 when none is left. */
int64_t pkvo_alloc_block(OPool *p)
{
    if (p->n_free == 0)
        return -1;
    int64_t id = p->free_stack[--p->n_free];
    p->refcnt[id] = 1;
    return id;
}

/* Drop one reference; at zero the id goes back on the free stack. */
static void drop_ref(OPool *p, int64_t id)
{
    p->refcnt[id] -= 1;
    if (p->refcnt[id] == 0)
        p->free_stack[p->n_free++] = id;
}

/* Number of page-table entries, over all live sequences, that name id. */
static int page_table_holders(const OPool *p, int64_t id)
{
    int n = 0;
    for (int s = 0; s < p->max_seqs; s++) {
        const OSeq *q = &p->seqs[s];
        if (!q->alive)
            continue;
        for (int pg = 0; pg < q->n_pages; pg++)
            if (q->pt[pg] == id)
                n++;
    }
    return n;
}

/*
 * [P4] KAT part: a block handed out by alloc_block is given back with
 * unref_block and its id is recycled.  Reading: unref_block releases only
 * such references -- the block's count minus the page-table entries that
 * name it; those are released by truncate and free.  Anything else (an id
 * out of range, a free id, a block whose remaining references are all page
 * table entries) is refused with BAD_ARG and changes nothing.
 */
int pkvo_unref_block(OPool *p, int64_t id)
{
    if (id < 0 || id >= p->n_blocks)
        return O_BAD_ARG;
    if (p->refcnt[id] - page_table_holders(p, id) <= 0)
        return O_BAD_ARG;
    drop_ref(p, id);
    return O_OK;
}

/*
 * Reorder the free stack so the next pops return ids[0], ids[1], ...
 * ids must be a permutation of exactly the ids that are free now.
 */
int pkvo_set_free_order(OPool *p, const int64_t *ids, int n)
{
    if (n != p->n_free)
        return O_BAD_ARG;
    char *seen = (char *)calloc((size_t)p->n_blocks, 1);
    for (int i = 0; i < n; i++) {
        int64_t b = ids[i];
        if (b < 0 || b >= p->n_blocks || p->refcnt[b] != 0 || seen[b]) {
            free(seen);
            return O_BAD_ARG;
        }
        seen[b] = 1;
    }
    free(seen);
    for (int i = 0; i < n; i++)
        p->free_stack[n - 1 - i] = ids[i];
    return O_OK;
}

static OSeq *get_seq(OPool *p, int s)
{
    if (s < 0 || s >= p->max_seqs || !p->seqs[s].alive)
        return NULL;
    return &p->seqs[s];
}

static int lowest_free_seq(const OPool *p)
{
    for (int s = 0; s < p->max_seqs; s++)
        if (!p->seqs[s].alive)
            return s;
    return -1;
}

/* A new empty sequence that may grow to max_tokens rows. */
int pkvo_seq_new(OPool *p, int max_tokens)
{
    if (max_tokens <= 0)
        return -O_BAD_ARG;
    int s = lowest_free_seq(p);
    if (s < 0)
        return -O_CAPACITY;
    OSeq *q = &p->seqs[s];
    free(q->pt);
    q->pt = (int64_t *)calloc((size_t)ceil_div(max_tokens, p->block_size),
                              sizeof(int64_t));
    q->alive = 1;
    q->seq_len = 0;
    q->max_tokens = max_tokens;
    q->n_pages = 0;
    return s;
}

/* Release pages from the last one back to page keep, then set the length. */
static void release_tail(OPool *p, OSeq *q, int keep)
{
    for (int pg = q->n_pages - 1; pg >= keep; pg--)
        drop_ref(p, q->pt[pg]);
    if (q->n_pages > keep)
        q->n_pages = keep;
}

/* [P4] rewind: truncate to new_len (0 <= new_len <= seq_len). */
int pkvo_seq_truncate(OPool *p, int s, int new_len)
{
    OSeq *q = get_seq(p, s);
    if (!q)
        return O_ERR_SEQ;
    if (new_len < 0 || new_len > q->seq_len)
        return O_BAD_ARG;
    release_tail(p, q, ceil_div(new_len, p->block_size));
    q->seq_len = new_len;
    return O_OK;
}

int pkvo_seq_free(OPool *p, int s)
{
    OSeq *q = get_seq(p, s);
    if (!q)
        return O_ERR_SEQ;
    release_tail(p, q, 0);
    q->seq_len = 0;
    q->alive = 0;
    return O_OK;
}

/* [P4] fork: the child shares every written page; each gains a reference. */
int pkvo_seq_fork(OPool *p, int s)
{
    OSeq *src = get_seq(p, s);
    if (!src)
        return -O_ERR_SEQ;
    int c = lowest_free_seq(p);
    if (c < 0)
        return -O_CAPACITY;
    OSeq *dst = &p->seqs[c];
    free(dst->pt);
    dst->pt = (int64_t *)calloc((size_t)ceil_div(src->max_tokens, p->block_size),
                                sizeof(int64_t));
    dst->alive = 1;
    dst->seq_len = src->seq_len;
    dst->max_tokens = src->max_tokens;
    dst->n_pages = ceil_div(src->seq_len, p->block_size);
    for (int pg = 0; pg < dst->n_pages; pg++) {
        dst->pt[pg] = src->pt[pg];
        p->refcnt[src->pt[pg]] += 1;
    }
    return c;
}

/* All ids valid, alive and pairwise distinct. */
static int check_batch(OPool *p, const int *seqs, int M)
{
    for (int r = 0; r < M; r++) {
        if (!get_seq(p, seqs[r]))
            return O_ERR_SEQ;
        for (int r2 = 0; r2 < r; r2++)
            if (seqs[r2] == seqs[r])
                return O_ERR_SEQ;
    }
    return O_OK;
}

/*
 * ensure_append -- make room for n more rows in every sequence of the batch
 * and make every page those rows will land in private.
 * For each sequence, in batch order: every existing page in the write range
 * [seq_len / B, ceil((seq_len + n) / B)) that is shared is replaced by a
 * fresh copy (ascending page order); then fresh pages are appended until
 * ceil((seq_len + n) / B) pages exist.  The ids needed are counted first by
 * running the same steps on a scratch copy of the reference counts, and if
 * the free stack is short nothing is changed.
 */
int pkvo_ensure_append(OPool *p, const int *seqs, int M, int n)
{
    if (M <= 0 || n <= 0)
        return O_BAD_DIM;
    int rc = check_batch(p, seqs, M);
    if (rc)
        return rc;
    for (int r = 0; r < M; r++) {
        OSeq *q = get_seq(p, seqs[r]);
        if (q->seq_len + n > q->max_tokens)
            return O_CAPACITY;
    }
    const int B = p->block_size;
    int *tmp = (int *)malloc(sizeof(int) * (size_t)p->n_blocks);
    memcpy(tmp, p->refcnt, sizeof(int) * (size_t)p->n_blocks);
    long need = 0;
    for (int r = 0; r < M; r++) {
        OSeq *q = get_seq(p, seqs[r]);
        int first = q->seq_len / B;
        int want = ceil_div(q->seq_len + n, B);
        for (int pg = first; pg < want && pg < q->n_pages; pg++) {
            if (tmp[q->pt[pg]] > 1) {
                tmp[q->pt[pg]] -= 1;
                need += 1;
            }
        }
        if (want > q->n_pages)
            need += want - q->n_pages;
    }
    free(tmp);
    if (need > p->n_free)
        return O_OOM;

    const size_t bf = block_floats(p);
    for (int r = 0; r < M; r++) {
        OSeq *q = get_seq(p, seqs[r]);
        int first = q->seq_len / B;
        int want = ceil_div(q->seq_len + n, B);
        for (int pg = first; pg < want && pg < q->n_pages; pg++) {
            int64_t old = q->pt[pg];
            if (p->refcnt[old] > 1) {
                int64_t fresh = pkvo_alloc_block(p);
                if (p->k) {
                    memcpy(p->k + (size_t)fresh * bf, p->k + (size_t)old * bf,
                           sizeof(float) * bf);
                    memcpy(p->v + (size_t)fresh * bf, p->v + (size_t)old * bf,
                           sizeof(float) * bf);
                }
                p->refcnt[old] -= 1;
                q->pt[pg] = fresh;
            }
        }
        while (q->n_pages < want)
            q->pt[q->n_pages++] = pkvo_alloc_block(p);
    }
    return O_OK;
}

/* Row (seq s, layer, position pos) of the store; pos must be < n_pages*B. */
static float *row_ptr(float *base, const OPool *p, const OSeq *q, int layer,
                      int pos)
{
    const int B = p->block_size;
    const int64_t blk = q->pt[pos / B];
    const size_t kv_dim = (size_t)p->n_kv_heads * p->head_dim;
    return base + (size_t)blk * block_floats(p) +
           ((size_t)layer * B + (size_t)(pos % B)) * kv_dim;
}

/*
 * append_layer -- write row t of sequence seqs[r] (input row r*n + t) at
 * position seq_len + t of the given layer.  Every target page must exist
 * (ensure_append ran) and be private.
 */
int pkvo_append_layer(OPool *p, const int *seqs, int M, int n, int layer,
                      const float *K_new, const float *V_new)
{
    if (M <= 0 || n <= 0)
        return O_BAD_DIM;
    int rc = check_batch(p, seqs, M);
    if (rc)
        return rc;
    if (layer < 0 || layer >= p->n_layers)
        return O_BAD_ARG;
    const int B = p->block_size;
    for (int r = 0; r < M; r++) {
        OSeq *q = get_seq(p, seqs[r]);
        if (q->seq_len + n > q->n_pages * B)
            return O_ERR_SEQ;
        for (int pg = q->seq_len / B; pg < ceil_div(q->seq_len + n, B); pg++)
            if (p->refcnt[q->pt[pg]] != 1)
                return O_ERR_SEQ;
    }
    if (!p->k)
        return O_OK; /* metadata-only pool */
    const size_t kv_dim = (size_t)p->n_kv_heads * p->head_dim;
    for (int r = 0; r < M; r++) {
        OSeq *q = get_seq(p, seqs[r]);
        for (int t = 0; t < n; t++) {
            memcpy(row_ptr(p->k, p, q, layer, q->seq_len + t),
                   K_new + ((size_t)r * n + t) * kv_dim, sizeof(float) * kv_dim);
            memcpy(row_ptr(p->v, p, q, layer, q->seq_len + t),
                   V_new + ((size_t)r * n + t) * kv_dim, sizeof(float) * kv_dim);
        }
    }
    return O_OK;
}

/* seq_len += n for every sequence, once per step after all layers. */
int pkvo_advance(OPool *p, const int *seqs, int M, int n)
{
    if (M <= 0 || n <= 0)
        return O_BAD_DIM;
    int rc = check_batch(p, seqs, M);
    if (rc)
        return rc;
    for (int r = 0; r < M; r++) {
        OSeq *q = get_seq(p, seqs[r]);
        if (q->seq_len + n > q->max_tokens)
            return O_CAPACITY;
        if (q->seq_len + n > q->n_pages * p->block_size)
            return O_ERR_SEQ;
    }
    for (int r = 0; r < M; r++)
        get_seq(p, seqs[r])->seq_len += n;
    return O_OK;
}

/*
 * attn_paged -- for each row r: attend sequence seqs[r]'s n_q newest rows
 * (already appended, not yet advanced) over seq_len + n_q keys of `layer`,
 * gathered through its page table.  Q and out are [M * n_q, n_heads*head_dim]
 * with row r*n_q + i for query i of sequence seqs[r].
 */
int pkvo_attn_paged(OPool *p, const int *seqs, int M, int n_q, int layer,
                    int n_heads, int n_kv_heads, int head_dim, const float *Q,
                    int causal, float scale, float *out)
{
    if (M <= 0 || n_q <= 0 || n_heads <= 0 || n_kv_heads <= 0 || head_dim <= 0)
        return O_BAD_DIM;
    if (n_heads % n_kv_heads != 0)
        return O_BAD_GQA;
    if (n_kv_heads != p->n_kv_heads || head_dim != p->head_dim)
        return O_BAD_DIM;
    int rc = check_batch(p, seqs, M);
    if (rc)
        return rc;
    if (layer < 0 || layer >= p->n_layers)
        return O_BAD_ARG;
    if (!p->k)
        return O_BAD_ARG;
    for (int r = 0; r < M; r++) {
        OSeq *q = get_seq(p, seqs[r]);
        if (q->seq_len + n_q > q->n_pages * p->block_size)
            return O_ERR_SEQ;
    }
    const size_t q_dim = (size_t)n_heads * head_dim;
    for (int r = 0; r < M; r++) {
        OSeq *q = get_seq(p, seqs[r]);
        const int total_k = q->seq_len + n_q;
        const float **kr = (const float **)malloc(sizeof(float *) * (size_t)total_k);
        const float **vr = (const float **)malloc(sizeof(float *) * (size_t)total_k);
        for (int j = 0; j < total_k; j++) {
            kr[j] = row_ptr(p->k, p, q, layer, j);
            vr[j] = row_ptr(p->v, p, q, layer, j);
        }
        attend(Q + (size_t)r * n_q * q_dim, kr, vr, n_q, total_k, n_heads,
               n_kv_heads, head_dim, causal, scale, out + (size_t)r * n_q * q_dim);
        free(kr);
        free(vr);
    }
    return O_OK;
}

/*
 * pkvo_attn_with_paged -- [P1]'s nx_f32_attn_with_paged for one sequence:
 * checks in the page's order, append this layer's rows (failure -> 3), then
 * attend.
 */
int pkvo_attn_with_paged(const float *Q, const float *K_new,
                         const float *V_new, int n_tokens, int n_heads,
                         int n_kv_heads, int head_dim, OPool *p, int seq,
                         int layer, int causal, float scale, float *out)
{
    if (n_tokens <= 0 || n_heads <= 0 || n_kv_heads <= 0 || head_dim <= 0)
        return O_BAD_DIM;
    if (n_heads % n_kv_heads != 0)
        return O_BAD_GQA;
    if (!get_seq(p, seq))
        return O_ERR_SEQ;
    if (pkvo_append_layer(p, &seq, 1, n_tokens, layer, K_new, V_new) != O_OK)
        return O_ERR_SEQ;
    return pkvo_attn_paged(p, &seq, 1, n_tokens, layer, n_heads, n_kv_heads,
                           head_dim, Q, causal, scale, out);
}

/* ------------------------------------------------------------------------ */
/* Introspection, for state comparisons.                                     */
/* ------------------------------------------------------------------------ */

int pkvo_seq_len(OPool *p, int s)
{
    OSeq *q = get_seq(p, s);
    return q ? q->seq_len : -O_ERR_SEQ;
}

/* Copies up to cap page ids; returns the page count (or a negative code). */
int pkvo_seq_pages(OPool *p, int s, int64_t *out, int cap)
{
    OSeq *q = get_seq(p, s);
    if (!q)
        return -O_ERR_SEQ;
    for (int i = 0; i < q->n_pages && i < cap; i++)
        out[i] = q->pt[i];
    return q->n_pages;
}

int pkvo_refcounts(OPool *p, int32_t *out)
{
    for (int b = 0; b < p->n_blocks; b++)
        out[b] = p->refcnt[b];
    return p->n_blocks;
}

/* Free stack from bottom to top (the last element pops first). */
int pkvo_free_stack(OPool *p, int64_t *out, int cap)
{
    for (int i = 0; i < p->n_free && i < cap; i++)
        out[i] = p->free_stack[i];
    return p->n_free;
}

/* Logical row (layer, pos) of sequence s, both K and V (kv_dim floats). */
int pkvo_read_row(OPool *p, int s, int layer, int pos, float *k_out,
                  float *v_out)
{
    OSeq *q = get_seq(p, s);
    if (!q)
        return O_ERR_SEQ;
    if (!p->k || layer < 0 || layer >= p->n_layers || pos < 0 ||
        pos >= q->n_pages * p->block_size)
        return O_BAD_ARG;
    const size_t kv_dim = (size_t)p->n_kv_heads * p->head_dim;
    memcpy(k_out, row_ptr(p->k, p, q, layer, pos), sizeof(float) * kv_dim);
    memcpy(v_out, row_ptr(p->v, p, q, layer, pos), sizeof(float) * kv_dim);
    return O_OK;
}

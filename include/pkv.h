/*
 * pkv.h -- C ABI of libpkv: paged-KV grouped-query attention on AMD MI355X
 * (gfx950).
 *
 * What it computes.  A refcounted pool of fixed-size KV blocks holds the K
 * and V rows of many sequences; each sequence reads its rows back through a
 * page table of block ids.  Per layer, new K/V rows are appended, then query
 * head h attends with kv head h / (n_heads / n_kv_heads) over all cached rows
 * plus the new ones, query i sitting at position total_k - n_q + i
 * (offset-causal), and softmax(Q K^T * scale) V is written into an
 * [n_q, n_heads * head_dim] output.  ("nx_f32_attn_paged.nx source": header
 * comment and nx_f32_attn_with_paged; "nx_f32_gqa_attention.nx source":
 * header comment.)
 *
 * Step protocol ("nx_f32_attn_paged.nx source", caller contract in the header
 * comment; "nx_f32_llama_v4b.nx source", nx_f32_llama_stack_forward_v4b):
 *   pkv_ensure_append(batch, n)            once per step, before layer 0
 *   for each layer:
 *     pkv_append_layer(batch, n, layer, K_new, V_new)
 *     pkv_attn_paged_decode(...)           (n == 1)  or
 *     pkv_attn_paged_prefill(..., n_q = n)
 *     (for n == 1 both lines may be one pkv_attn_with_paged_decode(...))
 *   pkv_advance(batch, n)                  once per step, after all layers
 *
 * Conventions.
 *  - Status returns: 0 = OK, otherwise a PKV_ERR_* code.  Functions that
 *    return an id return it (>= 0) or the negated status code.
 *  - Every argument check runs before any state change or device work: a
 *    call that fails leaves the pool exactly as it was.
 *  - Pointers named *_dev are device pointers; all other pointers are host
 *    pointers.  The caller owns every buffer it passes and keeps device
 *    buffers alive until the work enqueued on `stream` has finished.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    All device work of one pool must go to one stream at a time; a call that
 *    names a different stream than the pool's previous call first waits for
 *    the previous stream to drain.
 *  - Host-side metadata changes when the call returns; device work is
 *    enqueued on `stream` and ordered with the caller's other work there.
 *  - A pool is not thread-safe: one host thread at a time per pool.
 *  - pool == NULL is rejected first with PKV_ERR_BAD_ARG (negated where the
 *    function returns an id).
 *  - All floating-point data is IEEE float32.
 *
 * Device layouts.
 *  - Pool storage: block-major [n_blocks][n_layers][2 (K,V)][n_kv_heads]
 *    [block_size][head_dim] float32 (pkv_pool_storage_bytes bytes).
 *  - Q and out rows: [rows, n_heads * head_dim]; head h occupies columns
 *    [h * head_dim, (h + 1) * head_dim).
 *  - K_new / V_new rows: [rows, n_kv_heads * head_dim].
 *  - Batched calls take `seqs[M]`; for n rows per sequence, input row
 *    r * n + t belongs to token t of sequence seqs[r].
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes.  0..3 are the four codes of "nx_f32_attn_paged.nx source"
 * (the NX_F32_AP_* constants); 4..8 name failures the pages do not. */
#define PKV_OK 0
#define PKV_ERR_BAD_DIM 1     /* a size <= 0, or head shape != the pool's  */
#define PKV_ERR_BAD_GQA 2     /* n_heads not a multiple of n_kv_heads      */
#define PKV_ERR_SEQ 3         /* bad/absent/duplicate sequence id, or rows
                                 not ensured / target block shared         */
#define PKV_ERR_OOM 4         /* not enough free blocks                     */
#define PKV_ERR_CAPACITY 5    /* beyond a sequence's max_tokens, or no
                                 free sequence id                           */
#define PKV_ERR_BAD_ARG 6     /* other bad argument (layer range, truncate
                                 length, unknown block, buffer too small,
                                 NULL pointer, metadata-only pool)          */
#define PKV_ERR_DEVICE 7      /* a HIP runtime call failed                  */
#define PKV_ERR_UNSUPPORTED 8 /* shape outside what the kernels handle      */
#define PKV_ERR_STATE 9       /* a debug state check failed (pkv_pool_set_checks) */

typedef struct pkv_pool pkv_pool;
typedef struct pkv_rope pkv_rope;

/* Human-readable name of a status code (static string). */
const char *pkv_strerror(int32_t code);

/* ------------------------------------------------------------------------ */
/* Pool and blocks                                                           */
/* ------------------------------------------------------------------------ */

/* Bytes of device storage a pool of this shape needs (0 on bad sizes).
 * ("nx_paged_kv_gate.nx source": nx_pkv_pool_new(n_blocks, n_layers, kv_dim);
 * the block size, hidden there, is an explicit parameter here.) */
size_t pkv_pool_storage_bytes(int32_t n_blocks, int32_t block_size,
                              int32_t n_layers, int32_t n_kv_heads,
                              int32_t head_dim);

/* Create a pool.  storage_dev (>= pkv_pool_storage_bytes bytes, 256-byte
 * aligned) is borrowed, never freed; the caller keeps it alive until
 * pkv_pool_free.  storage_dev == NULL makes a metadata-only pool: every
 * block, sequence and page-table call works and no device work is ever
 * done; pkv_append_layer runs its checks and then does nothing, and the
 * attention calls return PKV_ERR_BAD_ARG.  max_seqs bounds the number of
 * live sequence ids; the device page-table mirror gives each id at least 64
 * int32-addressed entries, so max_seqs * 64 must not exceed 2^31 - 1.
 * Makes no HIP call.  Returns NULL on a size <= 0, max_seqs too large,
 * storage_bytes below pkv_pool_storage_bytes, storage_dev not 256-byte
 * aligned, or host memory exhausted.
 * A fresh pool hands out block ids 0, 1, 2, ... in that order. */
pkv_pool *pkv_pool_new(int32_t n_blocks, int32_t block_size, int32_t n_layers,
                       int32_t n_kv_heads, int32_t head_dim, int32_t max_seqs,
                       void *storage_dev, size_t storage_bytes);

/* Wait for the pool's device work, then free its host metadata and the
 * small device/pinned buffers the library allocated for it. */
void pkv_pool_free(pkv_pool *pool);

/* Take a free block with one reference; -1 when none is free.
 * ("nx_paged_kv_gate.nx source", KAT part: ids 0,1,2 then -1 on a pool of 3;
 * a released id is handed out again.) */
int64_t pkv_alloc_block(pkv_pool *pool);

/* Debug state checks before device work, for hunting a corrupted pool
 * (they cost host time; off by default).  level 0: none.  level 1: before
 * every pkv_ensure_append copy launch, pkv_append_layer and attention call
 * (metadata-only pools included, for pkv_ensure_append and
 * pkv_append_layer), the host state the launch relies on: every page id of
 * the batch's rows in range, each block's reference count at least the
 * page-table entries naming it (which are at least one), every block new rows
 * land in held by its sequence alone, copy-on-append targets fresh; and the
 * batch's row descriptors and pending page-table patches, as built for the
 * device, against the host page tables and lengths.  level 2: also, before
 * each attention launch, the device page-table mirror rows of the batch are
 * read back (synchronizing the stream) and compared with the host page
 * tables.  A failed check returns PKV_ERR_STATE and launches nothing for
 * that call (host metadata a pkv_ensure_append has already changed stays
 * changed: a failure means the state was inconsistent).  PKV_ERR_BAD_ARG for
 * a level outside 0..2.  (The invariants are those of
 * "nx_paged_kv_gate.nx source": reference counts that follow the page tables
 * through fork, copy-on-append and truncate.) */
int32_t pkv_pool_set_checks(pkv_pool *pool, int32_t level);

/* Give back a reference taken by pkv_alloc_block; at zero the id returns to
 * the free stack, from which the most recently released id is taken first
 * ("nx_paged_kv_gate.nx source", KAT part: a released id is handed out
 * again).  Only such references can be dropped here: a block's count minus
 * the page-table entries that name it (those are released by
 * pkv_seq_truncate and pkv_seq_free).  PKV_ERR_BAD_ARG, with nothing
 * changed, for an id out of range, a free id, or a block whose remaining
 * references all belong to page tables. */
int32_t pkv_unref_block(pkv_pool *pool, int64_t id);

/* Placement control: afterwards, allocations return ids[0], ids[1], ... in
 * that order.  ids[0..n) must be a permutation of exactly the currently free
 * ids (PKV_ERR_BAD_ARG, with nothing changed, otherwise).  Used to scatter
 * sequences' pages across the pool with a seeded permutation. */
int32_t pkv_pool_set_free_order(pkv_pool *pool, const int64_t *ids,
                                int32_t n);

/* ------------------------------------------------------------------------ */
/* Rotary position embedding                                                 */
/*                                                                            */
/* "nx_f32_llama_v4b.nx source", nx_f32_llama_block_forward_v4b, RoPE step:  */
/* with rotary embedding on, every query head and every kv head of the new   */
/* rows is turned in the neox form at the row's position -- the sequence's   */
/* length for a decode row, length + t for token t of a chunk -- before K is */
/* appended and Q attends.  Here the turn is fused into the kernels: K rows  */
/* are turned inside pkv_append_layer's scatter (the pool stores turned K),  */
/* queries at load inside the attention kernels; V is never turned.  Pair    */
/* (x_i, x_{i + head_dim/2}) turns by pos * exp(-(2 i / head_dim) *          */
/* log_base) radians (log_base = ln of the rotary base, the page's           */
/* rope_log_base):                                                           */
/*   x_i' = x_i cos - x_{i+half} sin,  x_{i+half}' = x_i sin + x_{i+half} cos */
/* in double, rounded once to float.                                         */
/* ------------------------------------------------------------------------ */

/* Build the rotary table (cos, sin in double, [max_positions][head_dim / 2],
 * 8 * head_dim * max_positions bytes) on the current HIP device.  Returns
 * NULL for head_dim <= 0 or odd, log_base not finite and > 0,
 * max_positions <= 0, or a HIP failure.  Free with pkv_rope_free once no
 * pool or contiguous cache that names it has work left in flight. */
pkv_rope *pkv_rope_new(int32_t head_dim, double log_base,
                       int32_t max_positions);
void pkv_rope_free(pkv_rope *rope);

/* Turn rotary embedding on for the pool with this table (borrowed: it must
 * outlive the pool's use of it), or off with rope == NULL.  It applies to
 * every later pkv_append_layer (K) and attention call (Q); switch it only
 * between steps.  Errors: BAD_ARG (pool NULL), BAD_DIM (table head_dim !=
 * the pool's).  While on, a call whose rows reach position max_positions
 * or beyond fails with PKV_ERR_CAPACITY before any device work. */
int32_t pkv_pool_set_rope(pkv_pool *pool, const pkv_rope *rope);

/* ------------------------------------------------------------------------ */
/* Sequences                                                                 */
/* ------------------------------------------------------------------------ */

/* New empty sequence that may hold up to max_tokens rows; returns the lowest
 * unused id, -PKV_ERR_BAD_ARG for max_tokens <= 0, -PKV_ERR_CAPACITY when
 * max_seqs ids are live or when the device page-table mirror could not
 * address the new page table with int32 offsets: max_seqs times the longest
 * page table of any sequence (ceil(max_tokens / block_size), rounded up to a
 * multiple of 64) must not exceed 2^31 - 1.  Nothing changes on an error.
 * ("nx_paged_kv_gate.nx source": nx_pkv_seq_new.) */
int32_t pkv_seq_new(pkv_pool *pool, int32_t max_tokens);

/* Release every page of the sequence (last page first) and retire its id. */
int32_t pkv_seq_free(pkv_pool *pool, int32_t seq);

/* New sequence sharing the first ceil(seq_len / block_size) pages of `seq`;
 * each shared block gains one reference.  Returns the new id or a negated
 * code.  ("nx_paged_kv_gate.nx source", FORK part: the shared first block
 * has reference count 2.) */
int32_t pkv_seq_fork(pkv_pool *pool, int32_t seq);

/* Rewind to new_len rows (0 <= new_len <= seq_len, else PKV_ERR_BAD_ARG):
 * pages past ceil(new_len / block_size) are released, last page first.
 * ("nx_paged_kv_gate.nx source": header "truncate unref" and REWIND part.) */
int32_t pkv_seq_truncate(pkv_pool *pool, int32_t seq, int32_t new_len);

/* ------------------------------------------------------------------------ */
/* Step protocol                                                             */
/* ------------------------------------------------------------------------ */

/* Reserve room for n_new rows in every sequence of seqs[0..M) and make every
 * block those rows will land in private.  Per sequence, in batch order:
 * each existing page in [seq_len / B, ceil((seq_len + n_new) / B)) whose
 * block is shared is replaced by a fresh copy (ascending page order; the
 * copy is enqueued on `stream`), then fresh pages are added until
 * ceil((seq_len + n_new) / B) exist.  The ids this takes over the whole
 * batch are counted first; if fewer are free, PKV_ERR_OOM and nothing
 * changes.  Errors: BAD_DIM (M or n_new <= 0), SEQ (bad or repeated id),
 * CAPACITY (seq_len + n_new > max_tokens), OOM.
 * ("nx_f32_attn_paged.nx source", caller contract; "nx_f32_llama_v4b.nx
 * source", the capacity + copy-on-write loop before the layers.) */
int32_t pkv_ensure_append(pkv_pool *pool, const int32_t *seqs, int32_t M,
                          int32_t n_new, void *stream);

/* Write K_new_dev / V_new_dev rows [M * n_new, n_kv_heads * head_dim] at
 * positions seq_len .. seq_len + n_new - 1 of `layer` for each sequence
 * (one coalesced scatter kernel).  Errors, in this order: BAD_DIM (M or
 * n_new <= 0), SEQ (bad or repeated id), BAD_ARG (layer out of range), SEQ
 * (rows not ensured, or a target block shared), CAPACITY (rotary table too
 * short), BAD_ARG (NULL pointer).  With rotary embedding on, K rows are
 * stored turned at their positions.
 * ("nx_f32_attn_paged.nx source": nx_pkv_append_layer in
 * nx_f32_attn_with_paged, step 1.) */
int32_t pkv_append_layer(pkv_pool *pool, const int32_t *seqs, int32_t M,
                         int32_t n_new, int32_t layer, const float *K_new_dev,
                         const float *V_new_dev, void *stream);

/* seq_len += n for every sequence, once per step after all layers.
 * Errors: BAD_DIM, SEQ (bad id, or beyond the ensured pages), CAPACITY.
 * ("nx_f32_llama_v4b.nx source": nx_pkv_advance after the layer loop.) */
int32_t pkv_advance(pkv_pool *pool, const int32_t *seqs, int32_t M,
                    int32_t n);

/* ------------------------------------------------------------------------ */
/* Attention                                                                 */
/* ------------------------------------------------------------------------ */

/* Device workspace bytes pkv_attn_paged_decode needs for this batch (split
 * partial results); depends only on each sequence's length and n_heads.
 * Returns 0 if no workspace is needed, (size_t)-1 on bad arguments. */
size_t pkv_decode_workspace_bytes(pkv_pool *pool, const int32_t *seqs,
                                  int32_t M, int32_t n_heads);

/* Batched decode: one new query row per sequence, already appended with
 * pkv_append_layer and not yet advanced, so total_k = seq_len + 1 and every
 * key is visible.  Q_dev, out_dev: [M, n_heads * head_dim], row r for
 * seqs[r].  Long contexts are split into key ranges whose size follows from
 * the sequence's own length alone (256 rows below 2048 keys, 512 below
 * 6144, 1024 below 8192, 2048 above) and whose partial softmax states are merged in a fixed
 * order, so each output depends only on its own sequence (independent of M,
 * batch order and placement).
 * ws_dev: >= pkv_decode_workspace_bytes bytes (may be NULL when that is 0).
 * Errors in the pages' order: BAD_DIM (M, n_heads, n_kv_heads, head_dim
 * <= 0, or head shape != the pool's), BAD_GQA, SEQ, then BAD_ARG (layer,
 * metadata-only pool), SEQ (rows not appended), CAPACITY (rotary table too
 * short), BAD_ARG (NULL pointer, workspace too small), UNSUPPORTED.  With
 * rotary embedding on, each query is turned at position seq_len (+ i).
 * ("nx_f32_llama_v4b.nx source": per-row nx_f32_attn_with_paged with n_q = 1
 * and causal = 1; "nx_f32_attn_paged.nx source": the attention body.) */
int32_t pkv_attn_paged_decode(pkv_pool *pool, const int32_t *seqs, int32_t M,
                              int32_t layer, int32_t n_heads,
                              int32_t n_kv_heads, int32_t head_dim,
                              const float *Q_dev, float scale, float *out_dev,
                              void *ws_dev, size_t ws_bytes, void *stream);

/* pkv_attn_paged_decode for callers that cannot allocate memory during the
 * call (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same checks, kernels and results (bit for bit),
 * but no workspace argument and no allocation of any kind -- the split
 * partials and the batch's row descriptors live in a fixed device array
 * built into the library (one per GPU, 1 MiB for descriptors + 64 MiB for
 * partials, held from the first use of the library's kernels on that GPU
 * until the process ends), and the descriptors reach it as kernel arguments
 * (one small launch per 896 ints) instead of through a staging buffer.
 * Every call on one GPU shares that array: calls whose device work overlaps
 * on one GPU (other streams, other pools, other threads) race and must be
 * serialised by the caller.  Nothing in the array needs to start at zero.
 * Errors as pkv_attn_paged_decode (minus the workspace ones), then
 * PKV_ERR_UNSUPPORTED if the pool's device page-table mirror would first
 * have to grow (it is sized by the pool's first device call after a
 * pkv_seq_new with a longer max_tokens than any before: run
 * pkv_append_layer first, as the step protocol does), PKV_ERR_CAPACITY if
 * the batch's descriptors or partials exceed the array's regions, and
 * PKV_ERR_DEVICE.  Kernel timing (pkv_profile_*) covers its launches only
 * while events made by pkv_profile_enable remain. */
int32_t pkv_attn_paged_decode_noalloc(pkv_pool *pool, const int32_t *seqs,
                                      int32_t M, int32_t layer,
                                      int32_t n_heads, int32_t n_kv_heads,
                                      int32_t head_dim, const float *Q_dev,
                                      float scale, float *out_dev,
                                      void *stream);

/* Append, then attend, for one new row per sequence: the pages' per-layer
 * wrapper (append this layer's K/V rows, then paged GQA attention over
 * every row including the new one) as one call.  It runs
 * pkv_append_layer(pool, seqs, M, 1, layer, K_new_dev, V_new_dev, stream)
 * and then pkv_attn_paged_decode(...) with the same arguments (the same
 * launches, so the same pool bytes and output bits), after checking the
 * arguments of both.  K_new_dev, V_new_dev: [M, n_kv_heads * head_dim], row
 * r for seqs[r]; Q_dev, out_dev as for pkv_attn_paged_decode; ws_dev:
 * >= pkv_decode_workspace_bytes bytes.  Rows must be ensured
 * (pkv_ensure_append(.., 1, ..)) and not yet advanced.
 * Errors, in the pages' order: BAD_DIM (M, n_heads, n_kv_heads, head_dim
 * <= 0, or head shape != the pool's), BAD_GQA, SEQ (bad or repeated id),
 * then BAD_ARG (layer out of range), SEQ (rows not ensured, or a target
 * block shared), CAPACITY (rotary table too short), BAD_ARG (metadata-only
 * pool, NULL pointer, workspace too small), DEVICE.  Nothing is launched on
 * an argument error.
 * ("nx_f32_attn_paged.nx source": nx_f32_attn_with_paged -- append, then
 * attention per query head -- with n_q = 1.) */
int32_t pkv_attn_with_paged_decode(pkv_pool *pool, const int32_t *seqs,
                                   int32_t M, int32_t layer, int32_t n_heads,
                                   int32_t n_kv_heads, int32_t head_dim,
                                   const float *Q_dev, const float *K_new_dev,
                                   const float *V_new_dev, float scale,
                                   float *out_dev, void *ws_dev,
                                   size_t ws_bytes, void *stream);

/* pkv_attn_with_paged_decode for pkv_attn_paged_decode_shared: after the
 * checks of both calls, pkv_append_layer of one row per sequence, then the
 * shared-prefix decode (the same launches, so the same pool bytes and
 * output bits).  ws_dev: >= pkv_decode_shared_workspace_bytes bytes.
 * Errors as
 * pkv_attn_with_paged_decode.  ("nx_f32_attn_paged.nx source":
 * nx_f32_attn_with_paged, with the fork sharing of "nx_paged_kv_gate.nx
 * source".) */
int32_t pkv_attn_with_paged_decode_shared(pkv_pool *pool, const int32_t *seqs,
                                          int32_t M, int32_t layer,
                                          int32_t n_heads, int32_t n_kv_heads,
                                          int32_t head_dim, const float *Q_dev,
                                          const float *K_new_dev,
                                          const float *V_new_dev, float scale,
                                          float *out_dev, void *ws_dev,
                                          size_t ws_bytes, void *stream);

/* Device workspace bytes pkv_attn_paged_decode_shared needs for this batch
 * (prefix and split partial results); 0 if none, (size_t)-1 on bad
 * arguments. */
size_t pkv_decode_shared_workspace_bytes(pkv_pool *pool, const int32_t *seqs,
                                         int32_t M, int32_t n_heads);

/* Batched decode that reads shared prefixes once ("nx_paged_kv_gate.nx
 * source", fork: forked sequences hold the same blocks, by reference count,
 * for their common rows).  Computes what pkv_attn_paged_decode computes.
 * Rows of the batch whose page tables begin with the same full pages (at
 * least 16 of them) form a group; the group's common prefix is attended once
 * per kv head for all members' queries (MFMA), each row's remaining keys by
 * decode waves of the same launch, and the partial results are merged.  Outputs agree with
 * pkv_attn_paged_decode within the float tolerance, not bit for bit, and a
 * row's bits depend on the group it falls in (which other rows are in the
 * batch).  Needs head_dim 128 and 16-row pages with a decode group of 1, 2,
 * 4 or 8; other shapes run pkv_attn_paged_decode.  ws_dev: >=
 * pkv_decode_shared_workspace_bytes bytes.  Errors as
 * pkv_attn_paged_decode. */
int32_t pkv_attn_paged_decode_shared(pkv_pool *pool, const int32_t *seqs,
                                     int32_t M, int32_t layer, int32_t n_heads,
                                     int32_t n_kv_heads, int32_t head_dim,
                                     const float *Q_dev, float scale,
                                     float *out_dev, void *ws_dev,
                                     size_t ws_bytes, void *stream);

/* Device workspace bytes pkv_attn_paged_verify needs for n_q queries per
 * sequence (split partial results); 0 if none, (size_t)-1 on bad arguments. */
size_t pkv_verify_workspace_bytes(pkv_pool *pool, const int32_t *seqs,
                                  int32_t M, int32_t n_q, int32_t n_heads);

/* Multi-query decode: n_q new rows per sequence (appended, not advanced),
 * offset-causal -- query i sits at position seq_len + i and sees keys
 * 0 .. seq_len + i -- e.g. verifying n_q drafted tokens in one step, after
 * which pkv_seq_truncate rewinds the rejected ones ("nx_paged_kv_gate.nx
 * source": header, "truncate unref" as the speculative-decode rewind; the
 * result is the prefill's, "nx_f32_attn_paged.nx source" header comment).
 * Q_dev, out_dev: [M * n_q, n_heads * head_dim], row r * n_q + i.  Keys are
 * cut into splits sized from the sequence's own length (as in decode for
 * n_q <= 4, twice that above), merged in a fixed order, so each output
 * depends only on its own sequence.  Split kernel when
 * n_q * (n_heads / n_kv_heads) <= 32 with head_dim 128 and 16-row pages
 * (n_q == 1 runs pkv_attn_paged_decode's kernels, bit for bit); other shapes
 * run the prefill kernels and need no workspace.  ws_dev: >=
 * pkv_verify_workspace_bytes bytes.  Errors as pkv_attn_paged_decode plus
 * BAD_DIM for n_q <= 0. */
int32_t pkv_attn_paged_verify(pkv_pool *pool, const int32_t *seqs, int32_t M,
                              int32_t n_q, int32_t layer, int32_t n_heads,
                              int32_t n_kv_heads, int32_t head_dim,
                              const float *Q_dev, float scale, float *out_dev,
                              void *ws_dev, size_t ws_bytes, void *stream);

/* Chunked prefill: n_q new rows per sequence (appended, not advanced),
 * total_k = seq_len + n_q; with causal != 0 query i sees keys
 * 0 .. total_k - n_q + i, otherwise all total_k keys.  Q_dev, out_dev:
 * [M * n_q, n_heads * head_dim], row r * n_q + i for query i of seqs[r].
 * Errors as pkv_attn_paged_decode plus BAD_DIM for n_q <= 0.
 * ("nx_f32_attn_paged.nx source": header comment, offset-causal rule, and
 * nx_f32_attn_with_paged.) */
int32_t pkv_attn_paged_prefill(pkv_pool *pool, const int32_t *seqs,
                               int32_t M, int32_t n_q, int32_t layer,
                               int32_t n_heads, int32_t n_kv_heads,
                               int32_t head_dim, const float *Q_dev,
                               int32_t causal, float scale, float *out_dev,
                               void *stream);

/* ------------------------------------------------------------------------ */
/* Contiguous twin (the same kernels reading a contiguous cache)             */
/*                                                                            */
/* "nx_f32_attn_paged.nx source" (header comment) and "nx_paged_kv_gate.nx   */
/* source" (EQUIV part) define the paged path as the contiguous path with    */
/* only the row storage changed, and require the two to agree bit for bit.   */
/* These entry points run the same kernels with a contiguous address map,    */
/* so that agreement can be checked on the GPU.                              */
/* ------------------------------------------------------------------------ */

/* A contiguous cache of n_slots sequences: device layout
 * [n_slots][n_layers][2 (K,V)][n_kv_heads][max_seq][head_dim] float32. */
typedef struct pkv_contig {
    void *base_dev;
    int32_t n_slots;
    int32_t n_layers;
    int32_t n_kv_heads;
    int32_t max_seq;
    int32_t head_dim;
    int32_t block_size; /* rows per page the kernels iterate by: give the
                           paged pool's block size to get identical bits */
    const pkv_rope *rope; /* rotary table as pkv_pool_set_rope, or NULL;
                             its head_dim must equal head_dim (else
                             PKV_ERR_BAD_ARG) */
} pkv_contig;

/* Bytes of the contiguous cache above (0 on bad sizes). */
size_t pkv_contig_bytes(int32_t n_slots, int32_t n_layers, int32_t n_kv_heads,
                        int32_t max_seq, int32_t head_dim);

/* Write rows [M * n_new, kv_dim] of slot slots[r] at positions
 * seq_lens[r] .. seq_lens[r] + n_new - 1 of `layer`.  seq_lens, slots: host
 * arrays of M entries. */
int32_t pkv_contig_append(const pkv_contig *cache, const int32_t *slots,
                          const int32_t *seq_lens, int32_t M, int32_t n_new,
                          int32_t layer, const float *K_new_dev,
                          const float *V_new_dev, void *stream);

/* Workspace for pkv_attn_contig_decode given per-row seq_lens. */
size_t pkv_contig_decode_workspace_bytes(const int32_t *seq_lens, int32_t M,
                                         int32_t n_heads, int32_t n_kv_heads,
                                         int32_t head_dim);

/* As pkv_attn_paged_decode with total_k = seq_lens[r] + 1 over slot
 * slots[r].  Bit-identical to the paged call on the same rows. */
int32_t pkv_attn_contig_decode(const pkv_contig *cache, const int32_t *slots,
                               const int32_t *seq_lens, int32_t M,
                               int32_t layer, int32_t n_heads,
                               int32_t n_kv_heads, int32_t head_dim,
                               const float *Q_dev, float scale, float *out_dev,
                               void *ws_dev, size_t ws_bytes, void *stream);

/* Workspace for pkv_attn_contig_verify given per-row seq_lens. */
size_t pkv_contig_verify_workspace_bytes(const int32_t *seq_lens, int32_t M,
                                         int32_t n_q, int32_t n_heads,
                                         int32_t n_kv_heads, int32_t head_dim);

/* As pkv_attn_paged_verify with total_k = seq_lens[r] + n_q over slot
 * slots[r].  Bit-identical to the paged call on the same rows. */
int32_t pkv_attn_contig_verify(const pkv_contig *cache, const int32_t *slots,
                               const int32_t *seq_lens, int32_t M, int32_t n_q,
                               int32_t layer, int32_t n_heads,
                               int32_t n_kv_heads, int32_t head_dim,
                               const float *Q_dev, float scale, float *out_dev,
                               void *ws_dev, size_t ws_bytes, void *stream);

/* As pkv_attn_paged_prefill with total_k = seq_lens[r] + n_q over slot
 * slots[r].  Bit-identical to the paged call on the same rows. */
int32_t pkv_attn_contig_prefill(const pkv_contig *cache, const int32_t *slots,
                                const int32_t *seq_lens, int32_t M,
                                int32_t n_q, int32_t layer, int32_t n_heads,
                                int32_t n_kv_heads, int32_t head_dim,
                                const float *Q_dev, int32_t causal,
                                float scale, float *out_dev, void *stream);

/* ------------------------------------------------------------------------ */
/* Introspection (bitwise state comparisons)                                 */
/* ------------------------------------------------------------------------ */

/* Current length of a sequence, or -PKV_ERR_SEQ. */
int32_t pkv_seq_len(pkv_pool *pool, int32_t seq);

/* Copies up to cap block ids of the page table; returns the page count
 * (which may exceed cap) or -PKV_ERR_SEQ. */
int32_t pkv_seq_pages(pkv_pool *pool, int32_t seq, int64_t *out, int32_t cap);

/* Copies the n_blocks reference counts; returns n_blocks. */
int32_t pkv_pool_refcounts(pkv_pool *pool, int32_t *out);

/* Copies up to cap free ids from the bottom of the free stack to its top
 * (the last one is taken next); returns the number of free ids. */
int32_t pkv_pool_free_stack(pkv_pool *pool, int64_t *out, int32_t cap);

/* ------------------------------------------------------------------------ */
/* Kernel timing                                                             */
/* ------------------------------------------------------------------------ */

/* Kernel ids for pkv_profile_read. */
#define PKV_K_APPEND 0
#define PKV_K_DECODE 1   /* the split decode kernel */
#define PKV_K_MERGE 2    /* the merge of the decode key splits */
#define PKV_K_PREFILL 3
#define PKV_K_COW 4
#define PKV_K_VERIFY 5   /* the split multi-query kernel */
#define PKV_K_PREFIX 6   /* the shared-prefix decode kernel (prefix and own
                            keys in one launch) */
#define PKV_K_COUNT 7

/* on != 0: record a HIP event pair on the launch stream around every kernel
 * the pool launches; on == 0: stop.  Either way, clears the totals (after
 * waiting for the pool's stream).  Switching on makes the events for the
 * next 128 timed launches up front (creating a HIP event can take the host
 * hundreds of microseconds, which would otherwise land inside timed steps);
 * events are reused by later profiling runs. */
int32_t pkv_profile_enable(pkv_pool *pool, int32_t on);

/* Which kernels profiling times: bit k of mask selects kernel id k (all by
 * default).  Each timed launch adds two event records to the stream, so a
 * caller timing one kernel of a step can leave the others untimed. */
int32_t pkv_profile_kernels(pkv_pool *pool, uint32_t mask);

/* Wait for the recorded events and report the summed kernel time (ms) and
 * launch count of one kernel id since profiling was enabled. */
int32_t pkv_profile_read(pkv_pool *pool, int32_t kernel, double *total_ms,
                         int64_t *launches);

/* The kernel form last launched under kernel id `kernel` -- the template
 * instance, e.g. "decode_fast_kernel<4, PagedMap, true>" (GQA group, address
 * map, deep form) -- written NUL-terminated into out[0..cap) (truncated to
 * fit).  Returns the name's full length (0 before any launch) or a negated
 * code.  Recorded whether or not profiling is on. */
int32_t pkv_profile_kernel_name(pkv_pool *pool, int32_t kernel, char *out,
                                int32_t cap);

/* Wait for the recorded events and copy the duration (ms) of each of the
 * first cap launches of one kernel id, in launch order; returns the number
 * of launches recorded (which may exceed cap) or a negated code. */
int32_t pkv_profile_samples(pkv_pool *pool, int32_t kernel, float *out_ms,
                            int32_t cap);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */

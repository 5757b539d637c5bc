/*
 * zipage.h -- C ABI of the MI355X (gfx950) Compressed-PagedAttention
 * compression library.
 *
 * The operation is one KV-cache compression step of Zipage (arXiv 2603.08743,
 * "Zipage: Maintain High Request Concurrency for LLM Reasoning through
 * Compressed PagedAttention"), as described by the summary pages cited below:
 *   [zh] gist.science/zh/paper/2603.08743, technical summary
 *   [de] gist.science/de/paper/2603.08743, technical summary
 *   [es] gist.science/es/paper/2603.08743, technical summary
 *   [fr] gist.science/fr/paper/2603.08743, technical summary
 *
 * Conventions for every call:
 *   - All pointers named "device" point to GPU memory owned by the caller; the
 *     library never allocates, frees or synchronises device memory or streams
 *     (the one exception, zp_workspace_error, is documented as synchronous).
 *   - `stream` is a hipStream_t passed as void*; NULL is the null stream.
 *     Work is enqueued asynchronously; pointers must stay valid until it ends.
 *   - Every argument check runs before anything is enqueued. On an error
 *     status nothing was enqueued and no output was touched. The message of
 *     the last error on the calling thread is returned by zp_last_error().
 *   - Device tables are checked by the kernels as they read them: a block id
 *     outside [0, num_blocks), a token count outside its allowed range or a
 *     slot outside [0, num_slots) makes the affected (request, layer, head)
 *     unit skip all memory writes except the markers keep_idx[u][0] = -1 and
 *     first_hole[u] = -1 (when that output is requested), and records
 *     ZP_EDEVICE in the workspace. zp_update_global leaves such units alone.
 *   - No C++ exception crosses this interface.
 *   - The calls that enqueue work (zp_compress, zp_update_global, the decode
 *     and capture calls, zp_redundancy_full) allocate nothing, synchronise
 *     nothing and issue no memset, so a caller may record them into a HIP
 *     graph and replay it (per-launch timing, zp_timing_enable, must be off
 *     while capturing). zp_workspace_error synchronises and stays outside.
 */
#ifndef ZIPAGE_H
#define ZIPAGE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t zp_status;

#define ZP_OK            0
#define ZP_EINVAL       -1  /* bad shape, pointer, alignment or value        */
#define ZP_EUNSUPPORTED -2  /* valid but not built: head_dim, block size ... */
#define ZP_EWORKSPACE   -3  /* workspace missing or too small                */
#define ZP_ENOSPACE     -4  /* free list exhausted (no state was changed)    */
#define ZP_EHIP         -5  /* the HIP runtime reported an error             */
#define ZP_EDEVICE      -6  /* a kernel found a bad device table entry       */
#define ZP_ESYNC        -7  /* workgroups of a split unit stopped waiting on
                               each other (bounded wait passed); the call's
                               outputs are incomplete: every unit's K/V rows
                               and global row are either fully compacted or
                               untouched, but which is not reported, so the
                               batch's requests must be prefilled again     */

/* element types */
#define ZP_F32  0
#define ZP_BF16 1

/* zp_params.flags */
#define ZP_NONCAUSAL      (1u << 0) /* window rows see all n tokens           */
#define ZP_PROTECT_WINDOW (1u << 1) /* the last w tokens are always kept      */
#define ZP_WINDOW_RING    (1u << 2) /* q_window rows form a ring: the query of
                                       position p sits in row p mod w (the
                                       layout zp_capture_queries writes)     */
#define ZP_UPDATE_GLOBAL  (1u << 3) /* zp_compress also applies the global-
                                       score update of zp_update_global in
                                       the same kernel (then that call must
                                       not follow for this batch)            */
#define ZP_SPLIT_UNITS    (1u << 4) /* zp_compress spreads every unit over up
                                       to 8 workgroups where that schedule
                                       applies (same results, up to the
                                       rounding of the attention sums)       */

/* A paged KV pool: k and v are device arrays laid out
 * [layers][num_blocks][kv_heads][block_size][head_dim] of `dtype`, 16-byte
 * aligned. A block id names the same block in every layer and head, so one
 * block table serves a request in all layers ([zh] §2: the method builds on
 * PagedAttention's block tables). */
typedef struct {
  void*   k;
  void*   v;
  int32_t num_blocks;
  int32_t layers;
  int32_t kv_heads;
  int32_t block_size;   /* b; the library supports 16                       */
  int32_t head_dim;     /* d; the library supports 64 and 128               */
  int32_t dtype;        /* ZP_F32 or ZP_BF16                                */
} zp_kv_pool;

/* Parameters of one compression call.
 *   n_max    -- N_max, the per-request block cap, 2..1024 (N_max*b is at
 *               most 16384); a request compresses when it holds N_max full
 *               blocks and keeps k = (N_max-1)*b tokens in its first N_max-1
 *               blocks ([zh] §2.1, [de] §2).
 *   window   -- w, the number of most recent query states used to score
 *               ([zh] §2.1, [de] §2, [es] §2).
 *   q_heads  -- query heads; must be a multiple of kv_heads. Query head
 *               h*G+g (G = q_heads/kv_heads) reads KV head h.
 *   q_dtype  -- element type of the query windows (ZP_F32 or ZP_BF16).
 *   w_attn, w_global, w_red -- score s = w_attn*attn + w_global*global
 *               - w_red*red (the pages name the three parts, [zh] §2.1,
 *               without a formula; 1, 0.5, 0.5 is the documented default).
 *   sm_scale -- softmax scale; <= 0 selects 1/sqrt(head_dim).
 *   flags    -- ZP_NONCAUSAL, ZP_PROTECT_WINDOW, ZP_WINDOW_RING,
 *               ZP_UPDATE_GLOBAL. */
typedef struct {
  int32_t  n_max;
  int32_t  window;
  int32_t  q_heads;
  int32_t  q_dtype;
  float    w_attn;
  float    w_global;
  float    w_red;
  float    sm_scale;
  uint32_t flags;
} zp_params;

/* The requests of one compression call (R = num_reqs). Device arrays:
 *   slot[R]        -- query-slot row of each request: selects its window in
 *                     q_window and its row of global scores ([zh] §2.2: only
 *                     requests holding a query slot are compressed). The
 *                     entries are distinct within a call: the kernels reject
 *                     every request whose slot another request of the call
 *                     also names, as a bad table entry (ZP_EDEVICE; for
 *                     zp_update_global: such units are left alone).
 *   n_tokens[R]    -- tokens held, n; must satisfy n_max*b <= n <= n_cap and
 *                     ceil(n/b) <= max_blocks (n > n_max*b: prefill overshoot).
 *   src_table[R][max_blocks] -- current block table (logical -> physical).
 *   dst_table[R][n_max]      -- block table after compression. For a request
 *                     with n_pinned == 0 it must equal src_table's first n_max
 *                     entries (in-place compaction). With n_pinned == S > 0,
 *                     entries [0,S) equal the shared blocks, entries
 *                     [S, n_max-1) are fresh target blocks that alias no
 *                     source block, entry n_max-1 is any block (the new tail).
 *   n_pinned[R]    -- S, the leading shared blocks, kept whole and never
 *                     written ([zh] §2.2, [de] §2, [fr] §2.C).
 *                     The blocks a request writes -- src_table entries
 *                     [S, ceil(n/b)) when it compacts in place, dst_table
 *                     entries [S, n_max-1) when it writes targets -- belong
 *                     to that request alone: no other request of the call
 *                     reads or writes them (zp_bm_plan_compress guarantees
 *                     it; the kernels do not check it).
 *   seq_pos[R]     -- optional (NULL: n_tokens), read with ZP_WINDOW_RING
 *                     only: sequence position P of the request's next token,
 *                     the position zp_capture_queries rings by. Window row i
 *                     (the i-th of the last w queries) is ring row
 *                     (P - w + i) mod w; P >= w. After a compression the
 *                     cache holds fewer tokens than the sequence, so P and
 *                     n_tokens differ.
 * Host fields: num_reqs, max_blocks, num_slots (rows of q_window and of
 * global_scores) and n_cap (length of a global-score row and of the attn /
 * red / score output rows; n_cap <= 16384). */
typedef struct {
  int32_t        num_reqs;
  int32_t        max_blocks;
  int32_t        num_slots;
  int32_t        n_cap;
  const int32_t* slot;
  const int32_t* n_tokens;
  const int32_t* src_table;
  const int32_t* dst_table;
  const int32_t* n_pinned;
  const int32_t* seq_pos;
} zp_batch;

/* Outputs of zp_compress, one row per unit u = (r*layers + l)*kv_heads + h.
 *   keep_idx[U][k]  (required) kept logical positions, ascending.
 *   attn[U][n_cap]  (required) window attention of every token, entries
 *                   [0, n) written; consumed by zp_update_global.
 *   red[U][n_cap]   (optional, NULL) lightning redundancy.
 *   score[U][n_cap] (optional, NULL) combined score, +inf where pinned.
 *   first_hole[U]   (optional, NULL) first evicted position h. */
typedef struct {
  int32_t* keep_idx;
  float*   attn;
  float*   red;
  float*   score;
  int32_t* first_hole;
} zp_compress_out;

/* Bytes of device workspace zp_compress needs for num_reqs requests with
 * these params: 256 (the error word and padding), or, with ZP_SPLIT_UNITS on
 * a bf16 pool, the split-unit schedule's size (about 11.5 MB, whatever the
 * batch: the error word, a group ticket and 256 group exchange slots).
 * zp_compress also accepts a 256-byte workspace with ZP_SPLIT_UNITS; it then
 * runs the one-workgroup schedule. A workspace serves one call at a time:
 * calls that may overlap (on different streams) need their own.
 * Errors: ZP_EINVAL for a NULL argument or non-positive sizes. */
zp_status zp_compress_workspace_bytes(const zp_kv_pool* pool,
                                      const zp_params* params,
                                      int32_t num_reqs, size_t* bytes);

/* One compression step for every (request, layer, KV head) unit of `batch`
 * ([zh] §2.1, [de] §2, [es] §2, [fr] §2.A; kernels: [zh] §2.3):
 *   1. attn_t: mean over the w*G window rows of softmax(q.k*scale)_t, causal
 *      by default (window row i sits at position n-w+i);
 *   2. red_t: mean cosine similarity of k_t to the other keys of its block
 *      (lightning redundancy, O(N b^2) for N blocks: [zh] §2.1, [fr] §2.E);
 *   3. s_t = w_attn*attn_t + w_global*global_t - w_red*red_t, +inf for
 *      pinned tokens (shared prefix; the window with ZP_PROTECT_WINDOW);
 *   4. keep the k = (N_max-1)*b best tokens (higher s first, then lower
 *      position) and write them ascending to keep_idx;
 *   5. move kept K and V rows, in order, to logical rows [0, k) through
 *      dst_table: in place for n_pinned == 0, into the target blocks
 *      otherwise; shared blocks are never written ([zh] §2.2).
 * q_window: device [num_slots][layers][w][q_heads][head_dim] of q_dtype.
 * global_scores: device [num_slots][layers][kv_heads][n_cap] fp32 (read only
 * here unless ZP_UPDATE_GLOBAL is set, then updated in place as by
 * zp_update_global). workspace: device, 256-byte aligned, at least
 * zp_compress_workspace_bytes; it also receives the device error word.
 * Schedules. By default one workgroup scores, selects and compacts a whole
 * unit: units whose keys take at most 512 KiB (n_cap * head_dim * element
 * bytes) run as 4-wave workgroups, two per compute unit, larger ones as
 * 8-wave workgroups, one per compute unit. The environment variable
 * ZIPAGE_KEY_GROUPS, read at each call, forces the 4-wave (value 2) or the
 * 8-wave shape (value 4); both give results within the attention rounding
 * of each other. With ZP_SPLIT_UNITS, a bf16 call with n_cap <= 4096 (w*G <= 128) or
 * n_cap <= 2048 (w*G <= 192) and a workspace of zp_compress_workspace_bytes
 * splits every unit over up to 8 workgroups, one per slice of 512 (256)
 * tokens: each keeps its slice's keys on chip, the workgroups exchange their
 * per-row softmax normalisers and their eviction candidates through the
 * workspace, and every K/V row is read once. Its grid holds one workgroup
 * per CU and the workgroups of a unit wait on each other, so two such calls
 * must not run concurrently on one device (they could hold every CU between
 * them and wait until the bounded wait ends with ZP_ESYNC). Both schedules
 * give the same keep sets and bytes; attention values may differ in the last
 * bits (summation order). The split schedule's waits on other
 * workgroups are bounded: if one ever passes its limit (a few seconds), the
 * kernel stops and the workspace error word becomes ZP_ESYNC. The
 * environment variable ZP_SPLIT_SPIN_LIMIT, read at each call, lowers that
 * limit to the given number of polls (0 to 4194304; other values are
 * ignored); it exists to exercise the ZP_ESYNC path.
 * Errors: ZP_EINVAL, ZP_EUNSUPPORTED (head_dim not 64/128, block_size not 16,
 * w*G > 192 -- 64 for fp32 with head_dim 128 --, n_cap > 16384, or, for fp32
 * with head_dim 128 only, n_cap above about 6100: the per-token scores of a
 * unit live in on-chip memory beside the key ring), ZP_EWORKSPACE, ZP_EHIP.
 * Nothing is written when an error is returned. */
zp_status zp_compress(const zp_kv_pool* pool, const zp_batch* batch,
                      const void* q_window, float* global_scores,
                      const zp_params* params, const zp_compress_out* out,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Global-score update after zp_compress on the same stream ([zh] §2.1 global
 * score from past attention; update kernel [zh] §2.3): for every unit,
 * g'_t = g_{keep[t]} + attn_{keep[t]} for t < k and g'_t = 0 for
 * t in [k, n_cap), in place in global_scores (the row of slot[r]).
 * Errors: ZP_EINVAL, ZP_EUNSUPPORTED, ZP_EHIP. */
zp_status zp_update_global(float* global_scores, const zp_kv_pool* pool,
                           const zp_batch* batch, const zp_compress_out* out,
                           const zp_params* params, void* stream);

/* Reads the device error word of a workspace after the caller's stream work
 * has finished: synchronises `stream`, stores ZP_OK, ZP_EDEVICE or ZP_ESYNC
 * in *code and clears the word. A call that met both a bad table entry and a
 * wait past its limit reports either one. Errors: ZP_EINVAL, ZP_EHIP. */
zp_status zp_workspace_error(void* workspace, void* stream, int32_t* code);

/* Decode attention over a paged cache, the consumer of the compressed blocks
 * ([zh] §2.3: decoding runs PagedAttention over the blocks):
 * out[r][l][hq][:] = softmax(q[r][l][hq] . K^T * scale) V over the seq_lens[r]
 * tokens of request r, with K, V read through block_tables.
 * out: device fp32 [num_reqs][layers][q_heads][head_dim]; q: device
 * [num_reqs][layers][q_heads][head_dim] of params->q_dtype; block_tables:
 * device [num_reqs][max_blocks]; seq_lens: device [num_reqs], 1 <= len <=
 * max_blocks*b. Only params->q_heads, q_dtype and sm_scale are read.
 * Errors: ZP_EINVAL, ZP_EUNSUPPORTED, ZP_EHIP. */
zp_status zp_paged_decode(float* out, const void* q, const zp_kv_pool* pool,
                          const int32_t* block_tables, int32_t max_blocks,
                          const int32_t* seq_lens, int32_t num_reqs,
                          const zp_params* params, void* stream);

/* Decode step with the new token appended ([zh] §2.3: decoding appends to the
 * request's tail block): for every (r, l, kv head h) the new token's rows
 * k_new[r][l][h][:] and v_new[r][l][h][:] are written to position seq_lens[r]
 * (block block_tables[r][seq_lens[r] / b], slot seq_lens[r] mod b) and out is
 * the attention of q over the seq_lens[r] + 1 tokens, the new one included.
 * seq_lens[r] counts the tokens cached before the call (0 allowed) and is not
 * changed; ceil((seq_lens[r] + 1) / b) <= max_blocks. k_new, v_new: device
 * [num_reqs][layers][kv_heads][head_dim] of the pool dtype, 16-byte aligned.
 * A unit with a bad length or block id writes nothing (neither the slot nor
 * out). Errors: as zp_paged_decode. */
zp_status zp_paged_decode_append(float* out, const void* q, const void* k_new,
                                 const void* v_new, const zp_kv_pool* pool,
                                 const int32_t* block_tables, int32_t max_blocks,
                                 const int32_t* seq_lens, int32_t num_reqs,
                                 const zp_params* params, void* stream);

/* Split-K decode for long contexts with few units: each (request, layer, kv
 * head) is spread over `splits` waves (1..256), each taking a contiguous range
 * of the unit's blocks; a second kernel merges their partial (max, sum, P.V)
 * with the usual softmax rescaling. k_new / v_new: NULL, or an append as in
 * zp_paged_decode_append. workspace: device, 256-byte aligned, at least
 * zp_decode_workspace_bytes(pool, params, num_reqs, splits) bytes (0 for
 * splits == 1). Errors: as zp_paged_decode, plus ZP_EWORKSPACE. */
zp_status zp_decode_workspace_bytes(const zp_kv_pool* pool, const zp_params* params,
                                    int32_t num_reqs, int32_t splits, size_t* bytes);
zp_status zp_paged_decode_split(float* out, const void* q, const void* k_new,
                                const void* v_new, const zp_kv_pool* pool,
                                const int32_t* block_tables, int32_t max_blocks,
                                const int32_t* seq_lens, int32_t num_reqs,
                                const zp_params* params, int32_t splits, void* workspace,
                                size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * split-K decode as zp_paged_decode_split, with its split partials in a
 * static device array of ZP_DECODE_STATIC_BYTES owned by the library (each
 * GPU the library runs on holds one copy until the process ends) instead of
 * a caller workspace. The call allocates nothing and issues no memset; the
 * caller still passes every input and output. Calls that overlap on one GPU
 * (on different streams, or from several threads) share that array and
 * race: serialise them. The array keeps the last call's partials; nothing
 * in it needs clearing between calls. Call with the stream's device current.
 * Errors: as zp_paged_decode_split, with ZP_EWORKSPACE when the partials,
 * num_reqs * layers * q_heads * splits * (head_dim + 2) * 4 bytes, exceed
 * ZP_DECODE_STATIC_BYTES (nothing is enqueued then). */
#define ZP_DECODE_STATIC_BYTES (64u << 20)
zp_status zp_paged_decode_split_static(float* out, const void* q, const void* k_new,
                                       const void* v_new, const zp_kv_pool* pool,
                                       const int32_t* block_tables, int32_t max_blocks,
                                       const int32_t* seq_lens, int32_t num_reqs,
                                       const zp_params* params, int32_t splits,
                                       void* stream);

/* All-pairs key redundancy, an ablation of the lightning score ([zh] §2.1,
 * [fr] §2.E: the original score compared every pair of cached keys, O(N^2 b^2)
 * for N blocks of b; lightning keeps the pairs inside a block, O(N b^2)).
 * For every unit of `batch` the full n x n cosine matrix of its keys is
 * formed (norm products clamped at 1e-8, the diagonal dropped) and each token
 * gets red_block[u][t], the mean over the other tokens of its block (equal
 * to zp_compress's red, up to rounding), and, when red_all is not NULL,
 * red_all[u][t], the mean over all other tokens. Rows [0, n) of
 * [U][n_cap] fp32 outputs are written; only src_table and n_tokens of the
 * batch are read. Nothing is moved or selected. Each pair of key tiles is
 * formed once; red_all's sums gather contributions from several workgroups
 * by float atomic adds, so they can differ between calls in the last bits
 * (fp32 addition order). Without red_all only the block-diagonal tiles are
 * formed. workspace: as zp_compress (its error word; a bad table entry gives
 * ZP_EDEVICE there, and that unit's red_all rows are left at 0).
 * Errors: as zp_compress. */
zp_status zp_redundancy_full(float* red_block, float* red_all, const zp_kv_pool* pool,
                             const zp_batch* batch, const zp_params* params,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Query-window capture, the step before compression ([zh] §2.2, [de] §2: only
 * requests that hold a query slot keep their recent queries; [zh] §2.1: the
 * last w queries score the cache). For every request r with a slot
 * (0 <= slot[r] < num_slots) and pos[r] >= 0, the post-RoPE queries of its
 * new token at position pos[r] are written for every layer l to
 *   q_window[slot[r]][l][pos[r] mod w][:][:]
 * so the window of a slot is a ring over the last w positions; zp_compress
 * reads it with ZP_WINDOW_RING. Requests without a slot (slot[r] < 0, the
 * slot-free decoding of [zh] §2.2) and any with a slot or position out of
 * range are skipped.
 * q_window: device [num_slots][layers][w][q_heads][head_dim]; q: device
 * [num_reqs][layers][q_heads][head_dim]; both of params->q_dtype, 16-byte
 * aligned. slot, pos: device [num_reqs] int32. Only params->window, q_heads
 * and q_dtype are read. Errors: ZP_EINVAL, ZP_EUNSUPPORTED (head_dim not
 * 64/128), ZP_EHIP. */
zp_status zp_capture_queries(void* q_window, const void* q, const int32_t* slot,
                             const int32_t* pos, int32_t num_reqs, int32_t layers,
                             int32_t num_slots, int32_t head_dim,
                             const zp_params* params, void* stream);

/* ---------------------------------------------------------------------------
 * Host-side block bookkeeping (no GPU calls). A block manager owns the free
 * list and the reference counts of a pool of num_blocks blocks. The free list
 * is a LIFO stack; a fresh manager pops id 0 first. Not thread-safe: the
 * caller serialises calls on one manager.
 * ------------------------------------------------------------------------ */
typedef struct zp_bm zp_bm;
typedef struct zp_plan zp_plan;

/* NULL on a bad size or out of memory. */
zp_bm* zp_bm_create(int32_t num_blocks);
void zp_bm_destroy(zp_bm* bm);

/* Pops n blocks into ids[n] (refcount 1 each). ZP_ENOSPACE leaves the
 * manager unchanged. */
zp_status zp_bm_alloc(zp_bm* bm, int32_t n, int32_t* ids);
/* One more user of a held block (a shared prefix, [de] §2). */
zp_status zp_bm_incref(zp_bm* bm, int32_t id);
/* One user fewer for each id; blocks reaching 0 are pushed in array order. */
zp_status zp_bm_release(zp_bm* bm, int32_t n, const int32_t* ids);
int32_t zp_bm_free_count(const zp_bm* bm);
/* -1 for an id out of range. */
int32_t zp_bm_refcount(const zp_bm* bm, int32_t id);
/* Copies the free stack bottom to top into ids (at most cap); returns the
 * number of free blocks. */
int32_t zp_bm_free_list(const zp_bm* bm, int32_t* ids, int32_t cap);

/* Plans one compression call ([zh] §2.1 trigger; [zh] §2.2 shared prefix):
 * host_tables[R][max_blocks], n_tokens[R] on the host. For every request,
 * S = the leading run of blocks with refcount > 1 (at most n_max-1).
 *   S == 0: dst_tables[r] = its first n_max blocks (in place);
 *   S  > 0: dst_tables[r] = [shared 0..S-1, n_max-1-S targets popped now in
 *           logical order, old block n_max-1 as the tail].
 * Blocks that compression frees (old private blocks S..n_max-2 when S > 0,
 * then every block past n_max) are recorded in the plan, in logical order,
 * and pushed only by zp_bm_commit. Outputs dst_tables[R][n_max] and
 * n_pinned[R] (= S) on the host. Every block a request holds after its
 * shared run ([S, ceil(n/b))) is rewritten in place, kept as the tail or
 * freed, so it must have refcount 1 and appear once in the whole call
 * ([de] §2: blocks with a count above one stay intact).
 * Errors: ZP_EINVAL (bad sizes, n_tokens below n_max*b, a block id out of
 * range, a block after the shared run with refcount other than 1 or listed
 * twice), ZP_ENOSPACE (not enough free blocks for the targets). On an error
 * nothing changed and *plan is NULL. */
zp_status zp_bm_plan_compress(zp_bm* bm, int32_t num_reqs,
                              const int32_t* host_tables, int32_t max_blocks,
                              const int32_t* n_tokens, int32_t n_max,
                              int32_t block_size, int32_t* dst_tables,
                              int32_t* n_pinned, zp_plan** plan);
/* After the compression stream's work has finished (an event the caller
 * waited on): targets keep refcount 1, freed blocks get 0 and are pushed in
 * plan order, shared counts are unchanged. Consumes the plan. */
zp_status zp_bm_commit(zp_bm* bm, zp_plan* plan);
/* Abandons a plan: its targets go back on the stack (reverse pop order), so
 * the manager is as before the plan. Consumes the plan. */
zp_status zp_bm_abort(zp_bm* bm, zp_plan* plan);
/* Blocks the plan will free, in push order; returns their number (copies at
 * most cap into ids). */
int32_t zp_plan_freed(const zp_plan* plan, int32_t* ids, int32_t cap);
/* Targets the plan popped, in pop order; returns their number. */
int32_t zp_plan_targets(const zp_plan* plan, int32_t* ids, int32_t cap);

/* ---------------------------------------------------------------------------
 * Hybrid scheduling (host, no GPU calls): query slots, slot-free decoding,
 * preemption and a restricted mode ([zh] §2.2, [de] §2, [fr] §2.B), with
 * compression running beside decoding ([zh] §2.1, [fr] §2.D). The scheduler
 * owns a block manager of num_blocks blocks. Each zp_sched_step plans one
 * step in admission order:
 *   1. the first query_slots (M) running requests hold the M query slots;
 *   2. a slot holder with n >= N_max*b cached tokens that has captured w
 *      queries compresses (and does not decode) this step; target blocks of
 *      a shared-prefix compression are taken first, preempting slot-free
 *      requests if needed;
 *   3. every other request decodes one token, except a slot-free request
 *      with n >= N_max*b - w (its queries would have to be captured: it waits
 *      for a slot). A token that opens a block takes one from the free list;
 *      when it is empty the most recently admitted slot-free request is
 *      preempted (its blocks are released and it returns to the front of the
 *      waiting queue, to be prefilled again with prompt + generated tokens).
 *      With no slot-free request left the step is restricted: requests
 *      without a block wait and nothing is admitted;
 *   4. waiting requests are admitted FIFO while blocks last; a prompt of at
 *      least N_max*b - w tokens is admitted only if it gets a slot. Prompts of
 *      a prefix group share the group's cached prefix blocks.
 * The caller runs the plan's GPU work (prefill of admitted requests, query
 * capture and decode with append for the decode set, zp_compress +
 * zp_update_global for the compress set with dst tables and n_pinned from the
 * plan), then calls zp_sched_complete. Plan arrays are host memory owned by
 * the scheduler, valid until the next zp_sched_step; tables are rows of
 * max_blocks (compress_dst: rows of n_max), padded with -1. Not thread-safe.
 * ------------------------------------------------------------------------ */
typedef struct zp_sched zp_sched;

typedef struct {
  int32_t num_blocks;   /* blocks of the pool                               */
  int32_t block_size;   /* b                                                */
  int32_t n_max;        /* N_max                                            */
  int32_t window;       /* w                                                */
  int32_t query_slots;  /* M                                                */
  int32_t max_running;  /* cap on running requests                          */
  int32_t max_blocks;   /* table row width; >= ceil((prompt+gen)/b) of all;
                           max_blocks * block_size <= 2^30              */
} zp_sched_config;

typedef struct {
  int32_t restricted, max_blocks;
  int32_t num_admit;          /* prefill: write K/V of tokens [shared, len)  */
  const int32_t *admit_id, *admit_len, *admit_slot, *admit_table, *admit_shared;
  int32_t num_new_slots;      /* slots handed out: clear ring and global row */
  const int32_t* new_slot;
  int32_t num_decode;         /* one token each at cache position len,       */
  const int32_t *decode_id, *decode_slot, *decode_len, *decode_pos,
      *decode_table;          /* sequence position pos (ring row pos mod w)  */
  int32_t num_compress;       /* n tokens, next sequence position pos        */
  const int32_t *compress_id, *compress_slot, *compress_len, *compress_pos,
      *compress_src, *compress_dst, *compress_pinned;
  int32_t num_preempt;
  const int32_t* preempt_id;
} zp_sched_plan;

typedef struct {
  int64_t steps, tokens, compressions, preemptions, restricted_steps, admitted,
      finished;
  int32_t running, waiting, free_blocks;
} zp_sched_stats;

zp_sched* zp_sched_create(const zp_sched_config* cfg);   /* NULL on error   */
void zp_sched_destroy(zp_sched* s);
zp_bm* zp_sched_block_manager(zp_sched* s);              /* for inspection  */
/* A cached shared prefix of `blocks` blocks (1 <= blocks < n_max): allocated
 * now, one reference held by the cache for the scheduler's lifetime; its ids
 * are returned so the caller can fill their K/V. */
zp_status zp_sched_add_prefix(zp_sched* s, int32_t blocks, int32_t* group,
                              int32_t* block_ids);
/* Queue a request (ids unique, >= 0); group -1 or a prefix group whose
 * prefix the prompt starts with. */
zp_status zp_sched_submit(zp_sched* s, int32_t req_id, int32_t prompt_len,
                          int32_t gen_len, int32_t group);
zp_status zp_sched_step(zp_sched* s, zp_sched_plan* plan);
zp_status zp_sched_complete(zp_sched* s);
zp_status zp_sched_get_stats(const zp_sched* s, zp_sched_stats* stats);

/* ---------------------------------------------------------------------------
 * Kernel timing for measurement: while enabled, zp_compress,
 * zp_update_global and zp_paged_decode record a pair of HIP events around
 * every kernel they launch, on the launch stream. zp_timing_read waits for
 * the recorded events, and returns per kernel kind the launch count and the
 * summed milliseconds, then clears the record.
 * ------------------------------------------------------------------------ */
#define ZP_KERNEL_COMPRESS 0  /* score, select and K/V compaction            */
#define ZP_KERNEL_GLOBAL   1  /* global-score update                         */
#define ZP_KERNEL_DECODE   2  /* paged decode                                */
#define ZP_KERNEL_CAPTURE  3  /* query-window capture                        */
#define ZP_KERNEL_REDUNDANCY_FULL 4  /* all-pairs redundancy (ablation)      */
#define ZP_KERNEL_KINDS    5

zp_status zp_timing_enable(int32_t enable);
zp_status zp_timing_read(int32_t* launches /*[ZP_KERNEL_KINDS]*/,
                         double* total_ms /*[ZP_KERNEL_KINDS]*/);

/* Text of a status code; message of the last error on this thread. */
const char* zp_status_str(zp_status status);
const char* zp_last_error(void);
/* Library version string. */
const char* zp_version(void);

#ifdef __cplusplus
}
#endif
#endif /* ZIPAGE_H */

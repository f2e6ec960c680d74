/*
 * pkv.h -- C ABI of libpkv: a paged KV cache and PagedAttention decode for
 * AMD MI355X (gfx950).
 *
 * Sources the operations follow (cited by page title and section):
 *   [lesson]   "PagedAttention e continuous batching" (llmdeepdive lesson 7.8),
 *              section "01 · Conceito", paragraphs 1-9 (paragraph 1 opens
 *              "Você tem um acelerador de 80 GB", 3 "PagedAttention,
 *              introduzida com o vLLM", 6 "A indireção também habilita
 *              compartilhamento", 7 "A alocação resolve onde o estado
 *              mora", 8 "Acompanhe as métricas operacionais");
 *   [preview]  "04 — Hacia PagedAttention (vista previa)" (lynx-cortex,
 *              phase 22 theory), section "La idea de PagedAttention", steps 1-5
 *              and "Propiedades"; "Lo que deberías llevarte"; "Lo que la
 *              Fase 22 construye";
 *   [tutorial] "Paged Attention em Large Language Models LLMs" (acheiumaia),
 *              "Configurando as Constantes".
 *
 * Two halves:
 *   host    -- the block allocator.  A pool of fixed-size blocks with a free
 *              list, per-block reference counts, per-sequence block tables
 *              and copy-on-write.  Pure CPU code, no GPU calls.
 *   device  -- HIP kernels that write new K/V rows at their slots, copy whole
 *              blocks for copy-on-write, and run decode attention through the
 *              block tables.  Asynchronous on the caller's stream.
 *
 * Conventions
 *   - Every function returns a pkv_status.  On any error nothing changes
 *     (a request that does not fit is turned away when admitted, with a
 *     status, instead of failing later: [lesson] paragraph 7);
 *     pkv_last_error() gives a message for the calling thread.
 *   - The caller owns all device memory: the K/V pools, q, out, tables,
 *     context lengths, plans and workspaces.  The library never allocates
 *     device memory and never synchronises a stream.
 *   - A pool object is not thread-safe; use one thread per pool.
 *   - Slots: slot s of a pool is row s % block_size of block s / block_size.
 *   - "stream" is a hipStream_t passed as void*; NULL is the null stream.
 *   - Pool layout in device memory (a reading: the pages only say blocks may
 *     live anywhere): K and V are two arrays shaped
 *     [num_blocks][num_kv_heads][block_size][head_dim] of the pool dtype, so
 *     one (block, head) tile is one contiguous block_size*head_dim span.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_E_NO_BLOCKS = 1,   /* not enough free blocks; nothing changed       */
  PKV_E_BAD_SEQ = 2,     /* unknown or already freed sequence id          */
  PKV_E_BAD_ARG = 3,     /* invalid argument (null, size, geometry, dtype) */
  PKV_E_TABLE_FULL = 4,  /* a sequence would exceed max_blocks_per_seq    */
  PKV_E_HIP = 5,         /* a HIP launch failed                           */
  PKV_E_UNSUPPORTED = 6, /* valid, but not built (head_dim, dtype, ...)   */
  PKV_E_NO_SLOTS = 7     /* no free state slot (hybrid manager); nothing changed */
} pkv_status;

typedef enum { PKV_F32 = 0, PKV_F16 = 1, PKV_BF16 = 2 } pkv_dtype;

/* Pool geometry.  block_size is the tokens per block ([preview] step 1;
 * 16 in every workload here, and the only size the device kernels take). */
typedef struct {
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t max_blocks_per_seq; /* block-table capacity per sequence       */
  int32_t dtype;              /* pkv_dtype of the K/V pools and of q      */
} pkv_pool_desc;

/* Operational counters ([lesson] paragraph 8). */
typedef struct {
  int64_t free_blocks;
  int64_t used_blocks;
  int64_t alloc_failures;   /* calls refused for lack of free blocks      */
  int64_t tail_waste_slots; /* unused rows of last blocks, all sequences  */
  int64_t shared_blocks;    /* blocks with refcount > 1                   */
  int64_t cow_copies;       /* copy-on-write block copies queued so far   */
  int64_t forks;
  int64_t live_seqs;
} pkv_stats_t;

typedef struct pkv_pool pkv_pool;

/* Message describing the last error on this thread ("" if none). */
const char* pkv_last_error(void);

/* ---------------------------------------------------------------------------
 * Host: pool and allocator
 * ------------------------------------------------------------------------ */

/* Create a pool.  k_cache / v_cache are device arrays of the layout above,
 * 16-byte aligned (may both be NULL for allocator-only use; device calls then
 * fail with PKV_E_BAD_ARG).  free_order (host, num_blocks ids, a permutation; NULL =
 * 0..num_blocks-1) is the free list's initial content: the first block handed
 * out is free_order[0].  The free list is a stack: freed blocks are handed
 * out again most-recent first ([preview] step 4). */
pkv_status pkv_pool_create(const pkv_pool_desc* desc, void* k_cache, void* v_cache,
                           const int32_t* free_order, pkv_pool** out);
pkv_status pkv_pool_destroy(pkv_pool* pool);
/* Drop every sequence and restore the initial free list (the "reset" of the
 * cache API in [preview] "Lo que la Fase 22 construye").  Device contents are
 * left as they are. */
pkv_status pkv_pool_reset(pkv_pool* pool);
pkv_status pkv_pool_get_desc(const pkv_pool* pool, pkv_pool_desc* out);

/* New sequence holding n_tokens tokens (n_tokens >= 0): its block table
 * gets ceil(n_tokens / block_size) blocks taken from the free list, and
 * token t goes to row t % block_size of table entry t / block_size
 * ([preview] "La idea de PagedAttention", steps 2-3: one table per
 * sequence mapping logical blocks to physical ones, tokens filling blocks
 * in order).  Writes its id to *seq and, if slots != NULL, the slot of each
 * token to slots[0..n_tokens).  Fails with PKV_E_NO_BLOCKS, changing
 * nothing, when fewer blocks are free ([lesson] paragraph 7: admission is
 * decided in blocks and refused up front).  Ids count up from 0 and are
 * never reused. */
pkv_status pkv_seq_alloc(pkv_pool* pool, int32_t n_tokens, int32_t* seq, int64_t* slots);

/* Append n_tokens tokens to a sequence ([preview] step 3): a token goes into
 * the last block if it has room, otherwise into a newly taken block; nothing
 * already stored moves.  If the last block is partly filled and shared
 * (refcount > 1), the first token copies it first ([lesson] paragraph 6):
 * the appending sequence takes a fresh block, a (src, dst) copy is queued for
 * pkv_take_cow, and the source loses one reference. */
pkv_status pkv_seq_append(pkv_pool* pool, int32_t seq, int32_t n_tokens, int64_t* slots);

/* Append n_tokens to each of seqs[0..n_seqs) in that order, all or nothing.
 * slots (may be NULL) receives [n_seqs][n_tokens]. */
pkv_status pkv_seq_append_batch(pkv_pool* pool, const int32_t* seqs, int32_t n_seqs,
                                int32_t n_tokens, int64_t* slots);

/* New sequence sharing every block of parent (prefix sharing, parallel
 * samples; [lesson] paragraph 6, [preview] "Propiedades").  Takes no block:
 * every block's refcount goes up by one. */
pkv_status pkv_seq_fork(pkv_pool* pool, int32_t parent, int32_t* child);

/* New sequence sharing the first n_tokens tokens of `parent` (0 <= n_tokens
 * <= its length): the child's table is the parent's first
 * ceil(n_tokens / block_size) blocks, each gaining a reference; requests
 * with an identical prompt prefix point at the same read-only blocks
 * ([lesson] paragraph 6).  If n_tokens ends inside a block, the child's
 * first append copies that block (copy-on-write). */
pkv_status pkv_seq_fork_prefix(pkv_pool* pool, int32_t parent, int32_t n_tokens, int32_t* child);

/* Release a sequence ([preview] "La idea de PagedAttention", step 4: a
 * finished sequence returns its blocks to the free list; [lesson] paragraph
 * 6: reference counts decide when a shared block goes back to the pool):
 * each block of its table, front to back, loses one reference; blocks
 * reaching zero are pushed on the free list.  PKV_E_BAD_SEQ for an unknown
 * or already freed id (nothing changes). */
pkv_status pkv_seq_free(pkv_pool* pool, int32_t seq);

/* Batched retire / admit for a scheduler iteration (the same passages as
 * pkv_seq_free and pkv_seq_fork): pkv_seq_free on seqs[0 .. n_seqs) in
 * order, and pkv_seq_fork on parents[0 .. n) in order with the new ids in
 * children[0 .. n) (host arrays).  All or nothing: an unknown id
 * (PKV_E_BAD_SEQ) or an id given twice to the free (PKV_E_BAD_ARG) is found
 * before anything changes.  A parent may appear more than once. */
pkv_status pkv_seq_free_batch(pkv_pool* pool, const int32_t* seqs, int32_t n_seqs);
pkv_status pkv_seq_fork_batch(pkv_pool* pool, const int32_t* parents, int32_t n, int32_t* children);

pkv_status pkv_seq_length(const pkv_pool* pool, int32_t seq, int32_t* length);
/* Copy the sequence's block table to table[0..cap); *n = its length. */
pkv_status pkv_seq_table(const pkv_pool* pool, int32_t seq, int32_t* table, int32_t cap,
                         int32_t* n);
/* Slots of positions [first, first + n) of the sequence, slots[i] =
 * table[p / block_size] * block_size + p % block_size for p = first + i: the
 * gather list through which the paged cache is read ([preview] "La idea de
 * PagedAttention", step 5).  Fails (nothing written) unless
 * 0 <= first, 0 <= n and first + n <= the sequence's length. */
pkv_status pkv_seq_slots(const pkv_pool* pool, int32_t seq, int32_t first, int32_t n,
                         int64_t* slots);
/* Live sequence ids in ascending order. */
pkv_status pkv_live_seqs(const pkv_pool* pool, int32_t* ids, int32_t cap, int32_t* n);
/* Free blocks in the order they will be handed out next. */
pkv_status pkv_free_list(const pkv_pool* pool, int32_t* blocks, int32_t cap, int32_t* n);
/* Reference count of every block, refcounts[0..num_blocks). */
pkv_status pkv_refcounts(const pkv_pool* pool, int32_t* refcounts);
pkv_status pkv_stats(const pkv_pool* pool, pkv_stats_t* out);

/* Take the copy-on-write pairs queued since the last call ([lesson]
 * paragraph 6: when a branch diverges, copy-on-write gives it a new block
 * for the altered positions; the device half is pkv_copy_blocks), host
 * int32 pairs[i][0] = src, pairs[i][1] = dst.  If more than cap are queued, fails with PKV_E_BAD_ARG,
 * sets *n to the count and takes nothing.  Contract: enqueue pkv_copy_blocks
 * for these pairs, then pkv_write_kv for the appended tokens, before the next
 * append or fork; the pairs of one append batch never depend on each other. */
pkv_status pkv_take_cow(pkv_pool* pool, int32_t* pairs, int32_t cap, int32_t* n);

/* Block tables and context lengths of a batch, the arguments the attention
 * kernel takes to do its gathers itself ([preview] "La idea de
 * PagedAttention", step 5), written to host arrays
 * block_tables[n_seqs][table_stride] (row i = table of seqs[i], padded with
 * -1) and context_lens[n_seqs].  PKV_E_BAD_SEQ for an unknown id,
 * PKV_E_BAD_ARG if a table is wider than table_stride; nothing is written
 * then. */
pkv_status pkv_build_batch(const pkv_pool* pool, const int32_t* seqs, int32_t n_seqs,
                           int32_t* block_tables, int32_t table_stride, int32_t* context_lens);

/* ---------------------------------------------------------------------------
 * Host: continuous-batching scheduler with preemption
 * ------------------------------------------------------------------------ */

/* One iteration-level scheduler over one pool ("PagedAttention e continuous
 * batching", 01 · Conceito: composition revisited at every iteration
 * boundary, finished sequences leave, waiting ones enter, running ones
 * advance one token; the scheduler weighs free blocks, tokens per batch and
 * the prefill/decode mix, slicing long prefills; admission is decided in
 * blocks; paragraph 8 names the metrics kept here).
 * The pages give the goals, not the rules; the rules below are readings.
 *
 * Requests are known up front with an arrival iteration; the policy does
 * not look at output_len except to end a request.  A request's K/V length
 * is prompt_len + generated - 1 once it has generated >= 1 tokens.  Each
 * pkv_sched_step(), at iteration t:
 *   1. requests arriving at t join the back of the waiting queue (id order);
 *   2. every running sequence past its prefill needs room for one token,
 *      and the oldest running sequence still in prefill room for its next
 *      slice; while the blocks this needs exceed the free blocks, the most
 *      recently admitted running sequence is preempted (for that slice, only
 *      sequences newer than the prefill; for the decodes, any): its blocks are freed and it goes to the front of the
 *      waiting queue, to be recomputed (prefilled again over prompt_len +
 *      generated - 1 tokens) when readmitted.  So the oldest running
 *      request always advances and sliced prefills cannot deadlock;
 *   3. each of those sequences appends one token and generates one (DECODE
 *      item);
 *   4. budget = max_batch_tokens - decode tokens; running sequences still
 *      in prefill take, in admission order, min(rest, chunk_tokens, budget)
 *      tokens (PREFILL item), stopping at the first that does not fit in the
 *      free blocks;
 *   5. while budget > 0, the queue is not empty and fewer than max_running
 *      run: a head request that could never fit (its final length needs more
 *      blocks than the pool or a table holds) is rejected; otherwise it is
 *      admitted if its first slice fits, else admission stops (first come,
 *      first served).  If another running sequence of the same prefix_id has
 *      prefilled the prefix, the new sequence forks those prefix_len tokens
 *      (pkv_seq_fork_prefix: prefix hits) and prefills only the rest;
 *   6. a prefill that completes generates the request's first token (not
 *      again after a preemption); requests that reach output_len tokens
 *      finish; their sequences are freed at the start of the next step, so
 *      the items of a step stay valid until the next pkv_sched_step call
 *      (one more call after the last request finishes frees the rest).
 * Items list what the device must compute this iteration: (request, seq,
 * kind, first position, tokens); their K/V slots follow from the tables.
 * Copy-on-write pairs accumulate in the pool (pkv_take_cow). */
typedef struct {
  int32_t arrival;     /* iteration at which the request joins the queue    */
  int32_t prompt_len;  /* >= 1                                             */
  int32_t output_len;  /* tokens to generate, >= 1                        */
  int32_t klass;       /* request class, for metrics                      */
  int32_t prefix_id;   /* -1, or a shared-prompt-prefix id                 */
  int32_t prefix_len;  /* shared prefix tokens: a multiple of block_size,
                          0 <= prefix_len < prompt_len                     */
} pkv_request;

typedef struct {
  int32_t max_batch_tokens;  /* decode + prefill tokens per iteration       */
  int32_t chunk_tokens;      /* longest prefill slice per sequence per step */
  int32_t max_running;       /* running sequences at most                  */
} pkv_sched_config;

enum { PKV_ITEM_PREFILL = 0, PKV_ITEM_DECODE = 1 };
typedef struct {
  int32_t request;
  int32_t seq;
  int32_t kind;      /* PKV_ITEM_PREFILL or PKV_ITEM_DECODE */
  int32_t pos;       /* position of the first token computed */
  int32_t n_tokens;
} pkv_sched_item;

typedef struct {
  int32_t iteration;
  int32_t n_items;
  int32_t prefill_tokens;
  int32_t decode_tokens;
  int32_t admitted;
  int32_t preempted;
  int32_t finished;
  int32_t rejected;
} pkv_sched_step_info;

enum { PKV_REQ_PENDING = 0, PKV_REQ_WAITING = 1, PKV_REQ_RUNNING = 2, PKV_REQ_FINISHED = 3,
       PKV_REQ_REJECTED = 4 };
typedef struct {
  int32_t state;           /* PKV_REQ_*                                    */
  int32_t seq;             /* current sequence, or -1                      */
  int32_t admitted_at;     /* first admission iteration, or -1             */
  int32_t first_token_at;  /* iteration of the first generated token, or -1 */
  int32_t finished_at;     /* or -1                                        */
  int32_t generated;
  int32_t preemptions;
  int32_t prefix_hit_tokens;
} pkv_request_state;

typedef struct {
  int64_t iterations;
  int64_t waiting;
  int64_t running;
  int64_t finished;
  int64_t rejected;
  int64_t preemptions;
  int64_t prompt_tokens_admitted;  /* tokens each admission had to cover    */
  int64_t prefix_hit_tokens;       /* of those, served by shared blocks     */
  int64_t prefill_tokens;
  int64_t decode_tokens;
} pkv_sched_stats_t;

typedef struct pkv_sched pkv_sched;

/* reqs (host, n entries) are copied; request ids are their indices.  The
 * pool must hold no sequence the scheduler does not own while it runs. */
pkv_status pkv_sched_create(pkv_pool* pool, const pkv_sched_config* cfg, const pkv_request* reqs,
                            int32_t n, pkv_sched** out);
pkv_status pkv_sched_destroy(pkv_sched* s);
/* Run one iteration; items needs room for max_running entries. */
pkv_status pkv_sched_step(pkv_sched* s, pkv_sched_item* items, int32_t cap, pkv_sched_step_info* info);
pkv_status pkv_sched_request(const pkv_sched* s, int32_t request, pkv_request_state* out);
pkv_status pkv_sched_stats(const pkv_sched* s, pkv_sched_stats_t* out);

/* ---------------------------------------------------------------------------
 * Host: hybrid two-pool manager
 * ------------------------------------------------------------------------ */

/* A hybrid model keeps paged K/V only for its attention layers; its other
 * layers carry a recurrent state of fixed size per sequence, so a server
 * aware of the hybrid runs two pools with different lifecycles
 * ("PagedAttention e continuous batching", 01 · Conceito, paragraph 5).
 * pkv_hybrid pairs a K/V pool with a pool of num_slots state slots of
 * slot_bytes each (device memory at state_base, caller-owned; NULL for
 * host-only use).  A sequence admitted through it holds blocks and one
 * slot; a fork shares the parent's blocks (refcounts) but takes its own
 * slot and queues a (parent slot, child slot) copy, since the state changes
 * every step; free returns both.  Admission and fork are all-or-nothing
 * across the two pools and fail up front ([lesson] paragraph 7) with
 * PKV_E_NO_SLOTS or PKV_E_NO_BLOCKS.  The slot free list is a stack seeded
 * by slot_order (NULL = 0..num_slots-1; slot_order[0] is handed out first).
 * Sequences admitted here must be forked and freed here; appends go to the
 * K/V pool directly (pkv_seq_append). */
typedef struct pkv_hybrid pkv_hybrid;

typedef struct {
  int64_t free_slots;
  int64_t used_slots;
  int64_t refusals;      /* admissions / forks refused for lack of a slot or blocks */
  int64_t state_copies;  /* state copies queued so far */
} pkv_hybrid_stats_t;

pkv_status pkv_hybrid_create(pkv_pool* kv, int32_t num_slots, int64_t slot_bytes, void* state_base,
                             const int32_t* slot_order, pkv_hybrid** out);
pkv_status pkv_hybrid_destroy(pkv_hybrid* h);
pkv_status pkv_hybrid_admit(pkv_hybrid* h, int32_t n_tokens, int32_t* seq, int32_t* slot,
                            int64_t* slots);
pkv_status pkv_hybrid_fork(pkv_hybrid* h, int32_t parent, int32_t* child, int32_t* child_slot);
pkv_status pkv_hybrid_free(pkv_hybrid* h, int32_t seq);
pkv_status pkv_hybrid_slot(const pkv_hybrid* h, int32_t seq, int32_t* slot);
/* Queued (src slot, dst slot) state copies.  With pairs == NULL (or cap too
 * small) only *n is written and the queue is kept; otherwise the pairs are
 * written and the queue is cleared. */
pkv_status pkv_hybrid_take_copies(pkv_hybrid* h, int32_t* pairs, int32_t cap, int32_t* n);
pkv_status pkv_hybrid_stats(const pkv_hybrid* h, pkv_hybrid_stats_t* out);
/* Device: copy slot_bytes from slot pairs_dev[i][0] to slot pairs_dev[i][1]
 * (device int32 [n][2]); pairs naming a slot outside the pool are skipped.
 * Asynchronous on `stream`. */
pkv_status pkv_hybrid_copy_states(pkv_hybrid* h, const int32_t* pairs_dev, int32_t n, void* stream);

/* Split a joint memory budget into the two pools for sessions of
 * session_tokens tokens: a session costs ceil(session_tokens / block_size)
 * blocks of block_bytes plus one slot of slot_bytes ([lesson] paragraph 4's
 * arithmetic: 2 GiB of K/V + 144 MiB of state per 32,768-token session, ten
 * of which fit 23,859 MiB).  *sessions = budget / cost (floor); the state
 * pool gets that many slots and the K/V pool every whole block left. */
pkv_status pkv_hybrid_plan(int64_t budget_bytes, int64_t block_bytes, int32_t block_size,
                           int64_t slot_bytes, int64_t session_tokens, int32_t* sessions,
                           int32_t* num_blocks, int32_t* num_slots);

/* ---------------------------------------------------------------------------
 * Host: naive-vs-paged utilisation of one set of concurrent requests
 * ------------------------------------------------------------------------ */

/* The comparison the tutorial ("Paged Attention em Large Language Models
 * LLMs", opening paragraph and "Cache KV Ingênuo") sets up: a naive cache
 * reserves max_len tokens per request up front; the paged cache allocates
 * each request's tokens in block_size-token blocks.  The paged side runs
 * this library's allocator on a scratch host-only pool sized to fit (every
 * request allocated, statistics read, pool destroyed); the naive side is
 * n * max_len.  Token counts; lengths[i] in [1, max_len]. */
typedef struct {
  int64_t requests;
  int64_t tokens_used;
  int64_t naive_reserved_tokens;
  int64_t paged_blocks;
  int64_t paged_reserved_tokens;
  int64_t naive_waste_tokens;
  int64_t paged_waste_tokens;
} pkv_utilisation_t;

pkv_status pkv_utilisation(const int32_t* lengths, int32_t n, int32_t max_len, int32_t block_size,
                           pkv_utilisation_t* out);

/* ---------------------------------------------------------------------------
 * Host: decode plan
 * ------------------------------------------------------------------------ */

/* Split-K plan of a decode batch.  Each sequence's tokens are cut into
 * partitions of partition_tokens (a multiple of block_size; 0 selects
 * pkv_default_partition_tokens()).  One work item per (sequence, partition); items are ordered
 * longest first so that the GPU's in-order dispatch fills the tail with short
 * ones; equal lengths go partition-major (partition 0 of every sequence
 * first), so that sequences sharing a prefix read its blocks together.
 * Sequences with more than one partition write partial results that a
 * second kernel combines.
 *
 * plan (host int32, cap >= pkv_decode_plan_ints(...)) receives
 *   [0, 2*n_work)                     work items (seq index, partition index)
 *   [2*n_work, 2*n_work + num_seqs)   first partial index of each sequence,
 *                                     or -1 for single-partition sequences
 *   [.., + n_reduce)                  indices of multi-partition sequences.
 * Upload it unchanged and pass the device copy to pkv_paged_decode. */
typedef struct {
  int32_t num_seqs;
  int32_t block_size;
  int32_t partition_tokens;
  int32_t n_work;
  int32_t n_reduce;
  int32_t n_partials;
  int32_t plan_ints;
  int32_t max_context_len;
  /* K/V load policy hint, read by pkv_paged_decode: 0 (what pkv_decode_plan
   * sets) streams the tiles past the caches (nontemporal loads, the faster
   * choice when every tile is read once); 1 reads them through the caches
   * (4 waves per workgroup), for batches whose sequences share blocks, so
   * that the repeated reads of a shared prefix hit in L2.
   * pkv_prepare_decode sets 1 when at least a quarter of the batch's
   * context tokens lie in blocks held by more than one sequence.  Any value
   * gives the same results. */
  int32_t shared_kv;
  /* Shared-block section (pkv_decode_plan_shared; all 0 from
   * pkv_decode_plan): nodes of blocks held in common by several sequences
   * of the batch, read once for all of them by a separate launch. */
  int32_t n_nodes;             /* shared nodes (0: no shared section)          */
  int32_t n_wide_nodes;        /* the first n_wide_nodes are wide, the rest narrow */
  int32_t n_shared_items;      /* wide workgroups per KV head                   */
  int32_t n_narrow_items;      /* narrow workgroups per KV head                 */
  int32_t shared_chunk_blocks; /* smallest blocks per wide work item            */
  int32_t narrow_chunk_blocks; /* smallest blocks per narrow work item          */
  int32_t shared_group;        /* query heads per KV head the plan was made for */
  int32_t off_shared;          /* int offset of the shared section in the plan  */
  /* Mean blocks per work item, rounded up.  The decode gives short items
   * fewer waves per workgroup (4 from 16 blocks, 2 from 6, else 1) unless
   * PKV_DECODE_WAVES says otherwise. */
  int32_t item_blocks;
} pkv_decode_plan_info;

/* Upper bound of the plan length for these lengths. */
pkv_status pkv_decode_plan_ints(const int32_t* context_lens, int32_t num_seqs, int32_t block_size,
                                int32_t partition_tokens, int32_t* plan_ints);
pkv_status pkv_decode_plan(const int32_t* context_lens, int32_t num_seqs, int32_t block_size,
                           int32_t partition_tokens, int32_t* plan, int32_t cap,
                           pkv_decode_plan_info* info);

/* Split-K plan of a batch of live sequences of `pool` that reads every block
 * held in common by several of them once for all its holders ("PagedAttention
 * e continuous batching", 01 · Conceito, paragraph 6: requests with an
 * identical prompt prefix point at the same read-only blocks; "04 — Hacia
 * PagedAttention", Propiedades: prefix sharing comes free).
 *
 * The sequences' tables are taken from the pool as they stand.  Sequences
 * whose tables agree on a run of blocks form a node: blocks [j0, j1) of the
 * table of its first member, which every member holds at the same positions,
 * full in every member (a sequence's last block is never in a node).  Nodes
 * nest like a prefix tree: the members of a node share all blocks of its
 * ancestors.  A node of more than 16 (member, query head) columns is wide:
 * its blocks are cut into chunks and its members into column sets of
 * 128 / group sequences, each (chunk, column set, KV head) one workgroup
 * of the wide launch, which stages the chunk through LDS once for all the
 * set's columns.  A narrow node's blocks are cut into chunks, each (chunk,
 * KV head) one workgroup of the narrow launch, whose waves stream the
 * chunk's blocks for its columns.  Both write one split-K record per
 * member, query head and chunk.  A chunk is chunk_tokens / block_size
 * blocks (at least 64 for a narrow node), or, for chunk_tokens = 0, at
 * least 64 blocks, long nodes being cut into at most
 * 8 chunks (wide) or 4 (narrow); shared_chunk_blocks / narrow_chunk_blocks
 * give the smallest size of each kind and every node stores its own.  Every
 * sequence then attends over the rest of its blocks (from private_start) as
 * in pkv_decode_plan, and its records, shared ones first, are combined.
 * Nodes are built only when at least a quarter of the batch's context tokens
 * lie in them, for fp16 / bf16 pools of head_dim 128 and group = num_q_heads
 * / num_kv_heads dividing 16; otherwise the result is pkv_decode_plan's
 * (with shared_kv set as pkv_batch_shared_kv would).  chunk_tokens: a
 * multiple of block_size, or 0 (the sizes above; the environment variable
 * PKV_SHARED_CHUNK_TOKENS, read at every call, replaces 0 for tuning).  A
 * sequence's shared records (one per node chunk on its path) are capped at
 * PKV_MAX_SHARED_RECORDS: a node stops where the cap would be passed.
 *
 * Layout: pkv_decode_plan's, then, from info->off_shared when n_nodes > 0,
 *   [num_seqs]       private_start: first block of each sequence's own part
 *   [num_seqs]       n_shared: shared records of each sequence
 *   [num_seqs]       order: batch indices, each node's members contiguous
 *   [9 * n_nodes]    nodes (rep, j0, j1, first member in order, members,
 *                    first record, first item of its kind, column sets,
 *                    blocks per chunk), the n_wide_nodes wide ones first
 * where a member s of node v writes, for chunk c, the record at
 * part_offset[s] + first record + c.  Upload it unchanged. */
/* A sequence owns at most this many shared records (pkv_decode_plan_shared
 * stops a node early rather than pass it; workspace bounds count on it). */
#define PKV_MAX_SHARED_RECORDS 16
pkv_status pkv_decode_plan_shared_ints(const pkv_pool* pool, const int32_t* seqs, int32_t n_seqs,
                                       int32_t partition_tokens, int32_t* plan_ints);
pkv_status pkv_decode_plan_shared(const pkv_pool* pool, const int32_t* seqs, int32_t n_seqs,
                                  int32_t partition_tokens, int32_t num_q_heads, int32_t chunk_tokens,
                                  int32_t* plan, int32_t cap, pkv_decode_plan_info* info);

/* Device workspace bytes pkv_paged_decode needs for this plan: the split-K
 * partial records (from the workspace's start) and completion tickets for
 * num_seqs x num_q_heads (at its end; they must be zero before the first
 * launch and every launch leaves them zero).  A workspace reused by
 * launches of different shapes must be sized for the largest of them
 * (pkv_decode_workspace_bound does that), so that no launch's records
 * overlap another's tickets. */
size_t pkv_decode_workspace_bytes(const pkv_decode_plan_info* info, int32_t num_q_heads,
                                  int32_t head_dim);

/* Workspace bytes that suffice for every plan of at most max_seqs sequences
 * no longer than max_context_len tokens, pkv_decode_plan's and
 * pkv_decode_plan_shared's (each sequence may add PKV_MAX_SHARED_RECORDS
 * shared records), 0 on bad arguments; for callers that size the workspace
 * once. */
size_t pkv_decode_workspace_bound(int32_t max_seqs, int32_t max_context_len, int32_t block_size,
                                  int32_t partition_tokens, int32_t num_q_heads, int32_t head_dim);

/* Partition length that partition_tokens = 0 selects. */
int32_t pkv_default_partition_tokens(void);

/* Fill mode: a stepper created with partition_tokens = PKV_PARTITION_FILL
 * picks, at every iteration, the smallest partition that lets all of the
 * launch's workgroups be resident on the GPU at once
 * (pkv_decode_fill_partition over pkv_decode_occupancy), else the default.
 * pkv_prepare_decode_bytes, pkv_stepper_slot_bytes and
 * pkv_decode_workspace_bound size buffers for it as for PKV_FILL_MIN_TOKENS;
 * the plan functions themselves take concrete sizes only. */
#define PKV_PARTITION_FILL (-1)
#define PKV_FILL_MIN_TOKENS 512

/* Smallest multiple of block_size P >= min_tokens for which
 * workgroups_per_item * sum_i ceil(context_lens[i] / P) <= resident, i.e. a
 * split-K plan whose workgroups all fit on the GPU at once (one dispatch
 * round: no tail of a partly filled second round, and the finest split that
 * does so).  0 when even one partition per sequence needs more; the caller
 * then keeps its partition size.  Host only. */
int32_t pkv_decode_fill_partition(const int32_t* context_lens, int32_t num_seqs, int32_t block_size,
                                  int32_t workgroups_per_item, int64_t resident, int32_t min_tokens);

/* ---------------------------------------------------------------------------
 * Host: chunked-prefill plan
 * ------------------------------------------------------------------------ */

/* Work list of a chunked-prefill launch ("PagedAttention e continuous
 * batching", 01 · Conceito, the scheduler paragraph: long prefills are cut
 * into slices).  Sequence i brings q_lens[i] >= 1 new tokens that are the
 * last q_lens[i] of its context_lens[i] tokens (already appended and
 * written).  A tile is tile_tokens consecutive query tokens of one
 * sequence; tile_tokens is 128 / Gw with Gw the largest power of two <= 16
 * dividing H_q / H_kv (Gw query heads of one KV head share a tile).  A tile
 * whose last query attends more than max_keys keys (max_keys > 0) is split
 * into parts of at most max_keys keys (whole 32-key stages); max_keys = 0
 * never splits; max_keys < 0 splits only a launch that would have fewer
 * than 512 workgroups, with a limit that brings it to about 512 (at least
 * 1024 keys per part).  Each part is a work item, and the parts' partial softmax states are merged in the same
 * launch (workspace: pkv_prefill_workspace_bytes).  The kernel runs every
 * item for every KV head.  Items are ordered by decreasing number of keys,
 * except that a launch of at most 512 workgroups (items x KV heads x head
 * groups: two per CU of MI355X, one round) takes its second half in
 * increasing order, so that workgroups j and j + 256, which the dispatcher
 * puts on one CU, hold a long and a short item.
 *
 * plan (host int32, cap >= pkv_prefill_plan_ints(...)) receives
 *   [0, 6*n_work)                      items (sequence, tile, first stage,
 *                                       end stage, split tile index or -1,
 *                                       part index)
 *   [6*n_work, .. + num_seqs + 1)      q_start: first query row of each
 *                                       sequence in q / out (prefix sums)
 *   [.., + 2*n_split)                  per split tile (first partial, parts)
 * Upload it unchanged and pass the device copy to pkv_paged_prefill. */
typedef struct {
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t tile_tokens;
  int32_t n_work;
  int32_t total_q;
  int32_t max_context_len;
  int32_t plan_ints;
  int32_t n_split;     /* tiles split into several parts                 */
  int32_t n_partials;  /* parts of split tiles, summed                   */
} pkv_prefill_plan_info;

pkv_status pkv_prefill_plan_ints(const int32_t* q_lens, const int32_t* context_lens,
                                 int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t max_keys, int32_t* plan_ints);
pkv_status pkv_prefill_plan(const int32_t* q_lens, const int32_t* context_lens, int32_t num_seqs,
                            int32_t num_q_heads, int32_t num_kv_heads, int32_t max_keys,
                            int32_t* plan, int32_t cap, pkv_prefill_plan_info* info);
/* Device workspace bytes pkv_paged_prefill needs for this plan (0 when no
 * tile is split): one record per (part, head group, tile row): o[head_dim],
 * m, l as fp32 padded to whole 128-byte lines, from the workspace's start;
 * completion tickets [n_split][H_q / Gw] int32 at its end.  The tickets
 * must be zero before the first launch; every launch leaves them zero.  A
 * workspace reused by launches of different shapes must be sized for the
 * largest records plus the largest tickets. */
size_t pkv_prefill_workspace_bytes(const pkv_prefill_plan_info* info, int32_t head_dim);

/* ---------------------------------------------------------------------------
 * Host: one decode iteration's metadata in one staging buffer
 * ------------------------------------------------------------------------ */

/* Where pkv_prepare_decode put each array inside the staging buffer (byte
 * offsets from its start, each 256-byte aligned). */
typedef struct {
  int32_t n_seqs;
  int32_t append_tokens;
  int32_t n_pairs;       /* copy-on-write pairs taken by this call        */
  int32_t table_stride;
  int64_t off_slots;     /* int64 [n_seqs][append_tokens]                 */
  int64_t off_pairs;     /* int32 [n_pairs][2]                            */
  int64_t off_tables;    /* int32 [n_seqs][table_stride]                  */
  int64_t off_lens;      /* int32 [n_seqs]                                */
  int64_t off_plan;      /* int32 [plan.plan_ints]                        */
  int64_t bytes;         /* bytes used from the start of the buffer       */
  pkv_decode_plan_info plan;
} pkv_batch_layout;

/* Staging bytes pkv_prepare_decode needs at most for a batch of up to
 * max_seqs sequences whose tables fit table_stride blocks. */
size_t pkv_prepare_decode_bytes(int32_t max_seqs, int32_t append_tokens, int32_t table_stride,
                                int32_t block_size, int32_t partition_tokens);

/* The host half of a continuous-batching decode iteration ([lesson]
 * paragraph 7: running sequences advance one token per iteration), in one
 * call: append append_tokens (0 or more) to each of seqs[0..n_seqs) in that
 * order (pkv_seq_append_batch), take the copy-on-write pairs, build block
 * tables and context lengths (pkv_build_batch) and the split-K plan, all
 * written into the host buffer `staging` (ideally pinned) at the offsets
 * returned in *layout.  The plan is pkv_decode_plan_shared's for
 * num_q_heads > 0 (blocks held in common read once for their holders) and
 * pkv_decode_plan's with the load-policy hint for num_q_heads = 0.  Upload
 * the first layout->bytes bytes unchanged to a device buffer; the device
 * arrays then sit at the same offsets.  All or nothing: on error the pool is
 * unchanged. */
pkv_status pkv_prepare_decode(pkv_pool* pool, const int32_t* seqs, int32_t n_seqs,
                              int32_t append_tokens, int32_t table_stride,
                              int32_t partition_tokens, int32_t num_q_heads, void* staging,
                              size_t staging_bytes, pkv_batch_layout* layout);

/* The decode plan's K/V load-policy hint for a batch of live sequences
 * (pkv_decode_plan_info.shared_kv): 1 when at least a quarter of their
 * context tokens lie in blocks that more than one sequence holds (forked
 * prefixes), else 0.  pkv_prepare_decode applies the same rule after its
 * append; callers that plan with pkv_decode_plan can set the field from this.
 * Read only.  PKV_E_BAD_SEQ for an unknown sequence id. */
pkv_status pkv_batch_shared_kv(const pkv_pool* pool, const int32_t* seqs, int32_t n_seqs,
                               int32_t* shared_kv);

/* ---------------------------------------------------------------------------
 * One decode iteration in one call (host + device)
 * ------------------------------------------------------------------------ */

/* A stepper runs continuous-batching decode iterations ([lesson] paragraph 7:
 * at every iteration the running sequences advance one token) over a pool.
 * The caller provides PKV_STEPPER_SLOTS staging slots of slot_bytes each, in
 * pinned host memory (staging_host) and in device memory (staging_dev), the
 * decode workspace (zeroed before first use, pkv_decode_workspace_bytes for
 * the largest batch) and a copy stream (NULL: uploads go on the compute
 * stream).  The stepper creates two HIP events (one completion event per
 * group of four slots) and nothing else.  The compute stream never waits on
 * another stream; the host waits for each upload before launching (it
 * synchronises the copy stream, so give each stepper a copy stream of its
 * own or one that carries nothing slow), and for the iterations that last
 * used a slot before rewriting it.
 * All calls on one stepper must use the same compute stream.
 * partition_tokens: a concrete size, 0 (the default) or PKV_PARTITION_FILL
 * (re-chosen at every iteration from the batch's lengths after the append;
 * size slots and workspace with the same value). */
#define PKV_STEPPER_SLOTS 8
typedef struct pkv_stepper pkv_stepper;

size_t pkv_stepper_slot_bytes(int32_t max_seqs, int32_t table_stride, int32_t block_size,
                              int32_t partition_tokens);
pkv_status pkv_stepper_create(pkv_pool* pool, int32_t max_seqs, int32_t table_stride,
                              int32_t num_q_heads, int32_t partition_tokens, void* staging_host,
                              void* staging_dev, size_t slot_bytes, void* workspace,
                              size_t workspace_bytes, void* copy_stream, pkv_stepper** out);
/* Waits for the stepper's own uploads and launches to finish, then frees it. */
pkv_status pkv_stepper_destroy(pkv_stepper* stepper);

/* One iteration over seqs[0..n_seqs):
 *   host    pkv_prepare_decode (append one token to each sequence, take the
 *           copy-on-write pairs, tables, lengths, split-K plan) into the next
 *           staging slot; all or nothing, the pool is unchanged on error;
 *   upload  one async copy of the slot on the copy stream;
 *   stream  wait for that upload, pkv_copy_blocks for the pairs, then
 *           pkv_paged_decode with k_new/v_new (the appended tokens' rows,
 *           [n_seqs][num_kv_heads][head_dim]) stored and attended.
 * The host may run up to PKV_STEPPER_SLOTS iterations ahead of the device.
 * ev_before / ev_after: optional hipEvent_t attached to the decode dispatch
 * (start and end of the kernel's execution on `stream`); when the batch is
 * empty no kernel runs and they are not recorded.  layout_out / slot_out (optional) receive the iteration's
 * staging layout and slot index (the host slot stays readable until the slot
 * comes round again, PKV_STEPPER_SLOTS iterations later). */
pkv_status pkv_stepper_step(pkv_stepper* stepper, const int32_t* seqs, int32_t n_seqs,
                            const void* q, const void* k_new, const void* v_new, float* out,
                            float scale, void* stream, void* ev_before, void* ev_after,
                            pkv_batch_layout* layout_out, int32_t* slot_out);

/* ---------------------------------------------------------------------------
 * Device (HIP, gfx950): asynchronous on `stream`
 * ------------------------------------------------------------------------ */

/* Workgroups pkv_paged_decode launches per work item (KV heads x query-head
 * groups) and how many of its workgroups the current device holds resident
 * at once (the occupancy of the kernel this pool and head count select,
 * times the number of compute units): the inputs of
 * pkv_decode_fill_partition.  Makes no launch. */
pkv_status pkv_decode_occupancy(const pkv_pool* pool, int32_t num_q_heads, int32_t* workgroups_per_item,
                                int64_t* resident);

/* Copy-on-write copies ([lesson] paragraph 6): for each pair, K[dst] = K[src]
 * and V[dst] = V[src] over all heads and rows.  pairs: device int32
 * [n_pairs][2].  Pairs with an id outside the pool are skipped. */
pkv_status pkv_copy_blocks(const pkv_pool* pool, const int32_t* pairs, int32_t n_pairs,
                           void* stream);

/* Store new tokens' K and V rows at their slots ([preview] step 3; the
 * "reshape_and_cache" step of a decode iteration).  k_new, v_new: device
 * [n_tokens][num_kv_heads][head_dim] of the pool dtype; slot_mapping: device
 * int64 [n_tokens]; a negative slot skips the token, as does a slot outside
 * the pool.  Bit-exact copy. */
pkv_status pkv_write_kv(const pkv_pool* pool, const void* k_new, const void* v_new,
                        const int64_t* slot_mapping, int32_t n_tokens, void* stream);

/* Read tokens' K and V rows back out of the pool into dense arrays: the
 * "read" of the cache surface (append, read, reset) that the paged cache
 * keeps from the dense one ([preview] "Lo que la Fase 22 construye hacia la
 * Fase 27", first item).  k_out, v_out: device [n_tokens][num_kv_heads]
 * [head_dim] of the pool dtype, 16-byte aligned, written by the call;
 * slot_mapping: device int64 [n_tokens] (pkv_seq_slots gives a sequence's).
 * The inverse of pkv_write_kv: row t of k_out / v_out is the pool's row at
 * slot_mapping[t], bit for bit; a negative slot, or one outside the pool,
 * gives a row of zeros. */
pkv_status pkv_read_kv(const pkv_pool* pool, const int64_t* slot_mapping, int32_t n_tokens,
                       void* k_out, void* v_out, void* stream);

/* PagedAttention decode ([lesson] paragraph 3, [preview] step 5): for every
 * sequence i and query head h,
 *     out[i][h] = softmax_j(scale * q[i][h] . K_i[j][g]) . V_i[j][g]
 * over the context_lens[i] tokens of sequence i, where K_i / V_i row j is read
 * from the pool through block_tables[i][j / block_size] and
 * g = h / (num_q_heads / num_kv_heads).  Paging does not change the result of
 * dense attention ([preview] "Lo que deberías llevarte", item 2).
 *   q:            device [num_seqs][num_q_heads][head_dim], pool dtype, 16-byte aligned
 *   k_new, v_new: device [num_seqs][num_kv_heads][head_dim], pool dtype, or
 *                 both NULL.  When given, they are the K/V rows of each
 *                 sequence's newest token (position context_lens[i] - 1, the
 *                 token just appended, [preview] step 3): the kernel stores
 *                 them into the pool at that position and attends over them,
 *                 i.e. pkv_write_kv and decode in one launch.  Copy-on-write
 *                 copies of the same iteration must be enqueued before.
 *   out:          device float32 [num_seqs][num_q_heads][head_dim], 4-byte aligned
 *   block_tables: device int32 [num_seqs][table_stride]
 *   context_lens: device int32 [num_seqs]; every entry >= 1 and equal to the
 *                 lengths given to pkv_decode_plan
 *   plan, info:   device copy of the plan and its host-side info
 *   workspace:    device, 16-byte aligned, >= pkv_decode_workspace_bytes(info, ...) bytes.  Split-K
 *                 partial records fill it from its start; its last bytes
 *                 hold completion tickets, which must be zero before the
 *                 first call (allocate it zeroed) and which every call
 *                 leaves zero.  Calls that share a workspace must not
 *                 overlap in time.
 *   scale:        finite and > 0 (1/sqrt(head_dim) for the pages' attention),
 *                 else PKV_E_BAD_ARG.
 * One kernel launch: multi-partition sequences are combined by the last
 * workgroup of each sequence and head group to finish.
 * Arithmetic: fp32 accumulation and an online (running max) softmax; the
 * output is float32.  Table entries outside the pool read nothing.
 * Kernels: grouped-query batches (num_q_heads / num_kv_heads >= 2) of fp16 or
 * bf16 with head_dim 128 run the two products on the matrix cores (the
 * softmax weights enter them as fp16, or as a bf16 head plus a bf16
 * remainder); every other shape runs on the vector ALUs.  The environment
 * variable PKV_DECODE_MFMA=0, read at every call, selects the vector kernel
 * for all shapes. */
pkv_status pkv_paged_decode(const pkv_pool* pool, const void* q, const void* k_new,
                            const void* v_new, float* out, int32_t num_seqs, int32_t num_q_heads,
                            const int32_t* block_tables, int32_t table_stride,
                            const int32_t* context_lens, float scale, const int32_t* plan,
                            const pkv_decode_plan_info* info, void* workspace,
                            size_t workspace_bytes, void* stream);

/* The same decode as two launches, same arguments: the partition kernel
 * (writes out for single-partition sequences, partials to the workspace
 * otherwise; stores k_new/v_new like pkv_paged_decode), then a separate kernel
 * that combines the partials.  Kept for comparison and for callers that want
 * to schedule the combine apart. */
pkv_status pkv_paged_decode_partitions(const pkv_pool* pool, const void* q, const void* k_new,
                                       const void* v_new, float* out, int32_t num_seqs,
                                       int32_t num_q_heads, const int32_t* block_tables,
                                       int32_t table_stride, const int32_t* context_lens,
                                       float scale, const int32_t* plan,
                                       const pkv_decode_plan_info* info, void* workspace,
                                       size_t workspace_bytes, void* stream);
pkv_status pkv_paged_decode_reduce(const pkv_pool* pool, const void* q, const void* k_new,
                                   const void* v_new, float* out, int32_t num_seqs,
                                   int32_t num_q_heads, const int32_t* block_tables,
                                   int32_t table_stride, const int32_t* context_lens, float scale,
                                   const int32_t* plan, const pkv_decode_plan_info* info,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* pkv_paged_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments without the workspace, the same kernels
 * and results.  The split-K records and completion tickets live in a fixed
 * scratch array inside the library, PKV_NOALLOC_SCRATCH_BYTES on each GPU
 * the library runs on, held until the process ends; its device address is
 * looked up once per device, on that device's first call.  A batch whose
 * pkv_decode_workspace_bytes exceeds it is refused with PKV_E_BAD_ARG and
 * nothing is launched.  The call allocates nothing; it clears the tickets it
 * will use with a small kernel before the decode.  Every call on a GPU
 * shares that GPU's scratch: calls that overlap in time on one GPU (other
 * streams, other threads) race and must be serialised by the caller. */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
pkv_status pkv_paged_decode_noalloc(const pkv_pool* pool, const void* q, const void* k_new,
                                    const void* v_new, float* out, int32_t num_seqs,
                                    int32_t num_q_heads, const int32_t* block_tables,
                                    int32_t table_stride, const int32_t* context_lens, float scale,
                                    const int32_t* plan, const pkv_decode_plan_info* info,
                                    void* stream);

/* Causal attention of chunked-prefill queries through the block tables:
 * query t of sequence i (row q_start[i] + t of q and out) sits at position
 * context_lens[i] - q_lens[i] + t and attends to that sequence's positions
 * 0 .. that position ("PagedAttention e continuous batching", 01 · Conceito:
 * the kernel reads through the block table, paragraph 3; long prefills are
 * sliced, the scheduler paragraph).  The chunk's K/V must already be in the
 * pool (pkv_seq_append / pkv_write_kv).  q: device [total_q][H_q][head_dim]
 * in the pool dtype; out: device fp32 [total_q][H_q][head_dim] (q, out and
 * workspace 16-byte aligned, else PKV_E_BAD_ARG); block_tables
 * / context_lens as for decode; plan / info from pkv_prefill_plan (plan
 * uploaded); workspace (device, zeroed once, every launch leaves its
 * tickets zero) of at least pkv_prefill_workspace_bytes(info, head_dim)
 * bytes, may be NULL when no tile is split.  fp16 and bf16 pools, head_dim
 * 64 or 128 (else PKV_E_UNSUPPORTED); the products run on the matrix cores
 * with fp32 accumulation, the softmax weights rounded to fp16.  A bf16 pool's
 * V is converted to fp16 as it is staged (exact below 2^16 in magnitude), and
 * every bf16 call makes two launches: that pass, then an exact pass (V in
 * bf16, weights as a bf16 head + remainder) whose workgroups exit at once
 * unless the first pass met a V value of magnitude 2^16 or more.  The first
 * pass records that in one word per device inside the library, raised to
 * the call's number (numbers only grow), so concurrent calls can cause an
 * exact pass that was not needed but never skip one that was.  A captured
 * graph keeps the number the call had at capture: once one replay meets such
 * a value, every later replay of that graph also runs the exact pass (its
 * results stay exact).  Setting the environment variable
 * PKV_PREFILL_BF16_EXACT=1 runs the exact pass alone.
 * Asynchronous on `stream`; allocates nothing. */
pkv_status pkv_paged_prefill(const pkv_pool* pool, const void* q, float* out, int32_t num_seqs,
                             int32_t num_q_heads, const int32_t* block_tables, int32_t table_stride,
                             const int32_t* context_lens, float scale, const int32_t* plan,
                             const pkv_prefill_plan_info* info, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Measurement aid, not part of the decode path: reads every K/V tile that
 * pkv_paged_decode would read for this plan (the decode gathers tiles
 * through the block tables: "04 — Hacia PagedAttention", La idea de
 * PagedAttention, step 5), with the decode's work items, order and wave
 * layout, and none of its arithmetic; its duration is the gather ceiling a
 * decode launch is compared with.  mode: PKV_PROBE_REGS (tiles into two
 * alternating register sets, nontemporal loads, as the VALU decode),
 * PKV_PROBE_CACHED (the same with cached loads) or PKV_PROBE_LDS (tiles
 * loaded straight into a per-wave two-stage LDS ring, then read back; tiles
 * of at most 4 KiB).  waves: 1, 2 or 4 per workgroup.  lds_pad: unused
 * dynamic LDS bytes per workgroup (0 to 65536), which caps how many
 * workgroups a compute unit holds at once (occupancy sweeps).  plan / info: a
 * decode plan of pkv_decode_plan (no shared-block nodes), plan uploaded;
 * block_tables / context_lens as for decode.  out: device uint32
 * [info->n_work][num_kv_heads][waves], the XOR of every 32-bit word of the
 * K and V tiles of blocks b0 + w, b0 + w + waves, ... of the item's
 * partition [b0, b1) (all 16 rows of each block).  Errors: PKV_E_BAD_ARG,
 * PKV_E_UNSUPPORTED (block size other than 16, a tile that is not a
 * multiple of 1 KiB, or LDS mode with a tile over 4 KiB).  Asynchronous on
 * `stream`; allocates nothing. */
#define PKV_PROBE_REGS 0
#define PKV_PROBE_CACHED 1
#define PKV_PROBE_LDS 2
pkv_status pkv_gather_probe(const pkv_pool* pool, const int32_t* block_tables, int32_t table_stride,
                            const int32_t* context_lens, int32_t num_seqs, const int32_t* plan,
                            const pkv_decode_plan_info* info, int32_t mode, int32_t waves,
                            int32_t lds_pad, uint32_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */

/*
 * brs.h -- block-retrieval sparse attention over a long key/value memory.
 *
 * The library implements one decode/prefill step of the method shared by
 * MemLong (arXiv 2408.16967), InfLLM (arXiv 2402.04617), Landmark Attention
 * (Mohtashami & Jaggi, 2023) and RetrievalAttention (arXiv 2409.10516):
 *
 *   1. brs_mem_append      -- store new K/V rows and, for every block the
 *                             append completes, its representative vectors;
 *   2. brs_score_blocks    -- relevance of every candidate block to the query;
 *   3. brs_select_topk     -- the k best blocks per score head;
 *   4. brs_retrieval_attention -- exact softmax attention over the sinks,
 *                             the local window and the selected blocks;
 *   brs_retrieval_step        -- 2 to 4 in one call.
 *
 * Conventions shared by every call
 * --------------------------------
 * - All pointers to tensors are DEVICE pointers (HIP device memory) unless a
 *   parameter says "host".  The caller allocates and owns all of them; the
 *   library never allocates or frees device memory and never creates
 *   streams.  It keeps no state between calls, with two exceptions:
 *   brs_retrieval_step_static's workspace, a fixed device array the library
 *   holds on every GPU it runs on until the process ends, and the events
 *   armed by brs_profile_next_attention (per thread, until the next
 *   attention call takes them).
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *   device work is enqueued on it; results are ready once the caller has
 *   synchronised that stream.
 * - Every call validates its arguments on the host before it enqueues
 *   anything; a call that returns an error has enqueued nothing and changed
 *   nothing (brs_mem_append leaves m->length unchanged).
 * - Return value: BRS_OK (0) or a negative BRS_E_* code; brs_last_error()
 *   then gives a message (thread-local, valid until the next call on the
 *   same thread).
 * - Tensors are dense, row-major, with the shapes given below ([a][b][c]
 *   means c varies fastest).  "dtype" is the memory's brs_dtype.
 *
 * Memory layout (caller-owned, described by brs_memory)
 * -------------------------------------------------------
 *   k, v : [batch][n_kv_heads][capacity][row_stride]  dtype
 *          token t of (batch, head) is row t; columns [head_dim, row_stride)
 *          are padding that brs_mem_append sets to zero.
 *   reps : [batch][rep_heads][capacity / block_size][reps_per_block][rep_dim]
 *          rep_dtype; block b of a head covers tokens [b*B, (b+1)*B), B =
 *          block_size, and its representatives are written when the block
 *          is complete.
 * A block is the memory unit that is scored and retrieved as a whole (the
 * pages' "chunk", "memory unit", "block"); its tokens are one contiguous span
 * of rows, so a retrieved block is read with contiguous loads.
 */
#ifndef BRS_H_
#define BRS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BRS_VERSION 3

/* Storage types. */
typedef enum { BRS_F32 = 0, BRS_BF16 = 1 } brs_dtype;

/* How a block's representatives are obtained (MemLong 2.3.2, InfLLM
 * "method", Landmark Attention "proposed method"):
 *   BRS_REP_MEAN    R = 1: the mean of the block's keys, summed in float64
 *                   and rounded once (nearest-even) to dtype;
 *   BRS_REP_TOPNORM the R keys of the block with the largest L2 norm (squared
 *                   norms summed in float64; ties to the lower token), copied
 *                   unchanged, largest first -- a stand-in for InfLLM's
 *                   "tokens that received the most attention";
 *   BRS_REP_GIVEN   caller-supplied vectors of head_dim (Landmark keys);
 *   BRS_REP_EMBED   caller-supplied chunk embeddings of rep_dim, one per block
 *                   for the whole sequence (rep_heads = 1), scored by cosine
 *                   (MemLong's retriever embeddings);
 *   BRS_REP_ATTNSCORE the R keys of the block that received the most
 *                   attention while they were in the local window (InfLLM
 *                   "method": representative tokens chosen by their
 *                   attention scores).  brs_mem_append builds nothing; the
 *                   caller accumulates the attention with brs_window_mass
 *                   after each attention call and builds a block's
 *                   representatives with brs_reps_from_mass when the block
 *                   becomes a candidate. */
typedef enum {
  BRS_REP_MEAN = 0,
  BRS_REP_TOPNORM = 1,
  BRS_REP_GIVEN = 2,
  BRS_REP_EMBED = 3,
  BRS_REP_ATTNSCORE = 4
} brs_rep_mode;

enum {
  BRS_OK = 0,
  BRS_E_INVAL = -1,        /* bad shape, pointer, mode, alignment or range  */
  BRS_E_CAPACITY = -2,     /* append would exceed capacity                   */
  BRS_E_UNSUPPORTED = -3,  /* valid but outside what the kernels implement   */
  BRS_E_HIP = -4,          /* a HIP launch failed                            */
  BRS_E_EMPTY = -5,        /* some query would attend no token at all        */
  BRS_E_WORKSPACE = -6     /* workspace missing or too small                 */
};

/* Descriptor of one layer's memory.  All enums are stored as int32_t so the
 * layout is fixed for foreign-function callers.  Constraints (checked by
 * every call): batch, n_kv_heads, head_dim, block_size, reps_per_block,
 * rep_dim >= 1; row_stride >= head_dim; 0 <= length <= capacity;
 * rep_heads = n_kv_heads for MEAN/TOPNORM/GIVEN/ATTNSCORE and 1 for EMBED;
 * rep_dim = head_dim and rep_dtype = dtype unless rep_mode is EMBED;
 * reps_per_block = 1 for MEAN and EMBED; reps_per_block <= min(block_size,
 * 64) for TOPNORM and ATTNSCORE; row_stride * element size is a multiple of 4
 * bytes; k, v, reps non-NULL and 16-byte aligned. */
typedef struct brs_memory {
  int32_t dtype;           /* brs_dtype of k, v and the queries            */
  int32_t batch;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t row_stride;      /* elements between consecutive token rows      */
  int32_t block_size;      /* B, tokens per block                          */
  int32_t reps_per_block;  /* R                                            */
  int32_t rep_dim;
  int32_t rep_heads;
  int32_t rep_mode;        /* brs_rep_mode                                 */
  int32_t rep_dtype;       /* brs_dtype of reps                            */
  int32_t reserved;        /* must be 0                                    */
  int64_t capacity;        /* token rows per (batch, kv head)              */
  int64_t length;          /* tokens stored, equal for every batch row     */
  void* k;
  void* v;
  void* reps;
} brs_memory;

int brs_version(void);

/* Message for the last error on this thread ("" after success). */
const char* brs_last_error(void);

/* Host-only check of a descriptor (no device access). */
int brs_memory_check(const brs_memory* m);

/* Append n_new tokens (MemLong 2.3.2, "memorisation": K-V pairs are stored
 * together with the index-aligned representation of their chunk).
 *   k_new, v_new : [batch][n_kv_heads][n_new][head_dim] dtype, contiguous.
 *   reps_new     : for GIVEN/EMBED, the representatives of the blocks this
 *                  append completes, [batch][rep_heads][n_done][R][rep_dim]
 *                  rep_dtype, n_done = (length+n_new)/B - length/B; may be
 *                  NULL when n_done = 0; ignored for MEAN/TOPNORM, whose
 *                  representatives are computed from the stored keys, and
 *                  for ATTNSCORE, whose are built by brs_reps_from_mass.
 * On success enqueues the copies and representative builds and sets
 * m->length += n_new (host side).  BRS_E_CAPACITY if length + n_new >
 * capacity.  n_new = 0 is a no-op. */
int brs_mem_append(brs_memory* m, const void* k_new, const void* v_new, int64_t n_new,
                   const void* reps_new, void* stream);

/* Candidate blocks for a step with n_sink sinks and a window of the last
 * `window` tokens (InfLLM "method": the memory units hold what lies outside
 * the local window).  Host only.  Writes *lo, *hi such that block b is a
 * candidate iff lo <= b < hi: b is complete (b < length/B) and holds a token
 * outside [0, n_sink) and [length - window, length).  hi = lo means none. */
int brs_eligible_range(const brs_memory* m, int64_t n_sink, int64_t window, int64_t* lo,
                       int64_t* hi);

/* Score blocks [lo, hi) (Landmark Attention "proposed method": similarity of
 * the query with each block's landmark key; InfLLM "method": block-level
 * relevance; MemLong 2.3.2: cosine of the chunk embeddings).
 *   MEAN/TOPNORM/GIVEN (dot-max): qrep = q [batch][n_score_heads][head_dim]
 *     dtype, n_score_heads = the query heads Hq (a multiple of n_kv_heads;
 *     query head h reads kv head h / (Hq / n_kv_heads));
 *     score = max over the block's R representatives of q . rep.
 *   EMBED (cosine): qrep = [batch][rep_dim] rep_dtype, n_score_heads = 1;
 *     score = q.e / (|q| |e|), 0 if either norm is 0.
 * Products are exact and summed in float64, then rounded once to float32, so
 * the result does not depend on summation order.  No softmax scale.
 *   scores : [batch][n_score_heads][capacity / block_size] float32; only
 *            columns [lo, hi) are written.
 * Requires 0 <= lo <= hi <= length / block_size. */
int brs_score_blocks(const brs_memory* m, const void* qrep, int32_t n_score_heads, int64_t lo,
                     int64_t hi, float* scores, void* stream);

/* Scores for a selection shared by the query heads of each kv head (dot
 * scoring only; grouped-query attention): the score of block b for kv head g
 * is the maximum over the group's query heads h and the block's R
 * representatives of q_h . rep -- the block's best match with any head of
 * the group, combined by max as a block's representatives are (InfLLM
 * "method": block-level relevance; Landmark Attention "proposed method").
 * Exact products summed in float64, rounded once to float32; NaN in any dot
 * makes the score NaN.
 *   q      : [batch][n_q_heads][head_dim] dtype, as brs_score_blocks.
 *   scores : [batch][n_kv_heads][capacity / block_size] float32; columns
 *            [lo, hi) are written.
 * brs_select_topk with n_heads = n_kv_heads then gives one selection per kv
 * head (idx_heads = n_kv_heads in brs_retrieval_attention).  Errors as
 * brs_score_blocks; BRS_E_INVAL for EMBED memories. */
int brs_score_blocks_group(const brs_memory* m, const void* q, int32_t n_q_heads, int64_t lo, int64_t hi,
                           float* scores, void* stream);

/* Exact top-k per row of scores (MemLong 2.3.2: TopK of the scores, computed
 * exactly, 2.4.2).
 *   scores : [batch][n_heads][blocks_stride] float32, columns [lo, hi) read.
 *   idx    : [batch][n_heads][k] int32 -- the first min(k, hi-lo) blocks
 *            ordered by (score descending, block index ascending); NaN ranks
 *            below every number; -0 and +0 are equal; unused slots are -1.
 *   vals   : [batch][n_heads][k] float32 scores of idx (-inf in unused
 *            slots), or NULL.
 * Limits: 1 <= k <= 2048; hi - lo <= 1048576. */
int brs_select_topk(const float* scores, int32_t batch, int32_t n_heads, int64_t blocks_stride,
                    int64_t lo, int64_t hi, int32_t k, int32_t* idx, float* vals, void* stream);

/* Writes to *bytes (host) the workspace size brs_retrieval_attention needs
 * for these arguments -- a bound that does not depend on the contents of
 * idx.  Validates exactly as brs_retrieval_attention does and returns the
 * same error code for the same arguments. */
int brs_attention_workspace_bytes(const brs_memory* m, int32_t n_q_heads, int32_t n_q,
                                  int32_t idx_heads, int32_t k, int64_t n_sink, int64_t window,
                                  size_t* bytes);

/* Exact softmax attention over the attended set (InfLLM "method": local
 * tokens plus a few relevant memory units; MemLong Figure 3 and 2.3.4: the
 * retrieved chunks are visible in full, the local context causally;
 * RetrievalAttention "proposed method": attention restricted to the tokens
 * that matter).
 *   q    : [batch][n_q_heads][n_q][head_dim] dtype; query j sits at position
 *          N - n_q + j (N = m->length: the queries' own tokens are already
 *          appended).
 *   idx  : [batch][idx_heads][k] int32 block indices; idx_heads = n_q_heads
 *          (one list per query head), n_kv_heads (one list per kv head,
 *          shared by its query heads) or 1 (one list for all heads of a
 *          sequence).  Entries < 0 or >= N / block_size are skipped;
 *          duplicates count once.
 *   For query j of head h the attended set is the SET
 *      [0, n_sink) u [N - window, N) u  U_{b in idx} [bB, bB + B)
 *   restricted to positions <= N - n_q + j; head h reads kv head
 *   h / (n_q_heads / n_kv_heads).  Logits are scale * q.k; softmax and the
 *   weighted sum of V are accumulated in float32.
 *   out  : [batch][n_q_heads][n_q][head_dim] float32.  A query whose set is
 *          empty at run time (possible only when n_sink = window = 0 and
 *          every idx entry is skipped) gets zeros; when that is certain
 *          from the arguments alone the call returns BRS_E_EMPTY.
 *   lse  : [batch][n_q_heads][n_q] float32 or NULL: the natural log of each
 *          query's softmax denominator, log sum_t exp(scale * q.k_t) over
 *          its attended set (-inf for an empty set).
 *   workspace : device scratch of at least brs_attention_workspace_bytes()
 *          bytes, 256-byte aligned; its contents on entry do not matter.
 * n_q = 1 (decode) runs a split-K flash-decode; n_q > 1 with bf16 runs the
 * matrix-core prefill kernel. */
int brs_retrieval_attention(const brs_memory* m, const void* q, int32_t n_q_heads, int32_t n_q,
                            const int32_t* idx, int32_t idx_heads, int32_t k, int64_t n_sink,
                            int64_t window, float scale, float* out, float* lse, void* workspace,
                            size_t workspace_bytes, void* stream);

/* One whole step (score_blocks, select_topk, retrieval_attention) in one
 * call, with the candidate range of brs_eligible_range(n_sink, window):
 * identical results to the calls made in turn.
 *   select_heads : the selection lists per sequence.  Dot scores: n_q_heads
 *               (brs_score_blocks, one selection per query head) or
 *               n_kv_heads (brs_score_blocks_group, one selection per kv
 *               head shared by its query heads).  Cosine scores: 1 (one per
 *               sequence).
 *   q, out, lse : as brs_retrieval_attention (idx_heads = select_heads);
 *   qrep      : as brs_score_blocks (unused when k = 0);
 *   scores    : [batch][select_heads][capacity / block_size] float32;
 *   idx, vals : [batch][select_heads][k] as brs_select_topk (vals may be
 *               NULL; scores and idx may be NULL when k = 0);
 *   workspace : brs_attention_workspace_bytes(m, n_q_heads, n_q,
 *               select_heads, k, n_sink, window) bytes.
 * Errors as the separate calls; nothing is enqueued on error. */
int brs_retrieval_step(const brs_memory* m, const void* q, int32_t n_q_heads, int32_t n_q,
                       const void* qrep, int32_t select_heads, int32_t k, int64_t n_sink, int64_t window,
                       float scale, float* scores, int32_t* idx, float* vals, float* out, float* lse,
                       void* workspace, size_t workspace_bytes, void* stream);

/* brs_retrieval_step for callers that cannot allocate device memory -- code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc: the same step with the same results, its workspace taken from a
 * library-held device array of brs_static_scratch_bytes() bytes (16 MiB) per
 * GPU instead of a caller buffer.  Arguments, outputs and errors as
 * brs_retrieval_step without workspace / workspace_bytes; additionally
 * BRS_E_UNSUPPORTED when the step needs more workspace than the array holds
 * (brs_attention_workspace_bytes tells), and BRS_E_HIP if the array's address
 * cannot be obtained.  The array belongs to the device current at the call
 * (its address is looked up once per device); the stream must be on that
 * device.  It allocates nothing (no hipMalloc, hipFree or allocating library
 * call).  Every call on one GPU shares that GPU's array: calls that overlap
 * on one GPU (on different streams, or from several threads without ordering)
 * race on it.  Nothing in it needs to start at zero. */
int brs_retrieval_step_static(const brs_memory* m, const void* q, int32_t n_q_heads, int32_t n_q,
                              const void* qrep, int32_t select_heads, int32_t k, int64_t n_sink, int64_t window,
                              float scale, float* scores, int32_t* idx, float* vals, float* out, float* lse,
                              void* stream);

/* Bytes of the per-GPU array brs_retrieval_step_static works in. */
size_t brs_static_scratch_bytes(void);

/* Attention mass of the local window (InfLLM "method": the attention scores
 * each token receives decide which tokens represent its memory unit).  After
 * an attention call with queries q (same n_q_heads, n_q, scale) that wrote
 * lse, adds to every token t of the window [length - window, length)
 *     mass[b][g][t] += sum over the query heads h of kv head g and the
 *                      queries j that see t of exp(scale * q.k_t - lse)
 * -- the softmax weight t received, summed over the group's heads and the
 * call's queries.  Query j sits at position length - n_q + j and sees
 * positions <= its own (the window is always attended in full).
 *   q    : [batch][n_q_heads][n_q][head_dim] dtype, 16-byte aligned.
 *   lse  : [batch][n_q_heads][n_q] float32 from that attention call.
 *   mass : [batch][n_kv_heads][capacity] float32, caller-owned, zeroed by
 *          the caller once before the first token; read and written only
 *          at window tokens.
 * Weights are float32 (products of stored values summed in float32); a call
 * adds each token's sum once, in a fixed order (deterministic).  Any rep_mode;
 * window >= 1; n_q <= length. */
int brs_window_mass(const brs_memory* m, const void* q, int32_t n_q_heads, int32_t n_q, const float* lse,
                    int64_t window, float scale, float* mass, void* stream);

/* Representatives of blocks [b0, b1) from the accumulated mass (ATTNSCORE
 * memories): the R keys of each block with the largest mass, ties to the
 * lower token, copied unchanged, largest first, into reps (as TOPNORM does
 * with norms).  mass as in brs_window_mass; requires 0 <= b0 <= b1 <=
 * length / block_size.  The reading used by this library: a block's
 * representatives are built when it becomes a candidate (its first token
 * leaves the window), from the mass accumulated up to then. */
int brs_reps_from_mass(const brs_memory* m, const float* mass, int64_t b0, int64_t b1, void* stream);

/* Retrieval counters (MemLong 2.3.2, dynamic memory update: memory entries
 * are ranked by how often they are retrieved).  For every entry of
 * idx [batch][idx_heads][k] (a selection as brs_select_topk writes it)
 * naming a complete block, adds 1 to hits[b][block]:
 *   hits : [batch][capacity / block_size] int32, caller-owned, zeroed by the
 *          caller once; a count per block per sequence, summed over the
 *          selection lists (one per query head for dot scores).
 * Entries < 0 or >= length / block_size are skipped.  Integer atomics, so the
 * result does not depend on their order. */
int brs_count_hits(const brs_memory* m, const int32_t* idx, int32_t idx_heads, int32_t k, int32_t* hits,
                   void* stream);

/* Pruning on overflow (MemLong 2.3.2, dynamic memory update): copies what
 * survives of src into dst, which must have src's geometry (every field but
 * the pointers and length) and buffers of its own.  With nb = length / B
 * complete blocks and a partial tail of length - nb*B tokens:
 *   - the oldest floor(nb / 10) blocks are dropped and the newest floor(nb /
 *     10) kept;
 *   - blocks of the middle are evicted in order of (hits summed over the
 *     batch rows ascending, block index ascending) -- ties evict the older
 *     block -- until the kept blocks plus the tail fit in capacity / 2
 *     tokens, or none of the middle is left;
 *   - kept blocks keep their order; the tail follows them.
 * One decision is made for the whole memory (every batch row and head keeps
 * the same blocks, since all rows share one length).
 *   hits     : [batch][capacity / B] int32 counts of src (brs_count_hits).
 *   dst_hits : [batch][capacity / B] int32 or NULL: the kept blocks' counts
 *              at their new indices.
 *   plan     : [capacity / B] int32 scratch; on completion plan[b] is block
 *              b's new index, -1 if evicted (b < nb).
 * K, V, representatives and counts of the kept blocks are copied bit for bit;
 * dst's rows past its new length are left as they were.  Sets dst->length
 * (host side) on success.  BRS_E_UNSUPPORTED above 16384 middle blocks. */
int brs_mem_prune(const brs_memory* src, const int32_t* hits, brs_memory* dst, int32_t* dst_hits, int32_t* plan,
                  void* stream);

/* ---------------------------------------------------------------------------
 * Offload to host memory with a device cache of blocks (InfLLM "method": all
 * memory units are kept in CPU memory and the GPU keeps a cache of the units
 * used most, loading the units a step needs that it does not hold;
 * RetrievalAttention "proposed method": the KV cache is split between GPU and
 * CPU memory).
 *
 * The memory's k and v are then HOST memory: pinned and mapped (hipHostMalloc,
 * e.g. a torch tensor made with pin_memory=True), read and written by the
 * device through the same address.  brs_mem_append fills it as usual; the
 * representatives stay in device memory, so scoring and selection are
 * unchanged.  A caller-owned page pool in device memory caches blocks: */
typedef struct brs_page_cache {
  void* k;                 /* device [batch][n_kv_heads][n_pages * block_size][row_stride] dtype */
  void* v;                 /* device, as k                                                        */
  int32_t* page_of_block;  /* device [batch][n_kv_heads][capacity / block_size + 1]: page or -1   */
  int32_t* page_block;     /* device [batch][n_kv_heads][n_pages]: block held, -1 if free         */
  int32_t* page_rows;      /* device [batch][n_kv_heads][n_pages]: rows of that block copied      */
  int32_t* page_used;      /* device [batch][n_kv_heads][n_pages]: last step that needed the page */
  int32_t n_pages;         /* pages per (batch, kv head), 1 .. 2048                               */
  int32_t reserved;        /* must be 0                                                           */
} brs_page_cache;

/* Empties the cache (every table to "nothing cached").  Enqueued on stream.
 * Requires a valid memory descriptor for the geometry; row_stride * element
 * size a multiple of 16 bytes; capacity / block_size < 262144. */
int brs_cache_reset(const brs_memory* m, const brs_page_cache* c, void* stream);

/* Makes resident every block that brs_retrieval_attention_cached with the
 * same idx, idx_heads, k, n_sink and window will read, for every (batch, kv
 * head): the blocks holding sink or window tokens and the selected blocks
 * holding tokens outside both.  A needed block already cached keeps its page
 * (the rows a growing tail block gained since are copied); the others are
 * copied from host memory into pages that are free, else that were needed
 * least recently (lowest page_used, then lowest page index), among those this
 * step does not need.  page_used of every needed page becomes `step` (any
 * increasing counter).  fetched (device [batch][n_kv_heads] int32, or NULL)
 * gets += the blocks copied.  idx as brs_retrieval_attention (idx_heads = 1,
 * n_kv_heads or the query heads).  BRS_E_CAPACITY when n_pages is below the
 * blocks a step may need: ceil(S'/B) + the window's blocks + (lists of a kv
 * head) * k, with S' the sinks kept.  Enqueued on stream. */
int brs_cache_fetch(const brs_memory* m, const brs_page_cache* c, const int32_t* idx, int32_t idx_heads, int32_t k,
                    int64_t n_sink, int64_t window, int32_t step, int32_t* fetched, void* stream);

/* brs_retrieval_attention for an offloaded memory: K/V are read from the
 * cache's pages through page_of_block (after brs_cache_fetch with the same
 * selection), with results identical bit for bit to brs_retrieval_attention
 * over the same data resident in device memory.  Served by the kernels that
 * read K/V row by row: the slot-layout decode kernels (bfloat16, head_dim 64
 * or 128, any n_q whose rows they take) and the chunked-prefill kernel
 * (bfloat16, n_q >= 64, head_dim <= 128, k + 2 <= 256; InfLLM "method":
 * memory units stay offloaded during chunked prefill as well); other shapes
 * return BRS_E_UNSUPPORTED.  Workspace as brs_attention_workspace_bytes. */
int brs_retrieval_attention_cached(const brs_memory* m, const brs_page_cache* c, const void* q, int32_t n_q_heads,
                                   int32_t n_q, const int32_t* idx, int32_t idx_heads, int32_t k, int64_t n_sink,
                                   int64_t window, float scale, float* out, float* lse, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* Measurement hook: the next brs_retrieval_attention, brs_retrieval_step or
 * brs_window_mass call on this thread records `start_event` and `stop_event`
 * (hipEvent_t, passed as void*) at the begin and end of its main kernel (the
 * attention kernel; the mass kernel) on its stream, then forgets them.  In
 * the one-launch decode step the start is recorded when the score kernel
 * before it completes.  Pass NULLs to cancel. */
int brs_profile_next_attention(void* start_event, void* stop_event);

#ifdef __cplusplus
}
#endif

#endif /* BRS_H_ */

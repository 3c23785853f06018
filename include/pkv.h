/*
 * pkv.h - paged KV-cache attention for AMD Instinct MI355X (gfx950).
 *
 * A continuous-batching server keeps every request's attention keys and values
 * in fixed 16-token blocks of one shared FP16 pool; a per-request block table
 * maps logical block numbers to physical ones, a free list hands blocks out as
 * sequences grow, and reference counts let requests share prefix blocks
 * (LLM inference batching, faangrind.vercel.app: data model "KV pool",
 * "block_table", "ref_count", "free_list"; Build a continuous batching server,
 * scalablesystem.dev: "The KV Cache Block Manager (PagedAttention)" and
 * "PagedAttention Block Table Lookup").  Each decode step appends one token's
 * keys and values per row and attends over the row's blocks in place; a
 * prefill chunk attends causally over its paged prefix in the same step
 * (faangrind: "Prefill and decode share each step").
 *
 * This header is the whole boundary.  It uses plain C types only.
 *
 * Conventions for every call
 *  - Return value: PKV_OK (0) or a negative PKV_ERR_* code.  On error nothing
 *    has been launched or changed, and pkv_last_error() (thread-local) holds a
 *    message.  Scalar arguments are validated on the host before any launch.
 *    The one exception is PKV_ERR_HIP from a call that queues several
 *    launches or copies: what was queued before the refused one stays queued.
 *  - Device pointers are owned by the caller and must stay valid until the
 *    work queued on `stream` has finished.  The library never allocates or
 *    frees device memory and never synchronizes the stream.
 *  - `stream` is a hipStream_t passed as void*; NULL means the default stream.
 *  - Contents of device arrays (block ids, lengths, positions) are the
 *    caller's contract: they are not copied to the host.  Kernels bounds-check
 *    every block id against num_blocks and every table index against
 *    bt_stride, so a bad entry yields unspecified values for that row (or an
 *    append that is skipped) but never an out-of-bounds memory access.
 *  - The block pool object is single-owner and not thread-safe: a single
 *    scheduler thread drives the GPU and holds it (LLM inference batching,
 *    faangrind, scheduler step 3).
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = -1,   /* null pointer, negative count, index out of range */
  PKV_ERR_UNSUPPORTED = -2,   /* shape the kernels are not built for */
  PKV_ERR_OUT_OF_BLOCKS = -3, /* allocation larger than the free list; nothing allocated */
  PKV_ERR_DOUBLE_FREE = -4,   /* release or share of a block whose count is already 0 */
  PKV_ERR_BAD_BLOCK = -5,     /* block id outside [0, num_blocks) */
  PKV_ERR_WORKSPACE = -6,     /* workspace missing or smaller than the size query says */
  PKV_ERR_HIP = -7            /* the HIP runtime refused a launch; message kept */
};

/* Message for the last error on this thread ("" when the last call succeeded). */
const char* pkv_last_error(void);
/* Library version string. */
const char* pkv_version(void);

/* ------------------------------------------------------------------------
 * Host block pool: free list + reference counts.
 *
 * The free list is a stack: allocation pops ids from its top and release
 * pushes them back in the order given (scalablesystem.dev BlockManager;
 * Serving LLMs, sreshtalluri.github.io: "Paged KV memory" BlockPool).
 * A block's count is 1 after allocation, +1 per share, -1 per release; it
 * returns to the free list only at 0 (faangrind data model: ref_count exceeds
 * 1 while several samples share one prompt; failure list: a block freed
 * while still referenced leaks one user's text into another's answer).
 * Every call validates all of its ids before changing anything.
 * ---------------------------------------------------------------------- */
typedef struct pkv_pool pkv_pool;

/* Pool of num_blocks ids with free list 0..num_blocks-1; the first
 * allocation takes num_blocks-1.  *out receives a new pool owned by the
 * caller (release with pkv_pool_destroy). */
int pkv_pool_create(int32_t num_blocks, pkv_pool** out);

/* Pool of num_blocks ids whose free list is free_ids[0..n_free) with
 * free_ids[n_free-1] on top (allocated first), e.g. a shuffled list.  Ids must
 * be distinct and in range; ids not listed start allocated with count 1. */
int pkv_pool_create_from_list(int32_t num_blocks, const int32_t* free_ids, int32_t n_free, pkv_pool** out);

void pkv_pool_destroy(pkv_pool* pool);

/* Pop n ids into out_ids[0..n) (out_ids[0] = old top), each with count 1.
 * All or nothing: with fewer than n free, returns PKV_ERR_OUT_OF_BLOCKS and
 * changes nothing (Serving LLMs, "Paged KV memory": BlockPool.grow reports the
 * shortfall so that the scheduler preempts a sequence). */
int pkv_alloc(pkv_pool* pool, int32_t n, int32_t* out_ids);

/* Count +1 for each listed id (a new sharer of a prefix block).  Every id must
 * be allocated; otherwise PKV_ERR_DOUBLE_FREE / PKV_ERR_BAD_BLOCK and no
 * change. */
int pkv_ref(pkv_pool* pool, const int32_t* ids, int32_t n);

/* Count -1 for each listed id; an id reaching 0 is pushed on the free list, in
 * list order.  An id listed more times than its count is PKV_ERR_DOUBLE_FREE
 * and nothing changes. */
int pkv_free(pkv_pool* pool, const int32_t* ids, int32_t n);

/* Grow a block table so it covers num_tokens tokens: appends
 * ceil(num_tokens/16) - *table_len newly allocated ids to table[*table_len..]
 * and updates *table_len.  All or nothing (PKV_ERR_OUT_OF_BLOCKS); a table
 * that already covers num_tokens is left as is.  capacity bounds table. */
int pkv_grow(pkv_pool* pool, int32_t* table, int32_t* table_len, int32_t capacity, int32_t num_tokens);

/* One step's growth for a batch of rows, in one call: row r's table
 * tables[r * stride .. (r + 1) * stride) is grown as pkv_grow would grow it
 * to cover num_tokens[r] tokens, rows in order (a row takes a new block every
 * 16 tokens; faangrind scheduler step 7).  All arguments of every row are
 * checked first (PKV_ERR_INVALID_ARG, nothing changed).  Each row grows all
 * or nothing; at the first row the free list cannot cover, the call returns
 * PKV_ERR_OUT_OF_BLOCKS, that row and those after it unchanged, and the rows
 * before it grown -- the scheduler then preempts a sequence (Serving LLMs,
 * "Paged KV memory").  *rows_grown receives the number of rows processed. */
int pkv_grow_rows(pkv_pool* pool, int32_t* tables, int32_t stride, int32_t* table_lens, const int32_t* num_tokens,
                  int32_t num_rows, int32_t* rows_grown);

int32_t pkv_num_free(const pkv_pool* pool);
int32_t pkv_num_blocks(const pkv_pool* pool);
/* Count of block id, or -1 if id is out of range. */
int32_t pkv_ref_count(const pkv_pool* pool, int32_t id);
/* Copies up to cap ids of the free list, bottom first, into out; returns the
 * free-list length. */
int32_t pkv_free_list(const pkv_pool* pool, int32_t* out, int32_t cap);
/* ceil(num_tokens / 16) (scalablesystem.dev BlockManager.blocks_needed). */
int32_t pkv_blocks_needed(int32_t num_tokens);

/* ------------------------------------------------------------------------
 * Device KV pool descriptor.
 *
 * base points to caller-owned FP16 device memory laid out as
 *   [num_blocks][num_layers][2][num_heads][block_size][head_dim]
 * (faangrind data model: one block holds [32 layers, 2, 32 heads, 16 tokens,
 * 128] FP16; index 0 of the "2" axis is keys, 1 is values).
 * Supported: block_size == 16, head_dim == 128, 1 <= num_heads <= 128,
 * num_layers >= 1, num_blocks >= 1.  Offsets are 64-bit: a 7,152-block,
 * 32-layer pool is 60 GB.
 * ---------------------------------------------------------------------- */
typedef struct pkv_cache {
  void* base;
  int32_t num_blocks;
  int32_t num_layers;
  int32_t num_heads;
  int32_t block_size;
  int32_t head_dim;
} pkv_cache;

/* ------------------------------------------------------------------------
 * KV append.
 *
 * For each new token t < num_tokens of one step (the step's flat token list
 * tagged by request, faangrind data model: the step tensors positions and
 * request_of_token): row r = request_of_token[t], position p = positions[t],
 * block b = block_tables[r * bt_stride + p / 16], slot s = p % 16; copies the
 * bits of k_new[t] into pool[b][layer][0][:][s][:] and of v_new[t] into
 * pool[b][layer][1][:][s][:].  A row takes a new block every 16 tokens
 * (faangrind scheduler step 7), so the caller grows the table first.
 *   k_new, v_new  device FP16 [num_tokens][num_heads][128]
 *   positions, request_of_token  device int32 [num_tokens]
 *   block_tables  device int32 [num_rows][bt_stride]
 * Targets must be distinct and must not be shared blocks (count 1): shared
 * prefix blocks are immutable and a writer copies first (The inference
 * engine, wpnews.pro: copy-on-write when a branch diverges).  A token whose
 * row, position or block id is out of range is skipped.  num_tokens == 0 is a
 * no-op.  Bit-exact.
 * ---------------------------------------------------------------------- */
int pkv_append(const pkv_cache* cache, int32_t layer, const void* k_new, const void* v_new,
               const int32_t* positions, const int32_t* request_of_token, int32_t num_tokens,
               const int32_t* block_tables, int32_t num_rows, int32_t bt_stride, void* stream);

/* ------------------------------------------------------------------------
 * Decode attention.
 *
 * Row r has one query q[r] (device FP16 [num_rows][num_heads][128]) at
 * position context_lens[r]-1, and attends over its context_lens[r] cached
 * tokens including the token appended this step (Inference Infrastructure,
 * seeitflow.com: "Three iterations with the state written out").  For every
 * head: out = softmax_j((q . k_j) * scale) v_j over j < context_lens[r], read
 * through the block table in place (scalablesystem.dev "PagedAttention Block
 * Table Lookup": no contiguous copy).  Softmax statistics are kept per tile
 * so that tiles combine exactly (The inference engine, wpnews.pro: "IO-aware
 * attention and quantization attack different costs").  FP16 inputs, fp32
 * arithmetic, FP16 output rounded to nearest even:
 *   out  device FP16 [num_rows][num_heads][128]
 * Long contexts are split into fixed ranges of pkv_split_tokens() tokens whose
 * partial results a second pass merges; the split depends only on the row's
 * own length, so a row's output does not depend on its batch neighbours.
 *   context_lens       device int32 [num_rows], each in [1, max_context_len]
 *   max_context_len    host bound on context_lens, <= bt_stride * 16
 *   workspace          device memory of at least
 *                      pkv_decode_workspace_size(cache, num_rows, max_context_len)
 *                      bytes, 256-byte aligned; contents need no
 *                      initialisation and are scratch after the call.
 * A context_len outside [1, max_context_len] is clamped for memory safety and
 * gives unspecified output for that row.
 * ---------------------------------------------------------------------- */
size_t pkv_decode_workspace_size(const pkv_cache* cache, int32_t num_rows, int32_t max_context_len);
int pkv_decode_attention(const pkv_cache* cache, int32_t layer, void* out, const void* q,
                         const int32_t* block_tables, int32_t bt_stride, const int32_t* context_lens,
                         int32_t num_rows, int32_t max_context_len, float scale, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Tokens per split-K range of the decode kernel. */
int32_t pkv_split_tokens(void);

/* Decode with the step's append fused in.  Row r's new token sits at position
 * context_lens[r] - 1, and its keys and values are k_new[r] and v_new[r]
 * (device FP16 [num_rows][num_heads][128], 16-byte aligned).  The call writes
 * them into their slot, exactly as pkv_append with positions[r] =
 * context_lens[r] - 1 and request_of_token[r] = r.  It then returns
 * pkv_decode_attention's result: the same bits, in the pool and in out, as
 * those two calls in sequence.  The range that holds a row's last token takes
 * that token from k_new / v_new, so the step needs one launch fewer
 * (faangrind scheduler step 7: each decode row appends its token, then
 * attends).  Same contract and workspace as pkv_decode_attention; the
 * appended slot must not be in a shared block.  Rows with context_lens[r] < 1
 * or context_lens[r] > max_context_len break the length contract: they append
 * nothing (no pool byte changes for them) and their output is unspecified. */
int pkv_decode_attention_append(const pkv_cache* cache, int32_t layer, void* out, const void* q, const void* k_new,
                                const void* v_new, const int32_t* block_tables, int32_t bt_stride,
                                const int32_t* context_lens, int32_t num_rows, int32_t max_context_len, float scale,
                                void* workspace, size_t workspace_bytes, void* stream);

/* pkv_decode_attention_append for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, contract and result (the same pool bytes and
 * output bits) as pkv_decode_attention_append, without the workspace: the
 * split-K partials go to a scratch array the library holds on each GPU it runs
 * on, PKV_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, until the process ends.  The
 * call allocates nothing.  A call needing more scratch than that
 * (pkv_decode_workspace_size(cache, num_rows, max_context_len) bytes) returns
 * PKV_ERR_WORKSPACE before anything is launched.  All calls on one GPU share
 * its scratch array: calls whose work overlaps in time on one GPU (on
 * different streams, or from several threads) race and give unspecified
 * output; calls queued on one stream do not. */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int pkv_decode_attention_append_noalloc(const pkv_cache* cache, int32_t layer, void* out, const void* q,
                                        const void* k_new, const void* v_new, const int32_t* block_tables,
                                        int32_t bt_stride, const int32_t* context_lens, int32_t num_rows,
                                        int32_t max_context_len, float scale, void* stream);

/* ------------------------------------------------------------------------
 * Chunked-prefill attention mixed with decode rows in one call.
 *
 * Row r owns queries q[query_start[r] .. query_start[r+1]) (device FP16
 * [total_q][num_heads][128]); they are the last n_r = query_start[r+1] -
 * query_start[r] positions of its context, L_r - n_r .. L_r - 1 with
 * L_r = context_lens[r], and their keys and values were appended before the
 * call.  Query i of the row sits at p = L_r - n_r + i and attends causally to
 * keys 0..p (The inference engine, wpnews.pro, "Prefill and decode ask the
 * accelerator for different work": prefill attention is causal).  Rows with
 * n_r == 1 are decode rows; a prefill chunk and decode rows
 * share the step as a flat list of request-tagged tokens (faangrind "Prefill
 * and decode share each step").  The chunk's QK^T and PV products run on
 * MFMA matrix cores in FP16 with fp32 accumulation.
 *   out            device FP16 [total_q][num_heads][128]
 *   query_start    device int32 [num_rows + 1], query_start[0] = 0,
 *                  query_start[num_rows] = total_q
 *   context_lens   device int32 [num_rows], n_r <= L_r <= max_context_len
 *   max_q_per_row  host bound on n_r
 *   workspace      >= pkv_prefill_workspace_size(...) bytes, 256-byte aligned
 * Rows violating the bounds give unspecified output but no out-of-bounds
 * access.
 * ---------------------------------------------------------------------- */
size_t pkv_prefill_workspace_size(const pkv_cache* cache, int32_t num_rows, int32_t total_q,
                                  int32_t max_q_per_row, int32_t max_context_len);
int pkv_chunked_prefill_attention(const pkv_cache* cache, int32_t layer, void* out, const void* q,
                                  const int32_t* query_start, const int32_t* block_tables, int32_t bt_stride,
                                  const int32_t* context_lens, int32_t num_rows, int32_t total_q,
                                  int32_t max_q_per_row, int32_t max_context_len, float scale,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Grouped-query attention.
 *
 * The number of KV heads, not of query heads, sets the cache size; grouped-
 * query attention shares one K/V head among a group of query heads
 * (Inference Infrastructure, seeitflow.com: the KV-bytes formula and its
 * MHA / MQA / GQA note; The inference engine, wpnews.pro: grouped-query
 * attention lowers the KV-head count below the query-head count).  The pool
 * descriptor's num_heads is the number of KV heads; num_q_heads =
 * G * num_heads query heads attend, and query head h reads KV head h / G
 * (consecutive query heads form a group).  q and out are
 * [rows or tokens][num_q_heads][128]; everything else is as in
 * pkv_decode_attention / pkv_chunked_prefill_attention, which are these calls
 * with num_q_heads = num_heads.
 *   decode: G in {1, 2, 4, 8}, else PKV_ERR_UNSUPPORTED.  Each key and value
 *           of a KV head is read once for all G query heads of its group.
 *   prefill: any G with num_q_heads <= 1024.  Each query head's tile reads
 *           its group's K/V tile (from cache when the group's tiles run
 *           together); decode rows of the launch likewise.
 * The workspace sizes count query heads.
 * ---------------------------------------------------------------------- */
size_t pkv_decode_workspace_size_gqa(const pkv_cache* cache, int32_t num_q_heads, int32_t num_rows,
                                     int32_t max_context_len);
int pkv_decode_attention_gqa(const pkv_cache* cache, int32_t num_q_heads, int32_t layer, void* out, const void* q,
                             const int32_t* block_tables, int32_t bt_stride, const int32_t* context_lens,
                             int32_t num_rows, int32_t max_context_len, float scale, void* workspace,
                             size_t workspace_bytes, void* stream);
/* pkv_decode_attention_append with G query heads per KV head: k_new / v_new
 * are [num_rows][num_heads][128] (the pool's KV heads), q and out
 * [num_rows][num_q_heads][128]. */
int pkv_decode_attention_append_gqa(const pkv_cache* cache, int32_t num_q_heads, int32_t layer, void* out,
                                    const void* q, const void* k_new, const void* v_new,
                                    const int32_t* block_tables, int32_t bt_stride, const int32_t* context_lens,
                                    int32_t num_rows, int32_t max_context_len, float scale, void* workspace,
                                    size_t workspace_bytes, void* stream);
size_t pkv_prefill_workspace_size_gqa(const pkv_cache* cache, int32_t num_q_heads, int32_t num_rows,
                                      int32_t total_q, int32_t max_q_per_row, int32_t max_context_len);
int pkv_chunked_prefill_attention_gqa(const pkv_cache* cache, int32_t num_q_heads, int32_t layer, void* out,
                                      const void* q, const int32_t* query_start, const int32_t* block_tables,
                                      int32_t bt_stride, const int32_t* context_lens, int32_t num_rows,
                                      int32_t total_q, int32_t max_q_per_row, int32_t max_context_len, float scale,
                                      void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Shared-prefix decode.
 *
 * Prefix blocks are computed once, held immutable and shared by reference
 * count among every sequence whose prompt begins with them; in a multi-tenant
 * step every concurrent sequence reads that one prefix (Build a continuous
 * batching server, scalablesystem.dev, "Scaling and Performance"; Serving
 * LLMs, "Prefix caching").  pkv_decode_attention_prefix computes exactly what
 * pkv_decode_attention computes (every row attends over its own context), but
 * reads the prefix once per step for all rows that share it: for each head
 * and 256-token range of the prefix, the sharing rows' queries (32 at a time)
 * form one matrix-core tile, and their partial softmax statistics merge with
 * those of each row's own blocks.
 *   shares_prefix  device int32 [num_rows]; nonzero marks a row whose first
 *                  prefix_blocks table entries are the prefix's block ids
 *                  (the same ids for every marked row: the prefix's ids are
 *                  read from the first marked row's table).  A marked row
 *                  with L <= 16 * prefix_blocks is decoded like an unmarked
 *                  one.  May be NULL when prefix_blocks = 0.
 *   prefix_blocks  host int, 0 <= P <= bt_stride; the prefix is P full
 *                  blocks (16 P tokens).  P = 0 gives pkv_decode_attention's
 *                  result bit for bit.
 * Everything else is as in pkv_decode_attention (MHA: one query head per KV
 * head).  Unmarked rows give the same bits as in pkv_decode_attention.  A
 * marked row's ranges are the prefix's (16 blocks each, the last one possibly
 * shorter) followed by 16-block ranges from block P on; they depend only on
 * the row's length, its mark and P, so its output does not depend on the
 * other rows of the batch.  Rows whose marks break the contract give
 * unspecified output but no out-of-bounds access.
 * The workspace needs pkv_decode_workspace_size_prefix(...) bytes, 256-byte
 * aligned (it may be NULL when every row fits one range and P = 0).
 * ---------------------------------------------------------------------- */
size_t pkv_decode_workspace_size_prefix(const pkv_cache* cache, int32_t num_rows, int32_t max_context_len,
                                        int32_t prefix_blocks);
int pkv_decode_attention_prefix(const pkv_cache* cache, int32_t layer, void* out, const void* q,
                                const int32_t* block_tables, int32_t bt_stride, const int32_t* context_lens,
                                int32_t num_rows, int32_t max_context_len, float scale,
                                const int32_t* shares_prefix, int32_t prefix_blocks, void* workspace,
                                size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Device-side check of a step's metadata.
 *
 * The kernels above trust the contents of the device arrays, as the pages'
 * gather trusts its block table (scalablesystem.dev, "PagedAttention Block
 * Table Lookup"): a bad entry cannot make them touch memory outside their
 * buffers, but it gives a wrong answer, and a row reading another request's
 * blocks is on the faangrind failure list.  pkv_check_tables counts, on the
 * device, the entries that break the contract and leaves a report there; it
 * never synchronises the stream (read the report after the stream reaches
 * it).  The library calls it nowhere itself: it is for debugging and for
 * callers that want the check on every step.
 *   block_tables, bt_stride, context_lens, num_rows, max_context_len
 *                  as in pkv_decode_attention (scalars validated the same way)
 *   query_start    device int32 [num_rows + 1] of a chunked-prefill step, or
 *                  NULL to skip the query checks
 *   total_q        the prefill step's query count (used with query_start)
 *   report         device int32 [4], overwritten completely by the call:
 *     [0] rows whose length is outside [1, max_context_len]
 *     [1] table entries outside [0, num_blocks) among those the kernels read
 *         (the first ceil(min(L, max_context_len) / 16) of each row)
 *     [2] rows whose query range breaks the prefill contract: query_start[r]
 *         < 0, query_start[r + 1] > total_q, n_r < 1 or n_r > L (0 without
 *         query_start)
 *     [3] the smallest row with any violation, or -1
 * One workgroup; no global atomics, nothing to clear beforehand, so it can be
 * captured and replayed.  num_rows >= 1. */
int pkv_check_tables(const pkv_cache* cache, const int32_t* block_tables, int32_t bt_stride,
                     const int32_t* context_lens, int32_t num_rows, int32_t max_context_len,
                     const int32_t* query_start, int32_t total_q, int32_t* report, void* stream);

/* ------------------------------------------------------------------------
 * Whole-block copies.
 *
 * A block with all its layers is one contiguous region of the pool of
 * pkv_block_bytes(cache) = num_layers * 2 * num_heads * 16 * 128 * 2 bytes
 * (8 MiB for 32 layers x 32 heads); these calls move whole blocks.
 *
 * Copy-on-write: requests sharing prefix blocks hold them immutable, and a
 * branch that diverges inside a shared block takes a private copy of it
 * first (The inference engine, wpnews.pro, "Weights, activations, and KV
 * state occupy different ledgers" and "Paging turns variable sequences into
 * block tables").  pkv_copy_blocks copies block src_ids[i] to dst_ids[i] for
 * i < n, every layer, K and V, bit for bit.
 *   src_ids, dst_ids  device int32 [n]
 * The dst ids must be distinct and none may also be a src id of the same call
 * (otherwise the result is unspecified).  A pair with an id outside
 * [0, num_blocks) is skipped.  n == 0 is a no-op.  cache->base 16-byte
 * aligned.
 *
 * Swap: under memory pressure a scheduler may move a sequence's blocks to
 * host memory and restore them later instead of recomputing its prefill
 * (Build a continuous batching server, scalablesystem.dev, "Preemption and
 * Eviction: Recompute vs Swap"; Inference Infrastructure, seeitflow.com, "An
 * overload example").  pkv_swap_out copies block ids[i] to
 * host_dst + i * pkv_block_bytes(cache); pkv_swap_in copies
 * host_src + i * pkv_block_bytes(cache) to block ids[i].
 *   ids                host int32 [n], each in [0, num_blocks), else
 *                      PKV_ERR_BAD_BLOCK and nothing is queued
 *   host_dst/host_src  host memory of n * pkv_block_bytes(cache) bytes; pinned
 *                      (hipHostMalloc) for the copy to be asynchronous
 * The copies are queued on `stream` (one DMA copy per run of consecutive
 * ids); the host buffer must stay valid until they finish.  pkv_swap_in's ids
 * must be distinct.  If the HIP runtime refuses a copy after earlier runs
 * were queued, those runs stay queued and PKV_ERR_HIP is returned.
 * ---------------------------------------------------------------------- */
size_t pkv_block_bytes(const pkv_cache* cache); /* 0 for an invalid descriptor */
int pkv_copy_blocks(const pkv_cache* cache, const int32_t* src_ids, const int32_t* dst_ids, int32_t n,
                    void* stream);
int pkv_swap_out(const pkv_cache* cache, const int32_t* ids, int32_t n, void* host_dst, void* stream);
int pkv_swap_in(const pkv_cache* cache, const void* host_src, const int32_t* ids, int32_t n, void* stream);

/* ------------------------------------------------------------------------
 * 8-bit KV cache.
 *
 * An 8-bit cache halves the bytes of every cached token and the attention
 * read traffic, with a quality risk that grows with context length
 * (Inference Infrastructure, seeitflow.com, its paragraph on KV-cache
 * precision; The
 * inference engine, wpnews.pro, "IO-aware attention and quantization attack
 * different costs").  Codes are FP8 E4M3 (OCP format: bias 7, three mantissa
 * bits, largest finite 448, 0x7F NaN) with one fp32 scale per (token, head)
 * row of 128 values:
 *   s = amax / 448, code = nearest E4M3 of x * (448 / amax) (ties to the even
 *   mantissa, saturated at 448); a zero row has s = 0 and zero codes;
 *   a cached value reads back as decode(code) * s.
 *
 * codes   device uint8 [num_blocks][num_layers][2][num_heads][16][128]
 * scales  device fp32  [num_blocks][num_layers][2][num_heads][16]
 * both 16-byte aligned and caller-owned; index 0 of the "2" axis is keys.
 *
 * pkv_append_fp8 takes FP16 k_new / v_new and places them exactly as
 * pkv_append does (same arguments and contract); codes and scales are bit-
 * exact with the definition above.  pkv_decode_attention_fp8 is
 * pkv_decode_attention over the dequantized cache (same arguments; split-K
 * ranges of 512 tokens, which also depend only on the row's own length, and
 * a workspace of pkv_decode_workspace_size_fp8 bytes; fp32 arithmetic, FP16
 * output).
 * ---------------------------------------------------------------------- */
typedef struct pkv_cache8 {
  void* codes;
  void* scales;
  int32_t num_blocks;
  int32_t num_layers;
  int32_t num_heads;
  int32_t block_size;
  int32_t head_dim;
} pkv_cache8;

int pkv_append_fp8(const pkv_cache8* cache, int32_t layer, const void* k_new, const void* v_new,
                   const int32_t* positions, const int32_t* request_of_token, int32_t num_tokens,
                   const int32_t* block_tables, int32_t num_rows, int32_t bt_stride, void* stream);
size_t pkv_decode_workspace_size_fp8(const pkv_cache8* cache, int32_t num_rows, int32_t max_context_len);
int pkv_decode_attention_fp8(const pkv_cache8* cache, int32_t layer, void* out, const void* q,
                             const int32_t* block_tables, int32_t bt_stride, const int32_t* context_lens,
                             int32_t num_rows, int32_t max_context_len, float scale, void* workspace,
                             size_t workspace_bytes, void* stream);
/* pkv_decode_attention_append for the 8-bit cache: row r's new token (FP16
 * k_new[r], v_new[r], [num_rows][num_heads][128], 16-byte aligned) is
 * quantized and written at position context_lens[r] - 1 exactly as
 * pkv_append_fp8 would, and the result is pkv_decode_attention_fp8's: the
 * same codes, scales and output bits as those two calls in sequence, in one
 * launch fewer.  As in pkv_decode_attention_append, a row whose length lies
 * outside [1, max_context_len] appends nothing. */
int pkv_decode_attention_append_fp8(const pkv_cache8* cache, int32_t layer, void* out, const void* q,
                                    const void* k_new, const void* v_new, const int32_t* block_tables,
                                    int32_t bt_stride, const int32_t* context_lens, int32_t num_rows,
                                    int32_t max_context_len, float scale, void* workspace, size_t workspace_bytes,
                                    void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */

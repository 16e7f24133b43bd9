/*
 * pa.h — C ABI of the paged KV-cache attention library (gfx950 / MI355X).
 *
 * The operation: attention of each query token over a key/value cache that is
 * stored in fixed-size physical blocks and reached through a per-sequence
 * block table, plus the write of new tokens' K/V into the slots a block
 * manager chose. Sources, by page title and section:
 *   [P1] "vLLM推理引擎深度解析：从PagedAttention原理到高吞吐量部署的工程实践"
 *        §三 (PagedAttentionManager: block pool, block tables, append_token,
 *        share_prefix) and §五 (PagedAttention.forward: per sequence, look up
 *        the block table, read K and V from the physical blocks, scores
 *        q·k / sqrt(head_dim), softmax, weighted sum of V).
 *   [P2] "vLLM 原理与源码阅读", PagedAttention 显存管理 → Block 管理器
 *        (one block table per request, 16 tokens per block by default,
 *        copy-on-write for shared prefix blocks).
 *   [P3] "vLLM推理引擎深度实战", §1.2 PagedAttention原理 (BLOCK_SIZE = 16,
 *        a block holds K and V of its tokens for all heads), §5.3
 *        推理优化配置 (the chunked-prefill switch) and the introduction (FP8
 *        among the supported quantisation schemes).
 *
 * Common conventions
 *   - Every pointer argument is a DEVICE pointer owned by the caller, except
 *     `stream`, which is a hipStream_t passed as void* (NULL = null stream).
 *     The library allocates nothing, frees nothing, keeps no pointer after it
 *     returns and has no mutable global state; calls are thread-safe. The
 *     exceptions are the handle objects: a block manager (pa_bm_*) and a
 *     step graph (pa_graph_*) own their memory until destroyed.
 *   - Every call only enqueues work on `stream` and returns; stream order is
 *     what makes a cache write visible to a later attention call.
 *   - `dtype` is a pa_dtype_t. Element types: F32 = float, F16 = IEEE half,
 *     BF16 = bfloat16. All arithmetic accumulates in fp32; outputs are rounded
 *     to `dtype` with round-to-nearest-even.
 *   - K/V pool layout: physical block i of the K pool starts at element
 *     `k_cache + i * block_stride` and holds `[block_size][num_kv_heads]
 *     [head_dim]` contiguous elements, token-major as the per-block K and V
 *     planes of [P1] §五. The V pool is laid out the same way at `v_cache`.
 *     P1's interleaved per-block (2, block_size, heads, head_dim) tensor is
 *     the case v_cache = k_cache + block_size*num_kv_heads*head_dim and
 *     block_stride = 2*block_size*num_kv_heads*head_dim.
 *   - Block tables: int32 `[num_seqs][block_table_stride]`; entry i of row b is
 *     the physical block that holds logical block i (tokens 16i .. 16i+15) of
 *     sequence b. Only the first ceil(L_b / block_size) entries are read.
 *   - Supported shapes: block_size == 16; head_dim in {64, 128};
 *     num_q_heads % num_kv_heads == 0 with group G = num_q_heads/num_kv_heads
 *     in {1, 2, 4, 8}. Pointers must be 16-byte aligned and strides must be
 *     multiples of 16 bytes.
 *
 * Errors: every entry point returns a pa_status_t and never aborts. The host
 * checks O(1) arguments only (NULL pointers, enums, supported shapes,
 * alignment, workspace size). The CONTENTS of device index arrays are
 * preconditions: non-negative slots unique and < num_blocks*block_size;
 * tables covering ceil(L/16) entries < num_blocks; 0 <= L. The kernels never
 * read or write outside the pools when these are violated (out-of-range slots
 * are skipped, out-of-range table entries are read as block 0 and masked),
 * but the affected results are then undefined. `num_seqs == 0` (or
 * `num_tokens == 0`) returns PA_OK without launching.
 */
#ifndef PAGED_KV_CACHE_463_AMD_PA_H
#define PAGED_KV_CACHE_463_AMD_PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Symbols of the C ABI are the only ones the shared library exports. */
#define PA_API __attribute__((visibility("default")))

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL_PTR = 1,     /* a required pointer is NULL                          */
  PA_ERR_DTYPE = 2,        /* dtype is not a pa_dtype_t, or not supported here    */
  PA_ERR_SHAPE = 3,        /* a size or stride is negative or inconsistent        */
  PA_ERR_UNSUPPORTED = 4,  /* block_size, head_dim or group size not supported    */
  PA_ERR_WORKSPACE = 5,    /* split-KV workspace missing or too small             */
  PA_ERR_HIP = 6,          /* the HIP runtime reported an error at launch         */
  PA_ERR_ALIGNMENT = 7,    /* a pointer or stride is not 16-byte aligned          */
  PA_ERR_NO_BLOCKS = 8,    /* block manager: not enough free blocks (no change)   */
  PA_ERR_SEQUENCE = 9,     /* block manager: unknown request id, or one in use    */
  PA_ERR_SCRATCH = 10      /* needs more than the static split-KV scratch holds   */
} pa_status_t;

typedef enum { PA_DTYPE_F32 = 0, PA_DTYPE_F16 = 1, PA_DTYPE_BF16 = 2 } pa_dtype_t;

/* Human-readable name of a status code (static string, never NULL). */
PA_API const char* pa_status_string(int32_t status);

/* Library ABI version: major * 10000 + minor * 100 + patch. */
PA_API int32_t pa_version(void);

/*
 * pa_reshape_and_cache — write new tokens' K and V into their cache slots.
 * [P1] §三 append_token fixes where a new token goes (the last block of the
 * sequence while it has room, else a fresh block); [P1] §五 leaves the write
 * itself to the block manager. Slot s names physical block s / block_size,
 * row s % block_size.
 *
 *   key, value       [num_tokens][num_kv_heads][head_dim], row t at element
 *                    t * kv_token_stride (heads and dims contiguous in a row)
 *   kv_token_stride  elements between consecutive token rows (>= H_kv*D)
 *   k_cache, v_cache pools (layout above), written in place
 *   block_stride     elements between consecutive physical blocks (>= 16*H_kv*D)
 *   num_blocks       physical blocks in each pool
 *   slot_mapping     int32 [num_tokens]; negative entries are skipped
 *   dtype            any pa_dtype_t; the copy is bit-exact
 * slot_mapping may be NULL only when num_tokens == 0. Non-negative slots must
 * be unique (duplicates race; the result is then undefined).
 */
PA_API int32_t pa_reshape_and_cache(const void* key, const void* value, int64_t kv_token_stride,
                             void* k_cache, void* v_cache, int64_t block_stride,
                             int64_t num_blocks, const int32_t* slot_mapping, int64_t num_tokens,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int32_t dtype, void* stream);

/*
 * pa_decode — one query token per sequence attends over its cached tokens
 * ([P1] §五 PagedAttention.forward), single pass over the KV cache.
 *
 *   out              [num_seqs][num_q_heads][head_dim], dtype; must not alias inputs
 *   query            [num_seqs][num_q_heads][head_dim], dtype
 *   k_cache, v_cache pools (layout above), dtype
 *   block_tables     int32 [num_seqs][block_table_stride]
 *   context_lens     int32 [num_seqs]: L_b, tokens in cache INCLUDING this
 *                    step's new token (written by pa_reshape_and_cache first);
 *                    every cached position precedes the query, so no mask.
 *                    L_b == 0 yields an all-zero output row.
 *   scale            score scale (1/sqrt(head_dim) in [P1] §五)
 * Query head h reads K/V head h / G (contiguous groups; with G == 1 this is
 * the multi-head case of the pages).
 */
PA_API int32_t pa_decode(void* out, const void* query, const void* k_cache, const void* v_cache,
                  int64_t block_stride, int64_t num_blocks, const int32_t* block_tables,
                  int32_t block_table_stride, const int32_t* context_lens, int32_t num_seqs,
                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                  int32_t block_size, float scale, int32_t dtype, void* stream);

/*
 * Bytes of device workspace pa_decode_splitkv needs: per (sequence, query
 * head, partition) one fp32 partial output row of head_dim plus its running
 * max and normaliser, and one work counter. Returns 0 for non-positive sizes.
 */
PA_API size_t pa_decode_splitkv_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                         int32_t max_context_len, int32_t partition_size);

/*
 * pa_decode_splitkv — pa_decode for long contexts: the cached tokens of each
 * sequence are cut into partitions of `partition_size` logical tokens, each
 * partition computes (max score, sum of exponentials, unnormalised output),
 * and a second kernel merges them by log-sum-exp. The merged result is the
 * same softmax as pa_decode (the decomposition is exact in exact arithmetic).
 *
 * The plan follows P = ceil(max_context_len / partition_size). With P <= 16
 * a workgroup computes one (kv head, sequence, partition) at a time and a
 * sequence with a single partition is written directly, bit-identical to
 * pa_decode. With P > 16 one wave computes one partition; over a 16-bit
 * cache the four consecutive partitions that one workgroup takes are merged
 * (by the same log-sum-exp) before they reach the workspace, and a sequence
 * of at most four partitions is written directly; over an FP8 cache
 * (pa_decode_splitkv_fp8) every partition goes through the merge. Either
 * way a call's result depends only on its arguments' values (reruns are
 * bit-identical).
 *
 * Arguments as pa_decode, plus
 *   max_context_len  upper bound of context_lens (host-known); sequences
 *                    longer than this are a precondition violation: such a
 *                    sequence is cut after ceil(max_context_len /
 *                    partition_size) partitions (attention over its first
 *                    that many times partition_size tokens), and nothing is
 *                    written outside the workspace
 *   partition_size   tokens per partition, a positive multiple of 16
 *   workspace        device buffer of at least
 *                    pa_decode_splitkv_workspace_bytes(...) bytes, 16-byte
 *                    aligned; contents on entry are ignored. Calls that
 *                    share a workspace must not overlap (same stream, or
 *                    ordered by the caller)
 */
PA_API int32_t pa_decode_splitkv(void* out, const void* query, const void* k_cache, const void* v_cache,
                          int64_t block_stride, int64_t num_blocks, const int32_t* block_tables,
                          int32_t block_table_stride, const int32_t* context_lens,
                          int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, float scale, int32_t dtype,
                          int32_t max_context_len, int32_t partition_size, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * pa_decode_splitkv_noalloc — pa_decode_splitkv for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same computation, kernels and results
 * (bit for bit), with the workspace taken from a static device array of
 * PA_NOALLOC_SCRATCH_BYTES (80 MiB) that the library holds on every GPU it
 * runs on until the process ends. The call allocates nothing: no hipMalloc,
 * no hipFree, no allocating library routine. Its first call on a device looks
 * up that device's copy of the array.
 *
 * Arguments as pa_decode_splitkv without workspace / workspace_bytes. A call
 * whose pa_decode_splitkv_workspace_bytes(...) exceeds
 * PA_NOALLOC_SCRATCH_BYTES returns PA_ERR_SCRATCH and launches nothing (80 MiB
 * covers, e.g., 8 sequences x 64 query heads of 131072-token contexts in
 * 512-token partitions at head_dim 128, which need 65 MiB). The array keeps
 * the last call's contents; every call resets what must start at zero (its
 * work counter) with a kernel of its own. All calls on one GPU share the one
 * array: calls that overlap in time on that GPU (different streams, or host
 * threads without ordering) race and give undefined results.
 */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)80 << 20)
PA_API int32_t pa_decode_splitkv_noalloc(void* out, const void* query, const void* k_cache,
                                         const void* v_cache, int64_t block_stride, int64_t num_blocks,
                                         const int32_t* block_tables, int32_t block_table_stride,
                                         const int32_t* context_lens, int32_t num_seqs,
                                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                         int32_t block_size, float scale, int32_t dtype,
                                         int32_t max_context_len, int32_t partition_size, void* stream);

/*
 * pa_decode_step — one whole decode step in one launch: each sequence's new
 * token (key_new/value_new row b) is written at position L_b - 1 of its cache,
 * in the slot its block table names (row (L_b-1) % 16 of physical block
 * block_tables[b][(L_b-1) / 16], the append rule of [P1] §三), then every
 * sequence attends over its L_b cached tokens exactly as pa_decode does. The
 * result equals pa_reshape_and_cache with those slots followed by pa_decode;
 * no slot_mapping is needed, and a sequence with L_b == 0 writes nothing.
 *
 *   key_new, value_new  [num_seqs][num_kv_heads][head_dim] of dtype, row b at
 *                       element b * kv_token_stride (>= H_kv*D)
 *   k_cache, v_cache    written (the new rows) and read
 * Other arguments and errors as pa_decode. The workgroup of (sequence,
 * kv head) writes its own head's new row before reading the cache; the
 * table entry of position L_b - 1 must name a block no other sequence reads
 * (a shared block is copied first, see pa_copy_blocks).
 */
PA_API int32_t pa_decode_step(void* out, const void* query, const void* key_new, const void* value_new,
                       int64_t kv_token_stride, void* k_cache, void* v_cache, int64_t block_stride,
                       int64_t num_blocks, const int32_t* block_tables, int32_t block_table_stride,
                       const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size, float scale,
                       int32_t dtype, void* stream);

/*
 * Step graphs ([P3] §5.3 captures the decode step per batch size as a CUDA
 * graph; here a HIP graph). pa_graph_begin creates a capture stream (a
 * non-blocking stream of default priority) and starts recording it; library
 * calls issued on *capture_stream are recorded, not run, until pa_graph_end
 * instantiates them. pa_graph_launch replays the recording on `stream`.
 * Pointers, sizes and grids are frozen at capture; device memory (lengths,
 * tables, K/V, queries) is read at replay, so one graph serves every step of
 * a batch size whose buffers keep their addresses. A captured split-KV call
 * also freezes its max_context_len and the plan derived from it (partition
 * count, workspace layout, workgroup, span or wave items): capture it with a
 * max_context_len that bounds the lengths of every later replay, since a
 * sequence that grows past it is cut at the planned partitions (see
 * pa_decode_splitkv). Recordable calls: those
 * that only launch kernels (every call except pa_swap_blocks and the pa_bm_*
 * host calls). The graph owns its stream and executable until
 * pa_graph_destroy (which also abandons an unfinished recording). A graph is
 * not thread-safe; replays on one stream are ordered like any launch.
 * Errors: PA_ERR_NULL_PTR, PA_ERR_SHAPE (end without begin, launch before
 * end), PA_ERR_HIP (the runtime refused to capture or instantiate).
 */
typedef struct pa_graph pa_graph;
PA_API int32_t pa_graph_begin(pa_graph** graph, void** capture_stream);
PA_API int32_t pa_graph_end(pa_graph* graph);
PA_API int32_t pa_graph_launch(pa_graph* graph, void* stream);
PA_API void pa_graph_destroy(pa_graph* graph);

/*
 * FP8 KV cache. [P3] (introduction) lists FP8 among the quantisation schemes
 * the engine supports and gives no format; the format here is the OCP 8-bit
 * floating point E4M3 ("e4m3fn": bias 7, 3 mantissa bits, subnormals, no
 * infinities, NaN = S.1111.111, largest finite 448), one byte per element, in
 * the pool layout above with block_stride counted in bytes. Each kv head h has
 * two float32 scales: a stored code c stands for K = value(c) * k_scale[h]
 * (V likewise with v_scale[h]). k_scale and v_scale are DEVICE float32 arrays
 * [num_kv_heads], finite and > 0 (a precondition, not checked).
 */

/*
 * pa_reshape_and_cache_fp8 — pa_reshape_and_cache into an FP8 cache. Element
 * x of head h is stored as the e4m3 code nearest to fl32(x / scale[h]) (x
 * widened exactly to float32, one correctly rounded float32 division; ties to
 * the even mantissa; finite values beyond +-448 and infinities saturate to
 * +-448; NaN stays NaN; the sign of zero is kept).
 *
 *   key, value       [num_tokens][num_kv_heads][head_dim] of `dtype` (any
 *                    pa_dtype_t), row t at element t * kv_token_stride
 *   k_cache, v_cache FP8 pools, block_stride in bytes (>= 16*H_kv*D, a
 *                    multiple of 16)
 *   k_scale, v_scale float32 [num_kv_heads], device
 * Other arguments, slot rules and errors as pa_reshape_and_cache.
 */
PA_API int32_t pa_reshape_and_cache_fp8(const void* key, const void* value, int64_t kv_token_stride,
                                 void* k_cache, void* v_cache, int64_t block_stride,
                                 int64_t num_blocks, const int32_t* slot_mapping, int64_t num_tokens,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                 const float* k_scale, const float* v_scale, int32_t dtype,
                                 void* stream);

/*
 * pa_decode_fp8 — pa_decode over an FP8 cache: the same attention with K and
 * V dequantised as above. `dtype` (PA_DTYPE_F16 or PA_DTYPE_BF16) is the type
 * of query and out; cache codes are widened to it exactly, products
 * accumulate in fp32, k_scale[h] joins the score scale and v_scale[h] the
 * output. block_stride is in bytes. Returns PA_ERR_DTYPE for PA_DTYPE_F32.
 */
PA_API int32_t pa_decode_fp8(void* out, const void* query, const void* k_cache, const void* v_cache,
                      int64_t block_stride, int64_t num_blocks, const int32_t* block_tables,
                      int32_t block_table_stride, const int32_t* context_lens, int32_t num_seqs,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, float scale, const float* k_scale, const float* v_scale,
                      int32_t dtype, void* stream);

/*
 * pa_decode_splitkv_fp8 — pa_decode_splitkv over an FP8 cache (dequantised
 * as in pa_decode_fp8). Workspace size from pa_decode_splitkv_workspace_bytes,
 * which does not depend on the cache type; other arguments as
 * pa_decode_splitkv, block_stride in bytes.
 */
PA_API int32_t pa_decode_splitkv_fp8(void* out, const void* query, const void* k_cache,
                              const void* v_cache, int64_t block_stride, int64_t num_blocks,
                              const int32_t* block_tables, int32_t block_table_stride,
                              const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                              float scale, const float* k_scale, const float* v_scale,
                              int32_t dtype, int32_t max_context_len, int32_t partition_size,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_step_fp8 — pa_decode_step over an FP8 cache: the new rows (of
 * dtype, the query type) are quantised as in pa_reshape_and_cache_fp8, then
 * decode as pa_decode_fp8. block_stride is in bytes.
 */
PA_API int32_t pa_decode_step_fp8(void* out, const void* query, const void* key_new, const void* value_new,
                           int64_t kv_token_stride, void* k_cache, void* v_cache,
                           int64_t block_stride, int64_t num_blocks, const int32_t* block_tables,
                           int32_t block_table_stride, const int32_t* context_lens,
                           int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, float scale,
                           const float* k_scale, const float* v_scale, int32_t dtype,
                           void* stream);

/*
 * pa_copy_blocks — the device half of copy-on-write ([P2] Block 管理器: requests
 * that share a prompt prefix share its physical blocks, and a shared block is
 * copied only when one of them must write into it). For each (src, dst) pair,
 * the rows of block dst in both pools become those of block src, bit for bit.
 *
 *   k_cache, v_cache pools (layout above), written in place
 *   block_stride     elements between consecutive physical blocks (>= 16*H_kv*D)
 *   num_blocks       physical blocks in each pool
 *   num_kv_heads, head_dim, dtype   size of a block's rows: 16*H_kv*D elements
 *   pairs            int32 [num_pairs][2] (src, dst) in DEVICE memory; pairs
 *                    with an index outside [0, num_blocks) are skipped
 * Preconditions: no dst is the src or dst of another pair (the copies run in
 * parallel). pairs may be NULL only when num_pairs == 0.
 */
PA_API int32_t pa_copy_blocks(void* k_cache, void* v_cache, int64_t block_stride, int64_t num_blocks,
                              int32_t num_kv_heads, int32_t head_dim, int32_t dtype, const int32_t* pairs,
                              int64_t num_pairs, void* stream);

/*
 * pa_swap_blocks — move whole blocks between a device pool and a host pool
 * (the CPU swap space of [P3] §5.3): for each (src, dst) pair, block dst of
 * the destination pool becomes block src of the source pool. Either pool may
 * be device memory or pinned host memory (the copy engine moves the bytes;
 * runs of consecutive pairs are merged into one copy). Call once for K and
 * once for V.
 *
 *   dst_pool, dst_blocks   destination pool and its number of blocks
 *   src_pool, src_blocks   source pool and its number of blocks
 *   block_bytes            bytes per block (block_stride * element bytes)
 *   pairs                  int64 [num_pairs][2] (src, dst) in HOST memory
 * Every pair is checked on the host before any copy is issued: an index
 * outside its pool returns PA_ERR_SHAPE and moves nothing. Asynchronous on
 * `stream`; host memory that is not pinned makes the copies synchronous.
 */
PA_API int32_t pa_swap_blocks(void* dst_pool, int64_t dst_blocks, const void* src_pool, int64_t src_blocks,
                              int64_t block_bytes, const int64_t* pairs, int64_t num_pairs, void* stream);

/*
 * Host block manager ([P1] §三 PagedAttentionManager, with the copy-on-write of
 * [P2] Block 管理器). A physical block carries a share count. pa_bm_allocate
 * gives a new request ceil(num_tokens / block_size) blocks from the head of
 * the free list, or PA_ERR_NO_BLOCKS and nothing when fewer are free.
 * pa_bm_append adds one token: it fills the last block, takes a new block
 * from the head of the free list once that is full, and — when the last block
 * is shared and not full — takes a fresh block for it, lowers the shared
 * block's count and returns (cow_src, cow_dst), the pair pa_copy_blocks must
 * copy before the token's K/V are written (-1, -1 when no copy is needed);
 * *slot is the new token's slot for pa_reshape_and_cache. pa_bm_share_prefix
 * lets a new request `child` start with the first num_tokens tokens of `src`
 * by sharing the ceil(num_tokens / block_size) blocks that hold them;
 * pa_bm_fork shares all of them. pa_bm_free lowers the count of each block of
 * the request; a block at zero goes to the tail of the free list. Requests are
 * keyed by 64-bit ids; a refused call changes nothing. Not thread-safe: one
 * manager per host thread, or external locking.
 *
 *   pa_bm_create   free_order: a permutation of 0 .. num_blocks-1 giving the
 *                  initial free list (NULL: ascending); returns NULL on bad
 *                  arguments or when out of host memory
 *   pa_bm_block_table / pa_bm_free_list   copy up to `capacity` entries to
 *                  `out` (may be NULL) and return the full count (-1: unknown)
 *   pa_bm_slots    slots of positions pos0 .. pos0+count-1 of a request
 */
typedef struct pa_block_manager pa_block_manager;
PA_API pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order);
PA_API void pa_bm_destroy(pa_block_manager* m);
PA_API int32_t pa_bm_allocate(pa_block_manager* m, int64_t seq, int64_t num_tokens);
PA_API int32_t pa_bm_append(pa_block_manager* m, int64_t seq, int64_t* slot, int32_t* cow_src, int32_t* cow_dst);
PA_API int32_t pa_bm_share_prefix(pa_block_manager* m, int64_t src, int64_t child, int64_t num_tokens);
PA_API int32_t pa_bm_fork(pa_block_manager* m, int64_t parent, int64_t child);
PA_API int32_t pa_bm_free(pa_block_manager* m, int64_t seq);
PA_API int32_t pa_bm_num_free(const pa_block_manager* m);
PA_API int64_t pa_bm_seq_len(const pa_block_manager* m, int64_t seq);
PA_API int32_t pa_bm_block_table(const pa_block_manager* m, int64_t seq, int32_t* out, int32_t capacity);
PA_API int32_t pa_bm_ref_count(const pa_block_manager* m, int32_t block);
PA_API int32_t pa_bm_free_list(const pa_block_manager* m, int32_t* out, int32_t capacity);
PA_API int32_t pa_bm_slots(const pa_block_manager* m, int64_t seq, int64_t pos0, int64_t count, int32_t* out);

/*
 * Prefix caching ([P2] Prefix Caching → 自动检测与复用: the prompt content is
 * hashed into cache keys, a new request looks up the longest cached prefix,
 * only the rest needs its KV computed, and the hit blocks are shared through
 * the block counts). Block granular: the key of full block i of a prompt is a
 * 64-bit FNV-1a hash chained over block i-1's key and the block's own token
 * ids, standing for the whole prefix up to the block's end; a hit also checks
 * the stored parent key and tokens exactly. Partly filled blocks are never
 * cached.
 *
 *   pa_bm_allocate_cached  a new request for prompt `tokens` (int32 token ids,
 *                  num_tokens of them): shares the longest run of cached full
 *                  blocks from the prompt's start, takes fresh blocks from the
 *                  head of the free list for the rest, all or nothing
 *                  (PA_ERR_NO_BLOCKS changes nothing); *cached_tokens = the
 *                  number of leading tokens whose KV is already cached (a
 *                  multiple of block_size) — the caller computes and writes
 *                  KV for positions >= *cached_tokens only
 *   pa_bm_publish  enters the request's full blocks that hold tokens[0 ..
 *                  num_tokens) (at most its length) into the cache, once their
 *                  KV is written; a key already cached keeps its block, a
 *                  block is cached under one key at most; *added (may be
 *                  NULL) = entries added
 *   pa_bm_num_cached  entries in the cache
 * A cached block whose count drops to zero stays cached while it waits in the
 * free list (a hit takes it back out); taken from the free list for other
 * tokens it leaves the cache. Cached blocks are full, so appends never write
 * into them.
 */
PA_API int32_t pa_bm_allocate_cached(pa_block_manager* m, int64_t seq, const int32_t* tokens, int64_t num_tokens,
                              int64_t* cached_tokens);
PA_API int32_t pa_bm_publish(pa_block_manager* m, int64_t seq, const int32_t* tokens, int64_t num_tokens,
                      int32_t* added);
PA_API int32_t pa_bm_num_cached(const pa_block_manager* m);

/*
 * pa_prefill_chunked — a chunk of new query tokens per sequence attends over
 * the sequence's cache (prior tokens plus the chunk itself, already written
 * by pa_reshape_and_cache), on bf16/f16 matrix cores. The pages only name the
 * chunked-prefill switch ([P3] §5.3); the reading implemented: sequence b owns
 * query rows cu_q_lens[b] .. cu_q_lens[b+1]-1, and query i of the chunk sits
 * at absolute position seq_lens[b] - q_len_b + i; with `causal` it sees keys
 * 0 .. that position (itself included), otherwise all seq_lens[b] keys.
 *
 *   out              [num_q_tokens][num_q_heads][head_dim], dtype
 *   query            [num_q_tokens][num_q_heads][head_dim], dtype
 *   cu_q_lens        int32 [num_seqs + 1], cumulative chunk lengths, cu[0] = 0
 *   max_q_len        upper bound of the chunk lengths (host-known)
 *   num_q_tokens     cu_q_lens[num_seqs]
 *   seq_lens         int32 [num_seqs], keys in cache INCLUDING the chunk
 *   causal           0 or 1
 *   dtype            PA_DTYPE_BF16 or PA_DTYPE_F16
 * Preconditions beyond the common ones: 0 <= q_len_b <= min(max_q_len, seq_lens[b]),
 * cu_q_lens non-decreasing with cu_q_lens[num_seqs] <= num_q_tokens. A call that
 * violates them still touches only rows [0, num_q_tokens) (offsets are clamped
 * to it, a chunk longer than seq_lens[b] is cut to that length); the values of
 * the affected rows are then unspecified.
 */
PA_API int32_t pa_prefill_chunked(void* out, const void* query, const int32_t* cu_q_lens,
                           int32_t max_q_len, int64_t num_q_tokens, const void* k_cache,
                           const void* v_cache, int64_t block_stride, int64_t num_blocks,
                           const int32_t* block_tables, int32_t block_table_stride,
                           const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           float scale, int32_t causal, int32_t dtype, void* stream);

/*
 * pa_prefill_chunked_fp8 — pa_prefill_chunked over an FP8 (e4m3) cache written
 * by pa_reshape_and_cache_fp8: the same chunked attention over the dequantised
 * keys and values, value(code) * k_scale[h] and value(code) * v_scale[h] (the
 * FP8 reading of pa_decode_fp8). Queries and outputs are f16 or bf16; the
 * pools hold one byte per element and block_stride counts bytes; k_scale and
 * v_scale are float32 [num_kv_heads] device arrays (NULL: PA_ERR_NULL_PTR).
 * Other arguments, preconditions and errors as pa_prefill_chunked.
 */
PA_API int32_t pa_prefill_chunked_fp8(void* out, const void* query, const int32_t* cu_q_lens,
                               int32_t max_q_len, int64_t num_q_tokens, const void* k_cache,
                               const void* v_cache, int64_t block_stride, int64_t num_blocks,
                               const int32_t* block_tables, int32_t block_table_stride,
                               const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               float scale, int32_t causal, const float* k_scale, const float* v_scale,
                               int32_t dtype, void* stream);

/*
 * pa_read_kv_rows — read-bandwidth calibration beside the attention calls, not
 * part of the attention path: reads exactly the K and V rows that pa_decode
 * (partition_size == 0) or pa_decode_splitkv (partition_size > 0, the same
 * partitions) would read for these arguments — every cached token's row of
 * every kv head, through the block tables — with the same 16-byte
 * non-temporal loads and no arithmetic. Each wave stores an XOR of the words
 * it read into sink[some index < sink_words] (so the reads cannot be dropped;
 * the values carry no meaning). Timing it next to an attention call on the
 * same cache measures how fast the memory system delivers that access set.
 *
 *   cache_elem_bytes  1 (FP8 cache), 2 (f16/bf16) or 4 (f32)
 *   sink              device uint32 [sink_words], sink_words >= 1
 * Other arguments as pa_decode_splitkv; the split-KV walk supports up to 1024
 * sequences (PA_ERR_UNSUPPORTED beyond). Out-of-range table entries are read
 * as block 0; nothing outside the pools and sink is addressed.
 */
PA_API int32_t pa_read_kv_rows(const void* k_cache, const void* v_cache, int64_t block_stride, int64_t num_blocks,
                               const int32_t* block_tables, int32_t block_table_stride, const int32_t* context_lens,
                               int32_t num_seqs, int32_t num_kv_heads, int32_t head_dim, int32_t cache_elem_bytes,
                               int32_t max_context_len, int32_t partition_size, uint32_t* sink, int64_t sink_words,
                               void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_KV_CACHE_463_AMD_PA_H */

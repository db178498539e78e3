/*
 * paged_kv.h — C ABI of libpagedkv.so: a paged KV cache and its decode attention
 * for AMD Instinct MI355X (gfx950).
 *
 * Sources of the method (cited by page title and section):
 *   [DS]  deepsonar.com.cn, "PagedAttention de vLLM : comment la gestion de la VRAM
 *         soutient l'inférence des grands modèles" (§2.1 KV bytes; §2.2 blocks, block
 *         table, on-demand allocation; §2.3 reference counts and copy-on-write; §2.4
 *         free-block queue; §2.6 the block table handed to the attention kernel;
 *         §VII minimal skeleton).
 *   [CD]  chester-dev.com, "vLLM transforme la mémoire GPU en système d'exploitation
 *         pour LLM" (section on PagedAttention turning history into reusable blocks:
 *         logical order kept, physical placement scattered).
 *   [DL]  deeplearn.tn, "PagedAttention : comment optimiser la mémoire GPU lors de
 *         l'inférence des LLM" (worked allocation example with block size 4; the
 *         block-table section; PagedAttention vs. FlashAttention: tiles in on-chip
 *         memory with an incremental softmax).
 *
 * Conventions for every entry point:
 *   - Returns a paged_kv_status; never throws, never aborts.  On failure nothing is
 *     launched and host state is unchanged unless the entry point says otherwise;
 *     paged_kv_last_error() then describes the failure (thread-local string).
 *   - "device" pointers are HIP device memory owned by the caller unless stated;
 *     "host" pointers are ordinary process memory.  The library keeps no pointer
 *     to caller memory after a call returns, except the pool buffers handed to
 *     paged_kv_pool_create.
 *   - Device work is enqueued on `stream` (a hipStream_t passed as void*; NULL is the
 *     null stream) and is asynchronous: no call on the decode path synchronises the
 *     device.
 *   - A pool object is not thread-safe; calls on distinct pools may run concurrently.
 *
 * Memory layout of the KV pool (the pages leave it open; this is the library's):
 *   X = 16 / element bytes (8 for fp16/bf16, 4 for fp32); BS = block size.  A block of
 *   more than 16 tokens (BS a multiple of 16) is NS = BS / 16 sub-blocks of TB = 16
 *   tokens stored one after the other; up to 16 tokens NS = 1 and TB = BS.
 *   K pool: [num_blocks][num_kv_heads][NS][head_dim / X][TB][X]
 *   V pool: [num_blocks][num_kv_heads][NS][head_dim][TB]
 *   Element d of the key (value) of the token in slot `slot` = block * BS + offset,
 *   KV head h, is K[block][h][offset / TB][d / X][offset % TB][d % X]
 *   (V[block][h][offset / TB][d][offset % TB]).
 *   One (block, KV head) region of K or of V is BS * head_dim contiguous elements, and
 *   each 16-token sub-block of it 16 * head_dim.
 */
#ifndef PAGED_KV_H
#define PAGED_KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PAGED_KV_OK = 0,
    PAGED_KV_ERR_INVALID_ARG = 1,     /* null pointer, bad size, unsupported shape value */
    PAGED_KV_ERR_OUT_OF_BLOCKS = 2,   /* the free queue cannot supply the blocks needed */
    PAGED_KV_ERR_UNSUPPORTED = 3,     /* valid request the library has no kernel for */
    PAGED_KV_ERR_HIP = 4,             /* a HIP runtime call failed */
    PAGED_KV_ERR_NO_SUCH_SEQ = 5,     /* unknown or released sequence id */
    PAGED_KV_ERR_BUFFER_TOO_SMALL = 6 /* caller buffer (copies list, workspace) too small */
} paged_kv_status;

typedef enum { PAGED_KV_F32 = 0, PAGED_KV_F16 = 1, PAGED_KV_BF16 = 2 } paged_kv_dtype;

/* Pool shape.  block_size: tokens per block (any >= 1 for the allocator; 1, 16 or 32
 * for the device kernels: [DS] §2.2 gives 16 as the usual size, [DL] page-size section
 * of SGLang weighs 16/32 against 1).  dtype: element type of K and V (and of the
 * queries given to paged_attention_decode). */
typedef struct {
    int32_t num_blocks;
    int32_t block_size;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t dtype;      /* paged_kv_dtype */
    int32_t flags;      /* PAGED_KV_POOL_* bits */
} paged_kv_pool_desc;

/* Allocator only: no device memory is allocated or referenced by the pool object. */
#define PAGED_KV_POOL_HOST_ONLY 1
/* Prefix caching ([DS] §2.4, block pool and hash chain of V1; §VII step 5): the pool
 * keeps a map from chained block hash to physical block for full blocks written with
 * paged_kv_seq_append_tokens, and paged_kv_seq_create_prefix takes cached blocks over. */
#define PAGED_KV_POOL_PREFIX_CACHE 2

typedef struct paged_kv_pool paged_kv_pool; /* opaque host-side object */

/* ---------------------------------------------------------------- misc ---- */

/* Message for a status code (static string). */
const char* paged_kv_status_string(paged_kv_status status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* paged_kv_last_error(void);

/* [DS] §2.1: KV-cache bytes per token = 2 (K and V) x layers x KV heads x head dim x
 * bytes per element.  Returns 0 if any argument is negative. */
uint64_t paged_kv_bytes_per_token(int32_t layers, int32_t kv_heads, int32_t head_dim,
                                  int32_t dtype_bytes);

/* Bytes of one pool (K or V) for `desc`: num_blocks * num_kv_heads * block_size *
 * head_dim * element bytes.  0 if desc is invalid. */
size_t paged_kv_pool_bytes(const paged_kv_pool_desc* desc);

/* ------------------------------------------------------- pool + allocator ---- */

/* [DS] §2.2, §VII step 1: carve the KV memory into desc->num_blocks fixed-size blocks.
 *   free_order  host int32[num_blocks], a permutation of 0..num_blocks-1: the initial
 *               free-queue order, head first ([DS] §2.4: allocation takes the head).
 *               NULL = 0, 1, ..., num_blocks-1.
 *   k_pool, v_pool  device buffers of paged_kv_pool_bytes(desc) bytes each, owned by
 *               the caller and left untouched; or both NULL: the library allocates
 *               them (hipMalloc, contents set to all-ones bytes, i.e. NaN) and frees
 *               them in paged_kv_pool_destroy.  Ignored with PAGED_KV_POOL_HOST_ONLY.
 *   out         receives the pool object.
 * Errors: INVALID_ARG (sizes < 1, head_dim not a multiple of X, bad dtype, free_order
 * not a permutation, exactly one of k_pool/v_pool NULL), HIP (allocation failed). */
paged_kv_status paged_kv_pool_create(const paged_kv_pool_desc* desc, const int32_t* free_order,
                                     void* k_pool, void* v_pool, paged_kv_pool** out);

/* Release the pool object (and the buffers it allocated itself).  NULL is a no-op. */
void paged_kv_pool_destroy(paged_kv_pool* pool);

/* The pool's device buffers (NULL, NULL for a host-only pool) and its descriptor. */
paged_kv_status paged_kv_pool_buffers(const paged_kv_pool* pool, void** k_pool, void** v_pool);
paged_kv_status paged_kv_pool_get_desc(const paged_kv_pool* pool, paged_kv_pool_desc* desc);

/* New empty sequence.  Ids are 0, 1, 2, ... in create/fork order, never reused. */
paged_kv_status paged_kv_seq_create(paged_kv_pool* pool, int32_t* seq_id);

/* [DS] §2.3: new sequence sharing every block of `parent`; each shared block's
 * reference count goes up by one.  No block is copied here. */
paged_kv_status paged_kv_seq_fork(paged_kv_pool* pool, int32_t parent, int32_t* child);

/* [DS] §2.2, §2.3, §VII steps 2-3; [DL] worked example.  Reserve slots for n_tokens
 * new tokens of `seq`, in order.  A block is taken from the head of the free queue
 * only when the token lands at offset 0 of a new block.  If the sequence's last block
 * is partly filled and shared (count > 1), it is first copied to a fresh block: the
 * (source, destination) pair is reported and the sequence's table points at the copy.
 *   slots_out   host int32[n_tokens]: slot = physical block * block_size + offset.
 *   copies_out  host int32[2 * max_copies]: (src, dst) pairs, to be applied with
 *               paged_kv_copy_blocks before the new tokens are written (at most 1).
 *   n_copies    receives the number of pairs written.
 * Errors: NO_SUCH_SEQ; INVALID_ARG (n_tokens < 0, null outputs); OUT_OF_BLOCKS and
 * BUFFER_TOO_SMALL leave the allocator exactly as it was. */
paged_kv_status paged_kv_seq_append(paged_kv_pool* pool, int32_t seq, int32_t n_tokens,
                                    int32_t* slots_out, int32_t* copies_out, int32_t max_copies,
                                    int32_t* n_copies);

/* paged_kv_seq_append over several sequences, in order (one decode step appends one
 * token to each).  slots_out: host int32[sum(counts)] grouped by sequence in input
 * order; copies_out: host int32[2 * max_copies].  Stops at the first sequence that
 * fails: *n_done receives the number of sequences fully appended (their appends
 * stay); the failing one and those after it are unchanged. */
paged_kv_status paged_kv_append_batch(paged_kv_pool* pool, const int32_t* seqs,
                                      const int32_t* counts, int32_t n_seqs, int32_t* slots_out,
                                      int32_t* copies_out, int32_t max_copies, int32_t* n_copies,
                                      int32_t* n_done);

/* Release a sequence (finished, cancelled or preempted): its blocks, in logical order,
 * lose one reference; each block reaching zero goes to the tail of the free queue. */
paged_kv_status paged_kv_seq_free(paged_kv_pool* pool, int32_t seq);

/* [DS] §2.6: the block table handed to the attention kernel.  Writes host
 * int32 tables_out[n][max_blocks] (physical ids in logical order, padded with -1)
 * and host int32 context_lens_out[n] (tokens written).  INVALID_ARG if a table does
 * not fit max_blocks. */
paged_kv_status paged_kv_block_tables(const paged_kv_pool* pool, const int32_t* seq_ids,
                                      int32_t n, int32_t max_blocks, int32_t* tables_out,
                                      int32_t* context_lens_out);

/* Tokens and blocks of one sequence. */
paged_kv_status paged_kv_seq_info(const paged_kv_pool* pool, int32_t seq, int32_t* context_len,
                                  int32_t* num_blocks);

/* Reference count of a physical block (0 = free). */
paged_kv_status paged_kv_block_refcount(const paged_kv_pool* pool, int32_t block,
                                        int32_t* refcount);

/* Pool occupancy: free blocks, used blocks, and reserved-but-empty slots summed over
 * live sequences (block_size * blocks - tokens, < block_size per sequence: [DS] §2.2). */
paged_kv_status paged_kv_stats(const paged_kv_pool* pool, int64_t* num_free, int64_t* num_used,
                               int64_t* waste_slots);

/* ------------------------------------------------------- prefix caching ---- */

/* Chained block hash ([DS] §2.4): SHA-256 (FIPS 180-4) over the parent block's 32-byte
 * hash (NULL: 32 zero bytes, a sequence's first block), the n token ids as
 * little-endian int32 and extra_key as a little-endian int64, into out[32].  One
 * differing token changes the hash of its block and, through the parent, of every
 * later block. */
paged_kv_status paged_kv_block_hash(const uint8_t* parent, const int32_t* tokens, int32_t n,
                                    int64_t extra_key, uint8_t* out);

/* New sequence for a prompt of n token ids ([DS] §2.4, comparison block by block along
 * the hash chain; §VII step 5).  Walks the prompt's full blocks that lie inside its
 * first n-1 tokens (the last prompt token is always recomputed); each block whose
 * chained hash (with extra_key) is in the pool's map is taken over: its reference
 * count goes up and, if it was waiting in the free queue, it leaves the queue.  The
 * walk stops at the first miss.  *n_cached = tokens now held (a multiple of
 * block_size); the caller writes the rest with paged_kv_seq_append_tokens.  Errors:
 * PAGED_KV_ERR_UNSUPPORTED without PAGED_KV_POOL_PREFIX_CACHE; the pool is unchanged
 * on any error. */
paged_kv_status paged_kv_seq_create_prefix(paged_kv_pool* pool, const int32_t* prompt, int32_t n,
                                           int64_t extra_key, int32_t* seq_id, int32_t* n_cached);

/* paged_kv_seq_append with the new tokens' ids: on a prefix-caching pool, each block of
 * a sequence made by paged_kv_seq_create_prefix that this append fills gets its chained
 * hash and enters the map (unless the hash is already there).  A plain
 * paged_kv_seq_append to such a sequence stops its registration for good.  Taking a
 * block from the queue head evicts its cached hash first ([DS] §2.4: the queue order is
 * the LRU order).  Arguments and errors as paged_kv_seq_append. */
paged_kv_status paged_kv_seq_append_tokens(paged_kv_pool* pool, int32_t seq, const int32_t* tokens,
                                           int32_t n_tokens, int32_t* slots_out,
                                           int32_t* copies_out, int32_t max_copies,
                                           int32_t* n_copies);

/* Blocks in the hash map, blocks taken over by prompts so far, cached blocks evicted. */
paged_kv_status paged_kv_prefix_stats(const paged_kv_pool* pool, int64_t* cached_blocks,
                                      int64_t* hit_blocks, int64_t* evictions);

/* ------------------------------------------------------------ device ops ---- */

/* [DS] §2.3: copy-on-write copies.  For each of the n pairs (device int32[n][2],
 * (src, dst)), block dst of both pools becomes a copy of block src (all heads, all
 * slots).  Pairs with an id outside [0, num_blocks) are skipped.  Destinations must be
 * distinct and must not be sources in the same call.  n == 0 launches nothing. */
paged_kv_status paged_kv_copy_blocks(const paged_kv_pool_desc* desc, void* k_pool, void* v_pool,
                                     const int32_t* pairs, int32_t n, void* stream);

/* Write each new token's key and value into its slot ([DS] §2.2; [DL] worked example).
 *   key, value   device, element type desc->dtype, [num_tokens][num_kv_heads][head_dim]
 *                with token stride key_stride / value_stride elements (>= heads*dim;
 *                heads and dims contiguous).
 *   slot_mapping device int32[num_tokens]; -1 = padding, not written; slots outside
 *                [0, num_blocks * block_size) are not written either.
 * Layout of the destination: see the top of this file.  Requires block_size 1, 16 or
 * 32 and head_dim a multiple of X.  num_tokens == 0 launches nothing.  Two tokens with one
 * slot in a call: the surviving value is unspecified. */
paged_kv_status reshape_and_cache(const paged_kv_pool_desc* desc, const void* key,
                                  const void* value, int64_t key_stride, int64_t value_stride,
                                  void* k_pool, void* v_pool, const int32_t* slot_mapping,
                                  int32_t num_tokens, void* stream);

/* partition_tokens value that lets the library pick the schedule for the batch shape
 * (paged_attention_auto_partition_tokens). */
#define PAGED_KV_PARTITION_AUTO (-1)

/* A scheduling choice for paged_attention_decode below (what it computes is cited
 * there; the schedule changes only the summation order within tolerance).
 * The schedule PAGED_KV_PARTITION_AUTO picks, as a partition_tokens value: 0 (stream-K)
 * when the batch has at least 65536 (sequence, head unit, 16-token tile) tiles on the
 * bound max_context_len (64 per wave slot of the chip), else fixed partitions: 512
 * tokens when that gives at least 256 (sequence, head unit, partition) workgroups, one
 * per compute unit, else 256.  A head unit is a KV head for the MFMA kernels (fp16/bf16
 * with 2 to 16 query heads per KV head) and a query head otherwise.  Small batches go
 * to fixed partitions because stream-K then has few tiles per wave and merges many
 * pieces per unit at the end of the launch.  Depends on the arguments only (no device
 * state), so workspace sizing and the launches agree.  -1 if an argument is invalid. */
int32_t paged_attention_auto_partition_tokens(const paged_kv_pool_desc* desc, int32_t num_seqs,
                                              int32_t num_q_heads, int32_t max_context_len);

/* Bytes of workspace paged_attention_decode needs for this batch shape and pool (0 when
 * nothing needs merging).  Same partition_tokens convention as paged_attention_decode.
 * 0 if an argument is invalid. */
size_t paged_attention_workspace_bytes(const paged_kv_pool_desc* desc, int32_t num_seqs,
                                       int32_t num_q_heads, int32_t max_context_len,
                                       int32_t partition_tokens);

/* Paged decode attention ([DS] §2.2, §2.6; [CD]; [DL] PagedAttention vs.
 * FlashAttention): for every sequence s and query head h,
 *   out[s][h] = sum_t softmax_t(scale * q[s][h] . k_t) v_t  over the context_lens[s]
 * tokens of s, read through its block table; query head h uses KV head
 * h / (num_q_heads / num_kv_heads).
 *   out           device [num_seqs][num_q_heads][head_dim], type out_dtype (desc->dtype
 *                 or PAGED_KV_F32)
 *   q             device [num_seqs][num_q_heads][head_dim], type desc->dtype
 *   k_pool/v_pool device pools (layout above)
 *   block_tables  device int32[num_seqs][max_blocks_per_seq]; entries past a
 *                 sequence's last block are never read
 *   context_lens  device int32[num_seqs]
 *   max_context_len  host bound on every context_lens[s] (sizes the launch)
 *   partition_tokens 0: stream-K schedule — the batch's (sequence, head unit,
 *                 16-token tile) tiles are split evenly over a fixed set of waves
 *                 (one per resident wave slot on MI355X: 1024 or 3072 by kernel, fewer
 *                 for small batches) and the pieces of a
 *                 sequence's head unit cut by those splits are merged by log-sum-exp
 *                 (used for up to 8192 sequences; larger batches fall back to 512-token
 *                 partitions).  > 0: fixed split-K partitions of that many tokens
 *                 (multiple of 16), merged the same way.  PAGED_KV_PARTITION_AUTO (-1):
 *                 the value paged_attention_auto_partition_tokens returns for the same
 *                 arguments.  Other negative values: INVALID_ARG.
 *   workspace     device buffer of paged_attention_workspace_bytes(...) bytes (may be
 *                 NULL when that is 0).  Zero-fill it before its first use (e.g.
 *                 hipMemsetAsync): the stream-K schedule keeps one merge counter per
 *                 (sequence, head unit) at its start, and every call leaves them at
 *                 zero again; the rest is scratch.  So a workspace can be reused without zero-filling again as
 *                 long as no call has more counters (num_seqs x head units; a head unit
 *                 is a KV head for fp16/bf16 with 2..16 query heads per KV head, else a
 *                 query head) than a call made on it since the last zero-fill.  Calls
 *                 sharing one workspace must not overlap.
 * A sequence whose context_len is outside [1, max_context_len], or whose table holds
 * an id outside [0, num_blocks) below its length, gets NaN outputs; nothing outside
 * the buffers is read.  Requires block_size 1, 16 or 32, head_dim 64, 128 or 256,
 * num_q_heads % num_kv_heads == 0 and a group of at most 16 query heads.
 * Results do not depend on where blocks sit in the pool, nor on whether a block is
 * shared: the summation order follows logical token positions only. */
paged_kv_status paged_attention_decode(const paged_kv_pool_desc* desc, void* out, int32_t out_dtype,
                                       const void* q, const void* k_pool, const void* v_pool,
                                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       const int32_t* context_lens, int32_t num_seqs,
                                       int32_t num_q_heads, int32_t max_context_len, float scale,
                                       int32_t partition_tokens, void* workspace,
                                       size_t workspace_bytes, void* stream);

/* One decode step of a layer in a single launch where the schedule allows it: the cache
 * write of reshape_and_cache for one new token per sequence, then paged_attention_decode
 * over contexts that include that token.  deepsonar "PagedAttention de vLLM …" §2.2
 * (each new token's K/V lands in its sequence's current block, then the attention reads
 * the blocks through the table) and §2.6 (graph capture of the decode step: fewer
 * launches per layer).
 *   new_k, new_v  device [num_seqs][num_kv_heads][head_dim] of the pool dtype, rows
 *                 contiguous, 16-byte aligned: the new token of sequence s.
 *   slot_mapping  device int32 [num_seqs]: the pool slot of that token, which must be
 *                 the slot of position context_lens[s] - 1 in the sequence's table
 *                 (the allocator's append returns exactly that); -1 (or any slot
 *                 outside the pool) writes nothing.
 *   Every other argument as for paged_attention_decode, context_lens counting the new
 *   token.  The caller owns all buffers.
 * With fixed partitions and the matrix-core kernel (fp16/bf16, 2..16 query heads per KV
 * head) this is one kernel: the workgroup whose partition holds position ctx - 1
 * writes the token before reading, and the last workgroup of each (sequence, KV head)
 * to finish merges the partitions in partition order (same arithmetic as the merge
 * kernel; bit-identical to reshape_and_cache + paged_attention_decode when a sequence
 * has at most 16 partitions).  Otherwise (stream-K, the vector-ALU kernel) it launches
 * reshape_and_cache and then paged_attention_decode.  Errors as for
 * paged_attention_decode, plus PAGED_KV_ERR_INVALID_ARG for null or misaligned
 * new_k/new_v/slot_mapping; nothing is launched on an error. */
paged_kv_status paged_attention_decode_append(const paged_kv_pool_desc* desc, void* out,
                                              int32_t out_dtype, const void* q, const void* new_k,
                                              const void* new_v, const int32_t* slot_mapping,
                                              void* k_pool, void* v_pool,
                                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                                              const int32_t* context_lens, int32_t num_seqs,
                                              int32_t num_q_heads, int32_t max_context_len,
                                              float scale, int32_t partition_tokens, void* workspace,
                                              size_t workspace_bytes, void* stream);

/* paged_attention_decode for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, results and errors as paged_attention_decode (bit-identical outputs for
 * the same schedule), without the workspace: the partial results and merge counters
 * live in a static device array of the library, 64 MiB per device, held by every
 * device the library runs on until the process ends (1 MiB of it for counters, one
 * int32 per (sequence, head unit); 63 MiB for partial results).  A call that would need
 * more returns PAGED_KV_ERR_BUFFER_TOO_SMALL before launching anything.  It makes no
 * allocation of its own: the array's address is looked up once per device (first call
 * with that device current), its counters cleared there by a fill kernel on `stream`.
 * All calls on one device share the array and every call leaves the counters at zero,
 * so calls on one device must not overlap (two streams at once race on the array). */
paged_kv_status paged_attention_decode_static(const paged_kv_pool_desc* desc, void* out,
                                              int32_t out_dtype, const void* q, const void* k_pool,
                                              const void* v_pool, const int32_t* block_tables,
                                              int32_t max_blocks_per_seq,
                                              const int32_t* context_lens, int32_t num_seqs,
                                              int32_t num_q_heads, int32_t max_context_len,
                                              float scale, int32_t partition_tokens, void* stream);

/* The two halves of paged_attention_decode, exposed so each kernel can be timed on its
 * own.  With fixed partitions, paged_attention_partition writes `out` for sequences that
 * fit one partition and the per-partition (max, sum, weighted values) state of the
 * others into `workspace`, and paged_attention_reduce merges that state into `out`.
 * With the stream-K schedule the partition launch merges in-kernel and writes all of
 * `out`; paged_attention_reduce then only validates its arguments.
 * Arguments as for paged_attention_decode. */
paged_kv_status paged_attention_partition(const paged_kv_pool_desc* desc, void* out,
                                          int32_t out_dtype, const void* q, const void* k_pool,
                                          const void* v_pool, const int32_t* block_tables,
                                          int32_t max_blocks_per_seq, const int32_t* context_lens,
                                          int32_t num_seqs, int32_t num_q_heads,
                                          int32_t max_context_len, float scale,
                                          int32_t partition_tokens, void* workspace,
                                          size_t workspace_bytes, void* stream);
paged_kv_status paged_attention_reduce(const paged_kv_pool_desc* desc, void* out, int32_t out_dtype,
                                       const int32_t* context_lens, int32_t num_seqs,
                                       int32_t num_q_heads, int32_t max_context_len,
                                       int32_t partition_tokens, const void* workspace,
                                       size_t workspace_bytes, void* stream);

/* --------------------------------------------------- shared-prefix decode ---- */

/* Groups for paged_attention_decode_shared_prefix ([DS] §2.3: forked samples share the
 * prompt's blocks; [DS] §2.4: prefix-cache hits share cached blocks).  Walks the batch
 * in order and puts consecutive sequences in one group while all its members' tables
 * start with the same blocks for at least max(1, min_shared_tokens) tokens (and the
 * group has fewer than max_group members).  A group's shared length is its members'
 * common leading blocks times block_size, capped at the shortest member's length; a
 * group of one has shared length 0.
 *   seq_ids            host int32[n]: the batch, in the order the attention call uses
 *   group_start_out    host int32[n + 1]: members of group g are rows
 *                      group_start_out[g] .. group_start_out[g + 1] - 1 of the batch
 *   shared_tokens_out  host int32[n]: shared length of group g
 *   num_groups_out, max_shared_out: number of groups, longest shared length
 * Errors: INVALID_ARG (null pointers, n < 0, max_group < 1), NO_SUCH_SEQ. */
paged_kv_status paged_kv_shared_prefix_groups(const paged_kv_pool* pool, const int32_t* seq_ids,
                                              int32_t n, int32_t max_group,
                                              int32_t min_shared_tokens, int32_t* group_start_out,
                                              int32_t* shared_tokens_out, int32_t* num_groups_out,
                                              int32_t* max_shared_out);

/* Workspace bytes of paged_attention_decode_shared_prefix for this shape (0 if an
 * argument is invalid). */
size_t paged_attention_shared_prefix_workspace_bytes(const paged_kv_pool_desc* desc,
                                                     int32_t num_seqs, int32_t num_q_heads,
                                                     int32_t max_context_len, int32_t num_groups,
                                                     int32_t max_group, int32_t max_shared_tokens,
                                                     int32_t partition_tokens);

/* Paged decode attention for a batch whose sequences share prompt prefixes ([DS] §2.3
 * parallel sampling: the samples share the prompt's blocks by reference count; [DL]
 * concrete benefits, flexible sharing of the KV cache): the same result as
 * paged_attention_decode (within the attention tolerance; a different summation
 * order), but the shared tokens of each group are read from the pool once for all its
 * members.  The group's members times the query heads of a KV head form the columns of
 * the matrix products over each shared tile (at most 64: max_group x query heads per KV
 * head <= 64); each member's own tail is attended separately; a second launch merges,
 * per sequence and query head, the shared-part partitions with the tail partitions by
 * log-sum-exp.
 *   group_start    device int32[num_groups + 1]: non-decreasing, group_start[0] = 0,
 *                  group_start[num_groups] = num_seqs (as paged_kv_shared_prefix_groups
 *                  returns it)
 *   shared_tokens  device int32[num_groups]: tokens 0 .. shared_tokens[g] - 1 sit in the
 *                  same blocks in every member's table, and every member's context
 *                  holds at least that many tokens
 *   max_group, max_shared_tokens  host bounds on members per group and on shared_tokens
 *   partition_tokens  tokens per partition of the shared part and of each tail (a
 *                  multiple of 16; 0: chosen from the shape, the largest of 4096 (or the
 *                  longest context rounded up to 512), 2048, 1024 and 512 that leaves
 *                  about four workgroups per compute unit)
 *   workspace      device buffer of paged_attention_shared_prefix_workspace_bytes(...)
 *                  bytes (scratch; needs no zero-fill)
 * Other arguments as for paged_attention_decode.  A sequence for which the group
 * description does not hold (shared length above its length or above
 * max_shared_tokens, a table that differs from its group's first one over the shared
 * tokens, a group past the batch or larger than max_group) gets NaN outputs, as does one
 * with an invalid length; nothing outside the buffers is read.  Requires an fp16/bf16 pool with block_size 16 or 32, head_dim 64,
 * 128 or 256 and 2 to 16 query heads per KV head (UNSUPPORTED otherwise).  Results do
 * not depend on where blocks sit in the pool. */
paged_kv_status paged_attention_decode_shared_prefix(
    const paged_kv_pool_desc* desc, void* out, int32_t out_dtype, const void* q,
    const void* k_pool, const void* v_pool, const int32_t* block_tables,
    int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
    int32_t num_q_heads, int32_t max_context_len, float scale, const int32_t* group_start,
    const int32_t* shared_tokens, int32_t num_groups, int32_t max_group,
    int32_t max_shared_tokens, int32_t partition_tokens, void* workspace,
    size_t workspace_bytes, void* stream);

/* Causal multi-query attention over the pool: prefill, prefill in chunks, and the rest
 * of a prompt after a prefix-cache hit ([DS] §2.5: a request only counts how many of its
 * tokens are computed, so these are one operation; §2.6: it reads the blocks through
 * the table too; [DL] continuous batching section: the compute-heavy phase).  The last
 * n_s = q_start[s+1] - q_start[s] tokens of sequence s are queries; their K/V must
 * already be in the pool (reshape_and_cache), counted in context_lens[s].  Query i of
 * sequence s sits at position context_lens[s] - n_s + i and attends to keys 0 .. that
 * position.
 *   out           device [total][num_q_heads][head_dim], type out_dtype (desc->dtype or
 *                 PAGED_KV_F32); row q_start[s] + i is query i of sequence s
 *   q             device [total][num_q_heads][head_dim], type desc->dtype
 *   q_start       device int32[num_seqs + 1], non-decreasing, q_start[0] = 0 (rows of
 *                 out/q past q_start[num_seqs] are neither read nor written)
 *   block_tables, max_blocks_per_seq, context_lens: as for paged_attention_decode
 *   scale         score scale, > 0 (INVALID_ARG otherwise)
 *   max_q_len     host bound on every n_s (sizes the launch; 0 launches nothing)
 *   max_context_len  host bound on every context_lens[s], >= max_q_len
 * A sequence with n_s > context_lens[s] or context_lens[s] outside [1, max_context_len],
 * or whose table holds an id outside [0, num_blocks) below its length, gets NaN rows; a
 * sequence with n_s < 0 or n_s > max_q_len gets none written.  Requires an fp16/bf16
 * pool (UNSUPPORTED otherwise) with block_size 1, 16 or 32, head_dim 64, 128 or 256,
 * num_q_heads % num_kv_heads == 0 and at most 16 query heads per KV head; out, q and
 * the pools must be 16-byte aligned (INVALID_ARG otherwise).  Needs no workspace.
 * Results do not depend on where blocks sit in the pool. */
paged_kv_status paged_attention_prefill(const paged_kv_pool_desc* desc, void* out,
                                        int32_t out_dtype, const void* q, const int32_t* q_start,
                                        const void* k_pool, const void* v_pool,
                                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                                        const int32_t* context_lens, int32_t num_seqs,
                                        int32_t num_q_heads, int32_t max_q_len,
                                        int32_t max_context_len, float scale, void* stream);

/* ------------------------------------------------------------ measurement ---- */

/* A plain streaming read of `bytes` bytes at `buf` (device, 16-byte aligned, a multiple
 * of 16), with the access pattern of the attention kernels' K/V loads: 16-byte
 * nontemporal loads, 1 KiB contiguous per wave instruction, each wave streaming its own
 * contiguous run, two waves per SIMD.  Its rate is the measured read bandwidth that the
 * decode roofline is stated against beside the part's specified peak.  `sink` is a
 * device int32 that is written only in a case no real buffer reaches (it keeps the loads
 * alive).  Errors: INVALID_ARG. */
paged_kv_status paged_kv_read_bandwidth_probe(const void* buf, size_t bytes, void* sink,
                                              void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_KV_H */

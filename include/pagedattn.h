/*
 * pagedattn.h - C ABI of the MI355X (gfx950) paged decode attention library.
 *
 * The operation (devpress.csdn.net article on the vLLM architecture,
 * section 3 "PagedAttention kernel: from concept to CUDA"):
 *   part 1 gives the inputs: query[num_seqs, num_heads, head_size],
 *     block_tables[num_seqs, max_blocks_per_seq] and one pool per cache,
 *     k_cache/v_cache[num_physical_blocks, block_size, num_kv_heads, head_size];
 *   part 2 gives the flow: for each sequence take its block table, its actual
 *     length and the number of logical blocks, gather K/V from the physical
 *     blocks the table names, run standard attention of the query over them,
 *     write the output.
 * A block holds the K/V of 16 tokens (aiflowlearn.net vLLM course page,
 * section on cutting the KV cache into pages).
 *
 * Conventions for the device entry points (the host block manager pa_bm_*
 * at the end has its own):
 *  - All data pointers are DEVICE pointers owned by the caller; the library
 *    never allocates or frees, keeps no global state, and is re-entrant
 *    (paged_attention_decode_noalloc aside: it uses a device array of the
 *    library's own, see there).
 *  - Tensors are dense and row-major in the shapes given; q, caches and
 *    outputs share one element type (enum pa_dtype) except where an entry
 *    point says otherwise (fp8 pools).  Data pointers must be 16-byte
 *    aligned.
 *  - `stream` is a hipStream_t (NULL = the legacy default stream).  Calls only
 *    enqueue work on it; there is no host synchronisation.
 *  - Errors that the host can see (null pointer, unsupported size or type,
 *    bad partition size or flags, workspace too small, misalignment) are returned
 *    synchronously and nothing is launched.  A launch failure returns
 *    PA_ERR_HIP.  Device-side contract violations never fault: a sequence
 *    whose length is negative or exceeds max_blocks_per_seq * block_size, or
 *    whose first ceil(len / block_size) table entries are not all in
 *    [0, num_blocks), gets NaN in its output rows instead.
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = -1,  /* null pointer, negative size, bad shape relation, misalignment */
  PA_ERR_UNSUPPORTED = -2,  /* dtype / head_size / block_size / group size not built        */
  PA_ERR_WORKSPACE = -3,    /* split path without a large enough workspace                   */
  PA_ERR_HIP = -4,          /* the HIP runtime reported an error at launch                   */
  PA_ERR_NO_BLOCKS = -5,    /* block manager: not enough free blocks in the pool             */
  PA_ERR_CAPACITY = -6,     /* block manager: the sequence's table would exceed its maximum  */
  PA_ERR_SCRATCH = -7       /* paged_attention_decode_noalloc: the call needs more scratch
                               than PA_NOALLOC_SCRATCH_BYTES                                 */
} pa_status;

/* Element types.  PA_FP8_E4M3 (OCP 8-bit float, 1 sign, 4 exponent bits with
 * bias 7, 3 mantissa bits, no infinities, 0x7F/0xFF = NaN, largest finite
 * 448) is a pool type only: see paged_attention_decode_fp8,
 * reshape_and_cache_fp8 and copy_blocks. */
typedef enum { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2, PA_FP8_E4M3 = 3 } pa_dtype;

/* Flags of paged_attention_decode. */
enum {
  /* Physical blocks may be named by several sequences of the batch (shared
   * prefixes, copy-on-write): read K/V with the default cache policy so a
   * shared block stays cached for its other readers.  Without the flag K/V
   * are streamed with non-temporal loads (each block is read once per call). */
  PA_FLAG_SHARED_BLOCKS = 1
};

/* Human-readable name of a pa_status value (static string, never NULL). */
const char* pa_status_string(int status);

/*
 * Bytes of device workspace paged_attention_decode needs (an upper bound):
 *  partition_size > 0:
 *    256 + num_seqs * num_heads * ceil(max_seq_len / partition_size) * (head_size + 4) * 4
 *    (a 256-byte header holding a work-queue counter, then one fp32 partial
 *    record per partition: max, sum, 2 unused, output)
 *  partition_size == 0 (balanced split, bf16/fp16 KV):
 *    round_up(num_seqs * 16, 256) + 256 * num_heads * 2 * (head_size + 4) * 4
 *    (one 16-byte entry per sequence saying where its partial results are,
 *    then two partial records per range (the work is cut into 256 ranges)
 *    and query head; fp32 KV needs none).
 * Returns 0 for invalid sizes.  max_seq_len must be the value later passed to
 * paged_attention_decode, or max_blocks_per_seq * block_size if 0 is passed.
 */
size_t pa_decode_workspace_size(int num_seqs, int num_heads, int head_size,
                                int max_seq_len, int partition_size);

/*
 * Paged decode attention: one new query token per (sequence, head).
 *
 *   out[s, h, :] = sum_t softmax_t(scale * <query[s, h, :], K_t>) * V_t
 *
 * over the tokens t < seq_lens[s] of sequence s, where token t of KV head
 * g = h / (num_heads / num_kv_heads) is row
 *   k_cache[block_tables[s, t / block_size], t % block_size, g, :]
 * (and likewise for v_cache).  seq_lens[s] == 0 gives a zero output row.
 * Accumulation is fp32; for bf16/fp16 KV the softmax weights enter the
 * weighted sum of V rounded to the KV type (the sum of weights stays fp32).
 *
 *  out            [num_seqs, num_heads, head_size], written (dtype)
 *  query          [num_seqs, num_heads, head_size] (dtype)
 *  k_cache        [num_blocks, block_size, num_kv_heads, head_size] (dtype)
 *  v_cache        same shape and dtype as k_cache
 *  block_tables   int32 [num_seqs, max_blocks_per_seq]; only the first
 *                 ceil(seq_lens[s] / block_size) entries of row s are read
 *  seq_lens       int32 [num_seqs]
 *  head_size      64 or 128;  block_size: 16
 *  num_heads / num_kv_heads must be 1, 2, 4 or 8 (grouped-query attention)
 *  max_seq_len    upper bound on seq_lens (sizes the split grid and the
 *                 workspace); 0 means max_blocks_per_seq * block_size
 *  scale          softmax scale (usually 1/sqrt(head_size))
 *  dtype          pa_dtype of query, caches and out
 *  partition_size 0: the library splits the work.  For bf16/fp16 the whole
 *                 batch's blocks are cut into equal shares over the GPU
 *                 (sequences that straddle a share are merged by a second
 *                 kernel); needs a workspace; at most 16383 sequences.  For
 *                 fp32 one pass per (sequence, kv head), no workspace; so
 *                 too for bf16/fp16 with num_heads == num_kv_heads and at
 *                 least 1024 (sequence, kv head) pairs, longest sequence
 *                 first (the workspace is still required).  With
 *                 num_heads == num_kv_heads otherwise (fp8 pools
 *                 (paged_attention_decode_fp8) always, bf16/fp16 with fewer
 *                 pairs) the library picks a partition size (256 tokens, or
 *                 more where the records would not fit this workspace) and
 *                 runs the split below if that makes at least 1024
 *                 (sequence, partition, kv head) items; a length above
 *                 max_seq_len then breaks the contract (its row is NaN once
 *                 it runs past the partitions).
 *                 > 0: split context into partitions of this many tokens (a
 *                 multiple of block_size); a second kernel merges partitions
 *                 with log-sum-exp weights.  Needs a workspace.
 *  flags          0 or PA_FLAG_SHARED_BLOCKS
 *  workspace      device buffer of >= pa_decode_workspace_size(...) bytes,
 *                 256-byte aligned, NULL when none is needed.  Its contents
 *                 are scratch; calls that overlap in time need their own.
 */
int paged_attention_decode(void* out, const void* query, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, const int32_t* seq_lens,
                           int num_seqs, int num_heads, int num_kv_heads, int head_size,
                           int block_size, int max_blocks_per_seq, int num_blocks,
                           int max_seq_len, float scale, int dtype, int partition_size,
                           unsigned flags, void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_attention_decode without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  It computes exactly what
 * paged_attention_decode computes (same kernels, bit-identical results) and
 * takes the same arguments minus workspace and workspace_bytes.
 *
 * In place of the workspace it uses a device array of the library's own,
 * PA_NOALLOC_SCRATCH_BYTES (32 MiB) per device, which each device the
 * library runs on holds until the process ends; the call allocates nothing.
 * Its device address is looked up on the first call on each device (with
 * that device current).  Nothing in it has to start at zero: every call
 * writes what it reads.  All calls on one device share the array, so calls
 * that overlap in time on one device (two streams, or a launch still running
 * when the next is enqueued on another stream) race and corrupt each other's
 * results; calls in order on one stream are safe.
 *
 *  stream   a stream of the current device (or NULL); PA_ERR_INVALID_ARG if
 *           it belongs to another device.
 * Returns PA_ERR_SCRATCH, launching nothing, when the call would need more
 * than PA_NOALLOC_SCRATCH_BYTES (pa_decode_workspace_size gives the need),
 * The balanced split always fits when num_heads * (head_size + 4) <= 16256
 * (up to 64 heads of 128, any num_seqs it takes); the fixed split when
 * num_seqs * num_heads * partitions * (head_size + 4) * 4 <= 32 MiB.
 */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int paged_attention_decode_noalloc(void* out, const void* query, const void* k_cache, const void* v_cache,
                                   const int32_t* block_tables, const int32_t* seq_lens,
                                   int num_seqs, int num_heads, int num_kv_heads, int head_size,
                                   int block_size, int max_blocks_per_seq, int num_blocks,
                                   int max_seq_len, float scale, int dtype, int partition_size,
                                   unsigned flags, void* stream);

/*
 * Several new tokens per sequence, attending causally over the paged cache
 * (chunked prefill and speculative verification; yangyitao.com vLLM book
 * preface, overview list: prefill, decode and speculative decoding all give a
 * request N new tokens; is96.com essay: chunked prefill processes a long
 * prompt in pieces).
 *
 * Sequence s brings n_s = query_start[s+1] - query_start[s] query rows,
 * query[query_start[s] + i] for i < n_s: its last n_s tokens, whose K/V are
 * already in the pools (reshape_and_cache first).  Row i sits at position
 * p = seq_lens[s] - n_s + i and attends to tokens 0 .. p:
 *
 *   out[query_start[s] + i, h, :] = sum_{t <= p} softmax_t(scale <q, K_t>) V_t
 *
 * with K_t, V_t read through the block table as in paged_attention_decode
 * (kv head h / (num_heads / num_kv_heads)).  n_s == 1 is decode.
 *
 *  out, query     [num_query_tokens, num_heads, head_size] (dtype: PA_F16 or
 *                 PA_BF16; PA_F32 gives PA_ERR_UNSUPPORTED)
 *  query_start    int32 [num_seqs + 1], non-decreasing, query_start[0] = 0,
 *                 query_start[num_seqs] = num_query_tokens
 *  max_query_len  >= every n_s (sizes the grid and picks the path); 0 means
 *                 num_query_tokens
 *  workspace      device buffer of >= pa_prefill_workspace_size(...) bytes,
 *                 256-byte aligned (NULL when that size is 0); scratch, as for
 *                 paged_attention_decode
 *  other arguments as in paged_attention_decode.
 * When max_query_len * (num_heads / num_kv_heads) <= 32 (speculative
 * verification: each kv head's query rows fit two 16-row tiles) and num_seqs
 * <= 16383, the batch's blocks are split evenly over the GPU as in decode and
 * a second kernel merges partial results (needs the workspace; with two
 * tiles the K/V loads use the default cache policy whatever flags says,
 * since two waves read each line); otherwise two tiles per wave and 16 per
 * workgroup sharing K/V through LDS (from 32 sequences on, run longest
 * sequence first, which needs the workspace), or, for one tile (more than
 * 16383 sequences), one wave per tile.
 * Rows of a sequence with n_s > seq_lens[s], a length past its table row or a
 * block id outside the pool are NaN.  Rows beyond max_query_len are not
 * written.
 */
int paged_attention_prefill(void* out, const void* query, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* seq_lens, const int32_t* query_start,
                            int num_seqs, int num_query_tokens, int num_heads, int num_kv_heads, int head_size,
                            int block_size, int max_blocks_per_seq, int num_blocks, int max_query_len,
                            float scale, int dtype, unsigned flags, void* workspace, size_t workspace_bytes,
                            void* stream);

/* Workspace bytes paged_attention_prefill(_fp8) needs with these sizes (0:
 * none):  round_up(num_seqs * 16, 256) + 256 * num_kv_heads * 2 * 16 * tiles *
 * (head_size + 4) * 4 on the split path, tiles = ceil(max_query_len *
 * (num_heads / num_kv_heads) / 16); round_up(num_seqs * 4, 256) (the
 * longest-first order) on the LDS path with at least 32 sequences; else 0.
 * 0 for invalid sizes. */
size_t pa_prefill_workspace_size(int num_seqs, int num_query_tokens, int num_heads, int num_kv_heads,
                                 int head_size, int max_query_len);

/* paged_attention_prefill over fp8 (e4m3) pools with one scale per pool
 * (see paged_attention_decode_fp8). */
int paged_attention_prefill_fp8(void* out, const void* query, const void* k_cache, const void* v_cache,
                                const int32_t* block_tables, const int32_t* seq_lens, const int32_t* query_start,
                                int num_seqs, int num_query_tokens, int num_heads, int num_kv_heads,
                                int head_size, int block_size, int max_blocks_per_seq, int num_blocks,
                                int max_query_len, float scale, float k_scale, float v_scale, int dtype,
                                unsigned flags, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Scatter new tokens' K/V rows into their cache slots (csdn article,
 * section 4 point 3: gather-scatter in place of contiguous access; section 2
 * part 4: a new token joins its sequence's blocks).
 *
 *   for i < num_tokens with 0 <= slot_mapping[i] < num_blocks * block_size:
 *     k_cache[slot / block_size, slot % block_size, :, :] = key[i, :, :]
 *     v_cache[slot / block_size, slot % block_size, :, :] = value[i, :, :]
 *
 * Bytes are copied unchanged (bit-exact).  Negative slots mean "no write";
 * slots at or past num_blocks * block_size are skipped too.  Two tokens must
 * not share a slot (which write wins is then unspecified).
 *
 *  key, value       [num_tokens, num_kv_heads, head_size] (dtype)
 *  k_cache, v_cache [num_blocks, block_size, num_kv_heads, head_size], updated in place
 *  slot_mapping     int32 [num_tokens]
 */
int reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                      const int32_t* slot_mapping, int num_tokens, int num_kv_heads,
                      int head_size, int block_size, int num_blocks, int dtype, void* stream);

/*
 * FP8 KV cache.  The pages name quantisation as the way to fit more in less
 * memory (aiflowlearn.net vLLM course page, quantisation section: several
 * formats, none spelled out; yangyitao.com vLLM book preface, contents:
 * quantisation trades precision for speed).  Here the pools hold OCP fp8
 * e4m3 codes with one scale per pool: a stored code c means e4m3(c) * k_scale
 * in the K pool and e4m3(c) * v_scale in the V pool.
 *
 * paged_attention_decode_fp8 computes exactly what paged_attention_decode
 * computes, over those values: query and out are dtype (PA_F16 or PA_BF16;
 * PA_F32 gives PA_ERR_UNSUPPORTED), the pools are [num_blocks, block_size,
 * num_kv_heads, head_size] bytes.  Codes are widened exactly to dtype in
 * registers; k_scale enters the score scale and v_scale the final
 * normalisation.  k_scale and v_scale must be positive and finite.  Every
 * other argument, the workspace (same size) and the error behaviour are those
 * of paged_attention_decode.
 */
int paged_attention_decode_fp8(void* out, const void* query, const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, const int32_t* seq_lens,
                               int num_seqs, int num_heads, int num_kv_heads, int head_size,
                               int block_size, int max_blocks_per_seq, int num_blocks,
                               int max_seq_len, float scale, float k_scale, float v_scale, int dtype,
                               int partition_size, unsigned flags, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * Scatter with quantisation into fp8 pools: as reshape_and_cache, but each
 * element x of key (value) is stored as the e4m3 code
 *
 *   RNE_e4m3(saturate(x * inv)),  inv = (float)(1.0 / k_scale)  (1.0 / v_scale)
 *
 * where x * inv is an fp32 product, saturate clamps to [-448, 448] and keeps
 * NaN, and RNE_e4m3 rounds to the nearest e4m3 value, ties to the even code.
 * key/value are dtype (PA_F32, PA_F16 or PA_BF16); num_kv_heads * head_size
 * must be a multiple of 16.
 */
int reshape_and_cache_fp8(const void* key, const void* value, void* k_cache, void* v_cache,
                          const int32_t* slot_mapping, int num_tokens, int num_kv_heads, int head_size,
                          int block_size, int num_blocks, int dtype, float k_scale, float v_scale,
                          void* stream);

/*
 * Copy whole blocks inside both pools (the copies that copy-on-write queues,
 * see pa_bm_take_copies):
 *
 *   for i < num_pairs with src[i], dst[i] in [0, num_blocks):
 *     k_cache[dst[i]] = k_cache[src[i]];  v_cache[dst[i]] = v_cache[src[i]]
 *
 * (one block = block_size * num_kv_heads * head_size elements, copied
 * bit-exactly).  Pairs naming a block outside the pool are skipped.  The pairs
 * run in parallel: destinations must be distinct and no block may be both a
 * source and a destination in one call (true of the copies one batch of
 * appends queues when no fork happens in between).
 *
 *  k_cache, v_cache [num_blocks, block_size, num_kv_heads, head_size] (dtype, any
 *                   pa_dtype including PA_FP8_E4M3), device
 *  src, dst         int32 [num_pairs], device
 */
int copy_blocks(void* k_cache, void* v_cache, const int32_t* src, const int32_t* dst, int num_pairs,
                int num_kv_heads, int head_size, int block_size, int num_blocks, int dtype, void* stream);

/*
 * ---- Block manager (host memory, host calls; no GPU work) ----
 *
 * The paged KV cache's bookkeeping (devpress.csdn.net article on the vLLM
 * architecture, section 1: the KV-cache manager keeps one global pool of free
 * fixed-size blocks, answers a sequence's requests for blocks, keeps its
 * logical -> physical block table, and uses reference counts for
 * copy-on-write so blocks can be shared, e.g. by beam search; section 2 parts
 * 2 and 4: blocks are taken when a request is scheduled and again when a new
 * token needs a new block).  Freed blocks are handed out again first
 * (yangyitao.com vLLM book preface, "from OS to GPU" block-pool figure): the
 * pool is a stack; a new pool hands out block 0, then 1, 2, ...; a freed
 * sequence's blocks are pushed in table order.
 *
 * Token t of sequence s lives in slot table[t / block_size] * block_size +
 * t % block_size: the slot_mapping of reshape_and_cache, and (with the tables
 * from pa_bm_block_tables) the layout paged_attention_decode reads.
 *
 * Sequences are ids in [0, max_seqs).  Every call either succeeds or returns
 * an error and changes nothing.  A manager is not thread-safe; it owns only
 * host memory, released by pa_bm_destroy.  Slot arrays are host memory owned
 * by the caller.
 *
 * Copy-on-write: appending to a sequence whose last block is partly filled and
 * shared (reference count > 1) first gives it a fresh block in its place and
 * queues the pair (shared, fresh); the caller takes the queue
 * (pa_bm_take_copies), runs copy_blocks on it, and only then writes the new
 * tokens (reshape_and_cache).  A full shared block is never written, so
 * appending past it only takes a new block.  A queued copy whose destination
 * is freed before it is taken is dropped.
 */
typedef struct pa_block_manager pa_block_manager;

/* New manager with num_blocks free blocks; *out receives it (NULL on error).
 * PA_ERR_UNSUPPORTED if num_blocks * block_size does not fit in int32. */
int pa_bm_create(int num_blocks, int block_size, int max_seqs, int max_blocks_per_seq,
                 pa_block_manager** out);
void pa_bm_destroy(pa_block_manager* bm);

/* New sequence `seq` (a free id) holding num_tokens tokens: ceil(num_tokens /
 * block_size) blocks from the pool.  slots (NULL or num_tokens ints) receives
 * each token's slot.  PA_ERR_NO_BLOCKS / PA_ERR_CAPACITY when they do not fit. */
int pa_bm_allocate(pa_block_manager* bm, int seq, int num_tokens, int32_t* slots);

/* num_tokens more tokens at the end of `seq`; slots (NULL or num_tokens ints)
 * receives their slots.  Takes new blocks as the last one fills, after a
 * copy-on-write of a shared, partly filled last block (see above). */
int pa_bm_append_slots(pa_block_manager* bm, int seq, int num_tokens, int32_t* slots);

/* One decode step of a batch: one more token at the end of each seqs[i]
 * (distinct ids, in order), exactly as num_seqs calls of pa_bm_append_slots
 * with one token each; slots (NULL or num_seqs ints) receives the slots.  The
 * whole batch is checked first, so either every sequence grows or nothing
 * changes: PA_ERR_INVALID_ARG for an id that holds no sequence or appears
 * twice, else PA_ERR_CAPACITY if a table would exceed its maximum, else
 * PA_ERR_NO_BLOCKS if the pool cannot cover the new blocks and copies. */
int pa_bm_append_batch(pa_block_manager* bm, const int32_t* seqs, int num_seqs, int32_t* slots);

/* New sequence `child` (a free id) sharing every block of `parent`. */
int pa_bm_fork(pa_block_manager* bm, int parent, int child);

/* Release `seq`: reference counts drop; blocks that reach 0 return to the pool. */
int pa_bm_free(pa_block_manager* bm, int seq);

/* Free blocks in the pool (>= 0), or an error. */
int pa_bm_num_free_blocks(const pa_block_manager* bm);

/* The pool, bottom first (the next block handed out is the last one): returns
 * the count; PA_ERR_INVALID_ARG if capacity is too small. */
int pa_bm_free_list(const pa_block_manager* bm, int32_t* blocks, int capacity);

/* Reference count of a block, or PA_ERR_INVALID_ARG for an id outside the pool. */
int pa_bm_ref_count(const pa_block_manager* bm, int block);

/* Tokens held by `seq`, -1 if the id holds no sequence. */
int pa_bm_seq_len(const pa_block_manager* bm, int seq);

/* The batch seqs[0 .. num_seqs): row i of block_tables ([num_seqs,
 * max_blocks_per_seq], host) gets seqs[i]'s table padded with -1, and
 * seq_lens[i] its length: the block_tables / seq_lens of
 * paged_attention_decode after a copy to the device. */
int pa_bm_block_tables(const pa_block_manager* bm, const int32_t* seqs, int num_seqs,
                       int32_t* block_tables, int32_t* seq_lens);

/* Number of queued copies. */
int pa_bm_num_copies(const pa_block_manager* bm);

/* Move the queued copies (in the order they were queued) into src/dst (host,
 * capacity entries each) and clear the queue; returns the count.
 * PA_ERR_INVALID_ARG (nothing taken) if capacity is too small. */
int pa_bm_take_copies(pa_block_manager* bm, int32_t* src, int32_t* dst, int capacity);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */

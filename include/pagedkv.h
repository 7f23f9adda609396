/*
 * pagedkv.h - C ABI of libpagedkv: paged KV-cache decode attention for AMD MI355X (gfx950).
 *
 * The method is PagedAttention as described in three pages on continuous batching:
 *   [Serving] "Production Serving: Continuous Batching and PagedAttention" (llm-under-the-hood,
 *             project 17), The Concept; The Build, Step 4 (paged KV cache), Step 6 (attention
 *             over paged storage), Step 8 (prefix caching).
 *   [Chapter] "Continuous batching and PagedAttention" (how-ai-works, chapter 7),
 *             "How the scheduler works", "PagedAttention: KV cache memory".
 *   [Notes]   "Continuous batching and PagedAttention: serving many users from one GPU"
 *             (trefon notes), "Fragmentation: PagedAttention", "Prefill gets in the way".
 *
 * Every cached token of a sequence lives in a fixed 16-token physical block; a per-sequence block
 * table maps logical block j to a physical block id; each continuous-batching step appends the
 * step's K/V into slots and then attends over all cached tokens.
 *
 * Conventions shared by every call
 *   - Return value: PKV_OK (0) or a negative status.  pkv_last_error() returns a thread-local
 *     message for the last non-zero status of the calling thread.
 *   - Device calls take device pointers owned by the caller, enqueue work on `stream` (a
 *     hipStream_t; NULL = the default stream) and return without synchronising.  The library
 *     never allocates or frees device memory.  Argument checks happen on the host before any
 *     launch; a failed check launches nothing.  Launch failures return PKV_EHIP.
 *   - Device array CONTENTS (block ids, lengths, slots) are preconditions that the host cannot
 *     check without a synchronisation: block ids must lie in [0, num_blocks), 1 <= context length
 *     <= max_context_len, and the slots of one append call must be distinct.
 *   - Element types: PKV_F32, PKV_F16, PKV_BF16.  Queries, keys, values and caches of one call
 *     share one element type (`dtype`).
 *   - Cache layout (one layer; K and V are separate tensors, both indexed by physical block id):
 *         k_cache [num_blocks][num_kv_heads][K tile]                 see below
 *         v_cache [num_blocks][num_kv_heads][V tile]                 see below
 *     Slot s means block s / block_size, offset s % block_size.  One (block, head) tile of either
 *     tensor is contiguous (4 KiB at 16 x 128 bf16), and a whole block is one contiguous span.
 *     V tile: [block_size / 8][head_dim][8], i.e. element d of token t is at tile offset
 *     ((t / 8) * head_dim + d) * 8 + t % 8: eight consecutive tokens of one dimension are one
 *     16-byte operand of the P.V product, and the eight tokens of a half block own whole cache
 *     lines.
 *     K tile: the 16 x head_dim elements of one (block, head) are stored as 16-byte chunks
 *     (E = 16 / element size elements each, so head_dim * element size must be a multiple of 64
 *     bytes).  With token t = 8*hi + 4*set + low and chunk c = 4*cq + cr of the token's head
 *     vector, the chunks are stored in the nested order [cq][set][cr][hi][low], i.e. element d of
 *     token t is at tile offset (((cq*2 + set)*4 + cr)*8 + hi*4 + low)*E + d % E with c = d / E.
 *     This is the matrix-core operand order of the decode and prefill kernels: one 32-dimension
 *     k-step of eight tokens of a block is one contiguous 512-byte run.
 *     Neither tile is a [16][head_dim] array: callers treat a tile as opaque bytes (the Python
 *     binding's cache tensors are [num_blocks][num_kv_heads][16 * head_dim]) and write it only
 *     through paged_cache_append and the fused appends.
 *   - Grouped-query attention: query head h reads KV head h / (num_q_heads / num_kv_heads).
 *   - Supported kernel shapes: block_size 16, head_dim 64 or 128, num_q_heads / num_kv_heads in
 *     {1, 2, 4, 8}.  Other values return PKV_EUNSUPPORTED (paged_cache_append and
 *     paged_cache_copy_blocks accept any head_dim whose row is a multiple of 64 bytes).
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_OK 0
#define PKV_EINVAL (-1)       /* bad argument (null pointer, inconsistent sizes, unknown sequence) */
#define PKV_ENOMEM (-2)       /* the block pool cannot cover an allocation ([Serving] Step 4's out-of-pages error) */
#define PKV_EUNSUPPORTED (-3) /* shape or type the kernels do not implement */
#define PKV_EHIP (-4)         /* a HIP runtime call or kernel launch failed */

#define PKV_F32 0
#define PKV_F16 1
#define PKV_BF16 2

/* partition_size value: a batch-adaptive single pass (not batch invariant; see paged_attention_decode). */
#define PKV_SINGLE_PASS_ADAPTIVE (-1)

typedef void* pkv_stream_t; /* hipStream_t */

/* Thread-local message describing the last non-zero status returned to this thread. */
const char* pkv_last_error(void);

/* Library version, as major * 10000 + minor * 100 + patch. */
int32_t pkv_version(void);

/* ============================== device operations ============================== */

/*
 * paged_cache_append - scatter one call's K/V tokens into their slots.
 * [Serving] Step 4: token `pos` of a sequence is written at (page, pos % block_size) of the
 * page its page table names.  The slot of every token is computed on the host
 * (pkv_seq_append / pkv_build_slot_mapping); this call only moves bytes.
 *
 *   k_cache, v_cache  device, layout above; written at the given slots only.
 *   key, value        device, token t at key + t * key_stride elements, laid out [num_kv_heads][head_dim]
 *                     (a stride of 0 means num_kv_heads * head_dim, i.e. contiguous [T][Hkv][D]).
 *   slot_mapping      device int32 [T]; slot = block * block_size + offset; -1 skips the token.
 *   T                 tokens in this call (0 is a no-op).
 * Bit-exact copy; no arithmetic.  Slots must be distinct and < num_blocks * block_size.
 */
int paged_cache_append(void* k_cache, void* v_cache, const void* key, const void* value,
                       int64_t key_stride, int64_t value_stride, const int32_t* slot_mapping,
                       int32_t T, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                       int32_t num_blocks, int32_t dtype, pkv_stream_t stream);

/*
 * paged_cache_copy_blocks - whole-block copy of K and V for copy-on-write.
 * [Chapter] "PagedAttention: KV cache memory" and [Notes] "Fragmentation: PagedAttention":
 * sequences share physical blocks until they diverge; the block a sequence is about to write
 * while others still hold it is first copied (pkv_seq_append reports the pair).
 *
 *   src_dst   device int32 [n][2] = (source block, destination block) pairs, applied as one
 *             batch: no destination may be the source of another pair in the same call.
 * Copies every head and every slot of the block (stale tail slots included).  Bit-exact.
 */
int paged_cache_copy_blocks(void* k_cache, void* v_cache, const int32_t* src_dst, int32_t n,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            int32_t num_blocks, int32_t dtype, pkv_stream_t stream);

/*
 * paged_check_inputs - count the device-array values outside the kernels' contract.
 * [Serving] Step 4 (a sequence's pages in order; token pos at page pos // block_size, offset
 * pos % block_size) and Step 6 (attention over the stored tokens only).  The kernels clamp such
 * values (a wrong number, never an out-of-bounds access); this call reports them, on `stream`,
 * without synchronising.  It reads only inside the arrays it is given.
 *
 *   block_tables, context_lens  device int32 [B][max_blocks_per_seq] and [B], as passed to
 *                  paged_attention_decode (may be NULL when B is 0)
 *   slot_mapping   device int32 [T], as passed to paged_cache_append (may be NULL when T is 0)
 *   counts         device int32 [4], written (not accumulated):
 *                    [0] sequences whose length is outside [1, max_context_len] or longer than
 *                        max_blocks_per_seq * block_size,
 *                    [1] block-table entries among the first ceil(length / block_size) of a row
 *                        (at most the row) that are outside [0, num_blocks),
 *                    [2] the smallest sequence index counted in [0] or [1], 2147483647 when none,
 *                    [3] slots that are neither -1 nor in [0, num_blocks * block_size).
 * Not checked: repeated slots within one call, or a block listed twice.  PKV_EINVAL for negative
 * sizes, num_blocks or block_size <= 0, or a NULL pointer that a non-zero size needs.
 */
int paged_check_inputs(const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                       int32_t max_blocks_per_seq, int32_t max_context_len, const int32_t* slot_mapping, int32_t T,
                       int32_t num_blocks, int32_t block_size, int32_t* counts, pkv_stream_t stream);

/*
 * paged_probe_stream_read - a measuring aid, not part of the attention path: reads `bytes` of
 * device memory once with 16-byte nontemporal loads (the decode kernel's load form) over a
 * grid-stride walk, and writes nothing but (never, in practice) one word to `sink`.  Timing it
 * gives the HBM read bandwidth a plain streaming kernel achieves, the yardstick beside the 8 TB/s
 * nameplate for the bandwidth-bound decode ([Notes] "Continuous batching and PagedAttention:
 * serving many users from one GPU", "Why batching is almost free": every sequence's attention
 * reads its own KV cache, so decode time is set by bytes read).
 *   buf        device, 16-byte aligned; bytes a multiple of 16.
 *   sink       device uint32 (one word, caller-owned).
 *   workgroups grid size in [1, 65536] (256 threads each).
 * Enqueued on `stream`, no synchronisation.  PKV_EINVAL on a NULL pointer, misalignment or bad size.
 */
int paged_probe_stream_read(const void* buf, size_t bytes, uint32_t* sink, int32_t workgroups, pkv_stream_t stream);

/*
 * paged_attention_decode_workspace_bytes - device workspace paged_attention_decode needs.
 * 0 when partition_size is 0 or -1 (single pass).  Otherwise room for one (max, sum, unnormalised
 * output) partial per (sequence, query head, partition).
 */
size_t paged_attention_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                              int32_t max_context_len, int32_t partition_size);

/*
 * paged_attention_decode - one decode step of attention over the paged cache.
 * [Serving] Step 6: for every query head, score every cached token of its sequence (query . key
 * times `scale`), softmax the scores, and sum the values with those weights.  Only the first
 * context_lens[b] tokens take part; the unused tail of the last block is never read.
 *
 *   out            device [B][num_q_heads][head_dim] of out_dtype (PKV_F32 or `dtype`).
 *   query          device [B][num_q_heads][head_dim] of `dtype`.
 *   k_cache/v_cache device, layout above.
 *   block_tables   device int32 [B][max_blocks_per_seq]; row b lists sequence b's physical blocks
 *                  in logical order; entries past ceil(context_lens[b] / block_size) are not read.
 *   context_lens   device int32 [B]; tokens of sequence b, counting this step's appended token.
 *                  A sequence with no token (0, or a negative value) has nothing to attend to:
 *                  its rows of `out` are not written, and the other rows do not change.
 *   max_context_len host-known upper bound of context_lens (sizes the grid without a sync);
 *                  must not exceed max_blocks_per_seq * block_size.
 *   scale          score multiplier (1 / sqrt(head_dim) in the usual case).
 *   partition_size 0: one pass per (sequence, KV head).  Otherwise a multiple of block_size:
 *                  the context is cut into fixed partitions of that many tokens, each processed
 *                  independently, and the partial softmaxes are merged exactly (log-sum-exp).
 *                  At most 65535 partitions per sequence (PKV_EUNSUPPORTED beyond).
 *                  PKV_SINGLE_PASS_ADAPTIVE (-1): one pass whose split of the work inside a
 *                  workgroup follows the batch's max_context_len (fewer waves when it is at most
 *                  512), faster on batches of short contexts but not batch invariant.
 *                  Batch invariance (every value except -1): for a fixed partition_size, dtype,
 *                  out_dtype and head shape, a sequence's output bits depend only on its own
 *                  query, cached K/V and length - not on the other sequences, their number or
 *                  order, max_context_len, max_blocks_per_seq, host_context_lens, or whether the
 *                  step's token comes through the fused append.  Partition boundaries are token
 *                  positions and the waves per workgroup depend on partition_size alone.
 *                  [Chapter] "Continuous batching and PagedAttention", "Follow-up questions":
 *                  a reduction order that moves with the batch size is what makes outputs at
 *                  temperature 0 nondeterministic; batch-invariant kernels are the fix.
 *   workspace      device scratch of at least paged_attention_decode_workspace_bytes(...) bytes
 *                  (may be NULL when that is 0); contents on entry do not matter.
 *   host_context_lens  NULL, or a host copy of context_lens (B <= 512 entries): used only to
 *                  schedule the work, which shortens the launch's tail: sequences are handed out
 *                  by the size of their last partition (the whole context for a single pass),
 *                  largest first, and each sequence's partitions are rotated over the grid's
 *                  partition slices so that its last (ragged) one is dispatched in the final
 *                  slice.  The output does not depend on it, even when it disagrees with
 *                  context_lens (every partition's arithmetic is the same wherever it runs, and
 *                  the rotation covers every partition exactly once).
 * Accumulation is fp32 whatever the input type.
 */
int paged_attention_decode(void* out, int32_t out_dtype, const void* query, const void* k_cache,
                           const void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                           int32_t B, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                           int32_t max_context_len, float scale, int32_t partition_size,
                           void* workspace, size_t workspace_bytes, int32_t dtype,
                           const int32_t* host_context_lens, pkv_stream_t stream);

/*
 * paged_attention_decode_grouped - paged_attention_decode for batches in which sequences share
 * cached blocks.  [Chapter] "PagedAttention: KV cache memory": several samples of one answer, or
 * conversations with a common prefix, point at the same physical blocks (pkv_seq_fork,
 * pkv_prefix_lookup).  Sequences group_size * k .. group_size * k + group_size - 1 run in one
 * workgroup per KV head (and partition), their query heads side by side in the matrix columns; a
 * 32-token step whose two blocks are the same in every member's table is read from memory once
 * for the whole group, a step whose blocks differ is run once per member.  Order the batch so that
 * sequences sharing a prefix are adjacent; any batch is correct, sharing only saves reads.
 *   group_size  1 (exactly paged_attention_decode), or a size with group_size * (num_q_heads /
 *               num_kv_heads) equal to 8 or 16 (PKV_EUNSUPPORTED otherwise; bf16 / fp16 only).
 *   Other arguments as paged_attention_decode (no host_context_lens: groups run in batch order).
 * Output: bit for bit that of paged_attention_decode with the same partition_size, so the batch
 * invariance stated there holds here too, across group sizes as well.  K/V values must be finite
 * (a member's zero weights meet the other members' values in the shared products).
 */
int paged_attention_decode_grouped(void* out, int32_t out_dtype, const void* query, const void* k_cache,
                                   const void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                                   int32_t B, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                                   int32_t max_context_len, float scale, int32_t partition_size, void* workspace,
                                   size_t workspace_bytes, int32_t dtype, int32_t group_size, pkv_stream_t stream);

/*
 * paged_attention_decode_noalloc - paged_attention_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments without workspace / workspace_bytes, the same kernels and results, bit for bit.
 * The split-K partials live in a static device array of the library, PKV_NOALLOC_SCRATCH_BYTES
 * per GPU, held by each GPU the call runs on until the process ends; its address on a device is
 * looked up once, on the first call with that device current (the stream must belong to the
 * current device).  The call allocates nothing, then or later.
 *   - PKV_EINVAL, before anything else, when the partials need more than
 *     PKV_NOALLOC_SCRATCH_BYTES (paged_attention_decode_workspace_bytes(...) > the limit); a
 *     single pass (partition_size 0 or -1) needs none.
 *   - Every call on one GPU shares that GPU's array, and a call's partials are written and read
 *     by its own two launches: calls that overlap on one GPU (concurrent streams, or host threads)
 *     race.  Serialise them.  Nothing in the array needs an initial value.
 */
#define PKV_NOALLOC_SCRATCH_BYTES (16 * 1024 * 1024)
int paged_attention_decode_noalloc(void* out, int32_t out_dtype, const void* query, const void* k_cache,
                                   const void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                                   int32_t B, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                                   int32_t max_context_len, float scale, int32_t partition_size, int32_t dtype,
                                   const int32_t* host_context_lens, pkv_stream_t stream);

/*
 * paged_attention_decode_partitions / paged_attention_decode_reduce - the two launches of
 * paged_attention_decode when partition_size > 0, exposed separately (same arguments) so that a
 * caller can time or overlap them.  _partitions writes out[b] directly for every sequence that
 * fits in one partition and writes partials to the workspace for the others; _reduce merges the
 * partials of those others.  Calling _partitions then _reduce on one stream equals
 * paged_attention_decode.
 */
int paged_attention_decode_partitions(void* out, int32_t out_dtype, const void* query, const void* k_cache,
                                      const void* v_cache, const int32_t* block_tables,
                                      const int32_t* context_lens, int32_t B, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                      int32_t max_blocks_per_seq, int32_t num_blocks, int32_t max_context_len,
                                      float scale, int32_t partition_size, void* workspace,
                                      size_t workspace_bytes, int32_t dtype,
                                      const int32_t* host_context_lens, pkv_stream_t stream);
int paged_attention_decode_reduce(void* out, int32_t out_dtype, const int32_t* context_lens, int32_t B,
                                  int32_t num_q_heads, int32_t head_dim, int32_t max_context_len,
                                  int32_t partition_size, const void* workspace, size_t workspace_bytes,
                                  pkv_stream_t stream);

/*
 * paged_attention_decode_append - one decode step with the step's cache append fused in.
 * [Serving] Steps 4 and 6 in one launch: every sequence's newest token (position
 * context_lens[b] - 1) is written into its slot, block block_tables[b][(L - 1) / block_size],
 * offset (L - 1) % block_size (the slot pkv_seq_append / pkv_seqs_append reserved for it), and
 * attention over all context_lens[b] tokens uses that token's K/V straight from new_key /
 * new_value.  Same result, bit for bit, as paged_cache_append of those tokens followed by
 * paged_attention_decode; one launch fewer.
 *
 *   new_key, new_value device [B][num_kv_heads][head_dim] of `dtype`, 16-byte aligned.
 *   k_cache, v_cache   device, written at the B new slots only.
 *   Other arguments as paged_attention_decode.  The slots must be private to their sequences
 *   (copy-on-write copies done first) and distinct.  Every dtype: bf16 / fp16 in the matrix-core
 *   kernel, fp32 in the vector-ALU kernel (which also copies the rows into the slots).
 */
int paged_attention_decode_append(void* out, int32_t out_dtype, const void* query, const void* new_key,
                                  const void* new_value, void* k_cache, void* v_cache, const int32_t* block_tables,
                                  const int32_t* context_lens, int32_t B, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                                  int32_t num_blocks, int32_t max_context_len, float scale, int32_t partition_size,
                                  void* workspace, size_t workspace_bytes, int32_t dtype,
                                  const int32_t* host_context_lens, pkv_stream_t stream);
/* Its partition launch alone (then paged_attention_decode_reduce), as for paged_attention_decode. */
int paged_attention_decode_append_partitions(void* out, int32_t out_dtype, const void* query, const void* new_key,
                                             const void* new_value, void* k_cache, void* v_cache,
                                             const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                             int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                                             int32_t max_context_len, float scale, int32_t partition_size,
                                             void* workspace, size_t workspace_bytes, int32_t dtype,
                                             const int32_t* host_context_lens, pkv_stream_t stream);

/*
 * paged_attention_decode_newest - decode attention in which every sequence's newest token
 * (position context_lens[b] - 1) is taken from new_key / new_value instead of the cache, and the
 * cache is not written.  The caller stores those tokens with paged_cache_append, before, after,
 * or concurrently on another stream: this call never depends on the bytes of those slots, so the
 * append can overlap the attention.  Output bit for bit that of paged_attention_decode_append.
 * Arguments as paged_attention_decode_append (k_cache, v_cache read only).  Every dtype.
 */
int paged_attention_decode_newest(void* out, int32_t out_dtype, const void* query, const void* new_key,
                                  const void* new_value, const void* k_cache, const void* v_cache,
                                  const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                  int32_t max_blocks_per_seq, int32_t num_blocks, int32_t max_context_len,
                                  float scale, int32_t partition_size, void* workspace, size_t workspace_bytes,
                                  int32_t dtype, const int32_t* host_context_lens, pkv_stream_t stream);
/* Its partition launch alone (then paged_attention_decode_reduce). */
int paged_attention_decode_newest_partitions(void* out, int32_t out_dtype, const void* query, const void* new_key,
                                             const void* new_value, const void* k_cache, const void* v_cache,
                                             const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                             int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                                             int32_t max_context_len, float scale, int32_t partition_size,
                                             void* workspace, size_t workspace_bytes, int32_t dtype,
                                             const int32_t* host_context_lens, pkv_stream_t stream);

/*
 * paged_attention_prefill_chunk - causal attention of one prompt chunk against the paged cache.
 * [Chapter] "How the scheduler works" and [Notes] "Prefill gets in the way": a long prompt is
 * prefilled in chunks that fit a per-step token budget.  Row i of the chunk sits at absolute
 * position ctx_start + i and attends to positions 0 .. ctx_start + i of its sequence.  The
 * chunk's own K/V must already be appended (paged_cache_append) before this call.
 *
 *   out         device [C][num_q_heads][head_dim] of out_dtype (PKV_F32 or `dtype`).
 *   query       device [C][num_q_heads][head_dim] of `dtype` (bf16 and fp16 run on the matrix cores;
 *               PKV_F32 on the vector ALU, at most 65535 rows).
 *   block_table device int32 [>= ceil((ctx_start + C) / block_size)] of the one sequence.
 *   scale       positive and finite (PKV_EINVAL otherwise).
 * Accumulation is fp32.
 */
int paged_attention_prefill_chunk(void* out, int32_t out_dtype, const void* query, const void* k_cache,
                                  const void* v_cache, const int32_t* block_table, int32_t ctx_start,
                                  int32_t C, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t block_size, int32_t num_blocks, float scale, int32_t dtype,
                                  pkv_stream_t stream);

/*
 * paged_attention_mixed - one launch for a continuous-batching step's attention: a decode batch
 * and up to 16 prefill chunks ([Chapter] "How the scheduler works" and [Notes] "Prefill gets in the
 * way": a step carries the running sequences' decode tokens and a chunk of a new prompt).  The
 * decode part is paged_attention_decode (dec_group_size 1) or paged_attention_decode_grouped with
 * dec_partition_size; chunk i is paged_attention_prefill_chunk over its own table row; outputs
 * are bit for bit theirs.  Decode workgroups are dispatched first, so their cache streaming
 * overlaps the prefill tiles' matrix work.  With split-K partitions, the decode's log-sum-exp
 * merge (paged_attention_decode_reduce) is enqueued after the launch.  Either part may be empty
 * (B_dec = 0 or num_chunks = 0).
 *   decode:  dec_out [B_dec][Hq][D] (out_dtype), dec_query [B_dec][Hq][D], dec_block_tables
 *            [B_dec][dec_max_blocks], dec_context_lens [B_dec] (device); dec_max_context_len,
 *            host_dec_context_lens (NULL or a host copy, for the work order; ignored when grouped),
 *            dec_partition_size and workspace / workspace_bytes
 *            (paged_attention_decode_workspace_bytes(B_dec, Hq, D, dec_max_context_len,
 *            dec_partition_size)) as in paged_attention_decode.
 *            dec_group_size: 1, or the size with 8 matrix columns (8 / (Hq / Hkv) sequences; 2 when
 *            Hq / Hkv is 8) to run sequences dec_group_size to a workgroup and read the blocks they
 *            share once (paged_attention_decode_grouped).
 *   prefill: chunk i has host_chunk_lens[i] rows at positions host_ctx_starts[i] + r, packed one
 *            chunk after another in pre_query / pre_out ([sum of lengths][Hq][D]); its block table
 *            is row i of pre_block_tables [num_chunks][pre_max_blocks] (device); the chunks' K/V
 *            are already appended.  Starts and lengths are host arrays (they size the grid).
 *   group size Hq / Hkv in {1, 2, 4, 8}; bf16, fp16 or fp32; head_dim 64/128.  fp32 caches run
 *   the fp32 decode and prefill kernels' vector-ALU bodies (one wave per query head and sequence
 *   or chunk row; dec_group_size must be 1, else PKV_EUNSUPPORTED), bit for bit theirs.
 */
int paged_attention_mixed(void* dec_out, const void* dec_query, const int32_t* dec_block_tables,
                          const int32_t* dec_context_lens, int32_t B_dec, int32_t dec_max_blocks,
                          int32_t dec_max_context_len, const int32_t* host_dec_context_lens,
                          int32_t dec_partition_size, int32_t dec_group_size, void* workspace,
                          size_t workspace_bytes, void* pre_out, const void* pre_query,
                          const int32_t* pre_block_tables, int32_t pre_max_blocks, const int32_t* host_ctx_starts,
                          const int32_t* host_chunk_lens, int32_t num_chunks, int32_t out_dtype, const void* k_cache,
                          const void* v_cache, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size, int32_t num_blocks, float scale, int32_t dtype, pkv_stream_t stream);

/* ============================== FP8 K/V cache ============================== */
/*
 * An 8-bit cache halves the bytes a bandwidth-bound decode step reads and doubles the tokens that
 * fit ([Notes] "Continuous batching and PagedAttention: serving many users from one GPU", "Memory,
 * not compute, caps the batch").  Format: OCP 8-bit floating point E4M3 (bias 7, largest finite
 * 448, subnormals, no infinities).  Quantisation of each (token, KV head) row x of head_dim values,
 * K and V separately: amax = max |x_i|; scale s = amax / 448 (fp32, stored per slot);
 * code_i = E4M3 round-to-nearest-even(x_i * (448 / amax)) (0 when amax = 0); the cached value is
 * code_i * s.  A scale per slot means an append never rewrites the other tokens of its block.
 *
 * Layouts (device, caller-owned):
 *   k_cache  uint8 [num_blocks][Hkv][16 * head_dim]; within a (block, head) tile, byte (t, d) is at
 *            ((d / 64) * 2 + (t / 4) % 2) * 512 + ((t / 8) * 4 + t % 4) * 64 + d % 64.
 *   v_cache  uint8 [num_blocks][Hkv][head_dim][16] (dimension-major).
 *   k_scale, v_scale  fp32 [num_blocks][Hkv][16].
 * head_dim 64 or 128, block_size 16.  All four arrays 16-byte aligned.
 */

/*
 * paged_cache_append_fp8 - quantise the step's K/V rows and scatter them into their slots.
 *   key/value  device [T][num_kv_heads][head_dim] of in_dtype (PKV_F32/F16/BF16), token stride
 *              key_stride/value_stride elements (0 = contiguous).
 *   slot_mapping  device int32 [T], slot = block * 16 + offset; -1 = skip.  Slots must be unique.
 * Writes codes and both scales of every valid slot, nothing else.  Bit-exact with the definition.
 */
int paged_cache_append_fp8(void* k_cache, void* v_cache, void* k_scale, void* v_scale, const void* key,
                           const void* value, int64_t key_stride, int64_t value_stride, const int32_t* slot_mapping,
                           int32_t T, int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                           int32_t in_dtype, pkv_stream_t stream);

/* Copy-on-write copy of whole blocks of an fp8 cache: codes and scales (pairs as in paged_cache_copy_blocks). */
int paged_cache_copy_blocks_fp8(void* k_cache, void* v_cache, void* k_scale, void* v_scale, const int32_t* src_dst,
                                int32_t n, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                int32_t num_blocks, pkv_stream_t stream);

/*
 * paged_attention_decode_fp8 - paged_attention_decode over an fp8 cache: the same arguments and
 * guarantees (split-K, batch invariance, longest-first order, workspace from
 * paged_attention_decode_workspace_bytes), plus k_scale/v_scale; `q_dtype` is the query's type
 * (PKV_BF16 or PKV_F16), out_dtype PKV_F32 or q_dtype.  The result is attention over the values the
 * cache stands for (code * scale), accumulated in fp32.  _partitions is its first launch alone
 * (then paged_attention_decode_reduce).
 */
int paged_attention_decode_fp8(void* out, int32_t out_dtype, const void* query, const void* k_cache,
                               const void* v_cache, const void* k_scale, const void* v_scale,
                               const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int32_t max_blocks_per_seq, int32_t num_blocks, int32_t max_context_len, float scale,
                               int32_t partition_size, void* workspace, size_t workspace_bytes, int32_t q_dtype,
                               const int32_t* host_context_lens, pkv_stream_t stream);
int paged_attention_decode_fp8_partitions(void* out, int32_t out_dtype, const void* query, const void* k_cache,
                                          const void* v_cache, const void* k_scale, const void* v_scale,
                                          const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                          int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                                          int32_t max_context_len, float scale, int32_t partition_size,
                                          void* workspace, size_t workspace_bytes, int32_t q_dtype,
                                          const int32_t* host_context_lens, pkv_stream_t stream);

/*
 * paged_attention_decode_grouped_fp8 - paged_attention_decode_grouped over an fp8 cache.
 * [Chapter] "PagedAttention: KV cache memory" (samples and conversations sharing a prefix point at
 * the same physical blocks) over the quantised cache of [Notes] "Memory, not compute, caps the
 * batch".  Sequences group_size * k .. group_size * k + group_size - 1 run in one workgroup per KV
 * head (and partition), their query heads side by side in the matrix columns; a 32-token step
 * whose two blocks are the same in every member's table has its codes and scales read once for
 * the whole group.
 *   group_size  1 (exactly paged_attention_decode_fp8 without a work order), or a size with
 *               group_size * (num_q_heads / num_kv_heads) equal to 8 or 16 (PKV_EUNSUPPORTED
 *               otherwise).
 *   Other arguments as paged_attention_decode_fp8 (no host_context_lens: groups run in batch order).
 * Output: bit for bit that of paged_attention_decode_fp8 with the same partition_size.  Codes and
 * scales of every token some member of a group sees must be finite.
 */
int paged_attention_decode_grouped_fp8(void* out, int32_t out_dtype, const void* query, const void* k_cache,
                                       const void* v_cache, const void* k_scale, const void* v_scale,
                                       const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                                       int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                       int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                                       int32_t max_context_len, float scale, int32_t partition_size,
                                       void* workspace, size_t workspace_bytes, int32_t q_dtype,
                                       int32_t group_size, pkv_stream_t stream);

/*
 * paged_attention_decode_append_fp8 - paged_attention_decode_append over an fp8 cache: one decode
 * step with the step's quantising append fused in.  [Serving] Steps 4 and 6 in one launch, over
 * the quantised cache the [Notes] section "Memory, not compute, caps the batch" asks for: every
 * sequence's newest token (position context_lens[b] - 1) is quantised exactly as
 * paged_cache_append_fp8 quantises it (per (token, head): scale = amax / 448, codes = E4M3
 * nearest-even of x * (448 / amax)), its codes and scales are written into its slot, and
 * attention over all context_lens[b] tokens uses them.  Output, codes and scales equal, bit for
 * bit, paged_cache_append_fp8 of those tokens followed by paged_attention_decode_fp8.
 *   new_key, new_value device [B][num_kv_heads][head_dim] of q_dtype (bf16 or fp16), 16-byte aligned.
 *   k_cache, v_cache, k_scale, v_scale  device, written at the B new slots' blocks only (each
 *                  such block's code tiles and scale rows are stored back whole, the other slots
 *                  with the bytes they held).
 *   Other arguments as paged_attention_decode_fp8.  The slots must be private to their sequences
 *   (copy-on-write copies done first) and distinct.
 */
int paged_attention_decode_append_fp8(void* out, int32_t out_dtype, const void* query, const void* new_key,
                                      const void* new_value, void* k_cache, void* v_cache, void* k_scale,
                                      void* v_scale, const int32_t* block_tables, const int32_t* context_lens,
                                      int32_t B, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                                      int32_t max_context_len, float scale, int32_t partition_size,
                                      void* workspace, size_t workspace_bytes, int32_t q_dtype,
                                      const int32_t* host_context_lens, pkv_stream_t stream);

/*
 * paged_attention_prefill_chunk_fp8 - paged_attention_prefill_chunk over an fp8 cache: causal
 * attention of one prompt chunk ([Chapter] "How the scheduler works", [Notes] "Prefill gets in the
 * way") against the values the quantised cache stands for (code * scale).  The chunk's own K/V must
 * already be appended (paged_cache_append_fp8).
 *   out         device [C][num_q_heads][head_dim] of out_dtype (PKV_F32 or q_dtype).
 *   query       device [C][num_q_heads][head_dim] of q_dtype (PKV_BF16 or PKV_F16).
 *   k_cache, v_cache, k_scale, v_scale  the fp8 layouts above.
 *   block_table device int32 [>= ceil((ctx_start + C) / block_size)] of the one sequence.
 *   scale       positive and finite (PKV_EINVAL otherwise).
 * Codes are widened exactly to q_dtype for the matrix-core products; accumulation is fp32.
 */
int paged_attention_prefill_chunk_fp8(void* out, int32_t out_dtype, const void* query, const void* k_cache,
                                      const void* v_cache, const void* k_scale, const void* v_scale,
                                      const int32_t* block_table, int32_t ctx_start, int32_t C, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                      float scale, int32_t q_dtype, pkv_stream_t stream);

/*
 * paged_attention_mixed_fp8 - paged_attention_mixed over an fp8 cache: one launch for a step's
 * decode rows (paged_attention_decode_fp8) and up to 16 prefill chunks
 * (paged_attention_prefill_chunk_fp8); outputs are bit for bit theirs.  [Chapter] "How the
 * scheduler works" and [Notes] "Prefill gets in the way" (decodes and a prompt chunk in one step),
 * over the quantised cache of [Notes] "Memory, not compute, caps the batch".  Arguments as
 * paged_attention_mixed, except: no grouped decode (one sequence per decode workgroup); the
 * caches and k_scale / v_scale are the fp8 layouts above; q_dtype (PKV_BF16 or PKV_F16) is the type
 * of both queries, out_dtype PKV_F32 or q_dtype; the decode part follows paged_attention_decode_fp8's
 * rules (partition_size 0, -1 or a multiple of 16, workspace from
 * paged_attention_decode_workspace_bytes, longest-first order from host_dec_context_lens).  With
 * split-K partitions the log-sum-exp merge is enqueued after the launch.
 */
int paged_attention_mixed_fp8(void* dec_out, const void* dec_query, const int32_t* dec_block_tables,
                              const int32_t* dec_context_lens, int32_t B_dec, int32_t dec_max_blocks,
                              int32_t dec_max_context_len, const int32_t* host_dec_context_lens,
                              int32_t dec_partition_size, void* workspace, size_t workspace_bytes, void* pre_out,
                              const void* pre_query, const int32_t* pre_block_tables, int32_t pre_max_blocks,
                              const int32_t* host_ctx_starts, const int32_t* host_chunk_lens, int32_t num_chunks,
                              int32_t out_dtype, const void* k_cache, const void* v_cache, const void* k_scale,
                              const void* v_scale, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                              int32_t block_size, int32_t num_blocks, float scale, int32_t q_dtype,
                              pkv_stream_t stream);

/* ============================== host block pool ============================== */
/*
 * [Serving] Step 4: a pool of physical block ids with a free list; allocation takes the id at the
 * END of the free list and fails when it is empty; freeing puts the id back at the end; a
 * sequence owns a block table and a token count; the token at position pos opens a new block when
 * pos % block_size == 0.  Sharing with copy-on-write per [Chapter] "PagedAttention: KV cache
 * memory" and [Notes] "Fragmentation: PagedAttention":
 *   - fork gives a new sequence the parent's table and length and one more reference per block;
 *   - an append whose first token lands in a partially filled last block with refcount > 1 takes
 *     a fresh block, reports (old, new) for paged_cache_copy_blocks, and drops one reference of old;
 *   - free drops one reference per block in table order and returns a block to the free list
 *     when its count reaches 0 (a block registered in the prefix cache goes to its LRU instead).
 * Appends are all-or-nothing: PKV_ENOMEM leaves the pool unchanged.  With the prefix cache in
 * use, an allocation with an empty free list evicts (see pkv_prefix_insert), and PKV_ENOMEM means
 * the free list and the evictable blocks together are too few.  Sequence ids are the lowest
 * id not currently live.  The pool is host memory only, synchronous, and not thread-safe per
 * handle (different handles are independent).  It never touches the GPU.
 */
typedef struct pkv_pool pkv_pool;

/* free_order: NULL = 0..num_blocks-1, else a permutation of 0..num_blocks-1 (copied). */
int pkv_pool_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order, pkv_pool** out);
void pkv_pool_destroy(pkv_pool* pool);
int pkv_pool_num_free(const pkv_pool* pool, int32_t* out);
/* Copies the free list (bottom to top; the next allocation takes the last entry); *n = its length. */
int pkv_pool_free_list(const pkv_pool* pool, int32_t* out, int32_t capacity, int32_t* n);
int pkv_pool_refcount(const pkv_pool* pool, int32_t block, int32_t* out);

int pkv_seq_new(pkv_pool* pool, int32_t* seq_id);
int pkv_seq_fork(pkv_pool* pool, int32_t parent, int32_t* child);
/* Fresh blocks an append of n tokens would take, including a copy-on-write block. */
int pkv_seq_blocks_needed(const pkv_pool* pool, int32_t seq, int32_t n, int32_t* out);
/*
 * Reserve slots for n tokens of seq.  slots_out: host int32 [n].  cow_src_dst_out: host int32 [2],
 * written when *n_cow == 1 (at most one copy per append).  n == 0 is a no-op.
 */
int pkv_seq_append(pkv_pool* pool, int32_t seq, int32_t n, int32_t* slots_out, int32_t* cow_src_dst_out,
                   int32_t* n_cow);
/*
 * Batched append, sequence by sequence in the given order; each append is all-or-nothing.  On
 * PKV_ENOMEM, *done = the index of the sequence that did not fit (earlier ones are applied).
 * slots_out: host int32 [sum(counts)] in batch order; cow_out: host int32 [n][2];
 * *n_cow = pairs written.
 */
int pkv_seqs_append(pkv_pool* pool, const int32_t* seqs, const int32_t* counts, int32_t n,
                    int32_t* slots_out, int32_t* cow_out, int32_t* n_cow, int32_t* done);
int pkv_seq_free(pkv_pool* pool, int32_t seq);
int pkv_seq_len(const pkv_pool* pool, int32_t seq, int32_t* out);
int pkv_seq_num_blocks(const pkv_pool* pool, int32_t seq, int32_t* out);

/*
 * Block tables: tables_out host int32 [n][max_blocks], row b = the physical blocks of seqs[b] in
 * logical order padded with -1; lens_out host int32 [n] (may be NULL) = tokens of each.
 * PKV_EINVAL if a table is longer than max_blocks.
 */
int pkv_build_block_tables(const pkv_pool* pool, const int32_t* seqs, int32_t n, int32_t max_blocks,
                           int32_t* tables_out, int32_t* lens_out);
/*
 * Slot mapping: for each b, the slots of positions [starts[b], starts[b] + counts[b]) of seqs[b],
 * concatenated in batch order into slots_out (host int32 [sum(counts)]):
 * slot = table[pos / block_size] * block_size + pos % block_size.  Positions must be stored.
 */
int pkv_build_slot_mapping(const pkv_pool* pool, const int32_t* seqs, const int32_t* starts,
                           const int32_t* counts, int32_t n, int32_t* slots_out);

/* ============================== prefix cache ============================== */
/*
 * [Serving] Step 8 ("Prefix caching"): a request whose leading tokens are already held in blocks
 * shares them - the longest block-aligned prefix first - and each shared block gains a reference.
 * Blocks are registered by content: registered block k of a prefix is identified by the tokens of
 * the whole prefix up to and including its own block_size tokens.  Tokens are opaque host int32.
 *
 * pkv_prefix_insert - register seq's full blocks (the first min(n_tokens, length) / block_size)
 *   under the prefixes of `tokens` (the caller's token ids for the sequence's positions 0..).
 *   A prefix already registered keeps its block (seq's copy stays unregistered) and the walk goes
 *   on below it; the walk stops at a block already registered under a different prefix.  Only
 *   full blocks are registered, so a registered block is never written again.
 *   *n_registered (may be NULL) = seq's blocks newly registered.
 * pkv_prefix_lookup - start a new sequence (lowest free id) holding the longest registered
 *   block-aligned prefix of tokens[0 .. n_tokens) (possibly all of it, possibly none): its table
 *   is those blocks, its length *n_matched; each block gains a reference.  The caller appends the
 *   remaining tokens with pkv_seq_append as usual.
 * Release and eviction: a registered block whose count reaches 0 is not freed but waits on an LRU
 *   list (least recently released first); a lookup hit takes it off.  The registered blocks one
 *   pkv_seq_free releases join the list deepest first (reverse table order), so eviction shortens
 *   a registered prefix from its end.  An allocation that finds
 *   the free list empty evicts the LRU head: it and every registered block below it (prefixes
 *   extending through it) are unregistered; those below without references move from the LRU to
 *   the free list, least recently released first; the evicted block is the one allocated.
 * pkv_prefix_evictable - copy the LRU (front = next to evict) to out; *n = its length.
 * pkv_prefix_num_registered - number of registered blocks.
 */
int pkv_prefix_insert(pkv_pool* pool, int32_t seq, const int32_t* tokens, int32_t n_tokens, int32_t* n_registered);
int pkv_prefix_lookup(pkv_pool* pool, const int32_t* tokens, int32_t n_tokens, int32_t* seq_out, int32_t* n_matched);
int pkv_prefix_evictable(const pkv_pool* pool, int32_t* out, int32_t capacity, int32_t* n);
int pkv_prefix_num_registered(const pkv_pool* pool, int32_t* out);

#ifdef __cplusplus
}
#endif
#endif /* PAGEDKV_H */

/*
 * pkv -- paged key/value cache and decode attention for AMD MI355X (gfx950).
 *
 * C ABI. Plain pointers and sizes only. Host pointers are marked (host);
 * every other pointer is device memory that the CALLER allocates and owns:
 * the library never allocates or frees device memory. The one piece it holds
 * is the static scratch array of pkv_paged_attention_decode_noalloc
 * (PKV_NOALLOC_SCRATCH_BYTES per device, for the life of the process).
 *
 * Cache layout (both K and V): [num_blocks][num_kv_heads][block_size][head_dim],
 * row-major, head_dim innermost. Token t of a sequence lives in physical block
 * table[t / block_size], row t % block_size; its slot number is
 * physical_block * block_size + t % block_size.
 *
 * Sources: "vLLM and PagedAttention: Virtual Memory for LLM Serving" (slides 9-16)
 * and "Week 22 Day 2: High-Throughput Serving with vLLM & PagedAttention"
 * (sections 2-4), which state the problem: fixed-size blocks reached through a
 * per-sequence block table, one shared pool, allocation only when the last block
 * fills, reference-counted sharing with copy-on-write of the last block, and
 * attention computed block by block from non-contiguous blocks.
 *
 * Errors: every int-returning call returns a pkv_status. On failure nothing is
 * launched and no state changes; pkv_last_error() describes the failure
 * (thread-local, valid until the next call on the same thread).
 * Kernel calls enqueue on the given stream and return without waiting; only
 * launch-time errors are reported synchronously.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef PKV_HIP_STREAM_DEFINED
#define PKV_HIP_STREAM_DEFINED
typedef struct ihipStream_t *hipStream_t; /* same declaration as <hip/hip_runtime_api.h> */
#endif

typedef enum pkv_status {
    PKV_OK = 0,
    PKV_EINVAL = -1,      /* bad argument; nothing launched, nothing changed */
    PKV_ENOMEM = -2,      /* block pool exhausted; pool state unchanged */
    PKV_ENOSEQ = -3,      /* unknown sequence id */
    PKV_EHIP = -4,        /* HIP runtime / launch error */
    PKV_EUNSUPPORTED = -5,/* dtype / head_dim / block_size / group combination not built */
    PKV_EEXIST = -6       /* sequence id already in use */
} pkv_status;

typedef enum pkv_dtype {
    PKV_F32 = 0,
    PKV_F16 = 1,  /* IEEE binary16 */
    PKV_BF16 = 2  /* bfloat16 */
} pkv_dtype;

/* Attention flags. */
#define PKV_FLAG_SCALAR_GQA 1u /* use the one-query-head-per-workgroup kernel even when G > 1 */
/* The batch's sequences share blocks (a common prefix mapped by many block tables, slide 14:
 * a system prompt shared like a library): load all K/V through the caches, so that a block's
 * re-reads by the other sequences hit the L2 / last-level cache. Without it K/V are streamed
 * past the caches (non-temporal), which suits blocks read once per call, except the tokens the
 * cached_lens hint of pkv_paged_attention_decode names (the finer choice: only the shared
 * prefix goes through the caches). Paged cache only. */
#define PKV_FLAG_CACHED_KV 2u

/* partition_size value for the balanced split: the library cuts the whole batch's work into
 * equal shares, one per workgroup on the device (a (sequence, head) may be cut anywhere), and a
 * merge pass combines the rows cut between shares. Up to 4096 sequences. */
#define PKV_PARTITION_BALANCED (-1)

const char *pkv_last_error(void);
const char *pkv_version(void);

/* ======================================================================
 * Host block-pool allocator (the scheduler side; slides 10-16).
 * A pool is host-only state owned by one scheduler thread; not thread-safe.
 * ==================================================================== */
typedef struct pkv_pool pkv_pool;

/* One pool of num_blocks physical blocks of block_size tokens (slide 12: a single
 * shared pool takes the place of per-request reservations). free_order (host, nullable) is a permutation of
 * 0..num_blocks-1: the order in which free blocks are handed out (NULL = ascending).
 * Free blocks form a LIFO stack: a freed block is the next one handed out. */
int pkv_pool_create(int32_t num_blocks, int32_t block_size, const int32_t *free_order, pkv_pool **out);
void pkv_pool_destroy(pkv_pool *pool);
int32_t pkv_pool_num_blocks(const pkv_pool *pool);
int32_t pkv_pool_block_size(const pkv_pool *pool);
int32_t pkv_pool_num_free(const pkv_pool *pool);
/* Reference count of a physical block (number of sequences mapping it); -1 if out of range. */
int32_t pkv_block_ref_count(const pkv_pool *pool, int32_t block);

/* A new, empty sequence. PKV_EEXIST if seq_id is in use. */
int pkv_seq_add(pkv_pool *pool, int64_t seq_id);
/* Drop a sequence: every block's count is decremented; blocks reaching zero return to
 * the pool at once, in logical order (lesson note, section 4: finished sequences free
 * their blocks immediately). */
int pkv_seq_free(pkv_pool *pool, int64_t seq_id);
/* child shares all of parent's blocks: same table and length, every block's count + 1
 * (slide 14; lesson note section 3: sharing raises a block's count by one). */
int pkv_seq_fork(pkv_pool *pool, int64_t parent, int64_t child);
/* Length in tokens (>= 0), or PKV_ENOSEQ. */
int64_t pkv_seq_len(const pkv_pool *pool, int64_t seq_id);
/* Number of blocks of the sequence (>= 0), or PKV_ENOSEQ. */
int32_t pkv_seq_num_blocks(const pkv_pool *pool, int64_t seq_id);
/* Copy the sequence's block table (host out[cap]); returns the number of blocks or an error. */
int32_t pkv_seq_blocks(const pkv_pool *pool, int64_t seq_id, int32_t *out, int32_t cap);

/* Reserve n_tokens[i] new token slots at the end of each sequence seq_ids[i] (host arrays),
 * for all n_seqs sequences together: either every sequence gets its slots or, with
 * PKV_ENOMEM, none does and nothing changes (slide 15: all-or-nothing).
 *  - A block is taken only when the last one is full (slide 11).
 *  - If a sequence's last block is shared (count > 1) and partly filled, the sequence
 *    first gets a private copy: a new block dst, the pair (src, dst) is emitted, src's
 *    count drops by one (slide 13: copy-on-write duplicates the shared last block and
 *    nothing else). The last sharer
 *    left writes in place, so n sharers make n-1 copies.
 * Sequences are served in the order given; a sequence may appear once per call.
 * slots_out (host, int64[sum n_tokens]) receives the slots in request order;
 * cow_pairs_out (host, int32[2*max_pairs]) receives (src, dst) pairs, their count in
 * *n_pairs_out. More pairs than max_pairs: PKV_EINVAL, nothing changes.
 * The caller must run pkv_copy_blocks on the pairs before pkv_reshape_and_cache writes
 * the new tokens (same stream). */
int pkv_seq_append(pkv_pool *pool, const int64_t *seq_ids, const int32_t *n_tokens, int32_t n_seqs,
                   int64_t *slots_out, int32_t *cow_pairs_out, int32_t max_pairs, int32_t *n_pairs_out);

/* Prefix cache (the lesson note, section 3.1: when many requests open with the same system
 * prompt, a cryptographic digest per prompt block finds blocks the pool already holds; the new
 * request maps them and raises their counts, and their keys and values are not computed again).
 * Digest of full prompt block j: SHA-256 of (digest of block j-1, or 32 zero bytes for j = 0)
 * followed by the block's block_size token ids as little-endian int32: equal digests mean
 * equal prefixes. Only full prompt blocks are hashed. A hashed block that falls free keeps its
 * digest and contents: free blocks without a digest are handed out first (the usual LIFO
 * order), then hashed free blocks, least recently freed first, each losing its digest. A
 * digest names one block: a new prompt block whose digest another block holds (a later block
 * of a chain whose earlier block was evicted) takes the digest over, and the other block
 * becomes an ordinary one (on the LIFO stack if free). */

/* Chained digests of the full blocks of tokens[n_tokens] into digests_out[32 * k], k =
 * n_tokens / block_size full blocks (returned); PKV_EINVAL if k > max_blocks. Host only. */
int pkv_prompt_digests(const int32_t *tokens, int64_t n_tokens, int32_t block_size, uint8_t *digests_out,
                       int64_t max_blocks);

/* Add sequence seq_id with a prompt of n_tokens token ids (host arrays). Its leading full
 * blocks whose digests the pool holds are mapped and counted (a hit on a free hashed block
 * takes it back from the free list); the rest get blocks as pkv_seq_append would, each new
 * full block registered under its digest. slots_out (host, int64[n_tokens]) receives -1 for
 * the n_cached_out leading tokens whose keys and values are already in the cache (a negative
 * slot is skipped by pkv_reshape_and_cache) and the slot of every other token.
 * PKV_EEXIST: seq_id exists; PKV_ENOMEM: not enough free blocks (nothing changes). */
int pkv_seq_add_prompt(pkv_pool *pool, int64_t seq_id, const int32_t *tokens, int32_t n_tokens, int64_t *slots_out,
                       int32_t *n_cached_out);

/* Blocks the pool holds a digest for (in use or free). */
int32_t pkv_pool_num_cached(const pkv_pool *pool);

/* Move n sequences (host array seq_ids, distinct) from pool src to pool dst, all or nothing:
 * the preemption and recovery of slide 15 (the newest request leaves at once and comes back
 * by swap), with src and dst the device pool and a host pool, either way round.
 *  - Every distinct block the sequences map gets one dst block, in first-use order (sequence
 *    order, then logical order); its dst count is the number of moved sequences mapping it,
 *    so sharing among them (forks, slide 14) survives the move.
 *  - The sequences then leave src as pkv_seq_free would, in the order given: a block that a
 *    sequence left behind still maps is copied but stays in src.
 *  - pairs_out (host, int32[2*max_pairs]) receives the (src block, dst block) pairs, their
 *    count in *n_pairs_out; the caller copies them (pkv_swap_blocks) before dst writes the
 *    sequences' next tokens or src hands the freed blocks out again (same stream).
 * PKV_ENOSEQ: a sequence not in src; PKV_EEXIST: a sequence already in dst; PKV_ENOMEM: dst
 * has fewer free blocks than needed; PKV_EINVAL: duplicates, more pairs than max_pairs,
 * different block sizes, or src == dst. On any error nothing changes. */
int pkv_seq_migrate(pkv_pool *src, pkv_pool *dst, const int64_t *seq_ids, int32_t n, int32_t *pairs_out,
                    int32_t max_pairs, int32_t *n_pairs_out);

/* Block tables of n sequences as a dense host array tables_out[n][max_blocks] (row i for
 * seq_ids[i]), padded with pad_value past each sequence's blocks, and their lengths in
 * ctx_out[n] (host). A sequence with more than max_blocks blocks: PKV_EINVAL.
 * The caller uploads both to the device every step (slide 16: workers receive the
 * block tables with every step). */
int pkv_build_block_tables(const pkv_pool *pool, const int64_t *seq_ids, int32_t n, int32_t max_blocks,
                           int32_t pad_value, int32_t *tables_out, int32_t *ctx_out);

/* Shared prefix of n sequences, from the reference counts (lesson note section 3.1: sharing a
 * block increments its count; slide 14: sequences share blocks): out[i] (host) = the tokens of
 * seq_ids[i] that lie in its leading blocks with a count above one, i.e.
 * min(length, block_size * j) for the first j blocks of its table that are all shared. The
 * cached_lens hint of pkv_paged_attention_decode. An unknown sequence: PKV_ENOSEQ, out unchanged. */
int pkv_shared_prefix_lens(const pkv_pool *pool, const int64_t *seq_ids, int32_t n, int32_t *out);

/* ======================================================================
 * Device kernels. dtype is a pkv_dtype; all tensors of one call share it.
 * ==================================================================== */

/* Write new tokens' keys and values into their slots (slide 11: a new token goes into
 * the free slot of the last block).
 *  key, value:   [num_tokens][num_kv_heads][head_dim], token rows key_stride / value_stride
 *                elements apart (>= num_kv_heads*head_dim; lets K and V be views of a
 *                fused projection output).
 *  k_cache, v_cache: the caches, num_blocks blocks each.
 *  slot_mapping: device int64[num_tokens]; a negative slot is skipped (padding).
 * Byte-exact copy. Slots >= num_blocks*block_size are skipped by the kernel (a caller
 * error). Duplicate non-negative slots in one call are a caller error (result
 * unspecified); with PKV_DEBUG_VALIDATE=1 both are PKV_EINVAL, launching nothing
 * (slot_mapping copied to the host after the stream's earlier work). Pointers must be
 * 16-byte aligned and strides*elt multiples of 16. */
int pkv_reshape_and_cache(const void *key, const void *value, int64_t key_stride, int64_t value_stride,
                          void *k_cache, void *v_cache, int64_t num_blocks, const int64_t *slot_mapping,
                          int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                          int32_t dtype, hipStream_t stream);

/* Copy whole blocks for copy-on-write (slide 13): for each pair p, block pairs[2p+1]
 * becomes a byte copy of block pairs[2p], in the K and the V cache of every layer.
 *  k_caches, v_caches: host arrays of num_layers device pointers.
 *  pairs: host int32[2*num_pairs] (src, dst), e.g. straight from pkv_seq_append.
 *  block_bytes: bytes of one block of one cache (num_kv_heads*block_size*head_dim*elt).
 * Checked on the host: every block in [0, num_blocks), dst values distinct, no dst equal
 * to any src (so the order of copies cannot matter); otherwise PKV_EINVAL. */
int pkv_copy_blocks(void *const *k_caches, void *const *v_caches, int32_t num_layers, int64_t num_blocks,
                    int64_t block_bytes, const int32_t *pairs, int32_t num_pairs, hipStream_t stream);

/* Copy whole blocks from one pool's caches to another's: for each pair p and cache c, block
 * pairs[2p+1] of dst_caches[c] becomes a byte copy of block pairs[2p] of src_caches[c]. The
 * copy half of preemption by swap (slide 15): with the pairs from pkv_seq_migrate, a device
 * pool's caches to a host pool's (swap out) or back (swap in).
 *  src_caches, dst_caches: host arrays of num_caches pointers (e.g. K and V of every layer),
 *    each device memory or pinned host memory (allocated pinned through the HIP runtime; the
 *    GPU reads or writes it over the host link), holding src_num_blocks / dst_num_blocks
 *    blocks of block_bytes bytes; 16-byte aligned, block_bytes a multiple of 16.
 *  pairs: host int32[2*num_pairs] (src block, dst block).
 * One kernel launch per 8 caches and 224 pairs, on `stream`; pageable host memory is never
 * touched by the device.
 * PKV_EINVAL, with nothing launched: a block outside its pool, a destination block twice, a
 * pointer that is neither device nor pinned host memory or whose allocation is smaller than
 * its pool, a source overlapping its destination, bad sizes or alignment. */
int pkv_swap_blocks(const void *const *src_caches, void *const *dst_caches, int32_t num_caches,
                    int64_t src_num_blocks, int64_t dst_num_blocks, int64_t block_bytes, const int32_t *pairs,
                    int32_t num_pairs, hipStream_t stream);

/* Bytes of fp32 workspace a split mode needs:
 *  partition_size > 0: R = num_seqs * num_q_heads * ceil(max_context_len / partition_size) partition
 *                      rows of (head_dim + 2) floats. With head_dim 128, num_q_heads >= 2 and a
 *                      device to query, room for the grouped-query kernel's persistent schedule
 *                      follows: (align4(R * 130) + 8 * CU * min(num_q_heads, 16) * 130 + 4097
 *                      + num_seqs * num_q_heads) * 4, CU = the current device's compute units
 *                      (the rows padded to 16 bytes, one slot per wave and head of a group, the
 *                      prefix sums, a flag per row). Otherwise R * (head_dim + 2) * 4;
 *  PKV_PARTITION_BALANCED: W * (2 * num_q_heads * (head_dim + 2) * 4 + 8) + 4097 * 4, where W is
 *                          2 * the current device's compute units (0 if the device cannot be queried);
 *  partition_size == 0: 0. */
size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                  int32_t max_context_len, int32_t partition_size);

/* Decode attention over the paged cache, one query token per sequence (slide 9: attention
 * evaluated one block at a time, keys and values read from physically scattered blocks):
 *   for each sequence s and query head h (kv head h / (num_q_heads/num_kv_heads)):
 *   out[s][h] = softmax_t(scale * q[s][h] . K_t) . V_t over t < context_lens[s],
 *   K_t, V_t read from block block_tables[s][t / block_size], row t % block_size.
 *  out, q:        device [num_seqs][num_q_heads][head_dim], 16-byte aligned; out is written in
 *                 dtype (RNE).
 *  block_tables:  device int32[num_seqs][max_blocks_per_seq]; entries past a sequence's
 *                 last block are never read (so they may hold anything).
 *  context_lens:  device int32[num_seqs]; a sequence with length 0 gets zeros.
 *  max_context_len: host bound on context_lens, sizes the launch.
 *  partition_size: 0 = one pass per (sequence, head). > 0 (a multiple of block_size):
 *                 each (sequence, head) is cut into parts of that many tokens, each part's
 *                 attention computed on its own, then the parts merged by log-sum-exp. The
 *                 grouped-query matrix-core kernel (up to 4096 sequences) streams the parts on a
 *                 persistent schedule and merges the parts of a row that one workgroup held
 *                 whole in the same launch; other rows go through workspace to a merge pass.
 *                 Its rounding then depends on the compute-unit count, as in the balanced mode.
 *                 PKV_PARTITION_BALANCED: the batch's tiles are shared out evenly (see above),
 *                 then the same kind of merge; rounding then depends on the device's
 *                 compute-unit count (results are still reproducible on one device).
 *  workspace:     device, >= pkv_decode_workspace_bytes(...) bytes, 16-byte aligned;
 *                 may be NULL when partition_size == 0.
 *  flags:         PKV_FLAG_SCALAR_GQA and/or PKV_FLAG_CACHED_KV, or 0; other bits are PKV_EINVAL.
 *  cached_lens:   NULL, or device int32[num_seqs]: a load-policy hint. The first cached_lens[s]
 *                 tokens of sequence s sit in blocks other sequences of the batch also read (a
 *                 shared prefix; slide 14 and lesson note section 3.1: sharing is tracked by
 *                 reference counts, e.g. pkv_shared_prefix_lens). Their K/V loads go through
 *                 the caches, so the re-reads hit L2 instead of HBM; the other tokens are
 *                 loaded non-temporally. Any value is allowed (negative: none; past the length:
 *                 all). Not read with PKV_FLAG_CACHED_KV, which sends every load through the
 *                 caches. Neither changes any arithmetic: results are bit-identical with or
 *                 without them.
 * Device-side guards (never faults on bad tables, but the result is then unspecified):
 * lengths are clamped to [0, min(max_context_len, max_blocks_per_seq*block_size)] and a
 * table entry outside [0, num_blocks) contributes no tokens.
 * With the environment variable PKV_DEBUG_VALIDATE=1 the call first copies context_lens and
 * block_tables to the host (synchronising the stream; not for graph capture) and returns
 * PKV_EINVAL, launching nothing, for a length outside [0, max_context_len], a length needing
 * more than max_blocks_per_seq blocks, a used table entry outside [0, num_blocks), or an array
 * that is not device memory.
 * Supported: dtype f32/f16/bf16; head_dim 64 or 128; block_size 8, 16 or 32;
 * num_q_heads a multiple of num_kv_heads. */
int pkv_paged_attention_decode(void *out, const void *q, const void *k_cache, const void *v_cache,
                               int64_t num_blocks, const int32_t *block_tables, int32_t max_blocks_per_seq,
                               const int32_t *context_lens, int32_t max_context_len, int32_t num_seqs,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               float scale, int32_t partition_size, void *workspace, size_t workspace_bytes,
                               int32_t dtype, uint32_t flags, const int32_t *cached_lens, hipStream_t stream);

/* One decode step in one call: the cache write of pkv_reshape_and_cache for each sequence's new
 * token, then pkv_paged_attention_decode over the cache with that token in it (slide 11: each step
 * writes the new token's key and value into the free slot of the sequence's last block; slide 9:
 * attention block by block). Results and cache bytes are those of the two calls in that order.
 * One launch on the one-query-head kernel; the grouped-query matrix-core path writes the new rows
 * with a launch of its own first (measured faster there).
 *  new_k, new_v:  device [num_seqs][num_kv_heads][head_dim] in dtype, contiguous, 16-byte aligned:
 *                 the key and value of sequence s's token at position context_lens[s] - 1.
 *  slot_mapping:  device int64[num_seqs]: that token's slot, block_tables[s][t / block_size] *
 *                 block_size + t % block_size for t = context_lens[s] - 1 (pkv_seq_append gives
 *                 it), or negative: not written, and attention reads that row from the cache
 *                 (which must then hold the token already). A slot past num_blocks *
 *                 block_size is treated as negative; a sequence of length 0 has no such token,
 *                 so its slot must be negative.
 *  k_cache, v_cache: written at those slots (one row per kv head) and read.
 *  everything else: as for pkv_paged_attention_decode.
 * In one launch, attention takes each sequence's last row from new_k/new_v rather than from the
 * cache: no value the launch computes with comes from a location it writes. (The lanes of that row
 * still issue their load of its old cache bytes, which may race with the row's store by another
 * workgroup; a select replaces the loaded value before any arithmetic, so the race cannot reach a
 * result.) A slot that is not the slot of position
 * context_lens[s] - 1 is a caller error (the results then differ from the two calls);
 * PKV_DEBUG_VALIDATE=1 reports it as PKV_EINVAL, with the checks of the decode call. */
int pkv_paged_attention_decode_step(void *out, const void *q, const void *new_k, const void *new_v,
                                    const int64_t *slot_mapping, void *k_cache, void *v_cache, int64_t num_blocks,
                                    const int32_t *block_tables, int32_t max_blocks_per_seq,
                                    const int32_t *context_lens, int32_t max_context_len, int32_t num_seqs,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                    float scale, int32_t partition_size, void *workspace, size_t workspace_bytes,
                                    int32_t dtype, uint32_t flags, const int32_t *cached_lens, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): pkv_paged_attention_decode without the workspace
 * arguments. A split (partition_size != 0) takes its workspace from a static device array of
 * PKV_NOALLOC_SCRATCH_BYTES bytes that the library holds on each device it runs on until the
 * process ends (its address is looked up once per device, on the first call there). Same kernels,
 * same workspace layout, so results are bit-identical to pkv_paged_attention_decode with a
 * caller-provided workspace.
 *  All arguments: as for pkv_paged_attention_decode.
 *  PKV_EINVAL, launching nothing, when pkv_decode_workspace_bytes(...) for this call exceeds
 *  PKV_NOALLOC_SCRATCH_BYTES; PKV_EHIP when the array's address cannot be obtained.
 * The call allocates nothing (no hipMalloc, no host allocation) unless PKV_DEBUG_VALIDATE=1, whose
 * host copies it shares with the other entry points. Nothing in the array needs clearing between
 * calls: every value a split's merge pass reads is written by the same call first. Every call on
 * one device shares that device's array and leaves its contents behind, so calls that may overlap
 * on one device (different streams, or several host threads) race and must be serialised by the
 * caller, e.g. by issuing them on one stream. */
#define PKV_NOALLOC_SCRATCH_BYTES (128u * 1024u * 1024u)
int pkv_paged_attention_decode_noalloc(void *out, const void *q, const void *k_cache, const void *v_cache,
                                       int64_t num_blocks, const int32_t *block_tables, int32_t max_blocks_per_seq,
                                       const int32_t *context_lens, int32_t max_context_len, int32_t num_seqs,
                                       int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                       int32_t block_size, float scale, int32_t partition_size, int32_t dtype,
                                       uint32_t flags, const int32_t *cached_lens, hipStream_t stream);

/* Prefill (chunked) attention over the paged cache: the last n_s = query_start[s+1] -
 * query_start[s] tokens of each sequence s are queries, and query i of s, at position
 * p = context_lens[s] - n_s + i, attends causally to the keys at positions 0 .. p, earlier
 * chunks and shared prefix blocks included (slide 3: the prompt is processed in parallel;
 * slides 9 and 10: keys and values fetched block by block through the block table). The
 * queries' own keys and values must already be in the cache (pkv_reshape_and_cache).
 *   out[r][h] = softmax_t(scale * q[r][h] . K_t) . V_t over t <= p, for row r = query_start[s] + i
 *  out, q: [num_tokens][num_q_heads][head_dim], dtype, out written with RNE; rows past
 *          query_start[num_seqs] are not touched.
 *  query_start: device int32[num_seqs + 1], query_start[0] = 0, non-decreasing,
 *               query_start[num_seqs] <= num_tokens; n_s <= context_lens[s].
 *  num_tokens: rows of q and out (>= 0). max_query_len: host bound on n_s (sizes the launch).
 *  block_tables, context_lens, max_context_len, scale: as for pkv_paged_attention_decode.
 *  flags: 0.
 * The grouped-query matrix-core kernel generalised: a wave owns 16 (query token, query head)
 * rows of one kv head and walks every key tile up to its last row's position.
 * Supported: f16/bf16, head_dim 128, block_size 16 or 32, num_q_heads a multiple of
 * num_kv_heads. Device-side guards (caller errors; never a fault, but that sequence gets no
 * output): a sequence with n_s > context_lens[s], or whose rows query_start[s] ..
 * query_start[s+1] - 1 do not lie inside [0, num_tokens). PKV_DEBUG_VALIDATE=1 reports these,
 * query_start[0] != 0 and n_s > max_query_len as PKV_EINVAL, with the checks of the decode call
 * (query_start and context_lens copied to the host, synchronising the stream). */
int pkv_paged_attention_prefill(void *out, const void *q, const void *k_cache, const void *v_cache,
                                int64_t num_blocks, const int32_t *block_tables, int32_t max_blocks_per_seq,
                                const int32_t *context_lens, const int32_t *query_start, int32_t num_tokens,
                                int32_t max_query_len, int32_t max_context_len, int32_t num_seqs,
                                int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                float scale, int32_t dtype, uint32_t flags, hipStream_t stream);

/* The same attention over a contiguous cache, the layout paging replaces (slide 19 prices
 * the indirection against it): k, v are [num_seqs][num_kv_heads][lmax][head_dim] and token t
 * of (s, kv head) is row t of that slab. Same kernels, same tiling; only the address of a
 * tile differs. Lengths are clamped to [0, min(max_context_len, lmax)]; with
 * PKV_DEBUG_VALIDATE=1 a length above either is PKV_EINVAL (context_lens copied to the host). */
int pkv_contiguous_attention_decode(void *out, const void *q, const void *k, const void *v, int32_t lmax,
                                    const int32_t *context_lens, int32_t max_context_len, int32_t num_seqs,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, float scale,
                                    int32_t partition_size, void *workspace, size_t workspace_bytes,
                                    int32_t dtype, uint32_t flags, hipStream_t stream);

/* ======================================================================
 * Continuous-batching memory simulator (host only; the memory side of iteration-level
 * scheduling, lesson note "Week 22 Day 2" section 4, under the paged and the contiguous
 * scheme; slides 6, 7 and 15).
 * ==================================================================== */

/* Integers per trace row, in this order:
 *   step, running, waiting        step index; requests in the batch and in the queue after
 *                                 the step's admissions
 *   used                          slots holding a real token (sum of the running lengths)
 *   held, free, largest_free      slots given to running requests, slots not given, and the
 *                                 most one request could take (paged: all free slots)
 *   admitted, preempted, finished, decoded
 *                                 requests admitted, evicted, finished and decoding this step
 *   blocked_need                  slots the queue head asked for when admission stopped for
 *                                 memory, else 0 (external fragmentation: free >= blocked_need
 *                                 > largest_free)
 *   final_sum                     sum of the running requests' final lengths P + O */
#define PKV_SIM_FIELDS 13

/* Requests (host arrays of n_requests): arrival step (>= 0, non-decreasing), prompt length P
 * and output length O (both >= 1). A request holds P tokens after its prefill and P + O after
 * its O-th decode step, when it finishes; a fresh request admitted at step t, never evicted,
 * finishes at step t + O.
 * One step: arrivals join the queue tail; every running request appends one token; finished
 * requests are freed at once; the queue head is admitted while it fits and fewer than
 * max_batch requests run (strict queue order); one trace row is written. The run ends after
 * the step at which every request has finished.
 * trace_out: host int64[max_steps * PKV_SIM_FIELDS], rows of the steps run (*n_steps_out of them);
 * finish_out: host int64[n_requests], the step each request finished at.
 * PKV_EINVAL for bad arguments, a request that can never fit, or a run longer than max_steps
 * (outputs then unspecified). */

/* Paged: a pool of num_blocks blocks of block_size slots (this library's allocator, fresh,
 * ascending free order). A decode step appends one token to every running request in one
 * all-or-nothing batch; if the pool is short, the newest running request is freed whole and
 * returns to the queue head (slide 15), and the batch is tried again. An evicted request keeps
 * its generated tokens and recomputes them: its next prefill writes P + (tokens generated).
 * Admission needs ceil(tokens / block_size) + watermark_blocks free blocks. Every request must
 * satisfy ceil((P + O) / block_size) + watermark_blocks <= num_blocks. */
int pkv_sim_paged(int32_t num_blocks, int32_t block_size, int32_t watermark_blocks, int32_t max_batch,
                  const int32_t *arrival, const int32_t *prompt_len, const int32_t *output_len, int32_t n_requests,
                  int64_t max_steps, int64_t *trace_out, int64_t *n_steps_out, int64_t *finish_out);

/* Contiguous: capacity slots in one linear range; admission reserves reserve_len[i] slots
 * (P + O <= reserve_len[i] <= capacity; a system that does not know O reserves the maximum
 * length, lesson note section 1) in the lowest-addressed free run that holds them (first fit),
 * released on finish and merged with free neighbours. Nothing is evicted. */
int pkv_sim_contiguous(int64_t capacity, int32_t max_batch, const int32_t *arrival, const int32_t *prompt_len,
                       const int32_t *output_len, const int32_t *reserve_len, int32_t n_requests, int64_t max_steps,
                       int64_t *trace_out, int64_t *n_steps_out, int64_t *finish_out);

/* ======================================================================
 * Measurement companion (not part of the method).
 * ==================================================================== */

/* Read `bytes` of device memory at src once, with the 16-byte non-temporal loads the attention
 * kernels use, and nothing else: timing it gives the device's achievable streaming-read rate,
 * the context for an attention GB/s figure next to the datasheet HBM peak.
 *  src: device, 16-byte aligned; bytes a multiple of 16.
 *  sink: device, 16-byte aligned, 4 bytes; written only in the (practically impossible) case
 *        that the buffer's XOR-fold equals 0x9e3779b9, which keeps the loads live.
 * PKV_EINVAL for NULL or misaligned arguments. */
int pkv_read_probe(const void *src, size_t bytes, void *sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* PKV_H */

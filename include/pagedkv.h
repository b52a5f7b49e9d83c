/*
 * pagedkv -- paged KV-cache attention for AMD Instinct MI355X (gfx950).
 *
 * Attention for the current query tokens over a K/V cache that lives in
 * fixed-size physical blocks and is reached through a per-sequence block
 * table (cnblogs "paged attention", sections 2, 3 and 5; "08. PagedAttention",
 * sections "borrowing OS paging" and "why the name").
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Return value: PKV_OK (0) or a negative PKV_ERR_* code; no call throws.
 *    pkv_status_string() names a code.
 *  - Device pointers are caller-owned device memory (this library allocates
 *    no device memory; the caller sizes workspaces with the *_size calls).
 *    Host pointers are caller-owned host memory and are not retained.
 *  - GPU calls only enqueue work on `stream` (a hipStream_t; NULL = the
 *    default stream) and return at once.  Argument checks are synchronous and
 *    host-side; a failed check enqueues nothing.  A launch failure reports
 *    PKV_ERR_HIP.
 *  - Cache layout: k_cache and v_cache are [num_blocks][num_kv_heads]
 *    [block_size][head_dim] arrays of `dtype` elements.  Token slot s lives in
 *    physical block s / block_size at offset s % block_size.
 *  - Block tables are int32 [num_seqs][max_blocks_per_seq]; entry lb is the
 *    physical block of logical block lb (tokens lb*B .. lb*B+B-1).  Entries
 *    past ceil(context_len / block_size) may be read but are never
 *    dereferenced, and never change a result (pad them with -1).  Table
 *    contents are trusted: an entry outside [0, num_blocks) is not
 *    dereferenced; the output rows that attend a key of such a block are
 *    NaN, and no other row changes.
 *  - Query head h reads KV head h / (num_heads / num_kv_heads).
 *  - Device pointers to element arrays must be 16-byte aligned
 *    (PKV_ERR_ALIGN otherwise); int32 arrays need 4-byte alignment.
 *  - Supported shapes (PKV_ERR_UNSUPPORTED otherwise): dtype f32 or bf16;
 *    head_dim 16, 32, 64 or 128; block_size a power of two from 1 to 256;
 *    num_heads / num_kv_heads in {1, 2, 4, 8} with head_dim * elem_bytes
 *    / 16 >= that ratio.  Prefill: bf16, head_dim 64 or 128, any of those
 *    block sizes, and num_blocks * num_kv_heads * block_size < 2^32 (pool
 *    rows are indexed in 32 bits; a pool that size exceeds one GPU's HBM).
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_ABI_VERSION 1

#define PKV_OK 0
#define PKV_ERR_INVALID (-1)     /* bad argument (null, negative size, bad id) */
#define PKV_ERR_UNSUPPORTED (-2) /* shape or dtype outside the compiled set */
#define PKV_ERR_ALIGN (-3)       /* device pointer not 16-byte aligned */
#define PKV_ERR_NO_BLOCKS (-4)   /* free list too short; state unchanged */
#define PKV_ERR_STATE (-5)       /* allocator state inconsistent with the request */
#define PKV_ERR_HIP (-6)         /* a HIP runtime call or kernel launch failed */
#define PKV_ERR_WORKSPACE (-7)   /* workspace missing or smaller than required */

#define PKV_DTYPE_F32 0
#define PKV_DTYPE_BF16 1

/* Version of this interface (PKV_ABI_VERSION). */
int pkv_abi_version(void);

/* Static string naming a status code. */
const char* pkv_status_string(int status);

/* ------------------------------------------------------------------------
 * kv_write: store each new token's K and V at its slot.
 * "08. PagedAttention", section "why the name": slot =
 * block_table[logical block] * block_size + offset, and a small GPU kernel
 * writes every token's K/V to its slot.
 *
 *   k_new, v_new   device, [num_tokens][num_kv_heads][head_dim] of dtype
 *   slot_mapping   device int32 [num_tokens]; a negative slot skips the token;
 *                  slots must be < num_blocks * block_size and distinct
 *                  (duplicates race; out-of-range slots are skipped)
 *   k_cache, v_cache  device caches (layout above), updated in place
 * Bitwise copy of the token rows; nothing else in the caches changes.
 * ---------------------------------------------------------------------- */
int pkv_kv_write(const void* k_new, const void* v_new, const int32_t* slot_mapping, int num_tokens,
                 void* k_cache, void* v_cache, int num_blocks, int num_kv_heads, int block_size,
                 int head_dim, int dtype, void* stream);

/* ------------------------------------------------------------------------
 * copy_blocks: copy-on-write block copies.  intelliparadigm.com article,
 * section 2.3: when a sequence modifies a shared block, a new block is
 * allocated and the original block's contents are copied into it.
 *
 *   pairs   device int32 [num_pairs][2] = (src, dst) physical blocks
 * For each pair, every slot of every head of block dst in both caches becomes
 * a bitwise copy of block src.  Destinations must be distinct and must not
 * appear as sources (the allocator below only produces such lists); pairs
 * with an id outside [0, num_blocks) are skipped.
 * ---------------------------------------------------------------------- */
int pkv_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int num_pairs, int num_blocks,
                    int num_kv_heads, int block_size, int head_dim, int dtype, void* stream);

/* ------------------------------------------------------------------------
 * swap_out / swap_in: move whole blocks between the device pools and host
 * memory, for preemption by swapping (intelliparadigm.com article, sections
 * 3.1 and 6.1: blocks of a preempted request go to CPU memory and come back
 * later; "08. PagedAttention", section "what it does not solve").
 *
 *   block_ids        device int32 [num]: physical blocks, in the order of the
 *                    host buffers
 *   host_k, host_v   host memory [num][num_kv_heads][block_size][head_dim]
 *                    of dtype, pinned (hipHostMalloc or torch pin_memory) so
 *                    the GPU reads / writes it directly; 16-byte aligned;
 *                    caller-owned and not to be touched until the call has
 *                    completed on `stream`
 * swap_out: host[i] = cache[block_ids[i]]; swap_in: cache[block_ids[i]] =
 * host[i]; K and V, every head and slot, bitwise.  Ids outside
 * [0, num_blocks) are skipped; swap_in's ids must be distinct.
 * ---------------------------------------------------------------------- */
int pkv_swap_out(const void* k_cache, const void* v_cache, const int32_t* block_ids, int num, int num_blocks,
                 int num_kv_heads, int block_size, int head_dim, int dtype, void* host_k, void* host_v,
                 void* stream);

int pkv_swap_in(void* k_cache, void* v_cache, const int32_t* block_ids, int num, int num_blocks, int num_kv_heads,
                int block_size, int head_dim, int dtype, const void* host_k, const void* host_v, void* stream);

/* ------------------------------------------------------------------------
 * paged_attention_decode: one query token per sequence.
 * out[s][h] = softmax(scale * q[s][h] . K_s^T) V_s over the first
 * context_lens[s] tokens of sequence s, K_s / V_s read through the block
 * table (cnblogs section 5: position -> logical block -> physical block; the
 * attention formula itself is unchanged, cnblogs section 6).
 *
 *   out            device [num_seqs][num_heads][head_dim] of dtype (written)
 *   q              device [num_seqs][num_heads][head_dim] of dtype
 *   block_tables   device int32 [num_seqs][max_blocks_per_seq]
 *   context_lens   device int32 [num_seqs]; the count includes the token this
 *                  step wrote.  <= 0 gives zeros; values above
 *                  max_blocks_per_seq * block_size are clamped to it.
 *   workspace      device scratch of at least pkv_decode_workspace_size(...)
 *                  bytes, private to this call until it completes on `stream`;
 *                  its contents need no initialisation
 * Accumulation is fp32.  Long contexts are split across wavefronts; partial
 * results are merged with their log-sum-exp weights in a second kernel.
 * ---------------------------------------------------------------------- */
/* Returns 0 for unsupported shapes.  The size depends on the decode grid:
 * a fixed number of workgroups per compute unit, which the environment
 * variable PKV_DECODE_WG_PER_CU (1..8) overrides.  Size the workspace with
 * the same setting as the calls that use it; a call whose grid needs more
 * than workspace_bytes returns PKV_ERR_WORKSPACE and launches nothing. */
size_t pkv_decode_workspace_size(int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                                 int block_size, int max_blocks_per_seq, int dtype);

int pkv_paged_attention_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, int max_blocks_per_seq,
                               const int32_t* context_lens, int num_seqs, int num_heads,
                               int num_kv_heads, int head_dim, int block_size, int num_blocks,
                               float scale, int dtype, void* workspace, size_t workspace_bytes,
                               void* stream);

/* Append and attend in one call: the kv_write of one new token per sequence
 * ("08. PagedAttention", section "why the name": slot = block_table[logical
 * block] * block_size + offset) followed by pkv_paged_attention_decode, for
 * the usual decode step in which every sequence's new token is its last.
 * For each sequence s with p = context_lens[s] - 1 >= 0:
 *   - k_new[s], v_new[s] (device, [num_seqs][num_kv_heads][head_dim] of
 *     dtype) are stored at slot block_tables[s][p / block_size] *
 *     block_size + p % block_size of k_cache / v_cache;
 *   - out[s] is the decode of q[s] over positions 0 .. p, position p taking
 *     those K/V.
 * The result, output and caches, is bit for bit that of pkv_kv_write of the
 * same rows at those slots and then pkv_paged_attention_decode.  Other
 * arguments, the workspace (sized by pkv_decode_workspace_size) and the
 * errors are those of pkv_paged_attention_decode; k_new and v_new must be
 * 16-byte aligned.
 * The caller guarantees that the slot belongs to sequence s alone in this
 * call: a block shared by several sequences is copied before a write
 * (copy-on-write), as the allocator arranges; another sequence reading the
 * slot in the same call could see either value.
 * Sequences with context_lens[s] <= 0 write nothing and give zeros.  Those
 * with context_lens[s] > max_blocks_per_seq * block_size have no slot for
 * the new token: they write nothing and attend their first
 * max_blocks_per_seq * block_size tokens from the cache, as the decode does.
 * When the block id of position p lies outside [0, num_blocks), nothing is
 * written and the sequence's rows come out NaN, as in the decode. */
int pkv_paged_attention_decode_append(void* out, const void* q, const void* k_new, const void* v_new,
                                      void* k_cache, void* v_cache, const int32_t* block_tables,
                                      int max_blocks_per_seq, const int32_t* context_lens, int num_seqs,
                                      int num_heads, int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                      float scale, int dtype, void* workspace, size_t workspace_bytes,
                                      void* stream);

/* Sliding-window decode: as pkv_paged_attention_decode, but sequence s
 * attends only its last min(window, context_lens[s]) tokens (streaming with
 * a sliding window whose old blocks are reclaimed: intelliparadigm.com
 * article, section 5.2).  Table entries of blocks that lie wholly before
 * the window are never read, so pkv_seq_trim may have released them (-1).
 * window must be > 0 (PKV_ERR_INVALID otherwise); the workspace is sized by
 * pkv_decode_workspace_size as for the full decode. */
int pkv_paged_attention_decode_window(void* out, const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_tables, int max_blocks_per_seq,
                                      const int32_t* context_lens, int num_seqs, int num_heads, int num_kv_heads,
                                      int head_dim, int block_size, int num_blocks, int window, float scale,
                                      int dtype, void* workspace, size_t workspace_bytes, void* stream);

/* Decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): as
 * pkv_paged_attention_decode, with the same arguments minus the workspace.
 * The partial results live in a device array of this library, one copy per
 * GPU, PKV_DECODE_SCRATCH_BYTES large and held until the process ends; its
 * address is looked up on the first call on each device.  The call makes no
 * allocation of any kind.  A batch whose partials need more than that
 * (pkv_decode_workspace_size above it) returns PKV_ERR_WORKSPACE and
 * launches nothing.  Every call on one GPU shares its array: calls that may
 * run at the same time on one GPU (other streams, other threads) race and
 * must be ordered by the caller.  Nothing in the array needs to start at
 * zero; it keeps the last call's contents. */
#define PKV_DECODE_SCRATCH_BYTES (32u << 20)
int pkv_paged_attention_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                                       const int32_t* block_tables, int max_blocks_per_seq,
                                       const int32_t* context_lens, int num_seqs, int num_heads, int num_kv_heads,
                                       int head_dim, int block_size, int num_blocks, float scale, int dtype,
                                       void* stream);

/* ------------------------------------------------------------------------
 * paged_attention_prefill: a causal query chunk over a cached prefix.
 * Query i of sequence s (rows cu_q_lens[s] .. cu_q_lens[s+1]-1 of q) sits at
 * position context_lens[s] - C_s + i, C_s = cu_q_lens[s+1] - cu_q_lens[s],
 * and attends keys 0 .. that position inclusive.  The chunk's K/V must
 * already be in the cache (pkv_kv_write).  Block-wise computation of scores
 * and merging of partial results: intelliparadigm.com article, section 2.2.
 *
 *   out, q         device [total_q][num_heads][head_dim], bf16
 *   cu_q_lens      device int32 [num_seqs + 1], cu_q_lens[0] = 0, nondecreasing,
 *                  cu_q_lens[num_seqs] = total_q
 *   max_q_len      host bound on every C_s (sizes the launch); >= 1 when
 *                  total_q > 0 (PKV_ERR_INVALID otherwise).  Rows past
 *                  ceil(max_q_len / 256) * 256 of a longer chunk are written
 *                  as NaN, never left unwritten.
 *   context_lens   device int32 [num_seqs], each >= C_s
 * ---------------------------------------------------------------------- */
int pkv_paged_attention_prefill(void* out, const void* q, const int32_t* cu_q_lens, int total_q,
                                int max_q_len, const void* k_cache, const void* v_cache,
                                const int32_t* block_tables, int max_blocks_per_seq,
                                const int32_t* context_lens, int num_seqs, int num_heads,
                                int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                float scale, int dtype, void* stream);

/* ------------------------------------------------------------------------
 * paged_attention_decode_shared: decode for a batch whose sequences share a
 * prompt (parallel sampling, beam search).  Branches forked from one prompt
 * hold its blocks together, by reference count (intelliparadigm.com
 * article, section 2.3; "08. PagedAttention", section "what else paging
 * solves"); the pages store such a prompt once (cnblogs "paged attention",
 * section 9), and this call also reads it once per step: the query heads of
 * all members of a group are stacked against each shared block.  The result
 * is that of pkv_paged_attention_decode on the same inputs (the same
 * formula; only the order of the sums differs).
 *
 *   group_start    device int32 [num_groups + 1]: group i is the sequences
 *                  group_start[i] .. group_start[i+1] - 1 of the batch;
 *                  group_start[0] = 0, increasing, group_start[num_groups] =
 *                  num_seqs; each group holds 1 ..
 *                  pkv_decode_shared_max_members(num_heads, num_kv_heads)
 *                  sequences (members past that come out NaN)
 *   shared_blocks  device int32 [num_groups]: the number of leading table
 *                  entries that are the same block in every member of the
 *                  group and lie wholly inside every member's context
 *                  (pkv_shared_prefix_groups computes both arrays)
 * Other arguments as pkv_paged_attention_decode; no workspace: one launch,
 * one workgroup per (group, kv head).  bf16, head_dim 128, block_size a
 * power of two from 16 to 256 (PKV_ERR_UNSUPPORTED otherwise).
 * ---------------------------------------------------------------------- */
int pkv_paged_attention_decode_shared(void* out, const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* block_tables, int max_blocks_per_seq,
                                      const int32_t* context_lens, int num_seqs, const int32_t* group_start,
                                      const int32_t* shared_blocks, int num_groups, int num_heads, int num_kv_heads,
                                      int head_dim, int block_size, int num_blocks, float scale, int dtype,
                                      void* stream);

/* Largest group pkv_paged_attention_decode_shared takes for this head
 * layout: min(8, 16 / (num_heads / num_kv_heads)); 0 for an invalid one. */
int pkv_decode_shared_max_members(int num_heads, int num_kv_heads);

/* ------------------------------------------------------------------------
 * gather_units: a measurement aid, not part of the attention path.  Reads
 * every listed unit once and computes nothing else, so its rate is the HBM
 * bandwidth ceiling of the paged access pattern (a table lookup, then a
 * contiguous run per block; "08. PagedAttention", section "block size":
 * smaller blocks mean more scattered reads).
 *
 *   pool_a, pool_b   device pools of pool_units units of unit_kib KiB each
 *                    (pool_b may be NULL; when given, unit i is read from both)
 *   unit_ids         device int32 [num_units]: units to read; an id outside
 *                    [0, pool_units) reads unit 0 instead (nothing outside
 *                    the pools is ever read)
 *   unit_kib         a power of two from 1 to 4096
 *   sink             device uint32 [sink_words], sink_words >= 4: one folded
 *                    word per wavefront (keeps the loads live; no meaning)
 * ---------------------------------------------------------------------- */
int pkv_gather_units(const void* pool_a, const void* pool_b, const int32_t* unit_ids, int num_units, int unit_kib,
                     int64_t pool_units, void* sink, int sink_words, void* stream);

/* ------------------------------------------------------------------------
 * Host block allocator: builds block tables, slot mappings and copy lists.
 * Never touches the GPU.  Not thread-safe; one handle per owner.
 *
 * Policy (the pages fix the semantics; the order is this library's reading
 * so results are reproducible):
 *  - free list = LIFO stack; init_order[0] (or block 0) is popped first;
 *  - append: a new block only when the last one is full (cnblogs section 8);
 *    the first write into a block shared by several sequences copies it to a
 *    fresh block (copy-on-write, intelliparadigm.com section 2.3), the last
 *    holder writes in place;
 *  - fork(parent, child, f): child shares the parent's first ceil(f/B)
 *    blocks (ref + 1) and has length f ("08. PagedAttention", section "what
 *    else paging solves": shared blocks carry a reference count);
 *  - free: blocks are released in reverse logical order; a block whose
 *    count reaches 0 goes back on the free list at once (cnblogs section 7).
 * ---------------------------------------------------------------------- */
typedef struct pkv_alloc pkv_alloc;

typedef struct pkv_stats {
    int32_t num_blocks;
    int32_t block_size;
    int32_t num_free;
    int32_t num_used;       /* blocks with ref > 0 */
    int32_t num_seqs;
    int32_t num_shared;     /* blocks with ref > 1 */
    int64_t logical_tokens; /* sum of sequence lengths */
    int64_t table_slots;    /* sum over sequences of table length * block_size */
} pkv_stats;

/* init_order: host int32 [num_blocks] permutation or NULL (0, 1, 2, ...).
 * Returns NULL on invalid arguments or out of host memory. */
pkv_alloc* pkv_alloc_create(int num_blocks, int block_size, const int32_t* init_order);
void pkv_alloc_destroy(pkv_alloc* a);

/* New empty sequence.  PKV_ERR_INVALID if the id exists. */
int pkv_seq_add(pkv_alloc* a, int64_t seq);

/* Reserve slots for n new tokens.  slots_out: host int32 [n] (written).
 * copy_pairs_out: host int32 [copy_cap][2] receiving (src, dst) copies that
 * must be applied (pkv_copy_blocks) before the tokens are written; one append
 * produces at most one copy.  *num_copies_out gets the count.  A write into
 * a -1 entry (a block released by pkv_seq_trim and shared as a hole by a
 * fork) takes a fresh block there, as a write past the table does, with no
 * copy.  Atomic: on PKV_ERR_NO_BLOCKS or any error nothing changes. */
int pkv_seq_append(pkv_alloc* a, int64_t seq, int n, int32_t* slots_out, int32_t* copy_pairs_out,
                   int copy_cap, int* num_copies_out);

/* Prefix caching: append n tokens whose ids are known (host int32
 * tokens[n]).  cnblogs section 9: a prompt shared by many requests is stored
 * once; "08. PagedAttention", section "what else paging solves": only full
 * blocks are shared, by reference count.
 * Every full block of a sequence whose appends all carried token ids is
 * named by a chained hash: FNV-1a (64-bit) over the previous full block's
 * hash (8 bytes little endian; 0 before the first block) followed by the
 * block's token ids (4 bytes each, little endian).  A block this append
 * covers whole, whose hash and token ids match a cached block, reuses that
 * block (ref + 1; a cached block with count 0 is taken back off the free
 * list) as long as every earlier new block of the append did too; its
 * tokens get slot -1 in slots_out (their K/V are already in the cache:
 * pkv_kv_write skips negative slots) and are counted in *num_cached_out.
 * Hits are decided on the cache as it was before the call.  Other tokens
 * are placed as pkv_seq_append places them, copy-on-write included.  A
 * block filled by this append is filed under its hash unless the hash is
 * cached already.  A block that leaves the free list for any other reason
 * loses its cache entry.  A sequence that ever takes a plain pkv_seq_append
 * (or was forked inside a block) no longer takes part.  Atomic like
 * pkv_seq_append. */
int pkv_seq_append_tokens(pkv_alloc* a, int64_t seq, const int32_t* tokens, int n, int32_t* slots_out,
                          int* num_cached_out, int32_t* copy_pairs_out, int copy_cap, int* num_copies_out);

/* Sliding-window reclamation (intelliparadigm.com article, section 5.2):
 * release every block of the sequence that lies wholly before position
 * keep_from (logical blocks lb with (lb + 1) * block_size <= keep_from),
 * last first, as pkv_seq_free would; their table entries become -1 (a hole
 * that no kernel reads) and the length is unchanged.  *freed_out counts the
 * entries released by this call.  PKV_ERR_INVALID if keep_from is outside
 * [0, length]; PKV_ERR_STATE if the sequence is swapped out.  Forks share
 * holes as holes; swapping a trimmed sequence moves its live blocks only
 * (its block list carries -1 at the holes, which the swap kernels skip). */
int pkv_seq_trim(pkv_alloc* a, int64_t seq, int64_t keep_from, int* freed_out);

/* Number of blocks filed in the prefix cache. */
int pkv_prefix_cache_size(const pkv_alloc* a, int* entries_out);

/* child := first fork_pos tokens of parent, sharing its blocks.
 * PKV_ERR_INVALID for an unknown parent, an existing child or
 * fork_pos outside [0, len(parent)]. */
int pkv_seq_fork(pkv_alloc* a, int64_t parent, int64_t child, int fork_pos);

/* Release a sequence.  PKV_ERR_INVALID if unknown; PKV_ERR_STATE on a
 * reference-count underflow (never happens through this API). */
int pkv_seq_free(pkv_alloc* a, int64_t seq);

/* Swap a sequence out: blocks_out (host int32 [cap]) receives its table in
 * logical order -- the blocks to copy to host memory with pkv_swap_out
 * before they are reused -- and *num_out its length; the blocks are then
 * released exactly as pkv_seq_free would, and the sequence keeps its length
 * but holds no blocks.  Append, fork and pkv_build_block_tables on a swapped
 * sequence give PKV_ERR_STATE; pkv_seq_free drops it.
 * Swap it back in: takes *num_out fresh blocks off the free list (logical
 * order; PKV_ERR_NO_BLOCKS and no change if too few are free) and writes
 * them to blocks_out: host buffer i goes to block blocks_out[i]
 * (pkv_swap_in).  PKV_ERR_STATE if the sequence is not swapped out. */
int pkv_seq_swap_out(pkv_alloc* a, int64_t seq, int32_t* blocks_out, int cap, int* num_out);
int pkv_seq_swap_in(pkv_alloc* a, int64_t seq, int32_t* blocks_out, int cap, int* num_out);

int pkv_seq_len(const pkv_alloc* a, int64_t seq, int64_t* len_out);

/* Copy a sequence's table (host int32 [cap]); *len_out = its length in
 * blocks.  PKV_ERR_INVALID if cap is too small. */
int pkv_get_block_table(const pkv_alloc* a, int64_t seq, int32_t* out, int cap, int* len_out);

/* Padded batch export: tables_out host int32 [num_seqs][max_blocks_per_seq]
 * (pad -1), context_lens_out host int32 [num_seqs]. */
int pkv_build_block_tables(const pkv_alloc* a, const int64_t* seqs, int num_seqs,
                           int max_blocks_per_seq, int32_t* tables_out, int32_t* context_lens_out);

/* Groups of a batch for pkv_paged_attention_decode_shared (forks of one
 * prompt hold its blocks together: intelliparadigm.com article, section
 * 2.3).  Walking the batch in order, a group is a sequence and the ones
 * right after it whose first table entry is the same physical block, at
 * most max_members of them; its shared block count is the number of leading
 * table entries that are the same live block in every member and lie
 * wholly inside every member's context (0 for a one-member group).
 *   group_start_out    host int32 [num_seqs + 1] (num_groups + 1 written)
 *   shared_blocks_out  host int32 [num_seqs] (num_groups written)
 * PKV_ERR_INVALID for an unknown sequence, PKV_ERR_STATE for a swapped one. */
int pkv_shared_prefix_groups(const pkv_alloc* a, const int64_t* seqs, int num_seqs, int max_members,
                             int32_t* group_start_out, int32_t* shared_blocks_out, int* num_groups_out);

int pkv_alloc_stats(const pkv_alloc* a, pkv_stats* out);

/* Inspection for tests: reference count of a block; the free stack from top
 * to bottom (host int32 [cap]). */
int pkv_block_ref(const pkv_alloc* a, int block, int* ref_out);
int pkv_free_list(const pkv_alloc* a, int32_t* out, int cap, int* len_out);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */

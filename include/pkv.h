/*
 * pkv.h - paged KV cache with shared-prefix decode attention for AMD gfx950 (C ABI).
 *
 * Two device operations and the host bookkeeping that feeds them:
 *
 *   pkv_kv_append          write each new token's K/V into the slot named by a slot
 *                          mapping, after copying the valid rows of shared,
 *                          partly filled tail blocks (copy-on-write).
 *   pkv_paged_decode_attn  one query token per sequence attends to the sequence's
 *                          cached K/V through its block table (grouped-query heads);
 *                          optional cascade plan: blocks shared by several sequences
 *                          are read once for all of them.
 *
 *   pkv_pool_* / pkv_seq_* host block pool with reference counts, fork, append
 *                          planning (slots + copy-on-write list) and free.
 *   pkv_plan_*             host cascade planner: finds the blocks that several block
 *                          tables share and lays out the shared-prefix work.
 *   pkv_radix_*            host prefix cache: a radix tree of cached token runs and
 *                          their blocks, longest-prefix match, locks, LRU or
 *                          score/depth leaf eviction.
 *
 * Sources.  "The Reasoning Engine Meltdown" (atozofsoftwareengineering.blog):
 * §2.1 defines attention, softmax(Q K^T / sqrt(d_k)) V, the decode step (the new
 * query attends to all cached keys and values) and the KV-size formula
 * 2*L*H*d_h*S*P; §5 the page table with reference counts, zero-copy fork,
 * copy-on-write and free-on-zero; §6 the manager's API and error conventions.
 * "Dismantling the Memory Wall" (blog.bako.co): section "PagedAttention: The
 * Virtual Memory Analogy for GPUs" fixes 16-token blocks and the block table
 * (token t is in logical block t / block_size); section "Copy-on-Write and
 * Advanced Decoding Strategies" the sharing of prompt blocks among beams with a
 * new block only on divergence; section "RadixAttention" the longest shared
 * prefix reused across requests, which the cascade pass exploits.
 *
 * Conventions for every function:
 *   - Status codes are returned synchronously; on any non-OK status
 *     pkv_last_error() holds a message (thread-local, valid until the next call
 *     on the same thread).  Nothing is changed when a call fails.
 *   - Device pointers are caller-owned device memory (e.g. torch tensors).  The
 *     device calls enqueue work on `stream` (a hipStream_t; NULL = the default
 *     stream), never synchronize and never allocate device memory.
 *   - Pools and plans are library-owned host objects; destroy them explicitly.
 *     They are not thread-safe: one thread at a time per object.
 *   - dtype: PKV_F16 (IEEE binary16) or PKV_BF16; q, K and V share it.
 *   - Page layout: k_pages and v_pages are [num_blocks][block_size][num_kv_heads]
 *     [head_dim] elements, row-major; token slot s is block s / block_size, row
 *     s % block_size.
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
  PKV_ERR_INVALID = -1,     /* bad argument: null pointer, negative size, inconsistent shape */
  PKV_ERR_OOM = -2,         /* block pool exhausted; the pool is unchanged */
  PKV_ERR_NOT_FOUND = -3,   /* unknown sequence id where one is required (fork parent, append) */
  PKV_ERR_UNSUPPORTED = -4, /* dtype / head_dim / block_size / group not built into the library */
  PKV_ERR_HIP = -5,         /* the HIP runtime reported an error while enqueueing */
  PKV_ERR_WORKSPACE = -6    /* workspace smaller than pkv_decode_workspace_bytes() */
} pkv_status;

typedef enum { PKV_F16 = 0, PKV_BF16 = 1 } pkv_dtype;

/* Flags a decode call or-s into its optional device status word (see
 * pkv_paged_decode_attn): the call still returns a result, but not the definition's
 * for the rows concerned. */
typedef enum {
  PKV_STATUS_LEN_CLAMPED = 1, /* some seq_lens[b] outside [0, min(max_seq_len, max_blocks_per_seq*block_size)]:
                                 the row attended to the clamped length */
  PKV_STATUS_BAD_BLOCK = 2    /* some block id read from a table (or a plan node) outside [0, num_blocks):
                                 its tokens got zero weight */
} pkv_status_flag;

typedef struct pkv_pool pkv_pool;
typedef struct pkv_plan pkv_plan;
typedef struct pkv_radix pkv_radix;

/* Leaf eviction order of the prefix cache (pkv_radix_create). */
typedef enum {
  PKV_EVICT_LRU = 0,  /* least recently used first */
  PKV_EVICT_RSBCM = 1 /* lowest score / (depth + 1) first, then least recently used */
} pkv_evict_policy;

/* Message for the last non-OK status on this thread ("" if none). */
const char* pkv_last_error(void);

/* Library version string. */
const char* pkv_version(void);

/* ------------------------------------------------------------------------------------------
 * Device operation 1: append new tokens' K/V (with copy-on-write).
 *
 * Defined by "The Reasoning Engine Meltdown", §5 (writes land only in pages the
 * writer owns; a shared page is copied first) and "Dismantling the Memory Wall",
 * "Copy-on-Write and Advanced Decoding Strategies" (a branch gets its own block
 * when it diverges).  The copies and slots come from pkv_plan_append().
 *
 * Effect, in this order as far as the result is concerned:
 *   1. for c in [0, num_cow): rows [0, cow_rows[c]) of block cow_src[c] are copied
 *      to block cow_dst[c], for K and V, all heads;
 *   2. for i in [0, num_tokens): if slot_mapping[i] >= 0, token slot
 *      slot_mapping[i] of k_pages / v_pages is set to k_new[i] / v_new[i].
 * One launch does both: a plan from pkv_plan_append() never makes step 2 write a
 * row that step 1 reads or writes, so the two cannot race.  Slots < 0 are
 * skipped (padding); slots >= num_blocks*block_size and copies naming blocks
 * outside [0, num_blocks) or rows outside [0, block_size] are skipped by the
 * device (never written), so a bad plan cannot write out of bounds.
 *
 *   k_pages, v_pages  device, [num_blocks][block_size][num_kv_heads][head_dim], dtype
 *   k_new, v_new      device, [num_tokens][num_kv_heads][head_dim], dtype
 *   slot_mapping      device, int64 [num_tokens]
 *   cow_src, cow_dst, cow_rows  device, int32 [num_cow] (may be NULL when num_cow == 0)
 * Requirements: num_kv_heads*head_dim*2 bytes a multiple of 16; 16-byte aligned
 * pointers.  Errors: PKV_ERR_INVALID, PKV_ERR_UNSUPPORTED, PKV_ERR_HIP.
 * ---------------------------------------------------------------------------------------- */
pkv_status pkv_kv_append(void* k_pages, void* v_pages, int64_t num_blocks, int32_t block_size,
                         int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                         const void* k_new, const void* v_new, int32_t num_tokens,
                         const int64_t* slot_mapping,
                         const int32_t* cow_src, const int32_t* cow_dst, const int32_t* cow_rows,
                         int32_t num_cow, void* stream);

/* ------------------------------------------------------------------------------------------
 * Device operation 2: single-token decode attention over a paged KV cache.
 *
 * Defined by "The Reasoning Engine Meltdown", §2.1 (softmax(Q K^T / sqrt(d_k)) V;
 * the decode query attends to all cached K_{1:t}, V_{1:t}) and "Dismantling the
 * Memory Wall", "PagedAttention ..." (token t of row b is row t % block_size of
 * physical block block_tables[b][t / block_size]).
 *
 *   out[b][h][:] = sum_t softmax_t(scale * <q[b][h], K_b[t][h / group]>) * V_b[t][h / group]
 *
 * over t in [0, seq_lens[b]), group = num_q_heads / num_kv_heads (query head h
 * reads KV head h / group).  A row with seq_lens[b] == 0 gets out = 0.  Table
 * entries past ceil(seq_lens[b] / block_size) are never read.
 *
 *   q             device, [batch][num_q_heads][head_dim], dtype
 *   k_pages/v_pages  device, [num_blocks][block_size][num_kv_heads][head_dim], dtype
 *   block_tables  device, int32 [batch][max_blocks_per_seq]
 *   seq_lens      device, int32 [batch]
 *   max_seq_len   host int >= every seq_lens[b] (sizes the split grid; lengths above it
 *                 are clamped to it, and to max_blocks_per_seq*block_size, on the device)
 *   scale         softmax scale (1/sqrt(head_dim) for standard attention)
 *   plan          NULL: every row is decoded on its own (split-K over its tokens).
 *                 Non-NULL: a cascade plan built by pkv_plan_build() from the same
 *                 block tables and lengths and uploaded with pkv_plan_upload(); the
 *                 shared blocks are then read once per KV head for all rows sharing
 *                 them, and each row's own remainder is decoded split-K.
 *   workspace     device scratch of at least pkv_decode_workspace_bytes(...) bytes
 *                 (fp32 partial results); contents on entry are ignored.
 *   out           device, float32 [batch][num_q_heads][head_dim]
 *   status        device int32 word, or NULL: the call or-s PKV_STATUS_* flags into it
 *                 when an input is outside the definition's domain (a length clamped, a
 *                 block id out of range).  Never cleared by the call: zero it first to
 *                 see one call's flags.
 * Supported: block_size 16; head_dim 64 or 128; group in {1, 2, 4, 8}; num_blocks >= 1
 * when batch > 0.  Block ids outside [0, num_blocks) are never dereferenced: their
 * tokens get zero weight (block 0 is read in their place, so a block 0 holding
 * non-finite values could still reach the output) and PKV_STATUS_BAD_BLOCK is set.
 * With a plan, max_seq_len below the tokens its shared nodes cover is PKV_ERR_INVALID.
 * Errors: PKV_ERR_INVALID, PKV_ERR_UNSUPPORTED, PKV_ERR_WORKSPACE, PKV_ERR_HIP.
 * ---------------------------------------------------------------------------------------- */
pkv_status pkv_paged_decode_attn(const void* q, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t dtype,
                                 const void* k_pages, const void* v_pages, int64_t num_blocks,
                                 int32_t block_size,
                                 const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* seq_lens, int32_t max_seq_len, float scale,
                                 const pkv_plan* plan, void* workspace, size_t workspace_bytes,
                                 float* out, int32_t* status, void* stream);

/* Append and decode in one launch: pkv_kv_append of one new token per row (with the
 * copy-on-write of a partly filled shared last block) followed by pkv_paged_decode_attn,
 * as in "The Reasoning Engine Meltdown", §5 (a write lands only in a block its row
 * owns) and §2.1 (the decode query attends to every cached token, the new one included).
 *
 * block_tables and seq_lens are the tables AFTER the append (as pkv_plan_append and
 * pkv_export_tables leave them): row b's new token is its token seq_lens[b] - 1, in
 * row (seq_lens[b] - 1) % 16 of its last block D = block_tables[b][(seq_lens[b]-1)/16].
 *   k_new/v_new  device, [batch][num_kv_heads][head_dim], dtype, 16-byte aligned: the
 *                new token's K and V, written into that row of D.
 *   cow_src      device, int32 [batch]: the block D was copied from on write (rows
 *                [0, (seq_lens[b]-1) % 16) of cow_src[b] are copied into D), or -1.
 * Everything else as for pkv_paged_decode_attn (16-bit pages only); out equals
 * pkv_kv_append followed by pkv_paged_decode_attn up to float rounding order, and the
 * pages afterwards are bit-identical.  Rows with seq_lens[b] == 0, above max_seq_len or
 * above max_blocks_per_seq * 16 append nothing; copy-on-write sources outside
 * [0, num_blocks) are ignored.  A plan must come from the post-append tables: one that
 * puts a row's last token in a shared node is rejected with PKV_ERR_INVALID.  Workspace:
 * pkv_decode_workspace_bytes.  Errors: as pkv_paged_decode_attn. */
pkv_status pkv_paged_decode_attn_append(const void* q, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t dtype, void* k_pages, void* v_pages,
                                        int64_t num_blocks, int32_t block_size, const int32_t* block_tables,
                                        int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t max_seq_len,
                                        const void* k_new, const void* v_new, const int32_t* cow_src, float scale,
                                        const pkv_plan* plan, void* workspace, size_t workspace_bytes, float* out,
                                        int32_t* status, void* stream);

/* Bytes of device workspace pkv_paged_decode_attn needs for these sizes (and plan,
 * which may be NULL).  Returns 0 for invalid arguments (see pkv_last_error). */
size_t pkv_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t max_seq_len, const pkv_plan* plan);

/* pkv_paged_decode_attn for callers that cannot allocate device memory (code under
 * stream capture, tight serving loops, harnesses that forbid allocation): the same
 * computation and kernels, with the partial results in a fixed scratch array of
 * PKV_NOALLOC_SCRATCH_BYTES that the library holds on each device it runs on (from
 * its first use on that device until the process ends) instead of a caller workspace.
 * The caller still passes q, pages, tables, lengths, out (and the optional status
 * word); the call allocates nothing and calls no allocating routine.
 *   Limit: sizes whose pkv_decode_workspace_bytes(...) exceeds the scratch are refused
 *   with PKV_ERR_WORKSPACE before anything is enqueued.
 *   Sharing: every call on one device uses that device's one scratch array; calls whose
 *   execution overlaps on one device (other streams, other threads) race and must be
 *   ordered by the caller.  Nothing in the scratch needs clearing between calls.
 * Errors: as pkv_paged_decode_attn (PKV_ERR_HIP also when the scratch address cannot be
 * resolved). */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
pkv_status pkv_paged_decode_attn_noalloc(const void* q, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t dtype, const void* k_pages, const void* v_pages,
                                         int64_t num_blocks, int32_t block_size, const int32_t* block_tables,
                                         int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t max_seq_len,
                                         float scale, const pkv_plan* plan, float* out, int32_t* status,
                                         void* stream);

/* ------------------------------------------------------------------------------------------
 * Host block pool ("The Reasoning Engine Meltdown", §5 and §6).
 *
 * Blocks have reference counts.  The free list is a FIFO seeded by `free_order`
 * (a permutation of [0, num_blocks), NULL for 0, 1, 2, ...): allocation takes
 * from the front, freed blocks go to the back, in table order.  Sequence ids are
 * arbitrary int64 keys.  Not thread-safe.
 * ---------------------------------------------------------------------------------------- */

/* Returns NULL on invalid arguments (free_order not a permutation, sizes <= 0). */
pkv_pool* pkv_pool_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order);
void pkv_pool_destroy(pkv_pool* pool);

/* New root sequence of num_tokens tokens: ceil(num_tokens/block_size) blocks with
 * count 1.  PKV_ERR_OOM (nothing changed) if too few blocks are free;
 * PKV_ERR_INVALID if seq exists or num_tokens < 0. */
pkv_status pkv_seq_alloc(pkv_pool* pool, int64_t seq, int32_t num_tokens);

/* New sequence starting on cached blocks (a prefix-cache hit): its table is
 * prefix_blocks[0..num_prefix_blocks) (each count + 1; each must be allocated)
 * followed by fresh blocks up to ceil(num_tokens/block_size).  num_tokens must be
 * at least num_prefix_blocks*block_size.  PKV_ERR_OOM (nothing changed) if too few
 * blocks are free; PKV_ERR_INVALID for an existing seq or a bad prefix. */
pkv_status pkv_seq_alloc_prefix(pkv_pool* pool, int64_t seq, const int32_t* prefix_blocks,
                                int32_t num_prefix_blocks, int32_t num_tokens);

/* child gets a copy of parent's block table (a partly filled last block included)
 * and the same length; every block's count goes up by one; no KV data moves.
 * PKV_ERR_NOT_FOUND for an unknown parent, PKV_ERR_INVALID if child exists. */
pkv_status pkv_seq_fork(pkv_pool* pool, int64_t parent, int64_t child);

/* Drop the sequence: counts go down in table order, a block reaching 0 goes to
 * the back of the free list.  An unknown id is a no-op (PKV_OK). */
pkv_status pkv_seq_free(pkv_pool* pool, int64_t seq);

/* Append one token to each of seqs[0..n) in that order (a sequence at most once).
 * For each: pos = len; j = pos / block_size; off = pos % block_size;
 *   off == 0                 -> a new block is appended to the table;
 *   off > 0, count(t[j]) > 1 -> copy-on-write: a new block Y gets rows [0, off) of
 *                               t[j] (one entry of the cow_* outputs), count(t[j])
 *                               drops by one, t[j] = Y;
 *   slot_out[i] = t[j]*block_size + off; len += 1.
 * The batch is all-or-nothing: PKV_ERR_OOM with nothing changed if the free list
 * cannot cover it.  cow_src/cow_dst/cow_rows need room for n entries; *num_cow
 * receives the count.  row_cow_src (host int32 [n], may be NULL): entry i is the
 * block sequence i's last block was copied from on write in this batch, -1 if
 * none (the per-row form pkv_paged_decode_attn_append takes).
 * PKV_ERR_NOT_FOUND for an unknown id. */
pkv_status pkv_plan_append(pkv_pool* pool, const int64_t* seqs, int32_t n, int64_t* slot_out,
                           int32_t* cow_src, int32_t* cow_dst, int32_t* cow_rows, int32_t* num_cow,
                           int32_t* row_cow_src);

/* Write the block tables ([n][max_blocks], padded with -1) and lengths of seqs. */
pkv_status pkv_export_tables(const pkv_pool* pool, const int64_t* seqs, int32_t n, int32_t max_blocks,
                             int32_t* tables_out, int32_t* lens_out);

int32_t pkv_seq_len(const pkv_pool* pool, int64_t seq);     /* -1 if unknown */
/* Copy up to cap entries of seq's block table; returns its block count (-1 if unknown,
 * -2 if swapped out). */
int32_t pkv_seq_table(const pkv_pool* pool, int64_t seq, int32_t* out, int32_t cap);
int32_t pkv_refcount(const pkv_pool* pool, int32_t block);  /* -1 if out of range */
int32_t pkv_free_count(const pkv_pool* pool);
int32_t pkv_num_seqs(const pkv_pool* pool);
/* Copy up to cap free-list entries, front first; returns the free count. */
int32_t pkv_free_list(const pkv_pool* pool, int32_t* out, int32_t cap);

/* ------------------------------------------------------------------------------------------
 * Swap space ("Dismantling the Memory Wall", "Cross-Tier Memory Offloading": KV blocks
 * that overflow the GPU move down to CPU memory and are brought back before attention
 * needs them).
 *
 * The pool keeps host slots (one block each, in caller-owned pinned host buffers) with
 * their own FIFO free list.  A swap-out moves the blocks a sequence holds alone
 * (count 1), in table order, to host slots from the front of the host list and returns
 * those device blocks to the back of the device free list; blocks it shares stay on the
 * device with its reference.  A swap-in takes a device block from the front of the
 * device list for each host-resident entry and returns the slot to the back of the host
 * list.  Both are all-or-nothing (PKV_ERR_OOM with nothing changed) and return the
 * copies that pkv_copy_blocks must perform, on the stream that later reads or reuses
 * the blocks.  A swapped-out sequence cannot be appended to, forked, exported or cached
 * (PKV_ERR_INVALID); freeing it returns its host slots in table order and drops its
 * remaining device references.
 * ---------------------------------------------------------------------------------------- */

/* Once per pool: num_host_slots host slots, free list seeded by host_order (a
 * permutation, NULL for 0, 1, 2, ...).  PKV_ERR_INVALID if already set. */
pkv_status pkv_pool_set_host_slots(pkv_pool* pool, int32_t num_host_slots, const int32_t* host_order);

/* Copies (device_blocks_out[i] -> host_slots_out[i]), *num_copies of them; capacity
 * must cover the sequence's unshared blocks. */
pkv_status pkv_seq_swap_out(pkv_pool* pool, int64_t seq, int32_t* device_blocks_out, int32_t* host_slots_out,
                            int32_t capacity, int32_t* num_copies);
/* Copies (host_slots_out[i] -> device_blocks_out[i]). */
pkv_status pkv_seq_swap_in(pkv_pool* pool, int64_t seq, int32_t* host_slots_out, int32_t* device_blocks_out,
                           int32_t capacity, int32_t* num_copies);
int32_t pkv_seq_is_swapped(const pkv_pool* pool, int64_t seq);  /* 1, 0, or -1 if unknown */
/* Up to cap table entries (block ids, or host slots where on_host_out[i] = 1); returns
 * the entry count, -1 if unknown. */
int32_t pkv_seq_placement(const pkv_pool* pool, int64_t seq, int32_t* ids_out, int8_t* on_host_out, int32_t cap);
int32_t pkv_host_free_count(const pkv_pool* pool);
/* Copy up to cap host free-list entries, front first; returns the count. */
int32_t pkv_host_free_list(const pkv_pool* pool, int32_t* out, int32_t cap);

/* Device op: whole-block copies between two block arrays, each in device memory or in
 * pinned host memory (hipHostMalloc, torch pin_memory), e.g. K and V pages (and FP8
 * scale arrays) to and from host slot buffers.  For i < n and each array k <
 * num_arrays (1..4): block dst_ids[i] of dst[k] = block src_ids[i] of src[k],
 * block_bytes[k] bytes each (a positive multiple of 16; arrays 16-byte aligned;
 * dst[k] holds dst_blocks blocks, src[k] src_blocks).  dst, src and block_bytes are
 * host arrays of num_arrays entries; dst_ids and src_ids are int32 arrays of n
 * entries in device or pinned host memory.  Ids outside [0, dst_blocks) /
 * [0, src_blocks) are skipped; repeated destinations race.  Memory that HIP does not
 * know as device memory or as device-mapped host memory is refused
 * (PKV_ERR_INVALID).  max_workgroups > 0 caps the launch (the work-groups loop over
 * the blocks), leaving the rest of the chip to kernels that run beside the copy, e.g.
 * a prefetch on a second stream under decode; 0 launches one work-group per block
 * and array.  One launch on `stream`; no synchronization. */
pkv_status pkv_copy_blocks(int32_t num_arrays, void* const* dst, const void* const* src, const int64_t* block_bytes,
                           int64_t dst_blocks, int64_t src_blocks, const int32_t* dst_ids, const int32_t* src_ids,
                           int32_t n, int32_t max_workgroups, void* stream);

/* The same copies as runtime copies: one hipMemcpyAsync per run of consecutive ids on
 * both sides (the runtime picks the engine; ROCm 7 runs them as short blit kernels).
 * Many short copies interleave with a long kernel on another stream, where one
 * pkv_copy_blocks launch holding compute units would delay it: the prefetch path
 * under decode.  dst_ids / src_ids are HOST int32 arrays here; an id out of range is
 * PKV_ERR_INVALID (nothing enqueued).  Each run costs a host enqueue (about 10 us), so
 * scattered single blocks are slow to issue; host block arrays must be pinned. */
pkv_status pkv_copy_blocks_memcpy(int32_t num_arrays, void* const* dst, const void* const* src,
                               const int64_t* block_bytes, int64_t dst_blocks, int64_t src_blocks,
                               const int32_t* dst_ids, const int32_t* src_ids, int32_t n, void* stream);

/* ------------------------------------------------------------------------------------------
 * Prefix cache ("Dismantling the Memory Wall", "RadixAttention: The Tree of Life
 * for Agentic Swarms": a radix tree keeps the KV of finished requests, a new
 * request reuses its longest cached prefix, a request in flight locks its node and
 * the node's ancestors, and eviction takes least recently used unlocked leaves;
 * "RKSC - Reasoning-Aware KV Cache Sharing en Confident Early Exit", §2 C "RSBCM":
 * evict the lowest branch_score / (depth + 1) first).
 *
 * The tree caches whole blocks of a pool: keys are token ids compared in runs of
 * block_size, so a partly filled last block is never cached, and each cached
 * block holds one reference in the pool (it survives the sequences that wrote
 * it).  Node ids are int64 handles; the root is 0; ids are never reused.  Time is
 * a logical clock (one tick per match or insert).  Not thread-safe; destroy the
 * cache before its pool.
 * ---------------------------------------------------------------------------------------- */

/* NULL on a null pool or an unknown policy (pkv_evict_policy). */
pkv_radix* pkv_radix_create(pkv_pool* pool, int32_t policy);
/* Drops every cached block's reference (nodes in increasing id order), then frees. */
void pkv_radix_destroy(pkv_radix* cache);
/* Same release as destroy; the cache stays usable and empty. */
pkv_status pkv_radix_clear(pkv_radix* cache);

/* Longest cached prefix of tokens[0..num_tokens), in whole blocks.  Where the match
 * ends inside a node, the node is split there (the new upper node gets a new id),
 * so *node_out ends exactly at the match (0 if nothing matched).  Every node on the
 * path gets the current time.  *matched_tokens = matched blocks * block_size;
 * blocks_out (optional; room for num_tokens/block_size ids) gets their block ids.
 * A caller that must compute at least one token passes num_tokens - 1. */
pkv_status pkv_radix_match(pkv_radix* cache, const int32_t* tokens, int32_t num_tokens, int32_t* matched_tokens,
                           int32_t* blocks_out, int32_t blocks_cap, int64_t* node_out);

/* Cache the full blocks of a sequence: tokens[0..num_tokens) with its block table
 * blocks[0..num_blocks) (num_blocks >= num_tokens/block_size; each of those blocks
 * allocated in the pool).  Where the path is cached the tree keeps its own blocks
 * (the caller's duplicates stay the caller's); the rest becomes one new leaf under
 * the last matched node and the tree takes one pool reference per adopted block.
 * Path nodes take the current time and max(score, their score); the new leaf takes
 * (score, depth).  *node_out: the node that ends at the last full block;
 * *adopted_out: blocks adopted.  score must be finite, depth >= 0. */
pkv_status pkv_radix_insert(pkv_radix* cache, const int32_t* tokens, int32_t num_tokens, const int32_t* blocks,
                            int32_t num_blocks, double score, int32_t depth, int64_t* node_out,
                            int32_t* adopted_out);

/* lock_ref + 1 / - 1 on the node and every ancestor below the root (a locked node is
 * never evicted).  Unlock of an unlocked node is PKV_ERR_INVALID with nothing
 * changed; an unknown id is PKV_ERR_NOT_FOUND. */
pkv_status pkv_radix_lock(pkv_radix* cache, int64_t node);
pkv_status pkv_radix_unlock(pkv_radix* cache, int64_t node);

/* Branch score for the RSBCM order: the node's score becomes `score` and every
 * ancestor's is raised to at least `score`. */
pkv_status pkv_radix_set_score(pkv_radix* cache, int64_t node, double score);

/* Remove unlocked leaves one at a time, in the cache's policy order (ties: smaller
 * id), until num_blocks blocks went back to the pool's free list or no unlocked
 * leaf is left.  Removing a leaf drops the tree's reference on each of its blocks
 * in key order (blocks still used by sequences stay allocated) and may make its
 * parent a leaf.  *released_out: blocks that reached the free list; the first
 * evicted_cap evicted ids go to evicted_out, *num_evicted_out counts all. */
pkv_status pkv_radix_evict(pkv_radix* cache, int32_t num_blocks, int32_t* released_out, int64_t* evicted_out,
                           int32_t evicted_cap, int32_t* num_evicted_out);

/* Batched admission for a scheduler, one call per batch.  Request i is the token run
 * tokens[offsets[i] .. offsets[i+1]) (at least one token) and becomes sequence
 * seqs[i] (new ids, no repeats).  In order, each request matches all but its last
 * token, locks the match, evicts (blocks needed - free blocks) when the pool is short,
 * and starts its sequence on the matched blocks plus fresh ones; the first request
 * that still does not fit is unlocked and ends the batch.  matched_out / node_out get
 * the matched tokens and the locked node of each admitted request; *num_admitted
 * counts them (a short count is not an error).  The caller writes K/V for positions
 * from matched_out[i] on (pkv_seq_table gives the slots). */
pkv_status pkv_radix_admit(pkv_radix* cache, const int32_t* tokens, const int64_t* offsets, int32_t n,
                           const int64_t* seqs, int32_t* matched_out, int64_t* node_out, int32_t* num_admitted);

/* Batched completion: for each i, cache sequence seqs[i]'s full blocks under the token
 * run tokens[offsets[i] .. offsets[i+1]) (at most the sequence's length) with
 * scores[i] / depths[i] (NULL: 0), unlock nodes[i] (its admission node) and free the
 * sequence.  Every entry is checked first; on an error nothing changes. */
pkv_status pkv_radix_finish(pkv_radix* cache, const int32_t* tokens, const int64_t* offsets, int32_t n,
                            const int64_t* seqs, const int64_t* nodes, const double* scores, const int32_t* depths);

int32_t pkv_radix_num_nodes(const pkv_radix* cache);       /* the root included */
int32_t pkv_radix_cached_blocks(const pkv_radix* cache);   /* blocks the tree references */
int32_t pkv_radix_evictable_blocks(const pkv_radix* cache); /* blocks in nodes with lock_ref 0 */
/* Copy up to cap node ids in increasing order; returns the node count. */
int32_t pkv_radix_node_ids(const pkv_radix* cache, int64_t* out, int32_t cap);
/* A node's parent (-1 for the root), lock_ref, last access time, score, depth,
 * number of blocks, block ids and tokens (outputs optional; blocks_out needs room
 * for the block count, tokens_out for block count * block_size). */
pkv_status pkv_radix_node_info(const pkv_radix* cache, int64_t node, int64_t* parent, int32_t* lock_ref,
                               int64_t* last_access, double* score, int32_t* depth, int32_t* num_blocks,
                               int32_t* blocks_out, int32_t blocks_cap, int32_t* tokens_out, int32_t tokens_cap);

/* ------------------------------------------------------------------------------------------
 * Cascade planner ("Dismantling the Memory Wall", "RadixAttention": a prefix tree
 * of shared token sequences whose KV is referenced, not copied; "The Reasoning
 * Engine Meltdown", §5: branches point at the same physical pages).
 *
 * From host copies of the block tables and lengths, build a trie over (logical
 * block index, physical block id).  Every maximal run of *full* blocks that the
 * same set of >= min_members rows shares becomes a node; each row's blocks after
 * its last node are its private remainder.  The decode then reads each node's
 * blocks once per KV head for all of its rows (matrix-core pass) and writes one
 * partial result per (row, head, node), merged with the remainder's partials.
 * ---------------------------------------------------------------------------------------- */

/* Returns NULL on invalid arguments (see pkv_last_error).  min_members >= 2. */
pkv_plan* pkv_plan_build(const int32_t* block_tables, const int32_t* seq_lens, int32_t batch,
                         int32_t max_blocks_per_seq, int32_t block_size, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t min_members);
void pkv_plan_destroy(pkv_plan* plan);

/* Bytes of device memory the plan's tables need. */
size_t pkv_plan_device_bytes(const pkv_plan* plan);

/* Copy the plan's tables into caller-owned device memory `device_buf` (at least
 * pkv_plan_device_bytes bytes) on `stream` and bind it to the plan.  The copy is
 * ordered on `stream`; later decode calls on other streams must be ordered
 * after it by the caller. */
pkv_status pkv_plan_upload(pkv_plan* plan, void* device_buf, size_t bytes, void* stream);

/* Plan inspection (host): number of shared nodes, shared tokens summed over
 * nodes, tokens each row reads through nodes. */
int32_t pkv_plan_num_nodes(const pkv_plan* plan);
/* For node i: number of blocks, number of member rows; copies its block ids and
 * member rows into the given arrays when non-NULL (sized by the returned counts). */
pkv_status pkv_plan_node(const pkv_plan* plan, int32_t node, int32_t* num_blocks, int32_t* num_members,
                         int32_t* blocks_out, int32_t* members_out);
/* Token pieces node i is cut into (each piece is a separate work item and a
 * separate partial per member row and query head); -1 for a bad index. */
int32_t pkv_plan_node_pieces(const pkv_plan* plan, int32_t node);
/* For query row r (a sequence for a decode plan, a query token for an extend
 * plan): tokens covered by its shared nodes (a decode row's remainder starts
 * there) and the number of partial slots its nodes use. */
pkv_status pkv_plan_row(const pkv_plan* plan, int32_t row, int32_t* shared_tokens, int32_t* depth);

/* ------------------------------------------------------------------------------------------
 * FP8 pages.  "The Reasoning Engine Meltdown" names FP8 (and FP4) quantization of
 * the KV cache among the ways to fit deep search trees in memory (§3, and its
 * closing outlook); the format and granularity are this library's choice:
 *   - codes: OCP E4M3 ("fn": largest finite 448, subnormals down to 2^-9), one byte
 *     per element, k_pages / v_pages [num_blocks][block_size][num_kv_heads][head_dim];
 *   - scales: float32 [num_blocks][num_kv_heads][block_size], one per token row and
 *     KV head, a power of two 2^k with k the smallest integer (clamped to
 *     [-126, 127]) such that max|x| / 2^k <= 448 over the head vector (k = 0 for an
 *     all-zero vector); a code's value times its scale is the stored element;
 *   - an appended token's head vector x is stored as round-to-nearest-even(x / 2^k)
 *     (exact scaling, then the nearest E4M3 value, ties to even), so appending never
 *     re-quantizes earlier rows.
 * Halves the KV bytes the decode streams.
 * ---------------------------------------------------------------------------------------- */

/* As pkv_kv_append, for FP8 pages: copy-on-write copies codes and scales of rows
 * [0, cow_rows[c]); each new token (k_new / v_new [num_tokens][num_kv_heads][head_dim]
 * in src_dtype, PKV_F16 or PKV_BF16) is quantized into its slot.  head_dim 64 or
 * 128.  Errors: PKV_ERR_INVALID, PKV_ERR_UNSUPPORTED, PKV_ERR_HIP. */
pkv_status pkv_kv_append_fp8(void* k_pages, void* v_pages, float* k_scales, float* v_scales, int64_t num_blocks,
                             int32_t block_size, int32_t num_kv_heads, int32_t head_dim, int32_t src_dtype,
                             const void* k_new, const void* v_new, int32_t num_tokens, const int64_t* slot_mapping,
                             const int32_t* cow_src, const int32_t* cow_dst, const int32_t* cow_rows, int32_t num_cow,
                             void* stream);

/* As pkv_paged_decode_attn, over FP8 pages: K and V elements are code value x scale;
 * q is q_dtype (PKV_F16 or PKV_BF16) and the arithmetic is that of the 16-bit path
 * (every E4M3 value is exact in both 16-bit types).  With a cascade plan the shared
 * blocks go through the matrix-core pass, their codes widened to q's type in LDS, the
 * K scale applied to each score and the V scale folded into each weight.  With q in
 * f16 that weight (at most 2^8 times the V scale) is held in f16 for the matrix-core
 * products: V scales up to 2^8, which is what pkv_kv_append_fp8 writes from f16 data,
 * keep it finite, and a product above the largest finite f16 is clamped to it.  The
 * scale arrays must be 16-byte aligned (a token group's four scales are read as one
 * vector).  Workspace: pkv_decode_workspace_bytes(..., plan).  Errors as
 * pkv_paged_decode_attn. */
pkv_status pkv_paged_decode_attn_fp8(const void* q, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t q_dtype, const void* k_pages, const void* v_pages,
                                     const float* k_scales, const float* v_scales, int64_t num_blocks,
                                     int32_t block_size, const int32_t* block_tables, int32_t max_blocks_per_seq,
                                     const int32_t* seq_lens, int32_t max_seq_len, float scale, const pkv_plan* plan,
                                     void* workspace, size_t workspace_bytes, float* out, int32_t* status,
                                     void* stream);

/* ------------------------------------------------------------------------------------------
 * Device operation 3: multi-token (extend) attention over a paged KV cache.
 *
 * Several new tokens per sequence, each attending causally to its sequence's
 * cache: the verification pass of "RKSC" (gist.science summary, §1: a generated
 * branch is scored with one forward pass over its tokens, while branches share
 * their prefix) and "Dismantling the Memory Wall", "Chunked Prefill" (a prompt
 * is processed in token slices, each slice attending to what is cached before
 * it).  Row b's q_lens[b] new tokens are the last q_lens[b] of its seq_lens[b]
 * cached tokens (they were appended first); query token i of row b, at position
 * p = seq_lens[b] - q_lens[b] + i, gets
 *
 *   out[r][h][:] = sum_{t <= p} softmax_t(scale * <q[r][h], K_b[t][h / group]>) V_b[t][h / group]
 *
 * with r = q_lens[0] + ... + q_lens[b-1] + i (query rows packed in row order).
 * All of it runs on the matrix cores: blocks that several rows share are read
 * once for all of their query tokens (as in the decode cascade), and each row's
 * remaining blocks once for all of its own query tokens.
 *
 * The plan (pkv_plan_build_extend, then pkv_plan_upload) carries the block ids,
 * so the call takes no tables:
 *   q            device, [num_query_rows][num_q_heads][head_dim], dtype
 *   k_pages/v_pages  device, [num_blocks][block_size][num_kv_heads][head_dim], dtype
 *   workspace    device scratch of at least pkv_extend_workspace_bytes(plan, head_dim)
 *                bytes; contents on entry are ignored
 *   out          device, float32 [num_query_rows][num_q_heads][head_dim]
 * Supported: block_size 16; head_dim 64 or 128; group in {1, 2, 4, 8}.
 * Errors: PKV_ERR_INVALID, PKV_ERR_UNSUPPORTED, PKV_ERR_WORKSPACE, PKV_ERR_HIP.
 * ---------------------------------------------------------------------------------------- */
pkv_status pkv_paged_extend_attn(const void* q, int32_t num_query_rows, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t dtype, const void* k_pages, const void* v_pages,
                                 int64_t num_blocks, int32_t block_size, float scale, const pkv_plan* plan,
                                 void* workspace, size_t workspace_bytes, float* out, void* stream);

/* As pkv_paged_extend_attn, over FP8 pages (codes as for pkv_paged_decode_attn_fp8,
 * scales float32 [num_blocks][num_kv_heads][block_size], 16-byte aligned); q is
 * q_dtype (PKV_F16 or PKV_BF16).  Codes are widened to q's type in LDS (exact), the K
 * scale multiplies each score, the V scale each weight. */
pkv_status pkv_paged_extend_attn_fp8(const void* q, int32_t num_query_rows, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t q_dtype, const void* k_pages, const void* v_pages,
                                     const float* k_scales, const float* v_scales, int64_t num_blocks,
                                     int32_t block_size, float scale, const pkv_plan* plan, void* workspace,
                                     size_t workspace_bytes, float* out, void* stream);

/* Plan for pkv_paged_extend_attn from host copies of the block tables
 * ([batch][max_blocks_per_seq]), lengths and query-token counts (0 <= q_lens[b]
 * <= seq_lens[b]; rows with q_lens[b] == 0 take no part).  Shared nodes are
 * found as in pkv_plan_build among the rows with query tokens.  Returns NULL on
 * invalid arguments (see pkv_last_error). */
pkv_plan* pkv_plan_build_extend(const int32_t* block_tables, const int32_t* seq_lens, const int32_t* q_lens,
                                int32_t batch, int32_t max_blocks_per_seq, int32_t block_size, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t min_members);

/* Bytes of device workspace pkv_paged_extend_attn needs with this plan (0 and
 * an error for a decode plan). */
size_t pkv_extend_workspace_bytes(const pkv_plan* plan, int32_t head_dim);

/* Query rows of a plan: the batch for a decode plan, the summed q_lens for an
 * extend plan; -1 for NULL. */
int32_t pkv_plan_num_query_rows(const pkv_plan* plan);

/* The plan's device image (what pkv_plan_upload copies), for inspection on the
 * host: copies it into out when capacity (int32 entries) suffices, writes the
 * offsets of its sections (row info, nodes, node blocks, members, items) and the
 * partial slots per query row into offsets[0..5], and returns the image length
 * (-1 for NULL).  Node records are 8 ints (block offset, blocks, member offset,
 * members, pieces, blocks per piece, first token position, tokens holding data),
 * member entries 3 (query row, slot of piece 0, last attended position or
 * INT32_MAX), work items 4 (node or -1, KV head, first tile row, piece). */
int64_t pkv_plan_image(const pkv_plan* plan, int32_t* out, int64_t capacity, int64_t* offsets);

/* Query rows of one work item of the plan's matrix-core pass (a work item's first
 * row is a multiple of it): 64 for decode plans, 128 for extend plans. -1 for NULL. */
int32_t pkv_plan_rows_per_item(const pkv_plan* plan);

/* Where the plan's device image holds the work-item records the matrix-core pass
 * reads (the same work items as the items section, each made self-contained so that
 * a work-group's first K/V and query loads need one read of its record): returns the
 * record section's offset in int32 entries (a multiple of 4) and stores the ints per
 * record in *ints_per_item (if non-NULL); -1 for NULL.  A record is a 16-int header
 * (KV head or -1 for an idle item, first tile row, piece, index of the piece's first
 * block in the node-block section, blocks in the piece, query rows of the node, logical
 * position of the piece's first token, tokens of the piece holding data, the ids of the
 * piece's first 4 blocks or -1, 4 zeros), then 4 ints per member row of the tile
 * (query row or -1 past the node's members, partial slot of this piece, last attended
 * position or INT32_MAX, 0).  An idle item's record has head -1, no blocks, no rows,
 * ids -1 and every member row -1.  For inspection; the layout follows the plan's kind and
 * may change with the library version. */
int64_t pkv_plan_item_records(const pkv_plan* plan, int32_t* ints_per_item);

/* ------------------------------------------------------------------------------------------
 * Kernel timing (for measurement).  When enabled, every kernel launch of the
 * library is bracketed with HIP events on its own stream; pkv_timing_read()
 * synchronizes those events and returns the summed duration and count per
 * kernel since the last reset.  Kernel ids: 0 append, 1 split-K decode,
 * 2 partial merge, 3 cascade / extend matrix-core pass, 4 block copy.  Costs two
 * event records per launch when on.
 * ---------------------------------------------------------------------------------------- */
/* Measurement yardstick: read `bytes` (a multiple of 16) of device memory `buf` as
 * a plain streaming read (16-byte loads, `grid` work-groups of 256 threads; 0 picks
 * 2048) on `stream`.  `sink` (one device uint32) is written only in a case that
 * practically never happens.  Time it with events to get the chip's read-stream
 * ceiling beside the decode kernels' rates. */
pkv_status pkv_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int32_t grid, void* stream);

enum { PKV_KERNEL_APPEND = 0, PKV_KERNEL_DECODE_SPLIT = 1, PKV_KERNEL_MERGE = 2, PKV_KERNEL_CASCADE = 3,
       PKV_KERNEL_COPY = 4, PKV_NUM_KERNELS = 5 };
pkv_status pkv_timing_enable(int32_t on);
pkv_status pkv_timing_reset(void);
pkv_status pkv_timing_read(int32_t kernel, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */

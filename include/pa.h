/*
 * pa.h -- paged KV-cache attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libpa.so: a slot-mapped store of new keys/values into a cache made
 * of fixed-size blocks, paged decode attention (one query token per sequence,
 * or a few with causal masking among them) and causal varlen prefill
 * attention over the same paged cache, whole-block copies (copy-on-write
 * inside a pool, swap between pools), and the host-side block manager that
 * produces block tables and slot mappings.
 *
 * What the operations compute (no code is taken from these sources):
 *   - nano-vllm hub page (pomoai.com), section "Attention + Triton Kernel":
 *     keys/values computed for new tokens are written into preallocated cache
 *     blocks through a per-token slot mapping;
 *   - same page, section "KV Cache block management": blocks hold a fixed
 *     256 tokens;
 *   - CSDN essay comparing nanoVLLM and vLLM, first section (KV-cache
 *     management): a per-sequence block table maps logical blocks to physical
 *     blocks that need not be contiguous; a new block is taken when a sequence
 *     reaches 256k+1 tokens, so a sequence of n tokens owns ceil(n/256) blocks;
 *   - same essay, third section (attention computation): the attention is the
 *     exact softmax(scale * q K^T) V, computed in tiles kept on chip;
 *   - same essay, reading vLLM's attention module: prefill (many tokens per
 *     sequence, compute-bound) and decode (one token per sequence, bound by
 *     reading the cache) are separate kernels.
 *
 * Conventions shared by every entry point
 *   bf16        : IEEE bfloat16, passed as raw 16-bit patterns.
 *   D           : head_dim; only 128 is supported.
 *   block_size  : tokens per cache block; only 256 is supported.
 *   Hkv, Hq     : key/value heads and query heads; G = Hq / Hkv must be
 *                 1, 2, 4 or 8 and query head h reads kv head h / G
 *                 (contiguous grouped-query heads).
 *   slot        : a cache position; slot s is row (s % block_size) of physical
 *                 block (s / block_size).
 *   K cache     : bf16 [num_blocks][Hkv][D/8][block_size][8]; element (slot s,
 *                 kv head g, dim d) sits at
 *                 ((((s/bs)*Hkv + g)*(D/8) + d/8)*bs + s%bs)*8 + d%8.
 *                 Each 16-byte chunk holds 8 consecutive dims of one token, and
 *                 one block-head is one contiguous 64 KiB tile.
 *   V cache     : bf16 [num_blocks][Hkv][block_size][D]; element (s, g, d) sits
 *                 at (((s/bs)*Hkv + g)*bs + s%bs)*D + d.
 *   block_table : int32 [batch][max_blocks_per_seq], row-major; entry
 *                 [b][j] is the physical block of tokens j*bs .. j*bs+bs-1 of
 *                 sequence b.  Only the first ceil(context_lens[b]/bs) entries
 *                 of a row are read.
 *
 * Memory and streams
 *   Every array argument of a GPU call is a DEVICE pointer owned by the
 *   caller (host arrays are marked as such: the validators, pa_swap_blocks'
 *   pair list, the block manager).  The GPU calls allocate nothing; the
 *   library keeps only cached device attributes, the debug-check switch and
 *   the fixed per-device scratch array of pa_decode_append_noalloc, and is
 *   thread-safe (a block manager serialises its own calls; overlapping
 *   pa_decode_append_noalloc calls on one device are the exception).  Every call is
 *   asynchronous on `stream` (a hipStream_t passed as void*; NULL = the null
 *   stream) on the current device.  The caller orders a store before the
 *   attention that reads it by issuing both on one stream.
 *
 * Errors
 *   Entry points return PA_OK or a negative PA_ERR_* code.  All argument checks
 *   run on the host before anything is launched; on an error nothing is
 *   launched and pa_last_error_detail() describes it (thread-local).  An empty
 *   batch (num_tokens == 0, batch == 0) is a successful no-op.  No C++
 *   exception crosses the ABI.
 *
 * Data preconditions (not checked on the host -- pa_set_debug_checks turns on
 * device-side checks of them; device code never reads or writes outside the
 * arrays whatever the data, but the affected outputs are then unspecified):
 *   - slots are < num_blocks*block_size (a negative slot means "skip");
 *   - no two tokens of one pa_store_kv call share a slot;
 *   - block_table entries that are read lie in [0, num_blocks);
 *   - 0 <= context_lens[b] <= max_blocks_per_seq*block_size;
 *   - for prefill, 0 <= q_len_b <= context_lens[b].
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_BLOCK_SIZE 256
#define PA_HEAD_DIM 128
#define PA_K_CHUNK 8

enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL_PTR = -1,      /* a required pointer is NULL */
  PA_ERR_BAD_SHAPE = -2,     /* negative sizes, Hq % Hkv != 0, ... */
  PA_ERR_UNSUPPORTED = -3,   /* head_dim != 128, block_size != 256, G not 1/2/4/8 */
  PA_ERR_ALIGN = -4,         /* a bf16 array is not 16-byte aligned */
  PA_ERR_WORKSPACE = -5,     /* workspace missing or too small */
  PA_ERR_HIP = -6,           /* the HIP runtime reported an error */
  PA_ERR_SLOT_RANGE = -7,    /* pa_validate_slots: a slot >= num_slots */
  PA_ERR_DUPLICATE_SLOT = -8, /* pa_validate_slots: two tokens share a slot */
  PA_ERR_BLOCK_CONFLICT = -9, /* pa_validate_block_pairs: a block written twice, or read and written */
  PA_ERR_NO_BLOCKS = -10,     /* block manager: not enough free blocks */
  PA_ERR_PRECONDITION = -11   /* debug checks: a data-dependent precondition is violated */
};

/*
 * pa_store_kv -- write each new token's keys and values into its cache slot.
 *
 * For every i < num_tokens with slot_mapping[i] >= 0, copies the bits of
 * k_new[i][g][0..D) into the K cache and v_new[i][g][0..D) into the V cache at
 * slot slot_mapping[i], for every kv head g.  Tokens whose slot is negative
 * are skipped.  A bit copy: the cache afterwards holds exactly the input bits.
 *
 *   k_new, v_new  : bf16 [num_tokens][num_kv_heads][head_dim], 16-B aligned.
 *   slot_mapping  : int32 [num_tokens].
 *   k_cache, v_cache : the pools, layouts above, num_blocks blocks each.
 *   Source: nano-vllm hub page, "Attention + Triton Kernel" (slot mapping into
 *   preallocated blocks); CSDN essay, first section (block table).
 */
int pa_store_kv(const void* k_new, const void* v_new, const int32_t* slot_mapping,
                int64_t num_tokens, void* k_cache, void* v_cache, int64_t num_blocks,
                int32_t block_size, int32_t num_kv_heads, int32_t head_dim, void* stream);

/*
 * pa_decode_workspace_size -- bytes of device workspace pa_decode needs for a
 * batch of this shape on the current device (split-context partial results).
 * Returns 0 for shapes pa_decode would reject.
 */
size_t pa_decode_workspace_size(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size);

/*
 * pa_decode -- attention of one new query token per sequence over its whole
 * paged context.
 *
 * For sequence b and query head h (kv head g = h / G), with n = context_lens[b]
 * and K_b[j], V_b[j] the cached key/value of position j (read through
 * block_table[b]):
 *   s_j = scale * <q[b][h], K_b[j][g]>   for j < n
 *   out[b][h] = sum_j exp(s_j - max s) V_b[j][g] / sum_j exp(s_j - max s)
 * rounded to bf16 (nearest even) from fp32 accumulators.  n == 0 gives a zero
 * row.  The new token must already be stored (pa_store_kv on the same stream).
 * Long contexts are cut into chunks whose partial (max, sum, weighted V) states
 * are merged; the result does not depend on the cut beyond rounding.
 *
 *   out           : bf16 [batch][num_q_heads][head_dim], 16-B aligned.
 *   q             : bf16 [batch][num_q_heads][head_dim], 16-B aligned.
 *   k_cache, v_cache, block_table : see above; max_blocks_per_seq = row length.
 *   context_lens  : int32 [batch].
 *   max_context_len : an upper bound of context_lens used to size the launch
 *                   (must be <= max_blocks_per_seq*block_size).
 *   scale         : the logit scale (e.g. 1/sqrt(head_dim)); finite.
 *   workspace     : >= pa_decode_workspace_size(...) bytes of device memory,
 *                   256-B aligned.  It holds partial results from its start
 *                   (scratch, no clearing needed) and one arrival counter per
 *                   (sequence, kv head) at its end, which must be zero before
 *                   the first call (zero-fill the whole workspace once) and
 *                   which every call resets to zero.  A workspace sized for
 *                   the largest call of a series (batch, heads) serves every
 *                   call of the series, in any order, when every call passes
 *                   the same workspace_bytes (the allocation's size: the
 *                   counters' place is taken from it).  Calls that overlap in
 *                   time must not share a workspace.
 *   Source: CSDN essay, first and third sections; vLLM decode kernel
 *   description in the same essay.
 */
int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_table, int32_t max_blocks_per_seq,
              const int32_t* context_lens, int32_t batch, int32_t max_context_len,
              int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
              int64_t num_blocks, float scale, void* workspace, size_t workspace_bytes,
              void* stream);

/*
 * pa_decode_append -- one decode step in one launch: the store of each
 * sequence's new token and the decode attention over its context.
 *
 * For sequence b with n = context_lens[b] >= 1 (n counts the new token), the
 * token at position n-1 is new: its rows k_new[b], v_new[b] are written into
 * the caches at slot block_table[b][(n-1)/block_size]*block_size +
 * (n-1)%block_size, and out[b] is pa_decode's result over positions 0 .. n-1
 * with that position's key and value taken from k_new / v_new.  The result
 * equals pa_store_kv (with those slots) followed by pa_decode, up to rounding
 * order: positions 0 .. n-2 are read from the cache and the new token is
 * folded in as one more partial state; nothing reads position n-1 of the
 * cache during the call.  n == 0: a zero row and nothing stored.  A position
 * whose block-table entry lies outside the pool contributes nothing and is
 * not stored (as pa_decode and pa_store_kv treat such blocks).
 *
 *   k_new, v_new  : bf16 [batch][num_kv_heads][head_dim], 16-B aligned, not
 *                   NULL when batch > 0.
 *   k_cache, v_cache : the pools, written at the new positions.
 *   workspace     : >= pa_decode_workspace_size(...) bytes; same rules as
 *                   pa_decode's workspace.
 *   Other arguments as for pa_decode.
 *   Source: nano-vllm hub page, "Attention + Triton Kernel" (store through the
 *   slot mapping, then attend) and "KV Cache block management" (the slot
 *   formula); CSDN essay, first and third sections (the decode kernel).
 */
int pa_decode_append(void* out, const void* q, const void* k_new, const void* v_new, void* k_cache,
                     void* v_cache, const int32_t* block_table, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, int32_t batch, int32_t max_context_len,
                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                     int64_t num_blocks, float scale, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * pa_decode_append_noalloc -- pa_decode_append without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  It
 * allocates nothing: the partial records and arrival counters live in a
 * library-owned device array of PA_DECODE_NOALLOC_SCRATCH_BYTES bytes, which
 * every device the library runs on holds from the library's load until the
 * process ends.  The first call on a device clears it with a kernel on
 * `stream` (no memset); every call leaves its counters at zero again.
 *
 * Same arguments (minus the workspace), results and cache writes as
 * pa_decode_append.  A batch whose workspace (pa_decode_workspace_size)
 * exceeds the array -- about 750 sequences at 8 kv heads and up to 4 q heads
 * per kv head, fewer at 8 -- returns PA_ERR_WORKSPACE with nothing launched.
 * All calls on one device share the one array: calls that overlap in time
 * on one device (concurrent streams or threads) race and must not be made.
 */
#define PA_DECODE_NOALLOC_SCRATCH_BYTES 16777216
int pa_decode_append_noalloc(void* out, const void* q, const void* k_new, const void* v_new,
                             void* k_cache, void* v_cache, const int32_t* block_table,
                             int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t batch,
                             int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale,
                             void* stream);

/*
 * pa_decode_multi -- decode of q_per_seq new tokens per sequence at once
 * (speculative verification: the drafted tokens and the next one scored in
 * one pass), each attending causally to the cache.
 *
 * Query row i (0 <= i < q_per_seq) of sequence b is the token at position
 * context_lens[b] - q_per_seq + i and attends to the cached positions
 * 0 .. context_lens[b] - q_per_seq + i of its sequence (the same bottom-right
 * causal rule as pa_prefill; the K/V of all context_lens[b] positions,
 * including the new tokens, must already be in the cache).  Softmax and
 * rounding as in pa_decode; q_per_seq = 1 is exactly pa_decode.
 *
 *   out, q        : bf16 [batch * q_per_seq][num_q_heads][head_dim], row
 *                   b * q_per_seq + i, 16-B aligned.
 *   q_per_seq     : 1 .. 32, with q_per_seq * num_q_heads / num_kv_heads <= 32
 *                   (else PA_ERR_UNSUPPORTED): the rows of one (sequence, kv
 *                   head) are processed together -- up to 4 like the query
 *                   heads of one kv head in pa_decode (q_per_seq = 1: up to
 *                   8), 5 to 16 as one block of 16 rows and 17 to 32 as one
 *                   block of 32 rows on the matrix cores (P rounded to bf16
 *                   before P.V, as in pa_prefill).
 *   context_lens  : int32 [batch], each >= q_per_seq for meaningful rows (a
 *                   row whose position is negative sees no key and is zero).
 *   workspace     : >= pa_decode_multi_workspace_size(...) bytes; same rules
 *                   as pa_decode's workspace.
 *   Other arguments as for pa_decode.
 *   Source: CSDN essay, first and third sections (the decode kernel), and
 *   its section on speculative decoding (drafted tokens checked in one
 *   pass); the causal rule of the prefill description on the same pages.
 */
size_t pa_decode_multi_workspace_size(int32_t batch, int32_t q_per_seq, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size);
int pa_decode_multi(void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_table, int32_t max_blocks_per_seq,
                    const int32_t* context_lens, int32_t batch, int32_t q_per_seq,
                    int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                    int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_prefill_workspace_size -- bytes of device workspace pa_prefill needs for
 * these sizes (0 when no query block can be split: contexts of at most
 * 1024 tokens, i.e. max_blocks_per_seq <= 4).  Also 0 for invalid arguments;
 * pa_prefill then reports the error.
 */
size_t pa_prefill_workspace_size(int32_t batch, int64_t total_q_rows, int32_t max_seqlen_q,
                                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t max_blocks_per_seq);

/*
 * pa_prefill -- causal varlen attention of prompt tokens over the paged cache.
 *
 * Sequence b owns query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 (q_len_b of
 * them).  Query row i of sequence b is the token at position
 * a = context_lens[b] - q_len_b + i and attends to the cached positions 0..a of
 * the same sequence (bottom-right aligned causal mask, so a cached prefix is
 * seen in full), with the same softmax formula as pa_decode.  The K/V of all
 * context_lens[b] positions must already be in the cache.
 *
 *   out, q        : bf16 [total_q_rows][num_q_heads][head_dim], 16-B aligned.
 *   cu_seqlens_q  : int32 [batch+1], non-decreasing, cu_seqlens_q[0] = 0,
 *                   cu_seqlens_q[batch] = total_q_rows (if it is larger, no
 *                   query block is split, which is slower but still correct).
 *   context_lens  : int32 [batch].
 *   max_seqlen_q  : an upper bound of q_len_b (sizes the launch).
 *   workspace     : DEVICE, 256-B aligned, at least pa_prefill_workspace_size
 *                   bytes (may be NULL when that is 0): scratch for the
 *                   partial states of query blocks whose context is split
 *                   across workgroups (a second kernel on the same stream
 *                   merges them), and, when the query lengths are ragged
 *                   (total_q_rows < batch * max_seqlen_q) and contexts may
 *                   exceed 4 blocks, for the order in which the workgroups
 *                   take the query blocks: longest first, written by a
 *                   small kernel on the same stream before the attention
 *                   kernel.  No initial contents are needed.  Calls that
 *                   overlap in time must not share a workspace.
 *   Source: nano-vllm hub page, "Scheduler" (prefill fills the cache with the
 *   prompt); CSDN essay, reading vLLM's attention module (prefill kernel);
 *   the split-context merge follows the decode description in the same essay.
 */
int pa_prefill(void* out, const void* q, const int32_t* cu_seqlens_q,
               const int32_t* context_lens, int32_t batch, int32_t max_seqlen_q,
               int64_t total_q_rows, const void* k_cache, const void* v_cache,
               const int32_t* block_table, int32_t max_blocks_per_seq, int32_t num_q_heads,
               int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
               float scale, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_copy_blocks -- copy whole cache blocks inside one pool (copy-on-write of
 * a block shared by several sequences before one of them extends it).
 *
 * For every pair i < n_pairs with (src, dst) = (pairs[2i], pairs[2i+1]), both
 * indexes in [0, num_blocks) and src != dst: block dst of the K cache and of
 * the V cache (all kv heads) receives a bit copy of block src.  Pairs with an
 * index outside the pool (e.g. -1 padding) or src == dst are skipped.
 *
 *   k_cache, v_cache : the pools, layouts above, num_blocks blocks each.
 *   pairs         : DEVICE int32 [n_pairs][2], 4-B aligned.
 *   Precondition (not checked on the device; pa_validate_block_pairs checks
 *   it on the host): no block is the destination of two pairs or both a
 *   source and a destination in one call -- otherwise the result depends on
 *   the order of the copies.
 *   Source: CSDN essay comparing nanoVLLM and vLLM, first section (blocks
 *   are allocated per sequence through the block table; vLLM's block
 *   management).
 */
int pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int64_t n_pairs,
                   int64_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                   int32_t head_dim, void* stream);

/*
 * pa_swap_blocks -- copy whole blocks between two pools of the same layout,
 * typically the device cache and a pinned host cache (swap-out for
 * preemption and swap-in when the sequence resumes).
 *
 * For every pair i, block host_pairs[2i+1] of (dst_k, dst_v) receives a bit
 * copy of block host_pairs[2i] of (src_k, src_v).  Runs of pairs whose source
 * and destination both advance by one block become one transfer.  The copies
 * are asynchronous DMA transfers on `stream` (no kernel); host pools should be
 * pinned (hipHostMalloc) for them to overlap with other work.
 *
 *   src_k, src_v, dst_k, dst_v : pools with src_num_blocks / dst_num_blocks
 *                   blocks, each a device pointer or a host pointer known to
 *                   the HIP runtime; source and destination pools are
 *                   different allocations.
 *   host_pairs    : HOST int32 [n_pairs][2] (src block, dst block); every
 *                   index must lie in its pool (else PA_ERR_SLOT_RANGE and
 *                   nothing is copied).  Destinations should be distinct.
 *   Source: CSDN essay comparing nanoVLLM and vLLM, first and closing
 *   sections (vLLM swaps KV cache out to CPU memory under memory pressure
 *   and back in later; nano-vllm has no swap).
 */
int pa_swap_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                   const int32_t* host_pairs, int64_t n_pairs, int64_t src_num_blocks,
                   int64_t dst_num_blocks, int32_t block_size, int32_t num_kv_heads,
                   int32_t head_dim, void* stream);

/*
 * pa_validate_block_pairs -- host-side check of a pa_copy_blocks pair list
 * (HOST int32 [n_pairs][2]).  Pairs that pa_copy_blocks skips (a negative
 * index or src == dst) are ignored.  Returns PA_ERR_SLOT_RANGE if an index is
 * >= num_blocks, PA_ERR_BLOCK_CONFLICT if a block is the destination of two
 * pairs or both a source and a destination, PA_OK otherwise.
 */
int pa_validate_block_pairs(const int32_t* host_pairs, int64_t n_pairs, int64_t num_blocks);

/*
 * Host block manager -- the bookkeeping that produces block tables and slot
 * mappings for the calls above (host memory only; no GPU work).
 *
 * Source: nano-vllm hub page, "KV Cache block management" (blocks of a fixed
 * 256 tokens, allocated and released with reference counts); CSDN essay
 * comparing nanoVLLM and vLLM, first section (a per-sequence block table of
 * physical blocks allocated on demand: a sequence takes a new block each time
 * its length reaches 256k+1).
 *
 * Sequences are named by caller-chosen int64 ids.  Free blocks are handed out
 * first-in first-out, starting from block 0 (released blocks join the end).
 * Every call is serialised by a mutex inside the manager; all pointers are
 * HOST pointers.  Errors return a negative PA_ERR_* code (detail in
 * pa_last_error_detail) and leave the manager unchanged.
 */
typedef struct pa_block_manager pa_block_manager;

/* A manager of num_blocks blocks of block_size tokens (every slot must fit
 * an int32); NULL on bad arguments. */
pa_block_manager* pa_bm_create(int64_t num_blocks, int32_t block_size);
void pa_bm_destroy(pa_block_manager* bm);

/* Blocks currently free (-1 for a NULL manager). */
int64_t pa_bm_num_free(pa_block_manager* bm);

/* New sequence `seq` holding num_tokens tokens (e.g. a prompt):
 * ceil(num_tokens / block_size) blocks.  PA_ERR_NO_BLOCKS if too few are
 * free, PA_ERR_BAD_SHAPE if seq exists. */
int pa_bm_allocate(pa_block_manager* bm, int64_t seq, int64_t num_tokens);

/* One more token for `seq`: *slot_out receives its cache slot.  When the new
 * length is k*block_size + 1 a new block is taken; otherwise, if the last
 * block is shared with another sequence, a private copy is taken first and
 * copy_pair_out[0..1] = (shared block, new block) -- the caller copies it
 * with pa_copy_blocks before storing; else copy_pair_out = (-1, -1). */
int pa_bm_append(pa_block_manager* bm, int64_t seq, int32_t* slot_out, int32_t* copy_pair_out);

/* pa_bm_append for every sequence of a decode step, in the order given, as one
 * all-or-nothing call: slots_out[i] receives the slot of seqs[i]'s new token;
 * the copy pairs the step produced are packed into pairs_out[0 .. 2*k) (room
 * for 2*n int32 must be there) and *n_pairs_out = k -- a list ready for
 * pa_copy_blocks, which must run before the step's tokens are stored.  The
 * blocks the batch needs are counted first: PA_ERR_NO_BLOCKS if too few are
 * free, PA_ERR_BAD_SHAPE if a sequence is unknown or listed twice; either way
 * nothing changes. */
int pa_bm_append_batch(pa_block_manager* bm, const int64_t* seqs, int32_t n, int32_t* slots_out,
                       int32_t* pairs_out, int32_t* n_pairs_out);

/* `child` shares every block of `parent` (reference counts + 1). */
int pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child);

/* Release `seq`: reference counts - 1; blocks reaching zero become free. */
int pa_bm_free(pa_block_manager* bm, int64_t seq);

/* Tokens held by `seq` (-1 if unknown). */
int64_t pa_bm_seq_len(pa_block_manager* bm, int64_t seq);

/* Rows of an int32 [n][max_blocks_per_seq] block table (-1 padded) for the
 * n sequences seqs[0..n); PA_ERR_BAD_SHAPE if one needs more columns. */
int pa_bm_block_table(pa_block_manager* bm, const int64_t* seqs, int32_t n, int32_t* table_out,
                      int32_t max_blocks_per_seq);

/* Cache slots of positions first_pos .. first_pos+count-1 of `seq`. */
int pa_bm_slot_mapping(pa_block_manager* bm, int64_t seq, int64_t first_pos, int64_t count,
                       int32_t* slots_out);

/*
 * Debug checks of the data-dependent preconditions on the device.  When on
 * (environment variable PA_DEBUG=1 at the first call, or this call), every
 * pa_store_kv, pa_decode, pa_decode_multi and pa_prefill first runs a small
 * kernel on its stream that checks the device-resident inputs -- slots
 * inside the pool; context_lens inside [0, min(max_context_len,
 * max_blocks_per_seq * block_size)]; every block-table entry a sequence uses
 * inside [0, num_blocks); for pa_prefill cu_seqlens_q[0] = 0, 0 <= q_len_b
 * <= min(context_lens[b], max_seqlen_q) and cu_seqlens_q[batch] =
 * total_q_rows; for pa_decode_multi context_lens[b] >= q_per_seq -- then
 * SYNCHRONISES the stream and returns PA_ERR_PRECONDITION (detail naming the
 * violated conditions) without launching the call's own kernels.  Duplicate
 * slots are left to pa_validate_slots.  Not for use under graph capture.
 * Returns the previous setting (1 on, 0 off).
 */
int pa_set_debug_checks(int enabled);

/*
 * pa_set_decode_waves -- testing aid: fix the number of runs (waves) the
 * decode calls (pa_decode, pa_decode_append, pa_decode_append_noalloc,
 * pa_decode_multi) cut their work list into, so that one input can be
 * decoded under different split-context plans: 1 streams every (sequence,
 * kv head) whole in one wave, larger counts cut the contexts into more
 * partial states (at most 8 per compute unit, the count every workspace is
 * sized for; a larger value is clamped to it).  0 (the default) restores the
 * automatic count.  Results differ between plans by rounding only.  Applies
 * to calls made after it, from any thread.  Returns the previous setting.
 */
int pa_set_decode_waves(int32_t waves);

/* Name of a status code ("PA_OK", "PA_ERR_NULL_PTR", ...); never NULL. */
const char* pa_status_string(int status);

/* Detail of the last error returned on this thread ("" if none). */
const char* pa_last_error_detail(void);

/*
 * pa_validate_slots -- host-side check of a slot mapping (a debugging aid for
 * the store's data preconditions).  host_slots is a HOST array of n slots.
 * Returns PA_ERR_SLOT_RANGE if some slot is >= num_slots, PA_ERR_DUPLICATE_SLOT
 * if two non-negative slots are equal, PA_OK otherwise.
 */
int pa_validate_slots(const int32_t* host_slots, int64_t n, int64_t num_slots);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
